"""Format variants (aissn.com 量化粒度 and 对称/非对称量化): group
sizes 32 and 256 beside 64 and 128, and the symmetric map (zero-point 0 as
the signed code, stored as code + 8 with zero-point 8).

Quantize: bit-exact against the oracle. Linear layer: relative Frobenius
error <= 1e-3 and |y - y_ref| <= 1e-2 * (|y_ref| + 1) per element, on every
path (GEMV, skinny with and without K splits, GEMM and its stream-K form).
Scale search: the oracle's alpha.
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import (assert_linear_close, assert_quant_equal, check_search, dev, host,  # noqa: E402
                             say)


def gpu_quantize(w16, G, cs=None, symmetric=False):
    qw, sc, zr = awq.awq_quantize(dev(w16), G, None if cs is None else dev(cs.astype(np.float32)),
                                  symmetric=symmetric)
    torch.cuda.synchronize()
    return host(qw).view(np.uint32), host(sc), host(zr)


@pytest.mark.parametrize("N,K,G", [(N, K, G) for G in (32, 256, 512)
                                   for (N, K) in ((11008, 4096), (4096, 11008), (77, 1536)) if K % G == 0])
def test_quantize_group_sizes_bit_exact(N, K, G):
    """Every shape whose K the group size divides (11008 = 43 * 256)."""
    lay = synth.decode_layer(N, K, 0, G)
    say("quantize G", G, N, K)
    assert_quant_equal(gpu_quantize(lay["w"], G), oracle.quantize(lay["w"], G))


@pytest.mark.parametrize("G", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("scaled", [False, True])
def test_quantize_symmetric_bit_exact(G, scaled):
    N, K = 1000, 2048
    lay = synth.make_layer(N, K, 0, seed=[150, G], w_std=0.02, salient_frac=0.01)
    cs = None
    if scaled:
        rng = np.random.default_rng([151, G])
        cs = (np.abs(rng.standard_normal(K)) + 0.1).astype(np.float32)
    say("quantize symmetric G", G, "scaled" if scaled else "")
    got = gpu_quantize(lay["w"], G, cs, symmetric=True)
    exp = oracle.quantize_symmetric(lay["w"], G, cs)
    assert_quant_equal(got, exp)
    assert np.all(got[2] == 8)


def linear_cases():
    # (label, M, N, K, path, with workspace)
    return [
        ("gemv", 1, 11008, 4096, awq.PATH_GEMV, False),
        ("gemv", 3, 257, 2048, awq.PATH_GEMV, False),
        ("skinny", 16, 4096, 4096, awq.PATH_SKINNY, True),
        ("skinny", 16, 1000, 2048, awq.PATH_SKINNY, False),
        ("skinny", 40, 300, 1024, awq.PATH_SKINNY, True),
        ("gemm", 300, 700, 2048, awq.PATH_GEMM, False),
        ("gemm-streamk", 512, 1000, 4096, awq.PATH_GEMM, True),
    ]


@pytest.mark.parametrize("symmetric", [False, True])
@pytest.mark.parametrize("G", [32, 256])
@pytest.mark.parametrize("case", linear_cases(), ids=lambda c: f"{c[0]}-M{c[1]}-{c[2]}x{c[3]}")
def test_linear_paths_group_sizes(case, G, symmetric):
    label, M, N, K, path, with_ws = case
    lay = synth.make_layer(N, K, M, seed=[152, M, N, K, G, int(symmetric)], w_std=0.02)
    say("linear", label, M, N, K, "G", G, "sym" if symmetric else "asym")
    qw, sc, zr = (oracle.quantize_symmetric if symmetric else oracle.quantize)(lay["w"], G)
    ws = awq.gemm_workspace(M, N, K) if with_ws else None
    y = awq.awq_gemm(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G, path=path, workspace=ws)
    assert_linear_close(host(y), oracle.linear_ref(lay["x"], qw, sc, zr, G))


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("symmetric", [False, True])
def test_linear_paths_symmetric_smaller_groups(G, symmetric):
    """The other two group sizes through the automatic choice, symmetric and
    asymmetric (a ragged 5 x 333 x 1216 product: skinny or GEMV)."""
    M, N, K = 5, 333, 1216 if G == 64 else 1184
    lay = synth.make_layer(N, K, M, seed=[153, G, int(symmetric)], w_std=0.02)
    qw, sc, zr = (oracle.quantize_symmetric if symmetric else oracle.quantize)(lay["w"], G)
    y = awq.awq_gemm(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G)
    assert_linear_close(host(y), oracle.linear_ref(lay["x"], qw, sc, zr, G))


@pytest.mark.parametrize("G", [32, 256, 512])
def test_scale_search_group_sizes(G):
    lay = synth.make_layer(256, 512, 512, seed=[154, G], w_std=0.02, w_mult=1.0)
    w, x = lay["w"], lay["x"]
    losses_o, best_o, s_o = oracle.scale_search(w, x, G)
    losses_f, _, _ = oracle.scale_search(w, x, G, f16_activations=True)
    losses, best, s = awq.awq_scale_search(dev(w), dev(x), G)
    say("search G", G, "gpu", best, "oracle", best_o)
    check_search(losses, best, host(s), losses_o, best_o, s_o, losses_f)


@pytest.mark.parametrize("symmetric", [False, True])
@pytest.mark.parametrize("case", [c for c in linear_cases() if c[0] != "skinny"] +
                         [("auto", 16, 1000, 2048, awq.PATH_AUTO, False), ("auto", 40, 300, 1024, awq.PATH_AUTO, True)],
                         ids=lambda c: f"{c[0]}-M{c[1]}-{c[2]}x{c[3]}")
def test_linear_paths_group_512(case, symmetric):
    """G = 512 (the largest group size): GEMV, GEMM and its stream-K form; the
    skinny kernel stops at G = 256, so batched decode shapes take the
    automatic choice (GEMV or GEMM)."""
    label, M, N, K, path, with_ws = case
    G = 512
    lay = synth.make_layer(N, K, M, seed=[155, M, N, K, int(symmetric)], w_std=0.02)
    say("linear G=512", label, M, N, K, "sym" if symmetric else "asym")
    qw, sc, zr = (oracle.quantize_symmetric if symmetric else oracle.quantize)(lay["w"], G)
    ws = awq.gemm_workspace(M, N, K) if with_ws else None
    y = awq.awq_gemm(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G, path=path, workspace=ws)
    assert_linear_close(host(y), oracle.linear_ref(lay["x"], qw, sc, zr, G))


def test_skinny_refuses_group_512():
    lay = synth.make_layer(64, 1024, 16, seed=[156], w_std=0.02)
    qw, sc, zr = oracle.quantize(lay["w"], 512)
    with pytest.raises(awq.AwqError):
        awq.awq_gemm(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), 512, path=awq.PATH_SKINNY)
