"""W8A16 (aissn.com "INT8 vs INT4" and "INT8 实战": 8-bit weights, fp16
activations) through the C ABI against the oracle.

Quantize: bit-exact (codes, scales, zero-points). Linear layer: relative
Frobenius error <= 1e-3 and |y - y_ref| <= 1e-2 * (|y_ref| + 1) per element,
on the GEMV and the MFMA GEMM (with and without stream-K), ragged shapes
included.
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import assert_linear_close, dev, extreme_quotient_rows, host, say  # noqa: E402


def gpu_quantize_w8(w16, G, cs=None, symmetric=False):
    qw, sc, zr = awq.awq_quantize_w8(dev(w16), G, None if cs is None else dev(cs.astype(np.float32)),
                                     symmetric=symmetric)
    torch.cuda.synchronize()
    return host(qw).view(np.uint32), host(sc), host(zr)


def assert_equal_bits(got, exp):
    for a, b in zip(got, exp):
        a, b = np.asarray(a), np.asarray(b)
        assert a.shape == b.shape
        n_bad = int(np.count_nonzero(a.view(np.uint8) != b.view(np.uint8)))
        assert n_bad == 0, f"{n_bad} mismatching bytes"


@pytest.mark.parametrize("G", [64, 128, 256, 512])
@pytest.mark.parametrize("symmetric", [False, True])
def test_quantize_w8_bit_exact(G, symmetric):
    lay = synth.make_layer(1000, 2048, 0, seed=[210, G], w_std=0.02)
    say("quantize w8 G", G, "sym" if symmetric else "asym")
    assert_equal_bits(gpu_quantize_w8(lay["w"], G, symmetric=symmetric),
                      oracle.quantize_w8(lay["w"], G, symmetric=symmetric))


def test_quantize_w8_full_size_and_scaled():
    lay = synth.decode_layer(11008, 4096, 0, 128)
    assert_equal_bits(gpu_quantize_w8(lay["w"], 128), oracle.quantize_w8(lay["w"], 128))
    rng = np.random.default_rng(211)
    cs = (np.abs(rng.standard_normal(4096)) + 0.1).astype(np.float32)
    w = lay["w"][:700]
    assert_equal_bits(gpu_quantize_w8(w, 128, cs), oracle.quantize_w8(w, 128, cs))


@pytest.mark.parametrize("M,N,K,G,path,with_ws", [
    (1, 11008, 4096, 128, awq.PATH_AUTO, False),      # GEMV, one-shot rows
    (1, 4096, 11008, 128, awq.PATH_AUTO, False),      # GEMV, streaming ring
    (3, 257, 2048, 64, awq.PATH_GEMV, False),
    (8, 1000, 1536, 512, awq.PATH_AUTO, False),
    (16, 4096, 4096, 128, awq.PATH_AUTO, True),       # batched decode on the GEMM
    (300, 700, 2048, 256, awq.PATH_GEMM, False),
    (512, 1000, 4096, 128, awq.PATH_GEMM, True),      # stream-K
    (2048, 11008, 4096, 128, awq.PATH_AUTO, False),   # prefill shape
])
@pytest.mark.parametrize("symmetric", [False, True])
def test_linear_w8(M, N, K, G, path, with_ws, symmetric):
    lay = synth.make_layer(N, K, M, seed=[212, M, N, K, G], w_std=0.02)
    say("linear w8", M, N, K, "G", G, "path", path, "sym" if symmetric else "asym")
    qw, sc, zr = oracle.quantize_w8(lay["w"], G, symmetric=symmetric)
    ws = awq.gemm_workspace(M, N, K) if with_ws else None
    y = awq.awq_gemm_w8(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G, path=path, workspace=ws)
    assert_linear_close(host(y), oracle.linear_ref_w8(lay["x"], qw, sc, zr, G))


def test_w8_one_hot_is_exact_on_gemv():
    """x = e_k picks column k of the dequantized weight: exact on the GEMV
    (the fp32 sum of one exact product)."""
    N, K, G = 300, 1024, 128
    lay = synth.make_layer(N, K, 0, seed=[213], w_std=0.02)
    qw, sc, zr = oracle.quantize_w8(lay["w"], G)
    w_hat = oracle.dequantize_w8(qw, sc, zr, G, K)
    x = np.zeros((4, K), dtype=np.float16)
    ks = [0, 77, 512, 1023]
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = host(awq.awq_gemm_w8(dev(x), dev(qw.view(np.int32)), dev(sc), dev(zr), G, path=awq.PATH_GEMV))
    exp = w_hat[:, ks].T.astype(np.float16)
    assert np.array_equal(y.view(np.uint16), exp.view(np.uint16))


@pytest.mark.parametrize("symmetric", [False, True])
def test_quantize_w8_extreme_quotients_bit_exact(symmetric):
    """The 255-level map on groups whose quotients are far from the codes
    (constant, offset and outlier groups)."""
    w = extreme_quotient_rows(128)
    for G in (64, 128):   # W8 group sizes start at 64
        assert_equal_bits(gpu_quantize_w8(w, G, symmetric=symmetric), oracle.quantize_w8(w, G, symmetric=symmetric))
