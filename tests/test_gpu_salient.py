"""Mixed precision with fp16 salient channels (blog.ohmyagent.ai "技术实现" 1
and "混合精度设计"; xxmr.cn §2.2), through the C ABI against the oracle.

Selection and the stored form: bit-exact (indices, packed codes, scales,
zero-points, fp16 side columns). Mixed linear layer: relative Frobenius
error <= 1e-3 and |y - y_ref| <= 1e-2 * (|y_ref| + 1) per element on every
path. Losses: within 2e-6 relative of the oracle (no activation is rescaled
here, so only fp32 accumulation separates them), the same channels.
"""

import base64
import hashlib
import json
import os

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import LOSS_RTOL_F16, assert_linear_close, dev, fp32_loss_rtol, host, say  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("K,n", [(4096, 41), (11008, 110), (28672, 287), (1000, 1000), (300, 7), (64, 0)])
def test_select_matches_oracle_with_ties(K, n):
    rng = np.random.default_rng([190, K])
    m = rng.integers(0, 50, size=K).astype(np.float64) / 8.0 + 1e-8    # many equal values
    say("select", K, n)
    idx = awq.select_salient(dev(m), n)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx).astype(np.int64), oracle.salient_channels(m, n))


def test_select_from_activations_finds_planted_channels():
    lay = synth.make_layer(64, 4096, 512, seed=[191], w_std=0.02)
    m = awq.awq_activation_absmean(dev(lay["x"]))
    idx = host(awq.select_salient(m, 41)).astype(np.int64)
    assert np.array_equal(idx, oracle.salient_channels(oracle.activation_absmean(lay["x"]), 41))
    assert np.array_equal(np.sort(idx), lay["salient"])


def random_channels(K, n, seed):
    """Distinct channels, including the first and last and neighbours that
    share a packed word."""
    rng = np.random.default_rng(seed)
    base = [0, K - 1, 8, 9, 10, 15]
    rest = rng.choice(np.arange(16, K - 1), n - len(base), replace=False)
    return np.concatenate([base, rest]).astype(np.int32)


@pytest.mark.parametrize("G", [32, 128, 512])
@pytest.mark.parametrize("symmetric", [False, True])
def test_quantize_salient_bit_exact(G, symmetric):
    N, K = 1000, 2048
    lay = synth.make_layer(N, K, 0, seed=[192, G], w_std=0.02)
    idx = random_channels(K, 25, [193, G])
    say("quantize salient G", G, "sym" if symmetric else "asym")
    qw, sc, zr, ws = awq.awq_quantize_salient(dev(lay["w"]), G, dev(idx), symmetric=symmetric)
    torch.cuda.synchronize()
    eqw, esc, ezr, ews = oracle.quantize_salient(lay["w"], G, idx, symmetric)
    assert np.array_equal(host(qw).view(np.uint32), eqw)
    assert np.array_equal(host(sc).view(np.uint16), esc.view(np.uint16))
    assert np.array_equal(host(zr).view(np.uint16), ezr.view(np.uint16))
    assert np.array_equal(host(ws).view(np.uint16), ews.view(np.uint16))


@pytest.mark.parametrize("M,N,K,path,with_ws", [
    (1, 11008, 4096, awq.PATH_AUTO, False),     # decode GEMV
    (3, 257, 2048, awq.PATH_GEMV, False),
    (16, 4096, 4096, awq.PATH_AUTO, True),      # skinny
    (300, 700, 2048, awq.PATH_GEMM, False),     # ragged GEMM
    (2048, 1000, 1024, awq.PATH_GEMM, True),    # more rows than one side tile
])
def test_mixed_linear(M, N, K, path, with_ws):
    G = 128
    lay = synth.make_layer(N, K, M, seed=[194, M, N, K], w_std=0.02)
    n = oracle.salient_count(K)
    idx = np.sort(lay["salient"]).astype(np.int32)[:n]
    say("mixed linear", M, N, K, "path", path, "n", n)
    qw, sc, zr, ws = oracle.quantize_salient(lay["w"], G, idx)
    w_ws = awq.gemm_workspace(M, N, K) if with_ws else None
    y = awq.awq_gemm_salient(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), dev(idx), dev(ws), G,
                             path=path, workspace=w_ws)
    assert_linear_close(host(y), oracle.linear_salient_ref(lay["x"], qw, sc, zr, G, idx, ws))


def test_apply_adds_in_place_and_skips_nothing():
    """apply on a zero y gives the side product alone; n = 0 leaves y."""
    M, N, K = 70, 300, 512
    rng = np.random.default_rng(195)
    x = rng.standard_normal((M, K)).astype(np.float16)
    idx = random_channels(K, 40, 196)
    ws = (rng.standard_normal((40, N)) * 0.1).astype(np.float16)
    y = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    awq.awq_salient_apply(dev(x), dev(idx), dev(ws), y)
    ref = x.astype(np.float64)[:, idx] @ ws.astype(np.float64)
    assert_linear_close(host(y), ref)
    before = y.clone()
    awq.awq_salient_apply(dev(x), dev(idx[:0]), dev(ws[:0]), y)
    assert torch.equal(before, y)


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("symmetric", [False, True])
def test_salient_loss_matches_oracle(G, symmetric):
    lay = synth.make_layer(256, 1024, 512, seed=[197, G], w_std=0.02)
    w, x = lay["w"], lay["x"]
    n = oracle.salient_count(1024)
    say("salient loss G", G, "sym" if symmetric else "asym")
    lr, ls, idx = awq.awq_salient_loss(dev(w), dev(x), G, n, symmetric=symmetric)
    idx_o = oracle.salient_channels(oracle.activation_absmean(x), n)
    assert np.array_equal(host(idx).astype(np.int64), idx_o)
    lr_o = oracle.salient_loss(w, x, G, [], symmetric=symmetric)
    ls_o = oracle.salient_loss(w, x, G, idx_o, symmetric=symmetric)
    say("rtn", lr, lr_o, "salient", ls, ls_o)
    tol_r = fp32_loss_rtol(x, w, oracle.mixed_weight(w, G, [], symmetric))
    tol_s = fp32_loss_rtol(x, w, oracle.mixed_weight(w, G, idx_o, symmetric))
    assert abs(lr - lr_o) <= tol_r * lr_o
    assert abs(ls - ls_o) <= tol_s * ls_o
    assert ls < lr


def test_salient_loss_zero_channels_is_rtn():
    lay = synth.make_layer(200, 512, 333, seed=[198], w_std=0.02)
    lr, ls, idx = awq.awq_salient_loss(dev(lay["w"]), dev(lay["x"]), 128, 0)
    assert idx.numel() == 0 and lr == ls


@pytest.mark.timeout(600)
def test_salient_loss_full_size():
    """The scale search's workload (W[11008, 4096], X[65536, 4096]) against
    the stored oracle values."""
    path = os.path.join(GOLDEN, "salient_7b_mlp_wmult1.json")
    with open(path) as f:
        g = json.load(f)
    lay = synth.search_layer(w_mult=1.0)
    w, x = lay["w"], lay["x"]
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(w).tobytes())
    h.update(np.ascontiguousarray(x).tobytes())
    assert h.hexdigest() == g["inputs_sha256"], "generator output changed"
    say("salient loss full size", w.shape, x.shape)
    lr, ls, idx = awq.awq_salient_loss(dev(w), dev(x), 128, g["n_salient"])
    idx_o = np.frombuffer(base64.b64decode(g["idx_i64_b64"]), dtype="<i8")
    assert np.array_equal(host(idx).astype(np.int64), idx_o)
    say("rtn", lr, g["loss_rtn"], "salient", ls, g["loss_salient"])
    assert abs(lr - g["loss_rtn"]) <= LOSS_RTOL_F16 * g["loss_rtn"]
    assert abs(ls - g["loss_salient"]) <= LOSS_RTOL_F16 * g["loss_salient"]


def test_salient_loss_few_tokens():
    """T <= 8 takes the side product's decode form (the fp32 subtract)."""
    lay = synth.make_layer(300, 1024, 5, seed=[199], w_std=0.02)
    w, x = lay["w"], lay["x"]
    lr, ls, idx = awq.awq_salient_loss(dev(w), dev(x), 128, 10)
    idx_o = oracle.salient_channels(oracle.activation_absmean(x), 10)
    assert np.array_equal(host(idx).astype(np.int64), idx_o)
    ls_o = oracle.salient_loss(w, x, 128, idx_o, use_gram=False)
    tol = fp32_loss_rtol(x, w, oracle.mixed_weight(w, 128, idx_o))
    say("few-token salient loss deviation", abs(ls - ls_o) / ls_o, "bar", tol)
    assert abs(ls - ls_o) <= tol * ls_o
