"""Parity of the skinny MFMA kernel (4 < M <= 64, path 3 and the automatic
choice for that range) with the CPU oracle: relative Frobenius error <= 1e-3
and |y - y_ref| <= 1e-2 * (|y_ref| + 1) per element, with the K splits a
workspace enables and without them (one block per column tile, K staged in
LDS-sized phases when it does not fit at once). A one-hot input reproduces
the dequantized column exactly (one nonzero term, one scale multiply, one
fp16 rounding).
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import DEV, assert_linear_close, dev, host, sampled_rows, say  # noqa: E402


def skinny(x, qw, sc, zr, G, ws=None, out=None, path=awq.PATH_SKINNY):
    return awq.awq_gemm(x, qw, sc, zr, G, path=path, out=out, workspace=ws)


def skinny_no_workspace(args):
    """Path 3 without a workspace: one block per column tile over all of K."""
    return host(skinny(*args))


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("N,K", synth.DECODE_SHAPES)
def test_decode_m16_against_oracle(N, K, split):
    """With a workspace the skinny kernel splits K; without one the
    automatic choice runs one block per column tile over K in phases."""
    lay = synth.decode_layer(N, K, 16)
    say("skinny decode M=16", N, K, "split" if split else "auto, no workspace")
    qw, sc, zr = oracle.quantize(lay["w"], 128)
    args = (dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), 128)
    if split:
        y = skinny(*args, ws=awq.gemm_workspace(16, N, K))
    else:
        y = awq.awq_gemm(*args)
    assert_linear_close(host(y), oracle.linear_ref(lay["x"], qw, sc, zr, 128))


@pytest.mark.parametrize("G", synth.SWEEP_G)
@pytest.mark.parametrize("N,K", synth.SWEEP_SHAPES)
def test_sweep_m32_split_full_size_sampled(N, K, G):
    """M = 32 on the 13B/70B shapes through the automatic choice with a
    workspace (K split); sampled output columns against the oracle."""
    lay = synth.sweep_layer(N, K, 32, G)
    say("skinny sweep M=32 split", N, K, G)
    qw, sc, zr = awq.awq_quantize(dev(lay["w"]), G)
    ws = awq.gemm_workspace(32, N, K)
    y = host(awq.awq_gemm(dev(lay["x"]), qw, sc, zr, G, workspace=ws))
    rows = sampled_rows(N, 128, N + K + G)
    eq = oracle.quantize(lay["w"][rows], G)
    assert_linear_close(y[:, rows], oracle.linear_ref(lay["x"], *eq, G))


@pytest.mark.parametrize("M,N,K,G", [
    (5, 1, 64, 64), (8, 100, 128, 128), (16, 130, 192, 64), (17, 257, 640, 64), (31, 129, 1216, 64),
    (32, 300, 2048, 128), (33, 77, 384, 128), (48, 1000, 512, 64), (64, 200, 4096, 128), (64, 3, 11008, 128),
    # whole K in one block's LDS at the limit, and just past it (split only)
    (16, 600, 3840, 128), (16, 600, 3968, 128), (16, 300, 3200, 64), (16, 300, 3264, 64),
    (20, 513, 1920, 64), (20, 513, 1984, 64), (40, 260, 1024, 128), (40, 260, 1152, 128),
])
def test_skinny_ragged_against_oracle(M, N, K, G):
    lay = synth.make_layer(N, K, M, seed=[130, M, N, K, G], w_std=0.02)
    say("skinny ragged", M, N, K, G)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    y_ref = oracle.linear_ref(lay["x"], qw, sc, zr, G)
    args = (dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G)
    assert_linear_close(skinny_no_workspace(args), y_ref)
    assert_linear_close(host(skinny(*args, ws=awq.gemm_workspace(M, N, K))), y_ref)
    assert_linear_close(host(awq.awq_gemm(*args)), y_ref)     # automatic choice


@pytest.mark.parametrize("M,N,K,G", [
    (16, 300, 8192, 128),     # 3 phases of 24 groups (ring depth 8)
    (9, 257, 11008, 64),
    (33, 130, 6144, 256),     # 4 row blocks of 16, ring depth 4
    (64, 100, 5120, 32),
    (17, 513, 28672, 128),
    (6, 4096, 11008, 128),    # the decode down projection at a small batch
])
def test_skinny_phases_against_oracle(M, N, K, G):
    """K beyond one block's LDS without a workspace: staged in phases that
    are a multiple of the weight ring's depth, the last one partial."""
    lay = synth.make_layer(N, K, M, seed=[133, M, N, K, G], w_std=0.02)
    say("skinny phases", M, N, K, G)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    y_ref = oracle.linear_ref(lay["x"], qw, sc, zr, G)
    args = (dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G)
    assert_linear_close(skinny_no_workspace(args), y_ref)
    assert_linear_close(host(awq.awq_gemm(*args)), y_ref)     # automatic choice, no workspace


def test_skinny_phases_one_hot_is_exact():
    """One-hot rows over a K of 3 phases pick single dequantized columns in
    every phase, exactly."""
    N, K, G = 200, 8192, 128
    lay = synth.make_layer(N, K, 0, seed=[134], w_std=0.02)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    w_hat = oracle.dequantize(qw, sc, zr, G, K)
    ks = [0, 1, 3071, 3072, 3073, 5000, 6143, 6144, 8191, 4096, 128, 7000, 2047, 6200, 999, 7999]
    x = np.zeros((len(ks), K), dtype=np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = host(skinny(dev(x), dev(qw.view(np.int32)), dev(sc), dev(zr), G))
    assert np.array_equal(y, w_hat[:, ks].T.astype(np.float16))


@pytest.mark.parametrize("split", [False, True])
def test_skinny_one_hot_is_exact(split):
    N, K, G = 384, 1024, 128
    lay = synth.make_layer(N, K, 0, seed=[131], w_std=0.02)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    w_hat = oracle.dequantize(qw, sc, zr, G, K)
    ks = [0, 1, 7, 8, 127, 128, 200, 511, 512, 700, 1000, 1023, 64, 300, 900, 5, 33]
    x = np.zeros((len(ks), K), dtype=np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    ws = awq.gemm_workspace(len(ks), N, K) if split else None
    y = host(skinny(dev(x), dev(qw.view(np.int32)), dev(sc), dev(zr), G, ws))
    assert np.array_equal(y, w_hat[:, ks].T.astype(np.float16))


def test_skinny_deterministic_shared_workspace_and_guard_band():
    G = 128
    shapes = [(16, 4096, 4096), (40, 1000, 2048), (9, 11008, 512), (16, 4096, 4096)]
    ws = awq.gemm_workspace(64, 11008, 4096)
    first = None
    for i, (M, N, K) in enumerate(shapes):
        lay = synth.make_layer(N, K, M, seed=[132, M, N, K], w_std=0.02)
        say("skinny shared workspace", i, M, N, K)
        qw, sc, zr = oracle.quantize(lay["w"], G)
        buf = torch.full((M * N + 2048,), 7.0, dtype=torch.float16, device=DEV)
        y = buf[1024:1024 + M * N].view(M, N)
        skinny(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G, ws, out=y)
        torch.cuda.synchronize()
        b = host(buf)
        assert np.all(b[:1024] == 7.0) and np.all(b[1024 + M * N:] == 7.0)
        assert_linear_close(host(y), oracle.linear_ref(lay["x"], qw, sc, zr, G))
        if i == 0:
            first = y.clone()
        if i == len(shapes) - 1:
            assert torch.equal(y, first)


def test_skinny_graph_replay_matches_eager():
    M, N, K, G = 16, 4096, 4096, 128
    lay = synth.make_layer(N, K, M, seed=[133], w_std=0.02)
    x = dev(lay["x"])
    qw, sc, zr = awq.awq_quantize(dev(lay["w"]), G)
    ws = awq.gemm_workspace(M, N, K)
    e = skinny(x, qw, sc, zr, G, ws).clone()
    y = torch.empty_like(e)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            skinny(x, qw, sc, zr, G, ws, out=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    w2 = dev(synth.make_layer(512, 512, 0, seed=[134])["w"])
    for r in range(4):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        awq.awq_quantize(w2, 128)
        torch.cuda.synchronize()
        assert torch.equal(y, e), r
