"""Parity of the stream-K MFMA GEMM (awq_gemm_ex with a workspace) with the
CPU oracle, on the same bar as the other linear-layer tests: relative
Frobenius error <= 1e-3 and |y - y_ref| <= 1e-2 * (|y_ref| + 1) per element.

A workspace makes the library split the K loop of output tiles across thread
blocks whenever the tile count leaves resident blocks idle, which is the case
for every shape below on a 256-CU device. A split tile's partial sums are
added in a fixed order, so repeated calls give identical bits, and the
workspace is left ready for the next call without clearing.
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import DEV, assert_linear_close, dev, host, sampled_rows, say  # noqa: E402


def assert_close_per_element(y1, y0):
    """A split product against the unsplit one (the same sums in another fp32
    order): the linear-layer bar with y0 as the reference, per element."""
    a, b = y1.double(), y0.double()
    assert bool(torch.all((a - b).abs() <= 1e-2 * (b.abs() + 1)))
    assert float(torch.linalg.norm(a - b)) <= 1e-3 * float(torch.linalg.norm(b))


def gemm_ws(x, qw, sc, zr, G, ws, out=None):
    return awq.awq_gemm(x, qw, sc, zr, G, path=awq.PATH_GEMM, out=out, workspace=ws)


@pytest.mark.parametrize("N,K", synth.PREFILL_SHAPES)
def test_prefill_stream_k_full_size_sampled(N, K):
    """M = 2048 prefill: sampled output columns against the oracle, repeated
    calls bit-identical, and within fp32 summation order of the unsplit GEMM."""
    M, G = synth.PREFILL_M, 128
    lay = synth.prefill_layer(N, K)
    say("prefill stream-k", N, K)
    x = dev(lay["x"])
    qw, sc, zr = awq.awq_quantize(dev(lay["w"]), G)
    ws = awq.gemm_workspace(M, N, K)
    y1 = gemm_ws(x, qw, sc, zr, G, ws).clone()
    y2 = gemm_ws(x, qw, sc, zr, G, ws)
    y0 = awq.awq_gemm(x, qw, sc, zr, G, path=awq.PATH_GEMM)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    rows = sampled_rows(N, 192, N + 7)
    eq = oracle.quantize(lay["w"][rows], G)
    assert_linear_close(host(y1)[:, rows], oracle.linear_ref(lay["x"], *eq, G))
    assert_close_per_element(y1, y0)


@pytest.mark.parametrize("M,N,K,G", [
    (256, 128, 4096, 128),     # one tile, split four ways
    (17, 33, 4096, 64),        # one ragged tile
    (300, 1000, 2048, 128),    # 2 x 8 tiles, ragged rows and columns
    (513, 257, 640, 64),       # K steps = 20: segment edges fall inside groups
    (1000, 700, 1216, 64),     # 19 K steps per tile, odd segment lengths
    (2048, 640, 4096, 128),    # 40 tiles
    (300, 640, 13824, 128),    # 216 K steps per tile: six segments of 36
    (513, 257, 12288, 64),     # 192 K steps: six segments of 32, ragged tiles
])
def test_stream_k_ragged_against_oracle(M, N, K, G):
    lay = synth.make_layer(N, K, M, seed=[120, M, N, K, G], w_std=0.02)
    say("stream-k ragged", M, N, K, G)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    ws = awq.gemm_workspace(M, N, K)
    y = host(gemm_ws(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G, ws))
    assert_linear_close(y, oracle.linear_ref(lay["x"], qw, sc, zr, G))


def test_stream_k_workspace_shared_across_calls():
    """One workspace, sized for the largest call, serves calls of decreasing
    and increasing size back to back without clearing; each result matches
    the oracle and a repeat of the first call gives the same bits."""
    G = 64
    shapes = [(1024, 1536, 1024), (130, 200, 3072), (640, 384, 512), (1024, 1536, 1024)]
    ws = awq.gemm_workspace(1024, 1536, 3072)
    first = None
    for i, (M, N, K) in enumerate(shapes):
        lay = synth.make_layer(N, K, M, seed=[121, M, N, K], w_std=0.02)
        say("stream-k shared workspace", i, M, N, K)
        qw, sc, zr = oracle.quantize(lay["w"], G)
        y = gemm_ws(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G, ws)
        torch.cuda.synchronize()
        assert_linear_close(host(y), oracle.linear_ref(lay["x"], qw, sc, zr, G))
        if i == 0:
            first = y.clone()
        if i == len(shapes) - 1:
            assert torch.equal(y, first)


def test_stream_k_does_not_write_outside_y():
    M, N, K, G = 77, 300, 1024, 128
    lay = synth.make_layer(N, K, M, seed=[122], w_std=0.02)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    buf = torch.full((M * N + 2048,), 7.0, dtype=torch.float16, device=DEV)
    y = buf[1024:1024 + M * N].view(M, N)
    ws = awq.gemm_workspace(M, N, K)
    gemm_ws(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G, ws, out=y)
    torch.cuda.synchronize()
    b = host(buf)
    assert np.all(b[:1024] == 7.0) and np.all(b[1024 + M * N:] == 7.0)
    assert_linear_close(host(y), oracle.linear_ref(lay["x"], qw, sc, zr, G))


def test_stream_k_graph_replay_matches_eager():
    """Captured in a HIP graph, the split GEMM (whose tile counters reset
    inside the kernel, no memset node) gives the eager bits on every replay."""
    M, N, K, G = 2048, 1024, 2048, 128
    lay = synth.make_layer(N, K, M, seed=[123], w_std=0.02)
    x = dev(lay["x"])
    qw, sc, zr = awq.awq_quantize(dev(lay["w"]), G)
    ws = awq.gemm_workspace(M, N, K)
    e = gemm_ws(x, qw, sc, zr, G, ws).clone()
    y = torch.empty_like(e)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            gemm_ws(x, qw, sc, zr, G, ws, out=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    w2 = dev(synth.make_layer(512, 512, 0, seed=[124])["w"])
    for r in range(4):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        awq.awq_quantize(w2, 128)
        torch.cuda.synchronize()
        assert torch.equal(y, e), r


@pytest.mark.parametrize("M,N,K,G", [
    (8192, 8192, 4096, 128),     # 1024 tiles of 256 x 256: the one-block-per-CU geometry
    (12000, 17000, 1024, 64),    # ragged rows and columns on that geometry
    (1280, 8320, 1024, 128),     # 165 tiles: one round, cheaper wide than as 330 narrow tiles
    (1100, 8000, 2048, 64),      # the same with ragged rows and columns
])
def test_wide_tiles_sampled(M, N, K, G):
    """Shapes whose rounds of 256 x 256 tiles cost less than those of the
    256 x 128 tile take the 512-thread geometry without a workspace:
    sampled output columns against the oracle."""
    lay = synth.make_layer(N, K, M, seed=[121, M, N, K, G], w_std=0.02)
    say("wide tiles", M, N, K, G)
    x = dev(lay["x"])
    qw, sc, zr = awq.awq_quantize(dev(lay["w"]), G)
    y = awq.awq_gemm(x, qw, sc, zr, G, path=awq.PATH_GEMM)
    rows = sampled_rows(N, 160, N + 11)
    eq = oracle.quantize(lay["w"][rows], G)
    assert_linear_close(host(y)[:, rows], oracle.linear_ref(lay["x"], *eq, G))


def test_wide_tiles_w8():
    M, N, K, G = 8192, 8192, 1024, 128
    lay = synth.make_layer(N, K, M, seed=[122], w_std=0.02)
    qw, sc, zr = oracle.quantize_w8(lay["w"], G)
    y = awq.awq_gemm_w8(dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G, path=awq.PATH_GEMM)
    rows = sampled_rows(N, 160, N + 13)
    assert_linear_close(host(y)[:, rows], oracle.linear_ref_w8(lay["x"], qw[rows], sc[rows], zr[rows], G))


@pytest.mark.parametrize("M,N,K,G", [
    (1536, 11008, 4096, 128),   # 516 tiles: 512 whole, the last 4 split over every slot
    (2048, 8320, 1024, 128),    # 520 tiles, a tail of 8
    (2000, 8300, 2048, 64),     # the same with ragged rows and columns
    (1792, 11008, 4096, 128),   # 602 tiles, a tail of 90
])
def test_hybrid_tail_sampled(M, N, K, G):
    """More than one round of tiles with a short last round: the whole rounds
    run one tile per block and only the last round's tiles are split.
    Sampled output columns against the oracle (the last tiles' columns
    included), repeated calls bit-identical, and within fp32 summation order
    of the unsplit GEMM."""
    lay = synth.make_layer(N, K, M, seed=[140, M, N, K, G], w_std=0.02)
    say("hybrid tail", M, N, K, G)
    x = dev(lay["x"])
    qw, sc, zr = awq.awq_quantize(dev(lay["w"]), G)
    ws = awq.gemm_workspace(M, N, K)
    y1 = gemm_ws(x, qw, sc, zr, G, ws).clone()
    y2 = gemm_ws(x, qw, sc, zr, G, ws)
    y0 = awq.awq_gemm(x, qw, sc, zr, G, path=awq.PATH_GEMM)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    rows = np.unique(np.concatenate([sampled_rows(N, 160, M + N), np.arange(max(0, N - 300), N)]))
    eq = oracle.quantize(lay["w"][rows], G)
    assert_linear_close(host(y1)[:, rows], oracle.linear_ref(lay["x"], *eq, G))
    assert_close_per_element(y1, y0)
