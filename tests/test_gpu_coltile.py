"""Parity of the column-tile MFMA kernel (path 4: one block per 16, 32 or 64
output columns over all of K, for 2 <= M <= 32) with the CPU oracle: relative
Frobenius error <= 1e-3 and |y - y_ref| <= 1e-2 * (|y_ref| + 1) per element,
on the decode shapes, ragged shapes (N not a multiple of 16, rows past M,
few groups per wave, every group size it takes, blocks of several tiles
whose last tiles lie partly or wholly past N) and a one-hot input, which
reproduces the dequantized column exactly (one nonzero product per
column, one scale multiply, one fp16 rounding)."""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import assert_linear_close, dev, host, say  # noqa: E402


def coltile(x16, qw, sc, zr, G):
    y = awq.awq_gemm(dev(x16), dev(qw.view(np.int32)), dev(sc), dev(zr), G, path=awq.PATH_COLTILE)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("M", [2, 4, 8, 16])
@pytest.mark.parametrize("N,K", synth.DECODE_SHAPES)
def test_decode_shapes_against_oracle(N, K, M):
    lay = synth.decode_layer(N, K, M)
    say("column tiles", M, N, K)
    qw, sc, zr = oracle.quantize(lay["w"], 128)
    assert_linear_close(coltile(lay["x"], qw, sc, zr, 128), oracle.linear_ref(lay["x"], qw, sc, zr, 128))


@pytest.mark.parametrize("M,N,K,G", [
    (2, 1, 128, 128),         # one column, one group: seven of the eight waves idle
    (3, 17, 256, 64),         # a ragged second tile
    (5, 100, 1024, 32),       # 32 groups of 32
    (7, 250, 2560, 256),      # ten groups of 256
    (16, 1000, 6144, 128),
    (17, 333, 1536, 64),      # two row blocks, rows past M in the second
    (32, 4111, 4096, 128),
    (9, 77, 28672, 128),      # long K: 28 groups per wave
    # several 16-column tiles per block (each x operand read feeds them all)
    (16, 11000, 4096, 128),   # three tiles per block; the last block holds one tile, 8 columns wide
    (16, 6000, 4096, 128),    # two tiles per block; the last block's second tile past N
    (8, 13800, 5120, 128),    # two tiles at 8 rows (rows of 40 groups)
    (32, 10250, 4096, 128),   # three tiles, 32 rows; the last block's second tile 10 columns wide
    (16, 11000, 4096, 256),   # three tiles at G = 256 (two groups in flight)
    (32, 11000, 4096, 256),   # 32 rows at G = 256: two tiles
    (16, 13800, 2048, 128),   # four tiles (one round of blocks); the last block's third tile 8 wide
    (32, 14000, 1024, 64),    # four tiles at 32 rows
    (32, 9000, 2048, 64),     # three tiles, G = 64, a ragged last tile
    (24, 20000, 512, 32),     # three tiles over two rounds of blocks, G = 32
])
def test_ragged_against_oracle(M, N, K, G):
    lay = synth.make_layer(N, K, M, seed=[220, M, N, K, G], w_std=0.02)
    say("column tiles ragged", M, N, K, G)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    assert_linear_close(coltile(lay["x"], qw, sc, zr, G), oracle.linear_ref(lay["x"], qw, sc, zr, G))


@pytest.mark.parametrize("symmetric", [False, True])
def test_symmetric_map(symmetric):
    M, N, K, G = 6, 300, 2048, 128
    lay = synth.make_layer(N, K, M, seed=[221, int(symmetric)], w_std=0.02)
    qw, sc, zr = (oracle.quantize_symmetric if symmetric else oracle.quantize)(lay["w"], G)
    assert_linear_close(coltile(lay["x"], qw, sc, zr, G), oracle.linear_ref(lay["x"], qw, sc, zr, G))


def test_one_hot_rows_return_dequantized_columns():
    N, K, G = 40, 512, 64
    lay = synth.make_layer(N, K, 0, seed=[222], w_std=0.02)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    w_hat = oracle.dequantize(qw, sc, zr, G, K)
    ks = [0, 7, 63, 64, 200, 301, 511]
    x = np.zeros((len(ks), K), dtype=np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = coltile(x, qw, sc, zr, G)
    assert np.array_equal(y, w_hat[:, ks].T.astype(np.float16))


@pytest.mark.parametrize("M,N,K,G", [(13, 45, 1024, 128), (16, 10250, 4096, 128)])
def test_guard_band_and_repeatability(M, N, K, G):
    lay = synth.make_layer(N, K, M, seed=[223, M, N], w_std=0.02)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    buf = torch.full((M * N + 2048,), 7.0, dtype=torch.float16, device="cuda")
    y = buf[1024:1024 + M * N].view(M, N)
    args = (dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr), G)
    awq.awq_gemm(*args, path=awq.PATH_COLTILE, out=y)
    y2 = awq.awq_gemm(*args, path=awq.PATH_COLTILE)
    torch.cuda.synchronize()
    b = host(buf)
    assert np.all(b[:1024] == 7.0) and np.all(b[1024 + M * N:] == 7.0)
    assert torch.equal(y, y2)
    assert_linear_close(host(y), oracle.linear_ref(lay["x"], qw, sc, zr, G))
