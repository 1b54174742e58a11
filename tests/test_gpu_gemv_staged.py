"""The streaming GEMV with each block's (scale, zero) pairs staged in LDS.

On long rows (past the one-shot and few-row forms: three or more 2 KB items
per row, or two on layers of over 4096 rows) a single-layer GEMV launch stages the pairs of its block's rows once
as packed words, where (N K / G) is a multiple of 8 and the copy fits in LDS
beside x; other launches load each chunk's pair with the chunk. Both forms
compute the dequantization map of the xxmr.cn quantization article (§1.2)
inside y = x dequant(Wq)^T; outputs are held to the linear bar against the
oracle: relative Frobenius error <= 1e-3 and |y - y_ref| <= 1e-2 (|y_ref| + 1)
per element. The shapes cover both forms, ragged row counts, the pieces
loaded ahead of the weights and those loaded after them, both code widths.
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import assert_linear_close, dev, host, say  # noqa: E402


def run_gemv(x, q, G, bits):
    qw, sc, zr = q
    if bits == 4:
        y = awq.awq_gemm(dev(x), dev(qw.view(np.int32)), dev(sc), dev(zr), G, path=awq.PATH_GEMV)
    else:
        y = awq.awq_gemm_w8(dev(x), dev(qw.view(np.int32)), dev(sc), dev(zr), G, path=awq.PATH_GEMV)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("M,N,K,G,bits", [
    (2, 4004, 11008, 128, 4),     # two rows per wave, ragged last block
    (2, 4001, 11008, 128, 4),     # N K / G not a multiple of 8: pairs loaded per chunk
    (1, 4004, 11008, 128, 4),     # 3 items per row at M = 1: pairs loaded per chunk
    (2, 3000, 12288, 128, 4),
    (1, 8192, 28672, 64, 4),      # 448 groups per row: 3.5 pieces per thread ahead of the weights
    (2, 3000, 28672, 128, 4),
    (1, 6000, 20480, 32, 4),      # 640 groups per row: pieces past the first four per thread
    (1, 4096, 11008, 128, 8),     # W8 rows of 6 items
    (2, 777, 8192, 64, 8),
])
def test_gemv_streaming_pairs(M, N, K, G, bits):
    lay = synth.make_layer(N, K, M, seed=[230, N, K, G, bits], w_std=0.02)
    say("streaming gemv", M, N, K, G, "w%d" % bits)
    if bits == 4:
        q = oracle.quantize(lay["w"], G)
        ref = oracle.linear_ref(lay["x"], *q, G)
    else:
        q = oracle.quantize_w8(lay["w"], G)
        ref = oracle.linear_ref_w8(lay["x"], *q, G)
    assert_linear_close(run_gemv(lay["x"], q, G, bits), ref)


def test_gemv_streaming_pairs_do_not_leak_between_calls():
    """A block's staged pairs are its own rows' only: two layers of the same
    shape with different scales, called back to back, each match the oracle."""
    M, N, K, G = 2, 4096, 11008, 128
    for seed in (231, 232):
        lay = synth.make_layer(N, K, M, seed=[seed], w_std=0.02 if seed == 231 else 0.2)
        q = oracle.quantize(lay["w"], G)
        assert_linear_close(run_gemv(lay["x"], q, G, 4), oracle.linear_ref(lay["x"], *q, G))
