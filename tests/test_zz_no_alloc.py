"""awq_gemm_noalloc (the entry point that allocates nothing, its split
scratch held by the library) against awq_gemm_ex with a caller workspace,
through the C ABI, on two calls in a row (the second with a smaller input):
the linear-layer bar (relative Frobenius error <= 1e-3 and |y - y_ref| <=
1e-2 * (|y_ref| + 1) per element) against both awq_gemm_ex and the oracle,
and the same bits as awq_gemm_ex where both run the same split plan (the
skinny kernel, the column tiles and the GEMV).
"""

import ctypes

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import assert_linear_close, dev, host, say  # noqa: E402

G = 128


def noalloc(x, qw, sc, zr, y, path=awq.PATH_AUTO):
    """One awq_gemm_noalloc call through ctypes, into a preallocated y."""
    L = awq.load()
    M, K = x.shape
    N = qw.shape[0]
    st = L.awq_gemm_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(qw.data_ptr()),
                            ctypes.c_void_p(sc.data_ptr()), ctypes.c_void_p(zr.data_ptr()), M, N, K, G,
                            ctypes.c_void_p(y.data_ptr()), path,
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == awq.AWQ_OK, awq.load().awq_status_string(st).decode()


def run_pair(M, N, K, seed):
    lay = synth.make_layer(N, K, M, seed=[210, seed, M, N, K], w_std=0.02)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    x, q, s, z = dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr)
    ws = awq.gemm_workspace(M, N, K)
    y_ex = awq.awq_gemm(x, q, s, z, G, workspace=ws)
    y_na = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    noalloc(x, q, s, z, y_na)
    torch.cuda.synchronize()
    ref = oracle.linear_ref(lay["x"], qw, sc, zr, G)
    assert_linear_close(host(y_na), ref)
    assert_linear_close(host(y_na), host(y_ex).astype(np.float64))
    return y_na, y_ex


@pytest.mark.parametrize("first,second", [
    ((64, 4096, 4096), (40, 2048, 4096)),       # skinny, K split: 16 then 8 column tiles
    ((16, 11008, 4096), (9, 4096, 4096)),       # column tiles: no scratch
    ((48, 5120, 13824), (33, 4096, 11008)),     # skinny, 4 row blocks, long K
    ((3, 4096, 28672), (2, 1024, 28672)),       # long K: column tiles, then the skinny kernel (M = 2)
    ((1, 11008, 4096), (1, 4096, 4096)),        # GEMV: no scratch
    ((300, 2048, 1024), (130, 700, 512)),       # MFMA GEMM, unsplit here
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for i, (M, N, K) in enumerate((first, second)):
        say("noalloc call", i, M, N, K)
        y_na, y_ex = run_pair(M, N, K, i)
        if M <= 64:
            assert torch.equal(y_na, y_ex), (M, N, K)


def test_noalloc_is_repeatable_and_rejects_bad_arguments():
    M, N, K = 16, 4096, 4096
    lay = synth.make_layer(N, K, M, seed=[211], w_std=0.02)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    x, q, s, z = dev(lay["x"]), dev(qw.view(np.int32)), dev(sc), dev(zr)
    y1 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    y2 = torch.empty_like(y1)
    noalloc(x, q, s, z, y1)
    noalloc(x, q, s, z, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    L = awq.load()
    st = L.awq_gemm_noalloc(ctypes.c_void_p(x.data_ptr()), None, None, None, M, N, K, G,
                            ctypes.c_void_p(y1.data_ptr()), 0, None)
    assert st == 1   # AWQ_ERR_NULL
    st = L.awq_gemm_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                            ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(z.data_ptr()), M, N, K, 96,
                            ctypes.c_void_p(y1.data_ptr()), 0, None)
    assert st == 4   # AWQ_ERR_CONFIG: group size 96
