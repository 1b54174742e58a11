"""CPU-side checks of the C ABI: the library loads, exports every function
include/awq.h declares, and rejects bad arguments on the host (status codes,
nothing launched). Fake device addresses are never dereferenced because every
check here fails before a kernel would be enqueued."""

import ctypes
import os
import subprocess

import numpy as np
import pytest

import weight_only_int4_quantize_amd as awq

OK, NULL, SHAPE, ALIGN, CONFIG, WORKSPACE = 0, 1, 2, 3, 4, 5
FAKE = 0x10000          # aligned fake device address (never dereferenced)
FAKE_ODD = 0x10008      # 8-byte but not 16-byte aligned


@pytest.fixture(scope="module")
def L():
    return awq.load()


def test_library_exports_every_header_function(L):
    names = awq.header_functions()
    assert {"awq_quantize", "awq_gemm", "awq_scale_search"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", awq.lib_path()], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_library_is_built_for_gfx950_only():
    """The embedded offload bundle names gfx950 and no other GPU target."""
    import re
    with open(awq.lib_path(), "rb") as f:
        blob = f.read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-[a-z-]*(gfx[0-9a-f]+)", blob))
    assert targets == {b"gfx950"}


def test_status_strings(L):
    assert L.awq_status_string(OK) == b"AWQ_OK"
    for s in range(1, 7):
        assert L.awq_status_string(s).startswith(b"AWQ_ERR_")
    assert L.awq_status_string(99) == b"unknown awq_status"
    assert L.awq_version() == 100


@pytest.mark.parametrize("N,K,G,expect", [
    (16, 128, 16, CONFIG),      # unsupported group sizes (32 .. 512, powers of two, are supported)
    (16, 1024, 1024, CONFIG),
    (16, 96, 48, CONFIG),
    (16, 100, 64, SHAPE),       # K not a multiple of G
    (16, 0, 64, SHAPE),         # empty K
    (-1, 128, 64, SHAPE),
    (0, 128, 64, OK),           # empty N: nothing to do
])
def test_quantize_shape_checks(L, N, K, G, expect):
    assert L.awq_quantize(FAKE, None, N, K, G, FAKE, FAKE, FAKE, None) == expect


def test_quantize_ex_checks(L):
    q = L.awq_quantize_ex
    assert q(FAKE, None, 16, 128, 64, 2, 0.0, FAKE, FAKE, FAKE, None) == CONFIG     # unknown mode
    assert q(FAKE, None, 16, 128, 64, -1, 0.0, FAKE, FAKE, FAKE, None) == CONFIG
    assert q(FAKE, None, 16, 128, 64, 0, 0.25, FAKE, FAKE, FAKE, None) == CONFIG    # clip in [0, 0.25)
    assert q(FAKE, None, 16, 128, 64, 0, -0.01, FAKE, FAKE, FAKE, None) == CONFIG
    assert q(FAKE, None, 16, 128, 64, 1, float("nan"), FAKE, FAKE, FAKE, None) == CONFIG
    assert q(FAKE, None, 16, 128, 16, 1, 0.0, FAKE, FAKE, FAKE, None) == CONFIG     # group size
    assert q(FAKE, None, 16, 100, 64, 1, 0.01, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, None, 0, 128, 64, 1, 0.01, FAKE, FAKE, FAKE, None) == OK         # empty N
    assert q(None, None, 16, 128, 64, 1, 0.0, FAKE, FAKE, FAKE, None) == NULL
    assert q(FAKE_ODD, None, 16, 128, 64, 1, 0.0, FAKE, FAKE, FAKE, None) == ALIGN


def test_clip_search_checks(L):
    fr = np.array([0.0, 0.01], dtype=np.float64)
    f = fr.ctypes.data_as(ctypes.c_void_p)
    losses = np.zeros(2)
    lp = losses.ctypes.data_as(ctypes.c_void_p)
    best = ctypes.c_int(-1)
    bp = ctypes.addressof(best)
    need = L.awq_clip_search_workspace_bytes(256, 512, 1024, 128, 2, 0)
    need_s = L.awq_clip_search_workspace_bytes(256, 512, 1024, 128, 2, 1)
    assert need >= 1024 * 256 * 4 + 256 * 512 // 2 and need_s >= need + 1024 * 512 * 2
    assert L.awq_clip_search_workspace_bytes(256, 500, 1024, 128, 2, 0) == 0
    c = L.awq_clip_search
    assert c(FAKE, FAKE, None, 256, 512, 1024, 128, 0, f, 2, FAKE, need - 256, lp, bp, None) == WORKSPACE
    assert c(FAKE, FAKE, FAKE, 256, 512, 1024, 128, 0, f, 2, FAKE, need, lp, bp, None) == WORKSPACE  # scaled needs x/s
    assert c(FAKE, FAKE, None, 256, 512, 1024, 128, 3, f, 2, FAKE, need, lp, bp, None) == CONFIG
    assert c(FAKE, FAKE, None, 256, 512, 1024, 128, 0, f, 0, FAKE, need, lp, bp, None) == CONFIG
    bad = np.array([0.0, 0.3])
    assert c(FAKE, FAKE, None, 256, 512, 1024, 128, 0, bad.ctypes.data_as(ctypes.c_void_p), 2, FAKE, need, lp, bp,
             None) == CONFIG
    assert c(FAKE, FAKE, None, 256, 512, 0, 128, 0, f, 2, FAKE, need, lp, bp, None) == SHAPE
    assert c(FAKE, None, None, 256, 512, 1024, 128, 0, f, 2, FAKE, need, lp, bp, None) == NULL
    assert c(FAKE, FAKE, FAKE_ODD, 256, 512, 1024, 128, 0, f, 2, FAKE, need_s, lp, bp, None) == ALIGN


def test_quantize_null_and_alignment(L):
    assert L.awq_quantize(None, None, 4, 128, 128, FAKE, FAKE, FAKE, None) == NULL
    assert L.awq_quantize(FAKE, None, 4, 128, 128, None, FAKE, FAKE, None) == NULL
    assert L.awq_quantize(FAKE_ODD, None, 4, 128, 128, FAKE, FAKE, FAKE, None) == ALIGN
    assert L.awq_quantize(FAKE, FAKE_ODD, 4, 128, 128, FAKE, FAKE, FAKE, None) == ALIGN
    assert L.awq_quantize(FAKE, None, 4, 128, 128, FAKE, FAKE + 1, FAKE, None) == ALIGN


def test_gemm_checks(L):
    g = L.awq_gemm_path
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 16, 100, 64, FAKE, 0, None) == SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, -1, 16, 128, 64, FAKE, 0, None) == SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 16, 128, 96, FAKE, 0, None) == CONFIG
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 16, 128, 64, FAKE, 5, None) == CONFIG
    assert g(FAKE, FAKE, FAKE, FAKE, 33, 16, 128, 64, FAKE, 4, None) == CONFIG  # column tiles: M <= 32
    assert g(FAKE, FAKE, FAKE, FAKE, 16, 16, 512, 512, FAKE, 4, None) == CONFIG  # and G <= 256
    assert g(FAKE, FAKE, FAKE, FAKE, 65, 16, 128, 64, FAKE, 3, None) == CONFIG  # skinny is M <= 64
    assert g(FAKE, FAKE, FAKE, FAKE, 16, 16, 512, 512, FAKE, 3, None) == CONFIG  # and G <= 256
    assert g(FAKE, FAKE, FAKE, FAKE, 9, 16, 128, 64, FAKE, 1, None) == CONFIG   # GEMV is M <= 8
    assert g(FAKE, FAKE, FAKE, FAKE, 0, 16, 128, 64, FAKE, 0, None) == OK       # empty M
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 0, 128, 64, FAKE, 0, None) == OK        # empty N
    assert g(None, FAKE, FAKE, FAKE, 1, 16, 128, 64, FAKE, 0, None) == NULL
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 16, 128, 64, None, 0, None) == NULL
    assert g(FAKE_ODD, FAKE, FAKE, FAKE, 1, 16, 128, 64, FAKE, 0, None) == ALIGN
    assert g(FAKE, FAKE_ODD, FAKE, FAKE, 1, 16, 128, 64, FAKE, 0, None) == ALIGN
    assert L.awq_gemm(FAKE, FAKE, FAKE, FAKE, 1, 16, 128, 64, FAKE + 1, None) == ALIGN


def test_gemm_ex_workspace_checks(L):
    need = L.awq_gemm_workspace_bytes(2048, 4096, 4096)
    # two fp32 256x128 partial tiles per resident block, one counter per tile
    assert need >= 2 * 256 * 128 * 4 + (2048 // 256) * (4096 // 128) * 4
    assert L.awq_gemm_workspace_bytes(0, 4096, 4096) == 0
    assert L.awq_gemm_workspace_bytes(2048, 4096, -1) == 0
    assert L.awq_gemm_workspace_bytes(4096, 4096, 4096) >= need
    # skinny K splits: 16 rows x 128 columns of fp32 per split and column tile
    assert L.awq_gemm_workspace_bytes(16, 4096, 4096) >= 32 * 16 * 16 * 128 * 4
    g = L.awq_gemm_ex
    ws = 0x100000                                                      # 256-byte aligned fake address
    assert g(FAKE, FAKE, FAKE, FAKE, 2048, 4096, 4096, 128, FAKE, 2, ws, need - 1, None) == WORKSPACE
    assert g(FAKE, FAKE, FAKE, FAKE, 2048, 4096, 4096, 128, FAKE, 2, ws + 16, need, None) == ALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, 2048, 4096, 100, 128, FAKE, 2, ws, need, None) == SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, 2048, 4096, 4096, 96, FAKE, 2, ws, need, None) == CONFIG
    assert g(None, FAKE, FAKE, FAKE, 2048, 4096, 4096, 128, FAKE, 2, ws, need, None) == NULL
    assert g(FAKE, FAKE, FAKE, FAKE, 0, 4096, 4096, 128, FAKE, 2, ws, 0, None) == OK   # empty: no work


def test_absmean_checks(L):
    need = L.awq_activation_absmean_workspace_bytes(1000, 512)
    assert need >= 512 * 8
    assert L.awq_activation_absmean_workspace_bytes(0, 512) == 0
    assert L.awq_activation_absmean(FAKE, 1000, 512, FAKE, FAKE, need - 8, None) == WORKSPACE
    assert L.awq_activation_absmean(FAKE, 0, 512, FAKE, FAKE, need, None) == SHAPE
    assert L.awq_activation_absmean(FAKE, 10, 12, FAKE, FAKE, need, None) == SHAPE
    assert L.awq_activation_absmean(None, 10, 512, FAKE, FAKE, need, None) == NULL


def test_scale_search_checks(L):
    alphas = np.arange(20, dtype=np.float64) / 20
    a = alphas.ctypes.data_as(ctypes.c_void_p)
    losses = np.zeros(20)
    lp = losses.ctypes.data_as(ctypes.c_void_p)
    best = ctypes.c_int(-1)
    bp = ctypes.addressof(best)
    need = L.awq_scale_search_workspace_bytes(256, 512, 1024, 128, 20)
    # the layout holds at least Y (T x N fp32), x / s (T x K fp16) and the packed weight
    assert need >= 1024 * 256 * 4 + 1024 * 512 * 2 + 256 * 512 // 2
    assert L.awq_scale_search_workspace_bytes(256, 500, 1024, 128, 20) == 0
    s = L.awq_scale_search
    assert s(FAKE, FAKE, 256, 512, 1024, 128, a, 20, FAKE, need - 256, lp, bp, FAKE, None) == WORKSPACE
    assert s(FAKE, FAKE, 256, 512, 1024, 128, a, 0, FAKE, need, lp, bp, FAKE, None) == CONFIG
    assert s(FAKE, FAKE, 256, 512, 1024, 100, a, 20, FAKE, need, lp, bp, FAKE, None) == CONFIG
    assert s(FAKE, FAKE, 0, 512, 1024, 128, a, 20, FAKE, need, lp, bp, FAKE, None) == SHAPE
    assert s(FAKE, FAKE, 256, 512, 0, 128, a, 20, FAKE, need, lp, bp, FAKE, None) == SHAPE
    assert s(FAKE, None, 256, 512, 1024, 128, a, 20, FAKE, need, lp, bp, FAKE, None) == NULL
    # no grid (alphas NULL) is accepted: the call then fails only on the short workspace
    assert s(FAKE, FAKE, 256, 512, 1024, 128, None, 20, FAKE, need - 256, lp, bp, FAKE, None) == WORKSPACE
    assert s(FAKE, FAKE, 256, 512, 1024, 128, None, 0, FAKE, need, lp, bp, FAKE, None) == CONFIG
    bad = np.array([0.0, np.nan])
    assert s(FAKE, FAKE, 256, 512, 1024, 128, bad.ctypes.data_as(ctypes.c_void_p), 2, FAKE, need, lp, bp,
             FAKE, None) == CONFIG
    assert s(FAKE_ODD, FAKE, 256, 512, 1024, 128, a, 20, FAKE, need, lp, bp, FAKE, None) == ALIGN


def test_kernel_choice(L):
    """awq_gemm_kernel names the kernel each path takes, and refuses what a
    path cannot run (host logic only)."""
    k = L.awq_gemm_kernel
    k.restype = ctypes.c_int
    k.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_int] * 3
    assert k(1, 4096, 4096, 128, 0, 0) == 1            # decode: the GEMV
    assert k(4, 4096, 11008, 128, 0, 0) == 4           # column tiles
    assert k(4, 512, 11008, 128, 0, 0) == 1            # few long rows at 4 rows of x: the GEMV one-shot
    assert k(3, 1000, 8192, 64, 0, 1) == 1
    assert k(4, 2049, 5120, 128, 0, 0) == 4            # past one round of resident waves: column tiles
    assert k(4, 512, 4096, 128, 0, 0) == 4             # rows of one item: column tiles
    assert k(5, 512, 11008, 128, 0, 0) == 4            # 5 rows of x: column tiles
    assert k(16, 4096, 4096, 128, 0, 1) == 4
    assert k(16, 8192, 28672, 128, 0, 1) == 3          # large layer: the skinny kernel
    assert k(16, 8192, 28672, 128, 0, 0) == 4          # ... which without a workspace walks K in phases
    assert k(16, 5120, 13824, 128, 0, 1) == 3
    assert k(16, 13824, 5120, 128, 0, 1) == 4
    assert k(32, 11008, 4096, 128, 0, 1) == 4
    assert k(2048, 11008, 4096, 128, 0, 1) == 2        # prefill: the GEMM
    assert k(9, 64, 128, 64, 1, 0) == -1               # GEMV is M <= 8
    assert k(33, 64, 128, 64, 4, 0) == -1              # column tiles are M <= 32
    assert k(16, 64, 512, 512, 4, 0) == -1             # and G <= 256
    assert k(4, 64, 100, 64, 0, 0) == -1               # K % G
    assert k(0, 64, 128, 64, 0, 0) == -1


def test_salient_count_is_the_oracles(L):
    """The library's default salient-channel count (round(K / 100), ties to
    even) equals the oracle's for every width of the workloads and at ties."""
    import oracle
    L.awq_salient_count.restype = ctypes.c_int64
    L.awq_salient_count.argtypes = [ctypes.c_int64]
    for K in (1, 50, 150, 250, 512, 4096, 5120, 11008, 13824, 28672):
        assert L.awq_salient_count(K) == oracle.salient_count(K), K
    assert L.awq_salient_count(0) == 0
    assert L.awq_salient_count(4096) == 41


def test_binding_refuses_cpu_tensors():
    import torch
    w = torch.zeros(4, 128, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensor"):
        awq.awq_quantize(w, 128)


def test_oracle_is_not_reachable_from_the_package():
    """The product package never imports or reads the oracle."""
    pkg = os.path.dirname(awq.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                with open(os.path.join(root, f), encoding="utf-8") as fh:
                    text = fh.read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_salient_checks(L):
    """Argument checks of the mixed-precision entry points (no launch)."""
    sel = L.awq_select_salient
    assert sel(FAKE, 0, 1, FAKE, None) == SHAPE
    assert sel(FAKE, (1 << 17) + 8, 1, FAKE, None) == SHAPE          # K^2 selection is bounded
    assert sel(FAKE, 64, 65, FAKE, None) == SHAPE
    assert sel(FAKE, 64, -1, FAKE, None) == SHAPE
    assert sel(None, 64, 4, FAKE, None) == NULL
    assert sel(FAKE + 4, 64, 4, FAKE, None) == ALIGN
    assert sel(None, 64, 0, None, None) == OK                         # nothing to select
    q = L.awq_quantize_salient
    assert q(FAKE, 16, 256, 64, 2, FAKE, 4, FAKE, FAKE, FAKE, FAKE, None) == CONFIG   # mode
    assert q(FAKE, 16, 256, 48, 0, FAKE, 4, FAKE, FAKE, FAKE, FAKE, None) == CONFIG   # group size
    assert q(FAKE, 16, 256, 64, 0, FAKE, 257, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, 16, 256, 64, 0, None, 4, FAKE, FAKE, FAKE, FAKE, None) == NULL
    assert q(FAKE, 16, 256, 64, 0, FAKE, 4, FAKE, FAKE, FAKE, None, None) == NULL
    assert q(FAKE_ODD, 16, 256, 64, 0, FAKE, 4, FAKE, FAKE, FAKE, FAKE, None) == ALIGN
    assert q(FAKE, 0, 256, 64, 0, FAKE, 4, FAKE, FAKE, FAKE, FAKE, None) == OK        # empty N
    a = L.awq_salient_apply
    assert a(FAKE, FAKE, FAKE, 4, 16, 64, 65, FAKE, None) == SHAPE
    assert a(FAKE, FAKE, FAKE, -1, 16, 64, 4, FAKE, None) == SHAPE
    assert a(FAKE, None, FAKE, 4, 16, 64, 4, FAKE, None) == NULL
    assert a(FAKE + 1, FAKE, FAKE, 4, 16, 64, 4, FAKE, None) == ALIGN
    assert a(None, None, None, 0, 16, 64, 4, None, None) == OK                       # empty M
    assert a(None, None, None, 4, 16, 64, 0, None, None) == OK                       # no salient channel
    need = L.awq_salient_loss_workspace_bytes(256, 512, 1024, 128, 5)
    assert need >= 1024 * 256 * 4 + 256 * 512 // 2 + 5 * 256 * 2
    assert L.awq_salient_loss_workspace_bytes(256, 512, 1024, 128, 513) == 0
    lr, ls = ctypes.c_double(), ctypes.c_double()
    pr, ps = ctypes.addressof(lr), ctypes.addressof(ls)
    s = L.awq_salient_loss
    assert s(FAKE, FAKE, 256, 512, 1024, 128, 0, 5, FAKE, need - 256, pr, ps, None, None) == WORKSPACE
    assert s(FAKE, FAKE, 256, 512, 1024, 128, 2, 5, FAKE, need, pr, ps, None, None) == CONFIG
    assert s(FAKE, FAKE, 256, 1 << 18, 1024, 128, 0, 5, FAKE, need, pr, ps, None, None) == SHAPE
    assert s(FAKE, FAKE, 256, 512, 1024, 128, 0, 513, FAKE, need, pr, ps, None, None) == SHAPE
    assert s(FAKE, None, 256, 512, 1024, 128, 0, 5, FAKE, need, pr, ps, None, None) == NULL
    assert s(FAKE, FAKE, 256, 512, 1024, 128, 0, 5, FAKE, need, None, ps, None, None) == NULL
    assert s(FAKE, FAKE_ODD, 256, 512, 1024, 128, 0, 5, FAKE, need, pr, ps, None, None) == ALIGN


def test_w8_checks(L):
    q = L.awq_quantize_w8
    assert q(FAKE, None, 16, 256, 32, 0, FAKE, FAKE, FAKE, None) == CONFIG      # W8 takes G >= 64
    assert q(FAKE, None, 16, 256, 64, 2, FAKE, FAKE, FAKE, None) == CONFIG      # mode
    assert q(FAKE, None, 16, 200, 64, 0, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(None, None, 16, 256, 64, 0, FAKE, FAKE, FAKE, None) == NULL
    assert q(FAKE, FAKE_ODD, 16, 256, 64, 0, FAKE, FAKE, FAKE, None) == ALIGN
    assert q(FAKE, None, 0, 256, 64, 0, FAKE, FAKE, FAKE, None) == OK           # empty N
    g = L.awq_gemm_w8
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 16, 256, 32, FAKE, 0, None, 0, None) == CONFIG
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 16, 256, 64, FAKE, 3, None, 0, None) == CONFIG   # no skinny path
    assert g(FAKE, FAKE, FAKE, FAKE, 9, 16, 256, 64, FAKE, 1, None, 0, None) == CONFIG   # GEMV is M <= 8
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 16, 1 << 22, 64, FAKE, 2, None, 0, None) == CONFIG
    assert g(FAKE, FAKE, FAKE, FAKE, -1, 16, 256, 64, FAKE, 0, None, 0, None) == SHAPE
    assert g(FAKE, None, FAKE, FAKE, 4, 16, 256, 64, FAKE, 0, None, 0, None) == NULL
    assert g(FAKE_ODD, FAKE, FAKE, FAKE, 4, 16, 256, 64, FAKE, 0, None, 0, None) == ALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, 100, 16, 256, 64, FAKE, 2, FAKE, 16, None) == WORKSPACE
    assert g(FAKE, FAKE, FAKE, FAKE, 0, 16, 256, 64, FAKE, 0, None, 0, None) == OK


def test_grouped_rejects_bad_arguments(L):
    """awq_gemm_grouped's host checks, before any launch (host logic only)."""
    import ctypes as C
    g = L.awq_gemm_grouped
    g.restype = C.c_int
    g.argtypes = [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
                  C.c_int, C.c_void_p, C.c_void_p]
    P = C.c_void_p * 4
    ptrs = P(None, None, None, None)
    ns = (C.c_int64 * 4)(64, 64, 64, 64)
    assert g(None, 0, ptrs, ptrs, ptrs, ns, 1, 128, 64, ptrs, None) == 4      # n_layers < 1
    assert g(None, 5, ptrs, ptrs, ptrs, ns, 1, 128, 64, ptrs, None) == 4      # n_layers > 4
    assert g(None, 2, None, ptrs, ptrs, ns, 1, 128, 64, ptrs, None) == 1      # NULL array
    assert g(None, 2, ptrs, ptrs, ptrs, ns, 1, 100, 64, ptrs, None) == 2      # K % G
    assert g(None, 2, ptrs, ptrs, ptrs, ns, 1, 128, 96, ptrs, None) == 4      # group size
    assert g(None, 2, ptrs, ptrs, ptrs, ns, 1, 128, 64, ptrs, None) == 1      # NULL device pointers
    assert g(None, 2, ptrs, ptrs, ptrs, ns, 0, 128, 64, ptrs, None) == 0      # M = 0: no work
    big = (C.c_int64 * 4)(1 << 30, 1 << 30, 0, 0)
    assert g(None, 2, ptrs, ptrs, ptrs, big, 0, 128, 64, ptrs, None) == 2     # stacked rows past 2^31
