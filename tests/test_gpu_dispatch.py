"""The automatic kernel choice of awq_gemm: for batch sizes across every
regime (the GEMV, column tiles, the skinny kernel, the GEMM) and with and
without a workspace, the automatic call gives the same bits as the kernel
awq_gemm_kernel names, run by its explicit path, and meets the linear-layer
bar against the oracle (relative Frobenius error <= 1e-3 and |y - y_ref| <=
1e-2 * (|y_ref| + 1) per element)."""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import assert_linear_close, dev, host, say  # noqa: E402

PATH_OF = {"gemv": awq.PATH_GEMV, "gemm": awq.PATH_GEMM, "skinny": awq.PATH_SKINNY, "coltile": awq.PATH_COLTILE}
G = 128


@pytest.mark.parametrize("N,K", [(4096, 4096), (1000, 3072), (5120, 13824)])
@pytest.mark.parametrize("workspace", [False, True])
def test_automatic_choice_matches_named_kernel(N, K, workspace):
    lay = synth.make_layer(N, K, 80, seed=[240, N, K], w_std=0.02)
    qw, sc, zr = oracle.quantize(lay["w"], G)
    q, s, z = dev(qw.view(np.int32)), dev(sc), dev(zr)
    seen = set()
    for M in (1, 2, 3, 4, 5, 8, 9, 16, 17, 32, 33, 64, 80):
        x = lay["x"][:M]
        ws = awq.gemm_workspace(M, N, K) if workspace else None
        kern = awq.gemm_kernel(M, N, K, G, workspace=workspace)
        seen.add(kern)
        say("dispatch", M, N, K, "workspace" if workspace else "", kern)
        xd = dev(x)
        y_auto = awq.awq_gemm(xd, q, s, z, G, workspace=ws)
        y_named = awq.awq_gemm(xd, q, s, z, G, path=PATH_OF[kern], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_auto, y_named), (M, kern)
        if M in (1, 3, 9, 33, 80):
            assert_linear_close(host(y_auto), oracle.linear_ref(x, qw, sc, zr, G))
    assert len(seen) >= 3, seen
