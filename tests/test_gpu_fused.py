"""Fused projections of a decoder layer (the rskf.cn AWQ article, §3.4: a
quantized model loaded with its layers fused): q/k/v share their input and
run as one W[12288, 4096] product, gate/up as one W[22016, 4096] product.

Rows are output channels and groups run along K, so quantizing the
row-concatenated weight equals concatenating the quantized parts, bit for
bit; the fused product's outputs are then checked element by element against
the oracle (relative Frobenius error <= 1e-3 and |y - y_ref| <= 1e-2 *
(|y_ref| + 1)) at the decode batch sizes M = 1, 4 and 16, with and without a
workspace.
"""

import functools

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import assert_linear_close, assert_quant_equal, dev, host, say  # noqa: E402

G = 128
# (fused name, [(part, N)], K)
FUSED = {
    "qkv_proj": ([("q_proj", 4096), ("k_proj", 4096), ("v_proj", 4096)], 4096),
    "gate_up_proj": ([("gate_proj", 11008), ("up_proj", 11008)], 4096),
}


@functools.lru_cache(maxsize=None)
def fused_layer(name):
    """Each projection drawn with its own seed, then concatenated along N;
    the oracle quantizes each part on its own."""
    parts, K = FUSED[name]
    layers = [synth.make_layer(N, K, 0, seed=[6, j, N, K], w_std=0.02) for j, (_, N) in enumerate(parts)]
    w = np.concatenate([lay["w"] for lay in layers], axis=0)
    q_parts = [oracle.quantize(lay["w"], G) for lay in layers]
    eq = tuple(np.concatenate([q[i] for q in q_parts], axis=0) for i in range(3))
    return w, eq, layers[0]["salient"]


@pytest.mark.parametrize("name", sorted(FUSED))
def test_fused_quantize_is_concatenation_of_parts(name):
    w, eq, _ = fused_layer(name)
    say("fused quantize", name, w.shape)
    qw, sc, zr = awq.awq_quantize(dev(w), G)
    torch.cuda.synchronize()
    got = (host(qw).view(np.uint32), host(sc), host(zr))
    assert_quant_equal(got, eq)
    assert_quant_equal(got, oracle.quantize(w, G))


@pytest.mark.parametrize("workspace", [False, True])
@pytest.mark.parametrize("M", synth.DECODE_M)
@pytest.mark.parametrize("name", sorted(FUSED))
def test_fused_linear_every_output(name, M, workspace):
    w, eq, salient = fused_layer(name)
    N, K = w.shape
    x = synth.random_x(M, K, [7, N, K, M], salient)
    say("fused linear", name, M, N, K, "workspace" if workspace else "no workspace")
    ws = awq.gemm_workspace(M, N, K) if workspace else None
    y = awq.awq_gemm(dev(x), dev(eq[0].view(np.int32)), dev(eq[1]), dev(eq[2]), G, workspace=ws)
    torch.cuda.synchronize()
    assert_linear_close(host(y), oracle.linear_ref(x, *eq, G))
