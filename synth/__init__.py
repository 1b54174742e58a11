"""Seeded synthetic inputs shaped like the workloads on the AWQ pages.

Both the HIP path and the oracle are fed from here; this module holds no step
of the quantization method. The pages quantize Llama/Qwen checkpoints with
pile/c4/domain calibration text, none of which is available here, so these
Llama-shaped Gaussian tensors stand in for them. The salient-channel structure
(about 1 % of input channels carry much larger activations) follows the rskf.cn
AWQ article, §2.2, and "AWQ 模型量化技术：激活感知的权重量化革命", "显著权重识别".

Recipe:
  rng = np.random.default_rng(seed)       (PCG64)
  salient = rng.choice(K, round(frac*K), replace=False)   (drawn first)
  W = rng.standard_normal((N, K), float32) * w_std; W[:, salient] *= w_mult
  X = rng.standard_normal((M, K), float32);          X[:, salient] *= x_mult
  both cast to float16 with round-to-nearest-even.
"""

from __future__ import annotations

import numpy as np

# Llama-7B linear shapes (N, K): q/k/v/o, gate/up, down.
LLAMA7B_LAYER = (
    ("q_proj", 4096, 4096),
    ("k_proj", 4096, 4096),
    ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 11008, 4096),
    ("up_proj", 11008, 4096),
    ("down_proj", 4096, 11008),
)

# Distinct shapes of the decode sweep.
DECODE_SHAPES = ((4096, 4096), (11008, 4096), (4096, 11008))
# The same layer with its projections fused as a model loaded with fused
# layers runs them: q/k/v share x (N = 3 * 4096) and so do gate/up
# (N = 2 * 11008), so each group is one product.
LLAMA7B_LAYER_FUSED = (
    ("qkv_proj", 12288, 4096),
    ("o_proj", 4096, 4096),
    ("gate_up_proj", 22016, 4096),
    ("down_proj", 4096, 11008),
)
DECODE_M = (1, 4, 16)
# Prefill products: x[2048, K] . W[N, K]^T.
PREFILL_SHAPES = ((11008, 4096), (4096, 11008))
PREFILL_M = 2048
# 13B / 70B shapes of the larger sweep.
SWEEP_SHAPES = ((13824, 5120), (5120, 13824), (8192, 28672))
SWEEP_M = (1, 32, 512)
SWEEP_G = (64, 128)
# Scale search: one 7B MLP layer, 128 samples x 512 tokens of calibration.
SEARCH_SHAPE = (11008, 4096)
SEARCH_TOKENS = 128 * 512
SEARCH_N_ALPHA = 20


def case_seed(cfg: int, N: int, K: int, M: int, G: int):
    """Seed of one case: a list NumPy hashes into the PCG64 state."""
    return [int(cfg), int(N), int(K), int(M), int(G)]


def salient_channels(rng: np.random.Generator, K: int, frac: float = 0.01) -> np.ndarray:
    n = int(round(frac * K))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng.choice(K, n, replace=False))


def make_layer(N: int, K: int, M: int, *, seed, w_std: float = 0.02,
               salient_frac: float = 0.01, w_mult: float = 10.0,
               x_mult: float = 20.0):
    """One layer's weight W[N, K] and activations X[M, K] (float16)."""
    rng = np.random.default_rng(seed)
    idx = salient_channels(rng, K, salient_frac)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)
    if idx.size:
        w[:, idx] *= np.float32(w_mult)
    x = rng.standard_normal((M, K), dtype=np.float32) if M > 0 else np.zeros((0, K), np.float32)
    if idx.size and M > 0:
        x[:, idx] *= np.float32(x_mult)
    return {"w": w.astype(np.float16), "x": x.astype(np.float16), "salient": idx}


def tiny_layer():
    """W[512, 512] ~ N(0, 0.02), x[1, 512] ~ N(0, 1), seed 0, no salient
    channels: the small case the oracle finishes in well under a second."""
    return make_layer(512, 512, 1, seed=0, w_std=0.02, salient_frac=0.0)


def decode_layer(N: int, K: int, M: int, G: int = 128):
    return make_layer(N, K, M, seed=case_seed(2, N, K, M, G), w_std=0.02)


def prefill_layer(N: int, K: int, M: int = PREFILL_M, G: int = 128):
    return make_layer(N, K, M, seed=case_seed(3, N, K, M, G), w_std=0.02)


def sweep_layer(N: int, K: int, M: int, G: int):
    return make_layer(N, K, M, seed=case_seed(4, N, K, M, G), w_std=0.015)


def search_layer(T: int = SEARCH_TOKENS, N: int = SEARCH_SHAPE[0], K: int = SEARCH_SHAPE[1],
                 G: int = 128, w_mult: float = 1.0):
    """Calibration activations X[T, K] with 1 % salient channels x20 and one
    7B-shaped weight. The search workload states no salient structure for the
    weight, so by default W is plain N(0, 0.02) (w_mult = 1); w_mult = 10
    gives the decode workloads' weight recipe."""
    seed = case_seed(5, N, K, T, G) + ([] if w_mult == 1.0 else [int(w_mult)])
    return make_layer(N, K, T, seed=seed, w_std=0.02, w_mult=w_mult)


def random_x(M: int, K: int, seed, salient=None, x_mult: float = 20.0):
    """Extra activations for an existing layer (same salient channels)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if salient is not None and len(salient):
        x[:, salient] *= np.float32(x_mult)
    return x.astype(np.float16)
