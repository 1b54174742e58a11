"""Plain, slow CPU oracle for the AWQ W4A16 hot path.

TEST INFRASTRUCTURE. This module is imported only by the tests, by the smoke
check and by the benchmark's CPU-baseline leg. It never touches the HIP
library, and the HIP library never touches it.

Sources (the pages this follows):
  [P1] rskf.cn AWQ article (news/13914): §1.1 RTN baseline, §2.1
       "激活感知的缩放因子设计" (weights x s, activations / s, s searched to
       minimise the quantized-vs-original output difference), §2.2 salient
       channels, §2.3 / §4.1 scales folded ahead of inference.
  [P3] "模型量化实战：INT8/INT4、GPTQ、AWQ与精度-速度权衡", sections
       "量化粒度" (per-group, group_size=128) and "对称/非对称量化"
       (asymmetric: zero-point != 0).
  [P4] "AWQ 模型量化技术：激活感知的权重量化革命", "核心原理" (error =
       |Q(w) - w| x |activation|) and "Per-channel Scaling 优化".
  [P5] "模型量化:GGUF/AWQ/GPTQ部署方案", §1.2 "量化映射" (the affine map
       q = clamp(round(x/scale) + zero_point, 0, 2^bits - 1), its inverse
       x_hat = (q - zero_point) * scale, scale set by the weight range, and the
       worked example: range [-1, 1] -> scale 2/15), §1.4 "量化粒度"
       (128 weights per group).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * scale = (wmax - wmin) / 15 over the group's own [min, max], computed as an
    fp32 subtraction and an IEEE fp32 division; a range below 1e-5 is raised
    to 1e-5 so a constant group still has a non-zero scale.
  * the scale is stored as fp16 (round-to-nearest-even) and the codes are made
    with that stored fp16 value, so dequantization uses exactly the scale the
    codes were made with.
  * zero_point = clamp(rint(-wmin / scale), 0, 15), stored as an integer-valued
    fp16.
  * "round" is round-half-to-even (np.rint); rounding happens before the
    zero-point is added, as the formula on [P5 §1.2] is written.
  * packing: eight codes along K per uint32, code k = 8c + j in bits 4j..4j+3.
  * scale search: s = mean|x|^alpha per input channel, alpha_i = i / n_alpha;
    ties between alphas go to the smallest alpha.

Floating point: the quantizer's steps are taken in float32 exactly as the
reading states them (NumPy float32 division and subtraction are IEEE
correctly rounded, np.rint is half-to-even, astype(float16) is
round-to-nearest-even). Every matrix product is float64.
"""

from __future__ import annotations

import numpy as np

QMAX = 15                       # 2^bits - 1 for bits = 4   [P5 §1.2]
RANGE_FLOOR = np.float32(1e-5)  # degenerate-group guard (reading)
MEAN_FLOOR = 1e-8               # zero-activation-channel guard (reading)


def _check_groups(K: int, group_size: int) -> None:
    if group_size <= 0 or K % group_size != 0:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")


def group_quantize(w, group_size: int, channel_scale=None):
    """Group-wise asymmetric INT4 quantization of a weight matrix.

    Follows the affine map of [P5 §1.2] with per-group granularity of
    [P5 §1.4] / [P3 "量化粒度"] and a non-zero zero-point of
    [P3 "对称/非对称量化"].

    w:             [N, K] array (float16 weights; row n = output channel,
                   column k = input channel). Groups run along K.
    group_size:    G, the number of consecutive k sharing a scale/zero.
    channel_scale: optional float32 [K]; when given, the weights quantized are
                   float32(w[n, k] * channel_scale[k]) (AWQ's W * diag(s),
                   [P1 §2.1]), one IEEE float32 product per element.

    Returns (codes uint8 [N, K] in 0..15, scales float16 [N, K/G],
    zeros float16 [N, K/G]).
    """
    w32 = np.asarray(w).astype(np.float32)
    N, K = w32.shape
    _check_groups(K, group_size)
    if channel_scale is not None:
        cs = np.asarray(channel_scale, dtype=np.float32).reshape(1, K)
        w32 = w32 * cs                                  # float32 product
    wg = w32.reshape(N, K // group_size, group_size)

    # Range of each group: its own min and max.
    wmin = wg.min(axis=2)
    wmax = wg.max(axis=2)
    rng = np.maximum(wmax - wmin, RANGE_FLOOR)          # float32 subtraction
    # scale = range / (2^bits - 1), then stored as fp16.
    s32 = rng / np.float32(QMAX)                        # IEEE float32 divide
    s16 = s32.astype(np.float16)
    sf = s16.astype(np.float32)
    # zero-point: the integer that wmin maps to code 0 (held as an integer,
    # so a clamped -0.0 is stored as +0.0).
    z = np.clip(np.rint(-wmin / sf), 0, QMAX).astype(np.int32).astype(np.float32)
    # codes: round(x / scale) first, then add the zero-point, then clamp.
    q = np.rint(wg / sf[:, :, None]) + z[:, :, None]
    q = np.clip(q, 0, QMAX)
    codes = q.reshape(N, K).astype(np.uint8)
    return codes, s16, z.astype(np.float16)


def clip_position(group_size: int, clip_fraction: float):
    """Order-statistic position of the clip quantile: h = (G - 1) * p in
    float64, split into the integer i = floor(h) and the fraction
    f = float32(h - i). Positions past the middle of a group are refused."""
    if not (0.0 <= clip_fraction < 0.25):
        raise ValueError("clip_fraction must lie in [0, 0.25)")
    h = (group_size - 1) * float(clip_fraction)
    i = int(np.floor(h))
    return i, np.float32(h - i)


def clip_bounds(wg, group_size: int, clip_fraction: float):
    """The clip step of [P5 §1.5]: cut the extreme p of each group's values
    at both ends before the scale is taken (p = 1 % on the page).

    Reading: the bounds are the p and 1 - p quantiles of the group's G
    float32 values, linearly interpolated between order statistics (the
    usual percentile definition, NumPy's default method), with the lower one
    taken from the bottom and the upper one mirrored from the top, in this
    exact float32 order (no fused multiply-add):
      lo = x(i) + f * (x(i+1) - x(i))
      hi = x(G-1-i) - f * (x(G-1-i) - x(G-2-i))
    where x(0) <= ... <= x(G-1) are the sorted values and (i, f) come from
    clip_position. p = 0 gives lo = min, hi = max exactly.

    wg: float32 [N, groups, G] -> (lo, hi) float32 [N, groups]."""
    i, f = clip_position(group_size, clip_fraction)
    xs = np.sort(wg, axis=2)
    a0, a1 = xs[:, :, i], xs[:, :, i + 1]
    b0, b1 = xs[:, :, group_size - 1 - i], xs[:, :, group_size - 2 - i]
    lo = a0 + f * (a1 - a0)
    hi = b0 - f * (b0 - b1)
    return lo.astype(np.float32), hi.astype(np.float32)


def group_quantize_clipped(w, group_size: int, clip_fraction: float, channel_scale=None,
                           symmetric: bool = False):
    """Group-wise INT4 quantization after the clip step of [P5 §1.5]: the
    scale and zero-point come from the clipped bounds (lo, hi) instead of
    the group's min and max; values beyond them take the clamped codes 0 or
    15 (that is the clipping). Asymmetric: range = hi - lo, zero from lo, as
    in group_quantize. Symmetric: a = max(-lo, hi), as in
    group_quantize_symmetric. clip_fraction = 0 reproduces both exactly."""
    w32 = np.asarray(w).astype(np.float32)
    N, K = w32.shape
    _check_groups(K, group_size)
    if channel_scale is not None:
        cs = np.asarray(channel_scale, dtype=np.float32).reshape(1, K)
        w32 = w32 * cs
    wg = w32.reshape(N, K // group_size, group_size)
    lo, hi = clip_bounds(wg, group_size, clip_fraction)
    if symmetric:
        a = np.maximum(np.maximum(-lo, hi), RANGE_FLOOR)
        s16 = (a / np.float32(SYM_QMAX)).astype(np.float16)
        sf = s16.astype(np.float32)
        z = np.full(s16.shape, SYM_ZERO, dtype=np.float32)
    else:
        rng = np.maximum(hi - lo, RANGE_FLOOR)
        s16 = (rng / np.float32(QMAX)).astype(np.float16)
        sf = s16.astype(np.float32)
        z = np.clip(np.rint(-lo / sf), 0, QMAX).astype(np.int32).astype(np.float32)
    q = np.rint(wg / sf[:, :, None]) + z[:, :, None]
    q = np.clip(q, 0, QMAX)
    return q.reshape(N, K).astype(np.uint8), s16, z.astype(np.float16)


def quantize_clipped(w, group_size: int, clip_fraction: float, channel_scale=None, symmetric: bool = False):
    codes, s16, z16 = group_quantize_clipped(w, group_size, clip_fraction, channel_scale, symmetric)
    return pack_codes(codes), s16, z16


SYM_QMAX = 7                    # 2^(bits-1) - 1: the largest signed code used
SYM_ZERO = 8                    # stored zero-point of the symmetric form


def group_quantize_symmetric(w, group_size: int, channel_scale=None):
    """Group-wise symmetric INT4 quantization ([P3 "对称/非对称量化"]: the
    zero-point is 0, which the pages call simple and hardware friendly).

    Reading (the pages give no formula): the group's largest magnitude
    a = max|w| maps to +-7, so the map is odd, q(-w) = -q(w):
      s32 = max(a, 1e-5) / 7          (IEEE float32 divide; floor as R2)
      s16 = float16(s32)              (codes made with the stored scale)
      q   = clamp(rint(w / s16), -8, 7)
    stored in the asymmetric layout as code = q + 8 with zero-point 8, so
    x_hat = (code - 8) * s16 = q * s16 and every linear-layer path applies
    unchanged. Round first, then add the (fixed) zero-point, as in R5.

    Returns (codes uint8 [N, K] in 1..15, scales float16 [N, K/G],
    zeros float16 [N, K/G] all 8)."""
    w32 = np.asarray(w).astype(np.float32)
    N, K = w32.shape
    _check_groups(K, group_size)
    if channel_scale is not None:
        cs = np.asarray(channel_scale, dtype=np.float32).reshape(1, K)
        w32 = w32 * cs
    wg = w32.reshape(N, K // group_size, group_size)
    a = np.maximum(np.abs(wg).max(axis=2), RANGE_FLOOR)
    s32 = a / np.float32(SYM_QMAX)                      # IEEE float32 divide
    s16 = s32.astype(np.float16)
    sf = s16.astype(np.float32)
    q = np.rint(wg / sf[:, :, None]) + np.float32(SYM_ZERO)
    q = np.clip(q, 0, QMAX)
    codes = q.reshape(N, K).astype(np.uint8)
    z16 = np.full(s16.shape, SYM_ZERO, dtype=np.float16)
    return codes, s16, z16


def quantize_symmetric(w, group_size: int, channel_scale=None):
    """Symmetric form of quantize: (qweight, scales, zeros = 8)."""
    codes, s16, z16 = group_quantize_symmetric(w, group_size, channel_scale)
    return pack_codes(codes), s16, z16


def pack_codes(codes) -> np.ndarray:
    """Pack eight 4-bit codes along K into one uint32.

    Code of column k = 8c + j lands in bits 4j..4j+3 of word c (the plain
    little-endian nibble order; the pages give none).
    codes [N, K] (values 0..15) -> qweight uint32 [N, K/8].
    """
    c = np.asarray(codes).astype(np.uint32)
    N, K = c.shape
    if K % 8 != 0:
        raise ValueError("K must be a multiple of 8 to pack nibbles")
    c = c.reshape(N, K // 8, 8)
    out = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):
        out |= c[:, :, j] << np.uint32(4 * j)
    return out


def unpack_codes(qweight, K: int) -> np.ndarray:
    """Inverse of pack_codes: uint32 [N, K/8] -> uint8 codes [N, K]."""
    q = np.asarray(qweight, dtype=np.uint32)
    N = q.shape[0]
    out = np.empty((N, K // 8, 8), dtype=np.uint8)
    for j in range(8):
        out[:, :, j] = (q >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(N, K)


def quantize(w, group_size: int, channel_scale=None):
    """The library's quantize call: (qweight uint32 [N,K/8], scales fp16
    [N,K/G], zeros fp16 [N,K/G])."""
    codes, s16, z16 = group_quantize(w, group_size, channel_scale)
    return pack_codes(codes), s16, z16


def dequantize(qweight, scales, zeros, group_size: int, K: int) -> np.ndarray:
    """x_hat = (q - zero_point) * scale   [P5 §1.2], float64 [N, K].

    Every value is exact in float64 (a 4-bit difference times an fp16)."""
    codes = unpack_codes(qweight, K).astype(np.float64)
    N = codes.shape[0]
    _check_groups(K, group_size)
    s = np.asarray(scales).astype(np.float64)
    z = np.asarray(zeros).astype(np.float64)
    cg = codes.reshape(N, K // group_size, group_size)
    return ((cg - z[:, :, None]) * s[:, :, None]).reshape(N, K)


def linear_ref(x, qweight, scales, zeros, group_size: int) -> np.ndarray:
    """The W4A16 linear layer y = x . dequant(Wq)^T, float64 [M, N].

    x: [M, K] (float16 activations). One float64 matrix product."""
    x64 = np.asarray(x).astype(np.float64)
    K = x64.shape[1]
    w_hat = dequantize(qweight, scales, zeros, group_size, K)
    return x64 @ w_hat.T


# ---------------------------------------------------------------------------
# Activation-aware scale search   [P1 §2.1], [P4 "Per-channel Scaling 优化"]
# ---------------------------------------------------------------------------

def activation_absmean(x) -> np.ndarray:
    """m[k] = mean over tokens of |x[t, k]|, float64, floored at 1e-8."""
    x64 = np.abs(np.asarray(x).astype(np.float64))
    return np.maximum(x64.mean(axis=0), MEAN_FLOOR)


def alpha_grid(n_alpha: int = 20) -> np.ndarray:
    """alpha_i = i / n_alpha for i = 0..n_alpha-1, in float64."""
    return np.arange(n_alpha, dtype=np.float64) / float(n_alpha)


def channel_scales(m, alpha: float) -> np.ndarray:
    """s[k] = m[k]^alpha computed in float64, rounded to float32."""
    return np.power(np.asarray(m, dtype=np.float64), float(alpha)).astype(np.float32)


def searched_weight(w, s32, group_size: int) -> np.ndarray:
    """W_hat_alpha = dequant(Q(W . diag(s))) / s, float64 [N, K].

    Q(W diag(s)) (X / s)^T == X W_hat_alpha^T, so this is the effective
    weight the scaled layer applies to the unscaled activations."""
    w = np.asarray(w)
    K = w.shape[1]
    qw, sc, zr = quantize(w, group_size, channel_scale=s32)
    return dequantize(qw, sc, zr, group_size, K) / np.asarray(s32, np.float64)[None, :]


def search_loss_direct(w, x, s32, group_size: int) -> float:
    """L = || Q(W diag(s)) (X / s)^T - W X^T ||_F^2  (float64, direct form)."""
    w64 = np.asarray(w).astype(np.float64)
    x64 = np.asarray(x).astype(np.float64)
    y = x64 @ w64.T
    y_hat = x64 @ searched_weight(w, s32, group_size).T
    d = y_hat - y
    return float(np.sum(d * d))


def scaled_activations_f16(x, s32) -> np.ndarray:
    """fp16(X / s): the scaled activations as the W4A16 layer takes them.

    The search runs Q(W diag(s)) (X / s)^T on the W4A16 product, whose
    activations are fp16 (the "A16" of the layer, [P1 §1.3]), so X / s enters
    it rounded to fp16. Reading: one IEEE float32 division x / s per element
    (x is fp16, s float32), then round-to-nearest-even to fp16. Returned as
    float64 (exact)."""
    x32 = np.asarray(x).astype(np.float32)
    s = np.asarray(s32, dtype=np.float32).reshape(1, -1)
    return (x32 / s).astype(np.float16).astype(np.float64)


def search_loss_f16_activations(w, x, s32, group_size: int, clip_fraction: float = 0.0,
                                symmetric: bool = False) -> float:
    """L = || Q(W diag(s)) fp16(X / s)^T - W X^T ||_F^2 in float64, direct
    form: the scale search's loss with the scaled activations rounded to the
    fp16 the W4A16 layer takes (see scaled_activations_f16). It differs from
    search_loss_direct only by that rounding; with s a power of two per
    channel (or s = 1) the rounding is exact and the two agree.
    Q is the plain quantizer, or the clipped one when clip_fraction > 0 or
    symmetric is set."""
    w = np.asarray(w)
    K = w.shape[1]
    if clip_fraction == 0.0 and not symmetric:
        qw, sc, zr = quantize(w, group_size, channel_scale=s32)
    else:
        qw, sc, zr = quantize_clipped(w, group_size, clip_fraction, channel_scale=s32, symmetric=symmetric)
    w_q = dequantize(qw, sc, zr, group_size, K)
    y = np.asarray(x).astype(np.float64) @ w.astype(np.float64).T
    y_hat = scaled_activations_f16(x, s32) @ w_q.T
    d = y_hat - y
    return float(np.sum(d * d))


def gram(x) -> np.ndarray:
    """G = X^T X in float64 [K, K]."""
    x64 = np.asarray(x).astype(np.float64)
    return x64.T @ x64


def search_loss_gram(w, g, s32, group_size: int) -> float:
    """Same loss through the Gram matrix: with D = W_hat_alpha - W,
    ||D X^T||_F^2 = sum_n D_n G D_n^T = sum((D G) * D)."""
    d = searched_weight(w, s32, group_size) - np.asarray(w).astype(np.float64)
    return float(np.sum((d @ g) * d))


def scale_search(w, x, group_size: int, alphas=None, use_gram: bool = True, f16_activations: bool = False):
    """AWQ's per-input-channel scale search over an alpha grid.

    For every alpha: s = mean|x|^alpha, quantize W diag(s), and measure the
    squared output error against the unquantized layer. Returns
    (losses float64 [n_alpha], best index, best scales float32 [K]).
    The best index is the first minimum (ties go to the smallest alpha).
    f16_activations=True measures each loss with X / s rounded to fp16
    (search_loss_f16_activations, direct form) instead of exactly."""
    if alphas is None:
        alphas = alpha_grid(20)
    m = activation_absmean(x)
    g = gram(x) if (use_gram and not f16_activations) else None
    losses = np.empty(len(alphas), dtype=np.float64)
    for i, a in enumerate(alphas):
        s32 = channel_scales(m, a)
        if f16_activations:
            losses[i] = search_loss_f16_activations(w, x, s32, group_size)
        elif use_gram:
            losses[i] = search_loss_gram(w, g, s32, group_size)
        else:
            losses[i] = search_loss_direct(w, x, s32, group_size)
    best = int(np.argmin(losses))   # np.argmin returns the first minimum
    return losses, best, channel_scales(m, alphas[best])


def clipped_weight(w, group_size: int, clip_fraction: float, s32=None, symmetric: bool = False) -> np.ndarray:
    """W_hat_p = dequant(Q_p(W . diag(s))) / s in float64 [N, K], with Q_p
    the clipped quantizer, asymmetric or symmetric (s = 1 when s32 is None)."""
    w = np.asarray(w)
    K = w.shape[1]
    qw, sc, zr = quantize_clipped(w, group_size, clip_fraction, channel_scale=s32, symmetric=symmetric)
    w_hat = dequantize(qw, sc, zr, group_size, K)
    if s32 is not None:
        w_hat = w_hat / np.asarray(s32, np.float64)[None, :]
    return w_hat


def clip_search(w, x, group_size: int, fractions, s32=None, use_gram: bool = True, symmetric: bool = False,
                f16_activations: bool = False):
    """Search of the clip fraction p of [P5 §1.5] over a grid, by the same
    output loss as the scale search: for each p,
      L(p) = || Q_p(W diag(s)) (X / s)^T - W X^T ||_F^2
    (s = 1 without channel scales; Q_p asymmetric or symmetric). Returns
    (losses float64 [n], first index of the minimum). f16_activations=True
    (with s32) rounds X / s to fp16 as the W4A16 layer takes it, in the
    direct form."""
    g = gram(x) if (use_gram and not f16_activations) else None
    w64 = np.asarray(w).astype(np.float64)
    losses = np.empty(len(fractions), dtype=np.float64)
    for i, p in enumerate(fractions):
        if f16_activations:
            ones = np.ones(w64.shape[1], np.float32) if s32 is None else s32
            losses[i] = search_loss_f16_activations(w, x, ones, group_size, p, symmetric)
            continue
        d = clipped_weight(w, group_size, p, s32, symmetric) - w64
        if use_gram:
            losses[i] = float(np.sum((d @ g) * d))
        else:
            e = np.asarray(x).astype(np.float64) @ d.T
            losses[i] = float(np.sum(e * e))
    return losses, int(np.argmin(losses))


# ---------------------------------------------------------------------------
# Mixed precision: salient weights kept in fp16   [P4 "技术实现" 1 and
# "混合精度设计"], [P5 §2.2]
# ---------------------------------------------------------------------------

def salient_count(K: int, fraction: float = 0.01) -> int:
    """Number of salient input channels: the pages keep about 1 % of the
    weights; the reading is round(fraction * K) channels (41 of 4096)."""
    return int(round(fraction * K))


def salient_channels(m, n: int) -> np.ndarray:
    """The n input channels with the largest activation statistic m[k]
    (the pages pick the important weights from the activation distribution,
    at the 99th percentile), listed by descending m; equal m go by ascending
    channel index. A plain sort on the key (-m[k], k)."""
    m = np.asarray(m, dtype=np.float64).ravel()
    K = m.size
    if not 0 <= n <= K:
        raise ValueError("n must lie in [0, K]")
    order = sorted(range(K), key=lambda k: (-m[k], k))
    return np.asarray(order[:n], dtype=np.int64)


def mixed_weight(w, group_size: int, idx, symmetric: bool = False) -> np.ndarray:
    """The pages' recipe read literally, float64 [N, K]: quantize all of W
    (every group's range over all its G weights, salient ones included),
    dequantize, then put the original values back in the salient columns."""
    w = np.asarray(w)
    K = w.shape[1]
    qw, sc, zr = (quantize_symmetric if symmetric else quantize)(w, group_size)
    w_hat = dequantize(qw, sc, zr, group_size, K)
    idx = np.asarray(idx, dtype=np.int64)
    w_hat[:, idx] = w[:, idx].astype(np.float64)
    return w_hat


def quantize_salient(w, group_size: int, idx, symmetric: bool = False):
    """The stored form of the mixed-precision layer: the quantizer of
    group_quantize (or the symmetric one) on all of W, then the codes of the
    salient columns set to their group's zero-point, so that they dequantize
    to exactly 0, and the salient fp16 weights kept beside as
    w_salient[j, n] = W[n, idx[j]] (float16 [n_salient, N]).
    Returns (qweight, scales, zeros, w_salient)."""
    w16 = np.asarray(w).astype(np.float16)
    N, K = w16.shape
    codes, s16, z16 = (group_quantize_symmetric if symmetric else group_quantize)(w16, group_size)
    codes = codes.copy()
    idx = np.asarray(idx, dtype=np.int64)
    for k in idx:
        codes[:, k] = z16[:, k // group_size].astype(np.uint8)
    w_salient = np.ascontiguousarray(w16[:, idx].T)
    return pack_codes(codes), s16, z16, w_salient


def dequantize_salient(qweight, scales, zeros, group_size: int, K: int, idx, w_salient) -> np.ndarray:
    """Effective weight of the stored form, float64 [N, K]: the INT4 part
    (zero in the salient columns) plus the fp16 salient columns."""
    w_hat = dequantize(qweight, scales, zeros, group_size, K)
    idx = np.asarray(idx, dtype=np.int64)
    w_hat[:, idx] += np.asarray(w_salient).astype(np.float64).T
    return w_hat


def linear_salient_ref(x, qweight, scales, zeros, group_size: int, idx, w_salient) -> np.ndarray:
    """y = x . W_mixed^T in float64 [M, N]: the W4A16 product plus the
    fp16 side product x[:, idx] . w_salient."""
    x64 = np.asarray(x).astype(np.float64)
    K = x64.shape[1]
    return x64 @ dequantize_salient(qweight, scales, zeros, group_size, K, idx, w_salient).T


def salient_loss(w, x, group_size: int, idx, use_gram: bool = True, symmetric: bool = False) -> float:
    """Output loss of the mixed-precision layer, by the scale search's
    measure: || X W_mixed^T - X W^T ||_F^2 (float64)."""
    d = mixed_weight(w, group_size, idx, symmetric) - np.asarray(w).astype(np.float64)
    if use_gram:
        return float(np.sum((d @ gram(x)) * d))
    e = np.asarray(x).astype(np.float64) @ d.T
    return float(np.sum(e * e))


# ---------------------------------------------------------------------------
# W8A16: 8-bit weights, fp16 activations   [P3 "INT8 vs INT4" and "INT8 实战"
# (weight INT8 with activations kept in FP16/BF16)], the map of [P5 §1.2]
# with bits = 8
# ---------------------------------------------------------------------------

def group_quantize_bits(w, group_size: int, bits: int, channel_scale=None, symmetric: bool = False):
    """Group-wise quantization with 2^bits levels, written for any width.

    Asymmetric: scale = max(range, 1e-5) / (2^bits - 1) (IEEE float32),
    stored as fp16; zero = clamp(rint(-min / scale), 0, 2^bits - 1);
    code = clamp(rint(w / scale) + zero, 0, 2^bits - 1).
    Symmetric: scale = max(max|w|, 1e-5) / (2^(bits-1) - 1), stored as fp16,
    code = clamp(rint(w / scale) + 2^(bits-1), 0, 2^bits - 1) with stored
    zero-point 2^(bits-1).
    Returns (codes uint8 [N, K], scales float16 [N, K/G], zeros float16)."""
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    qmax = np.float32((1 << bits) - 1)
    half_levels = 1 << (bits - 1)
    w32 = np.asarray(w).astype(np.float32)
    N, K = w32.shape
    _check_groups(K, group_size)
    if channel_scale is not None:
        w32 = w32 * np.asarray(channel_scale, dtype=np.float32).reshape(1, K)
    wg = w32.reshape(N, K // group_size, group_size)
    if symmetric:
        a = np.maximum(np.abs(wg).max(axis=2), RANGE_FLOOR)
        sf = (a / np.float32(half_levels - 1)).astype(np.float16).astype(np.float32)
        z = np.full(sf.shape, np.float32(half_levels))
    else:
        wmin = wg.min(axis=2)
        rng = np.maximum(wg.max(axis=2) - wmin, RANGE_FLOOR)
        sf = (rng / qmax).astype(np.float16).astype(np.float32)
        z = np.clip(np.rint(-wmin / sf), 0, qmax).astype(np.int32).astype(np.float32)
    q = np.clip(np.rint(wg / sf[:, :, None]) + z[:, :, None], 0, qmax)
    return q.reshape(N, K).astype(np.uint8), sf.astype(np.float16), z.astype(np.float16)


def pack_codes8(codes) -> np.ndarray:
    """Four 8-bit codes along K per uint32: the code of column k = 4c + j in
    bits 8j..8j+7 of word c. codes [N, K] -> uint32 [N, K/4]."""
    c = np.asarray(codes).astype(np.uint32)
    N, K = c.shape
    if K % 4 != 0:
        raise ValueError("K must be a multiple of 4 to pack bytes")
    c = c.reshape(N, K // 4, 4)
    out = np.zeros((N, K // 4), dtype=np.uint32)
    for j in range(4):
        out |= c[:, :, j] << np.uint32(8 * j)
    return out


def unpack_codes8(qweight, K: int) -> np.ndarray:
    q = np.asarray(qweight, dtype=np.uint32)
    N = q.shape[0]
    out = np.empty((N, K // 4, 4), dtype=np.uint8)
    for j in range(4):
        out[:, :, j] = (q >> np.uint32(8 * j)) & np.uint32(0xFF)
    return out.reshape(N, K)


def quantize_w8(w, group_size: int, channel_scale=None, symmetric: bool = False):
    """W8 quantize call: (qweight uint32 [N, K/4], scales, zeros)."""
    codes, s16, z16 = group_quantize_bits(w, group_size, 8, channel_scale, symmetric)
    return pack_codes8(codes), s16, z16


def dequantize_w8(qweight, scales, zeros, group_size: int, K: int) -> np.ndarray:
    """x_hat = (q - zero_point) * scale, float64 [N, K] (exact)."""
    codes = unpack_codes8(qweight, K).astype(np.float64)
    N = codes.shape[0]
    s = np.asarray(scales).astype(np.float64)
    z = np.asarray(zeros).astype(np.float64)
    cg = codes.reshape(N, K // group_size, group_size)
    return ((cg - z[:, :, None]) * s[:, :, None]).reshape(N, K)


def linear_ref_w8(x, qweight, scales, zeros, group_size: int) -> np.ndarray:
    """The W8A16 linear layer y = x . dequant(Wq)^T, float64 [M, N]."""
    x64 = np.asarray(x).astype(np.float64)
    return x64 @ dequantize_w8(qweight, scales, zeros, group_size, x64.shape[1]).T
