"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: the
worked example printed on "模型量化:GGUF/AWQ/GPTQ部署方案" §1.2, closed forms,
invariants of min-max affine quantization, constructed rounding ties,
structural special cases and brute force on tiny inputs.
"""

import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _row(values, K=128):
    w = np.zeros((1, K), dtype=np.float16)
    w[0, : len(values)] = np.asarray(values, dtype=np.float16)
    return w


# ---------------------------------------------------------------- worked example

def test_worked_example_matches_page():
    """§1.2 of the xxmr.cn page: range [-1, 1] -> scale 2/15 ~ 0.133;
    0.5 -> 4 -> ~0.53, error ~0.03."""
    g = _golden("worked_example_p5_s1_2.json")
    lo, hi = g["range"]
    w = _row([lo, hi, g["x"]])
    codes, s16, z16 = oracle.group_quantize(w, 128)
    scale = float(s16[0, 0])
    zp = int(z16[0, 0])
    # scale equals 2/15 to the printed digits
    assert abs(scale - g["scale"]) < 0.5 * 10 ** -g["printed_digits"]["scale"]
    assert abs(scale - g["scale_fraction"][0] / g["scale_fraction"][1]) < 1e-4
    # round(x / scale) is the page's 4 (the code before the zero point is added)
    assert int(codes[0, 2]) - zp == g["round_x_over_scale"]
    qw, sc, zr = oracle.quantize(w, 128)
    w_hat = oracle.dequantize(qw, sc, zr, 128, 128)
    x_hat = w_hat[0, 2]
    assert abs(x_hat - g["x_hat"]) < 0.5 * 10 ** -g["printed_digits"]["x_hat"]
    assert abs(abs(x_hat - g["x"]) - g["abs_error"]) < 0.5 * 10 ** -g["printed_digits"]["abs_error"]


def test_worked_example_exact_values():
    """The same example carried out exactly: fp32(2/15) = 0.13333334 rounds
    to the fp16 0x3044 = 0.13330078125; 1/0.13330078125 = 7.5018 -> zero
    point 8; 0.5 -> rint(3.7509) = 4 -> code 12 -> (12-8)*s = 0.533203125;
    1.0 saturates at code 15; -1.0 maps to code 0."""
    w = _row([-1.0, 1.0, 0.5])
    codes, s16, z16 = oracle.group_quantize(w, 128)
    assert s16[0, 0].view(np.uint16) == 0x3044
    assert float(s16[0, 0]) == 0.13330078125
    assert float(z16[0, 0]) == 8.0
    assert codes[0, 0] == 0 and codes[0, 1] == 15 and codes[0, 2] == 12
    qw, sc, zr = oracle.quantize(w, 128)
    w_hat = oracle.dequantize(qw, sc, zr, 128, 128)
    assert w_hat[0, 2] == 0.533203125
    assert w_hat[0, 1] == 7 * 0.13330078125
    assert w_hat[0, 0] == -8 * 0.13330078125


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("G", [64, 128])
def test_affine_invariants(G):
    lay = synth.make_layer(96, 1024, 0, seed=[11, G], w_std=0.02)
    w = lay["w"]
    codes, s16, z16 = oracle.group_quantize(w, G)
    assert codes.max() <= 15
    z = z16.astype(np.float64)
    assert np.all(z == np.rint(z)) and z.min() >= 0 and z.max() <= 15
    qw, sc, zr = oracle.quantize(w, G)
    w_hat = oracle.dequantize(qw, sc, zr, G, 1024)
    s = np.repeat(s16.astype(np.float64), G, axis=1)
    err = np.abs(w.astype(np.float64) - w_hat)
    clamped = (codes == 0) | (codes == 15)
    # round-to-nearest: error at most half a step (to fp32 rounding of w/s)
    assert np.all(err[~clamped] <= s[~clamped] * (0.5 + 1e-6))
    # groups straddle zero here: wmin lands on code 0, wmax on 14 or 15
    wg = w.astype(np.float32).reshape(96, -1, G)
    cg = codes.reshape(96, -1, G)
    assert np.all((wg.min(axis=2) < 0) & (wg.max(axis=2) > 0))
    cmin = np.take_along_axis(cg, wg.argmin(axis=2)[..., None], axis=2)[..., 0]
    cmax = np.take_along_axis(cg, wg.argmax(axis=2)[..., None], axis=2)[..., 0]
    assert np.all(cmin == 0)
    assert np.all((cmax == 14) | (cmax == 15))
    # clamped codes: error within half a step plus the fp16 rounding of the scale
    rng = (wg.max(axis=2) - wg.min(axis=2)).astype(np.float64)
    bound = s16.astype(np.float64) / 2 + 15 * np.abs(s16.astype(np.float64) - rng / 15)
    bound = np.repeat(bound, G, axis=1) * (1 + 1e-6)
    assert np.all(err[clamped] <= bound[clamped])


def test_constructed_ties_round_half_to_even():
    """With range [-1, 1] the scale is s = 273 * 2^-11 (fp16 0x3044), so
    (k + 1/2) s is an exact fp16 for k = 0..3 and w / s is exactly k + 1/2.
    Half-to-even gives 0, 2, 2, 4 (half-away-from-zero would give 1, 2, 3, 4)."""
    s = 0.13330078125
    ties = [(k + 0.5) * s for k in range(4)]
    assert all(float(np.float16(t)) == t for t in ties)
    w = _row([-1.0, 1.0] + ties + [-t for t in ties])
    codes, _, z16 = oracle.group_quantize(w, 128)
    zp = int(z16[0, 0])
    assert zp == 8
    assert [int(c) - zp for c in codes[0, 2:6]] == [0, 2, 2, 4]
    assert [int(c) - zp for c in codes[0, 6:10]] == [0, -2, -2, -4]


def test_round_before_adding_zero_point():
    """w / s = 0.5 + 2^-24 (one fp32 step above a tie). Rounding first gives
    1, then + 8 = 9; adding the zero point first would give 8.5 in fp32
    (the step at 8 is 2^-20) and round to 8."""
    s = np.float32(0.13330078125)
    c_tie = np.nextafter(np.float32(0.5) * s, np.float32(1))
    assert np.float32(c_tie / s) == np.float32(0.5) + np.float32(2.0 ** -24)
    w = _row([-1.0, 1.0, 1.0])
    cs = np.ones(128, dtype=np.float32)
    cs[2] = c_tie
    codes, s16, z16 = oracle.group_quantize(w, 128, channel_scale=cs)
    assert float(s16[0, 0]) == float(s)
    assert int(z16[0, 0]) == 8
    assert codes[0, 2] == 9


def test_fp16_subnormal_weights_are_not_flushed():
    """A group of fp16 subnormals quantizes with its own (tiny) range."""
    tiny = np.array([-6e-5, 6e-5, 3e-5, -1e-6], dtype=np.float16)
    assert np.all(np.abs(tiny.astype(np.float32)) < 6.104e-5)
    w = _row(tiny)
    codes, s16, z16 = oracle.group_quantize(w, 128)
    # range ~1.2e-4 gives a scale ~8e-6, far above the 1e-5/15 floor
    assert float(s16[0, 0]) > 5e-6
    qw, sc, zr = oracle.quantize(w, 128)
    w_hat = oracle.dequantize(qw, sc, zr, 128, 128)
    s = float(s16[0, 0])
    rng = float(np.float32(tiny.max()) - np.float32(tiny.min()))
    err = np.abs(w_hat[0, :4] - tiny.astype(np.float64))
    clamped = (codes[0, :4] == 0) | (codes[0, :4] == 15)
    assert np.all(err[~clamped] <= s * 0.5 * (1 + 1e-6))
    assert np.all(err[clamped] <= (s / 2 + 15 * abs(s - rng / 15)) * (1 + 1e-6))
    assert codes[0, 0] == 0 and codes[0, 1] == 15


# ---------------------------------------------------------------- special cases

def test_groups_run_along_k_and_rows_are_independent():
    """Per-group quantization of [N, K] equals quantizing every (row, group)
    slice as its own 1 x G matrix; per-channel is the G = K case."""
    lay = synth.make_layer(8, 512, 0, seed=[12], w_std=0.02)
    w = lay["w"]
    for G in (64, 128, 512):
        codes, s16, z16 = oracle.group_quantize(w, G)
        for n in range(8):
            for g in range(512 // G):
                c1, s1, z1 = oracle.group_quantize(w[n:n + 1, g * G:(g + 1) * G], G)
                assert np.array_equal(c1[0], codes[n, g * G:(g + 1) * G])
                assert s1[0, 0] == s16[n, g] and z1[0, 0] == z16[n, g]


def test_per_channel_is_textbook_minmax():
    """G = K: one scale per output channel, (max - min) / 15 of the row."""
    lay = synth.make_layer(16, 256, 0, seed=[13], w_std=0.02)
    w = lay["w"]
    codes, s16, z16 = oracle.group_quantize(w, 256)
    rows = w.astype(np.float32)
    expect = ((rows.max(axis=1) - rows.min(axis=1)) / np.float32(15)).astype(np.float16)
    assert np.array_equal(s16[:, 0], expect)
    assert np.all(codes[np.arange(16), rows.argmin(axis=1)] == 0)


def test_constant_group_uses_range_floor():
    w = np.zeros((2, 128), dtype=np.float16)
    w[1, :] = np.float16(0.25)
    codes, s16, z16 = oracle.group_quantize(w, 128)
    floor_scale = np.float16(np.float32(1e-5) / np.float32(15))
    assert s16[0, 0] == floor_scale and s16[1, 0] == floor_scale
    assert float(s16[0, 0]) > 0
    # zero group: every code equals the zero point 0
    assert z16[0, 0] == 0 and np.all(codes[0] == 0)
    # a positive constant saturates (zero point clamps to 0)
    assert z16[1, 0] == 0 and np.all(codes[1] == 15)


@pytest.mark.parametrize("j", [1, 2, 3, 5])
def test_power_of_two_equivariance(j):
    """W * 2^j: identical codes and zeros, scales exactly * 2^j."""
    lay = synth.make_layer(32, 512, 0, seed=[14, j], w_std=0.02)
    w = lay["w"]
    w2 = (w.astype(np.float32) * np.float32(2.0 ** j)).astype(np.float16)
    assert np.array_equal(w2.astype(np.float64), w.astype(np.float64) * 2.0 ** j)
    c1, s1, z1 = oracle.group_quantize(w, 128)
    c2, s2, z2 = oracle.group_quantize(w2, 128)
    assert np.array_equal(c1, c2) and np.array_equal(z1, z2)
    assert np.array_equal(s2.astype(np.float64), s1.astype(np.float64) * 2.0 ** j)


# ---------------------------------------------------------------- packing

def test_pack_nibble_order_by_hex_digits():
    """Word c holds codes 8c..8c+7, code 8c+j in hex digit j counted from the
    least significant end."""
    rng = np.random.default_rng(15)
    codes = rng.integers(0, 16, size=(5, 64)).astype(np.uint8)
    qw = oracle.pack_codes(codes)
    assert qw.dtype == np.uint32 and qw.shape == (5, 8)
    for n in range(5):
        for c in range(8):
            digits = format(int(qw[n, c]), "08x")[::-1]
            assert [int(d, 16) for d in digits] == list(codes[n, 8 * c:8 * c + 8])
    assert np.array_equal(oracle.unpack_codes(qw, 64), codes)


def test_storage_bits_per_weight():
    """4-bit codes + fp16 scale and zero per 128 weights = 4.25 bits/weight.
    A 7B model at 4 bits is 3.5 GB of codes (the xxmr.cn page's TL;DR and
    §1.1: 14 GB fp16 -> 3.5 GB int4)."""
    w = synth.make_layer(64, 1024, 0, seed=[16])["w"]
    qw, sc, zr = oracle.quantize(w, 128)
    bits = 8 * (qw.nbytes + sc.nbytes + zr.nbytes) / w.size
    assert bits == 4.25
    assert 7e9 * 2 / 1e9 == 14.0 and 7e9 * 4 / 8 / 1e9 == 3.5


# ---------------------------------------------------------------- linear layer

def _brute_linear(x, qw, sc, zr, G):
    """Triple loop over Python floats, unpacking codes through hex digits."""
    M, K = x.shape
    N = qw.shape[0]
    y = [[0.0] * N for _ in range(M)]
    for n in range(N):
        digits = []
        for c in range(K // 8):
            digits += [int(d, 16) for d in format(int(qw[n, c]), "08x")[::-1]]
        for m in range(M):
            acc = 0.0
            for k in range(K):
                wk = (digits[k] - float(zr[n, k // G])) * float(sc[n, k // G])
                acc += float(x[m, k]) * wk
            y[m][n] = acc
    return np.array(y)


def test_linear_ref_matches_brute_force():
    lay = synth.make_layer(24, 256, 3, seed=[17], w_std=0.02)
    qw, sc, zr = oracle.quantize(lay["w"], 64)
    y = oracle.linear_ref(lay["x"], qw, sc, zr, 64)
    yb = _brute_linear(lay["x"], qw, sc, zr, 64)
    assert y.shape == (3, 24)
    assert np.linalg.norm(y - yb) <= 1e-12 * np.linalg.norm(yb)


def test_linear_ref_one_hot_and_linearity():
    """A one-hot x times a returns a * (dequantized column) exactly; the error
    against the unquantized layer is then |w_hat - w| * |a|, the error model of
    "AWQ 模型量化技术" (核心原理)."""
    lay = synth.make_layer(16, 256, 2, seed=[18], w_std=0.02)
    w = lay["w"]
    qw, sc, zr = oracle.quantize(w, 128)
    w_hat = oracle.dequantize(qw, sc, zr, 128, 256)
    for k in (0, 77, 255):
        a = 3.0
        x = np.zeros((1, 256), dtype=np.float16)
        x[0, k] = a
        y = oracle.linear_ref(x, qw, sc, zr, 128)[0]
        assert np.array_equal(y, a * w_hat[:, k])
        assert np.allclose(np.abs(y - a * w[:, k].astype(np.float64)),
                           np.abs(w_hat[:, k] - w[:, k].astype(np.float64)) * abs(a), rtol=0, atol=1e-15)
    x1, x2 = lay["x"][0:1], lay["x"][1:2]
    y12 = oracle.linear_ref(np.vstack([x1, x2]), qw, sc, zr, 128)
    assert np.allclose(y12[0] + y12[1],
                       oracle.linear_ref(x1, qw, sc, zr, 128)[0] + oracle.linear_ref(x2, qw, sc, zr, 128)[0],
                       rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- scale search

def test_absmean_closed_form():
    x = np.zeros((6, 4), dtype=np.float16)
    x[:, 0] = 2.0
    x[:, 1] = [-1, 1, -1, 1, -1, 1]
    x[:3, 2] = -3.0
    # column 3 all zero -> floor
    m = oracle.activation_absmean(x)
    assert m.shape == (4,)
    assert np.array_equal(m, np.array([2.0, 1.0, 1.5, 1e-8]))


def test_alpha_grid_values():
    a = oracle.alpha_grid(20)
    assert len(a) == 20 and a[0] == 0.0 and a[1] == 0.05 and a[19] == 0.95
    assert np.all(np.diff(a) > 0)


def test_channel_scales_closed_form():
    m = np.array([4.0, 0.25, 1.0, 9.0])
    assert np.array_equal(oracle.channel_scales(m, 0.5), np.array([2.0, 0.5, 1.0, 3.0], dtype=np.float32))
    assert np.array_equal(oracle.channel_scales(m, 0.0), np.ones(4, dtype=np.float32))


def test_searched_weight_error_bound():
    """Q(W diag(s)) / s stays within half a (scaled) step of W per element
    (unclamped codes); multiplying by s instead of dividing would not."""
    lay = synth.make_layer(32, 512, 64, seed=[19], w_std=0.02)
    w, x = lay["w"], lay["x"]
    s = oracle.channel_scales(oracle.activation_absmean(x), 0.5)
    w_hat = oracle.searched_weight(w, s, 128)
    codes, s16, _ = oracle.group_quantize(w, 128, channel_scale=s)
    step = np.repeat(s16.astype(np.float64), 128, axis=1) / s.astype(np.float64)[None, :]
    err = np.abs(w_hat - w.astype(np.float64))
    ok = (codes > 0) & (codes < 15)
    assert np.all(err[ok] <= step[ok] * (0.5 + 1e-6))
    assert not np.all(err <= step * 0.5 * 1e-3)


def test_alpha_zero_is_rtn():
    """alpha = 0 gives s = 1: the searched weight is plain round-to-nearest
    group quantization (the rskf.cn article's §1.1 RTN baseline)."""
    lay = synth.make_layer(32, 256, 48, seed=[20], w_std=0.02)
    w, x = lay["w"], lay["x"]
    s0 = oracle.channel_scales(oracle.activation_absmean(x), 0.0)
    assert np.all(s0 == 1.0)
    qw, sc, zr = oracle.quantize(w, 128)
    rtn = oracle.dequantize(qw, sc, zr, 128, 256)
    assert np.array_equal(oracle.searched_weight(w, s0, 128), rtn)
    d = (x.astype(np.float64) @ (rtn - w.astype(np.float64)).T)
    assert np.isclose(oracle.search_loss_direct(w, x, s0, 128), np.sum(d * d), rtol=1e-12)


def test_loss_identity_input_is_weight_error():
    """X = I (T = K): the output error is the weight error itself."""
    K = 128
    w = synth.make_layer(16, K, 0, seed=[21])["w"]
    x = np.eye(K, dtype=np.float16)
    s = np.full(K, 1.0, dtype=np.float32)
    qw, sc, zr = oracle.quantize(w, 64)
    d = oracle.dequantize(qw, sc, zr, 64, K) - w.astype(np.float64)
    assert np.isclose(oracle.search_loss_direct(w, x, s, 64), np.sum(d * d), rtol=1e-12)


def test_gram_identity():
    """||D X^T||^2 == sum_n D_n (X^T X) D_n^T on T=512, N=256, K=512."""
    lay = synth.make_layer(256, 512, 512, seed=[22], w_std=0.02)
    w, x = lay["w"], lay["x"]
    g = oracle.gram(x)
    for a in (0.0, 0.35, 0.9):
        s = oracle.channel_scales(oracle.activation_absmean(x), a)
        ld = oracle.search_loss_direct(w, x, s, 128)
        lg = oracle.search_loss_gram(w, g, s, 128)
        assert abs(ld - lg) <= 1e-10 * ld


def test_f16_activation_loss_equals_exact_when_rounding_is_exact():
    """X / s rounded to fp16 is exact for s = 1 (alpha = 0) and for s a
    power of two per channel (no underflow at these magnitudes), so the
    fp16-activation loss then equals the exact direct loss (up to the fp64
    summation order of the two products, ~1e-11 relative here)."""
    lay = synth.make_layer(96, 256, 80, seed=[27], w_std=0.02)
    w, x = lay["w"], lay["x"]
    ones = np.ones(256, np.float32)
    la = oracle.search_loss_f16_activations(w, x, ones, 64)
    assert abs(la - oracle.search_loss_direct(w, x, ones, 64)) <= 1e-9 * la
    p2 = (2.0 ** np.random.default_rng(28).integers(-3, 4, 256)).astype(np.float32)
    lp = oracle.search_loss_f16_activations(w, x, p2, 64)
    assert abs(lp - oracle.search_loss_direct(w, x, p2, 64)) <= 1e-9 * lp
    # a generic s rounds: the two differ, by far less than the loss
    s = oracle.channel_scales(oracle.activation_absmean(x), 0.5)
    lg, ld = oracle.search_loss_f16_activations(w, x, s, 64), oracle.search_loss_direct(w, x, s, 64)
    assert lg != ld and abs(lg - ld) <= 1e-3 * ld


def test_f16_activation_loss_matches_brute_force():
    """Element-by-element loop on a tiny case: fp16(float32(x) / s) per
    activation, the dequantized weight per element, squared error summed."""
    lay = synth.make_layer(5, 64, 3, seed=[29], w_std=0.02)
    w, x = lay["w"], lay["x"]
    s = oracle.channel_scales(oracle.activation_absmean(x), 0.7)
    qw, sc, zr = oracle.quantize(w, 32, channel_scale=s)
    codes = oracle.unpack_codes(qw, 64)
    total = 0.0
    for t in range(3):
        for n in range(5):
            yh = 0.0
            y = 0.0
            for k in range(64):
                xs = float(np.float16(np.float32(x[t, k]) / np.float32(s[k])))
                wq = (float(codes[n, k]) - float(zr[n, k // 32])) * float(sc[n, k // 32])
                yh += xs * wq
                y += float(x[t, k]) * float(w[n, k])
            total += (yh - y) ** 2
    got = oracle.search_loss_f16_activations(w, x, s, 32)
    assert abs(got - total) <= 1e-11 * total


def test_f16_activation_search_matches_exact_choice():
    """On the small search cases the fp16 rounding of X / s moves the losses
    by under 1e-4 relative, far below the gap between the best two alphas,
    so both forms pick the same alpha."""
    lay = synth.make_layer(128, 512, 256, seed=[8], w_std=0.02, w_mult=1.0)
    w, x = lay["w"], lay["x"]
    le, be, _ = oracle.scale_search(w, x, 128)
    lf, bf, _ = oracle.scale_search(w, x, 128, f16_activations=True)
    assert be == bf
    assert np.all(np.abs(lf - le) <= 1e-4 * le)


def test_loss_invariant_to_power_of_two_factor_on_s():
    """Scaling every s by 2 changes no code, only the scales (exactly), so the
    loss does not depend on a global factor and s needs no normalisation."""
    lay = synth.make_layer(32, 256, 64, seed=[23], w_std=0.02)
    w, x = lay["w"], lay["x"]
    s = oracle.channel_scales(oracle.activation_absmean(x), 0.4)
    w1 = oracle.searched_weight(w, s, 128)
    w2 = oracle.searched_weight(w, s * np.float32(2), 128)
    assert np.array_equal(w1, w2)


def test_search_tie_goes_to_smallest_alpha():
    """|x| == 1 everywhere: m = 1, every alpha gives s = 1 and the same loss;
    the first alpha wins."""
    w = synth.make_layer(16, 256, 0, seed=[24])["w"]
    rng = np.random.default_rng(24)
    x = np.where(rng.random((32, 256)) < 0.5, -1.0, 1.0).astype(np.float16)
    losses, best, s = oracle.scale_search(w, x, 128)
    assert np.all(losses == losses[0]) and best == 0 and np.all(s == 1.0)


def test_search_beats_rtn_on_salient_channels():
    """With 1 % salient input channels (x20 activations) and plain Gaussian
    weights, the searched scale lowers the output error below plain RTN
    (alpha = 0), the pages' central claim (rskf.cn article §2.1-2.2), with an
    interior minimum. Both the direct and Gram routes agree."""
    lay = synth.make_layer(128, 1024, 512, seed=[25], w_std=0.02, w_mult=1.0)
    w, x = lay["w"], lay["x"]
    ld, bd, _ = oracle.scale_search(w, x, 128, use_gram=False)
    lg, bg, _ = oracle.scale_search(w, x, 128, use_gram=True)
    assert bd == bg
    assert np.allclose(ld, lg, rtol=1e-9)
    assert 0 < bd < 19
    assert ld[bd] < 0.6 * ld[0]


def test_search_keeps_rtn_when_salient_weights_set_the_range():
    """When the salient input channels also carry x10 weights, those weights
    already set their groups' ranges; scaling them up only coarsens the
    rest, so the loss rises with alpha and alpha = 0 wins."""
    lay = synth.make_layer(128, 1024, 512, seed=[25], w_std=0.02, w_mult=10.0)
    losses, best, _ = oracle.scale_search(lay["w"], lay["x"], 128)
    assert best == 0
    assert np.all(np.diff(losses) > 0)


def test_zero_point_is_positive_zero_when_clamped():
    """A group whose minimum is positive clamps its zero-point to 0, stored
    as +0.0 (the zero-point is an integer)."""
    w = _row([0.5, 0.75, 1.0] + [0.25] * 125)
    _, _, z16 = oracle.group_quantize(w, 128)
    assert z16[0, 0].view(np.uint16) == 0x0000
