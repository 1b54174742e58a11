"""Pins of the oracle's clip step (xxmr.cn §1.5: cut the extreme 1 % of a
distribution's values at both ends before taking the scale) and of the clip
search (the clip fraction chosen by the scale search's output loss)."""

import numpy as np
import pytest

import oracle
import synth


@pytest.mark.parametrize("G", [32, 64, 128, 256])
@pytest.mark.parametrize("symmetric", [False, True])
def test_zero_fraction_is_the_plain_quantizer(G, symmetric):
    lay = synth.make_layer(64, 1024, 0, seed=[160, G], w_std=0.02, salient_frac=0.01)
    got = oracle.quantize_clipped(lay["w"], G, 0.0, symmetric=symmetric)
    exp = (oracle.quantize_symmetric if symmetric else oracle.quantize)(lay["w"], G)
    for a, b in zip(got, exp):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def test_hand_worked_ramp():
    """Group 0, 1, ..., 127 at p = 1 %: h = 127 * 0.01 = 1.27, so
    lo = x(1) + 0.27 * (x(2) - x(1)) = 1.27 and hi = x(126) - 0.27 *
    (x(126) - x(125)) = 125.73 (both in fp32). range = 124.46, scale =
    fp16(124.46 / 15 = 8.2973) = 8.296875 (fp16 spacing 1/128 at 8);
    zero = rint(-1.27 / 8.296875) = rint(-0.153) = 0 (clamped from -0);
    value 0 -> code 0, value 127 -> rint(15.307) = 15, value 64 ->
    rint(7.714) = 8."""
    w = np.arange(128, dtype=np.float16).reshape(1, 128)
    lo, hi = oracle.clip_bounds(w.astype(np.float32).reshape(1, 1, 128), 128, 0.01)
    assert lo[0, 0] == np.float32(1.27) and hi[0, 0] == np.float32(125.73)
    codes, s16, z16 = oracle.group_quantize_clipped(w, 128, 0.01)
    assert float(s16[0, 0]) == 8.296875
    assert float(z16[0, 0]) == 0.0
    assert codes[0, 0] == 0 and codes[0, 127] == 15 and codes[0, 64] == 8


@pytest.mark.parametrize("G", [32, 128, 256])
@pytest.mark.parametrize("p", [0.01, 0.05, 0.1])
def test_bounds_are_the_linear_percentiles(G, p):
    """The bounds equal NumPy's linear-interpolation percentiles up to the
    float32 rounding of the interpolation (a few ulps of the group's
    spread)."""
    lay = synth.make_layer(16, 4 * G, 0, seed=[161, G, int(p * 100)], w_std=0.02)
    wg = lay["w"].astype(np.float32).reshape(16, 4, G)
    lo, hi = oracle.clip_bounds(wg, G, p)
    ref_lo = np.percentile(wg.astype(np.float64), 100 * p, axis=2)
    ref_hi = np.percentile(wg.astype(np.float64), 100 * (1 - p), axis=2)
    spread = (wg.max(axis=2) - wg.min(axis=2)).astype(np.float64)
    tol = 4 * np.finfo(np.float32).eps * spread
    assert np.all(np.abs(lo - ref_lo) <= tol) and np.all(np.abs(hi - ref_hi) <= tol)
    assert np.all(lo <= hi)


def test_clip_helps_a_group_with_one_outlier():
    """127 values ~ N(0, 0.02) and one at 1.0: the outlier sets the plain
    range (scale ~ 1/15), so most values share a handful of codes. Clipping
    1 % puts the range on the bulk: the error of the 127 others falls."""
    rng = np.random.default_rng(162)
    w = (rng.standard_normal((1, 128)) * 0.02).astype(np.float16)
    w[0, 77] = 1.0
    bulk = np.arange(128) != 77
    err = {}
    for p in (0.0, 0.01):
        qw, sc, zr = oracle.quantize_clipped(w, 128, p)
        e = oracle.dequantize(qw, sc, zr, 128, 128) - w.astype(np.float64)
        err[p] = float(np.sqrt(np.mean(e[0, bulk] ** 2)))
    assert err[0.01] < 0.25 * err[0.0]


def test_clip_search_gram_equals_direct_and_ties_go_first():
    lay = synth.make_layer(64, 256, 384, seed=[163], w_std=0.02, salient_frac=0.01)
    fr = [0.0, 0.005, 0.01, 0.02, 0.05]
    lg, bg = oracle.clip_search(lay["w"], lay["x"], 64, fr)
    ld, bd = oracle.clip_search(lay["w"], lay["x"], 64, fr, use_gram=False)
    np.testing.assert_allclose(lg, ld, rtol=1e-10)
    assert bg == bd
    # G = 64 with 0 < p < 1/63: h < 1, i = 0, and duplicated fractions give
    # duplicated losses; the first wins
    l2, b2 = oracle.clip_search(lay["w"], lay["x"], 64, [0.01, 0.01, 0.0])
    assert l2[0] == l2[1] and (b2 == 0 or b2 == 2)


def test_clip_search_with_channel_scales_matches_scaled_loss():
    """p = 0 with channel scales s is the scale search's loss at that s."""
    lay = synth.make_layer(64, 256, 256, seed=[164], w_std=0.02, salient_frac=0.01)
    m = oracle.activation_absmean(lay["x"])
    s32 = oracle.channel_scales(m, 0.5)
    lc, _ = oracle.clip_search(lay["w"], lay["x"], 128, [0.0], s32=s32)
    ls = oracle.search_loss_gram(lay["w"], oracle.gram(lay["x"]), s32, 128)
    assert lc[0] == pytest.approx(ls, rel=1e-12)


def test_symmetric_clip_search_at_zero_is_the_symmetric_loss():
    """The symmetric search at p = 0 scores the plain symmetric quantizer:
    its loss is || X (dequant(Q_sym(W)) - W)^T ||_F^2 computed directly, and
    a nonzero clip changes the loss."""
    lay = synth.make_layer(64, 256, 256, seed=[165], w_std=0.02, salient_frac=0.01)
    w, x = lay["w"], lay["x"]
    lc, _ = oracle.clip_search(w, x, 128, [0.0, 0.02], symmetric=True)
    qw, sc, zr = oracle.quantize_symmetric(w, 128)
    d = oracle.dequantize(qw, sc, zr, 128, 256) - np.asarray(w, np.float64)
    e = np.asarray(x, np.float64) @ d.T
    assert lc[0] == pytest.approx(float(np.sum(e * e)), rel=1e-10)
    la, _ = oracle.clip_search(w, x, 128, [0.0])
    assert lc[0] != la[0] and lc[1] != lc[0]
