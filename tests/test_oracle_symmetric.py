"""Pins of the oracle's symmetric INT4 quantizer (aissn.com "对称/非对称量化":
symmetric means zero-point 0). The reading: the group's largest magnitude a
maps to +-7, s32 = max(a, 1e-5) / 7 in fp32, the fp16-stored scale makes the
codes, q = clamp(rint(w / s16), -8, 7), stored as q + 8 with zero-point 8.
"""

import numpy as np
import pytest

import oracle
import synth


def test_hand_worked_group():
    """Group [-1, 1, 0.5, -0.5, 0.25, 0, 0, ...] (G = 128), by hand:
    1/7 in fp32 = 0.14285715 = 1.1428572 * 2^-3; the fp16 mantissa
    0.1428572 * 1024 = 146.29 rounds to 146, so s16 = 1.142578125 * 2^-3
    = 0.142822265625 (bits 0x3092). Then w / s16 = 1 / 0.142822265625
    = 7.0017 -> 7 -> code 15; 0.5 -> 3.50085 -> 4 -> code 12 (x_hat
    0.5712890625); -1 -> code 1; -0.5 -> code 4; 0.25 -> 1.75 -> 2 -> code
    10; 0 -> code 8."""
    w = np.zeros((1, 128), dtype=np.float16)
    w[0, :6] = [-1.0, 1.0, 0.5, -0.5, 0.25, 0.0]
    codes, s16, z16 = oracle.group_quantize_symmetric(w, 128)
    assert s16.view(np.uint16)[0, 0] == 0x3092
    assert float(s16[0, 0]) == 0.142822265625
    assert float(z16[0, 0]) == 8.0
    assert list(codes[0, :6]) == [1, 15, 12, 4, 10, 8]
    assert np.all(codes[0, 6:] == 8)
    qw, sc, zr = oracle.quantize_symmetric(w, 128)
    w_hat = oracle.dequantize(qw, sc, zr, 128, 128)
    assert w_hat[0, 2] == 0.5712890625
    assert w_hat[0, 1] == 0.999755859375 and w_hat[0, 0] == -0.999755859375


@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_odd_symmetry_and_no_clipping(G):
    """q(-w) = -q(w) exactly (RNE is odd), so codes(-W) = 16 - codes(W) with
    the same scales; no code is clipped, so |w - x_hat| <= s16 / 2 (up to the
    fp32 rounding of w / s16) everywhere, codes stay in 1..15 and every
    zero-point is 8."""
    lay = synth.make_layer(64, 1024, 0, seed=[140, G], w_std=0.02, salient_frac=0.01)
    w = lay["w"]
    c1, s1, z1 = oracle.group_quantize_symmetric(w, G)
    c2, s2, z2 = oracle.group_quantize_symmetric(-w, G)
    assert np.array_equal(s1.view(np.uint16), s2.view(np.uint16))
    assert np.array_equal(c2.astype(int), 16 - c1.astype(int))
    assert c1.min() >= 1 and c1.max() <= 15
    assert np.all(z1 == 8) and np.all(z2 == 8)
    qw = oracle.pack_codes(c1)
    w_hat = oracle.dequantize(qw, s1, z1, G, w.shape[1])
    sf = np.repeat(s1.astype(np.float64), G, axis=1)
    err = np.abs(w.astype(np.float64) - w_hat)
    assert np.all(err <= sf / 2 * (1 + 2.0 ** -20))
    # the largest magnitude of each group lands on code 1 or 15
    wg = np.abs(w.astype(np.float32)).reshape(64, -1, G)
    cg = c1.reshape(64, -1, G)
    top = np.take_along_axis(cg, wg.argmax(axis=2)[:, :, None], axis=2)[:, :, 0]
    assert np.all((top == 1) | (top == 15))


@pytest.mark.parametrize("j", [-3, 2])
def test_symmetric_power_of_two_equivariance(j):
    """Scaling W by 2^j scales a, s32 and s16 by 2^j exactly (no fp16
    overflow or underflow at these magnitudes), so the codes are identical."""
    lay = synth.make_layer(32, 512, 0, seed=[141, j + 8], w_std=0.02)
    w = lay["w"].astype(np.float32)
    w[np.abs(w) < 1e-3] = 0.0          # keep w * 2^j exact in fp16 (no subnormals)
    assert np.array_equal((w * 2.0 ** j).astype(np.float16).astype(np.float32), w * 2.0 ** j)
    c1, s1, _ = oracle.group_quantize_symmetric(w.astype(np.float16), 128)
    c2, s2, _ = oracle.group_quantize_symmetric((w * 2.0 ** j).astype(np.float16), 128)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2.astype(np.float64), s1.astype(np.float64) * 2.0 ** j)


def test_constant_zero_group_uses_floor():
    w = np.zeros((2, 128), dtype=np.float16)
    codes, s16, z16 = oracle.group_quantize_symmetric(w, 64)
    assert np.all(codes == 8) and np.all(z16 == 8)
    assert np.all(s16 == np.float16(np.float32(1e-5) / np.float32(7)))
