"""Pins of the oracle's W8A16 form (aissn.com "INT8 vs INT4" and "INT8 实战":
8-bit weights with fp16 activations; the affine map of xxmr.cn §1.2 with
bits = 8)."""

import numpy as np
import pytest

import oracle
import synth


@pytest.mark.parametrize("G", [32, 128])
def test_general_width_reproduces_the_int4_quantizers(G):
    """The width-generic quantizer at bits = 4 equals the two INT4
    quantizers, which are written separately."""
    lay = synth.make_layer(200, 1024, 0, seed=[200, G], w_std=0.02)
    for sym, ref in ((False, oracle.group_quantize), (True, oracle.group_quantize_symmetric)):
        got = oracle.group_quantize_bits(lay["w"], G, 4, symmetric=sym)
        exp = ref(lay["w"], G)
        for a, b in zip(got, exp):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def test_worked_example_at_8_bits():
    """xxmr.cn §1.2's example (range [-1, 1], value 0.5) with 256 levels,
    by hand: scale 2/255 = 0.00784313... rounds to fp16 1.00390625 * 2^-7
    (bits 0x2004); zero = rint(1 / 0.0078430176) = rint(127.502) = 128;
    0.5 -> rint(63.751) + 128 = 192 -> (192 - 128) * s = 0.501953125;
    1.0 -> rint(127.502) + 128 = 256, clamped to 255; -1.0 -> 0."""
    w = np.zeros((1, 128), dtype=np.float16)
    w[0, :4] = [-1.0, 1.0, 0.5, 0.0]
    codes, s16, z16 = oracle.group_quantize_bits(w, 128, 8)
    assert s16.view(np.uint16)[0, 0] == 0x2004
    assert float(z16[0, 0]) == 128.0
    assert codes[0, :4].tolist() == [0, 255, 192, 128]
    qw = oracle.pack_codes8(codes)
    w_hat = oracle.dequantize_w8(qw, s16, z16, 128, 128)
    assert w_hat[0, 2] == 0.501953125


def test_pack_order():
    codes = np.array([[0x01, 0x23, 0x45, 0x67, 0x89, 0xAB, 0xCD, 0xEF]], dtype=np.uint8)
    qw = oracle.pack_codes8(codes)
    assert qw.tolist() == [[0x67452301, 0xEFCDAB89]]
    assert np.array_equal(oracle.unpack_codes8(qw, 8), codes)


def test_error_bound_and_symmetry():
    lay = synth.make_layer(64, 512, 0, seed=[201], w_std=0.02, salient_frac=0.0)
    w64 = lay["w"].astype(np.float64)
    qw, sc, zr = oracle.quantize_w8(lay["w"], 128)
    err = np.abs(oracle.dequantize_w8(qw, sc, zr, 128, 512) - w64)
    s = np.repeat(sc.astype(np.float64), 128, axis=1)
    # asymmetric: within half a step (plus the fp16 scale's rounding over
    # at most 255 steps) wherever the zero-point was not clamped
    assert np.all(err <= 0.5 * s + 255 * s * 2.0 ** -11 + 1e-12)
    # symmetric map is odd: code(-w) - 128 = -(code(w) - 128)
    c1, _, _ = oracle.group_quantize_bits(lay["w"], 128, 8, symmetric=True)
    c2, _, _ = oracle.group_quantize_bits(-lay["w"], 128, 8, symmetric=True)
    assert np.array_equal(c1.astype(np.int32) - 128, -(c2.astype(np.int32) - 128))
    # 8 bits resolve 17x finer than 4 on the same groups
    qw4, sc4, zr4 = oracle.quantize(lay["w"], 128)
    err4 = np.abs(oracle.dequantize(qw4, sc4, zr4, 128, 512) - w64)
    assert err.max() < err4.max() / 8


def test_constant_group_and_brute_force_linear():
    rng = np.random.default_rng(202)
    w = (rng.standard_normal((3, 64)) * 0.1).astype(np.float16)
    w[1, :32] = np.float16(0.25)                       # a constant group
    x = rng.standard_normal((2, 64)).astype(np.float16)
    qw, sc, zr = oracle.quantize_w8(w, 32)
    codes = oracle.unpack_codes8(qw, 64)
    y = np.zeros((2, 3))
    for m in range(2):
        for n in range(3):
            y[m, n] = sum(float(x[m, k]) * (float(codes[n, k]) - float(zr[n, k // 32])) * float(sc[n, k // 32])
                          for k in range(64))
    np.testing.assert_allclose(oracle.linear_ref_w8(x, qw, sc, zr, 32), y, rtol=1e-12, atol=1e-12)
    # a constant positive group is the map's degenerate case: the range is
    # floored to 1e-5, the scale is fp16(1e-5 / 255), the zero-point clamps
    # to 0 and every code clamps to 255 (a range that does not contain 0
    # cannot be represented; groups of real weights always straddle 0)
    assert sc.view(np.uint16)[1, 0] == np.float16(np.float32(1e-5) / np.float32(255)).view(np.uint16)
    assert float(zr[1, 0]) == 0.0
    assert np.all(codes[1, :32] == 255)
