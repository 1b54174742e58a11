"""Pins of the oracle's mixed-precision form (blog.ohmyagent.ai "技术实现" 1
and "混合精度设计": the important 1 % of the weights, picked from the
activation distribution, stay in fp16 while the rest is quantized to 4 bits;
xxmr.cn §2.2)."""

import numpy as np
import pytest

import oracle
import synth


def test_selection_hand_worked():
    # descending m, equal m by ascending channel
    m = np.array([0.5, 2.0, 2.0, 1.0, 3.0, 2.0])
    assert oracle.salient_channels(m, 4).tolist() == [4, 1, 2, 5]
    assert oracle.salient_channels(m, 0).tolist() == []
    assert sorted(oracle.salient_channels(m, 6).tolist()) == list(range(6))
    with pytest.raises(ValueError):
        oracle.salient_channels(m, 7)


def test_selection_matches_lexsort_with_ties():
    rng = np.random.default_rng(170)
    m = rng.integers(0, 20, size=1000).astype(np.float64) / 4.0     # many ties
    order = np.lexsort((np.arange(m.size), -m))
    for n in (1, 10, 137, 1000):
        assert np.array_equal(oracle.salient_channels(m, n), order[:n])


def test_count_reading():
    assert oracle.salient_count(4096) == 41
    assert oracle.salient_count(11008) == 110
    assert oracle.salient_count(50) == 0


@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("symmetric", [False, True])
def test_stored_form_is_the_pages_recipe(G, symmetric):
    """Quantize everything, dequantize, put the original values back in the
    salient columns (the recipe read literally) == the stored form's
    effective weight (codes at the zero-point plus the fp16 side columns)."""
    lay = synth.make_layer(96, 1024, 0, seed=[171, G], w_std=0.02)
    idx = np.random.default_rng([172, G]).choice(1024, 17, replace=False)
    qw, sc, zr, ws = oracle.quantize_salient(lay["w"], G, idx, symmetric)
    lit = oracle.mixed_weight(lay["w"], G, idx, symmetric)
    assert np.array_equal(oracle.dequantize_salient(qw, sc, zr, G, 1024, idx, ws), lit)
    # outside the salient columns nothing changed: same scales, zeros, codes
    qw0, sc0, zr0 = (oracle.quantize_symmetric if symmetric else oracle.quantize)(lay["w"], G)
    assert np.array_equal(sc.view(np.uint16), sc0.view(np.uint16))
    assert np.array_equal(zr.view(np.uint16), zr0.view(np.uint16))
    c, c0 = oracle.unpack_codes(qw, 1024), oracle.unpack_codes(qw0, 1024)
    rest = np.setdiff1d(np.arange(1024), idx)
    assert np.array_equal(c[:, rest], c0[:, rest])
    # the INT4 part of a salient column is exactly zero; its fp16 part is W
    w_int = oracle.dequantize(qw, sc, zr, G, 1024)
    assert np.all(w_int[:, idx] == 0)
    assert np.array_equal(ws, lay["w"][:, idx].T)


def test_linear_brute_force():
    rng = np.random.default_rng(173)
    N, K, M, G = 5, 64, 3, 32
    w = (rng.standard_normal((N, K)) * 0.1).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    idx = np.array([7, 40, 3])
    qw, sc, zr, ws = oracle.quantize_salient(w, G, idx)
    codes = oracle.unpack_codes(qw, K)
    y = np.zeros((M, N))
    for mm in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                if k in idx:
                    wk = float(w[n, k])
                else:
                    g = k // G
                    wk = (float(codes[n, k]) - float(zr[n, g])) * float(sc[n, g])
                acc += float(x[mm, k]) * wk
            y[mm, n] = acc
    np.testing.assert_allclose(oracle.linear_salient_ref(x, qw, sc, zr, G, idx, ws), y, rtol=1e-12, atol=1e-12)


def test_loss_limits_and_forms():
    lay = synth.make_layer(64, 512, 384, seed=[174], w_std=0.02)
    w, x = lay["w"], lay["x"]
    # no salient channel: the plain (RTN) loss, alpha = 0 of the scale search
    l0 = oracle.salient_loss(w, x, 128, [])
    losses, _, _ = oracle.scale_search(w, x, 128, alphas=[0.0])
    assert l0 == pytest.approx(losses[0], rel=1e-12)
    # every channel salient: the layer is exact
    assert oracle.salient_loss(w, x, 128, np.arange(512)) == 0.0
    # Gram form == direct form
    idx = oracle.salient_channels(oracle.activation_absmean(x), 5)
    assert oracle.salient_loss(w, x, 128, idx) == pytest.approx(
        oracle.salient_loss(w, x, 128, idx, use_gram=False), rel=1e-10)


def test_planted_channels_are_found_and_help():
    """The generator scales 1 % of the input channels' activations by 20:
    they are exactly the channels the selection picks, and keeping them in
    fp16 lowers the output loss below plain RTN."""
    lay = synth.make_layer(128, 1024, 512, seed=[175], w_std=0.02)
    n = oracle.salient_count(1024)
    idx = oracle.salient_channels(oracle.activation_absmean(lay["x"]), n)
    assert np.array_equal(np.sort(idx), lay["salient"])
    l_mix = oracle.salient_loss(lay["w"], lay["x"], 128, idx)
    l_rtn = oracle.salient_loss(lay["w"], lay["x"], 128, [])
    assert l_mix < 0.5 * l_rtn
