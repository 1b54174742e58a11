"""Clip step and clip search (xxmr.cn §1.5: cut the extreme p of each
group's values at both ends before the scale is taken; the fraction chosen
by the scale search's output loss).

Clipped quantize: bit-exact against the oracle for every group size, both
maps, with and without channel scales, including groups full of ties.
Clip search: the scale search's bar. The oracle's best index, unless its two
lowest losses lie within 1e-6 relative (then either of them); losses within
1e-4 of the exact oracle and 2e-6 of its fp16-activation form.
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import assert_quant_equal, check_choice, dev, host, say  # noqa: E402

FRACTIONS = [0.0, 0.001, 0.002, 0.005, 0.01, 0.02, 0.05, 0.1, 0.2]


def gpu_quantize(w16, G, p, cs=None, symmetric=False):
    qw, sc, zr = awq.awq_quantize(dev(w16), G, None if cs is None else dev(cs.astype(np.float32)),
                                  symmetric=symmetric, clip_fraction=p)
    torch.cuda.synchronize()
    return host(qw).view(np.uint32), host(sc), host(zr)


def heavy_tailed(N, K, seed, scale=0.02):
    """Student-t (3 degrees of freedom) weights: a few large values per group,
    the case the clip step is for."""
    rng = np.random.default_rng(seed)
    return (rng.standard_t(3, size=(N, K)) * scale).astype(np.float16)


@pytest.mark.parametrize("G", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("symmetric", [False, True])
@pytest.mark.parametrize("p", [0.01, 0.05, 0.2])
def test_clipped_quantize_bit_exact(G, symmetric, p):
    w = heavy_tailed(600, 2048, [180, G, int(symmetric)])
    say("clipped quantize G", G, "sym" if symmetric else "asym", "p", p)
    assert_quant_equal(gpu_quantize(w, G, p, symmetric=symmetric),
                       oracle.quantize_clipped(w, G, p, symmetric=symmetric))


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("symmetric", [False, True])
def test_clipped_quantize_with_channel_scale(G, symmetric):
    lay = synth.make_layer(1000, 2048, 0, seed=[181, G], w_std=0.02, salient_frac=0.01)
    rng = np.random.default_rng([182, G])
    cs = (np.abs(rng.standard_normal(2048)) + 0.1).astype(np.float32)
    for p in (0.003, 0.01, 0.1):
        say("clipped quantize scaled G", G, "p", p)
        assert_quant_equal(gpu_quantize(lay["w"], G, p, cs, symmetric),
                           oracle.quantize_clipped(lay["w"], G, p, cs, symmetric))


@pytest.mark.parametrize("G", [32, 128, 256])
def test_clipped_quantize_ties_and_constant_groups(G):
    """Values on a coarse grid (many equal order statistics), whole groups
    of one value, and an all-zero row: the rank selection must pick the
    same order statistics as a sort."""
    rng = np.random.default_rng([183, G])
    N, K = 96, 1024
    w = (rng.integers(-3, 4, size=(N, K)) * 0.125).astype(np.float16)
    w[5, :G] = np.float16(0.25)
    w[7, G:2 * G] = np.float16(-1.5)
    w[9, :] = 0
    w[11, :] = np.float16(3.0)
    for p in (0.0, 0.01, 0.1, 0.24):
        for sym in (False, True):
            say("ties G", G, "p", p, "sym" if sym else "asym")
            assert_quant_equal(gpu_quantize(w, G, p, symmetric=sym),
                               oracle.quantize_clipped(w, G, p, symmetric=sym))


def test_clipped_quantize_full_size():
    """The decode layer's weight (11008 x 4096, G = 128) at p = 1 %."""
    lay = synth.decode_layer(11008, 4096, 0, 128)
    say("clipped quantize full size")
    assert_quant_equal(gpu_quantize(lay["w"], 128, 0.01), oracle.quantize_clipped(lay["w"], 128, 0.01))


def test_zero_clip_is_the_plain_kernel():
    lay = synth.decode_layer(4096, 4096, 0, 128)
    wd = dev(lay["w"])
    a = awq.awq_quantize(wd, 128)
    b = awq.awq_quantize(wd, 128, clip_fraction=0.0)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def check_clip_search(losses, best, losses_o, best_o, losses_f16=None):
    """The scale search's bar (check_choice): the oracle's index unless its
    two lowest losses are a near-tie; losses within the stated tolerances
    of the exact oracle and of its fp16-activation form."""
    check_choice(losses, best, losses_o, best_o, losses_f16)


@pytest.mark.parametrize("G", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("symmetric", [False, True])
def test_clip_search_matches_oracle(G, symmetric):
    N, K, T = 512, 1024, 512
    w = heavy_tailed(N, K, [184, G])
    x = np.random.default_rng([185, G]).standard_normal((T, K)).astype(np.float16)
    say("clip search G", G, "sym" if symmetric else "asym")
    losses, best = awq.awq_clip_search(dev(w), dev(x), FRACTIONS, G, symmetric=symmetric)
    losses_o, best_o = oracle.clip_search(w, x, G, FRACTIONS, symmetric=symmetric)
    losses_f, _ = oracle.clip_search(w, x, G, FRACTIONS, symmetric=symmetric, f16_activations=True)
    say("gpu best", best, "oracle best", best_o)
    check_clip_search(losses, best, losses_o, best_o, losses_f)


@pytest.mark.parametrize("symmetric", [False, True])
def test_clip_search_with_channel_scale(symmetric):
    """After the scale search: the clip is searched on W diag(s) against
    X / s, the loss measured against the unquantized W X^T."""
    lay = synth.make_layer(768, 1024, 640, seed=[186], w_std=0.02, salient_frac=0.01)
    w, x = lay["w"], lay["x"]
    s32 = oracle.channel_scales(oracle.activation_absmean(x), 0.5)
    say("clip search scaled", "sym" if symmetric else "asym")
    losses, best = awq.awq_clip_search(dev(w), dev(x), FRACTIONS, 128, channel_scale=dev(s32),
                                       symmetric=symmetric)
    losses_o, best_o = oracle.clip_search(w, x, 128, FRACTIONS, s32=s32, symmetric=symmetric)
    losses_f, _ = oracle.clip_search(w, x, 128, FRACTIONS, s32=s32, symmetric=symmetric, f16_activations=True)
    say("gpu best", best, "oracle best", best_o)
    check_clip_search(losses, best, losses_o, best_o, losses_f)


def test_clip_search_ragged_tokens_and_reused_workspace():
    """T not a multiple of any tile, N not a multiple of 256, and one
    workspace used by two searches of different sizes in a row."""
    G = 128
    w1, w2 = heavy_tailed(300, 768, [187]), heavy_tailed(130, 512, [188])
    x1 = np.random.default_rng([189]).standard_normal((333, 768)).astype(np.float16)
    x2 = np.random.default_rng([190]).standard_normal((77, 512)).astype(np.float16)
    fr = [0.0, 0.01, 0.05]
    L = awq.load()
    nbytes = L.awq_clip_search_workspace_bytes(300, 768, 333, G, len(fr), 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for w, x in ((w1, x1), (w2, x2)):
        say("clip search ragged", w.shape, x.shape)
        losses, best = awq.awq_clip_search(dev(w), dev(x), fr, G, workspace=ws)
        losses_o, best_o = oracle.clip_search(w, x, G, fr)
        check_clip_search(losses, best, losses_o, best_o)
