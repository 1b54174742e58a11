"""awq_gemm_grouped: layers that read the same activations (a decoder
layer's q / k / v and gate / up projections, which the rskf.cn AWQ
article's deployment fuses, §3.4) in one GEMV launch over their stacked
rows, each layer kept as its own tensors.

Every y_i meets the linear-layer bar against the oracle (relative Frobenius
error <= 1e-3 and |y - y_ref| <= 1e-2 * (|y_ref| + 1) per element), and
outputs packed side by side in one buffer show that no layer writes past its
own rows. At M <= 2 (one GEMV launch) each y_i also equals the layer's own
awq_gemm result bit for bit (the same per-row arithmetic in the same order);
at 3 <= M <= 32 (one column-tile launch) the stacked rows set the tile and
wave counts, so only repeatability is exact; larger batches run the layers
one awq_gemm call each, with the same bits.
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import weight_only_int4_quantize_amd as awq  # noqa: E402

from test_gpu_parity import assert_linear_close, dev, host, say  # noqa: E402


def layers_of(Ns, K, M, G, seed):
    """Layers with weights of their own seeds and one shared x."""
    lays = [synth.make_layer(N, K, 0, seed=[230, seed, j, N, K], w_std=0.02) for j, N in enumerate(Ns)]
    x = synth.make_layer(1, K, M, seed=[231, seed, M, K], w_std=0.02)["x"]
    qs = [oracle.quantize(lay["w"], G) for lay in lays]
    return x, qs


def run_grouped(x, qs, G):
    xd = dev(x)
    dl = [(dev(q[0].view(np.int32)), dev(q[1]), dev(q[2])) for q in qs]
    M = x.shape[0]
    Ns = [q[0].shape[0] for q in qs]
    # outputs side by side in one buffer between sentinels
    total = sum(M * N for N in Ns)
    buf = torch.full((total + 2048,), 7.0, dtype=torch.float16, device="cuda")
    outs, off = [], 1024
    for N in Ns:
        outs.append(buf[off:off + M * N].view(M, N))
        off += M * N
    awq.awq_gemm_grouped(xd, dl, G, outs=outs)
    singles = [awq.awq_gemm(xd, *d, G) for d in dl]
    torch.cuda.synchronize()
    b = host(buf)
    assert np.all(b[:1024] == 7.0) and np.all(b[1024 + total:] == 7.0)
    return [host(o) for o in outs], [host(s) for s in singles]


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("Ns", [(4096, 4096, 4096), (11008, 11008)], ids=["qkv", "gate_up"])
def test_decode_projections(Ns, M):
    K, G = 4096, 128
    say("grouped", Ns, K, M)
    x, qs = layers_of(Ns, K, M, G, 0)
    got, singles = run_grouped(x, qs, G)
    for q, g, s in zip(qs, got, singles):
        assert np.array_equal(g.view(np.uint16), s.view(np.uint16))
        assert_linear_close(g, oracle.linear_ref(x, *q, G))


@pytest.mark.parametrize("Ns,K,G,M", [
    ((100, 37, 0, 1000), 512, 64, 1),     # ragged layers, one empty
    ((1, 2, 3), 1536, 128, 2),            # rows fewer than a wave's
    ((1000, 3000), 11008, 128, 1),        # long rows: the persistent form
    ((777,), 4096, 32, 2),                # one layer
    ((300, 500, 700, 900), 2048, 256, 1), # four layers
    ((512, 512, 512), 11008, 128, 1),     # a split layer's q/k/v share: one-shot, three items per row
    ((512, 512, 512), 11008, 128, 2),     # the same at two rows of x
    ((1376, 1376), 5120, 64, 1),          # two items per row, one-shot
    ((640, 640, 640, 640), 13824, 128, 1),# stacked past one round (persistent), each alone one-shot
])
def test_ragged_layers(Ns, K, G, M):
    say("grouped ragged", Ns, K, G, M)
    x, qs = layers_of(Ns, K, M, G, 1)
    got, singles = run_grouped(x, qs, G)
    for q, g, s in zip(qs, got, singles):
        assert np.array_equal(g.view(np.uint16), s.view(np.uint16))
        if q[0].shape[0]:
            assert_linear_close(g, oracle.linear_ref(x, *q, G))


def run_grouped_twice(x, qs, G):
    """The grouped call's outputs (between sentinels) and whether a second
    call gives the same bits."""
    got, _ = run_grouped(x, qs, G)
    again, _ = run_grouped(x, qs, G)
    same = all(np.array_equal(a.view(np.uint16), b.view(np.uint16)) for a, b in zip(got, again))
    return got, same


@pytest.mark.parametrize("M", [4, 16])
@pytest.mark.parametrize("Ns", [(4096, 4096, 4096), (11008, 11008)], ids=["qkv", "gate_up"])
def test_batched_decode_projections(Ns, M):
    """3 <= M <= 32: one column-tile launch over the stacked layers, each
    layer on whole blocks of its own columns. The tile and wave counts follow
    the stacked rows, so the waves' K ranges (and the fp32 summation order)
    may differ from a single-layer call: each layer meets the linear-layer bar
    against the oracle, and repeated calls give the same bits."""
    K, G = 4096, 128
    say("grouped batched", Ns, K, M)
    x, qs = layers_of(Ns, K, M, G, 3)
    got, same = run_grouped_twice(x, qs, G)
    assert same
    for q, g in zip(qs, got):
        assert_linear_close(g, oracle.linear_ref(x, *q, G))


@pytest.mark.parametrize("Ns,K,G,M", [
    ((100, 37, 0, 1000), 512, 64, 3),      # ragged layers, one empty
    ((5, 17, 33), 1024, 32, 8),            # layers narrower than one tile
    ((777, 1500), 6144, 256, 16),          # G = 256
    ((300, 500, 700, 900), 2048, 128, 32), # four layers, 32 rows of x
    ((2000, 3000, 1000), 4096, 128, 12),   # several tiles per block, from the stacked rows
    ((512, 512, 512), 11008, 128, 4),      # few rows at 4 rows of x (alone each the GEMV): stacked column tiles
])
def test_batched_ragged_layers(Ns, K, G, M):
    say("grouped batched ragged", Ns, K, G, M)
    x, qs = layers_of(Ns, K, M, G, 4)
    got, same = run_grouped_twice(x, qs, G)
    assert same
    for q, g in zip(qs, got):
        if q[0].shape[0]:
            assert_linear_close(g, oracle.linear_ref(x, *q, G))


@pytest.mark.parametrize("M", [40, 64])
def test_batches_past_the_column_tiles_run_per_layer(M):
    """M > 32: one awq_gemm per layer, with its bits."""
    Ns, K, G = (4096, 1024), 4096, 128
    x, qs = layers_of(Ns, K, M, G, 2)
    got, singles = run_grouped(x, qs, G)
    for q, g, s in zip(qs, got, singles):
        assert np.array_equal(g.view(np.uint16), s.view(np.uint16))
        assert_linear_close(g, oracle.linear_ref(x, *q, G))



def _carve(buf, off, arr, dtype):
    """A view of `buf` at byte offset `off` holding a copy of arr."""
    a = np.ascontiguousarray(arr)
    t = buf[off:off + a.nbytes].view(dtype).view(a.shape)
    t.copy_(torch.from_numpy(a).view(dtype))
    return t


def _place(x, qs, gap):
    """x and each layer's (qweight, scales, zeros) carved from one buffer:
    x and layer 0 first, layers 1.. from byte `gap` on (gap 0: all packed
    one after another)."""
    step = lambda n: (n + 255) // 256 * 256
    sizes = [sum(step(a.nbytes) for a in q) for q in qs]
    head = step(x.nbytes) + sizes[0]
    total = max(head, gap) + sum(sizes[1:]) + 256
    try:
        buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    except RuntimeError as e:   # a box without that much free device memory
        pytest.skip(f"could not allocate {total} bytes: {e}")
    xd = _carve(buf, 0, x, torch.float16)
    off, layers = step(x.nbytes), []
    for j, q in enumerate(qs):
        if j == 1:
            off = max(off, gap)
        o = off
        qw = _carve(buf, o, q[0].view(np.int32), torch.int32)
        o += step(q[0].nbytes)
        sc = _carve(buf, o, q[1], torch.float16)
        o += step(q[1].nbytes)
        zr = _carve(buf, o, q[2], torch.float16)
        layers.append((qw, sc, zr))
        off += sizes[j]
    return buf, xd, layers


# Layers past 64 GiB of the lowest tensor take the full-pointer entries
FAR = 65 << 30


def _span(ts):
    ptrs = [t.data_ptr() for t in ts]
    return max(ptrs) - min(ptrs)


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("Ns", [(4096, 4096, 4096), (11008, 11008)], ids=["qkv", "gate_up"])
def test_grouped_both_argument_forms(Ns, M):
    """One-shot grouped launches pass every early pointer as a 32-bit offset
    (16-byte units) from the lowest when x and all layers' weights, scales
    and zero-points lie within 64 GiB of it, and as full pointers otherwise.
    The same layers placed both ways (carved from one buffer, packed or
    65 GiB apart) give the same bits, equal to each layer's own awq_gemm."""
    K, G = 4096, 128
    x, qs = layers_of(Ns, K, M, G, 5)
    results = []
    for gap in (0, FAR):
        buf, xd, layers = _place(x, qs, gap)
        span = _span([xd] + [t for d in layers for t in d])
        say("grouped argument forms: gap", gap, "span", span)
        assert (span < (1 << 36)) == (gap == 0)
        outs = [torch.empty((M, N), dtype=torch.float16, device="cuda") for N in Ns]
        awq.awq_gemm_grouped(xd, layers, G, outs=outs)
        singles = [awq.awq_gemm(xd, *d, G) for d in layers]
        torch.cuda.synchronize()
        results.append(([host(o) for o in outs], [host(t) for t in singles]))
        del buf, xd, layers
    for j, q in enumerate(qs):
        near, far, single = results[0][0][j], results[1][0][j], results[0][1][j]
        assert np.array_equal(near.view(np.uint16), single.view(np.uint16))
        assert np.array_equal(far.view(np.uint16), single.view(np.uint16))
        assert_linear_close(near, oracle.linear_ref(x, *q, G))


@pytest.mark.parametrize("M", [4, 16])
@pytest.mark.parametrize("Ns", [(4096, 4096, 4096), (11008, 11008)], ids=["qkv", "gate_up"])
def test_grouped_column_tiles_both_argument_forms(Ns, M):
    """The grouped column-tile launch (3 <= M <= 32) has the same two
    argument forms: 32-bit offsets (16-byte units) from the lowest tensor
    when a launch's tensors lie within 64 GiB, full pointers otherwise. The
    same layers placed both ways give the same bits, and each layer meets
    the linear bar."""
    K, G = 4096, 128
    x, qs = layers_of(Ns, K, M, G, 6)
    results = []
    for gap in (0, FAR):
        buf, xd, layers = _place(x, qs, gap)
        assert (_span([xd] + [t for d in layers for t in d]) < (1 << 36)) == (gap == 0)
        outs = [torch.empty((M, N), dtype=torch.float16, device="cuda") for N in Ns]
        awq.awq_gemm_grouped(xd, layers, G, outs=outs)
        torch.cuda.synchronize()
        results.append([host(o) for o in outs])
        del buf, xd, layers
    for j, q in enumerate(qs):
        assert np.array_equal(results[0][j].view(np.uint16), results[1][j].view(np.uint16))
        assert_linear_close(results[0][j], oracle.linear_ref(x, *q, G))
