"""Oracle pins for the two other gradient sources of the step: a stored
reduce-scatter output (ZeRO-2 with the collective run on its own, one summed
buffer per rank) and a gradient all-reduced in full (ZeRO-1, each rank reading
its own range of the full flat vector)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import casts as C
from oracle import plan as P
from oracle import step as O

F = np.float32


@pytest.mark.parametrize("psi,N", [(10, 4), (19_210, 4), (1_000_003, 8), (3, 5)])
def test_read_pieces_flat_closed_form(psi, N):
    """One flat bucket: rank r owns [r*S, (r+1)*S) of the vector padded to
    ceil(psi/N)*N (the handbook's flatten / pad / split), so reading a full
    buffer whose entry i is i gives exactly that range."""
    pl = P.make_plan([psi], N)
    S = -(-psi // N)
    full = np.arange(S * N, dtype=np.int64)
    for r in range(N):
        got = O.read_pieces(full, P.rank_segments(pl, r))
        assert np.array_equal(got, np.arange(r * S, (r + 1) * S))


@pytest.mark.parametrize("sizes,N,cap", [([7, 0, 30, 5, 5, 1], 3, 12), ([1] * 50, 7, 6),
                                         (list(range(1, 300)), 5, 1000), ([4099] * 9, 4, 5000)])
def test_read_pieces_cover_the_full_buffer_once(sizes, N, cap):
    """With buckets, the N ranks' pieces tile the padded buffer exactly once, and
    writing what was read back into an empty buffer rebuilds it."""
    pl = P.make_plan(sizes, N, cap)
    NS = pl.padded_numel
    full = np.arange(NS, dtype=np.int64)
    seen = np.zeros(NS, np.int64)
    rebuilt = np.full(NS, -1, np.int64)
    for r in range(N):
        segs = P.rank_segments(pl, r)
        got = O.read_pieces(full, segs)
        assert got.size == pl.shard_numel
        seen[got] += 1
        O.write_gather(rebuilt, segs, got)
    assert np.all(seen == 1)
    assert np.array_equal(rebuilt, full)


def _padded_grads(rng, pl, sizes, N):
    NS = pl.padded_numel
    pad = np.ones(NS, bool)
    for i, n in enumerate(sizes):
        pad[pl.tensor_offset[i]:pl.tensor_offset[i] + n] = False
    grads = [rng.normal(0, 1e-2, NS).astype(F) for _ in range(N)]
    for g in grads:
        g[pad] = 0
    master = rng.normal(0, 0.05, NS).astype(F)
    master[pad] = 0
    return grads, master, pad


@pytest.mark.parametrize("sizes,N,cap", [([3_333, 3_334, 3_333], 4, 0), ([1_000, 2_500, 700, 800], 8, 1_500)])
def test_zero1_union_equals_unsharded(sizes, N, cap):
    """ZeRO-1: every rank reads its range of the all-reduced (SUM) full gradient,
    divides by N and steps its shard; the gathered result is the unsharded step
    on the averaged gradient, bit for bit, and equals the ZeRO-2 step that sums
    the N ranks' pieces itself."""
    rng = np.random.default_rng(len(sizes) * 100 + N)
    pl = P.make_plan(sizes, N, cap)
    NS = pl.padded_numel
    grads, master, pad = _padded_grads(rng, pl, sizes, N)
    total = O.reduce_slices(grads, "f32")                      # the all-reduce (SUM)
    m = np.zeros(NS, F)
    v = np.zeros(NS, F)
    gather = np.zeros(NS, F)
    kw = dict(lr=1e-2, weight_decay=0.1, t=1)
    for r in range(N):
        segs = P.rank_segments(pl, r)
        p_r = O.read_pieces(master, segs)
        z = np.zeros_like(p_r)
        one = O.shard_step([O.read_pieces(total, segs)], "f32", "f32", N, p_r, z, z, **kw)
        two = O.shard_step([O.read_pieces(g, segs) for g in grads], "f32", "f32", N, p_r, z, z, **kw)
        assert np.array_equal(one.master.view(np.uint32), two.master.view(np.uint32))
        O.write_gather(gather, segs, one.params)
    whole = O.shard_step([O.average(total, N)], "f32", "f32", 1, master, m, v, **kw)
    assert np.array_equal(gather.view(np.uint32), whole.params.view(np.uint32))
    assert np.all(gather[pad].view(np.uint32) == 0)


@pytest.mark.parametrize("N", [2, 8, 64])
def test_stored_fp32_rs_output_equals_fused(N):
    """An fp32 reduce-scatter output, stored and then stepped (one buffer, divided
    by N), gives the fused step's result bit for bit when the collective summed
    in the same order."""
    rng = np.random.default_rng(N)
    S = 1_000
    slices = [rng.normal(0, 1e-3, S).astype(F) for _ in range(N)]
    p = rng.normal(0, 0.02, S).astype(F)
    m = rng.normal(0, 1e-4, S).astype(F)
    v = np.abs(rng.normal(0, 1e-6, S)).astype(F)
    kw = dict(lr=3e-4, weight_decay=0.1, t=7)
    fused = O.shard_step(slices, "f32", "f32", N, p, m, v, **kw)
    rs = O.reduce_slices(slices, "f32")
    stored = O.shard_step([rs], "f32", "f32", N, p, m, v, **kw)
    for a, b in ((fused.master, stored.master), (fused.m, stored.m), (fused.v, stored.v)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("kind", ["bf16", "f16"])
@pytest.mark.parametrize("N", [4, 8, 16])
def test_stored_16bit_rs_output_exact(kind, N):
    """A 16-bit reduce-scatter output holding the SUM: with slice values k*2^-10,
    |k| <= 7, every partial sum is exact in 8 significant bits, so the stored
    output is the exact sum, the step's g is the correctly rounded sum / N, and
    the result equals the fused step over the N slices."""
    rng = np.random.default_rng(N)
    S = 300
    ints = rng.integers(-7, 8, size=(N, S))
    vals = (ints * 2.0 ** -10).astype(F)
    slices = [C.narrow(vals[k], kind) for k in range(N)]
    rs = C.narrow(vals.sum(axis=0).astype(F), kind)
    assert np.array_equal(C.widen(rs, kind), vals.sum(axis=0).astype(F))   # exact
    g = O.average(O.reduce_slices([rs], kind), N)
    for j in range(S):
        want = F(float(Fraction(int(ints[:, j].sum()), 1024) / N))
        assert g[j] == want
    p = rng.normal(0, 0.02, S).astype(F)
    z = np.zeros(S, F)
    a = O.shard_step(slices, kind, kind, N, p, z, z, lr=1e-3, t=1)
    b = O.shard_step([rs], kind, kind, N, p, z, z, lr=1e-3, t=1)
    assert np.array_equal(a.master.view(np.uint32), b.master.view(np.uint32))
    assert np.array_equal(a.params, b.params)
