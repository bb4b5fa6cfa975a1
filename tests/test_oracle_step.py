"""Pins of the oracle step against closed forms, brute force, library optimizers and
the pages' own 4-rank check."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import casts as C
from oracle import plan as P
from oracle import step as O

F = np.float32


def rn32(x: Fraction) -> np.float32:
    """Exact round-to-nearest-even of a rational to fp32 (normal range)."""
    a = F(float(x))
    best = None
    for c in (np.nextafter(a, F(-np.inf)), a, np.nextafter(a, F(np.inf))):
        d = abs(Fraction(float(c)) - x)
        key = (d, int(np.array(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return F(best[1])


# ---------------------------------------------------------------------------
# reduce / average / unscale: brute force with exactly representable values
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("world", [1, 3, 4, 8, 16, 64])
def test_reduce_average_unscale_exact(kind, world):
    """Slices hold small integers times 2^-10 (exact in every format); the fp32
    sum is then exact and order-free, so the result is the correctly rounded
    exact rational sum / N * inv_scale."""
    rng = np.random.default_rng(world)
    S = 257
    ints = rng.integers(-120, 121, size=(world, S))
    vals = (ints * 2.0 ** -10).astype(np.float32)
    slices = [C.narrow(vals[k], kind) for k in range(world)]
    inv_scale = 2.0 ** -16 if kind == "f16" else 1.0
    g = O.unscale(O.average(O.reduce_slices(slices, kind), world), inv_scale)
    for j in range(S):
        exact = Fraction(int(ints[:, j].sum()), 1024) / world
        want = rn32(exact) * F(inv_scale)          # unscale by a power of two is exact
        assert g[j] == want, (j, g[j], want)


def test_reduce_order_is_ascending_rank():
    """The fp32 accumulation starts from slice 0 and adds slices 1..N-1 in order
    (the order itself is a convention; this pins that the oracle keeps it)."""
    big, small = F(2.0 ** 24), F(1.0)
    slices = [np.array([big], F), np.array([small], F), np.array([small], F)]
    # ((2^24 + 1) + 1) rounds each time to 2^24; any other order gives 2^24 + 2
    assert O.reduce_slices(slices, "f32")[0] == big
    assert O.reduce_slices(slices[::-1], "f32")[0] == big + 2


# ---------------------------------------------------------------------------
# overflow flag and skip
# ---------------------------------------------------------------------------

def _flag_of(slices, kind, world, inv_scale=1.0):
    return O.overflow(O.unscale(O.average(O.reduce_slices(slices, kind), world), inv_scale))


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
@pytest.mark.parametrize("kind", ["f32", "bf16", "f16"])
def test_flag_on_injected_nonfinite(bad, kind):
    rng = np.random.default_rng(7)
    vals = rng.normal(0, 1e-3, size=(4, 100)).astype(F)
    slices = [C.narrow(v, kind) for v in vals]
    assert not _flag_of(slices, kind, 4)
    hit = vals.copy()
    hit[2, 37] = bad
    assert _flag_of([C.narrow(v, kind) for v in hit], kind, 4)


def test_flag_from_fp16_overflow_on_rounding():
    """65520 rounds to +inf in fp16 (ties to even past 65504)."""
    s = np.array([65520.0, 1.0], dtype=F)
    bits = C.narrow(s, "f16")
    assert bits[0] == 0x7C00
    assert _flag_of([bits, C.narrow(np.zeros(2, F), "f16")], "f16", 2, 2.0 ** -16)


def test_flag_from_fp32_sum_overflow():
    """Finite bf16 slices whose fp32 sum exceeds FLT_MAX raise the flag."""
    x = C.narrow(np.array([3.0e38], F), "bf16")
    assert np.isfinite(C.widen(x, "bf16")).all()
    assert _flag_of([x, x], "bf16", 2)


def test_skip_leaves_state_bitwise():
    rng = np.random.default_rng(3)
    S, N = 64, 4
    vals = rng.normal(0, 1e-3, size=(N, S)).astype(F)
    vals[1, 5] = np.inf
    master = rng.normal(0, 0.02, S).astype(F)
    m = rng.normal(0, 1e-4, S).astype(F)
    v = np.abs(rng.normal(0, 1e-6, S)).astype(F)
    r = O.shard_step([C.narrow(x, "bf16") for x in vals], "bf16", "bf16", N, master, m, v,
                     lr=3e-4, weight_decay=0.1, t=5)
    assert r.flag
    for a, b in ((r.master, master), (r.m, m), (r.v, v)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(r.params, C.round_to_bf16(master))


# ---------------------------------------------------------------------------
# norm and clip
# ---------------------------------------------------------------------------

def test_sumsq_exact_and_partitioned():
    """Sum over the N shards of q equals the full-vector sum of squares (exact
    summation of the exactly-squared fp32 values)."""
    rng = np.random.default_rng(5)
    N, S = 16, 1000
    g = rng.normal(0, 1e-3, N * S).astype(F)
    exact = math.fsum(float(x) * float(x) for x in g)
    q = [O.sumsq(g[r * S:(r + 1) * S]) for r in range(N)]
    assert abs(math.fsum(q) - exact) <= 1e-13 * exact
    assert abs(O.sumsq(g) - exact) <= 1e-13 * exact


def test_clip_coefficient_cases():
    assert O.clip_coefficient(0.25, 1.0) == F(1.0)       # norm 0.5 <= 1
    assert O.clip_coefficient(1.0, 1.0) == F(1.0)        # norm == max_norm: no clip
    assert O.clip_coefficient(4.0, 1.0) == F(0.5)        # norm 2 -> 1/2
    assert O.clip_coefficient(100.0, 5.0) == F(0.5)      # norm 10, max 5
    assert O.clip_coefficient(123.0, 0.0) == F(1.0)      # disabled
    c = O.clip_coefficient(31.4, 1.0)
    assert abs(float(c) * math.sqrt(31.4) - 1.0) < 1e-7


def test_clip_scales_gradient_before_adam():
    rng = np.random.default_rng(9)
    N, S = 4, 300
    vals = rng.normal(0, 1e-3, size=(N, S)).astype(F)
    sl = [C.narrow(x, "bf16") for x in vals]
    st = dict(master=rng.normal(0, .02, S).astype(F), m=np.zeros(S, F), v=np.zeros(S, F))
    big = O.shard_step(sl, "bf16", "bf16", N, **st, lr=3e-4, t=1, max_norm=1e-4)
    g = big.g
    c = O.clip_coefficient(O.sumsq(g), 1e-4)
    assert float(c) < 1
    ref = O.adamw(st["master"], st["m"], st["v"], np.multiply(g, c, dtype=F),
                  O.adam_consts(3e-4, .9, .999, 1e-8, 0.0, 1))
    assert np.array_equal(big.master, ref[0]) and np.array_equal(big.m, ref[1])
    # a norm below max_norm gives c = 1 and the same bits as not clipping
    nc = O.shard_step(sl, "bf16", "bf16", N, **st, lr=3e-4, t=1)
    cl = O.shard_step(sl, "bf16", "bf16", N, **st, lr=3e-4, t=1, max_norm=1e3)
    assert cl.clip == F(1) and np.array_equal(nc.master, cl.master)


# ---------------------------------------------------------------------------
# Adam: closed forms
# ---------------------------------------------------------------------------

def _first_step_error(adamw_fn):
    """Max error of step 1 from m = v = 0 against the float64 closed form
    p' = (1 - lr wd) p - lr g / (|g| + eps), relative to lr."""
    rng = np.random.default_rng(1)
    S = 4096
    p = rng.normal(0, 0.05, S).astype(F)
    g = rng.normal(0, 1e-2, S).astype(F)
    lr, wd = 1e-2, 0.1
    c = O.adam_consts(lr, 0.9, 0.999, 1e-8, wd, 1)
    p2, m2, v2 = adamw_fn(p, np.zeros(S, F), np.zeros(S, F), g, c)
    gd = g.astype(np.float64)
    want = (1 - lr * wd) * p.astype(np.float64) - lr * gd / (np.abs(gd) + 1e-8)
    return float(np.max(np.abs(p2 - want)) / lr), p, p2, g


def test_first_step_closed_form():
    err, p, p2, g = _first_step_error(O.adamw)
    assert err < 2e-6
    # the step is about lr per element when |g| >> eps (handbook's Adam, t = 1)
    step = np.abs(p2.astype(np.float64) - (1 - 1e-3) * p)
    assert abs(step.mean() - 1e-2) < 1e-5
    big = np.abs(g) > 1e-5                       # |g| >> eps: |step| within 0.1% of lr
    assert big.mean() > 0.99 and step[big].min() > 0.999e-2 and step.max() <= 1e-2 * (1 + 1e-6)


@pytest.mark.parametrize("mutant", ["no_bias_correction", "sign", "swapped_betas", "eps_inside_sqrt"])
def test_first_step_pin_catches_planted_mistakes(mutant):
    def bad(p, m, v, g, c):
        import dataclasses
        if mutant == "no_bias_correction":
            c = dataclasses.replace(c, bc1=F(1), bc2=F(1))
        if mutant == "swapped_betas":
            c = dataclasses.replace(c, b1=c.b2, b2=c.b1, omb1=c.omb2, omb2=c.omb1)
        if mutant == "eps_inside_sqrt":
            m2 = c.b1 * m + c.omb1 * g
            v2 = c.b2 * v + c.omb2 * (g * g)
            u = (c.lr * (m2 / c.bc1)) / np.sqrt(v2 / c.bc2 + c.eps)
            return (c.dec * p - u).astype(F), m2, v2
        p2, m2, v2 = O.adamw(p, m, v, g, c)
        if mutant == "sign":
            p2 = (c.dec * p + (c.dec * p - p2)).astype(F)
        return p2, m2, v2
    err, *_ = _first_step_error(bad)
    assert err > 1e-3


def test_zero_gradient():
    """g = 0: m' = b1 m, v' = b2 v, and with m = v = 0 the master is only decayed
    (bitwise unchanged when wd = 0)."""
    rng = np.random.default_rng(2)
    S = 500
    p = rng.normal(0, 0.05, S).astype(F)
    z = np.zeros(S, F)
    for wd in (0.0, 0.1):
        c = O.adam_consts(1e-2, 0.9, 0.999, 1e-8, wd, 3)
        p2, m2, v2 = O.adamw(p, z, z, z, c)
        assert np.array_equal(p2, np.multiply(c.dec, p, dtype=F))
        assert not np.any(m2) and not np.any(v2)
        if wd == 0:
            assert np.array_equal(p2.view(np.uint32), p.view(np.uint32))


def test_three_steps_against_float64_moment_sums():
    """m_k = (1-b1) sum_i b1^(k-i) g_i and v_k = (1-b2) sum_i b2^(k-i) g_i^2 in
    float64, with the update recursion, agree with the fp32 oracle to fp32
    rounding after three steps."""
    rng = np.random.default_rng(4)
    S, lr, b1, b2, eps, wd = 2000, 1e-2, 0.9, 0.999, 1e-8, 0.05
    gs = [rng.normal(0, 1e-2, S).astype(F) for _ in range(3)]
    p = rng.normal(0, 0.05, S).astype(F)
    m = np.zeros(S, F)
    v = np.zeros(S, F)
    pd = p.astype(np.float64)
    for k in range(1, 4):
        p, m, v = O.adamw(p, m, v, gs[k - 1], O.adam_consts(lr, b1, b2, eps, wd, k))
        md = (1 - b1) * sum(b1 ** (k - i) * gs[i - 1].astype(np.float64) for i in range(1, k + 1))
        vd = (1 - b2) * sum(b2 ** (k - i) * gs[i - 1].astype(np.float64) ** 2
                            for i in range(1, k + 1))
        pd = (1 - lr * wd) * pd - lr * (md / (1 - b1 ** k)) / (np.sqrt(vd / (1 - b2 ** k)) + eps)
        assert np.max(np.abs(m - md) / np.abs(md).max()) < 1e-6
        assert np.max(np.abs(v - vd) / np.abs(vd).max()) < 1e-6
    assert np.max(np.abs(p - pd)) / lr < 1e-5


def test_adamw_matches_torch_adamw():
    """Decoupled weight decay agrees with torch.optim.AdamW (a library optimizer)."""
    rng = np.random.default_rng(6)
    S, lr, wd = 3000, 3e-4, 0.1
    p0 = rng.normal(0, 0.02, S).astype(F)
    gs = [rng.normal(0, 1e-3, S).astype(F) for _ in range(4)]
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd,
                            foreach=False)
    p, m, v = p0.copy(), np.zeros(S, F), np.zeros(S, F)
    for k, g in enumerate(gs, start=1):
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p, m, v = O.adamw(p, m, v, g, O.adam_consts(lr, 0.9, 0.999, 1e-8, wd, k))
    assert np.max(np.abs(p - tp.detach().numpy())) < 1e-3 * lr
    st = opt.state[tp]
    # moments can cancel across steps: compare against their scale, not elementwise
    mr, vr = st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()
    assert np.max(np.abs(m - mr)) < 1e-6 * np.abs(mr).max()
    assert np.max(np.abs(v - vr)) < 1e-6 * np.abs(vr).max()


# ---------------------------------------------------------------------------
# sharding: union of the N shard steps == the unsharded step; padding
# ---------------------------------------------------------------------------

def _full_rank_grads(rng, N, psi):
    return [rng.normal(0, 1e-2, psi).astype(F) for _ in range(N)]


@pytest.mark.parametrize("psi,N,cap", [(10_007, 4, 0), (19_210, 4, 0), (5_000, 8, 700),
                                       (3, 4, 0)])
def test_union_of_shards_equals_unsharded(psi, N, cap):
    """Stepping every rank's shard and gathering equals one step on the whole
    padded vector (N = 1 with the reduced gradient), bit for bit; padding stays +0."""
    rng = np.random.default_rng(psi)
    sizes = [psi // 3, psi - 2 * (psi // 3), psi // 3]
    pl = P.make_plan(sizes, N, cap)
    NS = pl.padded_numel
    grads = _full_rank_grads(rng, N, NS)
    master = rng.normal(0, 0.05, NS).astype(F)
    pad = np.ones(NS, bool)
    for i, n in enumerate(sizes):
        pad[pl.tensor_offset[i]:pl.tensor_offset[i] + n] = False
    for x in grads + [master]:
        x[pad] = 0
    m = np.zeros(NS, F)
    v = np.zeros(NS, F)
    gather = np.zeros(NS, F)
    for r in range(N):
        segs = P.rank_segments(pl, r)
        idx = np.concatenate([np.arange(go, go + ln) for go, _lo, ln, _v in segs])
        res = O.shard_step([gk[idx] for gk in grads], "f32", "f32", N, master[idx], m[idx], v[idx],
                           lr=1e-2, weight_decay=0.1, t=1)
        O.write_gather(gather, segs, res.params)
    # unsharded: reduce first (same order), then one N = 1 step over everything
    g_full = O.average(O.reduce_slices(grads, "f32"), N)
    one = O.shard_step([g_full], "f32", "f32", 1, master, m, v, lr=1e-2, weight_decay=0.1, t=1)
    assert np.array_equal(gather.view(np.uint32), one.params.view(np.uint32))
    assert np.all(gather[pad].view(np.uint32) == 0)
    # and the unsharded step agrees with torch.optim.AdamW on the reduced gradient
    tp = torch.nn.Parameter(torch.from_numpy(master.copy()))
    opt = torch.optim.AdamW([tp], lr=1e-2, weight_decay=0.1, foreach=False)
    tp.grad = torch.from_numpy(g_full.copy())
    opt.step()
    assert np.max(np.abs(gather - tp.detach().numpy())) < 1e-7


def test_pads_stay_positive_zero_over_steps():
    S = 16
    z = np.zeros(S, F)
    p, m, v = z.copy(), z.copy(), z.copy()
    for t in range(1, 4):
        r = O.shard_step([C.narrow(z, "bf16")] * 8, "bf16", "bf16", 8, p, m, v, lr=3e-4,
                         weight_decay=0.1, t=t)
        p, m, v = r.master, r.m, r.v
    for x in (p, m, v, r.params):
        assert np.all(x.view(np.uint32 if x.dtype == F else np.uint16) == 0)


# ---------------------------------------------------------------------------
# the handbook's 4-rank check, emulated in one process
# ---------------------------------------------------------------------------

def test_toy_four_ranks_match_torch_adam():
    """zero_check.py: 4 ranks each take 8 of 32 samples; after 3 steps the
    sharded Adam matches single-process torch.optim.Adam on the full batch
    (the page prints True for max |diff| < 1e-5)."""
    def make_model():
        torch.manual_seed(0)
        return torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(),
                                   torch.nn.Linear(256, 10))

    torch.manual_seed(123)
    X, Y = torch.randn(32, 64), torch.randint(0, 10, (32,))
    world = 4
    loss_fn = torch.nn.CrossEntropyLoss()
    ref, model = make_model(), make_model()
    opt_ref = torch.optim.Adam(ref.parameters(), lr=1e-2)
    params = list(model.parameters())
    pl = P.make_plan([p.numel() for p in params], world)
    NS, S = pl.padded_numel, pl.shard_numel

    def flat(ts):
        out = np.zeros(NS, F)
        out[:pl.psi] = torch.cat([t.detach().reshape(-1) for t in ts]).numpy()
        return out

    full = flat([p.data for p in params])
    state = [(full[r * S:(r + 1) * S].copy(), np.zeros(S, F), np.zeros(S, F)) for r in range(world)]
    for t in range(1, 4):
        opt_ref.zero_grad()
        loss_fn(ref(X), Y).backward()
        opt_ref.step()
        grads = []
        for r in range(world):                       # each rank's backward on its local batch
            model.zero_grad()
            loc = slice(r * 32 // world, (r + 1) * 32 // world)
            loss_fn(model(X[loc]), Y[loc]).backward()
            grads.append(flat([p.grad for p in params]))
        gather = np.zeros(NS, F)
        for r in range(world):
            mst, m, v = state[r]
            res = O.shard_step([gk[r * S:(r + 1) * S] for gk in grads], "f32", "f32", world,
                               mst, m, v, lr=1e-2, t=t)
            state[r] = (res.master, res.m, res.v)
            O.write_gather(gather, P.rank_segments(pl, r), res.params)
        off = 0
        with torch.no_grad():
            for p in params:
                p.copy_(torch.from_numpy(gather[off:off + p.numel()]).view_as(p))
                off += p.numel()
    diff = max((a - b).abs().max().item() for a, b in zip(ref.parameters(), model.parameters()))
    assert diff < 1e-5, diff
    assert P.state_bytes(pl) == 57_636


def test_signed_zero_inputs_and_the_sum_identity():
    """The generator's signed-zero option (used by the GPU's signed-zero parity
    cases) yields -0 and +0 at its positions and -0 in every slice at some; and
    -0 is the identity of IEEE fp32 addition, the fact the windowed sums rely
    on when they start from -0 instead of from slice 0."""
    import torch
    import workloads as W
    from oracle import plan as OP
    w = W.Workload(name="sz", tensors=(("x", (12 * 3001,)),), world=12, rank=11, bucket_cap=0,
                   grad_dtype="bf16", param_dtype="bf16", lr=1e-3, grad_signed_zero_frac=0.3, seed=5)
    pl = OP.make_plan(W.numels(w.tensors), w.world)
    lay = W.Layout(S=pl.shard_numel, segments=OP.rank_segments(pl, w.rank), tensor_flat_off=list(pl.tensor_offset))
    x = W.make_slices(w, lay, step=1).float()
    zero = x == 0
    neg = zero & torch.signbit(x)
    assert neg.any() and (zero & ~torch.signbit(x)).any()
    assert neg.all(dim=0).any()
    # the ordered sum from slice 0 equals the sum started at -0, bit for bit
    xs = x.numpy().astype(F)
    a = xs[0].copy()
    b = np.full(xs.shape[1], -0.0, F) + xs[0]
    for k in range(1, xs.shape[0]):
        a = a + xs[k]
        b = b + xs[k]
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.signbit(a[neg.all(dim=0).numpy()]).all()
    special = np.array([0.0, -0.0, 1e-45, -1e-45, 1.0, -3.5, np.inf, -np.inf, np.nan], F)
    assert np.array_equal((np.float32(-0.0) + special).view(np.uint32)[:-1], special.view(np.uint32)[:-1])
    assert np.isnan(np.float32(-0.0) + special[-1])
