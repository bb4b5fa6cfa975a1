"""GPU parity of the HIP step against the oracle, through the C ABI, at sizes the
oracle finishes in seconds (several 2048-element tiles and a ragged tail)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from gpu_harness import (CODE, RIGS, Rig, check_params, compare_step, from_storage, guards, plant_tail,
                         round_up, say, storage)
from oracle import casts as OC
from oracle import plan as OP
from oracle import step as OS

pytestmark = pytest.mark.gpu
F = np.float32


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    RIGS.clear()
    yield
    # no step of the test wrote a tiled state buffer past S (fused, clipped,
    # skipped and restore steps all ran on these buffers)
    bad = [r.w.name for r in RIGS if not r.tails_intact()]
    RIGS.clear()
    assert not bad, f"tiled state written past S: {bad}"


def _oracle_slices(sl_cpu, S, world):
    return [storage(sl_cpu[k, :S]) for k in range(world)]


SEP, TILED = Z.ZERO_STATE_SEPARATE, Z.ZERO_STATE_TILED
LAYOUTS = pytest.mark.parametrize("layout", [SEP, TILED], ids=["separate", "tiled"])


def _grads(rig: Rig, source: str, step: int):
    """One step's gradient: (device buffers, fused-call options, oracle slices).

    slices: the N ranks' [S] contributions (the fused reduce-scatter);
    stored: one stored [S] reduce-scatter output (row 0 of the slices);
    full:   one full flat gradient read at the rank's slots (ZeRO-1);
    full_n: N full flat gradients, summed in the step."""
    w = rig.w
    if source in ("slices", "stored"):
        sl_cpu, sl_dev = rig.slices(step)
        if source == "slices":
            return sl_dev, {}, _oracle_slices(sl_cpu, rig.S, w.world)
        return sl_dev, dict(count=1), [storage(sl_cpu[0, :rig.S])]
    count = {"full": 1, "full_n": w.world}[source]
    NS = rig.pl.padded_numel
    ldf = round_up(NS, 64)
    full = W.make_full_grads(w, NS, rig.lay.tensor_flat_off, count, step=step, ld=ldf)
    sl = [OS.read_pieces(storage(full[k, :NS]), rig.lay.segments) for k in range(count)]
    return full.to(rig.dev), dict(count=count, layout=Z.ZERO_GRAD_FULL, ld=ldf), sl


def run_workload(w: W.Workload, ld_align=64, rank=None, steps=None, layout=SEP, source="slices", table=False):
    """Run w.steps steps on the GPU and in the oracle; compare everything."""
    rig = Rig(w, ld_align=ld_align, rank=rank, layout=layout, table=table)
    w = rig.w
    say(f"workload {w.name} S={rig.S} N={w.world} rank={w.rank} grads={w.grad_dtype} "
        f"params={w.param_dtype} buckets={len(rig.lay.segments)} ld={rig.ld} layout={layout} "
        f"source={source} table={table}")
    p, m, v = rig.p0, rig.m0, rig.v0
    gather_ref = rig.gather0.copy()
    cur, nxt = rig.A, rig.B
    t = w.t0
    same = total = 0
    for step in range(1, (steps or w.steps) + 1):
        sl_dev, gkw, sl = _grads(rig, source, step)
        kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                  t=t + 1, inv_scale=1.0 / w.loss_scale)
        if w.max_norm > 0:
            rig.reduce_norm(sl_dev, **gkw)
            torch.cuda.synchronize()
            g_ref = OS.unscale(OS.average(OS.reduce_slices(sl, w.grad_dtype), w.world),
                               1.0 / w.loss_scale)
            g_gpu = rig.g.cpu().numpy()
            assert np.array_equal(g_gpu.view(np.uint32), g_ref.view(np.uint32)), "stash g"
            q_gpu = float(rig.sumsq.item())
            q_ref = OS.sumsq(g_ref)
            assert abs(q_gpu - q_ref) <= 1e-9 * q_ref, (q_gpu, q_ref)
            c_gpu = F(rig.clip.item())
            c_ref = OS.clip_coefficient(q_ref, w.max_norm)
            assert abs(int(c_gpu.view(np.int32)) - int(c_ref.view(np.int32))) <= 1
            assert c_gpu == OS.clip_coefficient(q_gpu, w.max_norm)
            rig.stash_step(cur, t + 1)
            res = OS.shard_step(sl, w.grad_dtype, w.param_dtype, w.world, p, m, v,
                                max_norm=w.max_norm, clip_override=c_gpu, **kw)
            out = cur
        else:
            rig.fused(sl_dev, cur, nxt, t + 1, **gkw)
            res = OS.shard_step(sl, w.grad_dtype, w.param_dtype, w.world, p, m, v, **kw)
            out = cur if res.flag else nxt
        torch.cuda.synchronize()
        flag = int(rig.flag.item())
        assert flag == int(res.flag), f"step {step}: flag {flag} vs oracle {res.flag}"
        gp, gm, gv = rig.unpack(out)
        g_used = res.g if w.max_norm <= 0 else np.multiply(res.g, res.clip, dtype=F)
        n, tot = compare_step(gp, gm, gv, res, p, m, v, g_used,
                              OS.adam_consts(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t + 1),
                              f"{w.name} step {step}")
        same, total = same + n, total + tot
        # gather buffer: this rank's pieces hold the new params, everything else untouched
        OS.write_gather(gather_ref, rig.lay.segments, res.params)
        got = rig.gather_np()
        mask = rig.slot_mask()
        assert np.array_equal(got[~mask].view(np.uint32 if got.dtype == F else np.uint16),
                              gather_ref[~mask].view(np.uint32 if got.dtype == F else np.uint16)), \
            "write outside the rank's slots"
        check_params(got[mask], gather_ref[mask], w.param_dtype, f"{w.name} step {step} params")
        if not res.flag:
            p, m, v = res.master, res.m, res.v
            t += 1
            if w.max_norm <= 0:
                cur, nxt = nxt, cur
    say(f"  bitwise-equal state elements: {same}/{total}")
    assert same == total, f"{total - same} state elements differ in the last bit"
    return rig


@LAYOUTS
@pytest.mark.parametrize("name", W.ORDER)
def test_small_workloads(name, layout):
    run_workload(W.SMALL[name], layout=layout)


def test_toy_all_ranks_union_equals_unsharded():
    """Every rank of the toy stepped on the GPU; the gathered parameters equal the
    oracle's single step over the whole padded vector."""
    w = W.TOY
    pl = OP.make_plan(W.numels(w.tensors), w.world)
    NS = pl.padded_numel
    gather = np.zeros(NS, F)
    full_slices = [np.zeros(NS, F) for _ in range(w.world)]
    full_master = np.zeros(NS, F)
    for r in range(w.world):
        rig = Rig(w, rank=r)
        sl_cpu, sl_dev = rig.slices(1)
        rig.fused(sl_dev, rig.A, rig.B, 1)
        torch.cuda.synchronize()
        assert rig.flag.item() == 0
        got = rig.gather_np()
        for goff, _lo, ln, _v in rig.lay.segments:
            gather[goff:goff + ln] = got[goff:goff + ln]
            for k in range(w.world):
                full_slices[k][goff:goff + ln] = sl_cpu[k, :ln].numpy()
            full_master[goff:goff + ln] = rig.p0
    one = OS.shard_step(full_slices, "f32", "f32", w.world, full_master, np.zeros(NS, F),
                        np.zeros(NS, F), lr=w.lr, t=1)
    assert np.array_equal(gather.view(np.uint32), one.params.view(np.uint32))
    assert np.all(gather[pl.psi:].view(np.uint32) == 0)


def _flat(psi, world, rank, g, p, seed=3, **kw):
    return W.Workload(name=f"flat{psi}_n{world}_r{rank}_{g}_{p}", tensors=(("x", (psi,)),),
                      world=world, rank=rank, bucket_cap=0, grad_dtype=g, param_dtype=p,
                      lr=1e-3, weight_decay=0.05, steps=2, seed=seed, **kw)


# shard sizes on either side of the one-workgroup path's limit (8192 elements)
SIZES = pytest.mark.parametrize("S", [5003, 20011], ids=["small", "large"])


@SIZES
@pytest.mark.parametrize("g", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("p", ["f32", "bf16", "f16"])
def test_dtype_matrix(g, p, S):
    run_workload(_flat(4 * S, 4, 3, g, p))
    if g == p:
        run_workload(_flat(4 * S, 4, 3, g, p), layout=TILED)


@pytest.mark.parametrize("world,rank,psi", [
    (1, 0, 12_347),          # N = 1: the whole vector
    (2, 1, 40_000),          # slot offset 0 mod 16 bytes
    (3, 2, 30_001),          # N not a power of two: a true IEEE division
    (8, 1, 8 * 5004),        # bf16 slot 8 mod 16
    (8, 2, 8 * 5003),        # bf16 slot 4 mod 16 (2 * 10006 = 20012)
    (8, 1, 8 * 5003 - 5),    # bf16 slot 2 mod 16 and padding at the end of rank 7
    (16, 15, 16 * 2049 - 9), # padding inside the last rank's shard
    (64, 63, 750_000),       # many slices
    (5, 4, 3),               # fewer elements than ranks: this rank is all padding
])
def test_world_and_alignment(world, rank, psi):
    run_workload(_flat(psi, world, rank, "bf16", "bf16"))
    run_workload(_flat(psi, world, rank, "bf16", "bf16"), layout=TILED)


# Every form of the slice sum, in the fused update and in the clipped path's
# reduction, at a shard of 10,007 elements: above the one-workgroup path's
# limit (8192), so the multi-workgroup kernels run, over five state tiles with
# a ragged end.  The fused update: 1, 2, 4 buffers at once; 16-bit 8 in the
# eight-element windowed sum; 16-bit 16, 32, 64 and fp32 8, 16, 32 in the
# compiled four-element windows; every other count in the run-time ring, whose
# tail differs with (N - W) mod W (W = 8 for 16-bit, 4 for fp32): the counts
# 9-15 and 17 reach every tail of the 16-bit ring, 5-7 and 9-11 those of the
# fp32 one, 3 the path below the window.  The reduction: 1, 2, 4, 8, 16, 32,
# 64 compiled (fp32 8 as two batches of 4), the other counts of four or more
# in its ring (W = 4), 3 in the runtime loop.
@pytest.mark.parametrize("world", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 24, 32, 48, 64])
@pytest.mark.parametrize("g", ["f32", "bf16", "f16"])
def test_batch_forms(world, g):
    psi = world * 10007
    p = "bf16" if g != "f32" else "f32"
    run_workload(_flat(psi, world, world - 1, g, p), layout=TILED)
    run_workload(_flat(psi, world, world // 2, g, p, max_norm=0.05), layout=TILED)


# Exact zeros of either sign in every slice (at a quarter of those positions -0
# in all slices, so the sum there is -0).  The oracle sums from slice 0; the
# windowed sums start from -0, which leaves every value unchanged under IEEE
# addition, +0 included, so the two agree bit for bit.  The clipped path's
# stash holds g itself and shows the sign of each zero sum.
@pytest.mark.parametrize("world", [3, 5, 8, 12, 16, 24, 64])
@pytest.mark.parametrize("g", ["f32", "bf16"])
def test_signed_zero_sums(world, g):
    w = dataclasses.replace(_flat(world * 10007, world, world - 1, g, g), grad_signed_zero_frac=0.3)
    run_workload(w, layout=TILED)
    run_workload(dataclasses.replace(w, max_norm=0.05), rank=world // 2, layout=TILED)


# The one-workgroup path (a shard of at most 8192 elements) sums any count in
# its runtime loop: a few counts, fused and clipped.
@pytest.mark.parametrize("world", [3, 8, 24, 64])
@pytest.mark.parametrize("g", ["f32", "bf16"])
def test_small_path_counts(world, g):
    psi = world * 4099
    run_workload(_flat(psi, world, world - 1, g, g), layout=TILED)
    run_workload(_flat(psi, world, world // 2, g, g, max_norm=0.05), layout=TILED)


# Large data-parallel degrees (the deep-dive page's Table 1 goes to N_d = 1024):
# the runtime-N reduction loop in batches of 16, a world that is not a power
# of two (an IEEE division), and the last rank, fused and clipped.
@SIZES
@pytest.mark.parametrize("world,g", [(128, "bf16"), (257, "f16"), (1024, "bf16")])
def test_large_world(world, g, S):
    psi = world * S - 7
    run_workload(_flat(psi, world, world - 1, g, g), layout=TILED)
    run_workload(_flat(psi, world, world // 3, g, g, max_norm=0.05), layout=TILED)


def test_loss_scaled_fp16():
    run_workload(_flat(64 * 3001, 64, 63, "f16", "f16", loss_scale=65536.0, grad_zero_frac=0.01))


@pytest.mark.parametrize("S", [4093, 16381])
def test_minimal_slice_stride(S):
    """Slices packed with the smallest 16-byte-aligned stride (ld = S rounded up to 8)."""
    run_workload(_flat(4 * S, 4, 1, "bf16", "bf16"), ld_align=8)


def test_many_buckets_several_launches():
    """More pieces than one launch addresses (multi-launch path)."""
    sizes = [(i * 37) % 211 + 5 for i in range(140)]
    w = W.Workload(name="many_buckets", tensors=tuple((f"t{i}", (n,)) for i, n in enumerate(sizes)),
                   world=3, rank=2, bucket_cap=150, grad_dtype="bf16", param_dtype="bf16",
                   lr=1e-3, weight_decay=0.1, steps=2, seed=9)
    pl = OP.make_plan(sizes, 3, 150)
    assert len(pl.buckets) > 60
    for layout in (SEP, TILED):
        run_workload(w, layout=layout)
        run_workload(dataclasses.replace(w, max_norm=1e-3, name="many_buckets_clip"), layout=layout)


@SIZES
@LAYOUTS
@pytest.mark.parametrize("bad", ["+inf", "-inf", "nan", "f16_overflow"])
@pytest.mark.parametrize("mode", ["fused", "stash"])
def test_overflow_skips_bitwise(bad, mode, layout, S):
    gk = "f16" if bad == "f16_overflow" else "bf16"
    w = _flat(8 * S, 8, 5, gk, gk, max_norm=(1.0 if mode == "stash" else 0.0))
    rig = Rig(w, layout=layout)
    say(f"overflow {bad} {mode}")
    sl_cpu, _ = rig.slices(1)
    val = {"+inf": float("inf"), "-inf": float("-inf"), "nan": float("nan"),
           "f16_overflow": 65520.0}[bad]
    sl_cpu[6, 1234] = torch.tensor(val).to(sl_cpu.dtype)
    sl_dev = sl_cpu.to("cuda")
    before = [x.clone() for x in rig.A]
    if mode == "fused":
        rig.B[0].fill_(7.0)
        if layout == TILED:
            plant_tail(rig.B[0], rig.S)
        rig.fused(sl_dev, rig.A, rig.B, 1)
    else:
        rig.reduce_norm(sl_dev)
        rig.stash_step(rig.A, 1)
    torch.cuda.synchronize()
    assert rig.flag.item() == 1
    for a, b in zip(rig.A, before):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert np.array_equal(rig.gather_np(), rig.gather0)


@SIZES
@LAYOUTS
@pytest.mark.parametrize("mode", ["fused", "stash"])
def test_forced_skip(mode, layout, S):
    w = _flat(4 * S, 4, 2, "bf16", "bf16", max_norm=(1.0 if mode == "stash" else 0.0))
    rig = Rig(w, layout=layout)
    _, sl_dev = rig.slices(1)
    skip = torch.ones(1, dtype=torch.int32, device="cuda")
    before = [x.clone() for x in rig.A]
    if mode == "fused":
        rig.B[-1].fill_(3.0)
        if layout == TILED:
            plant_tail(rig.B[0], rig.S)
        rig.fused(sl_dev, rig.A, rig.B, 1, skip=skip.data_ptr())
        torch.cuda.synchronize()
        assert rig.flag.item() == 1
        if layout == TILED:
            assert np.all(rig.unpack(rig.B)[2] == 3.0)
        else:
            assert torch.all(rig.B[-1] == 3.0)
    else:
        rig.reduce_norm(sl_dev)
        rig.stash_step(rig.A, 1, skip=skip.data_ptr())
        torch.cuda.synchronize()
    for a, b in zip(rig.A, before):
        assert torch.equal(a, b)
    assert np.array_equal(rig.gather_np(), rig.gather0)


@SIZES
@LAYOUTS
@pytest.mark.parametrize("why", ["inf", "skip_in"])
def test_skip_rewrites_slots(why, layout, S):
    """A fused step that is not applied leaves the rank's slots holding the
    rounded input master, whatever they held before (the slots start as a
    sentinel here, not as the rounded master the other tests start from), on
    both sides of the one-workgroup path's limit; outside the slots nothing
    changes."""
    w = _flat(4 * S + 1, 4, 3, "bf16", "bf16")
    rig = Rig(w, layout=layout)
    sl_cpu, _ = rig.slices(1)
    skip = None
    if why == "inf":
        sl_cpu[2, S // 2] = float("inf")
    else:
        skip = torch.ones(1, dtype=torch.int32, device="cuda")
    mask = rig.slot_mask()
    g0 = rig.gather0.copy()
    g0[mask] = 0x3F80 if w.param_dtype != "f32" else 1.0   # bf16 1.0: not the rounded master
    rig.gather.copy_(from_storage(g0, w.param_dtype).to("cuda"))
    rig.fused(sl_cpu.to("cuda"), rig.A, rig.B, 1, skip=None if skip is None else skip.data_ptr())
    torch.cuda.synchronize()
    assert rig.flag.item() == 1
    got = rig.gather_np()
    assert np.array_equal(got[~mask], g0[~mask]), "write outside the rank's slots"
    want = np.zeros_like(g0)
    OS.write_gather(want, rig.lay.segments, OC.narrow(rig.p0, w.param_dtype))
    assert np.array_equal(got[mask], want[mask]), "slots do not hold the rounded input master"


@SIZES
@LAYOUTS
def test_no_flag_applies_update_with_inf(layout, S):
    """Without an overflow flag nothing is checked: both paths apply the update
    with the non-finite gradient, as the oracle's AdamW does without its skip."""
    w = _flat(4 * S, 4, 1, "bf16", "bf16")
    rig = Rig(w, layout=layout)
    sl_cpu, _ = rig.slices(1)
    sl_cpu[1, 77] = float("inf")
    rig.fused(sl_cpu.to("cuda"), rig.A, rig.B, 1, overflow=False)
    torch.cuda.synchronize()
    sl = [storage(sl_cpu[k, :rig.S]) for k in range(4)]
    g = OS.unscale(OS.average(OS.reduce_slices(sl, "bf16"), 4), 1.0)
    with np.errstate(invalid="ignore", over="ignore"):
        p2, m2, v2 = OS.adamw(rig.p0, rig.m0, rig.v0, g, OS.adam_consts(w.lr, w.beta1, w.beta2, w.eps,
                                                                          w.weight_decay, 1))
    gp, gm, gv = rig.unpack(rig.B)
    # NaN bit patterns are not part of the contract (the CPU and the GPU make
    # different default NaNs): NaN where the oracle has NaN, bits elsewhere
    for a_, b_ in ((gp, p2), (gm, m2), (gv, v2)):
        nan = np.isnan(b_)
        assert np.array_equal(np.isnan(a_), nan)
        assert np.array_equal(a_[~nan].view(np.uint32), b_[~nan].view(np.uint32))
    assert np.isnan(gp[77]) and np.isinf(gm[77]) and np.isinf(gv[77])
    got = rig.gather_np()
    want = rig.gather0.copy()
    OS.write_gather(want, rig.lay.segments, OC.narrow(p2, "bf16"))
    is_nan16 = lambda x: ((x & 0x7F80) == 0x7F80) & ((x & 0x7F) != 0)
    assert np.array_equal(is_nan16(got), is_nan16(want))
    assert np.array_equal(got[~is_nan16(want)], want[~is_nan16(want)])


@SIZES
@LAYOUTS
def test_no_flag_in_place_matches(layout, S):
    """Fused step without an overflow flag, updated in place."""
    w = _flat(4 * S + 3, 4, 3, "bf16", "bf16")
    rig = Rig(w, layout=layout)
    sl_cpu, sl_dev = rig.slices(1)
    rig.fused(sl_dev, rig.A, rig.A, 1, overflow=False)
    torch.cuda.synchronize()
    res = OS.shard_step([storage(sl_cpu[k, :rig.S]) for k in range(4)], "bf16", "bf16", 4,
                        rig.p0, rig.m0, rig.v0, lr=w.lr, weight_decay=w.weight_decay, t=1)
    assert np.array_equal(rig.unpack(rig.A)[0].view(np.uint32), res.master.view(np.uint32))


def test_norm_deterministic_and_partitioned():
    w = _flat(16 * 200_003, 16, 7, "bf16", "bf16", max_norm=1.0)
    rig = Rig(w)
    _, sl_dev = rig.slices(1)
    bits = set()
    for _ in range(10):
        rig.reduce_norm(sl_dev)
        torch.cuda.synchronize()
        bits.add(rig.sumsq.cpu().numpy().view(np.uint64)[0])
        assert rig.flag.item() == 0
    assert len(bits) == 1
    # other ranks' share enters the norm: sqrt(q + other) decides the coefficient
    q = float(rig.sumsq.item())
    rig.reduce_norm(sl_dev, other=3 * q, max_norm=1e-3)
    torch.cuda.synchronize()
    want = F(1e-3 / np.sqrt(np.float64(q) + 3 * q))
    assert F(rig.clip.item()) == want
    rig.reduce_norm(sl_dev, max_norm=1e6)
    torch.cuda.synchronize()
    assert rig.clip.item() == 1.0


# ---------------------------------------------------------------------------
# other gradient sources: a stored reduce-scatter output (one summed [S]
# buffer) and a gradient all-reduced in full (ZeRO-1: full flat buffers read
# at the rank's slots)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("world", [8, 64])
@pytest.mark.parametrize("g", ["f32", "bf16", "f16"])
def test_stored_rs_output(g, world):
    p = "f32" if g == "f32" else "bf16"
    ls = 1024.0 if g == "f16" else 1.0
    run_workload(_flat(world * 5003, world, world - 1, g, p, loss_scale=ls), layout=TILED,
                 source="stored")
    run_workload(_flat(world * 5003, world, 1, g, p, loss_scale=ls, max_norm=0.01), layout=TILED,
                 source="stored")


def _ragged(world, rank, g, p, n_tensors, size, cap, seed=5):
    """Tensors of odd sizes packed into buckets: pieces start at every alignment
    in the full gradient, and vectors of 8 straddle piece boundaries."""
    sizes = [size + 37 * (i % 5) for i in range(n_tensors)]
    return W.Workload(name=f"ragged{n_tensors}x{size}_n{world}_r{rank}_{g}",
                      tensors=tuple((f"t{i}", (n,)) for i, n in enumerate(sizes)), world=world,
                      rank=rank, bucket_cap=cap, grad_dtype=g, param_dtype=p, lr=1e-3,
                      weight_decay=0.05, steps=2, seed=seed)


@pytest.mark.parametrize("source", ["full", "full_n"])
@pytest.mark.parametrize("g,p", [("bf16", "bf16"), ("f16", "f16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("case", [
    (4, 3, 7, 4099, 9000),      # a few buckets, S > 8192: the multi-workgroup update
    (4, 1, 7, 999, 3000),       # S <= 8192 in one launch group: the one-workgroup path
    (3, 2, 70, 97, 150),        # 70 buckets: several launch groups of at most 24 pieces
    (8, 0, 1, 100_003, 0),      # one flat bucket, rank 0
])
def test_full_gradient(case, g, p, source):
    world, rank, n, size, cap = case
    for layout in (SEP, TILED):
        run_workload(_ragged(world, rank, g, p, n, size, cap), layout=layout, source=source)


@pytest.mark.parametrize("inside", [True, False])
def test_full_gradient_overflow_only_in_own_pieces(inside):
    """+inf in the full gradient flags the step only when it falls in this rank's
    pieces; another rank's inf is not this rank's business."""
    w = _ragged(4, 2, "bf16", "bf16", 7, 4099, 9000)
    rig = Rig(w, layout=TILED)
    segs = rig.lay.segments
    goff, _lo, ln, _v = segs[1]
    at = goff + ln // 2 if inside else (goff + ln + 5 if rig.w.rank < 3 else goff - 5)
    NS = rig.pl.padded_numel
    full = W.make_full_grads(w, NS, rig.lay.tensor_flat_off, 1, step=1, inf_at=at)
    sl = [OS.read_pieces(storage(full[0, :NS]), segs)]
    assert bool(np.isinf(OC.widen(sl[0], "bf16")).any()) == inside
    rig.fused(full.to("cuda"), rig.A, rig.B, 1, count=1, layout=Z.ZERO_GRAD_FULL, ld=0)
    torch.cuda.synchronize()
    assert int(rig.flag.item()) == int(inside)
    res = OS.shard_step(sl, "bf16", "bf16", w.world, rig.p0, rig.m0, rig.v0, lr=w.lr,
                        weight_decay=w.weight_decay, t=1)
    assert res.flag == inside
    got = rig.unpack(rig.A if inside else rig.B)
    if inside:
        assert np.array_equal(got[0].view(np.uint32), rig.p0.view(np.uint32))
    else:
        assert np.array_equal(got[0].view(np.uint32), res.master.view(np.uint32))
    gref = rig.gather0.copy()
    OS.write_gather(gref, segs, res.params)
    assert np.array_equal(rig.gather_np(), gref)


# ---------------------------------------------------------------------------
# per-parameter dim-0 layout (FSDP2 fully_shard): one piece per parameter
# ---------------------------------------------------------------------------

def _dim0(tensors, world, rank, g, p, **kw):
    kw.setdefault("weight_decay", 0.05)
    return W.Workload(name=f"dim0_{len(tensors)}t_n{world}_r{rank}_{g}_{p}", tensors=tuple(tensors),
                      world=world, rank=rank, bucket_cap=0, grad_dtype=g, param_dtype=p, lr=1e-3,
                      steps=2, seed=11, plan_layout="dim0", **kw)


@pytest.mark.parametrize("rank", [0, 1])
def test_dim0_page_mlp(rank):
    """The handbook's FSDP2 example model on 2 ranks (weights (256, 64), (10, 256))."""
    tm = [("0.weight", (256, 64)), ("0.bias", (256,)), ("2.weight", (10, 256)), ("2.bias", (10,))]
    run_workload(_dim0(tm, 2, rank, "f32", "f32"), layout=TILED)
    run_workload(_dim0(tm, 2, rank, "bf16", "bf16"))


@pytest.mark.parametrize("source", ["slices", "stored", "full"])
@pytest.mark.parametrize("g,p", [("bf16", "bf16"), ("f16", "f16"), ("f32", "f32")])
@pytest.mark.parametrize("world,rank,n_layer", [(8, 7, 2), (8, 3, 4), (16, 0, 1)])
def test_dim0_gpt2_shapes(world, rank, n_layer, g, p, source):
    """GPT-2-shaped parameter lists (d = 64): 28 to 52 pieces, several launch
    groups, pieces of every size down to a few elements."""
    ts = W.gpt2(n_layer=n_layer, d=64, vocab=503, n_ctx=96)
    ls = 256.0 if g == "f16" else 1.0
    run_workload(_dim0(ts, world, rank, g, p, loss_scale=ls), layout=TILED, source=source)


def test_dim0_clipped():
    ts = W.gpt2(n_layer=3, d=64, vocab=503, n_ctx=96)
    run_workload(_dim0(ts, 8, 5, "bf16", "bf16", max_norm=0.02), layout=TILED)


# ---------------------------------------------------------------------------
# seeded random configurations: layout, sizes, world, rank, dtypes, source,
# clip and state layout drawn together
# ---------------------------------------------------------------------------

def _random_workload(seed):
    rng = np.random.default_rng(1000 + seed)
    world = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 64]))
    rank = int(rng.integers(0, world))
    g = str(rng.choice(["f32", "bf16", "f16"]))
    p = str(rng.choice(["f32", "bf16", "f16"]))
    dim0 = bool(rng.random() < 0.3)
    n_t = int(rng.integers(1, 40))
    if dim0:
        tensors = tuple((f"t{i}", tuple(int(x) for x in rng.integers(0, 60, size=int(rng.integers(1, 3)))))
                        for i in range(n_t))
    else:
        tensors = tuple((f"t{i}", (int(rng.integers(0, 3000)),)) for i in range(n_t))
    if sum(int(np.prod(s)) for _n, s in tensors) == 0:
        tensors = tensors + (("extra", (17,)),)
    cap = int(rng.choice([0, 0, 500, 2000, 7000]))
    source = str(rng.choice(["slices", "slices", "stored", "full", "full_n"]))
    clip = rng.random() < 0.3
    return W.Workload(name=f"random{seed}", tensors=tensors, world=world, rank=rank, bucket_cap=cap,
                      grad_dtype=g, param_dtype=p, lr=float(rng.choice([1e-3, 3e-4, 1e-2])),
                      weight_decay=float(rng.choice([0.0, 0.1])),
                      loss_scale=float(rng.choice([1.0, 256.0])) if g == "f16" else 1.0,
                      max_norm=0.01 if clip else 0.0, steps=2, seed=seed,
                      plan_layout="dim0" if dim0 else "flat"), source, int(rng.choice([SEP, TILED]))


@pytest.mark.parametrize("seed", range(64))
def test_random_configurations(seed):
    w, source, layout = _random_workload(seed)
    run_workload(w, layout=layout, source=source)


@pytest.mark.parametrize("case", ["ragged", "dim0_many", "flat"])
def test_full_gradient_clipped(case):
    """ZeRO-1 with global-norm clipping: the reduction pass reads the rank's
    pieces of the full gradient (several launches when the pieces exceed one
    launch's 192)."""
    if case == "ragged":
        w = _ragged(4, 2, "bf16", "bf16", 70, 97, 150)
    elif case == "dim0_many":
        w = _dim0(W.gpt2(n_layer=20, d=64, vocab=503, n_ctx=96), 8, 5, "bf16", "bf16")
    else:
        w = _ragged(8, 7, "f16", "f16", 1, 100_003, 0)
    w = dataclasses.replace(w, max_norm=0.02)
    for layout in (SEP, TILED):
        run_workload(w, layout=layout, source="full")


# ---------------------------------------------------------------------------
# the device piece table: one launch for any number of pieces
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("source", ["slices", "stored", "full"])
@pytest.mark.parametrize("clip", [False, True])
def test_piece_table_many_pieces(source, clip):
    """A dim-0 layout of 244 pieces per rank with the piece table attached: the
    whole shard in one launch, equal to the oracle (the same layout without
    the table takes two launches, covered above)."""
    w = _dim0(W.gpt2(n_layer=20, d=64, vocab=503, n_ctx=96), 8, 5, "bf16", "bf16",
              max_norm=(0.02 if clip else 0.0))
    for layout in (SEP, TILED):
        run_workload(w, layout=layout, source=source, table=True)


@pytest.mark.parametrize("source", ["full", "full_n"])
def test_piece_table_lifts_the_tile_limit(source):
    """300 one-element parameters and a large one on 2 ranks: the first
    2048-element tile holds more than 192 pieces, which the full-gradient
    reduction refuses without the table and serves with it."""
    tm = [(f"s{i}", (1,)) for i in range(300)] + [("big", (5000,))]
    w = _dim0(tm, 2, 1, "f32", "f32", max_norm=0.5)
    run_workload(w, layout=TILED, source=source, table=True)
    run_workload(dataclasses.replace(w, max_norm=0.0), layout=TILED, source=source, table=True)
