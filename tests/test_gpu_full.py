"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (slice stride rounded up to 64 elements, one-shot grids).

The optimizer state uses the benchmark's tiled layout.  Every element of the
rank's shard is compared with the oracle (master, m, v and the gather slots,
bit for bit; the clipped path's fp32 stash too), chunk by chunk on the host's
threads (tests/shard_check.py).  Besides: the gather buffer outside the rank's
pieces keeps its sentinel, the tiled state's positions past S keep theirs, the
overflow flag equals the oracle's over the whole shard, and the norm equals
both the oracle's and a float64 library sum over the GPU's reduced gradient."""
import numpy as np
import pytest
import torch

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from gpu_harness import CODE, oracle_layout, plant_tail, say, tail_intact
from shard_check import check_reduction, check_whole_shard, full_grads, outside_slots_untouched, shard_grads
from zero_sharded_mixed_plan_amd.optim import pack_state, state_arg_dict
from oracle import step as OS

pytestmark = pytest.mark.gpu
F = np.float32
SENTINEL = {"f32": 7.0, "bf16": -3.0, "f16": 5.0}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def _tiled_state(w, lay, plan, dev):
    p0, m0, v0 = W.make_state(w, lay, dev)
    A = pack_state(p0, m0, v0, plan.state_numel(Z.ZERO_STATE_TILED))
    del p0, m0, v0
    B = torch.empty_like(A)
    plant_tail(A, lay.S)
    plant_tail(B, lay.S)
    return A, B


@pytest.mark.parametrize("name", W.ORDER)
def test_full_size(name):
    w = W.FULL[name]
    pl, lay = oracle_layout(w)
    S = lay.S
    dev = torch.device("cuda")
    plan = Z.Plan(W.numels(w.tensors), w.world, w.bucket_cap)
    assert plan.shard_numel == S and plan.segments(w.rank) == lay.segments
    ld = (S + 63) // 64 * 64
    say(f"full {name}: S={S} N={w.world} rank={w.rank} pieces={len(lay.segments)} ld={ld}")
    layout = Z.ZERO_STATE_TILED
    A, B = _tiled_state(w, lay, plan, dev)
    pdt = W.torch_dtype(w.param_dtype)
    gather = torch.full((pl.padded_numel,), SENTINEL[w.param_dtype], dtype=pdt, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    clip = w.max_norm > 0
    if clip:
        g = torch.empty(S, dtype=torch.float32, device=dev)
        ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device=dev)
        sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        coef = torch.zeros(1, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    cur, nxt = A, B
    t = w.t0
    slices = None
    steps = 3 if w.inject_inf_step is not None else 1
    for step in range(1, steps + 1):
        slices = W.make_slices(w, lay, step=step, ld=ld, device=dev, out=slices)
        snap = cur.clone()          # the step's input state, for the oracle
        common = dict(rank=w.rank, gather=gather.data_ptr(), param_dtype=CODE[w.param_dtype],
                      lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                      weight_decay=w.weight_decay, step=t + 1)
        c32 = g_gpu = None
        if clip:
            Z.zero_reduce_shard(plan, slices.data_ptr(), ld, CODE[w.grad_dtype], 1.0 / w.loss_scale,
                                g.data_ptr(), ws.data_ptr(), True, st)
            Z.zero_shard_norm(plan, ws.data_ptr(), 0.0, w.max_norm, flag.data_ptr(),
                              sumsq.data_ptr(), coef.data_ptr(), st)
            a = Z.adam_args(g_stash=g.data_ptr(), clip_coef=coef.data_ptr(), skip_in=flag.data_ptr(),
                            **state_arg_dict(layout, [cur], [cur]), **common)
            Z.zero_adam_step(plan, a, st)
            torch.cuda.synchronize()
            c32, g_gpu = F(coef.item()), g
        else:
            a = Z.adam_args(grad=slices.data_ptr(), grad_ld=ld, grad_dtype=CODE[w.grad_dtype],
                            inv_scale=1.0 / w.loss_scale, overflow_out=flag.data_ptr(),
                            **state_arg_dict(layout, [cur], [nxt]), **common)
            Z.zero_adam_step(plan, a, st)
            torch.cuda.synchronize()
        flag_gpu = int(flag.item())
        injected = w.inject_inf_step == step
        say(f"  step {step}: flag {flag_gpu} (injected inf: {injected})")
        assert flag_gpu == int(injected)
        # a fused step leaves its result in the other buffer, unless it was not applied
        out = cur if (clip or flag_gpu) else nxt
        if not clip:
            assert torch.equal(cur.view(torch.int32), snap.view(torch.int32)), "input state changed"
        n, oracle_flag, q_ora = check_whole_shard(
            S=S, w=w, t=t + 1, grads_of=shard_grads(slices, w.world), state_in=snap, state_out=out,
            gather=gather, segments=lay.segments, flag=flag_gpu, c32=c32, g_gpu=g_gpu,
            chunk=(1 << 20 if w.world > 16 else 1 << 22), what=f"{name} step {step}")
        assert oracle_flag == bool(flag_gpu)
        say(f"  every element of [0, {n}) equal to the oracle bit for bit")
        if clip:
            q = float(sumsq.item())
            q_lib = float(sum(torch.sum(ch.double() ** 2).item() for ch in torch.split(g, 1 << 28)))
            assert abs(q - q_lib) <= 1e-9 * q_lib, (q, q_lib)
            assert abs(q - q_ora) <= 1e-9 * q_ora, (q, q_ora)
            assert c32 == OS.clip_coefficient(q, w.max_norm)
            say(f"  q={q:.6g} norm={np.sqrt(q):.6g} clip={float(c32):.6g}")
        del snap
        if not flag_gpu:
            t += 1
            if not clip:
                cur, nxt = nxt, cur
    assert outside_slots_untouched(gather, lay.segments, SENTINEL[w.param_dtype]), "write outside the slots"
    assert tail_intact(A, S) and tail_intact(B, S), "tiled state written past S"
    del A, B, gather, slices


# Shards just past the library's launch size (2^26 elements per launch; 2^23
# for the 64-buffer four-element form), so that a step runs as two launches
# with a short, ragged second one: the eight-element fused update (8 bf16
# slices, S = 8 mod 8 + 5), the 64-buffer form (S = 2 mod 4) and the clipped
# path (reduction of 16 bf16 slices, then the stash update).  Every element
# against the oracle, as above.
BOUNDARY_CASES = {
    "step8": dict(world=8, S=(1 << 26) + 3 * 2048 + 5, g="bf16", clip=False, loss_scale=1.0),
    "narrow64": dict(world=64, S=(1 << 23) + 2048 + 6, g="f16", clip=False, loss_scale=1024.0),
    "clip16": dict(world=16, S=(1 << 26) + 2048 + 7, g="bf16", clip=True, loss_scale=1.0),
}


@pytest.mark.parametrize("case", list(BOUNDARY_CASES))
def test_launch_boundaries(case):
    cfg = BOUNDARY_CASES[case]
    N, S_want = cfg["world"], cfg["S"]
    w = W.Workload(name=f"boundary_{case}", tensors=(("flat", (N * S_want - 3,)),), world=N, rank=N - 1,
                   bucket_cap=0, grad_dtype=cfg["g"], param_dtype=cfg["g"], lr=1e-3, weight_decay=0.1,
                   loss_scale=cfg["loss_scale"], max_norm=(0.05 if cfg["clip"] else 0.0), steps=1, seed=41,
                   m_sigma=1e-3, v_sigma=1e-6)
    pl, lay = oracle_layout(w)
    S = lay.S
    assert S == S_want
    dev = torch.device("cuda")
    plan = Z.Plan(W.numels(w.tensors), w.world, w.bucket_cap)
    assert plan.shard_numel == S and plan.segments(w.rank) == lay.segments
    ld = (S + 63) // 64 * 64
    say(f"launch boundary {case}: S={S} N={N} ld={ld}")
    layout = Z.ZERO_STATE_TILED
    A, B = _tiled_state(w, lay, plan, dev)
    pdt = W.torch_dtype(w.param_dtype)
    gather = torch.full((pl.padded_numel,), SENTINEL[w.param_dtype], dtype=pdt, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    slices = W.make_slices(w, lay, step=1, ld=ld, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    common = dict(rank=w.rank, gather=gather.data_ptr(), param_dtype=CODE[w.param_dtype], lr=w.lr,
                  beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=w.t0 + 1)
    c32 = g = None
    if cfg["clip"]:
        g = torch.empty(S, dtype=torch.float32, device=dev)
        ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device=dev)
        sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        coef = torch.zeros(1, dtype=torch.float32, device=dev)
        Z.zero_reduce_shard(plan, slices.data_ptr(), ld, CODE[w.grad_dtype], 1.0 / w.loss_scale,
                            g.data_ptr(), ws.data_ptr(), True, st)
        Z.zero_shard_norm(plan, ws.data_ptr(), 0.0, w.max_norm, flag.data_ptr(), sumsq.data_ptr(),
                          coef.data_ptr(), st)
        B.copy_(A)
        a = Z.adam_args(g_stash=g.data_ptr(), clip_coef=coef.data_ptr(), skip_in=flag.data_ptr(),
                        **state_arg_dict(layout, [B], [B]), **common)
    else:
        a = Z.adam_args(grad=slices.data_ptr(), grad_ld=ld, grad_dtype=CODE[w.grad_dtype],
                        inv_scale=1.0 / w.loss_scale, overflow_out=flag.data_ptr(),
                        **state_arg_dict(layout, [A], [B]), **common)
    Z.zero_adam_step(plan, a, st)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    if cfg["clip"]:
        c32 = F(coef.item())
    n, oracle_flag, q_ora = check_whole_shard(
        S=S, w=w, t=w.t0 + 1, grads_of=shard_grads(slices, w.world), state_in=A, state_out=B,
        gather=gather, segments=lay.segments, flag=0, c32=c32, g_gpu=g,
        chunk=(1 << 20 if w.world > 16 else 1 << 22), what=f"launch boundary {case}")
    assert not oracle_flag
    if cfg["clip"]:
        q = float(sumsq.item())
        assert abs(q - q_ora) <= 1e-9 * q_ora, (q, q_ora)
        assert c32 == OS.clip_coefficient(q, w.max_norm)
    say(f"  every element of [0, {n}) equal to the oracle bit for bit")
    assert outside_slots_untouched(gather, lay.segments, SENTINEL[w.param_dtype]), "write outside the slots"
    assert tail_intact(A, S) and tail_intact(B, S), "tiled state written past S"
    del A, B, gather, slices


# The benchmark's other forms of the GPT-2 step, at full size: one stored
# reduce-scatter output, one full all-reduced gradient (ZeRO-1), the
# per-parameter dim-0 layout (580 pieces), and the reduction pass alone.
VARIANTS = ["stored", "full", "dim0", "reduce_only"]


@pytest.mark.parametrize("variant", VARIANTS)
def test_full_size_gpt2_variants(variant):
    import dataclasses
    w = W.FULL["gpt2_1p5b_n8"]
    if variant == "dim0":
        w = dataclasses.replace(w, plan_layout="dim0")
    pl, lay = oracle_layout(w)
    S = lay.S
    dev = torch.device("cuda")
    plan = (Z.Plan.dim0([s for _n, s in w.tensors], w.world) if variant == "dim0"
            else Z.Plan(W.numels(w.tensors), w.world, w.bucket_cap))
    assert plan.shard_numel == S and plan.segments(w.rank) == lay.segments
    table = None
    if plan.num_buckets > 192:   # as the benchmark does: the device piece table, one launch
        table = torch.empty(plan.piece_table_bytes(), dtype=torch.uint8, device=dev)
        plan.attach_piece_table(w.rank, table.data_ptr(), table.numel())
    ld = (S + 63) // 64 * 64
    say(f"full gpt2 {variant}: S={S} pieces={len(lay.segments)} table={table is not None}")
    st = torch.cuda.current_stream().cuda_stream
    if variant == "reduce_only":
        slices = W.make_slices(w, lay, step=1, ld=ld, device=dev)
        g = torch.empty(S, dtype=torch.float32, device=dev)
        ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device=dev)
        sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        Z.zero_reduce_shard(plan, slices.data_ptr(), ld, CODE[w.grad_dtype], 1.0, g.data_ptr(),
                            ws.data_ptr(), True, st)
        Z.zero_shard_norm(plan, ws.data_ptr(), 0.0, 0.0, None, sumsq.data_ptr(), None, st)
        torch.cuda.synchronize()
        q_ora = check_reduction(S=S, w=w, grads_of=shard_grads(slices, w.world), g_gpu=g,
                                what="gpt2 reduce_only")
        q = float(sumsq.item())
        assert abs(q - q_ora) <= 1e-9 * q_ora, (q, q_ora)
        say(f"  every element of g over [0, {S}) equal to the oracle bit for bit; q={q:.6g}")
        return
    layout = Z.ZERO_STATE_TILED
    A, B = _tiled_state(w, lay, plan, dev)
    gather = torch.full((pl.padded_numel,), SENTINEL[w.param_dtype], dtype=W.torch_dtype(w.param_dtype),
                        device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    if variant == "stored":
        grads = W.make_slices(dataclasses.replace(w, world=1), lay, step=1, ld=ld, device=dev)
        gkw = dict(grad_ld=0, grad_count=1)
        grads_of = shard_grads(grads, 1)
    elif variant == "full":
        grads = W.make_full_grads(w, pl.padded_numel, lay.tensor_flat_off, 1, step=1, device=dev)
        gkw = dict(grad_ld=0, grad_count=1, grad_layout=Z.ZERO_GRAD_FULL)
        grads_of = full_grads(grads, 1, lay.segments)
    else:
        grads = W.make_slices(w, lay, step=1, ld=ld, device=dev)
        gkw = dict(grad_ld=ld)
        grads_of = shard_grads(grads, w.world)
    a = Z.adam_args(grad=grads.data_ptr(), grad_dtype=CODE[w.grad_dtype], inv_scale=1.0 / w.loss_scale,
                    overflow_out=flag.data_ptr(), rank=w.rank, gather=gather.data_ptr(),
                    param_dtype=CODE[w.param_dtype], lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                    weight_decay=w.weight_decay, step=w.t0 + 1, **gkw,
                    **state_arg_dict(layout, [A], [B]))
    Z.zero_adam_step(plan, a, st)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    n, oracle_flag, _ = check_whole_shard(S=S, w=w, t=w.t0 + 1, grads_of=grads_of, state_in=A, state_out=B,
                                          gather=gather, segments=lay.segments, flag=0,
                                          what=f"gpt2 {variant}")
    assert not oracle_flag
    say(f"  every element of [0, {n}) equal to the oracle bit for bit")
    assert outside_slots_untouched(gather, lay.segments, SENTINEL[w.param_dtype]), "write outside the slots"
    assert tail_intact(A, S) and tail_intact(B, S), "tiled state written past S"
    del A, B, gather, grads


@pytest.mark.parametrize("clip", [False, True])
def test_shard_beyond_int32(clip):
    """A shard longer than 2^31 elements (one flat tensor, N = 2, rank 1, a
    ragged end): every index in the kernels and the host is 64-bit.  Every
    element against the oracle; the gather buffer outside the rank's piece is
    untouched.  About 130 GB of device memory at the peak."""
    S_want = (1 << 31) + 4099
    w = W.Workload(name="beyond_int32", tensors=(("flat", (2 * S_want - 3,)),), world=2, rank=1, bucket_cap=0,
                   grad_dtype="bf16", param_dtype="bf16", lr=1e-3, weight_decay=0.1, steps=1, seed=29,
                   max_norm=(0.05 if clip else 0.0))
    pl, lay = oracle_layout(w)
    S = lay.S
    assert S > (1 << 31)
    dev = torch.device("cuda")
    plan = Z.Plan(W.numels(w.tensors), w.world, w.bucket_cap)
    assert plan.shard_numel == S
    ld = (S + 63) // 64 * 64
    say(f"beyond int32: S={S} clip={clip}")
    layout = Z.ZERO_STATE_TILED
    A, B = _tiled_state(w, lay, plan, dev)
    torch.cuda.empty_cache()
    gather = torch.full((pl.padded_numel,), SENTINEL["bf16"], dtype=torch.bfloat16, device=dev)
    slices = W.make_slices(w, lay, step=1, ld=ld, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    common = dict(rank=w.rank, gather=gather.data_ptr(), param_dtype=CODE["bf16"], lr=w.lr, beta1=w.beta1,
                  beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=w.t0 + 1)
    say("  inputs ready")
    c32 = g = None
    if clip:
        B.copy_(A)      # the clipped update runs in place on B; A keeps the input
        g = torch.empty(S, dtype=torch.float32, device=dev)
        ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device=dev)
        sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        coef = torch.zeros(1, dtype=torch.float32, device=dev)
        Z.zero_reduce_shard(plan, slices.data_ptr(), ld, CODE["bf16"], 1.0, g.data_ptr(), ws.data_ptr(), True, st)
        Z.zero_shard_norm(plan, ws.data_ptr(), 0.0, w.max_norm, flag.data_ptr(), sumsq.data_ptr(),
                          coef.data_ptr(), st)
        a = Z.adam_args(g_stash=g.data_ptr(), clip_coef=coef.data_ptr(), skip_in=flag.data_ptr(),
                        **state_arg_dict(layout, [B], [B]), **common)
        Z.zero_adam_step(plan, a, st)
        torch.cuda.synchronize()
        c32 = F(coef.item())
        del ws
    else:
        a = Z.adam_args(grad=slices.data_ptr(), grad_ld=ld, grad_dtype=CODE["bf16"], overflow_out=flag.data_ptr(),
                        **state_arg_dict(layout, [A], [B]), **common)
        Z.zero_adam_step(plan, a, st)
        torch.cuda.synchronize()
    assert int(flag.item()) == 0
    say("  step done")
    n, oracle_flag, q_ora = check_whole_shard(S=S, w=w, t=w.t0 + 1, grads_of=shard_grads(slices, w.world),
                                              state_in=A, state_out=B, gather=gather, segments=lay.segments,
                                              flag=0, c32=c32, g_gpu=g, what="beyond int32")
    assert not oracle_flag
    say(f"  every element of [0, {n}) equal to the oracle bit for bit")
    if clip:
        q = float(sumsq.item())
        assert abs(q - q_ora) <= 1e-9 * q_ora, (q, q_ora)
        assert c32 == OS.clip_coefficient(q, w.max_norm)
    assert outside_slots_untouched(gather, lay.segments, SENTINEL["bf16"]), "write outside the slot"
    assert tail_intact(A, S) and tail_intact(B, S), "tiled state written past S"
    del A, B, gather, slices, g
