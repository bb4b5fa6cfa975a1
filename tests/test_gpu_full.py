"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (slice stride rounded up to 64 elements, one-shot grids).

The optimizer state uses the benchmark's tiled layout.  The step is
elementwise, so the oracle computes sampled elements one by one:
2^18 random local indices plus every piece boundary and the shard's ends.
Properties that hold at any size cover the rest: the gather buffer outside the
rank's pieces is untouched, the overflow flag is exact, and the norm equals a
float64 library sum over the GPU's reduced gradient (whose sampled elements are
bit-exact against the oracle)."""
import numpy as np
import pytest
import torch

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from gpu_harness import CODE, check_params, compare_step, oracle_layout, say, storage
from zero_sharded_mixed_plan_amd.optim import pack_state, state_arg_dict
from oracle import casts as OC
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


def _sample_idx(S, segments, n=1 << 18, seed=0):
    rng = np.random.default_rng(seed)
    idx = [rng.integers(0, S, n)]
    edges = [0, S]
    for _goff, lo, ln, valid in segments:
        edges += [lo, lo + ln, lo + valid]
    for e in edges:
        idx.append(np.arange(max(0, e - 16), min(S, e + 16)))
    return np.unique(np.concatenate(idx)).astype(np.int64)


def _take(t, idx_dev):
    return storage(t.index_select(0, idx_dev))


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
    # the benchmark's state layout: tiles of master|m|v
    layout, T = Z.ZERO_STATE_TILED, Z.ZERO_STATE_TILE
    p0, m0, v0 = W.make_state(w, lay, dev)
    A = [pack_state(p0, m0, v0, plan.state_numel(layout))]
    del p0, m0, v0
    B = [torch.empty_like(A[0])]
    pdt = W.torch_dtype(w.param_dtype)
    gather = torch.full((pl.padded_numel,), SENTINEL[w.param_dtype], dtype=pdt, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    clip = w.max_norm > 0
    if clip:
        g = torch.empty(S, dtype=torch.float32, device=dev)
        ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device=dev)
        sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        coef = torch.zeros(1, dtype=torch.float32, device=dev)
    idx = _sample_idx(S, lay.segments, seed=w.seed)
    idx_dev = torch.from_numpy(idx).to(dev)
    # local index -> gather index for the sampled elements
    gidx = np.empty_like(idx)
    for goff, lo, ln, _v in lay.segments:
        sel = (idx >= lo) & (idx < lo + ln)
        gidx[sel] = idx[sel] - lo + goff
    gidx_dev = torch.from_numpy(gidx).to(dev)
    soff = (idx // T) * 3 * T + idx % T
    soff_dev = [torch.from_numpy(soff + i * T).to(dev) for i in range(3)]

    def take_state(bufs):
        return tuple(_take(bufs[0], soff_dev[i]) for i in range(3))
    st = torch.cuda.current_stream().cuda_stream
    cur, nxt = A, B
    t = w.t0
    slices = None
    steps = 3 if w.inject_inf_step is not None else 1
    for step in range(1, steps + 1):
        slices = W.make_slices(w, lay, step=step, ld=ld, device=dev, out=slices)
        p_in, m_in, v_in = take_state(cur)
        sl = [_take(slices[k, :S], idx_dev) for k in range(w.world)]
        common = dict(rank=w.rank, gather=gather.data_ptr(), param_dtype=CODE[w.param_dtype],
                      lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                      weight_decay=w.weight_decay, step=t + 1)
        kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                  t=t + 1, inv_scale=1.0 / w.loss_scale)
        if clip:
            Z.zero_reduce_shard(plan, slices.data_ptr(), ld, CODE[w.grad_dtype], 1.0 / w.loss_scale,
                                g.data_ptr(), ws.data_ptr(), True, st)
            Z.zero_shard_norm(plan, ws.data_ptr(), 0.0, w.max_norm, flag.data_ptr(),
                              sumsq.data_ptr(), coef.data_ptr(), st)
            a = Z.adam_args(g_stash=g.data_ptr(), clip_coef=coef.data_ptr(), skip_in=flag.data_ptr(),
                            **state_arg_dict(layout, cur, cur), **common)
            Z.zero_adam_step(plan, a, st)
            torch.cuda.synchronize()
            q = float(sumsq.item())
            q_lib = float(torch.sum(g.double() * g.double()).item())
            assert abs(q - q_lib) <= 1e-9 * q_lib, (q, q_lib)
            c32 = F(coef.item())
            assert c32 == OS.clip_coefficient(q, w.max_norm)
            res = OS.shard_step(sl, w.grad_dtype, w.param_dtype, w.world, p_in, m_in, v_in,
                                max_norm=w.max_norm, clip_override=c32, **kw)
            assert np.array_equal(_take(g, idx_dev).view(np.uint32), res.g.view(np.uint32))
            out = cur
            say(f"  q={q:.6g} norm={np.sqrt(q):.6g} clip={float(c32):.6g}")
        else:
            a = Z.adam_args(grad=slices.data_ptr(), grad_ld=ld, grad_dtype=CODE[w.grad_dtype],
                            inv_scale=1.0 / w.loss_scale, overflow_out=flag.data_ptr(),
                            **state_arg_dict(layout, cur, nxt), **common)
            Z.zero_adam_step(plan, a, st)
            torch.cuda.synchronize()
            res = OS.shard_step(sl, w.grad_dtype, w.param_dtype, w.world, p_in, m_in, v_in, **kw)
        flag_gpu = int(flag.item())
        injected = w.inject_inf_step == step
        say(f"  step {step}: flag {flag_gpu} (injected inf: {injected})")
        assert flag_gpu == int(injected)
        if not clip:
            # a sample may miss the injected element: the flag is decided on the whole shard
            out = cur if flag_gpu else nxt
        gp, gm, gv = take_state(out)
        if injected:
            for a_, b_ in ((gp, p_in), (gm, m_in), (gv, v_in)):
                assert np.array_equal(a_.view(np.uint32), b_.view(np.uint32))
        else:
            g_used = res.g if not clip else np.multiply(res.g, res.clip, dtype=F)
            n, tot = compare_step(gp, gm, gv, res, p_in, m_in, v_in, g_used,
                                  OS.adam_consts(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay,
                                                 t + 1), f"{name} step {step}")
            assert n == tot, f"{tot - n} sampled state elements differ in the last bit"
        # the sampled gather elements hold the rounded master the state now has
        want = OC.narrow(gp, w.param_dtype)
        got = _take(gather, gidx_dev)
        check_params(got, want, w.param_dtype, f"{name} step {step} params")
        if not flag_gpu:
            t += 1
            if not clip:
                cur, nxt = nxt, cur
    # nothing outside the rank's pieces was written
    sent = torch.tensor(SENTINEL[w.param_dtype], dtype=pdt, device=dev)
    prev = 0
    for goff, _lo, ln, _v in sorted(lay.segments):
        if goff > prev:
            assert bool(torch.all(gather[prev:goff] == sent)), f"write before piece at {goff}"
        prev = goff + ln
    if prev < pl.padded_numel:
        assert bool(torch.all(gather[prev:] == sent)), "write after the last piece"
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
    ld = (S + 63) // 64 * 64
    say(f"full gpt2 {variant}: S={S} pieces={len(lay.segments)}")
    idx = _sample_idx(S, lay.segments, seed=3)
    idx_dev = torch.from_numpy(idx).to(dev)
    gidx = np.empty_like(idx)
    for goff, lo, ln, _v in lay.segments:
        sel = (idx >= lo) & (idx < lo + ln)
        gidx[sel] = idx[sel] - lo + goff
    gidx_dev = torch.from_numpy(gidx).to(dev)
    st = torch.cuda.current_stream().cuda_stream
    kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, t=w.t0 + 1,
              inv_scale=1.0 / w.loss_scale)
    if variant == "reduce_only":
        slices = W.make_slices(w, lay, step=1, ld=ld, device=dev)
        g = torch.empty(S, dtype=torch.float32, device=dev)
        ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device=dev)
        Z.zero_reduce_shard(plan, slices.data_ptr(), ld, CODE[w.grad_dtype], 1.0, g.data_ptr(),
                            ws.data_ptr(), True, st)
        torch.cuda.synchronize()
        sl = [_take(slices[k, :S], idx_dev) for k in range(w.world)]
        want = OS.unscale(OS.average(OS.reduce_slices(sl, w.grad_dtype), w.world), 1.0)
        assert np.array_equal(_take(g, idx_dev).view(np.uint32), want.view(np.uint32))
        return
    layout, T = Z.ZERO_STATE_TILED, Z.ZERO_STATE_TILE
    p0, m0, v0 = W.make_state(w, lay, dev)
    A = [pack_state(p0, m0, v0, plan.state_numel(layout))]
    del p0, m0, v0
    B = [torch.empty_like(A[0])]
    gather = torch.full((pl.padded_numel,), SENTINEL[w.param_dtype], dtype=W.torch_dtype(w.param_dtype),
                        device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    soff = (idx // T) * 3 * T + idx % T
    p_in, m_in, v_in = (_take(A[0], torch.from_numpy(soff + i * T).to(dev)) for i in range(3))
    if variant == "stored":
        grads = W.make_slices(dataclasses.replace(w, world=1), lay, step=1, ld=ld, device=dev)
        gkw = dict(grad_ld=0, grad_count=1)
        sl = [_take(grads[0, :S], idx_dev)]
    elif variant == "full":
        grads = W.make_full_grads(w, pl.padded_numel, lay.tensor_flat_off, 1, step=1, device=dev)
        gkw = dict(grad_ld=0, grad_count=1, grad_layout=Z.ZERO_GRAD_FULL)
        sl = [_take(grads[0], gidx_dev)]
    else:
        grads = W.make_slices(w, lay, step=1, ld=ld, device=dev)
        gkw = dict(grad_ld=ld)
        sl = [_take(grads[k, :S], idx_dev) for k in range(w.world)]
    a = Z.adam_args(grad=grads.data_ptr(), grad_dtype=CODE[w.grad_dtype], inv_scale=1.0 / w.loss_scale,
                    overflow_out=flag.data_ptr(), rank=w.rank, gather=gather.data_ptr(),
                    param_dtype=CODE[w.param_dtype], lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                    weight_decay=w.weight_decay, step=w.t0 + 1, **gkw,
                    **state_arg_dict(layout, A, B))
    Z.zero_adam_step(plan, a, st)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    res = OS.shard_step(sl, w.grad_dtype, w.param_dtype, w.world, p_in, m_in, v_in, **kw)
    gp, gm, gv = (_take(B[0], torch.from_numpy(soff + i * T).to(dev)) for i in range(3))
    n, tot = compare_step(gp, gm, gv, res, p_in, m_in, v_in, res.g,
                          OS.adam_consts(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.t0 + 1),
                          f"gpt2 {variant}")
    assert n == tot, f"{tot - n} sampled state elements differ in the last bit"
    check_params(_take(gather, gidx_dev), OC.narrow(gp, w.param_dtype), w.param_dtype, f"gpt2 {variant}")
    # nothing outside the rank's pieces was written
    sent = torch.tensor(SENTINEL[w.param_dtype], dtype=gather.dtype, device=dev)
    written = torch.zeros(pl.padded_numel, dtype=torch.bool, device=dev)
    for goff, _lo, ln, _v in lay.segments:
        written[goff:goff + ln] = True
    assert bool(torch.all(gather[~written] == sent))
    del A, B, gather, grads


@pytest.mark.parametrize("clip", [False, True])
def test_shard_beyond_int32(clip):
    """A shard longer than 2^31 elements (one flat tensor, N = 2, rank 1, a
    ragged end): every index in the kernels and the host is 64-bit.  Sampled
    elements, including a window around 2^31 and the shard's end, against the
    oracle; the gather buffer outside the rank's piece is untouched.  About 100
    GB of device memory at the peak."""
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
    idx = np.unique(np.concatenate([_sample_idx(S, lay.segments, n=1 << 16, seed=5),
                                    np.arange((1 << 31) - 64, (1 << 31) + 64)])).astype(np.int64)
    idx_dev = torch.from_numpy(idx).to(dev)
    gidx_dev = torch.from_numpy(idx + lay.segments[0][0]).to(dev)
    layout, T = Z.ZERO_STATE_TILED, Z.ZERO_STATE_TILE
    p0, m0, v0 = W.make_state(w, lay, dev)
    A = [pack_state(p0, m0, v0, plan.state_numel(layout))]
    del p0, m0, v0
    torch.cuda.empty_cache()
    soff = (idx // T) * 3 * T + idx % T
    soff_dev = [torch.from_numpy(soff + i * T).to(dev) for i in range(3)]
    p_in, m_in, v_in = (_take(A[0], soff_dev[i]) for i in range(3))
    gather = torch.full((pl.padded_numel,), SENTINEL["bf16"], dtype=torch.bfloat16, device=dev)
    slices = W.make_slices(w, lay, step=1, ld=ld, device=dev)
    sl = [_take(slices[k, :S], idx_dev) for k in range(w.world)]
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    common = dict(rank=w.rank, gather=gather.data_ptr(), param_dtype=CODE["bf16"], lr=w.lr, beta1=w.beta1,
                  beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=w.t0 + 1)
    kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, t=w.t0 + 1,
              inv_scale=1.0)
    say("  inputs ready")
    if clip:
        g = torch.empty(S, dtype=torch.float32, device=dev)
        ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device=dev)
        sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        coef = torch.zeros(1, dtype=torch.float32, device=dev)
        Z.zero_reduce_shard(plan, slices.data_ptr(), ld, CODE["bf16"], 1.0, g.data_ptr(), ws.data_ptr(), True, st)
        Z.zero_shard_norm(plan, ws.data_ptr(), 0.0, w.max_norm, flag.data_ptr(), sumsq.data_ptr(),
                          coef.data_ptr(), st)
        a = Z.adam_args(g_stash=g.data_ptr(), clip_coef=coef.data_ptr(), skip_in=flag.data_ptr(),
                        **state_arg_dict(layout, A, A), **common)
        Z.zero_adam_step(plan, a, st)
        torch.cuda.synchronize()
        c32 = F(coef.item())
        res = OS.shard_step(sl, "bf16", "bf16", w.world, p_in, m_in, v_in, max_norm=w.max_norm,
                            clip_override=c32, **kw)
        assert np.array_equal(_take(g, idx_dev).view(np.uint32), res.g.view(np.uint32))
        q = float(sumsq.item())
        q_lib = float(sum(torch.sum(ch.double() ** 2).item() for ch in torch.split(g, 1 << 28)))
        assert abs(q - q_lib) <= 1e-9 * q_lib, (q, q_lib)
        out = A
        del g, ws
    else:
        B = [torch.empty_like(A[0])]
        a = Z.adam_args(grad=slices.data_ptr(), grad_ld=ld, grad_dtype=CODE["bf16"], overflow_out=flag.data_ptr(),
                        **state_arg_dict(layout, A, B), **common)
        Z.zero_adam_step(plan, a, st)
        torch.cuda.synchronize()
        res = OS.shard_step(sl, "bf16", "bf16", w.world, p_in, m_in, v_in, **kw)
        out = B
    assert int(flag.item()) == 0
    say("  step done")
    gp, gm, gv = (_take(out[0], soff_dev[i]) for i in range(3))
    g_used = res.g if not clip else np.multiply(res.g, res.clip, dtype=F)
    n, tot = compare_step(gp, gm, gv, res, p_in, m_in, v_in, g_used,
                          OS.adam_consts(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.t0 + 1), "beyond int32")
    assert n == tot, f"{tot - n} sampled state elements differ in the last bit"
    check_params(_take(gather, gidx_dev), OC.narrow(gp, "bf16"), "bf16", "beyond int32 params")
    goff = lay.segments[0][0]
    sent = torch.tensor(SENTINEL["bf16"], dtype=torch.bfloat16, device=dev)
    assert bool(torch.all(gather[:goff] == sent)) and bool(torch.all(gather[goff + S:] == sent))
    del A, out, gather, slices
