"""The entry point that allocates nothing (zero_reduce_norm_noalloc) against
the calls it stands for (zero_reduce_shard + zero_shard_norm with a caller
workspace): the same stash, overflow word, sum of squares and clip coefficient
bit for bit, on two calls in a row of which the second has a smaller shard
(the library's array keeps the first call's contents), with an injected inf on
the second; and a plan past the array's limit refused before anything runs."""
import numpy as np
import pytest
import torch

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from gpu_harness import CODE, oracle_layout, round_up, say
from zero_sharded_mixed_plan_amd.optim import StepCtl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _flat(psi, world, rank, seed):
    return W.Workload(name=f"noalloc{psi}", tensors=(("x", (psi,)),), world=world, rank=rank, bucket_cap=0,
                      grad_dtype="bf16", param_dtype="bf16", lr=1e-3, weight_decay=0.1, steps=1, seed=seed,
                      max_norm=1e-3)


def _both(w, inf_at=None, other=0.0):
    """Run the no-allocation call and the two-call form on the same slices;
    return both results as host arrays."""
    _pl, lay = oracle_layout(w)
    S = lay.S
    plan = Z.Plan(W.numels(w.tensors), w.world, w.bucket_cap)
    ld = (S + 63) // 64 * 64
    sl = W.make_slices(w, lay, step=1, ld=ld, device="cuda")
    if inf_at is not None:
        sl[inf_at[0], inf_at[1]] = float("inf")
    st = torch.cuda.current_stream().cuda_stream
    out = []
    for noalloc in (True, False):
        g = torch.full((S,), 7.0, dtype=torch.float32, device="cuda")
        flag = torch.full((1,), 9, dtype=torch.int32, device="cuda")
        q = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
        c = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        if noalloc:
            Z.zero_reduce_norm_noalloc(plan, sl.data_ptr(), ld, CODE["bf16"], 1.0, g.data_ptr(), other,
                                       w.max_norm, flag.data_ptr(), q.data_ptr(), c.data_ptr(), st)
        else:
            ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device="cuda")
            Z.zero_reduce_shard(plan, sl.data_ptr(), ld, CODE["bf16"], 1.0, g.data_ptr(), ws.data_ptr(), True, st)
            Z.zero_shard_norm(plan, ws.data_ptr(), other, w.max_norm, flag.data_ptr(), q.data_ptr(),
                              c.data_ptr(), st)
        torch.cuda.synchronize()
        out.append((g.cpu().numpy(), int(flag.item()), q.cpu().numpy(), c.cpu().numpy()))
    return S, out


def _same(S, out, what):
    (g1, f1, q1, c1), (g2, f2, q2, c2) = out
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32)), f"{what}: stash differs"
    assert f1 == f2, f"{what}: flag {f1} vs {f2}"
    assert q1.view(np.uint64)[0] == q2.view(np.uint64)[0], f"{what}: sum of squares {q1[0]} vs {q2[0]}"
    assert c1.view(np.uint32)[0] == c2.view(np.uint32)[0], f"{what}: coefficient {c1[0]} vs {c2[0]}"
    say(f"{what}: S={S} flag={f1} q={q1[0]:.6g} c={c1[0]:.6g} equal bit for bit")
    return f1


def test_noalloc_matches_workspace_calls_twice():
    # first call: a shard of many tiles; second: a smaller one with an inf, so
    # the array still holds the first call's partials past the second's tiles
    big = _flat(8 * 3_000_017, 8, 5, seed=11)
    small = _flat(8 * 200_003, 8, 2, seed=12)
    S1, out1 = _both(big, other=0.25)
    assert _same(S1, out1, "first call") == 0
    S2, out2 = _both(small, inf_at=(3, 123_457))
    assert S2 < S1
    assert _same(S2, out2, "second call, smaller, with an inf") == 1
    # and once more at the first size, finite
    S3, out3 = _both(big)
    assert _same(S3, out3, "third call") == 0


def test_noalloc_full_gradient_and_step_control():
    """The other arguments it forwards: one full all-reduced gradient read at
    the rank's pieces (ZeRO-1) of a multi-bucket layout, with the loss scale
    read from step control in device memory (the inv_scale argument is then
    ignored).  Same results as the two-call form, bit for bit."""
    w = W.Workload(name="noalloc_full", tensors=(("a", (70_001,)), ("b", (3,)), ("c", (257, 129)),
                                                   ("d", (40_000,))),
                   world=4, rank=2, bucket_cap=60_000, grad_dtype="f16", param_dtype="f16", lr=1e-3,
                   weight_decay=0.0, steps=1, seed=21, loss_scale=512.0, max_norm=0.5)
    pl, lay = oracle_layout(w)
    plan = Z.Plan(W.numels(w.tensors), w.world, w.bucket_cap)
    assert plan.num_buckets > 1
    NS = pl.padded_numel
    ldf = round_up(NS, 64)
    full = W.make_full_grads(w, NS, lay.tensor_flat_off, 1, step=1, ld=ldf, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    scaler = Z.Scaler(init_scale=w.loss_scale)
    out = []
    # (no allocation, step control): the first two runs take the loss scale from
    # the control block and ignore the inv_scale argument (123); the third passes
    # 1/512 as the argument and must give the same bits
    for noalloc, use_ctl in ((True, True), (False, True), (True, False)):
        ctl = StepCtl(0, w.lr, scaler.s, False, "cuda")
        g = torch.full((lay.S,), 7.0, dtype=torch.float32, device="cuda")
        flag = torch.full((1,), 9, dtype=torch.int32, device="cuda")
        q = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
        c = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        kw = dict(grad_count=1, grad_layout=Z.ZERO_GRAD_FULL, rank=w.rank, ctl=ctl.ptr if use_ctl else 0)
        inv = 123.0 if use_ctl else 1.0 / w.loss_scale
        if noalloc:
            Z.zero_reduce_norm_noalloc(plan, full.data_ptr(), ldf, CODE["f16"], inv, g.data_ptr(), 0.0,
                                       w.max_norm, flag.data_ptr(), q.data_ptr(), c.data_ptr(), st, **kw)
        else:
            ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device="cuda")
            Z.zero_reduce_shard(plan, full.data_ptr(), ldf, CODE["f16"], inv, g.data_ptr(), ws.data_ptr(),
                                True, st, **kw)
            Z.zero_shard_norm(plan, ws.data_ptr(), 0.0, w.max_norm, flag.data_ptr(), q.data_ptr(),
                              c.data_ptr(), st)
        torch.cuda.synchronize()
        out.append((g.cpu().numpy(), int(flag.item()), q.cpu().numpy(), c.cpu().numpy()))
    assert _same(lay.S, out[:2], "full gradient, step control") == 0
    assert _same(lay.S, [out[0], out[2]], "step control against the argument") == 0


def test_noalloc_refuses_a_shard_past_the_limit():
    cap = Z.zero_noalloc_max_shard()
    assert cap == 715_302_912
    plan = Z.Plan([cap + 1], 1)
    assert plan.shard_numel == cap + 1
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_norm_noalloc(plan, 1 << 40, cap + 1, CODE["bf16"], 1.0, 0, 0.0, 1.0, 0, 0, 0)
    assert e.value.code == Z.ZERO_EINVAL and "fixed array" in Z.zero_last_error()
