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
from gpu_harness import CODE, oracle_layout, say

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


def test_noalloc_refuses_a_shard_past_the_limit():
    cap = Z.zero_noalloc_max_shard()
    assert cap == 715_302_912
    plan = Z.Plan([cap + 1], 1)
    assert plan.shard_numel == cap + 1
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_norm_noalloc(plan, 1 << 40, cap + 1, CODE["bf16"], 1.0, 0, 0.0, 1.0, 0, 0, 0)
    assert e.value.code == Z.ZERO_EINVAL and "fixed array" in Z.zero_last_error()
