"""Randomised agreement of the library's planners with the oracle planners
(flat buckets and the per-parameter dim-0 layout) over many small tensor
lists, world sizes and bucket caps, including zero-size tensors."""
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import zero_sharded_mixed_plan_amd as Z
from oracle import plan as OP


def _same(p, o, world):
    assert (p.shard_numel, p.total_numel, p.padded_numel) == (o.shard_numel, o.psi, o.padded_numel)
    assert p.num_buckets == len(o.buckets)
    for b, ob in enumerate(o.buckets):
        assert p.bucket(b) == (ob.base, ob.numel, ob.padded, ob.shard, ob.first_tensor, ob.n_tensors)
    for i in range(len(o.numels)):
        assert p.tensor(i) == (o.tensor_bucket[i], o.tensor_offset[i])
    for r in sorted({0, world // 2, world - 1}):
        assert p.segments(r) == OP.rank_segments(o, r)


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(sizes=st.lists(st.integers(0, 5000), min_size=1, max_size=40).filter(lambda s: sum(s) > 0),
       world=st.integers(1, 70), cap=st.integers(-1, 6000))
def test_flat_planner_agrees(sizes, world, cap):
    _same(Z.Plan(sizes, world, cap), OP.make_plan(sizes, world, cap), world)


shape = st.lists(st.integers(0, 40), min_size=0, max_size=3).map(tuple)


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(shapes=st.lists(shape, min_size=1, max_size=25), world=st.integers(1, 33))
def test_dim0_planner_agrees(shapes, world):
    numels = []
    for s in shapes:
        n = 1
        for x in s:
            n *= x
        numels.append(n)
    if sum(numels) == 0:
        with pytest.raises(Z.ZeroError):
            Z.Plan.dim0(shapes, world)
        return
    _same(Z.Plan.dim0(shapes, world), OP.make_plan_dim0(shapes, world), world)
