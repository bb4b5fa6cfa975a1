"""Host parts of the runtime around the step, through the C ABI: the
loss-scale update against the oracle, the plan hash against its documented
definition, and the checkpoint calls' argument and file checks (each case is
rejected before any device memory is touched)."""
import os

import numpy as np
import pytest

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from ckpt_format import header, plan_hash
from oracle import plan as OP
from oracle import scaler as SC

F = np.float32
BASE = 1 << 40


@pytest.mark.parametrize("seed,interval,p,init", [(0, 3, 0.2, 65536.0), (1, 1, 0.5, 1.0), (2, 50, 0.02, 2.0 ** 24),
                                                  (3, 4, 0.95, 3.0e38), (4, 2, 0.0, 3.0e37)])
def test_scaler_matches_oracle(seed, interval, p, init):
    rng = np.random.default_rng(seed)
    flags = (rng.random(400) < p).tolist()
    c = Z.Scaler(init, 2.0, 0.5, interval)
    o = SC.ScalerState(scale=F(init), growth_tracker=0, growth_interval=interval)
    for fl in flags:
        c.update(fl)
        o = SC.update(o, fl)
        assert F(c.scale).view(np.uint32) == o.scale.view(np.uint32)
        assert c.growth_tracker == o.growth_tracker
        assert F(c.inv_scale) == SC.inv_scale(o)


@pytest.mark.parametrize("args", [(0.0, 2.0, 0.5, 10), (float("inf"), 2.0, 0.5, 10), (1.0, 1.0, 0.5, 10),
                                  (1.0, 2.0, 1.0, 10), (1.0, 2.0, 0.0, 10), (1.0, 2.0, 0.5, 0)])
def test_scaler_init_rejects(args):
    with pytest.raises(Z.ZeroError) as e:
        Z.Scaler(*args)
    assert e.value.code == Z.ZERO_EINVAL


def _oracle_hash(pl):
    return plan_hash(pl.world, list(pl.numels), [(b.numel, b.shard, b.n_tensors) for b in pl.buckets])


@pytest.mark.parametrize("make", [
    lambda: (Z.Plan(W.numels(W.toy_mlp()), 4), OP.make_plan(W.numels(W.toy_mlp()), 4)),
    lambda: (Z.Plan([10, 30, 5, 5, 1], 3, 12), OP.make_plan([10, 30, 5, 5, 1], 3, 12)),
    lambda: (Z.Plan.dim0([(256, 64), (256,), (10, 256), (10,)], 2),
             OP.make_plan_dim0([(256, 64), (256,), (10, 256), (10,)], 2)),
])
def test_plan_hash_definition(make):
    p, o = make()
    assert Z.zero_plan_hash(p) == _oracle_hash(o)


def test_plan_hash_separates_layouts():
    hs = {Z.zero_plan_hash(Z.Plan([1000, 24], 4)), Z.zero_plan_hash(Z.Plan([1000, 24], 8)),
          Z.zero_plan_hash(Z.Plan([1000, 24], 4, 500)), Z.zero_plan_hash(Z.Plan([24, 1000], 4)),
          Z.zero_plan_hash(Z.Plan.dim0([(250, 4), (24,)], 4))}
    assert len(hs) == 5
    assert Z.zero_plan_hash(Z.Plan([1000, 24], 4)) == Z.zero_plan_hash(Z.Plan([1000, 24], 4))


def _save(plan, path, **over):
    a = dict(rank=1, layout=Z.ZERO_STATE_SEPARATE, master=BASE, m=BASE + (1 << 32), v=BASE + (2 << 32))
    a.update(over)
    Z.zero_checkpoint_save(plan, a["rank"], path, a["layout"], a["master"], a["m"], a["v"], 3,
                           Z.Scaler().s)


@pytest.mark.parametrize("over,code", [
    (dict(rank=4), Z.ZERO_EINVAL), (dict(layout=5), Z.ZERO_EINVAL), (dict(m=0), Z.ZERO_EINVAL),
    (dict(layout=Z.ZERO_STATE_TILED), Z.ZERO_EINVAL),          # tiled takes master only
    (dict(master=BASE + 4), Z.ZERO_EALIGN),
])
def test_checkpoint_save_rejects(over, code, tmp_path):
    plan = Z.Plan([100], 4)
    with pytest.raises(Z.ZeroError) as e:
        _save(plan, str(tmp_path / "x"), **over)
    assert e.value.code == code, Z.zero_last_error()
    assert not os.path.exists(tmp_path / "x") and not os.path.exists(tmp_path / "x.tmp")


def test_checkpoint_save_rejects_inconsistent_meta(tmp_path):
    plan = Z.Plan([100], 4)
    bad = Z.Scaler().s
    bad.growth_tracker = bad.growth_interval
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_checkpoint_save(plan, 1, str(tmp_path / "x"), Z.ZERO_STATE_SEPARATE, BASE, BASE + (1 << 32),
                               BASE + (2 << 32), 3, bad)
    assert e.value.code == Z.ZERO_EINVAL
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_checkpoint_save(plan, 1, str(tmp_path / "x"), Z.ZERO_STATE_SEPARATE, BASE, BASE + (1 << 32),
                               BASE + (2 << 32), -1, Z.Scaler().s)
    assert e.value.code == Z.ZERO_EINVAL


def _load(plan, path, rank=1):
    return Z.zero_checkpoint_load(plan, rank, path, Z.ZERO_STATE_SEPARATE, BASE, BASE + (1 << 32),
                                  BASE + (2 << 32))


@pytest.mark.parametrize("case,code", [
    ("missing", Z.ZERO_EIO), ("magic", Z.ZERO_EIO), ("version", Z.ZERO_EIO), ("short", Z.ZERO_EIO),
    ("hash", Z.ZERO_EINVAL), ("world", Z.ZERO_EINVAL), ("S", Z.ZERO_EINVAL), ("rank", Z.ZERO_EINVAL),
    ("size", Z.ZERO_EIO), ("tracker", Z.ZERO_EIO), ("interval", Z.ZERO_EIO), ("backoff", Z.ZERO_EIO),
    ("scale", Z.ZERO_EIO),
])
def test_checkpoint_load_rejects_foreign_files(case, code, tmp_path):
    """Files that do not belong to this plan and rank are refused from the
    header alone (no file here is a valid shard, so no copy is attempted)."""
    plan = Z.Plan([100], 4)                          # S = 25
    h = Z.zero_plan_hash(plan)
    kw = dict(plan_h=h, world=4, rank=1, S=25)
    body = b"\0" * (3 * 25 * 4)
    if case == "magic":
        kw["magic"] = b"ZEROSHD0"
    elif case == "version":
        kw["version"] = 2
    elif case == "hash":
        kw["plan_h"] = h ^ 1
    elif case == "world":
        kw["world"] = 8
    elif case == "S":
        kw["S"] = 26
    elif case == "rank":
        kw["rank"] = 2
    elif case == "size":
        body = body[:-4]
    elif case == "tracker":
        kw.update(tracker=2000, interval=2000)
    elif case == "interval":
        kw.update(interval=0)
    elif case == "backoff":
        kw.update(backoff=1.5)
    elif case == "scale":
        kw.update(scale=float("nan"))
    path = tmp_path / "shard"
    if case != "missing":
        data = header(**kw) + body
        path.write_bytes(data[:60] if case == "short" else data)
    with pytest.raises(Z.ZeroError) as e:
        _load(plan, str(path))
    assert e.value.code == code, Z.zero_last_error()


def test_checkpoint_load_checks_sums_before_copying(tmp_path):
    """A file with a valid header and size whose data do not match its
    checksums is refused by the read-only pass, before any copy to the device:
    the destination pointers here are never dereferenced (there is no GPU), so
    reaching the copy would fail differently.  The same file with the right
    sums gets past that pass (and only then needs the device)."""
    from ckpt_format import fnv1a
    plan = Z.Plan([100], 4)                          # S = 25
    S = 25
    arrays = [np.arange(S, dtype=np.float32) * (k + 1) for k in range(3)]
    body = b"".join(a.tobytes() for a in arrays)
    sums = [fnv1a(a.tobytes()) for a in arrays]
    path = tmp_path / "shard"
    bad = list(sums)
    bad[1] ^= 1
    path.write_bytes(header(Z.zero_plan_hash(plan), 4, 1, S, sums=tuple(bad)) + body)
    with pytest.raises(Z.ZeroError) as e:
        _load(plan, str(path))
    assert e.value.code == Z.ZERO_EIO
    assert "checksum mismatch (nothing was copied" in Z.zero_last_error()
    path.write_bytes(header(Z.zero_plan_hash(plan), 4, 1, S, sums=tuple(sums)) + body)
    with pytest.raises(Z.ZeroError) as e:
        _load(plan, str(path))
    assert "checksum" not in Z.zero_last_error()
