"""The C ABI on the host: the library loads, exports every declared symbol, its
planner matches the oracle planner exactly, and bad arguments are rejected
before anything is enqueued (no GPU is touched here)."""
import ctypes
import os
import re

import pytest

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from oracle import plan as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "zero_shard.h"), encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert len(declared) >= 17
    L = ctypes.CDLL(Z._abi.LIB_PATH)
    missing = [n for n in declared if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(Z.EXPORTS) == declared


CASES = [(W.numels(w.tensors), w.world, w.bucket_cap) for w in W.FULL.values()] + \
        [(W.numels(w.tensors), w.world, w.bucket_cap) for w in W.SMALL.values()] + [
    ([3], 4, 0), ([5, 0, 7], 1, 0), ([8, 8], 4, 0), ([10, 30, 5, 5, 1], 3, 12), ([1] * 50, 7, 6),
    ([0, 5, 0, 0, 4, 0], 2, 3), ([7] * 40, 3, 7), (list(range(1, 300)), 5, 1000),
]


@pytest.mark.parametrize("sizes,world,cap", CASES)
def test_planner_matches_oracle(sizes, world, cap):
    o = OP.make_plan(sizes, world, cap)
    p = Z.Plan(sizes, world, cap)
    assert p.shard_numel == o.shard_numel
    assert p.total_numel == o.psi
    assert p.padded_numel == o.padded_numel
    assert p.num_buckets == len(o.buckets)
    assert p.num_tensors == len(sizes)
    for b, ob in enumerate(o.buckets):
        assert p.bucket(b) == (ob.base, ob.numel, ob.padded, ob.shard, ob.first_tensor, ob.n_tensors)
    for i in range(len(sizes)):
        assert p.tensor(i) == (o.tensor_bucket[i], o.tensor_offset[i])
    ranks = range(world) if world <= 16 else [0, 1, world // 2, world - 1]
    for r in ranks:
        assert p.segments(r) == OP.rank_segments(o, r)
    for stage in range(4):
        f, pb = p.bytes(stage)
        assert pb == OP.padded_model_state_bytes(o, stage)
        exact = OP.model_state_bytes(sum(sizes), world, stage)
        assert abs(f - float(exact)) <= 1e-12 * float(exact)


DIM0_CASES = [
    ([(256, 64), (256,), (10, 256), (10,)], 2),
    ([(256, 64), (256,), (10, 256), (10,)], 3),
    ([(0, 5), (3, 2), (0,), (4,), (), (7, 0), (1, 1, 9)], 4),
    ([(5,)], 8),
    ([(50257, 1600), (1024, 1600), (1600,), (1600, 4800), (4800,)], 8),
    ([tuple(s) for _n, s in W.gpt2(n_layer=2)], 64),
]


@pytest.mark.parametrize("shapes,world", DIM0_CASES)
def test_dim0_planner_matches_oracle(shapes, world):
    o = OP.make_plan_dim0(shapes, world)
    p = Z.Plan.dim0(shapes, world)
    assert (p.shard_numel, p.total_numel, p.padded_numel) == (o.shard_numel, o.psi, o.padded_numel)
    assert p.num_buckets == len(o.buckets) and p.num_tensors == len(shapes)
    for b, ob in enumerate(o.buckets):
        assert p.bucket(b) == (ob.base, ob.numel, ob.padded, ob.shard, ob.first_tensor, ob.n_tensors)
    for i in range(len(shapes)):
        assert p.tensor(i) == (o.tensor_bucket[i], o.tensor_offset[i])
    for r in (range(world) if world <= 8 else [0, 1, world - 1]):
        assert p.segments(r) == OP.rank_segments(o, r)


@pytest.mark.parametrize("bad", [dict(rows=[], rn=[], world=2), dict(rows=[0, 3], rn=[4, 0], world=2),
                                 dict(rows=[4], rn=[1], world=0), dict(rows=[-1], rn=[5], world=2),
                                 dict(rows=[1 << 40], rn=[1 << 20], world=2)])
def test_dim0_plan_rejects(bad):
    import ctypes as C
    n = len(bad["rows"])
    h = C.c_void_p()
    rc = Z.lib().zero_plan_dim0((C.c_int64 * max(n, 1))(*bad["rows"]), (C.c_int64 * max(n, 1))(*bad["rn"]),
                                n, bad["world"], C.byref(h))
    assert rc == Z.ZERO_EINVAL and not h.value
    assert "zero_plan_dim0" in Z.zero_last_error()


@pytest.mark.parametrize("bad", [dict(numels=[], world=2), dict(numels=[0, 0], world=2),
                                 dict(numels=[4], world=0), dict(numels=[-1, 5], world=2)])
def test_plan_rejects(bad):
    with pytest.raises(Z.ZeroError) as e:
        Z.Plan(bad["numels"], bad["world"])
    assert e.value.code == Z.ZERO_EINVAL
    assert "zero_plan" in Z.zero_last_error()


def test_accessors_reject_bad_indices():
    p = Z.Plan([10, 20], 4)
    for call in (lambda: p.bucket(1), lambda: p.tensor(2), lambda: p.rank_segment(4, 0),
                 lambda: p.rank_segment(0, -1), lambda: p.bytes(4)):
        with pytest.raises(Z.ZeroError):
            call()
    L = Z.lib()
    assert L.zero_plan_shard_numel(None) == -1
    assert L.zero_workspace_bytes(None) == 0


# fake, well-aligned device addresses: validation must fail before any use
BASE = 1 << 40


def _good(plan, **over):
    S = plan.shard_numel
    a = dict(rank=3, grad=BASE, grad_ld=S + (-S) % 8, grad_dtype=Z.ZERO_BF16,
             master_in=BASE + (1 << 32), m_in=BASE + (2 << 32), v_in=BASE + (3 << 32),
             master_out=BASE + (4 << 32), m_out=BASE + (5 << 32), v_out=BASE + (6 << 32),
             gather=BASE + (7 << 32), param_dtype=Z.ZERO_BF16, lr=1e-3, beta1=0.9, beta2=0.999,
             eps=1e-8, step=1, overflow_out=BASE + (8 << 32))
    a.update(over)
    return Z.adam_args(**a)


@pytest.mark.parametrize("over,code", [
    (dict(rank=4), Z.ZERO_EINVAL),
    (dict(rank=-1), Z.ZERO_EINVAL),
    (dict(master_in=None), Z.ZERO_EINVAL),
    (dict(gather=None), Z.ZERO_EINVAL),
    (dict(grad=None), Z.ZERO_EINVAL),
    (dict(grad_ld=10), Z.ZERO_EINVAL),
    (dict(grad_dtype=7), Z.ZERO_EINVAL),
    (dict(param_dtype=9), Z.ZERO_EINVAL),
    (dict(master_in=BASE + (1 << 32) + 4), Z.ZERO_EALIGN),
    (dict(grad=BASE + 8), Z.ZERO_EALIGN),
    (dict(grad_ld=4803), Z.ZERO_EALIGN),                 # 4803 bf16 = 9606 B stride
    (dict(gather=BASE + (7 << 32) + 1), Z.ZERO_EALIGN),
    (dict(step=0), Z.ZERO_EINVAL),
    (dict(beta1=1.0), Z.ZERO_EINVAL),
    (dict(lr=float("nan")), Z.ZERO_EINVAL),
    (dict(master_out=BASE + (1 << 32)), Z.ZERO_EINVAL),  # in place with an overflow flag
    (dict(m_out=BASE + (4 << 32)), Z.ZERO_EINVAL),       # two outputs overlap
    (dict(gather=BASE + (4 << 32) + 64), Z.ZERO_EINVAL),  # gather overlaps master_out
    (dict(v_out=BASE + 16), Z.ZERO_EINVAL),              # output overlaps the slices
    (dict(grad_count=-1), Z.ZERO_EINVAL),
    (dict(grad_layout=2), Z.ZERO_EINVAL),                # unknown gradient layout
    (dict(grad_layout=1, grad_count=1, grad=BASE + 1), Z.ZERO_EALIGN),  # element alignment
    (dict(grad_count=2, grad_ld=4803), Z.ZERO_EALIGN),   # stride not a 16-byte multiple
    (dict(grad_layout=1, grad_ld=19_000), Z.ZERO_EINVAL),  # 4 full buffers need ld >= 19,212
    (dict(grad_layout=1, grad_count=1,                   # a full buffer reaching master_out
          grad=BASE + (4 << 32) - 64), Z.ZERO_EINVAL),
    (dict(ctl=BASE + (9 << 32) + 4), Z.ZERO_EALIGN),      # step control must be 8-byte aligned
    (dict(ctl=BASE + (9 << 32), overflow_out=None), Z.ZERO_EINVAL),  # fused with ctl needs the flag
    (dict(ctl=BASE + (6 << 32) + 8), Z.ZERO_EINVAL),      # ctl inside v_out
    (dict(ctl=BASE + (1 << 32) - 40), Z.ZERO_EINVAL),     # ctl reaching into master_in
])
def test_step_validation(over, code):
    plan = Z.Plan(W.numels(W.toy_mlp()), 4)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_adam_step(plan, _good(plan, **over))
    assert e.value.code == code, Z.zero_last_error()


def test_in_place_allowed_without_flag_or_with_stash():
    """Exact in-place state is legal when the skip decision does not need the
    inputs afterwards; partial overlap never is (validated, then rejected only
    for the deliberately broken cases)."""
    plan = Z.Plan(W.numels(W.toy_mlp()), 4)
    part = _good(plan, overflow_out=None, master_out=BASE + (1 << 32) + 16)
    with pytest.raises(Z.ZeroError):
        Z.zero_adam_step(plan, part)


def test_reduce_and_norm_validation():
    plan = Z.Plan([100], 4)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_shard(plan, BASE, 32, Z.ZERO_BF16, 1.0, 0, 0, True)
    assert e.value.code == Z.ZERO_EINVAL          # no workspace
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_shard(plan, BASE + 2, 32, Z.ZERO_BF16, 1.0, 0, BASE, True)
    assert e.value.code == Z.ZERO_EALIGN
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_shard(plan, BASE, 16, Z.ZERO_BF16, 1.0, 0, BASE, True)
    assert e.value.code == Z.ZERO_EINVAL          # ld < S = 25
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_shard(plan, BASE, 32, Z.ZERO_BF16, 1.0, 0, BASE, True, grad_count=-2)
    assert e.value.code == Z.ZERO_EINVAL
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_shard(plan, BASE, 20, Z.ZERO_BF16, 1.0, 0, BASE, True, grad_count=2)
    assert e.value.code == Z.ZERO_EINVAL          # two buffers, ld < S
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_shard(plan, BASE, 32, Z.ZERO_BF16, 1.0, 0, BASE + (1 << 32), True, ctl=BASE + (2 << 32) + 4)
    assert e.value.code == Z.ZERO_EALIGN          # step control misaligned
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_shard(plan, BASE, 32, Z.ZERO_BF16, 1.0, 0, BASE + (1 << 32), True, ctl=BASE + (1 << 32) + 8)
    assert e.value.code == Z.ZERO_EINVAL          # step control inside the workspace
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_shard(plan, BASE, 32, Z.ZERO_BF16, float("inf"), 0, BASE + (1 << 32), True)
    assert e.value.code == Z.ZERO_EINVAL          # inv_scale must be finite without ctl
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_shard_norm(plan, BASE, -1.0, 1.0, 0, 0, 0)
    assert e.value.code == Z.ZERO_EINVAL
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_shard_norm(plan, BASE, 0.0, float("inf"), 0, 0, 0)
    assert e.value.code == Z.ZERO_EINVAL


def test_reduce_refuses_a_tile_with_too_many_pieces():
    """Full-gradient layout, 300 one-element pieces in the first 2048-element
    tile: refused before anything is enqueued."""
    plan = Z.Plan.dim0([(1,)] * 300 + [(5000,)], 2)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_shard(plan, BASE, 0, Z.ZERO_BF16, 1.0, 0, BASE + (1 << 32), True, grad_count=1,
                            grad_layout=Z.ZERO_GRAD_FULL, rank=1)
    assert e.value.code == Z.ZERO_EINVAL and "pieces" in Z.zero_last_error()
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_shard(plan, BASE, 0, Z.ZERO_BF16, 1.0, 0, BASE + (1 << 32), True, grad_count=1,
                            grad_layout=Z.ZERO_GRAD_FULL, rank=2)
    assert e.value.code == Z.ZERO_EINVAL and "rank" in Z.zero_last_error()


def test_state_numel():
    p = Z.Plan([10_000], 4)          # S = 2500 -> 2 tiles of 2048
    assert p.state_numel(Z.ZERO_STATE_SEPARATE) == 2500
    assert p.state_numel(Z.ZERO_STATE_TILED) == 2 * 3 * 2048
    with pytest.raises(Z.ZeroError):
        p.state_numel(7)


@pytest.mark.parametrize("over,code", [
    (dict(state_layout=1), Z.ZERO_EINVAL),                       # tiled takes master only
    (dict(state_layout=1, m_in=None, v_in=None, m_out=None, v_out=None,
          master_out=BASE + (1 << 32) + 4096), Z.ZERO_EINVAL),   # in/out buffers overlap
    (dict(state_layout=3), Z.ZERO_EINVAL),                       # unknown layout
])
def test_tiled_state_validation(over, code):
    plan = Z.Plan(W.numels(W.toy_mlp()), 4)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_adam_step(plan, _good(plan, **over))
    assert e.value.code == code, Z.zero_last_error()


@pytest.mark.parametrize("cname,pytype", [("zero_adam_args_t", Z.zero_adam_args_t),
                                           ("zero_scaler_t", Z.zero_scaler_t),
                                           ("zero_ckpt_meta_t", Z.zero_ckpt_meta_t),
                                           ("zero_step_ctl_t", Z.zero_step_ctl_t)])
def test_args_struct_layout_matches_header(cname, pytype, tmp_path):
    """The ctypes mirrors of the ABI structs have the header's field offsets
    and sizes (compiled with the host C compiler against include/zero_shard.h)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    fields = [f for f, _ in pytype._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "zero_shard.h"', "int main(void) {",
            f'  printf("%zu\\n", sizeof({cname}));']
    prog += [f'  printf("%zu\\n", offsetof({cname}, {f}));' for f in fields]
    prog += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(prog) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(pytype)
    for f, off in zip(fields, out[1:]):
        assert getattr(pytype, f).offset == off, f


@pytest.mark.parametrize("args,code", [((0, BASE, 64), Z.ZERO_EINVAL), ((BASE, BASE + 4096, 24), Z.ZERO_EINVAL),
                                       ((BASE + 8, BASE + 4096, 64), Z.ZERO_EALIGN),
                                       ((BASE, BASE + 32, 64), Z.ZERO_EINVAL),      # overlap
                                       ((BASE, BASE + 4096, -16), Z.ZERO_EINVAL)])
def test_stream_copy_validation(args, code):
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_stream_copy(*args)
    assert e.value.code == code


def test_piece_table_attach_validation():
    """The piece table's size and the attach call's checks (no device memory is
    touched: every case fails before the copy)."""
    plan = Z.Plan.dim0([(256, 64), (256,), (10, 256), (10,)], 2)
    assert plan.piece_table_bytes() == 16 * plan.num_buckets
    for args, code in (((2, BASE, 64), Z.ZERO_EINVAL),       # rank out of range
                       ((-1, BASE, 64), Z.ZERO_EINVAL),
                       ((1, BASE + 8, 64), Z.ZERO_EALIGN),   # 16-byte alignment
                       ((1, BASE, 63), Z.ZERO_EINVAL)):      # too small
        with pytest.raises(Z.ZeroError) as e:
            plan.attach_piece_table(*args)
        assert e.value.code == code, Z.zero_last_error()
    plan.attach_piece_table(0, 0, 0)                          # detaching needs no device
    assert Z.lib().zero_plan_piece_table_bytes(None) == 0


def test_noalloc_limit_is_host_arithmetic():
    """The no-allocation entry point's limit and its refusal need no GPU: the
    largest shard whose workspace fits the 4 MiB array (one float64 partial and
    one overflow word per 2048 elements, plus 3 KiB for the finalize) is
    349,269 tiles; one element more is refused before any HIP call."""
    cap = Z.zero_noalloc_max_shard()
    tiles = (Z.ZERO_NOALLOC_SCRATCH_BYTES - 256 * 8 - 256 * 4) // 12
    assert cap == tiles * 2048 == 715_302_912
    plan = Z.Plan([cap + 1], 1)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_reduce_norm_noalloc(plan, 1 << 40, cap + 1, Z.ZERO_BF16, 1.0, 0, 0.0, 1.0, 0, 0, 0)
    assert e.value.code == Z.ZERO_EINVAL and "fixed array" in Z.zero_last_error()
    assert str(cap) in Z.zero_last_error()
