"""Sharded checkpoints on the GPU: the file matches the device state element
for element (read back by an independent reader of the documented format),
loads into either state layout, restarts a run bit for bit, and is refused
when corrupt or written for another rank."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from ckpt_format import fnv1a, read
from gpu_harness import oracle_layout, plant_tail, say, tail_intact
from zero_sharded_mixed_plan_amd.optim import ZeroAdam, pack_state, unpack_state

pytestmark = pytest.mark.gpu
SEP, TILED = Z.ZERO_STATE_SEPARATE, Z.ZERO_STATE_TILED


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _state(S, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return [torch.randn(S, generator=g, dtype=torch.float32) for _ in range(3)]


def _device(layout, plan, arrays):
    if layout == TILED:
        return [pack_state(*[a.cuda() for a in arrays], plan.state_numel(TILED))]
    return [a.cuda() for a in arrays]


def _ptrs(layout, bufs):
    return (bufs[0].data_ptr(), 0, 0) if layout == TILED else tuple(b.data_ptr() for b in bufs)


def _host(layout, bufs, S):
    if layout == TILED:
        return [x.cpu().numpy() for x in unpack_state(bufs[0], S)]
    return [b.cpu().numpy() for b in bufs]


@pytest.mark.parametrize("src_layout,dst_layout", [(SEP, SEP), (SEP, TILED), (TILED, SEP), (TILED, TILED)])
@pytest.mark.parametrize("numels,world,rank", [([19_210], 4, 3), ([4_194_304 * 3 + 9_000], 3, 1),
                                               ([(1 << 22) * 2], 2, 1), ([((1 << 21) + 1) * 3], 3, 2)])
def test_save_read_load(src_layout, dst_layout, numels, world, rank, tmp_path):
    """A shard of a few thousand elements; one of about 4.2M (three 2M-element
    staging chunks that alternate between the two staging sets, a ragged last
    chunk and tile); exactly two full chunks; two chunks of which the last holds
    one element."""
    plan = Z.Plan(numels, world)
    S = plan.shard_numel
    say(f"checkpoint S={S} {src_layout}->{dst_layout}")
    arrays = _state(S, 5)
    src = _device(src_layout, plan, arrays)
    scaler = Z.Scaler(1024.0, 2.0, 0.5, 7)
    scaler.update(False)
    path = str(tmp_path / f"rank{rank}.zshd")
    Z.zero_checkpoint_save(plan, rank, path, src_layout, *_ptrs(src_layout, src), 42, scaler.s,
                           torch.cuda.current_stream().cuda_stream)
    assert not os.path.exists(path + ".tmp")
    f = read(path)
    assert (f["version"], f["header"], f["world"], f["rank"], f["S"], f["step"]) == (1, 128, world, rank, S, 42)
    assert f["plan_hash"] == Z.zero_plan_hash(plan)
    assert (f["scale"], f["growth_tracker"], f["growth_factor"], f["backoff_factor"], f["growth_interval"]) == \
        (1024.0, 1, 2.0, 0.5, 7)
    assert f["reserved"] == 0 and f["tail"] == b"\0" * 32 and f["size"] == 128 + 12 * S
    for k, name in enumerate(("master", "m", "v")):
        assert np.array_equal(f[name].view(np.uint32), arrays[k].numpy().view(np.uint32)), name
        if S < 100_000:
            assert f["sums"][k] == fnv1a(f[name].tobytes())
    dst = _device(dst_layout, plan, [torch.full((S,), 7.0) for _ in range(3)])
    if dst_layout == TILED:
        plant_tail(dst[0], S)
    meta = Z.zero_checkpoint_load(plan, rank, path, dst_layout, *_ptrs(dst_layout, dst),
                                  torch.cuda.current_stream().cuda_stream)
    assert meta.step == 42 and meta.scaler.scale == 1024.0 and meta.scaler.growth_tracker == 1
    for k, a in enumerate(_host(dst_layout, dst, S)):
        assert np.array_equal(a.view(np.uint32), arrays[k].numpy().view(np.uint32))
    if dst_layout == TILED:   # the last tile's positions past S are not written
        assert tail_intact(dst[0], S)


def test_corrupt_and_foreign_files(tmp_path):
    plan = Z.Plan([50_000], 4)
    S = plan.shard_numel
    bufs = _device(SEP, plan, _state(S, 1))
    st = torch.cuda.current_stream().cuda_stream
    path = str(tmp_path / "r2")
    Z.zero_checkpoint_save(plan, 2, path, SEP, *_ptrs(SEP, bufs), 3, Z.Scaler().s, st)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_checkpoint_load(plan, 1, path, SEP, *_ptrs(SEP, bufs), st)
    assert e.value.code == Z.ZERO_EINVAL                     # rank 2's shard
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_checkpoint_load(Z.Plan([50_000], 8), 2, path, SEP, *_ptrs(SEP, bufs), st)
    assert e.value.code == Z.ZERO_EINVAL                     # another plan
    raw = bytearray(open(path, "rb").read())
    raw[128 + 4 * S + 17] ^= 0x40                            # one bit of m
    open(path, "wb").write(bytes(raw))
    for b in bufs:            # the live state a failed load must leave alone
        b.fill_(7.0)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_checkpoint_load(plan, 2, path, SEP, *_ptrs(SEP, bufs), st)
    assert e.value.code == Z.ZERO_EIO and "checksum" in Z.zero_last_error()
    torch.cuda.synchronize()
    assert all(bool(torch.all(b == 7.0)) for b in bufs), "a corrupt file was copied into the state"


@pytest.mark.parametrize("layout", [SEP, TILED])
@pytest.mark.parametrize("clip", [False, True])
def test_restart_is_bit_exact(layout, clip, tmp_path):
    """Run 5 steps (one skipped on an overflow); separately run 3, save, load
    into a fresh optimizer and run the last 2: state, gather slots, t and the
    loss scale agree bit for bit."""
    w = dataclasses.replace(W.SMALL["llama_7b_n8"], grad_dtype="f16", param_dtype="f16",
                            loss_scale=1024.0, inject_inf_step=4, max_norm=(1e-3 if clip else 0.0))
    pl, lay = oracle_layout(w)
    S = lay.S
    master, _m, _v = W.make_state(w, lay, "cpu")

    def make():
        return ZeroAdam(W.numels(w.tensors), w.world, w.rank, lr=w.lr, weight_decay=w.weight_decay,
                        grad_dtype=torch.float16, param_dtype=torch.float16, max_norm=w.max_norm,
                        loss_scale=w.loss_scale, dynamic_loss_scale=True, growth_interval=2,
                        master=master.cuda(), state_layout=layout)

    def grads(opt, step):
        return W.make_slices(dataclasses.replace(w, loss_scale=opt.loss_scale), lay, step=step,
                             ld=(S + 63) // 64 * 64, device="cuda")

    a = make()
    for step in range(1, 6):
        a.step(grads(a, step))
    b = make()
    for step in range(1, 4):
        b.step(grads(b, step))
    path = str(tmp_path / "shard")
    b.save(path)
    c = make()
    c.load(path)
    assert (c.t, c.loss_scale, c.scaler.growth_tracker) == (b.t, b.loss_scale, b.scaler.growth_tracker)
    c.gather.copy_(b.gather)
    for step in range(4, 6):
        c.step(grads(c, step))
    assert a.skipped == 1 and c.skipped == 1
    assert (c.t, c.loss_scale) == (a.t, a.loss_scale)
    for x, y in zip(a.state(), c.state()):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(a.gather.view(torch.int16), c.gather.view(torch.int16))
