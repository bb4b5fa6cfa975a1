"""Step control in device memory (zero_step_ctl_t): the step count, the learning
rate and the loss scale live on the device, the library derives each step's
constants there and advances them after the step.

- a sequence of steps with overflows, loss-scale growth and backoff and a
  learning-rate change equals the oracle step by step, bit for bit;
- a captured pair of steps replayed for a whole loop (with an overflow in the
  middle) equals the host-controlled step, bit for bit;
- the constants computed on the device equal the host's float64 formulas
  rounded once to fp32, for many step counts and loss scales."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from gpu_harness import oracle_layout, say, storage
from oracle import casts as OC
from oracle import scaler as ORS
from oracle import step as OS
from zero_sharded_mixed_plan_amd.optim import ZeroAdam

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _opt(w, master, *, device_control, growth_interval, layout=Z.ZERO_STATE_TILED):
    return ZeroAdam(W.numels(w.tensors), w.world, w.rank, lr=w.lr, weight_decay=w.weight_decay,
                    grad_dtype=W.torch_dtype(w.grad_dtype), param_dtype=W.torch_dtype(w.param_dtype),
                    max_norm=w.max_norm, loss_scale=w.loss_scale, dynamic_loss_scale=True,
                    growth_interval=growth_interval, master=master.cuda(), state_layout=layout,
                    device_control=device_control)


def _bits(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint32)


# name -> the multi-workgroup fused path, the one-workgroup path (S <= 8192)
@pytest.mark.parametrize("name", ["llama_7b_n8", "toy_mlp_n4"])
@pytest.mark.parametrize("clip", [False, True])
@pytest.mark.parametrize("layout", [Z.ZERO_STATE_SEPARATE, Z.ZERO_STATE_TILED])
def test_sequence_matches_oracle(name, clip, layout):
    w = W.SMALL[name]
    gd = "f16" if w.grad_dtype != "f32" else "f32"
    w = dataclasses.replace(w, grad_dtype=gd, param_dtype=("f16" if gd == "f16" else "f32"),
                            loss_scale=1024.0, inject_inf_step=3, weight_decay=0.01,
                            max_norm=(1e-3 if clip else 0.0))
    pl, lay = oracle_layout(w)
    S = lay.S
    master, m0, v0 = W.make_state(w, lay, "cpu")
    opt = _opt(w, master, device_control=True, growth_interval=2, layout=layout)
    say(f"device control {name} S={S} clip={clip} layout={layout}")
    p, m, v = master.numpy(), m0.numpy(), v0.numpy()
    t, skipped = 0, 0
    sc = ORS.ScalerState(scale=F32(w.loss_scale), growth_tracker=0, growth_interval=2)
    lr = w.lr
    for step in range(1, 8):
        if step == 5:
            lr = w.lr * 0.5
            opt.lr = lr
        sl = W.make_slices(dataclasses.replace(w, loss_scale=float(sc.scale)), lay, step=step,
                           ld=(S + 63) // 64 * 64)
        assert opt.step(sl.cuda()) is None
        res = OS.shard_step([storage(sl[k, :S]) for k in range(w.world)], w.grad_dtype, w.param_dtype,
                            w.world, p, m, v, lr=lr, weight_decay=w.weight_decay, t=t + 1,
                            inv_scale=float(ORS.inv_scale(sc)), max_norm=w.max_norm,
                            clip_override=(F32(opt.clip.item()) if clip else None))
        assert res.flag == (step == w.inject_inf_step)
        gp, gm, gv = (x.cpu().numpy() for x in opt.state())
        for a, b, what in ((gp, res.master, "master"), (gm, res.m, "m"), (gv, res.v, "v")):
            assert np.array_equal(_bits(a), _bits(b)), f"step {step}: {what}"
        for goff, loff, ln, _v in lay.segments:
            got = storage(opt.gather[goff:goff + ln])
            assert np.array_equal(got, OC.narrow(gp[loff:loff + ln], w.param_dtype)), f"step {step}: slot"
        if res.flag:
            skipped += 1
        else:
            p, m, v, t = res.master, res.m, res.v, t + 1
        sc = ORS.update(sc, res.flag)
        c = opt.ctl.read()
        assert (c.step, c.skipped) == (t, skipped)
        assert (F32(c.scaler.scale), c.scaler.growth_tracker) == (sc.scale, sc.growth_tracker)
    assert float(sc.scale) == 4096.0      # grown three times, backed off once


@pytest.mark.parametrize("clip", [False, True])
def test_graph_replay_of_a_loop(clip):
    """One captured pair of steps, replayed eight times with new gradients
    written into the captured buffer between replays (one replay's gradients
    overflow), equals the host-controlled optimizer stepped eagerly."""
    w = dataclasses.replace(W.SMALL["gpt2_1p5b_n8"], grad_dtype="f16", param_dtype="f16", loss_scale=4096.0,
                            inject_inf_step=None, max_norm=(0.05 if clip else 0.0))
    pl, lay = oracle_layout(w)
    S = lay.S
    ld = (S + 63) // 64 * 64
    master, _m, _v = W.make_state(w, lay, "cpu")
    eager = _opt(w, master, device_control=False, growth_interval=3)
    graphed = _opt(w, master, device_control=True, growth_interval=3)
    warm = _opt(w, master, device_control=True, growth_interval=3)
    say(f"graph loop S={S} clip={clip}")
    buf = torch.zeros((w.world, ld), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # load every kernel once, outside the capture
        warm.step(buf)
        buf[0, 0] = float("inf")
        warm.step(buf)
        buf.zero_()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step(buf)
        graphed.step(buf)
    torch.cuda.synchronize()
    for r in range(8):
        sl = W.make_slices(dataclasses.replace(w, loss_scale=eager.loss_scale), lay, step=r + 1, ld=ld,
                           device="cuda")
        if r == 4:
            sl[3, S // 2] = float("inf")
        buf.copy_(sl)
        g.replay()
        eager.step(sl)
        eager.step(sl)
        torch.cuda.synchronize()
        for a, b in zip(eager.state(), graphed.state()):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"replay {r}: state"
        assert torch.equal(eager.gather.view(torch.int16), graphed.gather.view(torch.int16)), f"replay {r}"
        assert (graphed.t, graphed.skipped, graphed.loss_scale) == (eager.t, eager.skipped, eager.loss_scale)
    assert eager.skipped == 2 and eager.t == 14


def test_device_constants_match_host():
    """bc1, bc2, lr, 1 - lr*wd and 1/scale as the device computes them equal
    float64 formulas rounded once to fp32 (the host's and the oracle's), for
    step counts 1..3000, large powers of two and odd scales."""
    opt = ZeroAdam([64], 1, 0, lr=3e-4, betas=(0.9, 0.999), weight_decay=0.1, grad_dtype=torch.float32,
                   param_dtype=torch.float32, device_control=True)
    grads = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
    ts = list(range(1, 3001)) + [2 ** e for e in range(12, 41)] + [10 ** e + 7 for e in range(4, 12)]
    scales = [65536.0, 1024.0, 3.0, 0.1, 1e-3, 7.0e5]
    say(f"device constants over {len(ts)} step counts")
    bad = []
    for i, t in enumerate(ts):
        c = opt.ctl.read()
        c.step = t - 1
        c.scaler.scale = scales[i % len(scales)]
        c.lr = 3e-4 * (1.0 + (i % 7) / 10.0)
        c.dynamic = 0
        opt.ctl.write(c)
        opt.step(grads)
        k = list(opt.ctl.read().k)[:5]
        want = [F32(1.0 - math.pow(0.9, t)), F32(1.0 - math.pow(0.999, t)), F32(c.lr),
                F32(1.0 - c.lr * 0.1), F32(1.0 / float(F32(c.scaler.scale)))]
        if [F32(x) for x in k] != want:
            bad.append((t, k, want))
    assert not bad, bad[:5]


@pytest.mark.parametrize("table", [False, True])
@pytest.mark.parametrize("clip", [False, True])
def test_sequence_many_pieces_dim0(clip, table):
    """The FSDP2 dim-0 layout of a 20-layer model (more than 192 pieces per rank:
    without the piece table the update runs in several launches and the last
    restore pass advances the step control; with it, in one): five steps with
    an overflow, against the oracle."""
    w = W.Workload(name="dim0_many", tensors=tuple(W.gpt2(n_layer=20, d=64, vocab=503, n_ctx=96)), world=8,
                   rank=5, bucket_cap=0, grad_dtype="f16", param_dtype="f16", lr=1e-3, weight_decay=0.05,
                   loss_scale=512.0, steps=5, seed=17, plan_layout="dim0", inject_inf_step=2,
                   max_norm=(0.02 if clip else 0.0))
    pl, lay = oracle_layout(w)
    S = lay.S
    assert len(lay.segments) > 192
    master, m0, v0 = W.make_state(w, lay, "cpu")
    opt = ZeroAdam([s for _n, s in w.tensors], w.world, w.rank, lr=w.lr, weight_decay=w.weight_decay,
                   grad_dtype=torch.float16, param_dtype=torch.float16, max_norm=w.max_norm,
                   loss_scale=w.loss_scale, dynamic_loss_scale=True, growth_interval=2, master=master.cuda(),
                   layout="dim0", device_control=True, piece_table=table)
    say(f"device control dim0 S={S} pieces={len(lay.segments)} clip={clip} table={table}")
    p, m, v = master.numpy(), m0.numpy(), v0.numpy()
    t = 0
    sc = ORS.ScalerState(scale=F32(w.loss_scale), growth_tracker=0, growth_interval=2)
    for step in range(1, 6):
        sl = W.make_slices(dataclasses.replace(w, loss_scale=float(sc.scale)), lay, step=step,
                           ld=(S + 63) // 64 * 64)
        opt.step(sl.cuda())
        res = OS.shard_step([storage(sl[k, :S]) for k in range(w.world)], "f16", "f16", w.world, p, m, v,
                            lr=w.lr, weight_decay=w.weight_decay, t=t + 1, inv_scale=float(ORS.inv_scale(sc)),
                            max_norm=w.max_norm, clip_override=(F32(opt.clip.item()) if clip else None))
        gp, gm, gv = (x.cpu().numpy() for x in opt.state())
        for a, b, what in ((gp, res.master, "master"), (gm, res.m, "m"), (gv, res.v, "v")):
            assert np.array_equal(_bits(a), _bits(b)), f"step {step}: {what}"
        for goff, loff, ln, _v in lay.segments:
            assert np.array_equal(storage(opt.gather[goff:goff + ln]), OC.narrow(gp[loff:loff + ln], "f16"))
        if not res.flag:
            p, m, v, t = res.master, res.m, res.v, t + 1
        sc = ORS.update(sc, res.flag)
        c = opt.ctl.read()
        assert (c.step, F32(c.scaler.scale), c.scaler.growth_tracker) == (t, sc.scale, sc.growth_tracker)
    assert opt.skipped == 1
