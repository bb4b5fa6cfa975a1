"""The ZeroAdam object (loss scaling, skip bookkeeping, both state layouts, both
step paths) against the oracle over several steps."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from gpu_harness import oracle_layout, say, storage
from oracle import casts as OC
from oracle import step as OS
from zero_sharded_mixed_plan_amd.optim import ZeroAdam

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("layout", [Z.ZERO_STATE_SEPARATE, Z.ZERO_STATE_TILED])
@pytest.mark.parametrize("clip", [False, True])
def test_zero_adam_object(layout, clip):
    w = dataclasses.replace(W.SMALL["llama_7b_n8"], grad_dtype="f16", param_dtype="f16",
                            loss_scale=1024.0, steps=4, inject_inf_step=2,
                            max_norm=(1e-3 if clip else 0.0))
    pl, lay = oracle_layout(w)
    S = lay.S
    master, m0, v0 = W.make_state(w, lay, "cpu")
    opt = ZeroAdam(W.numels(w.tensors), w.world, w.rank, lr=w.lr, weight_decay=w.weight_decay,
                   grad_dtype=torch.float16, param_dtype=torch.float16, max_norm=w.max_norm,
                   loss_scale=w.loss_scale, dynamic_loss_scale=True, master=master.cuda(),
                   state_layout=layout)
    say(f"ZeroAdam S={S} layout={layout} clip={clip}")
    assert opt.state_bytes() == 12 * S
    p, m, v = master.numpy(), m0.numpy(), v0.numpy()
    t = 0
    scale = w.loss_scale
    for step in range(1, w.steps + 1):
        sl = W.make_slices(dataclasses.replace(w, loss_scale=scale), lay, step=step,
                           ld=(S + 63) // 64 * 64)
        ok = opt.step(sl.cuda())
        res = OS.shard_step([storage(sl[k, :S]) for k in range(w.world)], "f16", "f16", w.world,
                            p, m, v, lr=w.lr, weight_decay=w.weight_decay, t=t + 1,
                            inv_scale=1.0 / scale, max_norm=w.max_norm,
                            clip_override=(np.float32(opt.clip.item()) if clip else None))
        assert ok == (not res.flag) == (step != w.inject_inf_step)
        gp, gm, gv = (x.cpu().numpy() for x in opt.state())
        for a, b in ((gp, res.master), (gm, res.m), (gv, res.v)):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        goff = lay.segments[0][0]
        got = storage(opt.gather[goff:goff + S])
        assert np.array_equal(got, OC.narrow(gp, "f16"))
        if ok:
            p, m, v, t = res.master, res.m, res.v, t + 1
        else:
            scale *= 0.5
        assert opt.t == t and opt.loss_scale == scale
    assert opt.skipped == 1
