"""Steps of different plans in flight at once on different streams.

The library keeps no state of its own between launches: flags, workspaces,
stashes and piece tables are the caller's memory, and every launch goes on the
stream it is given.  So three plans stepping concurrently on three streams (a
fused step with ping-pong state, the clipped two-pass step, the 64-slice fp16
step) must give exactly the bits of the same steps run one after another on
one stream.  All streams are created at the default priority."""
import dataclasses

import pytest
import torch

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from gpu_harness import device_plan, oracle_layout, plant_tail, round_up, say, tail_intact
from zero_sharded_mixed_plan_amd.optim import dtype_code, pack_state, state_arg_dict, unpack_state

pytestmark = pytest.mark.gpu
STEPS = 3
NAMES = ["gpt2_1p5b_n8", "llama3_8b_n16_buckets", "flat_7p5b_n64"]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Run:
    """One plan's buffers and its step sequence, launched on a given stream."""

    def __init__(self, name):
        w = dataclasses.replace(W.SMALL[name], inject_inf_step=None)
        _pl, lay = oracle_layout(w)
        self.w, self.plan, S = w, device_plan(w), lay.S
        self.S = S
        self.ld = round_up(S, 64)
        self.slices = [W.make_slices(w, lay, step=s, ld=self.ld, device="cuda") for s in range(1, STEPS + 1)]
        p, m, v = W.make_state(w, lay, "cuda")
        self.init = pack_state(p, m, v, self.plan.state_numel(Z.ZERO_STATE_TILED))
        self.clip = w.max_norm > 0
        self.g = torch.empty(S, dtype=torch.float32, device="cuda")
        self.ws = torch.empty(self.plan.workspace_bytes(), dtype=torch.uint8, device="cuda")
        self.sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
        self.coef = torch.zeros(1, dtype=torch.float32, device="cuda")
        self.flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.gather = torch.zeros(self.plan.padded_numel, dtype=W.torch_dtype(w.param_dtype), device="cuda")

    def reset(self):
        self.state = [self.init.clone(), torch.empty_like(self.init)]
        for b in self.state:   # the positions past S are never written
            plant_tail(b, self.S)
        self.cur = 0
        self.gather.zero_()

    def step(self, s, st):
        w = self.w
        sl = self.slices[s]
        common = dict(rank=w.rank, gather=self.gather.data_ptr(), param_dtype=dtype_code(self.gather.dtype),
                      lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      step=w.t0 + s + 1)
        if self.clip:
            Z.zero_reduce_shard(self.plan, sl.data_ptr(), self.ld, dtype_code(sl.dtype), 1.0 / w.loss_scale,
                                self.g.data_ptr(), self.ws.data_ptr(), True, st)
            Z.zero_shard_norm(self.plan, self.ws.data_ptr(), 0.0, w.max_norm, self.flag.data_ptr(),
                              self.sumsq.data_ptr(), self.coef.data_ptr(), st)
            cur = [self.state[self.cur]]
            a = Z.adam_args(g_stash=self.g.data_ptr(), clip_coef=self.coef.data_ptr(),
                            skip_in=self.flag.data_ptr(), **state_arg_dict(Z.ZERO_STATE_TILED, cur, cur),
                            **common)
        else:   # finite data: every fused step commits, so the state buffers swap
            src, dst = [self.state[self.cur]], [self.state[1 - self.cur]]
            a = Z.adam_args(grad=sl.data_ptr(), grad_ld=self.ld, grad_dtype=dtype_code(sl.dtype),
                            inv_scale=1.0 / w.loss_scale, overflow_out=self.flag.data_ptr(),
                            **state_arg_dict(Z.ZERO_STATE_TILED, src, dst), **common)
            self.cur = 1 - self.cur
        Z.zero_adam_step(self.plan, a, st)

    def result(self):
        return (self.state[self.cur].clone(), self.gather.clone(), self.flag.clone())


def test_concurrent_streams_match_serial():
    runs = [Run(n) for n in NAMES]
    say("streams: " + ", ".join(f"{r.w.name} S={r.S}" for r in runs))
    # serial: every step of every plan on the current stream, one after another
    st0 = torch.cuda.current_stream().cuda_stream
    for r in runs:
        r.reset()
        for s in range(STEPS):
            r.step(s, st0)
    torch.cuda.synchronize()
    serial = [r.result() for r in runs]
    # concurrent: one stream per plan, launches interleaved step by step
    streams = [torch.cuda.Stream() for _ in runs]
    for r in runs:
        r.reset()
    torch.cuda.synchronize()
    for s in range(STEPS):
        for r, x in zip(runs, streams):
            with torch.cuda.stream(x):
                r.step(s, x.cuda_stream)
    torch.cuda.synchronize()
    for r, ref in zip(runs, serial):
        got = r.result()
        assert int(got[2].item()) == 0 and int(ref[2].item()) == 0, r.w.name
        # the S elements of master, m and v; past S the last tile keeps the
        # sentinel planted before the steps, in both buffers
        assert all(tail_intact(b, r.S) for b in r.state), f"{r.w.name}: tiled state written past S"
        for name, a, b in zip(("master", "m", "v"), unpack_state(got[0], r.S), unpack_state(ref[0], r.S)):
            diff = (a.view(torch.int32) != b.view(torch.int32)).nonzero().flatten().cpu()
            assert diff.numel() == 0, (f"{r.w.name} {name}: {diff.numel()} of {r.S} differ, first at "
                                       f"{diff[:8].tolist()}")
        assert torch.equal(got[1].view(torch.int16) if got[1].element_size() == 2 else got[1].view(torch.int32),
                           ref[1].view(torch.int16) if ref[1].element_size() == 2 else ref[1].view(torch.int32)), \
            r.w.name
