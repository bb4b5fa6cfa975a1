"""Shared helpers of the GPU parity tests: device buffers for one workload, the
HIP step through the C ABI, and comparisons with the oracle (tolerances of the
step's contract: fp32 state within 1e-6 relative to the largest term of the
operation that produced it, 16-bit parameters within 1 ulp, flags and layout
exact; the kernels are built to be bit-exact and the tests also count that)."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from zero_sharded_mixed_plan_amd.optim import pack_state, state_arg_dict, unpack_state
from oracle import casts as OC
from oracle import plan as OP
from oracle import step as OS

F = np.float32
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
CODE = {"f32": Z.ZERO_F32, "bf16": Z.ZERO_BF16, "f16": Z.ZERO_F16}


def say(*a):
    print("[gpu]", *a, flush=True)


def storage(t: torch.Tensor) -> np.ndarray:
    """Tensor -> numpy storage (float32, or uint16 bits for 16-bit types)."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_storage(a: np.ndarray, kind: str) -> torch.Tensor:
    if kind == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=F))
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(TORCH[kind])


def oracle_layout(w: W.Workload):
    if w.plan_layout == "dim0":
        pl = OP.make_plan_dim0([s for _n, s in w.tensors], w.world)
    else:
        pl = OP.make_plan(W.numels(w.tensors), w.world, w.bucket_cap)
    segs = OP.rank_segments(pl, w.rank)
    return pl, W.Layout(S=pl.shard_numel, segments=segs, tensor_flat_off=list(pl.tensor_offset))


def device_plan(w: W.Workload) -> Z.Plan:
    if w.plan_layout == "dim0":
        return Z.Plan.dim0([s for _n, s in w.tensors], w.world)
    return Z.Plan(W.numels(w.tensors), w.world, w.bucket_cap)


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


# ---------------------------------------------------------------------------
# comparisons
# ---------------------------------------------------------------------------

def _ordered16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _ordered32(x: np.ndarray) -> np.ndarray:
    b = x.view(np.uint32).astype(np.int64)
    return np.where(b & 0x80000000, -(b & 0x7FFFFFFF), b)


def check_params(gpu: np.ndarray, ref: np.ndarray, kind: str, what: str) -> int:
    """<= 1 ulp; returns the number of bit-identical elements."""
    if kind == "f32":
        d = np.abs(_ordered32(gpu.astype(F)) - _ordered32(ref.astype(F)))
    else:
        d = np.abs(_ordered16(gpu) - _ordered16(ref))
    bad = np.flatnonzero(d > 1)
    assert bad.size == 0, f"{what}: {bad.size} params differ by >1 ulp, first at {bad[:5]}"
    return int(np.sum(d == 0))


def check_state(gpu: np.ndarray, ref: np.ndarray, guard: np.ndarray, what: str) -> int:
    """|gpu - ref| <= 1e-6 * max(|ref|, guard); returns the bit-identical count."""
    g = gpu.astype(np.float64)
    r = ref.astype(np.float64)
    tol = 1e-6 * np.maximum(np.abs(r), guard.astype(np.float64))
    same_nan = np.isnan(g) & np.isnan(r)
    bad = np.flatnonzero(~same_nan & ~(np.abs(g - r) <= tol))
    assert bad.size == 0, (f"{what}: {bad.size} elements out of tolerance; first {bad[:5]}, "
                           f"gpu {gpu[bad[:3]]}, oracle {ref[bad[:3]]}")
    return int(np.sum(gpu.view(np.uint32) == ref.view(np.uint32)))


def guards(p, m, v, g, c: OS.AdamConsts):
    """Magnitude of the largest term of each output's last operation."""
    f = np.float32
    m2 = np.maximum(np.abs(c.b1 * m), np.abs(c.omb1 * g)).astype(f)
    v2 = np.maximum(np.abs(c.b2 * v), np.abs(c.omb2 * (g * g))).astype(f)
    pn, mn, vn = OS.adamw(p, m, v, g, c)
    u = np.abs(c.dec * p - pn)
    p2 = np.maximum(np.abs(c.dec * p), u).astype(f)
    return p2, m2, v2


def compare_step(gpu_p, gpu_m, gpu_v, res: OS.StepResult, p_in, m_in, v_in, g_used, consts, what):
    """Compare one step's state; returns (bitwise-equal count, total)."""
    if res.flag:
        for a, b, n in ((gpu_p, p_in, "master"), (gpu_m, m_in, "m"), (gpu_v, v_in, "v")):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{what}: {n} changed on skip"
        return gpu_p.size * 3, gpu_p.size * 3
    gp, gm, gv = guards(p_in, m_in, v_in, g_used, consts)
    n = check_state(gpu_p, res.master, gp, what + " master")
    n += check_state(gpu_m, res.m, gm, what + " m")
    n += check_state(gpu_v, res.v, gv, what + " v")
    return n, gpu_p.size * 3


# ---------------------------------------------------------------------------
# the tiled state's last tile past S
# ---------------------------------------------------------------------------

# Tiled state buffers hold ceil(S / 2048) whole tiles; the positions past S in
# the last tile's master, m and v belong to no element, and no kernel may read
# them into an element or write them.  Tests plant this value there and check
# that it is still there after every kind of step.
TAIL_SENTINEL = -31.5


def plant_tail(buf: torch.Tensor, S: int) -> None:
    """Write TAIL_SENTINEL to a tiled state buffer's positions past S."""
    T = Z.ZERO_STATE_TILE
    if S % T:
        buf.view(-1, 3, T)[-1, :, S % T:] = TAIL_SENTINEL


def tail_intact(buf: torch.Tensor, S: int) -> bool:
    """True if every position past S of a tiled buffer still holds the sentinel."""
    T = Z.ZERO_STATE_TILE
    if S % T == 0:
        return True
    return bool(torch.all(buf.view(-1, 3, T)[-1, :, S % T:] == TAIL_SENTINEL).item())


# ---------------------------------------------------------------------------
# one workload on the device
# ---------------------------------------------------------------------------

# every Rig made by the running test (the parity tests check their tiled
# buffers' tails after each test)
RIGS: list = []

class Rig:
    """Device buffers of one rank for workload w (inputs drawn on the CPU)."""

    def __init__(self, w: W.Workload, ld_align: int = 64, device="cuda", rank=None,
                 layout: int = Z.ZERO_STATE_SEPARATE, table: bool = False):
        if rank is not None:
            import dataclasses
            w = dataclasses.replace(w, rank=rank)
        self.w = w
        self.pl, self.lay = oracle_layout(w)
        self.S = self.lay.S
        self.plan = device_plan(w)
        self.table = None
        if table:   # the pieces from a device table: one launch for any number of pieces
            self.table = torch.empty(self.plan.piece_table_bytes(), dtype=torch.uint8, device=device)
            self.plan.attach_piece_table(w.rank, self.table.data_ptr(), self.table.numel())
        self.ld = round_up(self.S, ld_align)
        dev = torch.device(device)
        self.dev = dev
        master, m, v = W.make_state(w, self.lay, "cpu")
        self.p0, self.m0, self.v0 = master.numpy().copy(), m.numpy().copy(), v.numpy().copy()
        self.layout = layout
        if layout == Z.ZERO_STATE_TILED:
            n = self.plan.state_numel(layout)
            self.A = [pack_state(master.to(dev), m.to(dev), v.to(dev), n)]
            self.B = [torch.zeros(n, dtype=torch.float32, device=dev)]
            plant_tail(self.A[0], self.S)
            plant_tail(self.B[0], self.S)
        else:
            self.A = [x.to(dev) for x in (master, m, v)]
            self.B = [torch.zeros(self.S, dtype=torch.float32, device=dev) for _ in range(3)]
        RIGS.append(self)
        # gather buffer: a random bit pattern everywhere (to catch stray writes),
        # the rank's pieces hold the rounded initial master
        rng = np.random.default_rng(w.seed + 1)
        NS = self.pl.padded_numel
        if w.param_dtype == "f32":
            g = rng.normal(0, 1, NS).astype(F)
        else:
            g = rng.integers(0, 0x7C00, NS, dtype=np.uint16)
        OS.write_gather(g, self.lay.segments, OC.narrow(self.p0, w.param_dtype))
        self.gather0 = g.copy()
        self.gather = from_storage(g, w.param_dtype).to(dev)
        self.flag = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ws = torch.empty(self.plan.workspace_bytes(), dtype=torch.uint8, device=dev)
        self.g = torch.empty(self.S, dtype=torch.float32, device=dev)
        self.sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        self.clip = torch.zeros(1, dtype=torch.float32, device=dev)

    def slices(self, step: int):
        s = W.make_slices(self.w, self.lay, step=step, ld=self.ld, device="cpu")
        return s, s.to(self.dev)

    def common(self, t):
        w = self.w
        return dict(rank=w.rank, gather=self.gather.data_ptr(), param_dtype=CODE[w.param_dtype],
                    lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                    weight_decay=w.weight_decay, step=t)

    def state_args(self, src, dst):
        return state_arg_dict(self.layout, src, dst)

    def unpack(self, bufs):
        """(master, m, v) of a state buffer list as numpy [S] arrays."""
        if self.layout == Z.ZERO_STATE_TILED:
            return tuple(x.cpu().numpy() for x in unpack_state(bufs[0], self.S))
        return tuple(x.cpu().numpy() for x in bufs)

    def fused(self, sl_dev, src, dst, t, overflow=True, skip=None, count=0, layout=Z.ZERO_GRAD_SHARD,
              ld=None):
        """The fused step on gradient buffers sl_dev (rows at stride ld, default
        the rig's slice stride): count buffers (0 = N) in the given layout."""
        a = Z.adam_args(grad=sl_dev.data_ptr(), grad_ld=self.ld if ld is None else ld,
                        grad_dtype=CODE[self.w.grad_dtype], grad_count=count, grad_layout=layout,
                        inv_scale=1.0 / self.w.loss_scale,
                        overflow_out=self.flag.data_ptr() if overflow else None,
                        skip_in=skip, **self.state_args(src, dst), **self.common(t))
        Z.zero_adam_step(self.plan, a, torch.cuda.current_stream().cuda_stream)

    def reduce_norm(self, sl_dev, other=0.0, max_norm=None, count=0, layout=Z.ZERO_GRAD_SHARD, ld=None):
        st = torch.cuda.current_stream().cuda_stream
        Z.zero_reduce_shard(self.plan, sl_dev.data_ptr(), self.ld if ld is None else ld,
                            CODE[self.w.grad_dtype], 1.0 / self.w.loss_scale, self.g.data_ptr(),
                            self.ws.data_ptr(), True, st, grad_count=count, grad_layout=layout,
                            rank=self.w.rank)
        Z.zero_shard_norm(self.plan, self.ws.data_ptr(), other,
                          self.w.max_norm if max_norm is None else max_norm, self.flag.data_ptr(),
                          self.sumsq.data_ptr(), self.clip.data_ptr(), st)

    def stash_step(self, state, t, skip=True):
        a = Z.adam_args(g_stash=self.g.data_ptr(), clip_coef=self.clip.data_ptr(),
                        skip_in=self.flag.data_ptr() if skip is True else skip,
                        **self.state_args(state, state), **self.common(t))
        Z.zero_adam_step(self.plan, a, torch.cuda.current_stream().cuda_stream)

    def tails_intact(self) -> bool:
        """Tiled layout: both state buffers still hold the sentinel past S."""
        if self.layout != Z.ZERO_STATE_TILED:
            return True
        return tail_intact(self.A[0], self.S) and tail_intact(self.B[0], self.S)

    def gather_np(self):
        return storage(self.gather)

    def slot_mask(self):
        m = np.zeros(self.pl.padded_numel, bool)
        for goff, _lo, ln, _v in self.lay.segments:
            m[goff:goff + ln] = True
        return m
