"""ZeroAdam: one rank's sharded mixed-precision AdamW over torch device tensors.

The object mirrors the surface of the handbook's ZeroAdam ("ZeRO 与 FSDP：
切分优化器状态、梯度与参数", section "从零实现 ZeRO 的 Adam": constructor with
lr, betas, eps; step(); state_bytes()) for one rank on one GPU, with the mixed
precision parts of "PaddlePaddle ZeRO优化…" (section "混合精度才是最佳拍档":
scale, unscale, skip on overflow, update the scale).  torch supplies device
memory and the stream; every step of the computation runs in libzero_shard.so.

The reduce-scatter's input arrives as `slices`, an [N, ld] device tensor whose row
k holds rank k's gradient of this rank's shard (in a multi-GPU job these rows
are what the reduce-scatter would sum).  The new parameters land in this rank's
slots of `gather`, the all-gather buffer.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _abi

_CODES = {torch.float32: _abi.ZERO_F32, torch.bfloat16: _abi.ZERO_BF16, torch.float16: _abi.ZERO_F16}


def dtype_code(dt: torch.dtype) -> int:
    try:
        return _CODES[dt]
    except KeyError:
        raise TypeError(f"unsupported dtype {dt}") from None


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def pack_state(master: torch.Tensor, m: torch.Tensor, v: torch.Tensor, numel: int) -> torch.Tensor:
    """Three [S] fp32 arrays -> one tiled state buffer of `numel` elements
    (tiles of ZERO_STATE_TILE master, then m, then v; the last tile zero-padded)."""
    T = _abi.ZERO_STATE_TILE
    nt = numel // (3 * T)
    S = master.numel()
    buf = torch.zeros(numel, dtype=torch.float32, device=master.device)
    view = buf.view(nt, 3, T)
    pad = torch.zeros(nt * T, dtype=torch.float32, device=master.device)
    for i, x in enumerate((master, m, v)):
        pad[:S].copy_(x)
        view[:, i, :].copy_(pad.view(nt, T))
    return buf


def unpack_state(buf: torch.Tensor, S: int):
    """Tiled state buffer -> (master, m, v) as [S] copies."""
    T = _abi.ZERO_STATE_TILE
    view = buf.view(-1, 3, T)
    return tuple(view[:, i, :].reshape(-1)[:S].clone() for i in range(3))


def state_arg_dict(layout: int, src, dst) -> dict:
    """zero_adam_args_t state fields for lists of buffers (3 arrays, or 1 tiled buffer)."""
    if layout == _abi.ZERO_STATE_TILED:
        return dict(state_layout=layout, master_in=src[0].data_ptr(), master_out=dst[0].data_ptr())
    return dict(state_layout=layout, master_in=src[0].data_ptr(), m_in=src[1].data_ptr(),
                v_in=src[2].data_ptr(), master_out=dst[0].data_ptr(), m_out=dst[1].data_ptr(),
                v_out=dst[2].data_ptr())


class StepCtl:
    """A zero_step_ctl_t in device memory: step count, skip count, learning
    rate and loss scale that the step reads and advances on the device."""

    _LR = _abi.zero_step_ctl_t.lr.offset

    def __init__(self, step: int, lr: float, scaler: "_abi.zero_scaler_t", dynamic: bool, device):
        self.buf = torch.zeros(ctypes.sizeof(_abi.zero_step_ctl_t), dtype=torch.uint8, device=device)
        self.write(_abi.zero_step_ctl_t(step=int(step), skipped=0, lr=float(lr), scaler=scaler,
                                        dynamic=1 if dynamic else 0))

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()

    def read(self) -> "_abi.zero_step_ctl_t":
        """Host image, after the work queued on the current stream."""
        return _abi.zero_step_ctl_t.from_buffer_copy(self.buf.cpu().numpy().tobytes())

    def write(self, c: "_abi.zero_step_ctl_t") -> None:
        """Replace every field, in stream order."""
        self.buf.copy_(torch.frombuffer(bytearray(bytes(c)), dtype=torch.uint8))

    def set_lr(self, lr: float) -> None:
        """Rewrite the learning rate only, in stream order (no wait)."""
        v = torch.tensor([float(lr)], dtype=torch.float64).view(torch.uint8)
        self.buf[self._LR:self._LR + 8].copy_(v)


class ZeroAdam:
    """Sharded AdamW state and step of rank `rank` out of `world`.

    Without clipping the step is one fused pass over the gradient buffers and
    writes the new state into the second of two state buffers, which become
    current only if no gradient overflowed.  With max_norm > 0 the step is two
    passes: the reduced gradient and the norm partials first, then the update
    in place.  With dynamic_loss_scale the loss scale follows zero_scaler_t
    (backoff on an overflow, growth after `growth_interval` clean steps).

    layout "flat": `numels` are tensor sizes packed into flat buckets of
    `bucket_cap`; layout "dim0": `numels` are parameter shapes, each split on
    its first dimension (FSDP2 fully_shard).

    device_control=True keeps the step count, the learning rate and the loss
    scale in device memory (StepCtl): step() then never waits for the device
    (it returns None), a skipped step leaves the output state current, and the
    step can be captured in a HIP graph and replayed for every step.  t,
    skipped and loss_scale read the device copy (a wait).

    piece_table: attach the rank's piece table in device memory (default: when
    the layout has more than 192 pieces, the most one launch addresses from its
    kernel arguments).
    """

    def __init__(self, numels: Sequence, world: int, rank: int, *, lr: float,
                 betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.0,
                 bucket_cap: int = 0, grad_dtype=torch.bfloat16, param_dtype=torch.bfloat16,
                 max_norm: float = 0.0, loss_scale: float = 1.0, dynamic_loss_scale: bool = False,
                 growth_interval: int = 2000, master: Optional[torch.Tensor] = None,
                 gather: Optional[torch.Tensor] = None, device="cuda",
                 state_layout: int = _abi.ZERO_STATE_TILED, layout: str = "flat",
                 device_control: bool = False, piece_table: Optional[bool] = None):
        if layout == "dim0":
            self.plan = _abi.Plan.dim0(numels, world)
        elif layout == "flat":
            self.plan = _abi.Plan(numels, world, bucket_cap)
        else:
            raise ValueError("layout must be 'flat' or 'dim0'")
        self.world, self.rank = int(world), int(rank)
        self._lr, self.betas, self.eps, self.weight_decay = lr, tuple(betas), eps, weight_decay
        self.grad_dtype, self.param_dtype = grad_dtype, param_dtype
        self.max_norm = float(max_norm)
        self.dynamic = dynamic_loss_scale
        # a fixed scale is a scaler that is never updated
        self.scaler = _abi.Scaler(float(loss_scale), 2.0, 0.5, growth_interval)
        self._t = 0
        self._skipped = 0
        S = self.plan.shard_numel
        self.S = S
        dev = torch.device(device)
        f32 = dict(dtype=torch.float32, device=dev)
        n_sets = 1 if self.max_norm > 0 else 2
        self.layout = state_layout
        if state_layout == _abi.ZERO_STATE_TILED:
            n = self.plan.state_numel(state_layout)
            self._state = [[torch.zeros(n, **f32)] for _ in range(n_sets)]
        else:
            self._state = [[torch.zeros(S, **f32) for _ in range(3)] for _ in range(n_sets)]
        self._cur = 0
        if master is not None:
            if state_layout == _abi.ZERO_STATE_TILED:
                z = torch.zeros(S, **f32)
                self._state[0][0].copy_(pack_state(master.to(**f32), z, z, self._state[0][0].numel()))
            else:
                self._state[0][0].copy_(master)
        # many pieces (a dim-0 layout of a large model): the piece table in device
        # memory, so each step is one launch rather than one per 192 pieces
        self._table = None
        if piece_table or (piece_table is None and self.plan.num_buckets > 192):
            self._table = torch.empty(self.plan.piece_table_bytes(), dtype=torch.uint8, device=dev)
            self.plan.attach_piece_table(self.rank, self._table.data_ptr(), self._table.numel())
        self.gather = gather if gather is not None else torch.zeros(
            self.plan.padded_numel, dtype=param_dtype, device=dev)
        if self.gather.numel() != self.plan.padded_numel or self.gather.dtype != param_dtype:
            raise ValueError("gather buffer has the wrong size or dtype")
        self.flag = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ctl = StepCtl(0, lr, self.scaler.s, self.dynamic, dev) if device_control else None
        if self.max_norm > 0:
            self.g = torch.empty(S, **f32)
            self.ws = torch.empty(self.plan.workspace_bytes(), dtype=torch.uint8, device=dev)
            self.sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
            self.clip = torch.ones(1, **f32)

    @property
    def loss_scale(self) -> float:
        return self.ctl.read().scaler.scale if self.ctl else self.scaler.scale

    @property
    def t(self) -> int:
        """Steps applied."""
        return int(self.ctl.read().step) if self.ctl else self._t

    @property
    def skipped(self) -> int:
        """Steps not applied (overflow)."""
        return int(self.ctl.read().skipped) if self.ctl else self._skipped

    @property
    def lr(self) -> float:
        return self._lr

    @lr.setter
    def lr(self, value: float) -> None:
        """A new learning rate from the next step on (with device control, a
        write of the device copy in stream order)."""
        self._lr = float(value)
        if self.ctl:
            self.ctl.set_lr(self._lr)

    # -- state ---------------------------------------------------------------
    def state(self):
        """(master, m, v) of this rank as [S] tensors (copies for the tiled layout)."""
        cur = self._state[self._cur]
        if self.layout == _abi.ZERO_STATE_TILED:
            return unpack_state(cur[0], self.S)
        return tuple(cur)

    @property
    def master(self) -> torch.Tensor:
        return self.state()[0]

    @property
    def m(self) -> torch.Tensor:
        return self.state()[1]

    @property
    def v(self) -> torch.Tensor:
        return self.state()[2]

    def state_bytes(self) -> int:
        """fp32 master + m + v of this rank (the handbook's state_bytes())."""
        return 3 * 4 * self.S

    def segments(self):
        return self.plan.segments(self.rank)

    # -- sharded checkpoint ----------------------------------------------------
    def _ptrs(self):
        cur = self._state[self._cur]
        if self.layout == _abi.ZERO_STATE_TILED:
            return cur[0].data_ptr(), 0, 0
        return tuple(x.data_ptr() for x in cur)

    def save(self, path: str) -> None:
        """Write this rank's shard (master, m, v, t, loss-scale state) to `path`."""
        if self.ctl:
            c = self.ctl.read()
            t, sc = int(c.step), c.scaler
        else:
            t, sc = self._t, self.scaler.s
        _abi.zero_checkpoint_save(self.plan, self.rank, path, self.layout, *self._ptrs(), t, sc, _stream())

    def load(self, path: str) -> None:
        """Restore what save() wrote (same plan and rank; any state layout)."""
        meta = _abi.zero_checkpoint_load(self.plan, self.rank, path, self.layout, *self._ptrs(), _stream())
        self._t = int(meta.step)
        self.scaler.s = meta.scaler
        if self.ctl:
            c = self.ctl.read()
            c.step, c.scaler = meta.step, meta.scaler
            self.ctl.write(c)

    # -- step ----------------------------------------------------------------
    def step(self, grads: torch.Tensor, other_ranks_sumsq: float = 0.0, *, full: bool = False) -> Optional[bool]:
        """One step; returns False if it was skipped (None with device control,
        which does not wait for the device).

        grads: [C, ld] device tensor of C gradient buffers summed in the step and
        divided by N -- the N ranks' slices of this shard (C = N), or one stored
        reduce-scatter output (C = 1); with full=True, whole flat gradients in
        the gather layout (ld >= padded numel; C = 1 is ZeRO-1's all-reduced
        gradient).
        """
        need = self.plan.padded_numel if full else self.S
        if grads.dim() != 2 or grads.shape[0] < 1 or grads.shape[1] < need:
            raise ValueError(f"grads must be [C, ld >= {need}]")
        if grads.dtype != self.grad_dtype or grads.stride(1) != 1:
            raise ValueError("grads have the wrong dtype or layout")
        st = _stream()
        gcode = dtype_code(grads.dtype)
        count = int(grads.shape[0])
        ctl = self.ctl.ptr if self.ctl else 0
        inv = 1.0 if ctl else self.scaler.inv_scale
        b1, b2 = self.betas
        common = dict(rank=self.rank, gather=self.gather.data_ptr(),
                      param_dtype=dtype_code(self.param_dtype), lr=self._lr, beta1=b1, beta2=b2,
                      eps=self.eps, weight_decay=self.weight_decay, step=self._t + 1, ctl=ctl or None)
        if self.max_norm > 0:
            _abi.zero_reduce_shard(self.plan, grads.data_ptr(), grads.stride(0), gcode, inv,
                                   self.g.data_ptr(), self.ws.data_ptr(), True, st, grad_count=count,
                                   grad_layout=_abi.ZERO_GRAD_FULL if full else _abi.ZERO_GRAD_SHARD,
                                   rank=self.rank, ctl=ctl)
            _abi.zero_shard_norm(self.plan, self.ws.data_ptr(), other_ranks_sumsq, self.max_norm,
                                 self.flag.data_ptr(), self.sumsq.data_ptr(), self.clip.data_ptr(), st)
            cur = self._state[0]
            args = _abi.adam_args(g_stash=self.g.data_ptr(), clip_coef=self.clip.data_ptr(),
                                  skip_in=self.flag.data_ptr(),
                                  **state_arg_dict(self.layout, cur, cur), **common)
            _abi.zero_adam_step(self.plan, args, st)
            if ctl:
                return None
            ok = int(self.flag.item()) == 0
        else:
            src, dst = self._state[self._cur], self._state[1 - self._cur]
            args = _abi.adam_args(grad=grads.data_ptr(), grad_ld=grads.stride(0), grad_dtype=gcode,
                                  grad_count=count,
                                  grad_layout=_abi.ZERO_GRAD_FULL if full else _abi.ZERO_GRAD_SHARD,
                                  inv_scale=inv, overflow_out=self.flag.data_ptr(),
                                  **state_arg_dict(self.layout, src, dst), **common)
            _abi.zero_adam_step(self.plan, args, st)
            if ctl:                       # the output state is current either way
                self._cur = 1 - self._cur
                return None
            ok = int(self.flag.item()) == 0
            if ok:
                self._cur = 1 - self._cur
        if ok:
            self._t += 1
        else:
            self._skipped += 1
        if self.dynamic:
            self.scaler.update(not ok)
        return ok
