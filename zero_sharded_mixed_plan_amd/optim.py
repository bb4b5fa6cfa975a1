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
    """

    def __init__(self, numels: Sequence, world: int, rank: int, *, lr: float,
                 betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.0,
                 bucket_cap: int = 0, grad_dtype=torch.bfloat16, param_dtype=torch.bfloat16,
                 max_norm: float = 0.0, loss_scale: float = 1.0, dynamic_loss_scale: bool = False,
                 growth_interval: int = 2000, master: Optional[torch.Tensor] = None,
                 gather: Optional[torch.Tensor] = None, device="cuda",
                 state_layout: int = _abi.ZERO_STATE_TILED, layout: str = "flat"):
        if layout == "dim0":
            self.plan = _abi.Plan.dim0(numels, world)
        elif layout == "flat":
            self.plan = _abi.Plan(numels, world, bucket_cap)
        else:
            raise ValueError("layout must be 'flat' or 'dim0'")
        self.world, self.rank = int(world), int(rank)
        self.lr, self.betas, self.eps, self.weight_decay = lr, tuple(betas), eps, weight_decay
        self.grad_dtype, self.param_dtype = grad_dtype, param_dtype
        self.max_norm = float(max_norm)
        self.dynamic = dynamic_loss_scale
        # a fixed scale is a scaler that is never updated
        self.scaler = _abi.Scaler(float(loss_scale), 2.0, 0.5, growth_interval)
        self.t = 0
        self.skipped = 0
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
        self.gather = gather if gather is not None else torch.zeros(
            self.plan.padded_numel, dtype=param_dtype, device=dev)
        if self.gather.numel() != self.plan.padded_numel or self.gather.dtype != param_dtype:
            raise ValueError("gather buffer has the wrong size or dtype")
        self.flag = torch.zeros(1, dtype=torch.int32, device=dev)
        if self.max_norm > 0:
            self.g = torch.empty(S, **f32)
            self.ws = torch.empty(self.plan.workspace_bytes(), dtype=torch.uint8, device=dev)
            self.sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
            self.clip = torch.ones(1, **f32)

    @property
    def loss_scale(self) -> float:
        return self.scaler.scale

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
        _abi.zero_checkpoint_save(self.plan, self.rank, path, self.layout, *self._ptrs(), self.t,
                                  self.scaler.s, _stream())

    def load(self, path: str) -> None:
        """Restore what save() wrote (same plan and rank; any state layout)."""
        meta = _abi.zero_checkpoint_load(self.plan, self.rank, path, self.layout, *self._ptrs(), _stream())
        self.t = int(meta.step)
        self.scaler.s = meta.scaler

    # -- step ----------------------------------------------------------------
    def step(self, grads: torch.Tensor, other_ranks_sumsq: float = 0.0, *, full: bool = False) -> bool:
        """One step; returns False if it was skipped.

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
        inv = self.scaler.inv_scale
        b1, b2 = self.betas
        common = dict(rank=self.rank, gather=self.gather.data_ptr(),
                      param_dtype=dtype_code(self.param_dtype), lr=self.lr, beta1=b1, beta2=b2,
                      eps=self.eps, weight_decay=self.weight_decay, step=self.t + 1)
        if self.max_norm > 0:
            _abi.zero_reduce_shard(self.plan, grads.data_ptr(), grads.stride(0), gcode, inv,
                                   self.g.data_ptr(), self.ws.data_ptr(), True, st, grad_count=count,
                                   grad_layout=_abi.ZERO_GRAD_FULL if full else _abi.ZERO_GRAD_SHARD,
                                   rank=self.rank)
            _abi.zero_shard_norm(self.plan, self.ws.data_ptr(), other_ranks_sumsq, self.max_norm,
                                 self.flag.data_ptr(), self.sumsq.data_ptr(), self.clip.data_ptr(), st)
            cur = self._state[0]
            args = _abi.adam_args(g_stash=self.g.data_ptr(), clip_coef=self.clip.data_ptr(),
                                  skip_in=self.flag.data_ptr(),
                                  **state_arg_dict(self.layout, cur, cur), **common)
            _abi.zero_adam_step(self.plan, args, st)
            ok = int(self.flag.item()) == 0
        else:
            src, dst = self._state[self._cur], self._state[1 - self._cur]
            args = _abi.adam_args(grad=grads.data_ptr(), grad_ld=grads.stride(0), grad_dtype=gcode,
                                  grad_count=count,
                                  grad_layout=_abi.ZERO_GRAD_FULL if full else _abi.ZERO_GRAD_SHARD,
                                  inv_scale=inv, overflow_out=self.flag.data_ptr(),
                                  **state_arg_dict(self.layout, src, dst), **common)
            _abi.zero_adam_step(self.plan, args, st)
            ok = int(self.flag.item()) == 0
            if ok:
                self._cur = 1 - self._cur
        if ok:
            self.t += 1
        else:
            self.skipped += 1
        if self.dynamic:
            self.scaler.update(not ok)
        return ok
