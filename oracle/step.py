"""Oracle for one rank's step: reduce N gradient slices, average, unscale, check,
optionally clip, AdamW on the fp32 shard, round and write the gather slot.

The order of the operations and their notation follow zero_adam.py in the
handbook chapter "ZeRO 与 FSDP：切分优化器状态、梯度与参数" (section
"从零实现 ZeRO 的 Adam"):

  g = reduce_scatter(SUM of the ranks' gradients); g /= world; t += 1
  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g g
  m_hat = m / (1 - b1^t);  v_hat = v / (1 - b2^t)
  master -= lr * m_hat / (sqrt(v_hat) + eps)
  all_gather(master) -> full parameters

Mixed precision adds the loss-scale unscale and the overflow skip of
GradScaler ("PaddlePaddle ZeRO优化…", section "混合精度才是最佳拍档") and the
fp16/bf16 parameter copy written into the gather buffer ("论文专题讲解：ZeRO…",
section "显存账"; the parameter all-gather of "ZeRO-DP 三阶段").

Every array operation is one numpy float32 ufunc (one IEEE rounding, no fused
multiply-add).  Readings the pages leave open (each one a convention of this
oracle; "parity unpinned" where no pin can decide it):
  * summation order: slices are added in ascending rank order into an fp32
    accumulator that starts from slice 0 (parity unpinned);
  * unscale multiplies by fp32(1 / loss_scale) after the average;
  * the overflow flag is raised by any non-finite reduced gradient of the
    shard, padding included; a flagged step leaves master, m, v untouched and
    does not advance t;
  * weight decay is decoupled, p <- (1 - lr wd) p - u, applied to every element
    (the pages only name AdamW);
  * the global-norm clip (pages silent) scales g by min(1, max_norm / ||g||),
    with ||g|| accumulated in float64 over the unclipped, unscaled gradient and
    the coefficient rounded once to fp32 (parity unpinned);
  * host constants are computed in float64 and rounded once to fp32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np

from . import casts

F32 = np.float32


# ---------------------------------------------------------------------------
# gradient preparation
# ---------------------------------------------------------------------------

def reduce_slices(slices: Sequence[np.ndarray], kind: str) -> np.ndarray:
    """acc = widen(slice_0); acc = acc + widen(slice_k) for k = 1 .. N-1 (fp32).

    Stands in for the SUM of the reduce-scatter (zero_adam.py step()).
    """
    acc = casts.widen(slices[0], kind).astype(np.float32, copy=True)
    with np.errstate(over="ignore", invalid="ignore"):   # inf / NaN are data here
        for k in range(1, len(slices)):
            acc = np.add(acc, casts.widen(slices[k], kind), dtype=np.float32)
    return acc


def average(acc: np.ndarray, world: int) -> np.ndarray:
    """g = acc / N  (zero_adam.py: g /= self.world)."""
    return np.divide(acc, F32(world), dtype=np.float32)


def unscale(g: np.ndarray, inv_scale: float) -> np.ndarray:
    """g = g * fp32(1 / loss_scale)  (GradScaler's unscale before the step)."""
    return np.multiply(g, F32(inv_scale), dtype=np.float32)


def overflow(g: np.ndarray) -> bool:
    """True if any element of the shard's reduced gradient is inf or NaN."""
    return bool(np.any(~np.isfinite(g)))


def sumsq(g: np.ndarray) -> float:
    """q = sum_j float64(g_j)^2 over the shard (float64 accumulation)."""
    g64 = np.asarray(g, dtype=np.float32).astype(np.float64)
    return float(np.sum(g64 * g64))


def clip_coefficient(total_sumsq: float, max_norm: float) -> np.float32:
    """c = max_norm / ||g|| if ||g|| > max_norm else 1, ||g|| = sqrt(total) in
    float64; rounded once to fp32.  max_norm <= 0 disables clipping (c = 1)."""
    if max_norm <= 0:
        return F32(1.0)
    norm = math.sqrt(total_sumsq)
    c = max_norm / norm if norm > max_norm else 1.0
    return F32(c)


# ---------------------------------------------------------------------------
# AdamW
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class AdamConsts:
    lr: np.float32
    b1: np.float32
    b2: np.float32
    omb1: np.float32    # 1 - beta1
    omb2: np.float32    # 1 - beta2
    bc1: np.float32     # 1 - beta1^t
    bc2: np.float32     # 1 - beta2^t
    eps: np.float32
    dec: np.float32     # 1 - lr * weight_decay


def adam_consts(lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                t: int) -> AdamConsts:
    """Per-step scalars, computed in float64 and rounded once to fp32.  t is the
    1-based index of the step being taken (t += 1 before the update)."""
    if t < 1:
        raise ValueError("t counts from 1")
    return AdamConsts(lr=F32(lr), b1=F32(beta1), b2=F32(beta2), omb1=F32(1.0 - beta1),
                      omb2=F32(1.0 - beta2), bc1=F32(1.0 - beta1 ** t),
                      bc2=F32(1.0 - beta2 ** t), eps=F32(eps),
                      dec=F32(1.0 - lr * weight_decay))


def adamw(p: np.ndarray, m: np.ndarray, v: np.ndarray, g: np.ndarray,
          c: AdamConsts) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One AdamW update of fp32 arrays; returns (p', m', v')."""
    f = np.float32
    m2 = np.add(np.multiply(c.b1, m, dtype=f), np.multiply(c.omb1, g, dtype=f), dtype=f)
    v2 = np.add(np.multiply(c.b2, v, dtype=f),
                np.multiply(c.omb2, np.multiply(g, g, dtype=f), dtype=f), dtype=f)
    m_hat = np.divide(m2, c.bc1, dtype=f)
    v_hat = np.divide(v2, c.bc2, dtype=f)
    den = np.add(np.sqrt(v_hat, dtype=f), c.eps, dtype=f)
    u = np.divide(np.multiply(c.lr, m_hat, dtype=f), den, dtype=f)
    p2 = np.subtract(np.multiply(c.dec, p, dtype=f), u, dtype=f)
    return p2, m2, v2


# ---------------------------------------------------------------------------
# the whole shard step
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class StepResult:
    master: np.ndarray
    m: np.ndarray
    v: np.ndarray
    params: np.ndarray          # the rank's new low-precision parameters, [S]
    flag: bool                  # overflow: step skipped
    g: np.ndarray               # reduced, averaged, unscaled gradient (before clipping)
    sumsq: Optional[float]      # q of this shard (only when clipping)
    clip: np.float32            # coefficient applied (1 when not clipping)


def shard_step(slices: Sequence[np.ndarray], grad_kind: str, param_kind: str, world: int,
               master: np.ndarray, m: np.ndarray, v: np.ndarray, *, lr: float,
               beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
               weight_decay: float = 0.0, t: int, inv_scale: float = 1.0,
               max_norm: float = 0.0, other_sumsq: float = 0.0,
               clip_override: Optional[np.float32] = None) -> StepResult:
    """One rank's step over its local shard.

    slices: N arrays [S] (float32 for 'f32', uint16 bit patterns for 'bf16'/'f16').
    t: 1-based index of this step.  With max_norm > 0 the global norm combines
    this shard's q with other_sumsq (the other ranks' share); clip_override, when
    given, replaces the coefficient computed here (used to decouple element
    parity from a last-bit difference in a norm computed elsewhere).
    """
    g = unscale(average(reduce_slices(slices, grad_kind), world), inv_scale)
    flag = overflow(g)
    q = None
    c32 = F32(1.0)
    g_used = g
    if max_norm > 0:
        q = sumsq(g)
        c32 = clip_coefficient(q + other_sumsq, max_norm) if clip_override is None \
            else F32(clip_override)
        with np.errstate(invalid="ignore", over="ignore"):   # inf * 0 when the norm is inf
            g_used = np.multiply(g, c32, dtype=np.float32)
    if flag:
        return StepResult(master.copy(), m.copy(), v.copy(), casts.narrow(master, param_kind),
                          True, g, q, c32)
    c = adam_consts(lr, beta1, beta2, eps, weight_decay, t)
    p2, m2, v2 = adamw(master, m, v, g_used, c)
    return StepResult(p2, m2, v2, casts.narrow(p2, param_kind), False, g, q, c32)


def write_gather(gather: np.ndarray, segments, params: np.ndarray) -> None:
    """Copy the rank's [S] parameters into its pieces of the gather buffer.

    segments: (gather_off, local_off, seg_len, valid) per bucket; every element
    of a piece is written, padding included.
    """
    for goff, loff, seg_len, _valid in segments:
        gather[goff:goff + seg_len] = params[loff:loff + seg_len]


def read_pieces(full: np.ndarray, segments) -> np.ndarray:
    """The rank's [S] local gradient read out of a full flat gradient (ZeRO-1:
    gradients all-reduced in full, each rank updating only the range it owns;
    handbook chapter, section "三个级别"; "PaddlePaddle ZeRO优化…", section
    "第一层：只分片优化器状态（ZeRO-1）").  The rank's pieces sit where its
    parameter slots sit in the gather buffer, so this is write_gather read
    backwards.  segments: (gather_off, local_off, seg_len, valid) per bucket.
    """
    S = sum(seg_len for _g, _l, seg_len, _v in segments)
    out = np.empty(S, dtype=full.dtype)
    for goff, loff, seg_len, _valid in segments:
        out[loff:loff + seg_len] = full[goff:goff + seg_len]
    return out
