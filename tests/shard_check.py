"""Whole-shard comparison of one GPU step with the oracle, chunk by chunk.

Every element of the rank's shard is checked: the GPU's master, m and v (tiled
state layout) and the rank's gather slots against the oracle stepping the same
inputs, copied to the host a chunk at a time and stepped on a pool of host
threads (the step is elementwise, so the oracle's result for a chunk is its
result for those elements of the shard).  The overflow decision is the one
place where elements meet: the GPU's flag is taken as the whole shard's, each
chunk is checked against it, and the oracle's own flag (the OR over chunks) must
equal it.  The clipped path's stash is compared too, and the oracle's sum of
squares over the shard is returned for the norm check."""
from __future__ import annotations

import concurrent.futures as cf
import math
import os

import numpy as np
import torch

import zero_sharded_mixed_plan_amd as Z
from gpu_harness import check_params, compare_step, storage
from oracle import casts as OC
from oracle import step as OS

F = np.float32
T = Z.ZERO_STATE_TILE


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def state_chunk(buf: torch.Tensor, a: int, b: int):
    """(master, m, v) of local elements [a, b) of a tiled state buffer (a % T == 0)."""
    t0, t1 = a // T, -(-b // T)
    x = storage(buf[t0 * 3 * T:t1 * 3 * T]).reshape(-1, 3, T)
    return tuple(np.ascontiguousarray(x[:, i, :].reshape(-1)[:b - a]) for i in range(3))


def pieces_chunk(flat: torch.Tensor, segments, a: int, b: int) -> np.ndarray:
    """Elements of local [a, b) read from a buffer in the gather layout (the
    rank's slots, or a full flat gradient at the rank's pieces)."""
    parts = []
    for goff, lo, ln, _v in segments:
        x0, x1 = max(a, lo), min(b, lo + ln)
        if x0 < x1:
            parts.append(storage(flat[goff + x0 - lo:goff + x1 - lo]))
    return np.concatenate(parts)


def check_whole_shard(*, S, w, t, grads_of, state_in, state_out, gather, segments, flag,
                      c32=None, g_gpu=None, chunk=1 << 22, what=""):
    """Compare every element of one step with the oracle.

    grads_of(a, b): the oracle's gradient buffers for local [a, b) (host arrays).
    state_in: a tiled buffer holding the step's input state (taken before the
    step); state_out: the tiled buffer the step's result is in (for a skipped
    fused step, the input buffer).  flag: the GPU's overflow decision.  c32:
    the GPU's clip coefficient (clipped path), g_gpu: its fp32 stash.
    Returns (elements checked, oracle flag, oracle sum of squares or None)."""
    assert chunk % T == 0
    kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, t=t,
              inv_scale=1.0 / w.loss_scale)
    if c32 is not None:
        kw.update(max_norm=w.max_norm, clip_override=c32)
    consts = OS.adam_consts(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t)

    def work(a):
        b = min(S, a + chunk)
        sl = grads_of(a, b)
        p, m, v = state_chunk(state_in, a, b)
        res = OS.shard_step(sl, w.grad_dtype, w.param_dtype, w.world, p, m, v, **kw)
        gp, gm, gv = state_chunk(state_out, a, b)
        where = f"{what} [{a}, {b})"
        if g_gpu is not None:
            assert np.array_equal(storage(g_gpu[a:b]).view(np.uint32), res.g.view(np.uint32)), \
                f"{where}: stash g differs"
        if flag:
            # not applied: the state is the input bit for bit and the slots hold
            # the rounded input master
            for x, y, n in ((gp, p, "master"), (gm, m, "m"), (gv, v, "v")):
                assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), f"{where}: {n} changed on skip"
            want = OC.narrow(p, w.param_dtype)
        else:
            assert not res.flag, f"{where}: the oracle sees a non-finite g, the GPU did not"
            g_used = res.g if c32 is None else np.multiply(res.g, res.clip, dtype=F)
            n, tot = compare_step(gp, gm, gv, res, p, m, v, g_used, consts, where)
            assert n == tot, f"{where}: {tot - n} state elements differ in the last bit"
            want = res.params
        got = pieces_chunk(gather, segments, a, b)
        same = check_params(got, want, w.param_dtype, where + " params")
        assert same == b - a, f"{where}: {b - a - same} parameters differ in the last bit"
        q = OS.sumsq(res.g) if c32 is not None else None
        return b - a, res.flag, q

    with cf.ThreadPoolExecutor(workers()) as ex:
        out = list(ex.map(work, range(0, S, chunk)))
    n = sum(o[0] for o in out)
    assert n == S
    oracle_flag = any(o[1] for o in out)
    q = math.fsum(o[2] for o in out) if c32 is not None else None
    return n, oracle_flag, q


def shard_grads(slices: torch.Tensor, count: int):
    """grads_of for [count, ld] shard-layout buffers."""
    return lambda a, b: [storage(slices[k, a:b]) for k in range(count)]


def full_grads(full: torch.Tensor, count: int, segments):
    """grads_of for [count, ld] full flat gradients read at the rank's pieces."""
    return lambda a, b: [pieces_chunk(full[k], segments, a, b) for k in range(count)]


def outside_slots_untouched(gather: torch.Tensor, segments, sentinel) -> bool:
    """Every element of the gather buffer outside the rank's pieces still holds
    the sentinel it was filled with."""
    sent = torch.tensor(sentinel, dtype=gather.dtype, device=gather.device)
    prev = 0
    for goff, _lo, ln, _v in sorted(segments):
        if goff > prev and not bool(torch.all(gather[prev:goff] == sent)):
            return False
        prev = goff + ln
    return prev >= gather.numel() or bool(torch.all(gather[prev:] == sent))


def check_reduction(*, S, w, grads_of, g_gpu, chunk=1 << 22, what=""):
    """The reduction pass alone: every element of the GPU's fp32 g (sum over
    the buffers, / N, unscaled) against the oracle, bit for bit.  Returns the
    oracle's float64 sum of squares over the shard."""
    def work(a):
        b = min(S, a + chunk)
        g = OS.unscale(OS.average(OS.reduce_slices(grads_of(a, b), w.grad_dtype), w.world),
                       1.0 / w.loss_scale)
        assert np.array_equal(storage(g_gpu[a:b]).view(np.uint32), g.view(np.uint32)), \
            f"{what} [{a}, {b}): g differs"
        return OS.sumsq(g)

    with cf.ThreadPoolExecutor(workers()) as ex:
        return math.fsum(ex.map(work, range(0, S, chunk)))
