"""Oracle planner: tensor list -> padded flat buckets -> one rank's shard segments.

Layout (handbook chapter "ZeRO 与 FSDP", section "从零实现 ZeRO 的 Adam",
zero_adam.py): all parameters are flattened in list order into one vector,
zero-padded at the end to a multiple of the world size N, and split into N equal
contiguous pieces; the piece length is ceil(numel / N) and rank r owns the piece
starting at r * piece.

Buckets (parity unpinned — the pages only say that real ZeRO-2 reduce-scatters
gradients bucket by bucket during backward, same section, and that fused
temporary buffers should have a constant size, "ZeRO-R", C_B): with a positive
cap, tensors are packed greedily in list order into buckets; a bucket that
already holds elements is closed when adding the next tensor would take it past
the cap, so a tensor larger than the cap sits alone and no bucket is empty
(zero-size tensors join the open bucket).  Each bucket is then laid out exactly
like the single flat vector above.  A cap <= 0 gives one bucket, i.e. the plain flat vector.

Byte accounting (section "三个级别" of the same chapter; "ZeRO-DP 三阶段" of the
paper deep-dive): per-device model state for mixed-precision Adam with K = 12 is
16 Psi (plain data parallel), 4 Psi + 12 Psi / N (stage 1, optimizer states
sharded), 2 Psi + 14 Psi / N (stage 2, + gradients), 16 Psi / N (stage 3, +
parameters).
"""
from __future__ import annotations

import dataclasses
from fractions import Fraction
from typing import List, Sequence, Tuple


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclasses.dataclass(frozen=True)
class Bucket:
    first_tensor: int
    n_tensors: int
    numel: int      # B_b: elements of the tensors in this bucket
    shard: int      # S_b = ceil(B_b / N)
    padded: int     # P_b = N * S_b
    base: int       # offset of the bucket in the flat (gather) buffer


@dataclasses.dataclass(frozen=True)
class Plan:
    world: int
    numels: Tuple[int, ...]
    buckets: Tuple[Bucket, ...]
    tensor_bucket: Tuple[int, ...]
    tensor_offset: Tuple[int, ...]   # flat offset of each tensor in the gather buffer

    @property
    def psi(self) -> int:
        return sum(self.numels)

    @property
    def shard_numel(self) -> int:
        """S: length of every rank's local arrays (sum of the bucket shards)."""
        return sum(b.shard for b in self.buckets)

    @property
    def padded_numel(self) -> int:
        """Length of the full gather buffer (sum of the padded bucket lengths)."""
        return sum(b.padded for b in self.buckets)


def make_plan(numels: Sequence[int], world: int, bucket_cap: int = 0) -> Plan:
    numels = tuple(int(n) for n in numels)
    if world < 1:
        raise ValueError("world size must be >= 1")
    if len(numels) == 0 or any(n < 0 for n in numels) or sum(numels) == 0:
        raise ValueError("need at least one element")
    groups: List[List[int]] = []
    cur: List[int] = []
    cur_size = 0
    for i, n in enumerate(numels):
        if bucket_cap > 0 and n > 0 and cur_size > 0 and cur_size + n > bucket_cap:
            groups.append(cur)
            cur, cur_size = [], 0
        cur.append(i)
        cur_size += n
    groups.append(cur)

    buckets: List[Bucket] = []
    tensor_bucket = [0] * len(numels)
    tensor_offset = [0] * len(numels)
    base = 0
    for b, idx in enumerate(groups):
        size = sum(numels[i] for i in idx)
        shard = ceil_div(size, world)
        off = base
        for i in idx:
            tensor_bucket[i] = b
            tensor_offset[i] = off
            off += numels[i]
        buckets.append(Bucket(first_tensor=idx[0], n_tensors=len(idx), numel=size, shard=shard,
                              padded=world * shard, base=base))
        base += world * shard
    return Plan(world=world, numels=numels, buckets=tuple(buckets),
                tensor_bucket=tuple(tensor_bucket), tensor_offset=tuple(tensor_offset))


def make_plan_dim0(shapes: Sequence[Sequence[int]], world: int) -> Plan:
    """Per-parameter dim-0 layout (FSDP2 fully_shard: every parameter a tensor
    split on its first dimension; handbook chapter, section "ZeRO-3 与 FSDP").

    Each parameter of shape (rows, *rest) is its own bucket.  Its rows are padded
    to N * c with c = ceil(rows / N), rank r holding rows [r*c, (r+1)*c): S_b =
    c * prod(rest), P_b = N * S_b, and the bucket in the gather buffer is the
    padded parameter in row-major order.  A 0-d parameter counts as one row of
    one element.  A parameter with no elements adds no bucket: it sits, empty, at
    the end of the previous parameter's bucket (or the start of the next one).
    The generic rank_segments then gives each rank one piece per parameter.
    """
    if world < 1:
        raise ValueError("world size must be >= 1")
    rows, row_numel = [], []
    for sh in shapes:
        sh = tuple(int(x) for x in sh)
        if any(x < 0 for x in sh):
            raise ValueError("negative dimension")
        r = sh[0] if sh else 1
        k = 1
        for x in sh[1:]:
            k *= x
        rows.append(r)
        row_numel.append(k)
    numels = tuple(r * k for r, k in zip(rows, row_numel))
    if len(numels) == 0 or sum(numels) == 0:
        raise ValueError("need at least one element")
    # groups: each non-empty parameter opens one; empty ones join the open group
    groups: List[List[int]] = []
    for i, n in enumerate(numels):
        if n > 0 or not groups:
            groups.append([i])
        else:
            groups[-1].append(i)
    if numels[groups[0][0]] == 0:          # leading empties: merge into the first real group
        lead = groups.pop(0)
        groups[0] = lead + groups[0]
    buckets: List[Bucket] = []
    tensor_bucket = [0] * len(numels)
    tensor_offset = [0] * len(numels)
    base = 0
    for b, idx in enumerate(groups):
        main = [i for i in idx if numels[i] > 0][0]
        shard = ceil_div(rows[main], world) * row_numel[main]
        for i in idx:
            tensor_bucket[i] = b
            tensor_offset[i] = base + (numels[main] if i > main else 0)
        buckets.append(Bucket(first_tensor=idx[0], n_tensors=len(idx), numel=numels[main],
                              shard=shard, padded=world * shard, base=base))
        base += world * shard
    return Plan(world=world, numels=numels, buckets=tuple(buckets),
                tensor_bucket=tuple(tensor_bucket), tensor_offset=tuple(tensor_offset))


def dim0_local_shape(shape: Sequence[int], world: int, rank: int) -> Tuple[int, ...]:
    """Shape of rank r's local shard of a dim-0 sharded parameter: rows
    clamp(rows - r*c, 0, c) of c = ceil(rows / N), the rest unchanged (what
    fully_shard's to_local() returns; the padding rows are not part of it)."""
    shape = tuple(int(x) for x in shape)
    rows = shape[0] if shape else 1
    c = ceil_div(rows, world)
    mine = min(max(rows - rank * c, 0), c)
    return (mine,) + shape[1:] if shape else ((1,) if mine else (0,))


def rank_segments(plan: Plan, rank: int) -> List[Tuple[int, int, int, int]]:
    """Rank r's pieces, one per bucket: (gather_off, local_off, seg_len, valid).

    gather_off = base_b + r * S_b is where the piece sits in the gather buffer;
    local_off is where it sits in the rank's local arrays (pieces are
    concatenated in bucket order); valid = clamp(B_b - r * S_b, 0, S_b) counts the
    non-padding elements, which come first.
    """
    if not 0 <= rank < plan.world:
        raise ValueError("rank out of range")
    segs = []
    local = 0
    for b in plan.buckets:
        valid = min(max(b.numel - rank * b.shard, 0), b.shard)
        segs.append((b.base + rank * b.shard, local, b.shard, valid))
        local += b.shard
    return segs


def state_bytes(plan: Plan) -> int:
    """Bytes of one rank's fp32 master, m and v (zero_adam.py state_bytes)."""
    return 3 * 4 * plan.shard_numel


def model_state_bytes(psi: int, world: int, stage: int) -> Fraction:
    """Per-device model-state bytes, mixed-precision Adam (K = 12), exact.

    stage 0: plain data parallel, 16 Psi; 1: 4 Psi + 12 Psi/N; 2: 2 Psi + 14 Psi/N;
    3: 16 Psi / N.
    """
    psi_f, n = Fraction(psi), Fraction(world)
    if stage == 0:
        return 16 * psi_f
    if stage == 1:
        return 4 * psi_f + 12 * psi_f / n
    if stage == 2:
        return 2 * psi_f + 14 * psi_f / n
    if stage == 3:
        return 16 * psi_f / n
    raise ValueError("stage must be 0, 1, 2 or 3")


def padded_model_state_bytes(plan: Plan, stage: int) -> int:
    """The same accounting on the padded layout: N*S in place of Psi, S in place of Psi/N."""
    S = plan.shard_numel
    NS = plan.padded_numel
    if stage == 0:
        return 16 * NS
    if stage == 1:
        return 4 * NS + 12 * S
    if stage == 2:
        return 2 * NS + 14 * S
    if stage == 3:
        return 16 * S
    raise ValueError("stage must be 0, 1, 2 or 3")
