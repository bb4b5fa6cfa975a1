"""An independent reader and writer of the shard checkpoint format, written
from its description in include/zero_shard.h (128-byte little-endian header,
then master, m and v as fp32 in local order), and the 64-bit FNV-1a hash."""
import struct

import numpy as np

HEADER = 128
FNV_OFFSET = 1469598103934665603
FNV_PRIME = 1099511628211
MASK = (1 << 64) - 1


def fnv1a(data: bytes, h: int = FNV_OFFSET) -> int:
    """64-bit FNV-1a (plain loop: for inputs of up to a few MB)."""
    for b in data:
        h = ((h ^ b) * FNV_PRIME) & MASK
    return h


def plan_hash(world, numels, buckets):
    """buckets: (numel, shard, n_tensors) per bucket."""
    def i64(x):
        return struct.pack("<q", x)
    data = i64(world) + i64(len(numels)) + b"".join(i64(n) for n in numels) + i64(len(buckets))
    data += b"".join(i64(n) + i64(s) + i64(c) for n, s, c in buckets)
    return fnv1a(data)


def read(path):
    raw = open(path, "rb").read()
    h = raw[:HEADER]
    assert h[:8] == b"ZEROSHD1"
    version, hdr = struct.unpack_from("<II", h, 8)
    plan_h, world, rank, S, step = struct.unpack_from("<QiiqQ", h, 16)
    scale, tracker, growth, backoff, interval, zero = struct.unpack_from("<fiffiI", h, 48)
    sums = struct.unpack_from("<QQQ", h, 72)
    arrays = [np.frombuffer(raw, dtype="<f4", count=S, offset=HEADER + 4 * S * k) for k in range(3)]
    return dict(version=version, header=hdr, plan_hash=plan_h, world=world, rank=rank, S=S, step=step,
                scale=scale, growth_tracker=tracker, growth_factor=growth, backoff_factor=backoff,
                growth_interval=interval, reserved=zero, sums=sums, master=arrays[0], m=arrays[1],
                v=arrays[2], tail=h[96:], size=len(raw))


def header(plan_h, world, rank, S, step=0, scale=1.0, tracker=0, growth=2.0, backoff=0.5, interval=2000,
           sums=(0, 0, 0), magic=b"ZEROSHD1", version=1):
    h = bytearray(HEADER)
    h[:8] = magic
    struct.pack_into("<II", h, 8, version, HEADER)
    struct.pack_into("<QiiqQ", h, 16, plan_h, world, rank, S, step)
    struct.pack_into("<fiffiI", h, 48, scale, tracker, growth, backoff, interval, 0)
    struct.pack_into("<QQQ", h, 72, *sums)
    return bytes(h)
