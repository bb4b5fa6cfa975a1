"""The layout the planner produces is the one the collectives around the step
expect: N CPU processes over gloo reduce-scatter their full flat gradients
bucket by bucket (SUM), step their shards with the oracle, and all-gather the
new parameters.  Each process's reduce-scatter output is the summed gradient
at the planner's pieces (to the summation order of the collective), and the
gathered parameters equal one process stepping the whole vector with that
summed gradient, bit for bit (the handbook's zero_check.py, with buckets, run
as real processes)."""
import os
import socket

import numpy as np
import pytest
import torch

from oracle import plan as P
from oracle import step as O

F = np.float32
SIZES = [1_000, 2_500, 700, 801, 3]


def _port():
    s = socket.socket()
    s.bind(("127.0.0.1", 0))
    p = s.getsockname()[1]
    s.close()
    return p


def _grads(pl, rank, step):
    g = np.random.default_rng(100 * step + rank).normal(0, 1e-2, pl.padded_numel).astype(F)
    pad = np.ones(pl.padded_numel, bool)
    for i, n in enumerate(pl.numels):
        pad[pl.tensor_offset[i]:pl.tensor_offset[i] + n] = False
    g[pad] = 0
    return g


def _worker(rank, world, port, cap, outdir):
    import torch.distributed as dist
    os.environ["MASTER_ADDR"], os.environ["MASTER_PORT"] = "127.0.0.1", str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)
    pl = P.make_plan(SIZES, world, cap)
    segs = P.rank_segments(pl, rank)
    master_full = np.random.default_rng(7).normal(0, 0.05, pl.padded_numel).astype(F)
    p = O.read_pieces(master_full, segs)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    gather = torch.zeros(pl.padded_numel)
    rs_out = []
    for step in (1, 2, 3):
        g = torch.from_numpy(_grads(pl, rank, step))
        pieces = []
        for b, bk in enumerate(pl.buckets):          # one reduce-scatter per bucket
            out = torch.empty(bk.shard)
            dist.reduce_scatter_tensor(out, g[bk.base:bk.base + bk.padded].contiguous(),
                                       op=dist.ReduceOp.SUM)
            pieces.append(out.numpy())
        mine = np.concatenate(pieces)
        rs_out.append(mine.copy())
        res = O.shard_step([mine], "f32", "f32", world, p, m, v, lr=1e-2, weight_decay=0.1, t=step)
        p, m, v = res.master, res.m, res.v
        local = torch.from_numpy(res.params)
        for b, bk in enumerate(pl.buckets):          # all-gather each bucket's pieces
            goff, lo, ln, _v = segs[b]
            dist.all_gather_into_tensor(gather[bk.base:bk.base + bk.padded], local[lo:lo + ln].contiguous())
    np.savez(os.path.join(outdir, f"r{rank}.npz"), gather=gather.numpy(), rs=np.stack(rs_out))
    dist.destroy_process_group()


@pytest.mark.parametrize("world,cap", [(2, 0), (4, 1500), (3, 900)])
def test_collectives_around_the_step(world, cap, tmp_path):
    torch.multiprocessing.spawn(_worker, args=(world, _port(), cap, str(tmp_path)), nprocs=world, join=True)
    pl = P.make_plan(SIZES, world, cap)
    master = np.random.default_rng(7).normal(0, 0.05, pl.padded_numel).astype(F)
    m = np.zeros_like(master)
    v = np.zeros_like(master)
    outs = [np.load(tmp_path / f"r{r}.npz") for r in range(world)]
    for step in (1, 2, 3):
        total = np.zeros(pl.padded_numel, F)
        for r in range(world):
            total = np.add(total, _grads(pl, r, step), dtype=F)
        for r in range(world):   # each rank's reduce-scatter output is the sum at its pieces
            got = outs[r]["rs"][step - 1]
            want = O.read_pieces(total, P.rank_segments(pl, r))
            assert np.allclose(got, want, rtol=1e-6, atol=1e-8)   # summation order: ~1 ulp of 1e-2
    # the gathered parameters equal one process stepping the whole vector with
    # the summed gradient the collectives produced (reassembled from the ranks'
    # reduce-scatter outputs at their pieces), bit for bit
    for step in (1, 2, 3):
        g = np.zeros(pl.padded_numel, F)
        for r in range(world):
            O.write_gather(g, P.rank_segments(pl, r), outs[r]["rs"][step - 1])
        one = O.shard_step([g], "f32", "f32", world, master, m, v, lr=1e-2, weight_decay=0.1, t=step)
        master, m, v = one.master, one.m, one.v
    for r in range(world):
        assert np.array_equal(outs[r]["gather"].view(np.uint32), master.view(np.uint32))
