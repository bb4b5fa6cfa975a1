"""Pins of the per-parameter dim-0 layout (FSDP2 fully_shard) in the oracle
planner: the page's printed local shapes, PyTorch's own fully_shard on CPU over
gloo (local shapes and local data on every rank), and the sharding invariants."""
import os
import socket

import numpy as np
import pytest
import torch

from conftest import golden_rows
from oracle import plan as P
from oracle import step as O

F = np.float32


def test_page_printed_local_shapes():
    rows = golden_rows("fsdp2_local_shapes.txt")
    assert len(rows) == 2
    for full, world, rank, local in rows:
        full = tuple(int(x) for x in full.split(","))
        local = tuple(int(x) for x in local.split(","))
        assert P.dim0_local_shape(full, int(world), int(rank)) == local
        pl = P.make_plan_dim0([full], int(world))
        _goff, _lo, ln, valid = P.rank_segments(pl, int(rank))[0]
        assert ln == valid == local[0] * local[1]


SHAPES = [(256, 64), (256,), (10, 256), (10,), (7, 3, 5), (1, 9), (3,), (2, 4)]


def _fsdp2_worker(rank, world, port, shapes, outdir):
    import torch.distributed as dist
    from torch.distributed.device_mesh import init_device_mesh
    from torch.distributed.fsdp import fully_shard
    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)
    mesh = init_device_mesh("cpu", (world,))
    torch.manual_seed(0)
    mod = torch.nn.Module()
    mod.ps = torch.nn.ParameterList([torch.nn.Parameter(torch.randn(*s)) for s in shapes])
    fully_shard(mod, mesh=mesh)
    out = {}
    for i, p in enumerate(mod.ps):
        loc = p.to_local().detach()
        out[f"shape{i}"] = np.array(loc.shape, dtype=np.int64)
        out[f"data{i}"] = loc.reshape(-1).numpy().astype(F)
    np.savez(os.path.join(outdir, f"rank{rank}.npz"), **out)
    dist.destroy_process_group()


def _free_port():
    s = socket.socket()
    s.bind(("127.0.0.1", 0))
    port = s.getsockname()[1]
    s.close()
    return port


@pytest.mark.parametrize("world", [2, 3, 4])
def test_matches_pytorch_fully_shard(world, tmp_path):
    """Every rank's local shard from PyTorch's fully_shard equals the valid part
    of that rank's piece of the planner's layout, read from the parameters
    flattened into the padded gather layout."""
    torch.multiprocessing.spawn(_fsdp2_worker, args=(world, _free_port(), SHAPES, str(tmp_path)),
                                nprocs=world, join=True)
    torch.manual_seed(0)
    full = [torch.randn(*s).reshape(-1).numpy().astype(F) for s in SHAPES]
    pl = P.make_plan_dim0(SHAPES, world)
    flat = np.zeros(pl.padded_numel, F)
    for i, x in enumerate(full):
        flat[pl.tensor_offset[i]:pl.tensor_offset[i] + x.size] = x
    for r in range(world):
        got = np.load(tmp_path / f"rank{r}.npz")
        segs = P.rank_segments(pl, r)
        local = O.read_pieces(flat, segs)
        for i, s in enumerate(SHAPES):
            assert tuple(got[f"shape{i}"]) == P.dim0_local_shape(s, world, r), (i, r)
            _goff, lo, ln, valid = segs[pl.tensor_bucket[i]]
            assert np.array_equal(local[lo:lo + valid], got[f"data{i}"]), (i, r)
            assert np.all(local[lo + valid:lo + ln] == 0)       # padding rows


@pytest.mark.parametrize("world", [1, 2, 3, 8])
def test_gather_buffer_is_each_parameter_padded(world):
    """Each parameter's bucket in the gather buffer is the parameter padded to
    N * ceil(rows / N) rows, in row-major order, and the ranks' pieces tile it."""
    shapes = [(5, 3), (0, 4), (16,), (9, 2, 2), ()]
    pl = P.make_plan_dim0(shapes, world)
    for i, s in enumerate(shapes):
        b = pl.buckets[pl.tensor_bucket[i]]
        if pl.numels[i] == 0:
            continue
        rows = s[0] if s else 1
        rest = pl.numels[i] // rows
        assert b.padded == world * (-(-rows // world)) * rest
        assert pl.tensor_offset[i] == b.base
    seen = np.zeros(pl.padded_numel, int)
    for r in range(world):
        for goff, _lo, ln, _v in P.rank_segments(pl, r):
            seen[goff:goff + ln] += 1
    assert np.all(seen == 1)


def test_union_of_dim0_shards_equals_unsharded():
    """Stepping every rank's per-parameter pieces and gathering equals one step
    over the whole padded vector, bit for bit; padding rows stay +0."""
    world = 3
    shapes = [(256, 64), (256,), (10, 256), (10,)]
    pl = P.make_plan_dim0(shapes, world)
    NS = pl.padded_numel
    rng = np.random.default_rng(7)
    pad = np.ones(NS, bool)
    for i, n in enumerate(pl.numels):
        pad[pl.tensor_offset[i]:pl.tensor_offset[i] + n] = False
    g = rng.normal(0, 1e-2, NS).astype(F)
    master = rng.normal(0, 0.05, NS).astype(F)
    g[pad] = 0
    master[pad] = 0
    z = np.zeros(NS, F)
    gather = np.zeros(NS, F)
    for r in range(world):
        segs = P.rank_segments(pl, r)
        res = O.shard_step([O.read_pieces(g, segs)], "f32", "f32", 1, O.read_pieces(master, segs),
                           O.read_pieces(z, segs), O.read_pieces(z, segs), lr=1e-2, t=1)
        O.write_gather(gather, segs, res.params)
    one = O.shard_step([g], "f32", "f32", 1, master, z, z, lr=1e-2, t=1)
    assert np.array_equal(gather.view(np.uint32), one.params.view(np.uint32))
    assert np.all(gather[pad].view(np.uint32) == 0)
    # per-rank optimizer state: 12 bytes per local element, about 1/N of the padded total
    assert P.state_bytes(pl) == 12 * sum(b.shard for b in pl.buckets)
