"""Data-parallel training with the GPU step inside, as the handbook checks its
ZeroAdam ("ZeRO 与 FSDP：切分优化器状态、梯度与参数", zero_check.py): four
processes each run forward and backward of the page's MLP (Linear 64->256,
GELU, Linear 256->10) on their 8 of 32 samples, reduce-scatter the flat
gradient (SUM) over gloo, step their shard with the HIP library (the
reduce-scatter output is one stored buffer, divided by N in the step), and
all-gather the new parameters.  After three steps every process holds the same
model, within the page's 1e-5 of single-process torch.optim.Adam on the full
batch.  The four processes share the one GPU; gloo only sees host tensors."""
import os
import socket

import pytest
import torch

pytestmark = pytest.mark.gpu

WORLD = 4


def _port():
    s = socket.socket()
    s.bind(("127.0.0.1", 0))
    p = s.getsockname()[1]
    s.close()
    return p


def _model():
    torch.manual_seed(0)
    return torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(), torch.nn.Linear(256, 10))


def _data():
    torch.manual_seed(123)
    return torch.randn(32, 64), torch.randint(0, 10, (32,))


def _worker(rank, world, port, outdir, device_control):
    import torch.distributed as dist

    import zero_sharded_mixed_plan_amd as Z
    from zero_sharded_mixed_plan_amd.optim import ZeroAdam
    os.environ["MASTER_ADDR"], os.environ["MASTER_PORT"] = "127.0.0.1", str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)
    torch.cuda.set_device(0)
    model = _model()
    X, Y = _data()
    loss_fn = torch.nn.CrossEntropyLoss()
    params = list(model.parameters())
    numels = [p.numel() for p in params]
    psi = sum(numels)
    flat0 = torch.cat([p.detach().reshape(-1) for p in params])
    plan = Z.Plan(numels, world)
    S, NS = plan.shard_numel, plan.padded_numel
    goff, lo, ln, _valid = plan.segments(rank)[0]      # one bucket: the rank's slot r*S
    full = torch.zeros(NS)
    full[:psi] = flat0
    master = full[goff:goff + ln].cuda()
    opt = ZeroAdam(numels, world, rank, lr=1e-2, grad_dtype=torch.float32, param_dtype=torch.float32,
                   master=master, device_control=device_control)
    loc = slice(rank * 32 // world, (rank + 1) * 32 // world)
    for _t in range(3):
        model.zero_grad()
        loss_fn(model(X[loc]), Y[loc]).backward()
        g = torch.zeros(NS)
        g[:psi] = torch.cat([p.grad.reshape(-1) for p in params])
        mine = torch.empty(S)
        dist.reduce_scatter_tensor(mine, g, op=dist.ReduceOp.SUM)      # host tensors only
        ok = opt.step(mine.view(1, S).cuda())                          # one stored buffer, / N inside
        assert ok is None if device_control else ok
        piece = opt.gather[goff:goff + ln].cpu()                        # synchronous copy to host
        gathered = torch.empty(NS)
        dist.all_gather_into_tensor(gathered, piece)
        off = 0
        with torch.no_grad():
            for p in params:
                p.copy_(gathered[off:off + p.numel()].view_as(p))
                off += p.numel()
    assert opt.t == 3
    torch.save([p.detach().clone() for p in params], os.path.join(outdir, f"r{rank}.pt"))
    dist.destroy_process_group()


@pytest.mark.parametrize("device_control", [False, True])
def test_four_ranks_match_torch_adam(device_control, tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[gpu] data-parallel toy over gloo, 4 processes, device_control={device_control}", flush=True)
    torch.multiprocessing.spawn(_worker, args=(WORLD, _port(), str(tmp_path), device_control), nprocs=WORLD,
                                join=True)
    ref = _model()
    X, Y = _data()
    opt_ref = torch.optim.Adam(ref.parameters(), lr=1e-2)
    loss_fn = torch.nn.CrossEntropyLoss()
    for _t in range(3):
        opt_ref.zero_grad()
        loss_fn(ref(X), Y).backward()
        opt_ref.step()
    got = [torch.load(tmp_path / f"r{r}.pt", weights_only=True) for r in range(WORLD)]
    for r in range(1, WORLD):
        assert all(torch.equal(a, b) for a, b in zip(got[0], got[r])), f"rank {r} differs from rank 0"
    diff = max((a - b).abs().max().item() for a, b in zip(ref.parameters(), got[0]))
    assert diff < 1e-5, diff
