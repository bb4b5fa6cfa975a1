"""The step's launches can be captured in a HIP graph (no memset nodes: the
overflow flag is reset by a kernel) and replayed: every replay, with eager
work and synchronisation between replays, gives the eager result bit for bit.
The step's constants (bias corrections for step t, 1/N, 1/scale) are kernel
arguments, so a captured graph replays the steps it was captured with."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
import zero_sharded_mixed_plan_amd as Z
from gpu_harness import Rig, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(bufs):
    return [b.detach().clone().view(torch.int32) for b in bufs]


@pytest.mark.parametrize("clip", [False, True])
@pytest.mark.parametrize("name", ["gpt2_1p5b_n8", "toy_mlp_n4"])
def test_graph_replays_match_eager(name, clip):
    w = dataclasses.replace(W.SMALL[name], max_norm=(0.05 if clip else 0.0))
    eager = Rig(w, layout=Z.ZERO_STATE_TILED)
    graph = Rig(w, layout=Z.ZERO_STATE_TILED)
    _cpu, sl = eager.slices(1)
    sl2 = sl.clone()
    say(f"graph {name} clip={clip} S={eager.S}")

    def two_steps(rig, slices):
        if clip:
            for t in (1, 2):
                rig.reduce_norm(slices)
                rig.stash_step(rig.A, t)
        else:
            rig.fused(slices, rig.A, rig.B, 1)
            rig.fused(slices, rig.B, rig.A, 2)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):      # one eager warm-up on the capture stream
        two_steps(graph, sl2)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        two_steps(graph, sl2)
    torch.cuda.synchronize()
    # eager: the warm-up, then the same pair of steps once per replay
    two_steps(eager, sl)
    for replay in range(4):
        two_steps(eager, sl)
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(_bits(eager.A), _bits(graph.A)):
            assert torch.equal(a, b), f"replay {replay}: state differs"
        assert torch.equal(eager.gather.view(torch.int16) if eager.gather.dtype != torch.float32 else eager.gather,
                           graph.gather.view(torch.int16) if graph.gather.dtype != torch.float32 else graph.gather)
        assert int(eager.flag.item()) == int(graph.flag.item()) == 0
        del junk
