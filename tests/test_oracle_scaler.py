"""Pins of the loss-scale policy: the oracle against PyTorch's own update
routine (torch._amp_update_scale_, what torch.amp.GradScaler.update runs) on
random overflow sequences, and the closed cases."""
import numpy as np
import pytest
import torch

from oracle import scaler as SC

F = np.float32


def _torch_run(init, growth, backoff, interval, flags):
    s = torch.tensor([init], dtype=torch.float32)
    t = torch.tensor([0], dtype=torch.int32)
    out = []
    for fl in flags:
        torch._amp_update_scale_(s, t, torch.tensor([1.0 if fl else 0.0]), growth, backoff, interval)
        out.append((float(s.item()), int(t.item())))
    return out


@pytest.mark.parametrize("seed,interval,p", [(0, 3, 0.2), (1, 1, 0.5), (2, 2000, 0.001), (3, 7, 0.0),
                                             (4, 5, 0.9)])
def test_matches_torch_update(seed, interval, p):
    rng = np.random.default_rng(seed)
    n = 5000 if interval == 2000 else 300
    flags = (rng.random(n) < p).tolist()
    want = _torch_run(65536.0, 2.0, 0.5, interval, flags)
    s = SC.ScalerState(scale=F(65536.0), growth_tracker=0, growth_interval=interval)
    for fl, (ws, wt) in zip(flags, want):
        s = SC.update(s, fl)
        assert (float(s.scale), s.growth_tracker) == (ws, wt)


def test_closed_cases():
    s = SC.ScalerState(scale=F(1024.0), growth_tracker=0, growth_interval=2)
    s = SC.update(s, False)
    assert (s.scale, s.growth_tracker) == (1024.0, 1)
    s = SC.update(s, False)
    assert (s.scale, s.growth_tracker) == (2048.0, 0)
    s = SC.update(s, True)
    assert (s.scale, s.growth_tracker) == (1024.0, 0)
    assert SC.inv_scale(s) == F(2.0 ** -10)
    big = SC.ScalerState(scale=F(3e38), growth_tracker=0, growth_interval=1)
    assert SC.update(big, False).scale == F(3e38)          # growth past fp32 range: kept
    odd = SC.ScalerState(scale=F(3.0), growth_tracker=0, growth_factor=1.5, growth_interval=1)
    assert SC.update(odd, False).scale == F(4.5) == _torch_run(3.0, 1.5, 0.5, 1, [False])[0][0]
