"""The plain streaming copy (the bandwidth reference of the benchmark) copies
exactly, at sizes that end inside a workgroup's range and at zero."""
import pytest
import torch

import zero_sharded_mixed_plan_amd as Z

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 16, 8192 * 3 + 48, (1 << 24) + 2064])
def test_stream_copy(nbytes):
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    Z.zero_stream_copy(dst.data_ptr(), src.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert bool(torch.all(dst[nbytes:] == 0))
