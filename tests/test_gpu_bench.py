"""The benchmark's JSON line, produced on the GPU for the toy workload through
bench.run: the fields a report is read from (throughput, the roofline of the
dominant kernel, the oracle's host throughput) are present and consistent."""
import json

import pytest
import torch

import bench

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_bench_line_toy():
    res = bench.run("toy_mlp_n4", steps=3, warmup=1, with_cpu=True, copy_gbps=None)
    json.dumps(res)   # serialisable as the one-line report
    assert res["metric"] == bench.METRIC and res["unit"] == "elements/s"
    assert res["n_gpus"] == 1 and res["steps"] == 3 and res["warmup"] == 1 and res["data"] == "synthetic"
    c = res["config"]
    assert c["workload"] == "toy_mlp_n4" and c["shard_elements"] == 4803 and c["world"] == 4
    assert res["value"] == pytest.approx(4803 / (res["ms_per_step"] * 1e-3), rel=1e-12)
    r = res["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBPS
    assert r["achieved"] > 0 and r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-12)
    k_ms = c["kernel_ms"][r["kernel"]]   # reported to 1e-5 ms
    assert r["achieved"] == pytest.approx(r["bytes_per_element"] * 4803 / (k_ms * 1e-3) / 1e9,
                                          rel=1e-5 / k_ms)
    for k in c["kernel_ms"]:   # per-launch HIP-event times: min <= median, min <= mean
        assert 0 < c["kernel_ms_min"][k] <= c["kernel_ms_median"][k]
        assert c["kernel_ms_min"][k] <= c["kernel_ms"][k] + 1e-5
    assert c["hip_graph_ms_per_step"] is not None and c["hip_graph_ms_per_step"] > 0
    cb = res["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "elements/s" and cb["cores"] >= 1 and cb["value"] > 0
    assert cb["value_1thread"] > 0
