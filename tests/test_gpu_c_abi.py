"""The C ABI from a plain C program (tests/c/abi_step.c: HIP runtime API for
memory and the stream, no Python or torch in that process): the fused step and
the clipped step it runs on seeded inputs equal the oracle bit for bit, and the
clipped step whose first pass takes no workspace equals the clipped step."""
import dataclasses
import os
import subprocess

import numpy as np
import pytest

import workloads as W
from gpu_harness import oracle_layout, say, storage
from oracle import casts as OC
from oracle import step as OS

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c", "abi_step")
CODE = {"f32": 0, "bf16": 1, "f16": 2}


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(BIN):
        raise RuntimeError(f"{BIN} is missing: build it with `python -m zero_sharded_mixed_plan_amd.build`")


def _bits(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint32)


@pytest.mark.parametrize("name,g,p", [("gpt2_1p5b_n8", "bf16", "bf16"), ("toy_mlp_n4", "f32", "f32"),
                                      ("llama_7b_n8", "f16", "f16"), ("flat_7p5b_n64", "f16", "f16")])
def test_c_program_matches_oracle(name, g, p, tmp_path):
    w = dataclasses.replace(W.SMALL[name], grad_dtype=g, param_dtype=p, inject_inf_step=None, max_norm=0.02,
                            loss_scale=(1024.0 if g == "f16" else 1.0), weight_decay=0.1)
    pl, lay = oracle_layout(w)
    S = lay.S
    ld = (S + 63) // 64 * 64
    sl = W.make_slices(w, lay, step=1, ld=ld, device="cpu")
    master, m, v = (x.numpy() for x in W.make_state(w, lay, "cpu"))
    rng = np.random.default_rng(w.seed + 7)
    if p == "f32":
        gather = rng.normal(0, 1, pl.padded_numel).astype(np.float32)
    else:
        gather = rng.integers(0, 0x7C00, pl.padded_numel, dtype=np.uint16)
    OS.write_gather(gather, lay.segments, OC.narrow(master, p))
    gather0 = gather.copy()

    inp, out = tmp_path / "in", tmp_path / "out"
    inp.mkdir()
    out.mkdir()
    inv = float(np.float32(1.0 / w.loss_scale))
    cfg = dict(world=w.world, rank=w.rank, bucket_cap=w.bucket_cap, grad_dtype=CODE[g], param_dtype=CODE[p],
               ld=ld, lr=repr(w.lr), beta1=repr(w.beta1), beta2=repr(w.beta2), eps=repr(w.eps),
               weight_decay=repr(w.weight_decay), step=w.t0 + 1, inv_scale=repr(inv), max_norm=repr(w.max_norm),
               ntensors=len(w.tensors))
    (inp / "config.txt").write_text("".join(f"{k} {v}\n" for k, v in cfg.items()) +
                                    "numels " + " ".join(str(n) for n in W.numels(w.tensors)) + "\n")
    storage(sl).tofile(inp / "slices.bin")
    for arr, fn in ((master, "master.bin"), (m, "m.bin"), (v, "v.bin"), (gather, "gather.bin")):
        arr.tofile(inp / fn)

    say(f"C driver {name} S={S} N={w.world} {g}->{p}")
    r = subprocess.run([BIN, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")

    slices = [storage(sl[k, :S]) for k in range(w.world)]
    pdt = np.float32 if p == "f32" else np.uint16
    # fused step into separate output state
    res = OS.shard_step(slices, g, p, w.world, master, m, v, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                        weight_decay=w.weight_decay, t=w.t0 + 1, inv_scale=inv)
    assert (out / "fused_flag.txt").read_text().split() == ["0"]
    for fn, ref in (("fused_master.bin", res.master), ("fused_m.bin", res.m), ("fused_v.bin", res.v)):
        assert np.array_equal(_bits(np.fromfile(out / fn, dtype=np.float32)), _bits(ref)), fn
    want = gather0.copy()
    OS.write_gather(want, lay.segments, res.params)
    assert np.array_equal(np.fromfile(out / "fused_gather.bin", dtype=pdt).view(want.dtype), want)

    # clipped step in place, with the coefficient the GPU computed
    flag, q, c = (out / "clip.txt").read_text().split()
    resc = OS.shard_step(slices, g, p, w.world, master, m, v, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                         weight_decay=w.weight_decay, t=w.t0 + 1, inv_scale=inv, max_norm=w.max_norm,
                         clip_override=np.float32(float(c)))
    assert int(flag) == 0
    assert abs(float(q) - resc.sumsq) <= 1e-9 * resc.sumsq
    assert abs(float(c) / float(OS.clip_coefficient(resc.sumsq, w.max_norm)) - 1) < 1e-6
    for fn, ref in (("clip_master.bin", resc.master), ("clip_m.bin", resc.m), ("clip_v.bin", resc.v)):
        assert np.array_equal(_bits(np.fromfile(out / fn, dtype=np.float32)), _bits(ref)), fn
    want = gather0.copy()
    OS.write_gather(want, lay.segments, resc.params)
    assert np.array_equal(np.fromfile(out / "clip_gather.bin", dtype=pdt).view(want.dtype), want)

    # the same clipped step with the first pass that takes no workspace: the
    # same flag, sum of squares and coefficient, and the same outputs bit for bit
    assert (out / "noalloc.txt").read_text() == (out / "clip.txt").read_text()
    for fn in ("master.bin", "m.bin", "v.bin", "gather.bin"):
        assert (out / ("noalloc_" + fn)).read_bytes() == (out / ("clip_" + fn)).read_bytes(), fn
