#!/usr/bin/env python3
"""Benchmark: one rank's sharded mixed-precision AdamW step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]

A step is one pass of the whole hot path over one rank's shard: reduce the N
gradient slices, average, unscale, check for overflow (and, for the clipped
workload, the two-pass global-norm clip), AdamW on the fp32 master/m/v, and the
rounded parameters written into the rank's slots of the all-gather buffer.
Inputs are seeded synthetic data resident in HBM before the timed region.

Prints ONE JSON line (the default workload, the largest one: the Llama-7B-like
tensor list, N = 8, rank 7, a shard of 842,301,952 elements, bf16 slices and
parameters, fp32 master/m/v; the oracle is timed on one full step over it).
`--workload all` also writes one line per workload to stderr (and to --report
if given), and prints the default workload's line last on stdout; there the
oracle is timed on the host beside each of the five workloads (`cpu_baseline`:
a bounded sample of each, one whole step for the default workload).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT = "llama_7b_n8"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published peak
METRIC = "shard elements/sec of fused ZeRO AdamW step; achieved HBM GB/s vs peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def round_up(x, m):
    return (x + m - 1) // m * m


def _code_only(text: str) -> str:
    """C++ source without comments, trailing blanks or empty lines (string and
    character literals kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_hash() -> str:
    """Hash of the code (comments aside) of the kernels and their launch
    configuration: profiles taken on other code are not reported as current."""
    h = hashlib.sha256()
    for f in ("kernels.hip", "abi.cpp", "zero_internal.h"):
        with open(os.path.join(ROOT, "zero_sharded_mixed_plan_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes of the kernel's launches in one step (the update of a large
    shard is several launches) from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_step"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# the CPU oracle, timed on a bounded sample (cpu_baseline)
# ---------------------------------------------------------------------------

def cpu_baseline(w, slices, tiled_state, S, full_step=False, target_s=5.0, max_elems=1 << 26,
                 chunk=1 << 20):
    """The oracle as written, timed on the host's cores.  full_step: one whole
    step over all S elements of the rank's shard (inputs copied to the host
    first, the oracle's arithmetic alone is timed); otherwise a bounded sample,
    the first max_elems elements stepped repeatedly for about target_s.  Both
    also time one thread on the first chunk."""
    import concurrent.futures as cf

    import numpy as np
    import torch

    import zero_sharded_mixed_plan_amd as Z
    from oracle import step as OS

    threads = max(1, min(os.cpu_count() or 1, 16))
    if full_step:
        n = S
    else:
        n = min(S, max_elems)
        n -= n % chunk if n > chunk else 0
        n = max(n, min(S, chunk))
    T = Z.ZERO_STATE_TILE
    chunk = max(T, chunk // T * T)

    def host(t):
        t = t.detach().cpu().contiguous()
        if t.dtype in (torch.bfloat16, torch.float16):
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    t_copy = time.perf_counter()
    sl = [host(slices[k, :n]) for k in range(w.world)]
    st = host(tiled_state[:(n + T - 1) // T * 3 * T]).reshape(-1, 3, T)
    p, m, v = (np.ascontiguousarray(st[:, i, :].reshape(-1)[:n]) for i in range(3))
    del st
    t_copy = time.perf_counter() - t_copy
    kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              t=w.t0 + 1, inv_scale=1.0 / w.loss_scale, max_norm=w.max_norm)

    def work(a):
        b = min(n, a + chunk)
        OS.shard_step([s[a:b] for s in sl], w.grad_dtype, w.param_dtype, w.world, p[a:b], m[a:b],
                      v[a:b], **kw)
        return b - a

    done = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        while True:
            done += sum(ex.map(work, range(0, n, chunk)))
            if full_step or time.perf_counter() - t0 >= target_s or done >= 64 * n:
                break
    dt = time.perf_counter() - t0
    # the same oracle on one thread, over the first chunk
    one, t1 = 0, time.perf_counter()
    while True:
        one += work(0)
        if time.perf_counter() - t1 >= max(0.5, dt / 10) or one >= 64 * min(n, chunk):
            break
    dt1 = time.perf_counter() - t1
    what = (f"one full step over all {n} elements of the rank's shard" if full_step else
            f"first {n} of the shard's {S} elements, stepped {done // n} time(s)")
    return {"value": done / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} in {chunk}-element chunks on {threads} threads ({dt:.2f} s of "
                      f"wall time; inputs copied to the host beforehand in {t_copy:.1f} s, not timed)",
            "seconds": dt, "elements": done,
            "value_1thread": one / dt1,
            "sample_1thread": f"first {min(n, chunk)} elements, stepped {one // min(n, chunk)} time(s) "
                              f"on one thread ({dt1:.1f} s)"}


# ---------------------------------------------------------------------------
# one workload on the GPU
# ---------------------------------------------------------------------------

# Other forms of the same step on the GPT-2 shard (extra lines of --workload
# all): one stored reduce-scatter output read in place of the N slices, one
# full all-reduced gradient read at the rank's slots (ZeRO-1), the clipped
# path's reduction pass alone, and the per-parameter dim-0 layout (FSDP2
# fully_shard: 580 pieces, one per parameter).
VARIANTS = {
    "gpt2_1p5b_n8_stored_rs": ("gpt2_1p5b_n8", "stored", "flat"),
    "gpt2_1p5b_n8_zero1_full": ("gpt2_1p5b_n8", "full", "flat"),
    "gpt2_1p5b_n8_reduce_only": ("gpt2_1p5b_n8", "reduce_only", "flat"),
    "gpt2_1p5b_n8_fsdp2_dim0": ("gpt2_1p5b_n8", "slices", "dim0"),
}


def run(name, steps, warmup, with_cpu, copy_gbps=None, ld_pad=0):
    import dataclasses

    import torch

    import workloads as W
    import zero_sharded_mixed_plan_amd as Z
    from zero_sharded_mixed_plan_amd.optim import dtype_code, pack_state, state_arg_dict

    base, source, plan_layout = VARIANTS.get(name, (name, "slices", "flat"))
    w = W.FULL[base]
    layout = Z.ZERO_STATE_TILED
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if plan_layout == "dim0":
        w = dataclasses.replace(w, plan_layout="dim0")
        plan = Z.Plan.dim0([shape for _n, shape in w.tensors], w.world)
    else:
        plan = Z.Plan(W.numels(w.tensors), w.world, w.bucket_cap)
    table = None
    if plan.num_buckets > 192:   # as ZeroAdam does: the device piece table, one launch per step
        table = torch.empty(plan.piece_table_bytes(), dtype=torch.uint8, device=dev)
        plan.attach_piece_table(w.rank, table.data_ptr(), table.numel())
    S = plan.shard_numel
    lay = W.Layout(S=S, segments=plan.segments(w.rank), tensor_flat_off=plan.tensor_offsets())
    ld = round_up(S, 64) + ld_pad
    log(f"[bench] {name}: S={S} N={w.world} rank={w.rank} buckets={plan.num_buckets} "
        f"grads={w.grad_dtype} params={w.param_dtype} clip={w.max_norm}")

    t_gen = time.perf_counter()
    count, glayout, gld = 0, Z.ZERO_GRAD_SHARD, ld
    if source == "stored":        # one [S] buffer holding the summed gradient
        slices = W.make_slices(dataclasses.replace(w, world=1), lay, step=1, ld=ld, device=dev)
        count, gld = 1, 0
    elif source == "full":        # one full flat gradient [padded]
        slices = W.make_full_grads(w, plan.padded_numel, plan.tensor_offsets(), 1, step=1, device=dev)
        count, glayout, gld = 1, Z.ZERO_GRAD_FULL, 0
    else:
        slices = W.make_slices(w, lay, step=1, ld=ld, device=dev)
        if w.inject_inf_step is not None:   # time clean steps: draw the slices of a clean step
            slices = W.make_slices(w, lay, step=w.inject_inf_step + 1, ld=ld, device=dev, out=slices)
    n_read = w.world if count == 0 else count   # gradient buffers each step reads
    p0, m0, v0 = W.make_state(w, lay, dev)
    A = [pack_state(p0, m0, v0, plan.state_numel(layout))]
    del p0, m0, v0
    B = [torch.empty_like(A[0])]
    gather = torch.zeros(plan.padded_numel, dtype=W.torch_dtype(w.param_dtype), device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    clip = w.max_norm > 0
    reduce_only = source == "reduce_only"
    if clip or reduce_only:
        g = torch.empty(S, dtype=torch.float32, device=dev)
        ws = torch.empty(plan.workspace_bytes(), dtype=torch.uint8, device=dev)
        sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        coef = torch.zeros(1, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s")

    stream = torch.cuda.current_stream()
    st = stream.cuda_stream
    gb = Z.DTYPE_BYTES[dtype_code(W.torch_dtype(w.grad_dtype))]
    pb = Z.DTYPE_BYTES[dtype_code(W.torch_dtype(w.param_dtype))]
    common = dict(rank=w.rank, gather=gather.data_ptr(), param_dtype=dtype_code(gather.dtype),
                  lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)       # creates the underlying hipEvent
        return evs

    state = {"cur": A, "nxt": B, "t": w.t0}

    def step(ev=None):
        st = torch.cuda.current_stream().cuda_stream   # the capture stream while a graph is recorded
        t = state["t"] + 1
        if reduce_only:
            e0, e1 = ev if ev else (None, None)
            if e0 is not None:
                e0.record(stream)
            Z.zero_reduce_shard(plan, slices.data_ptr(), ld, dtype_code(slices.dtype),
                                1.0 / w.loss_scale, g.data_ptr(), ws.data_ptr(), True, st)
            if e1 is not None:
                e1.record(stream)
        elif clip:
            e_red0, e_red1, e_up0, e_up1 = ev if ev else (None,) * 4
            if e_red0 is not None:
                e_red0.record(stream)
            Z.zero_reduce_shard(plan, slices.data_ptr(), ld, dtype_code(slices.dtype),
                                1.0 / w.loss_scale, g.data_ptr(), ws.data_ptr(), True, st)
            if e_red1 is not None:
                e_red1.record(stream)
            Z.zero_shard_norm(plan, ws.data_ptr(), 0.0, w.max_norm, flag.data_ptr(),
                              sumsq.data_ptr(), coef.data_ptr(), st)
            cur = state["cur"]
            a = Z.adam_args(g_stash=g.data_ptr(), clip_coef=coef.data_ptr(), skip_in=flag.data_ptr(),
                            step=t, ev_begin=e_up0.cuda_event if e_up0 else None,
                            ev_end=e_up1.cuda_event if e_up1 else None,
                            **state_arg_dict(layout, cur, cur), **common)
            Z.zero_adam_step(plan, a, st)
        else:
            e0, e1 = ev if ev else (None, None)
            src, dst = state["cur"], state["nxt"]
            a = Z.adam_args(grad=slices.data_ptr(), grad_ld=gld, grad_dtype=dtype_code(slices.dtype),
                            grad_count=count, grad_layout=glayout,
                            inv_scale=1.0 / w.loss_scale, overflow_out=flag.data_ptr(), step=t,
                            ev_begin=e0.cuda_event if e0 else None,
                            ev_end=e1.cuda_event if e1 else None,
                            **state_arg_dict(layout, src, dst), **common)
            Z.zero_adam_step(plan, a, st)
            # the data are finite, so every step commits: swap without a host read
            state["cur"], state["nxt"] = dst, src
        state["t"] = t

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if int(flag.item()) != 0:
        raise RuntimeError("warm-up step overflowed on finite synthetic data")

    n_ev = 4 if (clip and not reduce_only) else 2
    evs = [new_events(n_ev) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if int(flag.item()) != 0:
        raise RuntimeError("timed step overflowed on finite synthetic data")

    ms_step = wall / steps * 1e3
    graph_ms = None
    if S <= (1 << 16) and not reduce_only:
        # a latency-bound shard: the same steps captured once in a HIP graph and
        # replayed, which removes the per-launch host overhead (the step's
        # constants are kernel arguments, so the replays repeat the captured steps)
        per = 10
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(per):
                step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per):
                step()
        torch.cuda.synchronize()
        reps = max(1, steps // per)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        if int(flag.item()) != 0:
            raise RuntimeError("a replayed step overflowed on finite synthetic data")
        graph_ms = g0.elapsed_time(g1) / (reps * per)
        del graph
    kernels, per_launch = {}, {}
    if reduce_only:
        red = [evs[i][0].elapsed_time(evs[i][1]) for i in range(steps)]
        per_launch["reduce_kernel"] = red
        kernels["reduce_kernel"] = (sum(red) / steps, w.world * gb + 4)
        bpe_total = w.world * gb + 4
    elif clip:
        red = [evs[i][0].elapsed_time(evs[i][1]) for i in range(steps)]
        upd = [evs[i][2].elapsed_time(evs[i][3]) for i in range(steps)]
        per_launch["reduce_kernel"], per_launch["step_kernel_stash"] = red, upd
        kernels["reduce_kernel"] = (sum(red) / steps, w.world * gb + 4)
        kernels["step_kernel_stash"] = (sum(upd) / steps, 4 + 24 + pb)
        bpe_total = w.world * gb + 24 + pb + 8
    else:
        upd = [evs[i][0].elapsed_time(evs[i][1]) for i in range(steps)]
        per_launch["step_kernel"] = upd
        kernels["step_kernel"] = (sum(upd) / steps, n_read * gb + 24 + pb)
        bpe_total = n_read * gb + 24 + pb
    dom = max(kernels, key=lambda k: kernels[k][0])
    k_ms, k_bpe = kernels[dom]
    achieved = k_bpe * S / (k_ms * 1e-3) / 1e9
    traffic = load_traffic(dom, name)
    out = {
        "metric": METRIC,
        "value": S / (ms_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the type the step computes in (every workload reduces, updates and
        # keeps its state in fp32); the storage types are in config below
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": name, "gradient_source": {"slices": "N slices (fused reduce-scatter)",
                                                  "stored": "one stored reduce-scatter output",
                                                  "full": "one full all-reduced gradient (ZeRO-1)",
                                                  "reduce_only": "N slices, reduction pass alone"}[source],
            "plan_layout": {"flat": "flat buckets", "dim0": "per-parameter dim-0 (FSDP2)"}[plan_layout],
            "piece_table": table is not None,
            "shard_elements": S, "world": w.world, "rank": w.rank,
            "grad_dtype": w.grad_dtype, "param_dtype": w.param_dtype, "state_dtype": "f32",
            "buckets": plan.num_buckets,
            "clip": clip and not reduce_only, "state_layout": "tiled",
            "algorithmic_bytes_per_element": bpe_total,
            "step_GBps": bpe_total * S / (ms_step * 1e-3) / 1e9,
            "kernel_ms": {k: round(v[0], 5) for k, v in kernels.items()},
            "kernel_ms_median": {k: round(sorted(v)[len(v) // 2], 5) for k, v in per_launch.items()},
            "kernel_ms_min": {k: round(min(v), 5) for k, v in per_launch.items()},
            "hip_graph_ms_per_step": graph_ms,
            "parallelism": "one rank of N (single GPU)",
            "stream_copy_GBps": copy_gbps,
            "dominant_kernel_of_stream_copy": (achieved / copy_gbps) if copy_gbps else None,
        },
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "bytes_per_element": k_bpe,
                     # achieved and traffic cover all of the kernel's launches in one
                     # step: a large shard is updated in several launches
                     "per": "step",
                     "traffic": traffic},
    }
    if with_cpu:
        # the headline workload: one whole oracle step over the shard; the
        # others: a bounded sample of theirs
        out["cpu_baseline"] = cpu_baseline(w, slices, state["cur"][0], S, full_step=(name == DEFAULT))
    del slices, A, B, gather
    torch.cuda.empty_cache()
    return out


def device_copy_gbps(gib=2.0, launches=10) -> float:
    """Bandwidth of the library's plain streaming copy (zero_stream_copy: the
    step's own non-temporal 16-byte loads and stores, one read and one write
    stream) on this GPU, bytes read + written per second: the practical ceiling
    a streaming kernel is compared with besides the published peak."""
    import torch

    import zero_sharded_mixed_plan_amd as Z
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream()
    Z.zero_stream_copy(dst.data_ptr(), src.data_ptr(), 4 * n, st.cuda_stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(launches):
        Z.zero_stream_copy(dst.data_ptr(), src.data_ptr(), 4 * n, st.cuda_stream)
    e1.record(st)
    torch.cuda.synchronize()
    if not torch.equal(dst, src):
        raise RuntimeError("zero_stream_copy produced a wrong copy")
    ms = e0.elapsed_time(e1) / launches
    del src, dst
    torch.cuda.empty_cache()
    return 8 * n / (ms * 1e-3) / 1e9


def copy_probe(steps, warmup, gib=4.0):
    """A plain device-to-device copy kernel of known size (torch's elementwise
    multiply by 1 over fp32): reference bandwidth on this GPU, and the counter
    calibration (HBM bytes read and written per launch are both 4 * n)."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch.mul(src, 1.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    out = {"probe": "copy", "elements": n, "bytes_read": 4 * n, "bytes_written": 4 * n,
           "ms_per_launch": ms, "GBps": 8 * n / (ms * 1e-3) / 1e9}
    print(json.dumps(out), flush=True)


def checkpoint_probe(name="gpt2_1p5b_n8", reps=2):
    """Sharded checkpoint of one rank's optimizer state (master, m, v in the
    tiled device layout; 12 B per shard element on disk plus a 128-byte header):
    save and load through the library, timed on the host clock, bytes of the
    file per second.  The loaded state must equal the saved one bit for bit."""
    import tempfile

    import torch

    import workloads as W
    import zero_sharded_mixed_plan_amd as Z
    from zero_sharded_mixed_plan_amd.optim import pack_state, unpack_state

    w = W.FULL[name]
    plan = Z.Plan(W.numels(w.tensors), w.world, w.bucket_cap)
    S = plan.shard_numel
    lay = W.Layout(S=S, segments=plan.segments(w.rank), tensor_flat_off=plan.tensor_offsets())
    p0, m0, v0 = W.make_state(w, lay, "cuda")
    A = pack_state(p0, m0, v0, plan.state_numel(Z.ZERO_STATE_TILED))
    del p0, m0, v0
    B = torch.full_like(A, float("nan"))
    sc = Z.Scaler(init_scale=w.loss_scale)
    st = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    nbytes = 12 * S + 128
    save_s, load_s = [], []
    with tempfile.TemporaryDirectory(dir=os.environ.get("TMPDIR", "/tmp")) as d:
        path = os.path.join(d, f"rank{w.rank}.zshard")
        for _ in range(reps):
            t0 = time.perf_counter()
            Z.zero_checkpoint_save(plan, w.rank, path, Z.ZERO_STATE_TILED, A.data_ptr(), 0, 0,
                                   w.t0, sc.s, st)
            save_s.append(time.perf_counter() - t0)
            if os.path.getsize(path) != nbytes:
                raise RuntimeError("checkpoint file has the wrong size")
            t0 = time.perf_counter()
            meta = Z.zero_checkpoint_load(plan, w.rank, path, Z.ZERO_STATE_TILED, B.data_ptr(), 0, 0, st)
            load_s.append(time.perf_counter() - t0)
            # the S valid elements of master, m and v (the load leaves the last
            # tile's positions past S alone)
            same = all(torch.equal(a.view(torch.int32), b.view(torch.int32))
                       for a, b in zip(unpack_state(A, S), unpack_state(B, S)))
            if int(meta.step) != w.t0 or not same:
                raise RuntimeError("loaded state differs from the saved state")
    out = {"metric": "sharded checkpoint of one rank's optimizer state (save / load)",
           "workload": name, "shard_elements": S, "file_bytes": nbytes,
           "save_s": min(save_s), "load_s": min(load_s),
           "save_GBps": nbytes / min(save_s) / 1e9, "load_GBps": nbytes / min(load_s) / 1e9,
           "note": "host clock; device -> pinned staging -> file (page cache), FNV-1a checksums; "
                   "the load verifies the checksums in a read-only pass before copying; the loaded "
                   "state is compared with the saved one bit for bit"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline")
    ap.add_argument("--report", default=None, help="append every workload's JSON line here")
    ap.add_argument("--copy-probe", action="store_true", help="time a plain copy kernel only")
    ap.add_argument("--checkpoint", action="store_true",
                    help="time a sharded checkpoint save and load of the default workload's state")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="first run a plain copy of known size (torch.neg over 2^28 fp32, 3 "
                         "launches) in this process, to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one rank on one GPU; --gpus {args.gpus} is not "
              "supported (the multi-GPU collectives are out of scope)", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.steps, args.warmup)
        return
    if args.checkpoint:
        checkpoint_probe()
        return
    if args.copy_calibrate:
        import torch
        src = torch.randn(1 << 28, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x torch.neg over 2^28 fp32 (1 GiB read + 1 GiB written)")
        del src, dst
    import workloads as W
    names = W.ORDER + list(VARIANTS) if args.workload == "all" else [args.workload]
    if args.workload != "all" and args.workload not in W.FULL and args.workload not in VARIANTS:
        sys.exit(f"unknown workload {args.workload}; one of {W.ORDER + list(VARIANTS)} or 'all'")
    copy_gbps = device_copy_gbps()
    log(f"[bench] plain streaming copy (zero_stream_copy): {copy_gbps:.0f} GB/s")
    lines = {}
    for nm in names:
        # the oracle is timed beside every one of the five workloads (bounded
        # samples), not beside the GPT-2 step's other forms
        res = run(nm, args.steps, args.warmup, with_cpu=(not args.no_cpu and (nm == DEFAULT or (
                      args.workload == "all" and nm in W.ORDER))),
                  copy_gbps=copy_gbps)
        lines[nm] = res
        if len(names) > 1:
            log(json.dumps(res))
        if args.report:
            with open(args.report, "a", encoding="utf-8") as f:
                f.write(json.dumps(res) + "\n")
    head = lines.get(DEFAULT) or lines[names[-1]]
    print(json.dumps(head), flush=True)


if __name__ == "__main__":
    main()
