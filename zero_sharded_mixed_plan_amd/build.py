"""Build libzero_shard.so (HIP kernels for gfx950 + C++ planner + C ABI) in-tree.

    python -m zero_sharded_mixed_plan_amd.build

The library is loaded into processes that already hold torch's HIP runtime
(torch supplies the device memory and streams), so the code object version is
pinned to one every ROCm 7 runtime loads.

Floating-point flags are part of the contract of the library: no contraction
into fused multiply-add, IEEE-correct fp32 division and square root, denormals
kept.  Packed-fp32 instructions are disabled for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libzero_shard.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("kernels.hip", "abi.cpp", "plan.cpp", "runtime.cpp", "noalloc.hip")]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    # per-kernel registers, scratch and occupancy as compiler remarks (parsed below)
    "-Rpass-analysis=kernel-resource-usage",
]
RESOURCES = os.path.join(PKG, "kernel_resources.txt")


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


# A plain C program that drives the library through include/zero_shard.h with
# memory from the HIP runtime API alone (no Python, no torch); the GPU tests
# run it.  Built with the host C compiler; the HIP headers need the platform
# macro that hipcc would define.
C_DRIVER_SRC = os.path.join(ROOT, "tests", "c", "abi_step.c")
C_DRIVER = os.path.join(ROOT, "tests", "c", "abi_step")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_driver(verbose: bool = False) -> str:
    """Compile the C driver against the built library; returns its path."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           "-o", C_DRIVER + ".tmp", C_DRIVER_SRC, "-L", PKG, "-lzero_shard",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../zero_sharded_mixed_plan_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C driver build failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(C_DRIVER + ".tmp", C_DRIVER)
    return C_DRIVER


def kernel_resources(remarks: str) -> dict:
    """{kernel: {field: value}} from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass-analysis", 1)[0].strip()
        key, _, val = body.partition(":")
        if key == "Function Name":
            cur = out.setdefault(val.strip(), {})
        elif cur is not None:
            cur[key.strip()] = val.strip()
    return out


def build(verbose: bool = False) -> str:
    """Compile the library; returns its path.  Always recompiles.  A kernel
    that spills to scratch memory fails the build: every kernel here streams
    from registers, and a spill has cost the step several percent."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    res = kernel_resources(r.stderr)
    with open(RESOURCES, "w") as f:
        for name in sorted(res):
            f.write(name + " " + " ".join(f"{k.replace(' ', '_')}={v}" for k, v in res[name].items()) + "\n")
    spills = [n for n, d in res.items()
              if d.get("ScratchSize [bytes/lane]", "0") != "0" or d.get("VGPRs Spill", "0") != "0"
              or d.get("SGPRs Spill", "0") != "0"]
    if not res:
        raise RuntimeError("hipcc printed no kernel resource usage")
    if spills:
        os.remove(tmp)
        raise RuntimeError("kernels spill to scratch memory: " + ", ".join(sorted(spills)))
    os.replace(tmp, LIB)
    build_c_driver(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
