"""The build's kernel-resource check (the compiler's resource-usage remarks are
parsed per kernel, and a kernel that spills to scratch fails the build), the
benchmark's profile hash, and its refusal of more than one GPU."""
from zero_sharded_mixed_plan_amd import build as B

REMARKS = """\
k.hip:10:1: remark: Function Name: _Z1av [-Rpass-analysis=kernel-resource-usage]
k.hip:10:1: remark:     VGPRs: 30 [-Rpass-analysis=kernel-resource-usage]
k.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:10:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
   10 | __global__ void a() {}
k.hip:20:1: remark: Function Name: _Z1bv [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark:     ScratchSize [bytes/lane]: 20 [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark:     VGPRs Spill: 5 [-Rpass-analysis=kernel-resource-usage]
k.hip:30:1: warning: something else
"""


def test_resource_remarks_parsed_per_kernel():
    r = B.kernel_resources(REMARKS)
    assert set(r) == {"_Z1av", "_Z1bv"}
    assert r["_Z1av"] == {"VGPRs": "30", "ScratchSize [bytes/lane]": "0", "VGPRs Spill": "0"}
    assert r["_Z1bv"]["ScratchSize [bytes/lane]"] == "20" and r["_Z1bv"]["VGPRs Spill"] == "5"


def test_the_resource_flag_is_part_of_the_build():
    assert "-Rpass-analysis=kernel-resource-usage" in B.FLAGS


def test_profile_hash_ignores_comments_only():
    """The source hash the benchmark compares with the committed profiles
    covers code, not comments: a comment edit keeps the profiles current, a
    code edit does not."""
    import bench
    code = 'int f(int x) {  // twice\n  /* the "sum" */ return x + x; // it\'s\n}\nconst char* s = "a // b";\n'
    base = bench._code_only(code)
    assert base == 'int f(int x) {\n   return x + x;\n}\nconst char* s = "a // b";'
    assert bench._code_only(code.replace("twice", "double it")) == base
    assert bench._code_only(code.replace("x + x", "x * 2")) != base


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one rank on one GPU: --gpus above 1 exits with a
    message before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
