"""CPU oracle for one rank's sharded mixed-precision Adam/AdamW step (ZeRO P_os / P_os+g).

TEST INFRASTRUCTURE.  This package is a plain, slow, obviously-correct CPU
statement of what the step computes, used to check the HIP implementation.  Only
the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code with the HIP path: no
kernels, headers, helpers, tables or constant generators; neither imports the
other.  Inputs come from the seeded generators in ``workloads``.

Sources (cited by page title and section):
  * "ZeRO 与 FSDP：切分优化器状态、梯度与参数" (handbook chapter), section
    "从零实现 ZeRO 的 Adam" (zero_adam.py, zero_check.py) and section "三个级别";
  * "论文专题讲解：ZeRO：大模型训练的零冗余状态优化", sections "显存账",
    "ZeRO-DP 三阶段", "Table 1: ZeRO-DP Memory", "Table 2: Maximum Model Size",
    "ZeRO-R" (C_B constant-size buffers);
  * the ZeRO stages explainer (guanweilu.cn/article/1460), sections
    "先算一笔账" and "Stage 1/2/3";
  * "PaddlePaddle ZeRO优化：降低分布式内存占用", section "混合精度才是最佳拍档"
    (GradScaler scale / step / update) and the opening (AdamW).

Floating point: the pages fix fp32 master weights and fp32 Adam moments
(mixed-precision Adam accounting), so the step is computed in numpy float32 with
exactly one IEEE rounding per operation and no fused multiply-add.  The global
gradient norm, on which the pages are silent, is accumulated in float64.

Parity pins: every function here is pinned by tests under tests/test_oracle_*.py
to values the pages print, closed forms, library routines or brute force.  The
readings that no page fixes (bucket rule, summation order, weight-decay form,
clip form, loss-scale policy) are conventions of this oracle and are marked
"parity unpinned" where they are defined.
"""

from . import casts, plan, step  # noqa: F401
