"""One rank's sharded mixed-precision Adam/AdamW step (ZeRO-DP P_os / P_os+g) on MI355X.

The computation runs in libzero_shard.so (hand-written HIP kernels for gfx950
behind a C ABI, include/zero_shard.h); this package is its thin Python binding
plus a small optimizer object over torch device tensors.  The library is loaded
on first use (any planner or device call), which fails loudly if it has not been
built; nothing here falls back to another implementation.
"""
from ._abi import (DTYPE_BYTES, DTYPE_CODES, EXPORTS, ZERO_BF16, ZERO_EALIGN, ZERO_EHIP,
                   ZERO_EINVAL, ZERO_EIO, ZERO_ENOMEM, ZERO_F16, ZERO_F32, ZERO_GRAD_FULL,
                   ZERO_GRAD_SHARD, ZERO_OK, ZERO_STATE_SEPARATE, ZERO_STATE_TILE, ZERO_STATE_TILED,
                   Plan, Scaler, ZeroError, adam_args, lib, zero_adam_args_t, zero_adam_step,
                   zero_checkpoint_load, zero_checkpoint_save, zero_ckpt_meta_t, zero_last_error,
                   zero_plan_hash, zero_reduce_shard, zero_scaler_t, zero_shard_norm, zero_step_ctl_t,
                   zero_stream_copy, zero_version, ZERO_NOALLOC_SCRATCH_BYTES, zero_noalloc_max_shard,
                   zero_reduce_norm_noalloc)

__all__ = [
    "DTYPE_BYTES", "DTYPE_CODES", "EXPORTS", "ZERO_BF16", "ZERO_EALIGN", "ZERO_EHIP", "ZERO_EINVAL",
    "ZERO_EIO", "ZERO_ENOMEM", "ZERO_F16", "ZERO_F32", "ZERO_GRAD_FULL", "ZERO_GRAD_SHARD", "ZERO_OK",
    "ZERO_STATE_SEPARATE", "ZERO_STATE_TILE", "ZERO_STATE_TILED", "Plan", "Scaler", "ZeroError",
    "adam_args", "lib", "zero_adam_args_t", "zero_adam_step", "zero_checkpoint_load",
    "zero_checkpoint_save", "zero_ckpt_meta_t", "zero_last_error", "zero_plan_hash",
    "zero_reduce_shard", "zero_scaler_t", "zero_shard_norm", "zero_step_ctl_t", "zero_stream_copy",
    "zero_version", "ZERO_NOALLOC_SCRATCH_BYTES", "zero_noalloc_max_shard", "zero_reduce_norm_noalloc",
]
