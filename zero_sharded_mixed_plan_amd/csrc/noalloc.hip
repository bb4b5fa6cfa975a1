// The clipped step's first pass and norm finalize for callers that cannot
// allocate device memory: the workspace of zero_reduce_shard / zero_shard_norm
// (one float64 partial and one overflow word per 2048 shard elements, plus the
// finalize's first-level sums) lives in a fixed array in the library's device
// memory instead of a caller-allocated buffer.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <string>

#include "zero_internal.h"

namespace {

// The workspace array.  Every GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// the device array: its device address comes from hipGetSymbolAddress, once
// per device, and only that address is ever passed to a kernel.
static_assert(ZERO_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[ZERO_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of the current device's array (looked up on the first
// call on that device, with that device current).
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return zk::fail(ZERO_EHIP, std::string("zero_reduce_norm_noalloc: hipGetDevice: ") +
                                                      hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return zk::fail(ZERO_EINVAL, "zero_reduce_norm_noalloc: device index " + std::to_string(dev) +
                                     " beyond the library's table of " + std::to_string(kMaxDevices));
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return zk::fail(ZERO_EHIP, std::string("zero_reduce_norm_noalloc: hipGetSymbolAddress: ") +
                                     hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return ZERO_OK;
}

}  // namespace

extern "C" int64_t zero_noalloc_max_shard(void) {
  // the largest S whose workspace fits the array (ws_bytes grows with S)
  int64_t lo = 0, hi = int64_t(1) << 40;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (zk::ws_bytes(mid) <= (size_t)ZERO_NOALLOC_SCRATCH_BYTES) lo = mid; else hi = mid - 1;
  }
  return lo;
}

extern "C" int zero_reduce_norm_noalloc(const zero_plan_t* plan, int32_t rank, const void* grad, int64_t grad_ld,
                                        int32_t grad_count, int32_t grad_layout, zero_dtype_t grad_dtype,
                                        float inv_scale, float* g_out, double other_ranks_sumsq, double max_norm,
                                        uint32_t* overflow_out, double* sumsq_out, float* clip_coef_out,
                                        zero_step_ctl_t* ctl, void* stream) {
  if (!plan) return zk::fail(ZERO_EINVAL, "zero_reduce_norm_noalloc: plan is NULL");
  const size_t need = zk::ws_bytes(plan->shard);
  if (need > (size_t)ZERO_NOALLOC_SCRATCH_BYTES)
    return zk::fail(ZERO_EINVAL, "zero_reduce_norm_noalloc: a shard of " + std::to_string(plan->shard) +
                                     " elements needs " + std::to_string(need) + " bytes of workspace; the "
                                     "library's fixed array holds " +
                                     std::to_string((long long)ZERO_NOALLOC_SCRATCH_BYTES) + " (at most " +
                                     std::to_string(zero_noalloc_max_shard()) +
                                     " elements): use zero_reduce_shard with a caller workspace");
  // the same argument checks as the two calls it stands for, before anything
  // is enqueued (the finalize's own checks are repeated here so that a bad
  // finalize argument does not leave the first pass enqueued)
  if (!std::isfinite(other_ranks_sumsq) || other_ranks_sumsq < 0)
    return zk::fail(ZERO_EINVAL, "zero_reduce_norm_noalloc: other_ranks_sumsq must be finite and >= 0");
  if (!std::isfinite(max_norm)) return zk::fail(ZERO_EINVAL, "zero_reduce_norm_noalloc: max_norm is not finite");
  if ((sumsq_out && reinterpret_cast<uintptr_t>(sumsq_out) % 8) ||
      (clip_coef_out && reinterpret_cast<uintptr_t>(clip_coef_out) % 4) ||
      (overflow_out && reinterpret_cast<uintptr_t>(overflow_out) % 4))
    return zk::fail(ZERO_EALIGN, "zero_reduce_norm_noalloc: misaligned output");
  void* ws = nullptr;
  int rc = scratch_ptr(&ws);
  if (rc) return rc;
  rc = zero_reduce_shard(plan, rank, grad, grad_ld, grad_count, grad_layout, grad_dtype, inv_scale, g_out, ws, 1,
                         ctl, stream);
  if (rc) return rc;
  return zero_shard_norm(plan, ws, other_ranks_sumsq, max_norm, overflow_out, sumsq_out, clip_coef_out, stream);
}
