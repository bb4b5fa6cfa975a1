// Internal declarations shared by the planner, the C ABI and the HIP launchers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "zero_shard.h"

struct zero_plan {
  int32_t world = 0;
  int64_t psi = 0;            // sum of tensor sizes
  int64_t shard = 0;          // S = sum_b S_b
  int64_t padded = 0;         // sum_b P_b
  std::vector<int64_t> numel;
  struct Bucket {
    int32_t first, count;
    int64_t numel, shard, padded, base, local_off;
  };
  std::vector<Bucket> buckets;
  std::vector<int32_t> tensor_bucket;
  std::vector<int64_t> tensor_offset;
  // optional device piece table (zero_plan_attach_piece_table)
  const void* table = nullptr;
  int32_t table_rank = -1;
  int32_t table_device = -1;
};

namespace zk {

// error state (thread-local message)
int fail(int code, const std::string& msg);

constexpr int kThreads = 256;   // threads per workgroup (4 wave64s)
constexpr int kVec = 8;         // elements per thread per tile
constexpr int kTile = kThreads * kVec;
constexpr int kMaxSeg = 192;    // gather pieces one launch of the update kernel can address
constexpr int kScanSeg = 24;    // up to this many pieces, a lane scans all of them
constexpr int kNormThreads = 256;     // threads of the norm finalize workgroups
constexpr int kNormGroups = 256;      // first-level workgroups of the norm finalize
constexpr int kStateTileShift = 11;   // tiled state: 2048 elements of master, m, v per tile
constexpr int64_t kStateTile = int64_t(1) << kStateTileShift;
constexpr int kStreamBlocksPerCU = 2; // resident workgroups per CU of the streaming kernels
constexpr int kStashBlocksPerCU = 5;  // ... of the update kernel that reads the fp32 stash
constexpr int kFewStreamBlocksPerCU = 3;  // ... of kernels that sum one or two gradient buffers
constexpr int kNarrowBlocksPerCU = 3;     // ... of the four-element fused form
constexpr int kNarrowWideBlocksPerCU = 2; // ... of that form with more than 64 raw gradient bytes per lane
constexpr int kNarrow64Threads = 1024;    // threads per workgroup of that form with 64 16-bit buffers (1 per CU)
constexpr int kReduceFewBlocksPerCU = 3;  // ... of the reduction pass with at most 128 raw gradient bytes per lane
// Slice loads a lane keeps in flight in the windowed sums, rather than one load
// per slice all issued at once.  Measured with the builds alternating on the
// same buffers; a window one or two slices smaller or larger was slower.
constexpr int kStepWindow = 6;       // eight-element fused update (8 bf16 slices: +2% on Llama-7B and GPT-2 shards)
constexpr int kReduceWindow = 4;     // eight-element reduction pass (16 bf16 slices: +0.5%)
constexpr int kNarrowWindow = 8;     // four-element form with 16 or 32 16-bit buffers (+2.8%, +0.7%)
// ... with 64 16-bit buffers, at 16 waves per CU: against 8 waves with a
// window of 8 (itself +1.3% over all at once), +1.2% and +3.6% on two parts; a
// window of 4 +0.6% and +2.5%, 5 or 6 -4 to -5% (48 wave-wide slice loads in
// flight per CU, against 64 before and 80 at a window of 5)
constexpr int kNarrow64Window = 3;
constexpr int kNarrowWindow32 = 4;   // four-element form with 8, 16 or 32 fp32 buffers (N = 8: +2.5%)
constexpr size_t kStaticLdsRoom = 1024;  // LDS left for a streaming kernel's own __shared__ arrays
// Elements per launch of the streaming kernels: a larger shard is processed in
// consecutive launches of this size on the caller's stream.  Measured with both
// builds alternating on the same buffers: a single launch over the Llama-7B
// shard (842M elements, 411K workgroups) streams 5% slower than the same
// work as 13 launches of 2^26 elements; the clipped Llama-3 step gains 1-2%;
// 2^23-2^24 per launch lose more to each launch's ramp and tail than they gain.
constexpr int64_t kLaunchElems = int64_t(1) << 26;
// The four-element form with 64 16-bit buffers (154 bytes per element) streams
// best in shorter launches: on the 7.5B N = 64 shard 2^23 elements per launch
// (14 launches) are 2.5% faster than 2^26, 2^22 and 2^24 about 2%, 2^21 0.5%
// slower; the eight-slice steps lose 1-8% at 2^23-2^25.
constexpr int64_t kLaunchElems64 = int64_t(1) << 23;
constexpr int kSmallThreads = 1024;   // one-workgroup path for small shards ...
constexpr int64_t kSmallShard = (int64_t)kSmallThreads * kVec;  // ... of at most this many elements

// A rank piece as seen by one launch: local elements [.., end) map to gather
// element (local index + delta).
struct Seg {
  int64_t end;
  int64_t delta;
};

struct AdamK {  // fp32 constants of one step
  float b1, b2, omb1, omb2, bc1, bc2, lr, eps, dec;
};

struct StepLaunch {
  // gradient source
  const void* grad;
  int64_t ld_bytes;       // slice stride in bytes
  int32_t grad_full;      // slices are full flat gradients read at the gather offsets
  int32_t n;              // slices summed
  int32_t n_pow2;         // the divisor N is a power of two: acc * (1/N) is the IEEE quotient
  float nf;               // float(N), N = the world size
  float recip_n;          // 1/N (exact when n_pow2)
  float inv_scale;
  const float* g_stash;   // stash mode when non-null
  const float* clip;      // stash mode multiplier (may be null)
  // state
  const float* p_in;
  const float* m_in;
  const float* v_in;
  float* p_out;
  float* m_out;
  float* v_out;
  int32_t st_shift;       // state addressing: (j >> st_shift) * st_stride + (j & st_mask)
  int64_t st_mask;
  int64_t st_stride;
  char* gather;
  AdamK c;
  const float* kdev;      // non-null: bc1, bc2, lr, dec, inv_scale from device memory instead
  const uint32_t* skip_in;
  uint32_t* overflow;
  int32_t restore;        // a step that is not applied copies the input state to the output
  // step control advanced by this launch (the one-workgroup step, which also
  // derives its constants from it, or the last restore pass), else null
  zero_step_ctl_t* ctl;
  double beta1, beta2, wd;  // float64 hyper-parameters for constants derived on the device
  // local vector range of this launch and its pieces
  int64_t S;              // shard length (elements at or past S do not exist)
  int64_t v_lo, v_hi;     // vectors [v_lo, v_hi) of kVec elements
  int32_t nseg;
  const Seg* table;       // non-null: the pieces are read from this device table, seg[] is unused
  Seg seg[kMaxSeg];
};

// passed by value as the kernel argument: within the 4 KiB kernel-argument limit
static_assert(sizeof(StepLaunch) <= 3584, "StepLaunch must fit the kernel-argument segment");

struct ReduceLaunch {
  const void* grad;
  int64_t ld_bytes;
  int32_t grad_full;      // slices are full flat gradients read at the gather offsets
  int32_t n;              // slices summed (the divisor is the world size, in nf)
  int32_t n_pow2;
  float nf, recip_n, inv_scale;
  const float* kdev;      // non-null: inv_scale from device memory (kdev[4]) instead
  float* g_out;
  uint32_t* ws_flags;     // [gridDim.x]
  double* ws_sums;        // [gridDim.x]
  int32_t want_sumsq;
  int64_t S;
  int64_t nvec;           // ceil(S / kVec)
  int64_t blk0;           // first tile (workgroup) of this launch
  int32_t nseg;           // pieces of this launch's tiles (full-gradient layout)
  const Seg* table;       // non-null: the pieces are read from this device table
  Seg seg[kMaxSeg];
};

static_assert(sizeof(ReduceLaunch) <= 3584, "ReduceLaunch must fit the kernel-argument segment");

struct NormLaunch {
  const uint32_t* ws_flags;
  const double* ws_sums;
  double* l2_sums;         // [kNormGroups]
  uint32_t* l2_flags;      // [kNormGroups]
  int64_t nblocks;
  int64_t chunk;           // partials per first-level workgroup
  double other_sumsq;
  double max_norm;
  uint32_t* overflow_out;
  double* sumsq_out;
  float* clip_out;
};

// gradient-preparation grid: one 8-element vector per thread, one workgroup per
// kTile elements; the workspace holds one fp64 partial and one overflow word per
// workgroup
// workgroup, then kNormGroups first-level sums and overflow words of the finalize
inline int64_t reduce_blocks(int64_t S) { return (S + kTile - 1) / kTile; }
inline size_t ws_l2_sums_offset() { return 0; }
inline size_t ws_l2_flags_offset() { return (size_t)kNormGroups * sizeof(double); }
inline size_t ws_sums_offset() { return ws_l2_flags_offset() + (size_t)kNormGroups * sizeof(uint32_t); }
inline size_t ws_flags_offset(int64_t S) { return ws_sums_offset() + (size_t)reduce_blocks(S) * sizeof(double); }
inline size_t ws_bytes(int64_t S) {
  return (ws_flags_offset(S) + (size_t)reduce_blocks(S) * sizeof(uint32_t) + 255) / 256 * 256;
}

// launchers (kernels.hip); return ZERO_OK or ZERO_EHIP
int launch_fill_u32(uint32_t* p, uint32_t value, void* stream);
int launch_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);
int launch_step(const StepLaunch& a, zero_dtype_t gt, zero_dtype_t pt, bool stash, void* stream);
int launch_recast(const StepLaunch& a, zero_dtype_t pt, const uint32_t* cond, void* stream);
int launch_small_step(const StepLaunch& a, zero_dtype_t gt, zero_dtype_t pt, void* stream);
int launch_reduce(const ReduceLaunch& a, zero_dtype_t gt, int64_t nblocks, void* stream);
int launch_norm(const NormLaunch& a, void* stream);
// step control in device memory: the constants of the step about to run
// (all of them, or with adam == 0 only inv_scale; reset_flag, if given, is
// zeroed too), and the advance after it
int launch_ctl_begin(zero_step_ctl_t* ctl, int adam, double beta1, double beta2, double weight_decay,
                     uint32_t* reset_flag, void* stream);
int launch_ctl_end(zero_step_ctl_t* ctl, const uint32_t* flag, void* stream);
int record_event(void* ev, void* stream);

}  // namespace zk
