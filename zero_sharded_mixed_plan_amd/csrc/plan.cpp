// Host planner: tensor list -> padded flat buckets -> per-rank pieces, and the
// ZeRO-DP model-state byte accounting.
//
// Layout of zero_adam.py ("ZeRO 与 FSDP：切分优化器状态、梯度与参数", section
// "从零实现 ZeRO 的 Adam"): flatten in list order, zero-pad to ceil(numel/N)*N,
// rank r owns the r-th of N equal contiguous pieces.  With a positive bucket cap
// the same layout is applied bucket by bucket (constant-size buffers, C_B of
// "论文专题讲解：ZeRO…", section "ZeRO-R"); tensors are packed greedily in order
// and a bucket that already holds elements is closed when the next non-empty
// tensor would take it past the cap.
#include <cstring>
#include <new>

#include "zero_internal.h"

using zk::fail;

extern "C" int zero_plan(const int64_t* numel, int32_t n_tensors, int32_t world,
                         int64_t bucket_cap, zero_plan_t** out) {
  if (!out) return fail(ZERO_EINVAL, "zero_plan: out is NULL");
  *out = nullptr;
  if (!numel || n_tensors <= 0) return fail(ZERO_EINVAL, "zero_plan: need at least one tensor");
  if (world < 1) return fail(ZERO_EINVAL, "zero_plan: world must be >= 1");
  int64_t psi = 0;
  for (int32_t i = 0; i < n_tensors; ++i) {
    if (numel[i] < 0) return fail(ZERO_EINVAL, "zero_plan: negative tensor size");
    if (numel[i] > (int64_t(1) << 52) || psi > (int64_t(1) << 52))
      return fail(ZERO_EINVAL, "zero_plan: sizes too large");
    psi += numel[i];
  }
  if (psi == 0) return fail(ZERO_EINVAL, "zero_plan: all tensors are empty");

  zero_plan_t* p = new (std::nothrow) zero_plan_t;
  if (!p) return fail(ZERO_ENOMEM, "zero_plan: out of host memory");
  try {
    p->world = world;
    p->psi = psi;
    p->numel.assign(numel, numel + n_tensors);
    p->tensor_bucket.resize(n_tensors);
    p->tensor_offset.resize(n_tensors);

    // greedy packing in list order
    int32_t first = 0;
    int64_t size = 0;
    auto close = [&](int32_t end) {
      zero_plan_t::Bucket b;
      b.first = first;
      b.count = end - first;
      b.numel = size;
      b.shard = (size + world - 1) / world;
      b.padded = b.shard * world;
      b.base = p->padded;
      b.local_off = p->shard;
      int64_t off = b.base;
      for (int32_t i = first; i < end; ++i) {
        p->tensor_bucket[i] = (int32_t)p->buckets.size();
        p->tensor_offset[i] = off;
        off += numel[i];
      }
      p->buckets.push_back(b);
      p->padded += b.padded;
      p->shard += b.shard;
      first = end;
      size = 0;
    };
    for (int32_t i = 0; i < n_tensors; ++i) {
      const int64_t n = numel[i];
      if (bucket_cap > 0 && n > 0 && size > 0 && size + n > bucket_cap) close(i);
      size += n;
    }
    close(n_tensors);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(ZERO_ENOMEM, "zero_plan: out of host memory");
  }
  *out = p;
  return ZERO_OK;
}

// Per-parameter dim-0 layout ("ZeRO 与 FSDP…", section "ZeRO-3 与 FSDP": fully_shard
// splits each parameter on its first dimension).  One bucket per non-empty
// parameter with its rows padded to a multiple of N; empty parameters ride
// along in a neighbouring bucket without adding to it.
extern "C" int zero_plan_dim0(const int64_t* rows, const int64_t* row_numel, int32_t n_tensors,
                              int32_t world, zero_plan_t** out) {
  if (!out) return fail(ZERO_EINVAL, "zero_plan_dim0: out is NULL");
  *out = nullptr;
  if (!rows || !row_numel || n_tensors <= 0) return fail(ZERO_EINVAL, "zero_plan_dim0: need at least one tensor");
  if (world < 1) return fail(ZERO_EINVAL, "zero_plan_dim0: world must be >= 1");
  const int64_t kMax = int64_t(1) << 52;
  int64_t psi = 0;
  for (int32_t i = 0; i < n_tensors; ++i) {
    if (rows[i] < 0 || row_numel[i] < 0) return fail(ZERO_EINVAL, "zero_plan_dim0: negative size");
    if (rows[i] > kMax || row_numel[i] > kMax || (row_numel[i] > 0 && rows[i] > kMax / row_numel[i]))
      return fail(ZERO_EINVAL, "zero_plan_dim0: sizes too large");
    psi += rows[i] * row_numel[i];
    if (psi > kMax) return fail(ZERO_EINVAL, "zero_plan_dim0: sizes too large");
  }
  if (psi == 0) return fail(ZERO_EINVAL, "zero_plan_dim0: all tensors are empty");

  zero_plan_t* p = new (std::nothrow) zero_plan_t;
  if (!p) return fail(ZERO_ENOMEM, "zero_plan_dim0: out of host memory");
  try {
    p->world = world;
    p->psi = psi;
    p->numel.resize(n_tensors);
    for (int32_t i = 0; i < n_tensors; ++i) p->numel[i] = rows[i] * row_numel[i];
    p->tensor_bucket.resize(n_tensors);
    p->tensor_offset.resize(n_tensors);
    // groups [first, end) each holding exactly one non-empty parameter
    int32_t first = 0;
    while (first < n_tensors) {
      int32_t main = first;
      while (p->numel[main] == 0) ++main;  // a non-empty one exists at or after `first`
      int32_t end = main + 1;
      while (end < n_tensors && p->numel[end] == 0) ++end;
      zero_plan_t::Bucket b;
      b.first = first;
      b.count = end - first;
      b.numel = p->numel[main];
      b.shard = (rows[main] + world - 1) / world * row_numel[main];
      b.padded = b.shard * world;
      b.base = p->padded;
      b.local_off = p->shard;
      for (int32_t i = first; i < end; ++i) {
        p->tensor_bucket[i] = (int32_t)p->buckets.size();
        p->tensor_offset[i] = b.base + (i > main ? b.numel : 0);
      }
      p->buckets.push_back(b);
      p->padded += b.padded;
      p->shard += b.shard;
      first = end;
    }
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(ZERO_ENOMEM, "zero_plan_dim0: out of host memory");
  }
  *out = p;
  return ZERO_OK;
}

extern "C" void zero_plan_free(zero_plan_t* plan) { delete plan; }

extern "C" int64_t zero_plan_shard_numel(const zero_plan_t* p) { return p ? p->shard : -1; }
extern "C" int64_t zero_plan_total_numel(const zero_plan_t* p) { return p ? p->psi : -1; }
extern "C" int64_t zero_plan_padded_numel(const zero_plan_t* p) { return p ? p->padded : -1; }
extern "C" int32_t zero_plan_world(const zero_plan_t* p) { return p ? p->world : -1; }
extern "C" int32_t zero_plan_num_buckets(const zero_plan_t* p) {
  return p ? (int32_t)p->buckets.size() : -1;
}
extern "C" int32_t zero_plan_num_tensors(const zero_plan_t* p) {
  return p ? (int32_t)p->numel.size() : -1;
}

extern "C" int zero_plan_bucket(const zero_plan_t* p, int32_t b, int64_t* base, int64_t* numel,
                                int64_t* padded, int64_t* shard, int32_t* first_tensor,
                                int32_t* n_tensors) {
  if (!p) return fail(ZERO_EINVAL, "zero_plan_bucket: plan is NULL");
  if (b < 0 || b >= (int32_t)p->buckets.size())
    return fail(ZERO_EINVAL, "zero_plan_bucket: bucket index out of range");
  const auto& B = p->buckets[b];
  if (base) *base = B.base;
  if (numel) *numel = B.numel;
  if (padded) *padded = B.padded;
  if (shard) *shard = B.shard;
  if (first_tensor) *first_tensor = B.first;
  if (n_tensors) *n_tensors = B.count;
  return ZERO_OK;
}

extern "C" int zero_plan_tensor(const zero_plan_t* p, int32_t i, int32_t* bucket,
                                int64_t* offset) {
  if (!p) return fail(ZERO_EINVAL, "zero_plan_tensor: plan is NULL");
  if (i < 0 || i >= (int32_t)p->numel.size())
    return fail(ZERO_EINVAL, "zero_plan_tensor: tensor index out of range");
  if (bucket) *bucket = p->tensor_bucket[i];
  if (offset) *offset = p->tensor_offset[i];
  return ZERO_OK;
}

extern "C" int zero_plan_rank_segment(const zero_plan_t* p, int32_t rank, int32_t b,
                                      int64_t* gather_off, int64_t* local_off, int64_t* valid) {
  if (!p) return fail(ZERO_EINVAL, "zero_plan_rank_segment: plan is NULL");
  if (rank < 0 || rank >= p->world)
    return fail(ZERO_EINVAL, "zero_plan_rank_segment: rank out of range");
  if (b < 0 || b >= (int32_t)p->buckets.size())
    return fail(ZERO_EINVAL, "zero_plan_rank_segment: bucket index out of range");
  const auto& B = p->buckets[b];
  const int64_t start = (int64_t)rank * B.shard;
  int64_t v = B.numel - start;
  v = v < 0 ? 0 : (v > B.shard ? B.shard : v);
  if (gather_off) *gather_off = B.base + start;
  if (local_off) *local_off = B.local_off;
  if (valid) *valid = v;
  return ZERO_OK;
}

extern "C" int zero_plan_bytes(const zero_plan_t* p, int32_t stage, double* formula_bytes,
                               int64_t* padded_bytes) {
  if (!p) return fail(ZERO_EINVAL, "zero_plan_bytes: plan is NULL");
  const double psi = (double)p->psi, n = (double)p->world;
  const int64_t S = p->shard, NS = p->padded;
  double f;
  int64_t pb;
  switch (stage) {
    case 0: f = 16.0 * psi; pb = 16 * NS; break;
    case 1: f = 4.0 * psi + 12.0 * psi / n; pb = 4 * NS + 12 * S; break;
    case 2: f = 2.0 * psi + 14.0 * psi / n; pb = 2 * NS + 14 * S; break;
    case 3: f = 16.0 * psi / n; pb = 16 * S; break;
    default: return fail(ZERO_EINVAL, "zero_plan_bytes: stage must be 0, 1, 2 or 3");
  }
  if (formula_bytes) *formula_bytes = f;
  if (padded_bytes) *padded_bytes = pb;
  return ZERO_OK;
}

extern "C" int64_t zero_state_numel(const zero_plan_t* p, int32_t layout) {
  if (!p) return -1;
  if (layout == ZERO_STATE_SEPARATE) return p->shard;
  if (layout == ZERO_STATE_TILED) return (p->shard + zk::kStateTile - 1) / zk::kStateTile * 3 * zk::kStateTile;
  return -1;
}

extern "C" size_t zero_workspace_bytes(const zero_plan_t* p) { return p ? zk::ws_bytes(p->shard) : 0; }
