// C ABI of the device operations: argument validation (before anything is
// enqueued), fp32 step constants, and the launch sequence of each call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cmath>
#include <cstdio>
#include <string>
#include <vector>

#include "zero_internal.h"

namespace zk {

static thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

}  // namespace zk

using zk::fail;

extern "C" const char* zero_last_error(void) { return zk::g_err.c_str(); }
extern "C" const char* zero_version(void) { return "zero_shard 0.1 (gfx950)"; }

namespace {

int dtype_bytes(zero_dtype_t t) {
  switch (t) {
    case ZERO_F32: return 4;
    case ZERO_BF16: return 2;
    case ZERO_F16: return 2;
  }
  return 0;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  uintptr_t lo, hi;
  const char* name;
};

bool overlaps(const Range& x, const Range& y) { return x.lo < y.hi && y.lo < x.hi; }

Range rng(const void* p, int64_t bytes, const char* name) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)bytes, name};
}

// Gradient-buffer checks shared by the fused step and the reduce pass.  count
// buffers of `len` elements each (the shard, or the full padded vector); the
// stride matters only when there are several.  Shard buffers start on 16-byte
// boundaries; full buffers need element alignment (each vector's alignment is
// checked in the kernel).
int check_grad(const char* fn, const void* grad, int64_t ld, int32_t count, zero_dtype_t gt, bool full,
               int64_t len) {
  const int gb = dtype_bytes(gt);
  if (gb == 0) return fail(ZERO_EINVAL, std::string(fn) + ": unsupported gradient dtype");
  if (!grad) return fail(ZERO_EINVAL, std::string(fn) + ": grad is NULL");
  if (count < 1) return fail(ZERO_EINVAL, std::string(fn) + ": grad_count must be >= 0 (0 = N)");
  if (count > 1 && ld < len)
    return fail(ZERO_EINVAL, std::string(fn) + ": grad_ld is smaller than one gradient buffer");
  if (count > 1 && (ld * gb) % 16 != 0)
    return fail(ZERO_EALIGN, std::string(fn) + ": grad_ld must be a multiple of 16 bytes");
  if (!aligned(grad, full ? (uintptr_t)gb : 16))
    return fail(ZERO_EALIGN, std::string(fn) + (full ? ": grad is not element aligned"
                                                     : ": slices must start on 16-byte boundaries"));
  return ZERO_OK;
}

// bytes spanned by the gradient buffers
int64_t grad_span(int64_t ld, int32_t count, int64_t len, int gb) {
  return ((int64_t)(count - 1) * ld + len) * gb;
}

// The plan's attached device piece table if it serves `rank` on the current
// device, else NULL.
const zk::Seg* piece_table_for(const zero_plan_t* plan, int32_t rank) {
  if (plan->table == nullptr || plan->table_rank != rank) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->table_device) return nullptr;
  return static_cast<const zk::Seg*>(plan->table);
}

// device address of ctl->k (address arithmetic only; ctl is device memory)
const float* ctl_consts(const zero_step_ctl_t* ctl) {
  return reinterpret_cast<const float*>(reinterpret_cast<const char*>(ctl) + offsetof(zero_step_ctl_t, k));
}

void slice_consts(int32_t n, int32_t* n_pow2, float* nf, float* recip) {
  *n_pow2 = (n & (n - 1)) == 0 ? 1 : 0;
  *nf = (float)n;
  *recip = (float)(1.0 / (double)n);
}

}  // namespace

extern "C" int zero_reduce_shard(const zero_plan_t* plan, int32_t rank, const void* grad, int64_t grad_ld,
                                 int32_t grad_count, int32_t grad_layout, zero_dtype_t grad_dtype,
                                 float inv_scale, float* g_out, void* ws, int32_t want_sumsq,
                                 zero_step_ctl_t* ctl, void* stream) {
  if (!plan) return fail(ZERO_EINVAL, "zero_reduce_shard: plan is NULL");
  if (!ws) return fail(ZERO_EINVAL, "zero_reduce_shard: workspace is NULL");
  if (!aligned(ws, 16)) return fail(ZERO_EALIGN, "zero_reduce_shard: workspace must be 16-byte aligned");
  const int64_t S = plan->shard;
  if (grad_count < 0) return fail(ZERO_EINVAL, "zero_reduce_shard: grad_count must be >= 0 (0 = N)");
  if (grad_layout != ZERO_GRAD_SHARD && grad_layout != ZERO_GRAD_FULL)
    return fail(ZERO_EINVAL, "zero_reduce_shard: unknown gradient layout");
  const bool full = grad_layout == ZERO_GRAD_FULL;
  if (full && (rank < 0 || rank >= plan->world)) return fail(ZERO_EINVAL, "zero_reduce_shard: rank out of range");
  const int32_t count = grad_count == 0 ? plan->world : grad_count;
  const int64_t glen = full ? plan->padded : S;
  int rc = check_grad("zero_reduce_shard", grad, grad_ld, count, grad_dtype, full, glen);
  if (rc) return rc;
  if (g_out && !aligned(g_out, 16)) return fail(ZERO_EALIGN, "zero_reduce_shard: g_out must be 16-byte aligned");
  if (!ctl && !std::isfinite(inv_scale)) return fail(ZERO_EINVAL, "zero_reduce_shard: inv_scale is not finite");
  if (ctl && !aligned(ctl, 8)) return fail(ZERO_EALIGN, "zero_reduce_shard: ctl must be 8-byte aligned");
  const Range gr = rng(grad, grad_span(grad_ld, count, glen, dtype_bytes(grad_dtype)), "grad");
  if (g_out && overlaps(gr, rng(g_out, S * 4, "g_out")))
    return fail(ZERO_EINVAL, "zero_reduce_shard: g_out overlaps the slices");
  if (ctl) {
    const Range cr = rng(ctl, sizeof(zero_step_ctl_t), "ctl");
    if (overlaps(cr, gr) || (g_out && overlaps(cr, rng(g_out, S * 4, "g_out"))) ||
        overlaps(cr, rng(ws, (int64_t)zk::ws_bytes(S), "ws")))
      return fail(ZERO_EINVAL, "zero_reduce_shard: ctl overlaps the gradient, g_out or the workspace");
  }
  zk::ReduceLaunch a{};
  a.grad = grad;
  a.ld_bytes = count > 1 ? grad_ld * dtype_bytes(grad_dtype) : 0;
  a.grad_full = full ? 1 : 0;
  a.n = count;
  slice_consts(plan->world, &a.n_pow2, &a.nf, &a.recip_n);
  a.inv_scale = ctl ? 1.0f : inv_scale;
  a.kdev = ctl ? ctl_consts(ctl) : nullptr;
  a.g_out = g_out;
  a.ws_flags = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + zk::ws_flags_offset(S));
  a.ws_sums = reinterpret_cast<double*>(static_cast<char*>(ws) + zk::ws_sums_offset());
  a.want_sumsq = want_sumsq ? 1 : 0;
  a.S = S;
  a.nvec = (S + zk::kVec - 1) / zk::kVec;
  const int64_t nblocks = zk::reduce_blocks(S);
  if (!full) {
    a.blk0 = 0;
    if (ctl && (rc = zk::launch_ctl_begin(ctl, 0, 0.0, 0.0, 0.0, nullptr, stream))) return rc;
    return zk::launch_reduce(a, grad_dtype, nblocks, stream);
  }
  // Full-gradient layout: with the device piece table one launch over every
  // tile; else launches over runs of whole tiles whose elements lie in at most
  // kMaxSeg pieces (each workgroup still writes its own partial).
  const auto& B = plan->buckets;
  const int nb = (int)B.size();
  if (const zk::Seg* table = piece_table_for(plan, rank)) {
    a.blk0 = 0;
    a.nseg = nb;
    a.table = table;
    if (ctl && (rc = zk::launch_ctl_begin(ctl, 0, 0.0, 0.0, 0.0, nullptr, stream))) return rc;
    return zk::launch_reduce(a, grad_dtype, nblocks, stream);
  }
  auto first_piece = [&](int64_t j) {  // first piece whose local end is past element j
    int lo = 0, hi = nb - 1;
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (B[mid].local_off + B[mid].shard > j) hi = mid; else lo = mid + 1;
    }
    return lo;
  };
  auto last_piece = [&](int64_t tt) {  // last piece holding an element of the tiles before tt
    return first_piece(std::min<int64_t>(tt * zk::kTile, S) - 1);
  };
  // plan every launch first, so a layout that cannot be covered is refused
  // before anything is enqueued
  struct Run { int64_t t0, t1; int f, l; };
  std::vector<Run> runs;
  for (int64_t t = 0; t < nblocks;) {
    const int f = first_piece(t * zk::kTile);
    if (last_piece(t + 1) - f + 1 > zk::kMaxSeg)
      return fail(ZERO_EINVAL, "zero_reduce_shard: more than " + std::to_string(zk::kMaxSeg) +
                                   " pieces inside one 2048-element tile of the full-gradient layout");
    // the largest t1 whose tiles [t, t1) span at most kMaxSeg pieces
    int64_t lo = t + 1, hi = nblocks;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo + 1) / 2;
      if (last_piece(mid) - f + 1 <= zk::kMaxSeg) lo = mid; else hi = mid - 1;
    }
    runs.push_back(Run{t, lo, f, last_piece(lo)});
    t = lo;
  }
  if (ctl && (rc = zk::launch_ctl_begin(ctl, 0, 0.0, 0.0, 0.0, nullptr, stream))) return rc;
  for (const Run& r : runs) {
    a.blk0 = r.t0;
    a.nseg = r.l - r.f + 1;
    for (int q = 0; q < a.nseg; ++q) {
      const auto& P = B[r.f + q];
      a.seg[q].end = P.local_off + P.shard;
      a.seg[q].delta = (P.base + (int64_t)rank * P.shard) - P.local_off;
    }
    rc = zk::launch_reduce(a, grad_dtype, r.t1 - r.t0, stream);
    if (rc) return rc;
  }
  return ZERO_OK;
}

extern "C" int zero_shard_norm(const zero_plan_t* plan, void* ws, double other_ranks_sumsq,
                               double max_norm, uint32_t* overflow_out, double* sumsq_out,
                               float* clip_coef_out, void* stream) {
  if (!plan) return fail(ZERO_EINVAL, "zero_shard_norm: plan is NULL");
  if (!ws) return fail(ZERO_EINVAL, "zero_shard_norm: workspace is NULL");
  if (!aligned(ws, 16)) return fail(ZERO_EALIGN, "zero_shard_norm: workspace must be 16-byte aligned");
  if (!std::isfinite(other_ranks_sumsq) || other_ranks_sumsq < 0)
    return fail(ZERO_EINVAL, "zero_shard_norm: other_ranks_sumsq must be finite and >= 0");
  if (!std::isfinite(max_norm)) return fail(ZERO_EINVAL, "zero_shard_norm: max_norm is not finite");
  if ((sumsq_out && !aligned(sumsq_out, 8)) || (clip_coef_out && !aligned(clip_coef_out, 4)) ||
      (overflow_out && !aligned(overflow_out, 4)))
    return fail(ZERO_EALIGN, "zero_shard_norm: misaligned output");
  zk::NormLaunch a{};
  char* wsb = static_cast<char*>(ws);
  a.ws_flags = reinterpret_cast<const uint32_t*>(wsb + zk::ws_flags_offset(plan->shard));
  a.ws_sums = reinterpret_cast<const double*>(wsb + zk::ws_sums_offset());
  a.l2_sums = reinterpret_cast<double*>(wsb + zk::ws_l2_sums_offset());
  a.l2_flags = reinterpret_cast<uint32_t*>(wsb + zk::ws_l2_flags_offset());
  a.nblocks = zk::reduce_blocks(plan->shard);
  a.chunk = (a.nblocks + zk::kNormGroups - 1) / zk::kNormGroups;
  a.other_sumsq = other_ranks_sumsq;
  a.max_norm = max_norm;
  a.overflow_out = overflow_out;
  a.sumsq_out = sumsq_out;
  a.clip_out = clip_coef_out;
  return zk::launch_norm(a, stream);
}

extern "C" int zero_adam_step(const zero_plan_t* plan, const zero_adam_args_t* args, void* stream) {
  if (!plan) return fail(ZERO_EINVAL, "zero_adam_step: plan is NULL");
  if (!args) return fail(ZERO_EINVAL, "zero_adam_step: args is NULL");
  const zero_adam_args_t& A = *args;
  const int64_t S = plan->shard;
  const int32_t N = plan->world;
  if (A.rank < 0 || A.rank >= N) return fail(ZERO_EINVAL, "zero_adam_step: rank out of range");
  const bool stash = A.g_stash != nullptr;
  zero_step_ctl_t* const ctl = A.ctl;  // step control in device memory, or NULL
  if (ctl && !aligned(ctl, 8)) return fail(ZERO_EALIGN, "zero_adam_step: ctl must be 8-byte aligned");
  if (ctl && !stash && !A.overflow_out)
    return fail(ZERO_EINVAL, "zero_adam_step: a fused step with ctl needs overflow_out");
  const int32_t count = A.grad_count == 0 ? N : A.grad_count;
  const bool full = A.grad_layout == ZERO_GRAD_FULL;
  const int64_t glen = full ? plan->padded : S;  // elements of one gradient buffer
  const int pb = dtype_bytes(A.param_dtype);
  if (pb == 0) return fail(ZERO_EINVAL, "zero_adam_step: unsupported parameter dtype");

  // state pointers and alignment
  const bool tiled = A.state_layout == ZERO_STATE_TILED;
  if (A.state_layout != ZERO_STATE_SEPARATE && !tiled)
    return fail(ZERO_EINVAL, "zero_adam_step: unknown state layout");
  const float* ins[3] = {A.master_in, A.m_in, A.v_in};
  float* outs[3] = {A.master_out, A.m_out, A.v_out};
  const int n_arrays = tiled ? 1 : 3;
  for (int i = 0; i < 3; ++i) {
    if (i >= n_arrays) {
      if (ins[i] || outs[i])
        return fail(ZERO_EINVAL, "zero_adam_step: the tiled state layout takes master_in/master_out only");
      continue;
    }
    if (!ins[i] || !outs[i]) return fail(ZERO_EINVAL, "zero_adam_step: state pointer is NULL");
    if (!aligned(ins[i], 16) || !aligned(outs[i], 16))
      return fail(ZERO_EALIGN, "zero_adam_step: state arrays must be 16-byte aligned");
  }
  if (!A.gather) return fail(ZERO_EINVAL, "zero_adam_step: gather is NULL");
  if (!aligned(A.gather, pb)) return fail(ZERO_EALIGN, "zero_adam_step: gather is not element aligned");
  if (stash) {
    if (!aligned(A.g_stash, 16)) return fail(ZERO_EALIGN, "zero_adam_step: g_stash must be 16-byte aligned");
    if (A.clip_coef && !aligned(A.clip_coef, 4)) return fail(ZERO_EALIGN, "zero_adam_step: clip_coef misaligned");
  } else {
    if (A.grad_layout != ZERO_GRAD_SHARD && A.grad_layout != ZERO_GRAD_FULL)
      return fail(ZERO_EINVAL, "zero_adam_step: unknown gradient layout");
    if (A.grad_count < 0) return fail(ZERO_EINVAL, "zero_adam_step: grad_count must be >= 0 (0 = N)");
    const int rc = check_grad("zero_adam_step", A.grad, A.grad_ld, count, A.grad_dtype, full, glen);
    if (rc) return rc;
    if (!ctl && !std::isfinite(A.inv_scale)) return fail(ZERO_EINVAL, "zero_adam_step: inv_scale is not finite");
  }
  if ((A.skip_in && !aligned(A.skip_in, 4)) || (A.overflow_out && !aligned(A.overflow_out, 4)))
    return fail(ZERO_EALIGN, "zero_adam_step: flag pointers must be 4-byte aligned");

  // hyper-parameters (with ctl, lr and step live in device memory)
  const double lr = ctl ? 0.0 : A.lr;
  const int64_t step = ctl ? 1 : A.step;
  if (!(std::isfinite(lr) && lr >= 0) || !(A.beta1 >= 0 && A.beta1 < 1) ||
      !(A.beta2 >= 0 && A.beta2 < 1) || !(std::isfinite(A.eps) && A.eps >= 0) ||
      !std::isfinite(A.weight_decay))
    return fail(ZERO_EINVAL, "zero_adam_step: bad hyper-parameters");
  if (step < 1) return fail(ZERO_EINVAL, "zero_adam_step: step counts from 1");

  // aliasing: outputs never overlap each other or the gather buffer; in the
  // fused step with an overflow flag they must not overlap any input either
  // (the inputs are what a skipped step keeps)
  const int64_t sb = (tiled ? zero_state_numel(plan, ZERO_STATE_TILED) : S) * 4;
  static const char* in_names[3] = {"master_in", "m_in", "v_in"};
  static const char* out_names[3] = {"master_out", "m_out", "v_out"};
  std::vector<Range> out_r, in_r;
  for (int i = 0; i < n_arrays; ++i) out_r.push_back(rng(outs[i], sb, out_names[i]));
  out_r.push_back(rng(A.gather, plan->padded * pb, "gather"));
  for (size_t i = 0; i < out_r.size(); ++i)
    for (size_t j = i + 1; j < out_r.size(); ++j)
      if (overlaps(out_r[i], out_r[j]))
        return fail(ZERO_EINVAL, std::string("zero_adam_step: ") + out_r[i].name + " overlaps " + out_r[j].name);
  for (int i = 0; i < n_arrays; ++i) in_r.push_back(rng(ins[i], sb, in_names[i]));
  if (stash)
    in_r.push_back(rng(A.g_stash, S * 4, "g_stash"));
  else
    in_r.push_back(rng(A.grad, grad_span(A.grad_ld, count, glen, dtype_bytes(A.grad_dtype)), "grad"));
  const bool strict = !stash && A.overflow_out != nullptr;
  for (size_t i = 0; i < in_r.size(); ++i) {
    for (size_t j = 0; j < out_r.size(); ++j) {
      if (!overlaps(in_r[i], out_r[j])) continue;
      const bool same = ((int)i < n_arrays && j == i && in_r[i].lo == out_r[j].lo);  // exact in-place update
      if (strict || !same)
        return fail(ZERO_EINVAL, std::string("zero_adam_step: ") + in_r[i].name + " overlaps " + out_r[j].name +
                                     (strict ? " (a fused step with an overflow flag needs separate output state)" : ""));
    }
  }
  if (ctl) {
    const Range cr = rng(ctl, sizeof(zero_step_ctl_t), "ctl");
    for (const std::vector<Range>* v : {&in_r, &out_r})
      for (const Range& r : *v)
        if (overlaps(cr, r)) return fail(ZERO_EINVAL, std::string("zero_adam_step: ctl overlaps ") + r.name);
  }

  // fp32 constants, rounded once from float64
  zk::StepLaunch L{};
  L.c.b1 = (float)A.beta1;
  L.c.b2 = (float)A.beta2;
  L.c.omb1 = (float)(1.0 - A.beta1);
  L.c.omb2 = (float)(1.0 - A.beta2);
  L.c.bc1 = (float)(1.0 - std::pow(A.beta1, (double)step));
  L.c.bc2 = (float)(1.0 - std::pow(A.beta2, (double)step));
  L.c.lr = (float)lr;
  L.c.eps = (float)A.eps;
  L.c.dec = (float)(1.0 - lr * A.weight_decay);
  if (!(L.c.bc1 > 0.0f) || !(L.c.bc2 > 0.0f))
    return fail(ZERO_EINVAL, "zero_adam_step: bias correction rounds to 0 in fp32");

  L.grad = A.grad;
  L.ld_bytes = (stash || count == 1) ? 0 : A.grad_ld * dtype_bytes(A.grad_dtype);
  L.grad_full = (!stash && full) ? 1 : 0;
  L.n = stash ? N : count;
  slice_consts(N, &L.n_pow2, &L.nf, &L.recip_n);
  L.inv_scale = ctl ? 1.0f : A.inv_scale;
  L.kdev = ctl ? ctl_consts(ctl) : nullptr;
  L.restore = (ctl && !stash) ? 1 : 0;
  L.ctl = nullptr;  // set on the launch that advances the step control
  L.beta1 = A.beta1;
  L.beta2 = A.beta2;
  L.wd = A.weight_decay;
  L.g_stash = A.g_stash;
  L.clip = A.clip_coef;
  if (tiled) {
    L.p_in = A.master_in;
    L.m_in = A.master_in + zk::kStateTile;
    L.v_in = A.master_in + 2 * zk::kStateTile;
    L.p_out = A.master_out;
    L.m_out = A.master_out + zk::kStateTile;
    L.v_out = A.master_out + 2 * zk::kStateTile;
    L.st_shift = zk::kStateTileShift;
    L.st_mask = zk::kStateTile - 1;
    L.st_stride = 3 * zk::kStateTile;
  } else {
    L.p_in = A.master_in;
    L.m_in = A.m_in;
    L.v_in = A.v_in;
    L.p_out = A.master_out;
    L.m_out = A.m_out;
    L.v_out = A.v_out;
    L.st_shift = 62;  // j >> 62 == 0 for every shard index: plain j
    L.st_mask = -1;
    L.st_stride = 0;
  }
  L.gather = static_cast<char*>(A.gather);
  L.skip_in = A.skip_in;
  L.overflow = stash ? nullptr : A.overflow_out;
  L.S = S;

  // Split the rank's pieces into launches of at most kMaxSeg pieces.  A launch
  // covers whole 8-element vectors; the vector holding a piece boundary goes to
  // the launch that lists both pieces.
  const int nb = (int)plan->buckets.size();
  struct Group { int64_t v_lo, v_hi; int first, count; };
  std::vector<Group> groups;
  const int64_t nvec = (S + zk::kVec - 1) / zk::kVec;
  const zk::Seg* table = piece_table_for(plan, A.rank);
  if (table) {  // every piece in one launch, read from the device table
    groups.push_back(Group{0, nvec, 0, nb});
  } else {
    int first = 0;
    int64_t v_lo = 0;
    while (first < nb) {
      const int last = first + zk::kMaxSeg < nb ? first + zk::kMaxSeg : nb;  // exclusive
      int64_t v_hi = nvec;
      if (last < nb) v_hi = plan->buckets[last].local_off / zk::kVec;
      groups.push_back(Group{v_lo, v_hi, first, last - first});
      // the next launch starts with the piece holding element 8*v_hi
      if (last < nb) {
        int nf = last;
        while (nf > first && plan->buckets[nf].local_off > v_hi * zk::kVec) --nf;
        first = nf;
      } else {
        first = nb;
      }
      v_lo = v_hi;
    }
  }

  // one launch's vector range and pieces: kernel arguments, or the table
  auto set_group = [&](const Group& g) {
    L.v_lo = g.v_lo;
    L.v_hi = g.v_hi;
    L.nseg = g.count;
    L.table = table;
    if (table) return;
    for (int s = 0; s < g.count; ++s) {
      const auto& B = plan->buckets[g.first + s];
      L.seg[s].end = B.local_off + B.shard;
      L.seg[s].delta = (B.base + (int64_t)A.rank * B.shard) - B.local_off;
    }
  };

  int rc = ZERO_OK;
  if (!stash && S <= zk::kSmallShard && groups.size() == 1) {
    // one workgroup decides the skip before writing: a single launch
    set_group(groups[0]);
    // the workgroup derives the step control's constants and advances it itself
    L.kdev = nullptr;
    L.ctl = ctl;
    rc = zk::record_event(A.ev_begin, stream);
    if (rc) return rc;
    rc = zk::launch_small_step(L, A.grad_dtype, A.param_dtype, stream);
    if (rc) return rc;
    return zk::record_event(A.ev_end, stream);
  }
  if (ctl)  // the constants, and the flag reset of a fused step, in one launch
    rc = zk::launch_ctl_begin(ctl, 1, A.beta1, A.beta2, A.weight_decay, strict ? A.overflow_out : nullptr, stream);
  else if (strict)
    rc = zk::launch_fill_u32(A.overflow_out, 0u, stream);
  if (rc) return rc;
  rc = zk::record_event(A.ev_begin, stream);
  if (rc) return rc;
  for (const Group& g : groups) {
    set_group(g);
    rc = zk::launch_step(L, A.grad_dtype, A.param_dtype, stash, stream);
    if (rc) return rc;
  }
  rc = zk::record_event(A.ev_end, stream);
  if (rc) return rc;
  if (strict) {
    for (const Group& g : groups) {
      L.ctl = (&g == &groups.back()) ? ctl : nullptr;  // the last restore pass advances the step control
      set_group(g);
      rc = zk::launch_recast(L, A.param_dtype, A.overflow_out, stream);
      if (rc) return rc;
    }
  }
  // the fused step advanced the step control in its restore pass
  if (ctl && stash) return zk::launch_ctl_end(ctl, A.skip_in, stream);
  return ZERO_OK;
}

extern "C" int64_t zero_plan_piece_table_bytes(const zero_plan_t* plan) {
  return plan ? (int64_t)plan->buckets.size() * (int64_t)sizeof(zk::Seg) : 0;
}

extern "C" int zero_plan_attach_piece_table(zero_plan_t* plan, int32_t rank, void* table, int64_t bytes) {
  if (!plan) return fail(ZERO_EINVAL, "zero_plan_attach_piece_table: plan is NULL");
  if (!table) {  // detach
    plan->table = nullptr;
    plan->table_rank = -1;
    plan->table_device = -1;
    return ZERO_OK;
  }
  if (rank < 0 || rank >= plan->world) return fail(ZERO_EINVAL, "zero_plan_attach_piece_table: rank out of range");
  const int64_t need = zero_plan_piece_table_bytes(plan);
  if (bytes < need)
    return fail(ZERO_EINVAL, "zero_plan_attach_piece_table: the table needs " + std::to_string(need) + " bytes");
  if (!aligned(table, 16)) return fail(ZERO_EALIGN, "zero_plan_attach_piece_table: table must be 16-byte aligned");
  std::vector<zk::Seg> host(plan->buckets.size());
  for (size_t b = 0; b < host.size(); ++b) {
    const auto& B = plan->buckets[b];
    host[b].end = B.local_off + B.shard;
    host[b].delta = (B.base + (int64_t)rank * B.shard) - B.local_off;
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipMemcpy(table, host.data(), (size_t)need, hipMemcpyHostToDevice);
  if (e != hipSuccess)
    return fail(ZERO_EHIP, std::string("zero_plan_attach_piece_table: ") + hipGetErrorString(e));
  plan->table = table;
  plan->table_rank = rank;
  plan->table_device = dev;
  return ZERO_OK;
}

extern "C" int zero_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (!dst || !src) return fail(ZERO_EINVAL, "zero_stream_copy: NULL pointer");
  if (bytes < 0 || bytes % 16 != 0) return fail(ZERO_EINVAL, "zero_stream_copy: bytes must be a multiple of 16");
  if (!aligned(dst, 16) || !aligned(src, 16)) return fail(ZERO_EALIGN, "zero_stream_copy: pointers must be 16-byte aligned");
  if (overlaps(rng(dst, bytes, "dst"), rng(src, bytes, "src")))
    return fail(ZERO_EINVAL, "zero_stream_copy: source and destination overlap");
  return zk::launch_stream_copy(dst, src, bytes, stream);
}
