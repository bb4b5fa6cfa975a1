// HIP kernels for gfx950 (CDNA4): one rank's sharded mixed-precision AdamW step.
//
// The step is a pure streaming update (well under one flop per byte), so it is
// bound by HBM bandwidth, not by the matrix cores: every kernel here is written
// for wide, coalesced global traffic.  In the eight-element forms each thread
// owns kVec = 8 consecutive elements, so every 16-bit gradient slice is read with
// one 16-byte load (two for fp32) and every fp32 state array with two; a wave64
// touches 1 KiB contiguous per 16-bit slice.  The narrow forms give a thread 4
// elements and half the bytes in flight, which streams faster for most buffer
// counts.  All loads of a tile are issued before the arithmetic so enough bytes
// are in flight to cover HBM latency.
//
// What is computed follows zero_adam.py ("ZeRO 与 FSDP：切分优化器状态、梯度与参数",
// section "从零实现 ZeRO 的 Adam"): SUM of the ranks' gradient pieces, / N, Adam on
// fp32 master/m/v, then the new parameters go to the all-gather buffer; plus the
// loss-scale unscale and overflow skip of mixed precision ("PaddlePaddle
// ZeRO优化…", section "混合精度才是最佳拍档") and decoupled weight decay (AdamW).
// Arithmetic is IEEE fp32, one rounding per operation: the build disables
// contraction into FMA, keeps denormals and uses correctly rounded div/sqrt.
#include <hip/hip_runtime.h>

#include <cstdio>

#include "zero_internal.h"

namespace zk {

using u32 = uint32_t;

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------

struct TF32 { static constexpr int bytes = 4; };
struct TBF16 { static constexpr int bytes = 2; };
struct TF16 { static constexpr int bytes = 2; };

// Cache hints.  Gradient slices are read exactly once per step and the gather
// slot is written once and only read by the all-gather, so both move with the
// non-temporal bit (measured on the GPT-2 1.5B shard: +4% over plain loads and
// stores; non-temporal hints on the fp32 state made it slower).
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void st_stream16(void* p, uint4 x) {
  const v4u y = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(y, reinterpret_cast<v4u*>(p));
}
__device__ __forceinline__ void st_stream8(void* p, uint2 x) {
  const v2u y = {x.x, x.y};
  __builtin_nontemporal_store(y, reinterpret_cast<v2u*>(p));
}
__device__ __forceinline__ void st_stream4(void* p, uint32_t x) {
  __builtin_nontemporal_store(x, reinterpret_cast<uint32_t*>(p));
}

// 8 elements of a slice, raw: one uint4 for 16-bit types, two for fp32.
template <class T>
struct Raw { uint4 q[T::bytes / 2]; };

template <class T>
__device__ __forceinline__ Raw<T> ld_raw(const char* p) {
  Raw<T> r;
#pragma unroll
  for (int i = 0; i < T::bytes / 2; ++i) r.q[i] = ld_stream16(p + 16 * i);
  return r;
}

// An empty asm that reads and writes the registers of r: code that uses r
// cannot be placed ahead of it.
template <class T>
__device__ __forceinline__ void pin_raw(Raw<T>& r) {
#pragma unroll
  for (int i = 0; i < T::bytes / 2; ++i) asm volatile("" : "+v"(r.q[i].x), "+v"(r.q[i].y), "+v"(r.q[i].z), "+v"(r.q[i].w));
}

__device__ __forceinline__ float bf16_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_bits(u32 h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <class T> __device__ __forceinline__ void widen8(const Raw<T>& r, float o[8]);

template <> __device__ __forceinline__ void widen8<TBF16>(const Raw<TBF16>& r, float o[8]) {
  const u32 w[4] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { o[2 * i] = bf16_lo(w[i]); o[2 * i + 1] = bf16_hi(w[i]); }
}
template <> __device__ __forceinline__ void widen8<TF16>(const Raw<TF16>& r, float o[8]) {
  const u32 w[4] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { o[2 * i] = f16_bits(w[i] & 0xffffu); o[2 * i + 1] = f16_bits(w[i] >> 16); }
}
template <> __device__ __forceinline__ void widen8<TF32>(const Raw<TF32>& r, float o[8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    o[4 * i + 0] = __uint_as_float(r.q[i].x);
    o[4 * i + 1] = __uint_as_float(r.q[i].y);
    o[4 * i + 2] = __uint_as_float(r.q[i].z);
    o[4 * i + 3] = __uint_as_float(r.q[i].w);
  }
}

// one element of a slice, widened
template <class T> __device__ __forceinline__ float ld_one(const char* p);
template <> __device__ __forceinline__ float ld_one<TF32>(const char* p) { return *reinterpret_cast<const float*>(p); }
template <> __device__ __forceinline__ float ld_one<TBF16>(const char* p) {
  return __uint_as_float((u32)(*reinterpret_cast<const uint16_t*>(p)) << 16);
}
template <> __device__ __forceinline__ float ld_one<TF16>(const char* p) {
  return f16_bits(*reinterpret_cast<const uint16_t*>(p));
}

// fp32 -> parameter storage, round to nearest even (hardware conversions)
__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  const uint16_t x = __builtin_bit_cast(uint16_t, (__bf16)a);
  const uint16_t y = __builtin_bit_cast(uint16_t, (__bf16)b);
  return (u32)x | ((u32)y << 16);
}
__device__ __forceinline__ u32 pack_f16(float a, float b) {
  const uint16_t x = __builtin_bit_cast(uint16_t, (_Float16)a);
  const uint16_t y = __builtin_bit_cast(uint16_t, (_Float16)b);
  return (u32)x | ((u32)y << 16);
}

// Store 8 parameters at dst, choosing the widest naturally aligned store the
// address allows (a rank's gather slot may sit at any element offset).
template <class PT> __device__ __forceinline__ void store_params8(char* dst, const float p[8]);

template <class PT>
__device__ __forceinline__ void store_words(char* dst, const u32* w) {
  constexpr int NW = PT::bytes * 2;  // 4 words for 16-bit, 8 for fp32
  const uintptr_t a = reinterpret_cast<uintptr_t>(dst);
  if ((a & 15) == 0) {
#pragma unroll
    for (int i = 0; i < NW; i += 4) st_stream16(dst + 4 * i, make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]));
  } else if ((a & 7) == 0) {
#pragma unroll
    for (int i = 0; i < NW; i += 2) st_stream8(dst + 4 * i, make_uint2(w[i], w[i + 1]));
  } else if ((a & 3) == 0) {
#pragma unroll
    for (int i = 0; i < NW; ++i) st_stream4(dst + 4 * i, w[i]);
  } else {  // 2-byte aligned 16-bit elements
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      reinterpret_cast<uint16_t*>(dst)[2 * i] = (uint16_t)(w[i] & 0xffffu);
      reinterpret_cast<uint16_t*>(dst)[2 * i + 1] = (uint16_t)(w[i] >> 16);
    }
  }
}
template <> __device__ __forceinline__ void store_params8<TBF16>(char* dst, const float p[8]) {
  const u32 w[4] = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
  store_words<TBF16>(dst, w);
}
template <> __device__ __forceinline__ void store_params8<TF16>(char* dst, const float p[8]) {
  const u32 w[4] = {pack_f16(p[0], p[1]), pack_f16(p[2], p[3]), pack_f16(p[4], p[5]), pack_f16(p[6], p[7])};
  store_words<TF16>(dst, w);
}
template <> __device__ __forceinline__ void store_params8<TF32>(char* dst, const float p[8]) {
  u32 w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = __float_as_uint(p[i]);
  store_words<TF32>(dst, w);
}

template <class PT> __device__ __forceinline__ void store_param1(char* dst, float p);
template <> __device__ __forceinline__ void store_param1<TF32>(char* dst, float p) { *reinterpret_cast<float*>(dst) = p; }
template <> __device__ __forceinline__ void store_param1<TBF16>(char* dst, float p) {
  *reinterpret_cast<uint16_t*>(dst) = __builtin_bit_cast(uint16_t, (__bf16)p);
}
template <> __device__ __forceinline__ void store_param1<TF16>(char* dst, float p) {
  *reinterpret_cast<uint16_t*>(dst) = __builtin_bit_cast(uint16_t, (_Float16)p);
}

// ---------------------------------------------------------------------------
// fp32 state
// ---------------------------------------------------------------------------

__device__ __forceinline__ void ld8(const float* p, float o[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void st8(float* p, const float o[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(o[0], o[1], o[2], o[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(o[4], o[5], o[6], o[7]);
}

// the fp32 gradient stash of the clipped path is written once here and read once
// by the update kernel; streaming it past the caches measured 2% faster
__device__ __forceinline__ void st8_stream(float* p, const float o[8]) {
  st_stream16(p, make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])));
  st_stream16(p + 4, make_uint4(__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])));
}

// ---------------------------------------------------------------------------
// the arithmetic of one element (shared by all paths of all kernels)
// ---------------------------------------------------------------------------

// g = (acc / N) * inv_scale: an IEEE quotient; for N a power of two the product
// with the exact reciprocal is the same correctly rounded value.
__device__ __forceinline__ float average_unscale(float acc, int n_pow2, float nf, float recip_n,
                                                 float inv_scale) {
  const float g = n_pow2 ? acc * recip_n : acc / nf;
  return g * inv_scale;
}

// The same for K elements, with the choice between the two quotients made once.
// Written per element, the choice became a branch per element, and the
// compiler deferred each element's sum into its own branch: every loaded slice
// then stayed in registers until the last element's turn.
template <int K>
__device__ __forceinline__ void average_unscale_k(const float (&acc)[K], float (&g)[K], int n_pow2, float nf,
                                                  float recip_n, float inv_scale) {
  if (n_pow2) {
#pragma unroll
    for (int e = 0; e < K; ++e) g[e] = (acc[e] * recip_n) * inv_scale;
  } else {
#pragma unroll
    for (int e = 0; e < K; ++e) g[e] = (acc[e] / nf) * inv_scale;
  }
}

__device__ __forceinline__ void adamw1(float& p, float& m, float& v, float g, const AdamK& c) {
  const float m2 = c.b1 * m + c.omb1 * g;
  const float v2 = c.b2 * v + c.omb2 * (g * g);
  const float m_hat = m2 / c.bc1;
  const float v_hat = v2 / c.bc2;
  const float den = __builtin_sqrtf(v_hat) + c.eps;
  const float u = (c.lr * m_hat) / den;
  p = c.dec * p - u;
  m = m2;
  v = v2;
}

// The constants that change from step to step come from the kernel arguments,
// or -- with the step control in device memory -- from what the begin kernel
// wrote there for this step: bc1, bc2, lr, dec, inv_scale.  No kernel writes
// them while a step runs, so they are read through the constant address space:
// scalar loads, which keep them off the vector memory counters.
typedef const __attribute__((address_space(4))) float* ConstF32;

__device__ __forceinline__ void step_consts(const float* kp, AdamK& c, float& inv_scale) {
  if (kp != nullptr) {
    const ConstF32 k = (ConstF32)kp;
    c.bc1 = k[0];
    c.bc2 = k[1];
    c.lr = k[2];
    c.dec = k[3];
    inv_scale = k[4];
  }
}

// Step control in device memory: the fp32 constants of step t = ctl->step + 1
// as the host computes them (float64, rounded once).  which = 0 or 1: the bias
// correction 1 - beta1^t or 1 - beta2^t (two lanes of one wave evaluate the two
// powers side by side); lr, dec = 1 - lr*wd and inv_scale = 1/scale below.
__device__ __forceinline__ float ctl_bias_correction(const zero_step_ctl_t* ctl, int which, double beta1,
                                                     double beta2) {
  const double t = (double)(ctl->step + 1);
  return (float)(1.0 - pow(which == 0 ? beta1 : beta2, t));
}

__device__ __forceinline__ float ctl_inv_scale(const zero_step_ctl_t* ctl) {
  return (float)(1.0 / (double)ctl->scaler.scale);
}

// After a step: the step count (or the skip count), then the loss scale by the
// host's zero_scaler_update rule.  One thread.
__device__ __forceinline__ void ctl_advance(zero_step_ctl_t* ctl, bool skipped) {
  if (skipped) ctl->skipped += 1;
  else ctl->step += 1;
  if (!ctl->dynamic) return;
  float scale = ctl->scaler.scale;
  int32_t tracker = ctl->scaler.growth_tracker;
  if (skipped) {
    scale = scale * ctl->scaler.backoff_factor;
    tracker = 0;
  } else {
    const int32_t n = tracker + 1;
    if (n >= ctl->scaler.growth_interval) {
      const float grown = scale * ctl->scaler.growth_factor;
      if (__builtin_isfinite(grown)) scale = grown;
      tracker = 0;
    } else {
      tracker = n;
    }
  }
  ctl->scaler.scale = scale;
  ctl->scaler.growth_tracker = tracker;
}

// Sum of N slices for 8 elements: acc = s_0, then acc += s_k in ascending k,
// for any N (the form used when no compile-time batch count fits, below).
// Every load of a batch of NB slices is issued before the first add and the
// next batch's loads go out before this batch's adds; the per-slice guards and
// the copy of the next batch into the current one make the compiler wait for
// all outstanding loads before each batch, so this form keeps at most two
// batches in flight and drains between them.
template <class T, int NB>
__device__ __forceinline__ void reduce8(const char* base, int64_t ld_bytes, int n, float acc[8]) {
  Raw<T> cur[NB], nxt[NB];
  int cnt = n < NB ? n : NB;
#pragma unroll
  for (int b = 0; b < NB; ++b)
    if (b < cnt) cur[b] = ld_raw<T>(base + (int64_t)b * ld_bytes);
  int k0 = 0;
  while (true) {
    const int k1 = k0 + cnt;
    const int rem = n - k1;
    const int cnt1 = rem < NB ? rem : NB;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (b < cnt1) nxt[b] = ld_raw<T>(base + (int64_t)(k1 + b) * ld_bytes);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < cnt) {
        float w[8];
        widen8<T>(cur[b], w);
        if (k0 == 0 && b == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = w[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = acc[e] + w[e];
        }
      }
    }
    if (cnt1 <= 0) break;
    for (int b = 0; b < NB; ++b) cur[b] = nxt[b];
    k0 = k1;
    cnt = cnt1;
  }
}

// The same sum when N is a whole number of batches, NBATCH = N / NB known at
// compile time.  The loop unrolls into straight-line code with two register
// buffers taking turns, so every load is unconditional, nothing is copied
// between buffers, and each add waits only for its own slice: while batch i is
// added, the loads of batch i + 1 are in flight.  (In the runtime-N form the
// compiler waits for every outstanding load before the first add of a batch.)
// ubase is uniform across the workgroup and toff is the lane's byte offset.
template <class T, int NB>
__device__ __forceinline__ void load_batch(Raw<T> (&r)[NB], const char* ubase, int64_t ld_bytes,
                                           uint32_t toff) {
#pragma unroll
  for (int b = 0; b < NB; ++b) r[b] = ld_raw<T>(ubase + (int64_t)b * ld_bytes + toff);
}

template <class T, int NB>
__device__ __forceinline__ void add_batch(const Raw<T> (&r)[NB], bool first, float acc[8]) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float w[8];
    widen8<T>(r[b], w);
    if (first && b == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = w[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + w[e];
    }
  }
}

// The windowed sum: slice K is added, then the load of slice K + WIN goes out,
// so a lane keeps WIN slice loads in flight rather than a whole batch; after()
// runs with the add that follows the last slice load (the caller's state loads
// go there).  A compile-time recursion, so every register array index is a
// constant, with a scheduling barrier after each step to keep that order.
template <class T, int N, int WIN, int K, class F>
__device__ __forceinline__ void window8(Raw<T> (&r)[N], const char* ubase, int64_t ld_bytes, uint32_t toff,
                                        float acc[8], F& after) {
  if constexpr (K < N) {
    pin_raw<T>(r[K]);   // slice K is widened here, not earlier
    float w[8];
    widen8<T>(r[K], w);
    if constexpr (K == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = w[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + w[e];
    }
    // the sum so far is pinned here: otherwise the compiler may defer these
    // adds past a branch in after() and so issue the whole window at once
#pragma unroll
    for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(acc[e]));
    if constexpr (K + WIN < N) r[K + WIN] = ld_raw<T>(ubase + (int64_t)(K + WIN) * ld_bytes + toff);
    if constexpr (K + WIN == N) after();
    __builtin_amdgcn_sched_barrier(0);
    window8<T, N, WIN, K + 1>(r, ubase, ld_bytes, toff, acc, after);
  }
}

// after_last_issue() runs once, right after the loads of the last batch are
// issued (the caller's state loads go there).  With a window WIN of fewer than
// N = NB * NBATCH slices, the windowed sum above instead.
template <class T, int NB, int NBATCH, int WIN, class F>
__device__ __forceinline__ void reduce8_fixed(const char* ubase, int64_t ld_bytes, uint32_t toff,
                                              float acc[8], F&& after_last_issue) {
  static_assert(NBATCH >= 1, "at least one batch");
  constexpr int N = NB * NBATCH;
  if constexpr (WIN > 0 && WIN < N) {
    Raw<T> w[N];
#pragma unroll
    for (int k = 0; k < WIN; ++k) {   // issued in slice order: the waits count loads in order
      w[k] = ld_raw<T>(ubase + (int64_t)k * ld_bytes + toff);
      __builtin_amdgcn_sched_barrier(0);
    }
    window8<T, N, WIN, 0>(w, ubase, ld_bytes, toff, acc, after_last_issue);
    return;
  }
  Raw<T> r[2][NB];
  load_batch<T, NB>(r[0], ubase, ld_bytes, toff);
  if (NBATCH == 1) after_last_issue();
#pragma unroll
  for (int i = 0; i < NBATCH; ++i) {
    if (i + 1 < NBATCH) {
      load_batch<T, NB>(r[(i + 1) & 1], ubase + (int64_t)(i + 1) * NB * ld_bytes, ld_bytes, toff);
      if (i + 2 == NBATCH) after_last_issue();
    }
    add_batch<T, NB>(r[i & 1], i == 0, acc);
    // keep later batches' loads below this batch's adds: at most two batches
    // (and the state) are in flight, which bounds the registers held
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The same windowed sum for a count n >= WIN known only at run time: a ring
// of WIN registers (slice k in r[k mod WIN]), whole groups of WIN steps in a
// loop, then one of WIN straight-line tails chosen by rho = (n - WIN) mod WIN:
// rho more steps that load, after(), and the WIN steps that only add.  The sum
// starts at -0, the identity of the addition, so every step is the same add
// and the result is that of the ordered sum bit for bit.
template <class T>
__device__ __forceinline__ void ring_add8(Raw<T>& r, float acc[8]) {
  float w[8];
  widen8<T>(r, w);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc[e] + w[e];
#pragma unroll
  for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(acc[e]));
}

template <class T, int WIN, int I, int E>
__device__ __forceinline__ void ring8_load_steps(Raw<T> (&r)[WIN], float acc[8], const char* base, int64_t ld,
                                                 int k0) {
  if constexpr (I < E) {
    ring_add8<T>(r[I], acc);
    r[I] = ld_raw<T>(base + (int64_t)(k0 + I + WIN) * ld);
    __builtin_amdgcn_sched_barrier(0);
    ring8_load_steps<T, WIN, I + 1, E>(r, acc, base, ld, k0);
  }
}

template <class T, int WIN, int R, int J>
__device__ __forceinline__ void ring8_drain(Raw<T> (&r)[WIN], float acc[8]) {
  if constexpr (J < WIN) {
    ring_add8<T>(r[(R + J) % WIN], acc);
    __builtin_amdgcn_sched_barrier(0);
    ring8_drain<T, WIN, R, J + 1>(r, acc);
  }
}

template <class T, int WIN, int R, class F>
__device__ __forceinline__ void ring8_tail_sel(int rho, Raw<T> (&r)[WIN], float acc[8], const char* base, int64_t ld,
                                               int k0, F& after) {
  if constexpr (R < WIN) {
    if (rho == R) {
      ring8_load_steps<T, WIN, 0, R>(r, acc, base, ld, k0);
      after();
      __builtin_amdgcn_sched_barrier(0);
      ring8_drain<T, WIN, R, 0>(r, acc);
      return;
    }
    ring8_tail_sel<T, WIN, R + 1>(rho, r, acc, base, ld, k0, after);
  }
}

template <class T, int WIN, class F>
__device__ __forceinline__ void reduce8_ring(const char* base, int64_t ld, int n, float acc[8], F&& after) {
  Raw<T> r[WIN];
#pragma unroll
  for (int i = 0; i < WIN; ++i) {   // issued in slice order: the waits count loads in order
    r[i] = ld_raw<T>(base + (int64_t)i * ld);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = -0.0f;
  const int groups = (n - WIN) / WIN;
  int k0 = 0;
  for (int gi = 0; gi < groups; ++gi, k0 += WIN) ring8_load_steps<T, WIN, 0, WIN>(r, acc, base, ld, k0);
  ring8_tail_sel<T, WIN, 0>((n - WIN) % WIN, r, acc, base, ld, k0, after);
}

template <class T>
__device__ __forceinline__ float reduce1(const char* base, int64_t ld_bytes, int n) {
  float acc = ld_one<T>(base);
  for (int k = 1; k < n; ++k) acc = acc + ld_one<T>(base + (int64_t)k * ld_bytes);
  return acc;
}

// Slices per load batch: 8 (one batch holds all of N <= 8), 16 for larger N;
// fp32 slices are twice as wide, so half as many.
template <class T, bool WIDE> struct Batch { static constexpr int value = WIDE ? 16 : 8; };
template <bool WIDE> struct Batch<TF32, WIDE> { static constexpr int value = WIDE ? 8 : 4; };

// Offset of local element j in the state arrays.  Separate [S] arrays: j.
// Tiled state (one buffer, tiles of master|m|v of kStateTile elements each):
// (j / tile) * 3 * tile + j % tile, with the m and v bases one and two tiles on.
// A vector of 8 never straddles a tile.
__device__ __forceinline__ int64_t state_off(const StepLaunch& a, int64_t j) {
  return (j >> a.st_shift) * a.st_stride + (j & a.st_mask);
}

// The value of x in the wave's first active lane: tells the compiler that a
// quantity computed the same way in every lane is uniform (scalar registers).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The launch's pieces that can hold a wave's local elements [lo, hi): a
// uniform binary search over the piece ends (increasing), so a lane's lookup
// below scans only the few pieces the wave touches, not all of them.
struct SegRange {
  int s0, s1;  // pieces s0 .. s1
};

// Piece i of the launch: from the kernel arguments, or from the device table
// attached to the plan (read through the constant address space: no kernel
// writes it, so the reads are scalar loads like those of the arguments).
typedef const __attribute__((address_space(4))) Seg* ConstSegs;

template <class LA>
__device__ __forceinline__ int64_t seg_end(const LA& a, int i) {
  return a.table != nullptr ? ((ConstSegs)a.table)[i].end : a.seg[i].end;
}
template <class LA>
__device__ __forceinline__ int64_t seg_delta(const LA& a, int i) {
  return a.table != nullptr ? ((ConstSegs)a.table)[i].delta : a.seg[i].delta;
}

template <class LA>
__device__ __forceinline__ SegRange wave_segs(const LA& a, int64_t lo, int64_t hi) {
  // a few pieces: scan them all (no chain of dependent argument loads)
  if (a.nseg <= kScanSeg) return SegRange{0, a.nseg - 1};
  int L = 0, R = a.nseg - 1;
  while (L < R) {  // first piece ending after lo
    const int M = (L + R) >> 1;
    if (seg_end(a, M) > lo) R = M; else L = M + 1;
  }
  const int s0 = L;
  R = a.nseg - 1;
  while (L < R) {  // first piece reaching hi
    const int M = (L + R) >> 1;
    if (seg_end(a, M) >= hi) R = M; else L = M + 1;
  }
  return SegRange{s0, L};
}

// the wave's pieces, from its first vector index (any lane's v minus its lane)
template <class LA>
__device__ __forceinline__ SegRange wave_segs_v(const LA& a, int64_t v) {
  const int64_t w0 = uniform64(v - (int64_t)(threadIdx.x & 63));
  return wave_segs(a, w0 * kVec, (w0 + 64) * kVec);
}

// gather index offset of local element j, j inside the wave's pieces
template <class LA>
__device__ __forceinline__ int64_t delta_of(const LA& a, const SegRange& r, int64_t j) {
  int64_t d = seg_delta(a, r.s0);
  for (int s = r.s0; s < r.s1; ++s)
    if (j >= seg_end(a, s)) d = seg_delta(a, s + 1);
  return d;
}

// Slice sum for 8 local elements whose gradient sits in full flat buffers at
// the gather offsets (the gradient all-reduced in full): one aligned vector
// per buffer when the 8 fall in one piece on a 16-byte boundary, else element
// by element (a piece boundary inside the 8, or a slot that is not 16-byte
// aligned).
template <class GT, int NB, class LA>
__device__ __forceinline__ void reduce8_pieces(const LA& a, const SegRange& sr, int64_t j0,
                                               float acc[8]) {
  const char* g = static_cast<const char*>(a.grad);
  const int64_t d0 = delta_of(a, sr, j0);
  const char* p = g + (j0 + d0) * GT::bytes;
  if (delta_of(a, sr, j0 + kVec - 1) == d0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
    reduce8<GT, NB>(p, a.ld_bytes, a.n, acc);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc[e] = reduce1<GT>(g + (j0 + e + delta_of(a, sr, j0 + e)) * GT::bytes, a.ld_bytes, a.n);
  }
}

// the gradient of local element j in slice 0
template <class GT, class LA>
__device__ __forceinline__ const char* grad_elem(const LA& a, const SegRange& sr, int64_t j) {
  return static_cast<const char*>(a.grad) + (j + (a.grad_full ? delta_of(a, sr, j) : 0)) * GT::bytes;
}

// ---------------------------------------------------------------------------
// the fused update kernel: N gradient buffers in
// ---------------------------------------------------------------------------

template <class GT, class PT, bool WIDE, int NBATCH>
__global__ __launch_bounds__(kThreads) void step_kernel(const StepLaunch a) {
  if (a.skip_in != nullptr && *a.skip_in != 0u) {
    // skipped by the caller: report it like an overflow so the caller keeps
    // its current state and the slots get their pre-step values
    if (a.overflow != nullptr && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(a.overflow, 1u);
    return;
  }
  const int64_t v = a.v_lo + (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (v >= a.v_hi) return;
  const int64_t j0 = v * kVec;
  // The wave's pieces are needed for the parameter stores only, except where
  // the gradient itself is read at gather offsets (the runtime-N form).  With
  // many pieces their search is a chain of dependent argument loads, so in the
  // compile-time form it runs after the slice loads have been issued, hidden
  // behind them (the FSDP2 layout of GPT-2: -2%).
  constexpr bool kLateSegs = NBATCH > 0;
  SegRange sr{0, -1};
  if constexpr (!kLateSegs) sr = wave_segs_v(a, v);
  AdamK c = a.c;
  float inv_scale = a.inv_scale;
  step_consts(a.kdev, c, inv_scale);

  float p[8], m[8], s[8], g[8];
  bool bad = false;
  if (j0 + kVec <= a.S) {
    const int64_t o0 = state_off(a, j0);
    auto load_state = [&]() {
      ld8(a.p_in + o0, p);
      ld8(a.m_in + o0, m);
      ld8(a.v_in + o0, s);
    };
    {
      constexpr int NB = Batch<GT, WIDE>::value;
      float acc[8];
      if constexpr (NBATCH > 0) {
        // the state loads go out once the last slice load has been issued, so
        // they hold no registers while the earlier slices stream in
        const char* ubase = static_cast<const char*>(a.grad) +
                            (a.v_lo + (int64_t)blockIdx.x * kThreads) * (kVec * GT::bytes);
        reduce8_fixed<GT, NB, NBATCH, kStepWindow>(ubase, a.ld_bytes, threadIdx.x * (uint32_t)(kVec * GT::bytes),
                                                   acc, [&]() {
                                        load_state();
                                        if constexpr (kLateSegs) sr = wave_segs_v(a, v);
                                      });
      } else {
        load_state();
        if (a.grad_full) reduce8_pieces<GT, NB>(a, sr, j0, acc);
        else reduce8<GT, NB>(static_cast<const char*>(a.grad) + j0 * GT::bytes, a.ld_bytes, a.n, acc);
      }
      average_unscale_k<8>(acc, g, a.n_pow2, a.nf, a.recip_n, inv_scale);
#pragma unroll
      for (int e = 0; e < 8; ++e) bad |= !__builtin_isfinite(g[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) adamw1(p[e], m[e], s[e], g[e], c);
    st8(a.p_out + o0, p);
    st8(a.m_out + o0, m);
    st8(a.v_out + o0, s);
    const int64_t d0 = delta_of(a, sr, j0);
    if (delta_of(a, sr, j0 + kVec - 1) == d0) {
      store_params8<PT>(a.gather + (j0 + d0) * PT::bytes, p);
    } else {  // the 8 elements straddle two gather pieces
#pragma unroll
      for (int e = 0; e < 8; ++e) store_param1<PT>(a.gather + (j0 + e + delta_of(a, sr, j0 + e)) * PT::bytes, p[e]);
    }
  } else {
    // the shard's ragged end: fewer than 8 elements, element by element
    if constexpr (kLateSegs) sr = wave_segs_v(a, v);
    for (int e = 0; e < 8; ++e) {
      const int64_t j = j0 + e;
      if (j >= a.S) break;
      const int64_t oj = state_off(a, j);
      float pe = a.p_in[oj], me = a.m_in[oj], ve = a.v_in[oj];
      const float acc = reduce1<GT>(grad_elem<GT>(a, sr, j), a.ld_bytes, a.n);
      const float ge = average_unscale(acc, a.n_pow2, a.nf, a.recip_n, inv_scale);
      bad |= !__builtin_isfinite(ge);
      adamw1(pe, me, ve, ge, c);
      a.p_out[oj] = pe;
      a.m_out[oj] = me;
      a.v_out[oj] = ve;
      store_param1<PT>(a.gather + (j + delta_of(a, sr, j)) * PT::bytes, pe);
    }
  }
  if (a.overflow != nullptr && bad) atomicOr(a.overflow, 1u);
}

// ---------------------------------------------------------------------------
// the update from the fp32 gradient stash (the clipped path's second pass)
// ---------------------------------------------------------------------------

// Four elements per lane: one 16-byte load each of g, master, m and v, so a
// lane holds half the bytes in flight of the eight-element form (about 5%
// faster at five resident workgroups per CU on the Llama-3 shard).  The stash
// is read once, past the caches.
__device__ __forceinline__ void ld4(const float* p, float o[4]) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
}
__device__ __forceinline__ void ld4_stream(const float* p, float o[4]) {
  const uint4 x = ld_stream16(p);
  o[0] = __uint_as_float(x.x); o[1] = __uint_as_float(x.y); o[2] = __uint_as_float(x.z); o[3] = __uint_as_float(x.w);
}
__device__ __forceinline__ void st4(float* p, const float o[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
}

// Store 4 parameters at dst with the widest naturally aligned stores.
template <class PT> __device__ __forceinline__ void store_params4(char* dst, const float p[4]);
__device__ __forceinline__ void store_words2(char* dst, u32 w0, u32 w1) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(dst);
  if ((a & 7) == 0) {
    st_stream8(dst, make_uint2(w0, w1));
  } else if ((a & 3) == 0) {
    st_stream4(dst, w0);
    st_stream4(dst + 4, w1);
  } else {  // 2-byte aligned 16-bit elements
    reinterpret_cast<uint16_t*>(dst)[0] = (uint16_t)(w0 & 0xffffu);
    reinterpret_cast<uint16_t*>(dst)[1] = (uint16_t)(w0 >> 16);
    reinterpret_cast<uint16_t*>(dst)[2] = (uint16_t)(w1 & 0xffffu);
    reinterpret_cast<uint16_t*>(dst)[3] = (uint16_t)(w1 >> 16);
  }
}
template <> __device__ __forceinline__ void store_params4<TBF16>(char* dst, const float p[4]) {
  store_words2(dst, pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]));
}
template <> __device__ __forceinline__ void store_params4<TF16>(char* dst, const float p[4]) {
  store_words2(dst, pack_f16(p[0], p[1]), pack_f16(p[2], p[3]));
}
template <> __device__ __forceinline__ void store_params4<TF32>(char* dst, const float p[4]) {
  const u32 w[4] = {__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]), __float_as_uint(p[3])};
  const uintptr_t a = reinterpret_cast<uintptr_t>(dst);
  if ((a & 15) == 0) {
    st_stream16(dst, make_uint4(w[0], w[1], w[2], w[3]));
  } else if ((a & 7) == 0) {
    st_stream8(dst, make_uint2(w[0], w[1]));
    st_stream8(dst + 8, make_uint2(w[2], w[3]));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) st_stream4(dst + 4 * i, w[i]);
  }
}

// g = g_stash * clip_coef, then AdamW and the slot write, as in the fused form.
// Lane t of the grid takes elements [4 q, 4 q + 4), q = 2 v_lo + t: the launch
// covers the same 8-element vectors [v_lo, v_hi) as the fused form.  A skipped
// step (skip_in set) writes nothing.
template <class PT>
__global__ __launch_bounds__(kThreads) void stash_step_kernel(const StepLaunch a) {
  if (a.skip_in != nullptr && *a.skip_in != 0u) return;
  const int64_t q = 2 * a.v_lo + (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t j0 = q * 4;
  if (q >= 2 * a.v_hi || j0 >= a.S) return;
  AdamK c = a.c;
  float unused = 0.0f;
  step_consts(a.kdev, c, unused);
  const float clip = a.clip != nullptr ? *a.clip : 1.0f;
  const int64_t w0 = uniform64(q - (int64_t)(threadIdx.x & 63));  // the wave's first group
  if (j0 + 4 <= a.S) {
    const int64_t o0 = state_off(a, j0);
    float p[4], m[4], v[4], g[4];
    ld4(a.p_in + o0, p);
    ld4(a.m_in + o0, m);
    ld4(a.v_in + o0, v);
    ld4_stream(a.g_stash + j0, g);
    const SegRange sr = wave_segs(a, w0 * 4, (w0 + 64) * 4);   // behind the loads
#pragma unroll
    for (int e = 0; e < 4; ++e) adamw1(p[e], m[e], v[e], g[e] * clip, c);
    st4(a.p_out + o0, p);
    st4(a.m_out + o0, m);
    st4(a.v_out + o0, v);
    const int64_t d0 = delta_of(a, sr, j0);
    if (delta_of(a, sr, j0 + 3) == d0) {
      store_params4<PT>(a.gather + (j0 + d0) * PT::bytes, p);
    } else {  // the 4 elements straddle two gather pieces
#pragma unroll
      for (int e = 0; e < 4; ++e) store_param1<PT>(a.gather + (j0 + e + delta_of(a, sr, j0 + e)) * PT::bytes, p[e]);
    }
  } else {
    // the shard's ragged end
    const SegRange sr = wave_segs(a, w0 * 4, (w0 + 64) * 4);
    for (int64_t j = j0; j < a.S; ++j) {
      const int64_t oj = state_off(a, j);
      float pe = a.p_in[oj], me = a.m_in[oj], ve = a.v_in[oj];
      adamw1(pe, me, ve, a.g_stash[j] * clip, c);
      a.p_out[oj] = pe;
      a.m_out[oj] = me;
      a.v_out[oj] = ve;
      store_param1<PT>(a.gather + (j + delta_of(a, sr, j)) * PT::bytes, pe);
    }
  }
}

// ---------------------------------------------------------------------------
// the narrow fused update: four elements per lane
// ---------------------------------------------------------------------------

// Four elements of a buffer, raw: 8 bytes for 16-bit types, 16 for fp32.
template <class T> struct Raw4 { uint2 q; };
template <> struct Raw4<TF32> { uint4 q; };

template <class T> __device__ __forceinline__ Raw4<T> ld_raw4(const char* p) {
  const v2u x = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
  return Raw4<T>{make_uint2(x.x, x.y)};
}
template <> __device__ __forceinline__ Raw4<TF32> ld_raw4<TF32>(const char* p) { return Raw4<TF32>{ld_stream16(p)}; }

template <class T> __device__ __forceinline__ void widen4(const Raw4<T>& r, float o[4]);
template <> __device__ __forceinline__ void widen4<TBF16>(const Raw4<TBF16>& r, float o[4]) {
  o[0] = bf16_lo(r.q.x); o[1] = bf16_hi(r.q.x); o[2] = bf16_lo(r.q.y); o[3] = bf16_hi(r.q.y);
}
template <> __device__ __forceinline__ void widen4<TF16>(const Raw4<TF16>& r, float o[4]) {
  o[0] = f16_bits(r.q.x & 0xffffu); o[1] = f16_bits(r.q.x >> 16);
  o[2] = f16_bits(r.q.y & 0xffffu); o[3] = f16_bits(r.q.y >> 16);
}
template <> __device__ __forceinline__ void widen4<TF32>(const Raw4<TF32>& r, float o[4]) {
  o[0] = __uint_as_float(r.q.x); o[1] = __uint_as_float(r.q.y);
  o[2] = __uint_as_float(r.q.z); o[3] = __uint_as_float(r.q.w);
}

// The windowed sum: slice K is added, then the load of slice K + WIN goes out,
// so a lane keeps WIN slice loads in flight instead of all C; the state loads
// go out with the add that follows the last slice load.  A compile-time
// recursion, so that every index into the register arrays is a constant, with
// a scheduling barrier after each step to keep that order.
template <class GT, int C, int WIN, int K>
__device__ __forceinline__ void window_sum(Raw4<GT> (&r)[C], float (&acc)[4], const char* base, int64_t ld,
                                           const StepLaunch& a, int64_t o0, float (&p)[4], float (&m)[4],
                                           float (&v)[4]) {
  if constexpr (K < C) {
    if constexpr (K == 0) {
      widen4<GT>(r[0], acc);
    } else {
      float w[4];
      widen4<GT>(r[K], w);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = acc[e] + w[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(acc[e]));   // the sum so far, pinned here
    if constexpr (K + WIN < C) r[K + WIN] = ld_raw4<GT>(base + (int64_t)(K + WIN) * ld);
    if constexpr (K + WIN == C) {
      ld4(a.p_in + o0, p);
      ld4(a.m_in + o0, m);
      ld4(a.v_in + o0, v);
    }
    __builtin_amdgcn_sched_barrier(0);
    window_sum<GT, C, WIN, K + 1>(r, acc, base, ld, a, o0, p, m, v);
  }
}

// The windowed sum for a buffer count n known only at run time, n >= WIN: a
// ring of WIN registers (slice k lives in r[k mod WIN]).  The running sum starts
// at -0, the identity of the addition, so every step is the same add.  Steps
// k < n - WIN add slice k and load slice k + WIN into the freed register; they
// run as a loop over whole groups of WIN steps (every ring index a constant)
// and a tail selected by rho = (n - WIN) mod WIN: rho more such steps, the
// state loads, then the WIN steps that only add.  No load is under a branch
// inside a group, so each add waits for its own slice only.
template <class GT>
__device__ __forceinline__ void ring_add(const Raw4<GT>& r, float (&acc)[4]) {
  float w[4];
  widen4<GT>(r, w);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = acc[e] + w[e];
#pragma unroll
  for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(acc[e]));   // the sum so far, pinned here
}

// steps I .. E - 1 of a group: add r[I], load slice k0 + I + WIN into r[I]
template <class GT, int WIN, int I, int E>
__device__ __forceinline__ void ring_load_steps(Raw4<GT> (&r)[WIN], float (&acc)[4], const char* base, int64_t ld,
                                                int k0) {
  if constexpr (I < E) {
    ring_add<GT>(r[I], acc);
    r[I] = ld_raw4<GT>(base + (int64_t)(k0 + I + WIN) * ld);
    __builtin_amdgcn_sched_barrier(0);
    ring_load_steps<GT, WIN, I + 1, E>(r, acc, base, ld, k0);
  }
}

// the last WIN steps, from ring phase R: add only
template <class GT, int WIN, int R, int J>
__device__ __forceinline__ void ring_drain(Raw4<GT> (&r)[WIN], float (&acc)[4]) {
  if constexpr (J < WIN) {
    ring_add<GT>(r[(R + J) % WIN], acc);
    __builtin_amdgcn_sched_barrier(0);
    ring_drain<GT, WIN, R, J + 1>(r, acc);
  }
}

template <class GT, int WIN, int R>
__device__ __forceinline__ void ring_tail(Raw4<GT> (&r)[WIN], float (&acc)[4], const char* base, int64_t ld, int k0,
                                          const StepLaunch& a, int64_t o0, float (&p)[4], float (&m)[4],
                                          float (&v)[4]) {
  ring_load_steps<GT, WIN, 0, R>(r, acc, base, ld, k0);
  ld4(a.p_in + o0, p);
  ld4(a.m_in + o0, m);
  ld4(a.v_in + o0, v);
  __builtin_amdgcn_sched_barrier(0);
  ring_drain<GT, WIN, R, 0>(r, acc);
}

template <class GT, int WIN, int R>
__device__ __forceinline__ void ring_tail_sel(int rho, Raw4<GT> (&r)[WIN], float (&acc)[4], const char* base,
                                              int64_t ld, int k0, const StepLaunch& a, int64_t o0, float (&p)[4],
                                              float (&m)[4], float (&v)[4]) {
  if constexpr (R < WIN) {
    if (rho == R) {
      ring_tail<GT, WIN, R>(r, acc, base, ld, k0, a, o0, p, m, v);
      return;
    }
    ring_tail_sel<GT, WIN, R + 1>(rho, r, acc, base, ld, k0, a, o0, p, m, v);
  }
}

template <class GT, int WIN>
__device__ __forceinline__ void window_sum_rt(const char* base, int64_t ld, int n, float (&acc)[4],
                                              const StepLaunch& a, int64_t o0, float (&p)[4], float (&m)[4],
                                              float (&v)[4]) {
  Raw4<GT> r[WIN];
#pragma unroll
  for (int i = 0; i < WIN; ++i) {   // issued in slice order: the waits count loads in order
    r[i] = ld_raw4<GT>(base + (int64_t)i * ld);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = -0.0f;
  const int groups = (n - WIN) / WIN;
  int k0 = 0;
  for (int gi = 0; gi < groups; ++gi, k0 += WIN) ring_load_steps<GT, WIN, 0, WIN>(r, acc, base, ld, k0);
  ring_tail_sel<GT, WIN, 0>((n - WIN) % WIN, r, acc, base, ld, k0, a, o0, p, m, v);
}

// A run-time count n < WIN: every load at once, then the adds.
template <class GT, int WIN>
__device__ __forceinline__ void small_sum_rt(const char* base, int64_t ld, int n, float (&acc)[4],
                                             const StepLaunch& a, int64_t o0, float (&p)[4], float (&m)[4],
                                             float (&v)[4]) {
  Raw4<GT> r[WIN];
#pragma unroll
  for (int i = 0; i < WIN; ++i)
    if (i < n) r[i] = ld_raw4<GT>(base + (int64_t)i * ld);
  ld4(a.p_in + o0, p);
  ld4(a.m_in + o0, m);
  ld4(a.v_in + o0, v);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = -0.0f;
#pragma unroll
  for (int i = 0; i < WIN; ++i)
    if (i < n) ring_add<GT>(r[i], acc);
}

// The fused update over C [S] gradient buffers, four elements per lane as in
// the stash-mode update: one load per buffer and one each of master, m and v,
// then the same sum (ascending k), arithmetic and stores as the eight-element
// form.  A lane holds half the bytes in flight of that form, which streams
// faster for most counts (GPT-2 1.5B shard: one stored output -4%, N = 2 -3%,
// N = 4 -12%, N = 32 -8%; 7.5B N = 64 -2%; Llama-7B N = 16 -6%; fp32 gradients
// -8 to -11%).  With WIN = 0 every load is issued before the first add; with
// WIN > 0 (16, 32 and 64 16-bit buffers, 8 fp32 ones) the windowed sum above
// keeps WIN slice loads in flight.
// Lane t takes elements [4 q, 4 q + 4), q = 2 v_lo + t.
template <class GT, class PT, int C, int TPB = kThreads, int WIN = 0>
__global__ __launch_bounds__(TPB) void narrow_step_kernel(const StepLaunch a) {
  static_assert(WIN == 0 || (WIN > 0 && (C == 0 || WIN < C)), "the window holds fewer loads than there are buffers");
  static_assert(C > 0 || WIN > 0, "a run-time buffer count takes the windowed sum");
  if (a.skip_in != nullptr && *a.skip_in != 0u) {
    if (a.overflow != nullptr && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(a.overflow, 1u);
    return;
  }
  const int64_t q = 2 * a.v_lo + (int64_t)blockIdx.x * TPB + threadIdx.x;
  const int64_t j0 = q * 4;
  if (q >= 2 * a.v_hi || j0 >= a.S) return;
  AdamK c = a.c;
  float inv_scale = a.inv_scale;
  step_consts(a.kdev, c, inv_scale);
  const int64_t w0 = uniform64(q - (int64_t)(threadIdx.x & 63));  // the wave's first group
  bool bad = false;
  if (j0 + 4 <= a.S) {
    const char* base = static_cast<const char*>(a.grad) + j0 * GT::bytes;
    const int64_t o0 = state_off(a, j0);
    float p[4], m[4], v[4], acc[4];
    SegRange sr;
    if constexpr (C == 0) {   // the buffer count a.n, known at run time
      sr = wave_segs(a, w0 * 4, (w0 + 64) * 4);
      if (a.n >= WIN) window_sum_rt<GT, WIN>(base, a.ld_bytes, a.n, acc, a, o0, p, m, v);
      else small_sum_rt<GT, WIN>(base, a.ld_bytes, a.n, acc, a, o0, p, m, v);
    } else if constexpr (WIN > 0) {
      Raw4<GT> r[C];
      sr = wave_segs(a, w0 * 4, (w0 + 64) * 4);   // scalar work, ahead of the window
#pragma unroll
      for (int k = 0; k < WIN; ++k) {   // issued in slice order: the waits count loads in order
        r[k] = ld_raw4<GT>(base + (int64_t)k * a.ld_bytes);
        __builtin_amdgcn_sched_barrier(0);
      }
      window_sum<GT, C, WIN, 0>(r, acc, base, a.ld_bytes, a, o0, p, m, v);
    } else {
      Raw4<GT> r[C];
#pragma unroll
      for (int k = 0; k < C; ++k) r[k] = ld_raw4<GT>(base + (int64_t)k * a.ld_bytes);
      ld4(a.p_in + o0, p);
      ld4(a.m_in + o0, m);
      ld4(a.v_in + o0, v);
      sr = wave_segs(a, w0 * 4, (w0 + 64) * 4);   // behind the loads
      widen4<GT>(r[0], acc);
#pragma unroll
      for (int k = 1; k < C; ++k) {
        float w[4];
        widen4<GT>(r[k], w);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = acc[e] + w[e];
      }
    }
    float g[4];
    average_unscale_k<4>(acc, g, a.n_pow2, a.nf, a.recip_n, inv_scale);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bad |= !__builtin_isfinite(g[e]);
      adamw1(p[e], m[e], v[e], g[e], c);
    }
    st4(a.p_out + o0, p);
    st4(a.m_out + o0, m);
    st4(a.v_out + o0, v);
    const int64_t d0 = delta_of(a, sr, j0);
    if (delta_of(a, sr, j0 + 3) == d0) {
      store_params4<PT>(a.gather + (j0 + d0) * PT::bytes, p);
    } else {  // the 4 elements straddle two gather pieces
#pragma unroll
      for (int e = 0; e < 4; ++e) store_param1<PT>(a.gather + (j0 + e + delta_of(a, sr, j0 + e)) * PT::bytes, p[e]);
    }
  } else {
    // the shard's ragged end
    const SegRange sr = wave_segs(a, w0 * 4, (w0 + 64) * 4);
    for (int64_t j = j0; j < a.S; ++j) {
      const int64_t oj = state_off(a, j);
      float pe = a.p_in[oj], me = a.m_in[oj], ve = a.v_in[oj];
      const float acc = reduce1<GT>(static_cast<const char*>(a.grad) + j * GT::bytes, a.ld_bytes, C > 0 ? C : a.n);
      const float g = average_unscale(acc, a.n_pow2, a.nf, a.recip_n, inv_scale);
      bad |= !__builtin_isfinite(g);
      adamw1(pe, me, ve, g, c);
      a.p_out[oj] = pe;
      a.m_out[oj] = me;
      a.v_out[oj] = ve;
      store_param1<PT>(a.gather + (j + delta_of(a, sr, j)) * PT::bytes, pe);
    }
  }
  if (a.overflow != nullptr && bad) atomicOr(a.overflow, 1u);
}

// A step that is not applied, with the step control in device memory: the
// output state gets the input state, so the output is current either way.
__device__ __forceinline__ void copy_state(const StepLaunch& a, int64_t j0, int cnt) {
  if (cnt == kVec) {
    const int64_t o0 = state_off(a, j0);
    float x[8];
    ld8(a.p_in + o0, x);
    st8(a.p_out + o0, x);
    ld8(a.m_in + o0, x);
    st8(a.m_out + o0, x);
    ld8(a.v_in + o0, x);
    st8(a.v_out + o0, x);
  } else {
    for (int e = 0; e < cnt; ++e) {
      const int64_t oj = state_off(a, j0 + e);
      a.p_out[oj] = a.p_in[oj];
      a.m_out[oj] = a.m_in[oj];
      a.v_out[oj] = a.v_in[oj];
    }
  }
}

// The rank's gather slots of cnt local elements from j0 get the rounded p
// (p[e] for e < cnt), with the widest stores a whole vector allows.
template <class PT>
__device__ __forceinline__ void store_slots(const StepLaunch& a, const SegRange& sr, int64_t j0, int cnt,
                                            const float p[8]) {
  if (cnt == kVec) {
    const int64_t d0 = delta_of(a, sr, j0);
    if (delta_of(a, sr, j0 + kVec - 1) == d0) {
      store_params8<PT>(a.gather + (j0 + d0) * PT::bytes, p);
      return;
    }
  }
  for (int e = 0; e < cnt; ++e) store_param1<PT>(a.gather + (j0 + e + delta_of(a, sr, j0 + e)) * PT::bytes, p[e]);
}

// Small shards (S <= kSmallShard) in one launch: one workgroup, one 8-element
// vector per thread.  Every thread reduces its slices first and keeps g in
// registers; a workgroup-wide OR of the overflow decides the skip before any
// output is written, so a skipped step needs no restore pass or flag reset
// (the two extra launches of the multi-workgroup path, which dominate a step
// this small).  A step that is not applied leaves what the multi-workgroup
// path leaves: with an overflow flag, the rank's slots hold the rounded input
// master (and with a.restore the output state holds the input state); without
// one, nothing is checked and the update is applied whatever g holds.
// (batches of 8 slices whatever N: 1024 threads leave 128 registers each)
template <class GT, class PT>
__global__ __launch_bounds__(kSmallThreads) void small_step_kernel(const StepLaunch a) {
  AdamK c = a.c;
  float inv_scale = a.inv_scale;
  step_consts(a.kdev, c, inv_scale);
  if (a.skip_in != nullptr && *a.skip_in != 0u) {
    if (a.overflow != nullptr && threadIdx.x == 0) *a.overflow = 1u;
    if (a.ctl != nullptr && threadIdx.x == 0) ctl_advance(a.ctl, true);
    const int64_t j = (int64_t)threadIdx.x * kVec, rest = a.S - j;
    if (rest <= 0) return;
    const int cnt = rest >= kVec ? kVec : (int)rest;
    if (a.restore) copy_state(a, j, cnt);
    if (a.overflow != nullptr) {   // the slots keep the pre-step parameters
      float p[8];
      for (int e = 0; e < cnt; ++e) p[e] = a.p_in[state_off(a, j + e)];
      store_slots<PT>(a, wave_segs_v(a, threadIdx.x), j, cnt, p);
    }
    return;
  }
  // With the step control in device memory the workgroup derives the step's
  // constants itself (the begin and end launches of the multi-workgroup path
  // are folded in): every thread takes 1/scale, the last two lanes -- the
  // least loaded, past the end of most shards -- the two powers and lr, dec,
  // published to the others by the overflow barrier below.
  __shared__ float s_k[4];
  if (a.ctl != nullptr) {
    inv_scale = ctl_inv_scale(a.ctl);
    const int i = kSmallThreads - 1 - (int)threadIdx.x;   // 0, 1 for the last two lanes
    if (i <= 1) {
      const float bc = ctl_bias_correction(a.ctl, i, a.beta1, a.beta2);
      s_k[i] = bc;
      a.ctl->k[i] = bc;
      if (i == 0) {
        const double lr = a.ctl->lr;
        s_k[2] = a.ctl->k[2] = (float)lr;
        s_k[3] = a.ctl->k[3] = (float)(1.0 - lr * a.wd);
        a.ctl->k[4] = inv_scale;
      }
    }
  }
  const int64_t j0 = (int64_t)threadIdx.x * kVec;
  const SegRange sr = wave_segs_v(a, threadIdx.x);
  const int64_t rest = a.S - j0;
  const int cnt = rest >= kVec ? kVec : (rest > 0 ? (int)rest : 0);
  float g[8];
  bool bad = false;
  // the state goes out with the gradient loads: the step is latency bound, and
  // only the stores wait for the skip decision
  float p[8], m[8], v[8];
  const int64_t o0 = state_off(a, j0);
  if (cnt == kVec) {
    ld8(a.p_in + o0, p);
    ld8(a.m_in + o0, m);
    ld8(a.v_in + o0, v);
  }
  if (cnt == kVec) {
    float acc[8];
    if (a.grad_full)
      reduce8_pieces<GT, Batch<GT, false>::value>(a, sr, j0, acc);
    else
      reduce8<GT, Batch<GT, false>::value>(static_cast<const char*>(a.grad) + j0 * GT::bytes, a.ld_bytes,
                                           a.n, acc);
    average_unscale_k<8>(acc, g, a.n_pow2, a.nf, a.recip_n, inv_scale);
  } else {
    for (int e = 0; e < 8; ++e) {
      g[e] = 0.0f;
      if (e < cnt) {
        const float acc = reduce1<GT>(grad_elem<GT>(a, sr, j0 + e), a.ld_bytes, a.n);
        g[e] = average_unscale(acc, a.n_pow2, a.nf, a.recip_n, inv_scale);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) bad |= !__builtin_isfinite(g[e]);
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (a.overflow != nullptr && threadIdx.x == 0) *a.overflow = any_bad ? 1u : 0u;
  if (a.ctl != nullptr) {
    c.bc1 = s_k[0];
    c.bc2 = s_k[1];
    c.lr = s_k[2];
    c.dec = s_k[3];
    if (threadIdx.x == 0) ctl_advance(a.ctl, any_bad != 0);
  }
  if (cnt == 0) return;
  if (any_bad && a.overflow != nullptr) {
    if (cnt == kVec) {
      if (a.restore) {
        st8(a.p_out + o0, p);
        st8(a.m_out + o0, m);
        st8(a.v_out + o0, v);
      }
    } else {
      if (a.restore) copy_state(a, j0, cnt);
      for (int e = 0; e < cnt; ++e) p[e] = a.p_in[state_off(a, j0 + e)];
    }
    store_slots<PT>(a, sr, j0, cnt, p);   // the slots keep the pre-step parameters
    return;
  }
  if (cnt == kVec) {
#pragma unroll
    for (int e = 0; e < 8; ++e) adamw1(p[e], m[e], v[e], g[e], c);
    st8(a.p_out + o0, p);
    st8(a.m_out + o0, m);
    st8(a.v_out + o0, v);
    store_slots<PT>(a, sr, j0, kVec, p);
  } else {
    for (int e = 0; e < cnt; ++e) {
      const int64_t j = j0 + e;
      const int64_t oj = state_off(a, j);
      float pe = a.p_in[oj], me = a.m_in[oj], ve = a.v_in[oj];
      adamw1(pe, me, ve, g[e], c);
      a.p_out[oj] = pe;
      a.m_out[oj] = me;
      a.v_out[oj] = ve;
      store_param1<PT>(a.gather + (j + delta_of(a, sr, j)) * PT::bytes, pe);
    }
  }
}

// On a skipped fused step: rewrite the rank's gather pieces from master_in, so
// they keep the pre-step parameters (and with a.restore copy the input state to
// the output).  A no-op unless *cond != 0, apart from the step control advance
// (a.ctl, one thread).
template <class PT>
__global__ __launch_bounds__(kThreads) void recast_kernel(const StepLaunch a, const u32* cond) {
  const u32 skipped = *cond;
  if (a.ctl != nullptr && blockIdx.x == 0 && threadIdx.x == 0) ctl_advance(a.ctl, skipped != 0u);
  if (skipped == 0u) return;
  for (int64_t v = a.v_lo + (int64_t)blockIdx.x * kThreads + threadIdx.x; v < a.v_hi;
       v += (int64_t)gridDim.x * kThreads) {
    const int64_t j0 = v * kVec;
    const SegRange sr = wave_segs_v(a, v);
    if (a.restore) copy_state(a, j0, j0 + kVec <= a.S ? kVec : (int)(a.S - j0));
    if (j0 + kVec <= a.S) {
      float p[8];
      ld8(a.p_in + state_off(a, j0), p);
      const int64_t d0 = delta_of(a, sr, j0);
      if (delta_of(a, sr, j0 + kVec - 1) == d0) {
        store_params8<PT>(a.gather + (j0 + d0) * PT::bytes, p);
      } else {
        for (int e = 0; e < 8; ++e) store_param1<PT>(a.gather + (j0 + e + delta_of(a, sr, j0 + e)) * PT::bytes, p[e]);
      }
    } else {
      for (int64_t j = j0; j < a.S; ++j)
        store_param1<PT>(a.gather + (j + delta_of(a, sr, j)) * PT::bytes, a.p_in[state_off(a, j)]);
    }
  }
}

// ---------------------------------------------------------------------------
// gradient preparation with per-workgroup overflow words and fp64 sums of g^2
// ---------------------------------------------------------------------------

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// NB slices per load batch, NBATCH batches known at compile time (0: any N:
// the run-time ring, or the runtime loop with batches of NB below its window
// and for the full-gradient source)
template <class GT, int NB, int NBATCH>
__global__ __launch_bounds__(kThreads) void reduce_kernel(const ReduceLaunch a) {
  // one 8-element vector per thread; workgroup b owns vectors [256 b, 256 b + 256),
  // so the partition (and every partial sum) depends only on S
  double sq = 0.0;
  bool bad = false;
  const int64_t blk = a.blk0 + blockIdx.x;   // this launch's tiles start at blk0
  const int64_t v = blk * kThreads + threadIdx.x;
  AdamK unused{};
  float inv_scale = a.inv_scale;
  step_consts(a.kdev, unused, inv_scale);
  if (v < a.nvec) {
    const int64_t j0 = v * kVec;
    // pieces are needed only to find the full-layout gradient
    const SegRange sr = a.grad_full ? wave_segs_v(a, v) : SegRange{0, -1};
    if (j0 + kVec <= a.S) {
      float acc[8], g[8];
      if constexpr (NBATCH > 0) {
        const char* ubase = static_cast<const char*>(a.grad) + blk * (kTile * GT::bytes);
        reduce8_fixed<GT, NB, NBATCH, kReduceWindow>(ubase, a.ld_bytes, threadIdx.x * (uint32_t)(kVec * GT::bytes),
                                                     acc, [] {});
      } else if (a.grad_full) {
        reduce8_pieces<GT, NB>(a, sr, j0, acc);
      } else if (a.n >= kReduceWindow) {   // the windowed sum with a run-time count
        reduce8_ring<GT, kReduceWindow>(static_cast<const char*>(a.grad) + j0 * GT::bytes, a.ld_bytes, a.n, acc,
                                        [] {});
      } else {
        reduce8<GT, NB>(static_cast<const char*>(a.grad) + j0 * GT::bytes, a.ld_bytes, a.n, acc);
      }
      average_unscale_k<8>(acc, g, a.n_pow2, a.nf, a.recip_n, inv_scale);
#pragma unroll
      for (int e = 0; e < 8; ++e) bad |= !__builtin_isfinite(g[e]);
      if (a.g_out != nullptr) st8_stream(a.g_out + j0, g);
      if (a.want_sumsq) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sq += (double)g[e] * (double)g[e];
      }
    } else {
      for (int64_t j = j0; j < a.S; ++j) {
        const float acc = reduce1<GT>(grad_elem<GT>(a, sr, j), a.ld_bytes, a.n);
        const float g = average_unscale(acc, a.n_pow2, a.nf, a.recip_n, inv_scale);
        bad |= !__builtin_isfinite(g);
        if (a.g_out != nullptr) a.g_out[j] = g;
        if (a.want_sumsq) sq += (double)g * (double)g;
      }
    }
  }
  // fixed-order workgroup reduction: xor-shuffle within each wave64, then the 4
  // wave results in index order
  __shared__ double s_sum[kThreads / 64];
  __shared__ u32 s_bad[kThreads / 64];
  sq = wave_sum(sq);
  const u32 wbad = __any(bad) ? 1u : 0u;
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_sum[wave] = sq;
    s_bad[wave] = wbad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    u32 f = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      t += s_sum[w];
      f |= s_bad[w];
    }
    a.ws_sums[blk] = t;
    a.ws_flags[blk] = f;
  }
}

// Finalize, in two fixed-order levels so the sum is the same run to run.
// Level 1: workgroup g of kNormGroups sums the per-workgroup partials in
// [g * chunk, (g + 1) * chunk) (strided per thread, then an LDS tree) and ORs the
// overflow words.  Level 2: one workgroup sums the kNormGroups level-1 results in
// index order, takes the norm and the clip coefficient.  Two launches: the
// kernel boundary makes level 1's results visible to every XCD.
__device__ __forceinline__ void block_sum_or(double& s, u32& f) {
  __shared__ double s_sum[kNormThreads];
  __shared__ u32 s_f[kNormThreads];
  s_sum[threadIdx.x] = s;
  s_f[threadIdx.x] = f;
  __syncthreads();
  for (int w = kNormThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      s_sum[threadIdx.x] += s_sum[threadIdx.x + w];
      s_f[threadIdx.x] |= s_f[threadIdx.x + w];
    }
    __syncthreads();
  }
  s = s_sum[0];
  f = s_f[0];
}

__global__ __launch_bounds__(kNormThreads) void norm_partial_kernel(const NormLaunch a) {
  const int64_t lo = (int64_t)blockIdx.x * a.chunk;
  const int64_t hi = lo + a.chunk < a.nblocks ? lo + a.chunk : a.nblocks;
  double s = 0.0;
  u32 f = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kNormThreads) {
    s += a.ws_sums[i];
    f |= a.ws_flags[i];
  }
  block_sum_or(s, f);
  if (threadIdx.x == 0) {
    a.l2_sums[blockIdx.x] = s;
    a.l2_flags[blockIdx.x] = f;
  }
}

__global__ __launch_bounds__(kNormThreads) void norm_final_kernel(const NormLaunch a) {
  double s = 0.0;
  u32 f = 0;
  for (int i = threadIdx.x; i < kNormGroups; i += kNormThreads) {
    s += a.l2_sums[i];
    f |= a.l2_flags[i];
  }
  block_sum_or(s, f);
  if (threadIdx.x == 0) {
    const double q = s;
    const double norm = __builtin_sqrt(q + a.other_sumsq);
    const double c = (a.max_norm > 0.0 && norm > a.max_norm) ? a.max_norm / norm : 1.0;
    if (a.overflow_out) *a.overflow_out = f ? 1u : 0u;
    if (a.sumsq_out) *a.sumsq_out = q;
    if (a.clip_out) *a.clip_out = (float)c;
  }
}

__global__ void fill_u32_kernel(u32* p, u32 value) {
  if (threadIdx.x == 0) *p = value;
}

// Step control, begin: the constants of the step about to run into ctl->k
// (and a reset of the fused step's overflow flag, which this launch replaces).
__global__ void ctl_begin_kernel(zero_step_ctl_t* ctl, int adam, double beta1, double beta2, double wd,
                                 u32* reset) {
  const int i = threadIdx.x;
  if (i > 1) return;
  if (adam) ctl->k[i] = ctl_bias_correction(ctl, i, beta1, beta2);
  if (i == 0) {
    if (adam) {
      const double lr = ctl->lr;
      ctl->k[2] = (float)lr;
      ctl->k[3] = (float)(1.0 - lr * wd);
    }
    ctl->k[4] = ctl_inv_scale(ctl);
    if (reset != nullptr) *reset = 0u;
  }
}

// Step control, end: the advance after a step whose flag is *flag (NULL: applied).
__global__ void ctl_end_kernel(zero_step_ctl_t* ctl, const u32* flag) {
  if (threadIdx.x == 0) ctl_advance(ctl, flag != nullptr && *flag != 0u);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    char buf[256];
    snprintf(buf, sizeof buf, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
    return fail(ZERO_EHIP, buf);
  }
  return ZERO_OK;
}

static size_t occupancy_lds(int per_cu);

// Plain streaming copy: each lane moves kCopyVecs 16-byte vectors (loads all
// issued before the stores), non-temporal both ways; one-shot grid.  Measured
// best of 1/2/4/8 vectors per lane at 2-6 resident workgroups per CU: two
// vectors at three workgroups (6.6 TB/s; with 8 vectors 5.5 TB/s -- the copy
// streams fastest with about 24 KiB of loads in flight per CU).
constexpr int kCopyVecs = 2;
constexpr int kCopyBlocksPerCU = 3;

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(uint4* __restrict__ dst,
                                                              const uint4* __restrict__ src, int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * kCopyVecs + threadIdx.x;
  uint4 x[kCopyVecs];
#pragma unroll
  for (int i = 0; i < kCopyVecs; ++i) {
    const int64_t k = base + (int64_t)i * kThreads;
    if (k < n16) x[i] = ld_stream16(src + k);
  }
#pragma unroll
  for (int i = 0; i < kCopyVecs; ++i) {
    const int64_t k = base + (int64_t)i * kThreads;
    if (k < n16) st_stream16(dst + k, x[i]);
  }
}

int launch_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return ZERO_OK;
  const int64_t per_block = (int64_t)kThreads * kCopyVecs;
  const unsigned blocks = (unsigned)((n16 + per_block - 1) / per_block);
  hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(kThreads), occupancy_lds(kCopyBlocksPerCU),
                     (hipStream_t)stream, static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16);
  return check_launch("copy");
}

int launch_fill_u32(u32* p, u32 value, void* stream) {
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, p, value);
  return check_launch("fill");
}

int launch_ctl_begin(zero_step_ctl_t* ctl, int adam, double beta1, double beta2, double weight_decay,
                     u32* reset_flag, void* stream) {
  hipLaunchKernelGGL(ctl_begin_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, ctl, adam, beta1, beta2,
                     weight_decay, reset_flag);
  return check_launch("step control (begin)");
}

int launch_ctl_end(zero_step_ctl_t* ctl, const u32* flag, void* stream) {
  hipLaunchKernelGGL(ctl_end_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, ctl, flag);
  return check_launch("step control (end)");
}

// The compile-time form (the windowed sum) for the one count the narrow form
// does not take in the shard layout, 16-bit N = 8; the runtime-N form for
// every other N and for the full-gradient source.
template <class GT, class PT, bool WIDE>
static void go_step_full(const StepLaunch& a, unsigned blocks, size_t lds, hipStream_t st) {
  constexpr int NB = Batch<GT, WIDE>::value;
  const int nbatch = (!a.grad_full && a.n % NB == 0) ? a.n / NB : 0;
  const dim3 g(blocks), b(kThreads);
  if constexpr (GT::bytes == 2 && !WIDE) {
    if (nbatch == 1) {
      hipLaunchKernelGGL((step_kernel<GT, PT, WIDE, 1>), g, b, lds, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((step_kernel<GT, PT, WIDE, 0>), g, b, lds, st, a);
}

// wide batches when N > 8 (the full-gradient source); the windowed sum for
// 16-bit N = 8
template <class GT, class PT>
static void go_step(const StepLaunch& a, unsigned blocks, size_t lds, hipStream_t st) {
  if (a.n > 8)
    go_step_full<GT, PT, true>(a, blocks, lds, st);
  else
    go_step_full<GT, PT, false>(a, blocks, lds, st);
}

// Resident workgroups per CU of the streaming kernels.  Fewer concurrent waves
// keep fewer DRAM pages open per stream.  Measured on the GPT-2 1.5B and
// Llama-7B shards, 2 workgroups (8 wave64s) per CU stream the fused update and
// the reduction 7-8% faster than 3 or 4, while 1 per CU is too few to cover
// the latency; the stash-mode update (four elements per lane) is best at 5
// (2: -20%, 3: -5%, 4: -1%, 6: -1% on the Llama-3 clipped step).
// The cap is imposed by reserving dynamic LDS the kernels do not otherwise use.
// The reservation sits halfway between the sizes at which per_cu + 1 and
// per_cu workgroups just fit, in 2 KiB steps, so that neither the allocation
// granularity nor a kernel's own small __shared__ arrays move the count: a
// reservation of exactly a third of the CU's LDS already admits only two.  A
// workgroup's dynamic plus static LDS must also stay within the per-workgroup
// limit, or the dispatch is invalid; kStaticLdsRoom is kept free for that.
static size_t occupancy_lds(int per_cu) {
  static thread_local int dev_cached = -1;
  static thread_local size_t lds_cu = 0, lds_block = 0;
  int dev = 0;
  if (per_cu <= 0 || hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev != dev_cached) {
    int v = 0, b = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess) v = 0;
    if (hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) b = 0;
    lds_cu = (size_t)v;
    lds_block = (size_t)b;
    dev_cached = dev;
  }
  const size_t fits = lds_cu / (size_t)per_cu;               // per_cu workgroups fit at or below
  const size_t excludes = lds_cu / (size_t)(per_cu + 1);     // per_cu + 1 cannot fit above
  if (fits <= kStaticLdsRoom) return 0;
  size_t r = ((fits - kStaticLdsRoom + excludes) / 2) / 2048 * 2048;
  if (lds_block > kStaticLdsRoom && r > lds_block - kStaticLdsRoom) r = lds_block - kStaticLdsRoom;
  if (lds_block <= kStaticLdsRoom || r <= excludes) return 0;  // no reservation that enforces the cap
  return r;
}

// Resident workgroups per CU of a kernel that sums n gradient buffers: with
// one or two the update moves few streams and three workgroups per CU stream
// faster than two (GPT-2 shard: +2.5% from one stored reduce-scatter output,
// +7% from one full all-reduced gradient).
static int stream_blocks_per_cu(int n) { return n <= 2 ? kFewStreamBlocksPerCU : kStreamBlocksPerCU; }

template <class GT>
static int dispatch_pt(const StepLaunch& a, zero_dtype_t pt, unsigned blocks, hipStream_t st) {
  const size_t lds = occupancy_lds(stream_blocks_per_cu(a.n));
  switch (pt) {
    case ZERO_F32: go_step<GT, TF32>(a, blocks, lds, st); return ZERO_OK;
    case ZERO_BF16: go_step<GT, TBF16>(a, blocks, lds, st); return ZERO_OK;
    case ZERO_F16: go_step<GT, TF16>(a, blocks, lds, st); return ZERO_OK;
  }
  return fail(ZERO_EINVAL, "unsupported parameter dtype");
}

// The narrow fused form serves the shard layout when its buffer count is
// compiled: 1, 2, 4, and 16, 32, 64 for 16-bit gradients or 8, 16, 32 for fp32
// (the eight-element form keeps 16-bit N = 8, where the windowed eight-element
// sum is faster, and fp32 N = 64).  fp32 N = 16 with a window of 4 slice loads
// runs 8% faster than the eight-element form's two windowed batches (GPT-2
// tensors).  Resident workgroups per CU: 3, or 2 when a lane's raw gradient
// bytes exceed 64, as measured.
static bool narrow_form(zero_dtype_t gt, int n, int grad_full) {
  if (grad_full) return false;
  return !(n == 8 && gt != ZERO_F32);
}

template <class GT, class PT>
static int go_narrow(const StepLaunch& a, int64_t nv, hipStream_t st) {
  const dim3 g((unsigned)((2 * nv + kThreads - 1) / kThreads)), b(kThreads);
  const size_t lds = occupancy_lds(a.n * 4 * GT::bytes > 64 ? kNarrowWideBlocksPerCU : kNarrowBlocksPerCU);
  if constexpr (GT::bytes == 2) {
    if (a.n == 64) {
      // 64 slices: one workgroup of kNarrow64Threads per CU, each lane with a
      // window of kNarrow64Window slice loads in flight
      const dim3 g2((unsigned)((2 * nv + kNarrow64Threads - 1) / kNarrow64Threads)), b2(kNarrow64Threads);
      hipLaunchKernelGGL((narrow_step_kernel<GT, PT, 64, kNarrow64Threads, kNarrow64Window>), g2, b2,
                         occupancy_lds(1), st, a);
      return ZERO_OK;
    }
  }
  switch (a.n) {
    case 1: hipLaunchKernelGGL((narrow_step_kernel<GT, PT, 1>), g, b, lds, st, a); return ZERO_OK;
    case 2: hipLaunchKernelGGL((narrow_step_kernel<GT, PT, 2>), g, b, lds, st, a); return ZERO_OK;
    case 4: hipLaunchKernelGGL((narrow_step_kernel<GT, PT, 4>), g, b, lds, st, a); return ZERO_OK;
    case 8:
      if constexpr (GT::bytes == 4) {
        hipLaunchKernelGGL((narrow_step_kernel<GT, PT, 8, kThreads, kNarrowWindow32>), g, b, lds, st, a);
        return ZERO_OK;
      }
      break;
    case 16:
      hipLaunchKernelGGL((narrow_step_kernel<GT, PT, 16, kThreads, GT::bytes == 4 ? kNarrowWindow32 : kNarrowWindow>), g,
                         b, lds, st, a);
      return ZERO_OK;
    case 32:
      hipLaunchKernelGGL((narrow_step_kernel<GT, PT, 32, kThreads, GT::bytes == 4 ? kNarrowWindow32 : kNarrowWindow>), g,
                         b, lds, st, a);
      return ZERO_OK;
  }
  // any other count: the run-time windowed sum
  hipLaunchKernelGGL((narrow_step_kernel<GT, PT, 0, kThreads, GT::bytes == 4 ? kNarrowWindow32 : kNarrowWindow>), g, b,
                     lds, st, a);
  return ZERO_OK;
}

template <class GT>
static int dispatch_narrow(const StepLaunch& a, zero_dtype_t pt, int64_t nv, hipStream_t st) {
  switch (pt) {
    case ZERO_F32: return go_narrow<GT, TF32>(a, nv, st);
    case ZERO_BF16: return go_narrow<GT, TBF16>(a, nv, st);
    case ZERO_F16: return go_narrow<GT, TF16>(a, nv, st);
  }
  return fail(ZERO_EINVAL, "unsupported parameter dtype");
}

// the stash-mode update: two 4-element groups per 8-element vector
static int dispatch_stash(const StepLaunch& a, zero_dtype_t pt, int64_t nv, hipStream_t st) {
  const dim3 g((unsigned)((2 * nv + kThreads - 1) / kThreads)), b(kThreads);
  const size_t lds = occupancy_lds(kStashBlocksPerCU);
  switch (pt) {
    case ZERO_F32: hipLaunchKernelGGL(stash_step_kernel<TF32>, g, b, lds, st, a); return ZERO_OK;
    case ZERO_BF16: hipLaunchKernelGGL(stash_step_kernel<TBF16>, g, b, lds, st, a); return ZERO_OK;
    case ZERO_F16: hipLaunchKernelGGL(stash_step_kernel<TF16>, g, b, lds, st, a); return ZERO_OK;
  }
  return fail(ZERO_EINVAL, "unsupported parameter dtype");
}

static int launch_step_range(const StepLaunch& a, zero_dtype_t gt, zero_dtype_t pt, bool stash, void* stream) {
  const int64_t nv = a.v_hi - a.v_lo;
  if (nv <= 0) return ZERO_OK;
  const unsigned blocks = (unsigned)((nv + kThreads - 1) / kThreads);
  hipStream_t st = (hipStream_t)stream;
  int rc;
  if (stash) {
    rc = dispatch_stash(a, pt, nv, st);
  } else if (narrow_form(gt, a.n, a.grad_full)) {
    switch (gt) {
      case ZERO_F32: rc = dispatch_narrow<TF32>(a, pt, nv, st); break;
      case ZERO_BF16: rc = dispatch_narrow<TBF16>(a, pt, nv, st); break;
      case ZERO_F16: rc = dispatch_narrow<TF16>(a, pt, nv, st); break;
      default: return fail(ZERO_EINVAL, "unsupported gradient dtype");
    }
  } else {
    switch (gt) {
      case ZERO_F32: rc = dispatch_pt<TF32>(a, pt, blocks, st); break;
      case ZERO_BF16: rc = dispatch_pt<TBF16>(a, pt, blocks, st); break;
      case ZERO_F16: rc = dispatch_pt<TF16>(a, pt, blocks, st); break;
      default: return fail(ZERO_EINVAL, "unsupported gradient dtype");
    }
  }
  if (rc != ZERO_OK) return rc;
  return check_launch("step");
}

// A shard larger than kLaunchElems (kLaunchElems64 for the 64-buffer
// four-element form) is updated in consecutive launches of at most that many
// elements, in order on the stream.
int launch_step(const StepLaunch& a0, zero_dtype_t gt, zero_dtype_t pt, bool stash, void* stream) {
  const bool n64 = !stash && gt != ZERO_F32 && a0.n == 64 && narrow_form(gt, a0.n, a0.grad_full);
  const int64_t kChunk = (n64 ? kLaunchElems64 : kLaunchElems) / kVec;   // vectors per launch
  if (a0.v_hi - a0.v_lo <= kChunk) return launch_step_range(a0, gt, pt, stash, stream);
  StepLaunch a = a0;
  for (int64_t lo = a0.v_lo; lo < a0.v_hi; lo += kChunk) {
    a.v_lo = lo;
    a.v_hi = a0.v_hi - lo < kChunk ? a0.v_hi : lo + kChunk;
    const int rc = launch_step_range(a, gt, pt, stash, stream);
    if (rc) return rc;
  }
  return ZERO_OK;
}

template <class GT>
static int small_pt(const StepLaunch& a, zero_dtype_t pt, hipStream_t st) {
  const dim3 g(1), b(kSmallThreads);
  switch (pt) {
    case ZERO_F32: hipLaunchKernelGGL((small_step_kernel<GT, TF32>), g, b, 0, st, a); return ZERO_OK;
    case ZERO_BF16: hipLaunchKernelGGL((small_step_kernel<GT, TBF16>), g, b, 0, st, a); return ZERO_OK;
    case ZERO_F16: hipLaunchKernelGGL((small_step_kernel<GT, TF16>), g, b, 0, st, a); return ZERO_OK;
  }
  return fail(ZERO_EINVAL, "unsupported parameter dtype");
}

int launch_small_step(const StepLaunch& a, zero_dtype_t gt, zero_dtype_t pt, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  int rc;
  switch (gt) {
    case ZERO_F32: rc = small_pt<TF32>(a, pt, st); break;
    case ZERO_BF16: rc = small_pt<TBF16>(a, pt, st); break;
    case ZERO_F16: rc = small_pt<TF16>(a, pt, st); break;
    default: return fail(ZERO_EINVAL, "unsupported gradient dtype");
  }
  if (rc != ZERO_OK) return rc;
  return check_launch("small step");
}

int launch_recast(const StepLaunch& a, zero_dtype_t pt, const u32* cond, void* stream) {
  const int64_t nv = a.v_hi - a.v_lo;
  if (nv <= 0) return ZERO_OK;
  int64_t b = (nv + kThreads - 1) / kThreads;
  const unsigned blocks = (unsigned)(b < 1024 ? b : 1024);
  hipStream_t st = (hipStream_t)stream;
  switch (pt) {
    case ZERO_F32: hipLaunchKernelGGL(recast_kernel<TF32>, dim3(blocks), dim3(kThreads), 0, st, a, cond); break;
    case ZERO_BF16: hipLaunchKernelGGL(recast_kernel<TBF16>, dim3(blocks), dim3(kThreads), 0, st, a, cond); break;
    case ZERO_F16: hipLaunchKernelGGL(recast_kernel<TF16>, dim3(blocks), dim3(kThreads), 0, st, a, cond); break;
    default: return fail(ZERO_EINVAL, "unsupported parameter dtype");
  }
  return check_launch("recast");
}

// The reduction's compiled forms: every whole number of batches of the usual
// size (8 16-bit or 4 fp32 slices, twice that for larger N) in 1, 2 or 4
// batches, summed in the window of kReduceWindow slice loads, and one batch of
// exactly N for N = 1, 2, 4 (the runtime loop, with its per-slice guards,
// reduced 4 bf16 slices of the GPT-2 shard at 3.3 TB/s).  Other counts take
// the ring (four or more) or the runtime loop (three), inside the NBATCH = 0
// instantiation.  Only reachable forms are instantiated.
template <class GT>
static void go_reduce(const ReduceLaunch& a, dim3 grid, size_t lds, hipStream_t st) {
  const dim3 blk(kThreads);
  constexpr int NS = Batch<GT, false>::value, NW = Batch<GT, true>::value;
  const int n = a.n;
  if (!a.grad_full) {
    if (n == 1) { hipLaunchKernelGGL((reduce_kernel<GT, 1, 1>), grid, blk, lds, st, a); return; }
    if (n == 2) { hipLaunchKernelGGL((reduce_kernel<GT, 2, 1>), grid, blk, lds, st, a); return; }
    if (n == NS) { hipLaunchKernelGGL((reduce_kernel<GT, NS, 1>), grid, blk, lds, st, a); return; }
    if constexpr (NS == 8) {   // 16-bit: 4 alone is below the usual batch
      if (n == 4) { hipLaunchKernelGGL((reduce_kernel<GT, 4, 1>), grid, blk, lds, st, a); return; }
    } else {                   // fp32: 8 is two batches of 4
      if (n == 2 * NS) { hipLaunchKernelGGL((reduce_kernel<GT, NS, 2>), grid, blk, lds, st, a); return; }
    }
    if (n > 8 && n % NW == 0) {
      switch (n / NW) {
        case 1:
          if constexpr (NS == 8) {   // fp32 reaches 8 = NW as two batches of 4, above
            hipLaunchKernelGGL((reduce_kernel<GT, NW, 1>), grid, blk, lds, st, a);
            return;
          }
          break;
        case 2: hipLaunchKernelGGL((reduce_kernel<GT, NW, 2>), grid, blk, lds, st, a); return;
        case 4: hipLaunchKernelGGL((reduce_kernel<GT, NW, 4>), grid, blk, lds, st, a); return;
        default: break;
      }
    }
  }
  // the run-time count: the ring, or the runtime loop below the window, with
  // batches of the usual size, twice that above 8 buffers
  if (n > 8) hipLaunchKernelGGL((reduce_kernel<GT, NW, 0>), grid, blk, lds, st, a);
  else hipLaunchKernelGGL((reduce_kernel<GT, NS, 0>), grid, blk, lds, st, a);
}

// Resident workgroups per CU of the reduction pass (eight elements per lane):
// three while a lane's raw gradient bytes stay within 128 (16-bit N <= 8, fp32
// N <= 4), else two.  Measured on the GPT-2 1.5B shard, 8 bf16 slices: 6.23
// against 5.70 TB/s at two; 16 bf16 slices (Llama-3 shard) are best at two.
static int reduce_blocks_per_cu(int n, int grad_bytes) {
  return n * kVec * grad_bytes <= 128 ? kReduceFewBlocksPerCU : kStreamBlocksPerCU;
}

// Tiles [a.blk0, a.blk0 + nblocks), in launches of at most kLaunchElems
// elements (kLaunchElems / kTile workgroups), in order on the stream.
int launch_reduce(const ReduceLaunch& a0, zero_dtype_t gt, int64_t nblocks, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int gb = gt == ZERO_F32 ? 4 : 2;
  const size_t lds = occupancy_lds(reduce_blocks_per_cu(a0.n, gb));
  constexpr int64_t kChunk = kLaunchElems / kTile;   // workgroups per launch
  ReduceLaunch a = a0;
  for (int64_t done = 0; done < nblocks; done += kChunk) {
    a.blk0 = a0.blk0 + done;
    const dim3 grid((unsigned)(nblocks - done < kChunk ? nblocks - done : kChunk));
    switch (gt) {
      case ZERO_F32: go_reduce<TF32>(a, grid, lds, st); break;
      case ZERO_BF16: go_reduce<TBF16>(a, grid, lds, st); break;
      case ZERO_F16: go_reduce<TF16>(a, grid, lds, st); break;
      default: return fail(ZERO_EINVAL, "unsupported gradient dtype");
    }
    const int rc = check_launch("reduce");
    if (rc) return rc;
  }
  return ZERO_OK;
}

int launch_norm(const NormLaunch& a, void* stream) {
  hipLaunchKernelGGL(norm_partial_kernel, dim3(kNormGroups), dim3(kNormThreads), 0, (hipStream_t)stream, a);
  int rc = check_launch("norm");
  if (rc) return rc;
  hipLaunchKernelGGL(norm_final_kernel, dim3(1), dim3(kNormThreads), 0, (hipStream_t)stream, a);
  return check_launch("norm");
}

int record_event(void* ev, void* stream) {
  if (ev == nullptr) return ZERO_OK;
  const hipError_t e = hipEventRecord((hipEvent_t)ev, (hipStream_t)stream);
  if (e != hipSuccess) {
    char buf[256];
    snprintf(buf, sizeof buf, "hipEventRecord: HIP error %d (%s)", (int)e, hipGetErrorString(e));
    return fail(ZERO_EHIP, buf);
  }
  return ZERO_OK;
}

}  // namespace zk
