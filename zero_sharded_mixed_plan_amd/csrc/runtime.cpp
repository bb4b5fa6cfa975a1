// Host runtime around the step: the dynamic loss-scale update, the plan hash
// and per-rank (sharded) checkpoints of the optimizer state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "zero_internal.h"

using zk::fail;

// ---------------------------------------------------------------------------
// loss scale
// ---------------------------------------------------------------------------

extern "C" int zero_scaler_init(zero_scaler_t* s, float init_scale, float growth_factor,
                                float backoff_factor, int32_t growth_interval) {
  if (!s) return fail(ZERO_EINVAL, "zero_scaler_init: scaler is NULL");
  if (!(std::isfinite(init_scale) && init_scale > 0.0f))
    return fail(ZERO_EINVAL, "zero_scaler_init: init_scale must be finite and > 0");
  if (!(std::isfinite(growth_factor) && growth_factor > 1.0f))
    return fail(ZERO_EINVAL, "zero_scaler_init: growth_factor must be > 1");
  if (!(backoff_factor > 0.0f && backoff_factor < 1.0f))
    return fail(ZERO_EINVAL, "zero_scaler_init: backoff_factor must be in (0, 1)");
  if (growth_interval < 1) return fail(ZERO_EINVAL, "zero_scaler_init: growth_interval must be >= 1");
  s->scale = init_scale;
  s->growth_tracker = 0;
  s->growth_factor = growth_factor;
  s->backoff_factor = backoff_factor;
  s->growth_interval = growth_interval;
  return ZERO_OK;
}

extern "C" int zero_scaler_update(zero_scaler_t* s, int32_t overflow) {
  if (!s) return fail(ZERO_EINVAL, "zero_scaler_update: scaler is NULL");
  if (overflow) {
    s->scale = s->scale * s->backoff_factor;
    s->growth_tracker = 0;
    return ZERO_OK;
  }
  const int32_t n = s->growth_tracker + 1;
  if (n >= s->growth_interval) {
    const float grown = s->scale * s->growth_factor;
    if (std::isfinite(grown)) s->scale = grown;
    s->growth_tracker = 0;
  } else {
    s->growth_tracker = n;
  }
  return ZERO_OK;
}

extern "C" float zero_scaler_inv_scale(const zero_scaler_t* s) {
  if (!s) return 0.0f;
  return (float)(1.0 / (double)s->scale);
}

// ---------------------------------------------------------------------------
// plan hash
// ---------------------------------------------------------------------------

namespace {

constexpr uint64_t kFnvOffset = 1469598103934665603ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

inline uint64_t fnv(uint64_t h, const void* p, size_t n) {
  const unsigned char* b = static_cast<const unsigned char*>(p);
  for (size_t i = 0; i < n; ++i) {
    h ^= b[i];
    h *= kFnvPrime;
  }
  return h;
}

// FNV-1a of three byte strings of equal length at once: the same three
// results as three separate passes, with three independent multiply chains in
// flight (the byte-serial hash is latency bound, about 1 GB/s per chain).
inline void fnv3(uint64_t h[3], const void* p0, const void* p1, const void* p2, size_t n) {
  const unsigned char* a = static_cast<const unsigned char*>(p0);
  const unsigned char* b = static_cast<const unsigned char*>(p1);
  const unsigned char* c = static_cast<const unsigned char*>(p2);
  uint64_t x = h[0], y = h[1], z = h[2];
  for (size_t i = 0; i < n; ++i) {
    x = (x ^ a[i]) * kFnvPrime;
    y = (y ^ b[i]) * kFnvPrime;
    z = (z ^ c[i]) * kFnvPrime;
  }
  h[0] = x;
  h[1] = y;
  h[2] = z;
}

inline uint64_t fnv_i64(uint64_t h, int64_t x) {
  unsigned char b[8];
  for (int i = 0; i < 8; ++i) b[i] = (unsigned char)((uint64_t)x >> (8 * i));  // little-endian bytes
  return fnv(h, b, 8);
}

}  // namespace

extern "C" uint64_t zero_plan_hash(const zero_plan_t* p) {
  if (!p) return 0;
  uint64_t h = kFnvOffset;
  h = fnv_i64(h, p->world);
  h = fnv_i64(h, (int64_t)p->numel.size());
  for (int64_t n : p->numel) h = fnv_i64(h, n);
  h = fnv_i64(h, (int64_t)p->buckets.size());
  for (const auto& b : p->buckets) {
    h = fnv_i64(h, b.numel);
    h = fnv_i64(h, b.shard);
    h = fnv_i64(h, b.count);
  }
  return h;
}

// ---------------------------------------------------------------------------
// checkpoints
// ---------------------------------------------------------------------------

namespace {

constexpr size_t kHeader = 128;
constexpr uint32_t kVersion = 1;
constexpr int64_t kChunk = int64_t(1) << 21;  // elements per staging chunk (a multiple of the state tile)
static_assert(kChunk % zk::kStateTile == 0, "chunks hold whole tiles");

void put_u32(unsigned char* h, size_t off, uint32_t x) {
  for (int i = 0; i < 4; ++i) h[off + i] = (unsigned char)(x >> (8 * i));
}
void put_u64(unsigned char* h, size_t off, uint64_t x) {
  for (int i = 0; i < 8; ++i) h[off + i] = (unsigned char)(x >> (8 * i));
}
uint32_t get_u32(const unsigned char* h, size_t off) {
  uint32_t x = 0;
  for (int i = 0; i < 4; ++i) x |= (uint32_t)h[off + i] << (8 * i);
  return x;
}
uint64_t get_u64(const unsigned char* h, size_t off) {
  uint64_t x = 0;
  for (int i = 0; i < 8; ++i) x |= (uint64_t)h[off + i] << (8 * i);
  return x;
}
void put_f32(unsigned char* h, size_t off, float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  put_u32(h, off, x);
}
float get_f32(const unsigned char* h, size_t off) {
  const uint32_t x = get_u32(h, off);
  float f;
  std::memcpy(&f, &x, 4);
  return f;
}

int hip_fail(const char* fn, const char* what, hipError_t e) {
  return fail(ZERO_EHIP, std::string(fn) + ": " + what + ": " + hipGetErrorString(e));
}

// Pinned host staging: two sets, each master, m, v of one chunk plus their
// tiled form.  Chunk c uses set c % 2, so the copy of one chunk runs while the
// host hashes and writes (or reads and hashes) the other; an event per set
// marks when its copy has finished.  Destruction waits for the stream, so no
// copy is still in flight into or out of freed memory on an error return.
struct Staging {
  float* buf = nullptr;
  hipEvent_t ev[2] = {nullptr, nullptr};
  hipStream_t st = nullptr;
  ~Staging() {
    if (buf) (void)hipStreamSynchronize(st);
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
    if (buf) (void)hipHostFree(buf);
  }
  hipError_t alloc(hipStream_t s) {
    st = s;
    for (hipEvent_t& e : ev) {
      const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipHostMalloc((void**)&buf, 12 * (size_t)kChunk * sizeof(float), 0);
  }
  float* arr(int set, int k) { return buf + (size_t)(set * 6 + k) * kChunk; }
  float* tiles(int set) { return buf + (size_t)(set * 6 + 3) * kChunk; }
};

struct File {
  FILE* f = nullptr;
  ~File() {
    if (f) std::fclose(f);
  }
};

int check_state_args(const char* fn, const zero_plan_t* plan, int32_t rank, const char* path,
                     int32_t layout, const void* master, const void* m, const void* v) {
  if (!plan) return fail(ZERO_EINVAL, std::string(fn) + ": plan is NULL");
  if (!path || !*path) return fail(ZERO_EINVAL, std::string(fn) + ": path is empty");
  if (rank < 0 || rank >= plan->world) return fail(ZERO_EINVAL, std::string(fn) + ": rank out of range");
  if (layout == ZERO_STATE_TILED) {
    if (!master || m || v)
      return fail(ZERO_EINVAL, std::string(fn) + ": the tiled state layout takes master only");
  } else if (layout == ZERO_STATE_SEPARATE) {
    if (!master || !m || !v) return fail(ZERO_EINVAL, std::string(fn) + ": state pointer is NULL");
  } else {
    return fail(ZERO_EINVAL, std::string(fn) + ": unknown state layout");
  }
  const void* ps[3] = {master, m, v};
  for (const void* p : ps)
    if (p && (reinterpret_cast<uintptr_t>(p) & 15) != 0)
      return fail(ZERO_EALIGN, std::string(fn) + ": state arrays must be 16-byte aligned");
  return ZERO_OK;
}

}  // namespace

extern "C" int zero_checkpoint_save(const zero_plan_t* plan, int32_t rank, const char* path,
                                    int32_t state_layout, const float* master, const float* m,
                                    const float* v, const zero_ckpt_meta_t* meta, void* stream) {
  const char* fn = "zero_checkpoint_save";
  int rc = check_state_args(fn, plan, rank, path, state_layout, master, m, v);
  if (rc) return rc;
  if (!meta) return fail(ZERO_EINVAL, std::string(fn) + ": meta is NULL");
  {
    const zero_scaler_t& c = meta->scaler;
    if (meta->step < 0 || !(c.scale >= 0.0f && std::isfinite(c.scale)) ||
        !(c.growth_factor > 1.0f && std::isfinite(c.growth_factor)) ||
        !(c.backoff_factor > 0.0f && c.backoff_factor < 1.0f) || c.growth_interval < 1 || c.growth_tracker < 0 ||
        c.growth_tracker >= c.growth_interval)
      return fail(ZERO_EINVAL, std::string(fn) + ": inconsistent step or loss-scale state");
  }
  const int64_t S = plan->shard;
  const bool tiled = state_layout == ZERO_STATE_TILED;
  hipStream_t st = (hipStream_t)stream;

  Staging stg;
  if (stg.alloc(st) != hipSuccess || !stg.buf) return fail(ZERO_ENOMEM, std::string(fn) + ": pinned staging");
  const std::string tmp = std::string(path) + ".tmp";
  File out;
  out.f = std::fopen(tmp.c_str(), "wb");
  if (!out.f) return fail(ZERO_EIO, std::string(fn) + ": cannot create " + tmp);
  unsigned char h[kHeader] = {};
  if (std::fwrite(h, 1, kHeader, out.f) != kHeader) return fail(ZERO_EIO, std::string(fn) + ": write failed");

  // payload: master, m, v regions; chunks of kChunk elements of all three at
  // once, the copy of chunk c + 1 in flight while chunk c is hashed and written
  uint64_t sum[3] = {kFnvOffset, kFnvOffset, kFnvOffset};
  const float* src[3] = {master, m, v};
  const int64_t nchunks = (S + kChunk - 1) / kChunk;
  auto issue = [&](int64_t c) -> hipError_t {  // chunk c: device -> staging set c % 2
    const int set = (int)(c & 1);
    const int64_t j0 = c * kChunk, n = (S - j0 < kChunk) ? S - j0 : kChunk;
    hipError_t e = hipSuccess;
    if (tiled) {
      const int64_t t0 = j0 / zk::kStateTile, nt = (n + zk::kStateTile - 1) / zk::kStateTile;
      e = hipMemcpyAsync(stg.tiles(set), master + t0 * 3 * zk::kStateTile,
                         (size_t)nt * 3 * zk::kStateTile * sizeof(float), hipMemcpyDeviceToHost, st);
    } else {
      for (int k = 0; k < 3 && e == hipSuccess; ++k)
        e = hipMemcpyAsync(stg.arr(set, k), src[k] + j0, (size_t)n * sizeof(float), hipMemcpyDeviceToHost, st);
    }
    return e == hipSuccess ? hipEventRecord(stg.ev[set], st) : e;
  };
  if (nchunks > 0) {
    const hipError_t e = issue(0);
    if (e != hipSuccess) return hip_fail(fn, "copy to host", e);
  }
  for (int64_t c = 0; c < nchunks; ++c) {
    const int set = (int)(c & 1);
    const int64_t j0 = c * kChunk, n = (S - j0 < kChunk) ? S - j0 : kChunk;
    // set (c + 1) % 2 was last used by chunk c - 1, which is written already
    hipError_t e = c + 1 < nchunks ? issue(c + 1) : hipSuccess;
    if (e == hipSuccess) e = hipEventSynchronize(stg.ev[set]);
    if (e != hipSuccess) return hip_fail(fn, "copy to host", e);
    if (tiled) {
      const float* tb = stg.tiles(set);
      for (int64_t i = 0; i < n; ++i) {
        const int64_t t = i / zk::kStateTile, r = i % zk::kStateTile;
        for (int k = 0; k < 3; ++k) stg.arr(set, k)[i] = tb[(t * 3 + k) * zk::kStateTile + r];
      }
    }
    fnv3(sum, stg.arr(set, 0), stg.arr(set, 1), stg.arr(set, 2), (size_t)n * sizeof(float));
    for (int k = 0; k < 3; ++k) {
      const long long off = (long long)kHeader + ((long long)k * S + j0) * (long long)sizeof(float);
      if (fseeko(out.f, (off_t)off, SEEK_SET) != 0 ||
          std::fwrite(stg.arr(set, k), sizeof(float), (size_t)n, out.f) != (size_t)n)
        return fail(ZERO_EIO, std::string(fn) + ": write failed (" + tmp + ")");
    }
  }

  std::memcpy(h, "ZEROSHD1", 8);
  put_u32(h, 8, kVersion);
  put_u32(h, 12, (uint32_t)kHeader);
  put_u64(h, 16, zero_plan_hash(plan));
  put_u32(h, 24, (uint32_t)plan->world);
  put_u32(h, 28, (uint32_t)rank);
  put_u64(h, 32, (uint64_t)S);
  put_u64(h, 40, (uint64_t)meta->step);
  put_f32(h, 48, meta->scaler.scale);
  put_u32(h, 52, (uint32_t)meta->scaler.growth_tracker);
  put_f32(h, 56, meta->scaler.growth_factor);
  put_f32(h, 60, meta->scaler.backoff_factor);
  put_u32(h, 64, (uint32_t)meta->scaler.growth_interval);
  for (int k = 0; k < 3; ++k) put_u64(h, 72 + 8 * k, sum[k]);
  if (fseeko(out.f, 0, SEEK_SET) != 0 || std::fwrite(h, 1, kHeader, out.f) != kHeader ||
      std::fflush(out.f) != 0)
    return fail(ZERO_EIO, std::string(fn) + ": write failed (" + tmp + ")");
  const int closed = std::fclose(out.f);
  out.f = nullptr;
  if (closed != 0 || std::rename(tmp.c_str(), path) != 0)
    return fail(ZERO_EIO, std::string(fn) + ": cannot replace " + path);
  return ZERO_OK;
}

extern "C" int zero_checkpoint_load(const zero_plan_t* plan, int32_t rank, const char* path,
                                    int32_t state_layout, float* master, float* m, float* v,
                                    zero_ckpt_meta_t* meta, void* stream) {
  const char* fn = "zero_checkpoint_load";
  int rc = check_state_args(fn, plan, rank, path, state_layout, master, m, v);
  if (rc) return rc;
  if (!meta) return fail(ZERO_EINVAL, std::string(fn) + ": meta is NULL");
  const int64_t S = plan->shard;
  const bool tiled = state_layout == ZERO_STATE_TILED;
  hipStream_t st = (hipStream_t)stream;

  File in;
  in.f = std::fopen(path, "rb");
  if (!in.f) return fail(ZERO_EIO, std::string(fn) + ": cannot open " + path);
  unsigned char h[kHeader];
  if (std::fread(h, 1, kHeader, in.f) != kHeader) return fail(ZERO_EIO, std::string(fn) + ": short header");
  if (std::memcmp(h, "ZEROSHD1", 8) != 0 || get_u32(h, 8) != kVersion || get_u32(h, 12) != kHeader)
    return fail(ZERO_EIO, std::string(fn) + ": not a shard checkpoint of this version");
  if (get_u64(h, 16) != zero_plan_hash(plan) || (int32_t)get_u32(h, 24) != plan->world ||
      (int64_t)get_u64(h, 32) != S)
    return fail(ZERO_EINVAL, std::string(fn) + ": the file was written for another plan");
  {
    const float sc = get_f32(h, 48), gf = get_f32(h, 56), bf = get_f32(h, 60);
    const int32_t tr = (int32_t)get_u32(h, 52), gi = (int32_t)get_u32(h, 64);
    if (!(sc >= 0.0f && std::isfinite(sc)) || !(gf > 1.0f && std::isfinite(gf)) || !(bf > 0.0f && bf < 1.0f) ||
        gi < 1 || tr < 0 || tr >= gi || get_u32(h, 68) != 0 || (int64_t)get_u64(h, 40) < 0)
      return fail(ZERO_EIO, std::string(fn) + ": corrupt header (step or loss-scale fields)");
  }
  if ((int32_t)get_u32(h, 28) != rank)
    return fail(ZERO_EINVAL, std::string(fn) + ": the file holds rank " + std::to_string(get_u32(h, 28)) +
                                 "'s shard");
  if (fseeko(in.f, 0, SEEK_END) != 0 ||
      (long long)ftello(in.f) != (long long)kHeader + 3LL * S * (long long)sizeof(float))
    return fail(ZERO_EIO, std::string(fn) + ": file size does not match the shard");

  const int64_t nchunks = (S + kChunk - 1) / kChunk;
  // Pass 1, host only and read only: the checksums are verified before
  // anything reaches the device, so a corrupt file leaves the caller's state
  // as it was.
  {
    const size_t len = (size_t)(S < kChunk ? S : kChunk);
    std::vector<float> buf;
    try {
      buf.resize(3 * len);
    } catch (const std::bad_alloc&) {
      return fail(ZERO_ENOMEM, std::string(fn) + ": host buffer");
    }
    uint64_t sum[3] = {kFnvOffset, kFnvOffset, kFnvOffset};
    for (int64_t c = 0; c < nchunks; ++c) {
      const int64_t j0 = c * kChunk, n = (S - j0 < kChunk) ? S - j0 : kChunk;
      for (int k = 0; k < 3; ++k) {
        const long long off = (long long)kHeader + ((long long)k * S + j0) * (long long)sizeof(float);
        if (fseeko(in.f, (off_t)off, SEEK_SET) != 0 ||
            std::fread(buf.data() + k * len, sizeof(float), (size_t)n, in.f) != (size_t)n)
          return fail(ZERO_EIO, std::string(fn) + ": read failed");
      }
      fnv3(sum, buf.data(), buf.data() + len, buf.data() + 2 * len, (size_t)n * sizeof(float));
    }
    for (int k = 0; k < 3; ++k)
      if (sum[k] != get_u64(h, 72 + 8 * k))
        return fail(ZERO_EIO, std::string(fn) + ": checksum mismatch (nothing was copied to the device)");
  }
  Staging stg;
  if (stg.alloc(st) != hipSuccess || !stg.buf) return fail(ZERO_ENOMEM, std::string(fn) + ": pinned staging");
  // Pass 2: the copy to the device (hashed again, in case the file changed
  // between the passes).
  uint64_t sum[3] = {kFnvOffset, kFnvOffset, kFnvOffset};
  float* dst[3] = {master, m, v};
  for (int64_t c = 0; c < nchunks; ++c) {
    const int set = (int)(c & 1);
    const int64_t j0 = c * kChunk, n = (S - j0 < kChunk) ? S - j0 : kChunk;
    // this set's staging was last used by the copy of chunk c - 2: wait for it
    if (c >= 2) {
      const hipError_t e = hipEventSynchronize(stg.ev[set]);
      if (e != hipSuccess) return hip_fail(fn, "copy to device", e);
    }
    for (int k = 0; k < 3; ++k) {
      const long long off = (long long)kHeader + ((long long)k * S + j0) * (long long)sizeof(float);
      if (fseeko(in.f, (off_t)off, SEEK_SET) != 0 ||
          std::fread(stg.arr(set, k), sizeof(float), (size_t)n, in.f) != (size_t)n)
        return fail(ZERO_EIO, std::string(fn) + ": read failed");
    }
    fnv3(sum, stg.arr(set, 0), stg.arr(set, 1), stg.arr(set, 2), (size_t)n * sizeof(float));
    hipError_t e = hipSuccess;
    if (tiled) {
      // whole tiles in one copy; a partial last tile (the shard's end) as its
      // three valid runs, so nothing past S is written
      const int64_t T = zk::kStateTile;
      const int64_t t0 = j0 / T, nfull = n / T, rest = n % T;
      float* tb = stg.tiles(set);
      for (int64_t t = 0; t < nfull + (rest ? 1 : 0); ++t)
        for (int k = 0; k < 3; ++k)
          for (int64_t r = 0; r < T; ++r) {
            const int64_t i = t * T + r;
            tb[(t * 3 + k) * T + r] = i < n ? stg.arr(set, k)[i] : 0.0f;
          }
      if (nfull > 0)
        e = hipMemcpyAsync(master + t0 * 3 * T, tb, (size_t)nfull * 3 * T * sizeof(float), hipMemcpyHostToDevice,
                           st);
      for (int k = 0; k < 3 && rest && e == hipSuccess; ++k)
        e = hipMemcpyAsync(master + ((t0 + nfull) * 3 + k) * T, tb + (nfull * 3 + k) * T,
                           (size_t)rest * sizeof(float), hipMemcpyHostToDevice, st);
    } else {
      for (int k = 0; k < 3 && e == hipSuccess; ++k)
        e = hipMemcpyAsync(dst[k] + j0, stg.arr(set, k), (size_t)n * sizeof(float), hipMemcpyHostToDevice, st);
    }
    if (e == hipSuccess) e = hipEventRecord(stg.ev[set], st);
    if (e != hipSuccess) return hip_fail(fn, "copy to device", e);
  }
  {
    const hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(fn, "copy to device", e);
  }
  for (int k = 0; k < 3; ++k)
    if (sum[k] != get_u64(h, 72 + 8 * k))
      return fail(ZERO_EIO, std::string(fn) + ": the file changed while it was loaded (the device state is "
                                              "now undefined)");
  meta->step = (int64_t)get_u64(h, 40);
  meta->scaler.scale = get_f32(h, 48);
  meta->scaler.growth_tracker = (int32_t)get_u32(h, 52);
  meta->scaler.growth_factor = get_f32(h, 56);
  meta->scaler.backoff_factor = get_f32(h, 60);
  meta->scaler.growth_interval = (int32_t)get_u32(h, 64);
  return ZERO_OK;
}
