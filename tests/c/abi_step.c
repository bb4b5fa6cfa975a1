/*
 * A plain C consumer of include/zero_shard.h: no Python and no torch.  Device
 * memory and the stream come from the HIP runtime API directly.
 *
 *   abi_step IN_DIR OUT_DIR
 *
 * IN_DIR holds a workload written by tests/test_gpu_c_abi.py:
 *   config.txt   "key value" lines: world rank bucket_cap grad_dtype param_dtype
 *                ld lr beta1 beta2 eps weight_decay step inv_scale max_norm
 *                ntensors, then "numels" followed by ntensors sizes
 *   slices.bin   N gradient slices of the rank's shard, [N, ld] in grad_dtype
 *   master.bin, m.bin, v.bin   fp32 [S]
 *   gather.bin   the full gather buffer, [padded] in param_dtype
 *
 * It runs the two forms of the step on the same inputs and writes
 *   OUT_DIR/fused_{master,m,v,gather}.bin and fused_flag.txt
 *     (zero_adam_step over the slices into separate output state), and
 *   OUT_DIR/clip_{master,m,v,gather}.bin and clip.txt (flag, q, coefficient)
 *     (zero_reduce_shard + zero_shard_norm + zero_adam_step in place), and
 *   OUT_DIR/noalloc_{master,m,v,gather}.bin and noalloc.txt
 *     (the same clipped step with zero_reduce_norm_noalloc, which takes no
 *     workspace, on a copy of the inputs).
 * Exit status 0 on success; on any error the message goes to stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zero_shard.h"

#define HIP_OK(call)                                                                    \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
      exit(2);                                                                          \
    }                                                                                   \
  } while (0)

#define ZERO_OK_OR_DIE(call)                                                            \
  do {                                                                                  \
    int rc_ = (call);                                                                   \
    if (rc_ != ZERO_OK) {                                                               \
      fprintf(stderr, "%s:%d: %s: [%d] %s\n", __FILE__, __LINE__, #call, rc_, zero_last_error()); \
      exit(3);                                                                          \
    }                                                                                   \
  } while (0)

typedef struct {
  int32_t world, rank, grad_dtype, param_dtype, ntensors;
  int64_t bucket_cap, ld, step;
  double lr, beta1, beta2, eps, weight_decay, max_norm;
  float inv_scale;
  int64_t* numels;
} config_t;

static void die(const char* what, const char* path) {
  fprintf(stderr, "%s: %s\n", what, path);
  exit(2);
}

static void read_config(const char* dir, config_t* c) {
  char path[4096], key[64];
  snprintf(path, sizeof path, "%s/config.txt", dir);
  FILE* f = fopen(path, "r");
  if (!f) die("cannot open", path);
  memset(c, 0, sizeof *c);
  while (fscanf(f, "%63s", key) == 1) {
    int ok = 1;
    if (!strcmp(key, "world")) ok = fscanf(f, "%d", &c->world);
    else if (!strcmp(key, "rank")) ok = fscanf(f, "%d", &c->rank);
    else if (!strcmp(key, "bucket_cap")) ok = fscanf(f, "%ld", &c->bucket_cap);
    else if (!strcmp(key, "grad_dtype")) ok = fscanf(f, "%d", &c->grad_dtype);
    else if (!strcmp(key, "param_dtype")) ok = fscanf(f, "%d", &c->param_dtype);
    else if (!strcmp(key, "ld")) ok = fscanf(f, "%ld", &c->ld);
    else if (!strcmp(key, "lr")) ok = fscanf(f, "%lf", &c->lr);
    else if (!strcmp(key, "beta1")) ok = fscanf(f, "%lf", &c->beta1);
    else if (!strcmp(key, "beta2")) ok = fscanf(f, "%lf", &c->beta2);
    else if (!strcmp(key, "eps")) ok = fscanf(f, "%lf", &c->eps);
    else if (!strcmp(key, "weight_decay")) ok = fscanf(f, "%lf", &c->weight_decay);
    else if (!strcmp(key, "step")) ok = fscanf(f, "%ld", &c->step);
    else if (!strcmp(key, "inv_scale")) ok = fscanf(f, "%f", &c->inv_scale);
    else if (!strcmp(key, "max_norm")) ok = fscanf(f, "%lf", &c->max_norm);
    else if (!strcmp(key, "ntensors")) ok = fscanf(f, "%d", &c->ntensors);
    else if (!strcmp(key, "numels")) {
      if (c->ntensors <= 0) die("numels before ntensors in", path);
      c->numels = (int64_t*)calloc((size_t)c->ntensors, sizeof(int64_t));
      for (int i = 0; i < c->ntensors && ok == 1; ++i) ok = fscanf(f, "%ld", &c->numels[i]);
    } else {
      die("unknown key in", path);
    }
    if (ok != 1) die("bad value in", path);
  }
  fclose(f);
  if (!c->numels) die("no numels in", path);
}

static size_t dtype_bytes(int32_t t) { return t == ZERO_F32 ? 4 : 2; }

/* host file -> new device buffer of exactly `bytes` bytes */
static void* load_device(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) die("cannot open", path);
  void* host = malloc(bytes ? bytes : 1);
  if (fread(host, 1, bytes, f) != bytes) die("short read", path);
  fclose(f);
  void* dev = NULL;
  HIP_OK(hipMalloc(&dev, bytes ? bytes : 16));
  HIP_OK(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice));
  free(host);
  return dev;
}

static void save_device(const char* dir, const char* name, const void* dev, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  void* host = malloc(bytes ? bytes : 1);
  HIP_OK(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
  FILE* f = fopen(path, "wb");
  if (!f) die("cannot create", path);
  if (fwrite(host, 1, bytes, f) != bytes) die("short write", path);
  fclose(f);
  free(host);
}

static void* dev_copy(const void* src, size_t bytes) {
  void* dev = NULL;
  HIP_OK(hipMalloc(&dev, bytes ? bytes : 16));
  HIP_OK(hipMemcpy(dev, src, bytes, hipMemcpyDeviceToDevice));
  return dev;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN_DIR OUT_DIR\n", argv[0]);
    return 1;
  }
  const char* in = argv[1];
  const char* out = argv[2];
  config_t c;
  read_config(in, &c);
  printf("%s\n", zero_version());

  zero_plan_t* plan = NULL;
  ZERO_OK_OR_DIE(zero_plan(c.numels, c.ntensors, c.world, c.bucket_cap, &plan));
  const int64_t S = zero_plan_shard_numel(plan);
  const int64_t padded = zero_plan_padded_numel(plan);
  const size_t gb = dtype_bytes(c.grad_dtype), pb = dtype_bytes(c.param_dtype);
  printf("S=%ld padded=%ld N=%d rank=%d\n", (long)S, (long)padded, c.world, c.rank);

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  void* slices = load_device(in, "slices.bin", (size_t)c.world * (size_t)c.ld * gb);
  float* master = (float*)load_device(in, "master.bin", (size_t)S * 4);
  float* m = (float*)load_device(in, "m.bin", (size_t)S * 4);
  float* v = (float*)load_device(in, "v.bin", (size_t)S * 4);
  void* gather = load_device(in, "gather.bin", (size_t)padded * pb);
  void* gather2 = dev_copy(gather, (size_t)padded * pb);
  float *master_o, *m_o, *v_o;
  HIP_OK(hipMalloc((void**)&master_o, (size_t)S * 4 + 16));
  HIP_OK(hipMalloc((void**)&m_o, (size_t)S * 4 + 16));
  HIP_OK(hipMalloc((void**)&v_o, (size_t)S * 4 + 16));
  uint32_t* flag;
  HIP_OK(hipMalloc((void**)&flag, 16));

  /* 1. the fused step: slices in, new state into separate arrays */
  zero_adam_args_t a;
  memset(&a, 0, sizeof a);
  a.rank = c.rank;
  a.grad = slices;
  a.grad_ld = c.ld;
  a.grad_dtype = (zero_dtype_t)c.grad_dtype;
  a.grad_count = 0;
  a.grad_layout = ZERO_GRAD_SHARD;
  a.inv_scale = c.inv_scale;
  a.state_layout = ZERO_STATE_SEPARATE;
  a.master_in = master;
  a.m_in = m;
  a.v_in = v;
  a.master_out = master_o;
  a.m_out = m_o;
  a.v_out = v_o;
  a.gather = gather;
  a.param_dtype = (zero_dtype_t)c.param_dtype;
  a.lr = c.lr;
  a.beta1 = c.beta1;
  a.beta2 = c.beta2;
  a.eps = c.eps;
  a.weight_decay = c.weight_decay;
  a.step = c.step;
  a.overflow_out = flag;
  ZERO_OK_OR_DIE(zero_adam_step(plan, &a, stream));
  HIP_OK(hipStreamSynchronize(stream));
  uint32_t h_flag = 0;
  HIP_OK(hipMemcpy(&h_flag, flag, 4, hipMemcpyDeviceToHost));
  save_device(out, "fused_master.bin", master_o, (size_t)S * 4);
  save_device(out, "fused_m.bin", m_o, (size_t)S * 4);
  save_device(out, "fused_v.bin", v_o, (size_t)S * 4);
  save_device(out, "fused_gather.bin", gather, (size_t)padded * pb);
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/fused_flag.txt", out);
    FILE* f = fopen(path, "w");
    if (!f) die("cannot create", path);
    fprintf(f, "%u\n", h_flag);
    fclose(f);
  }

  /* copies of the inputs for the third form, taken before the second updates in place */
  float* master_n = (float*)dev_copy(master, (size_t)S * 4);
  float* m_n = (float*)dev_copy(m, (size_t)S * 4);
  float* v_n = (float*)dev_copy(v, (size_t)S * 4);
  void* gather3 = dev_copy(gather2, (size_t)padded * pb);

  /* 2. the clipped step: reduce (fp32 g + per-tile partials), norm, update in place */
  float* g = NULL;
  void* ws = NULL;
  double* sumsq = NULL;
  float* coef = NULL;
  HIP_OK(hipMalloc((void**)&g, (size_t)S * 4 + 16));
  HIP_OK(hipMalloc(&ws, zero_workspace_bytes(plan)));
  HIP_OK(hipMalloc((void**)&sumsq, 16));
  HIP_OK(hipMalloc((void**)&coef, 16));
  ZERO_OK_OR_DIE(zero_reduce_shard(plan, c.rank, slices, c.ld, 0, ZERO_GRAD_SHARD, (zero_dtype_t)c.grad_dtype,
                                   c.inv_scale, g, ws, 1, NULL, stream));
  ZERO_OK_OR_DIE(zero_shard_norm(plan, ws, 0.0, c.max_norm, flag, sumsq, coef, stream));
  zero_adam_args_t b = a;
  b.grad = NULL;
  b.g_stash = g;
  b.clip_coef = coef;
  b.master_out = master;
  b.m_out = m;
  b.v_out = v;
  b.gather = gather2;
  b.skip_in = flag;
  b.overflow_out = NULL;
  ZERO_OK_OR_DIE(zero_adam_step(plan, &b, stream));
  HIP_OK(hipStreamSynchronize(stream));
  double h_q = 0.0;
  float h_c = 0.0f;
  HIP_OK(hipMemcpy(&h_flag, flag, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&h_q, sumsq, 8, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&h_c, coef, 4, hipMemcpyDeviceToHost));
  save_device(out, "clip_master.bin", master, (size_t)S * 4);
  save_device(out, "clip_m.bin", m, (size_t)S * 4);
  save_device(out, "clip_v.bin", v, (size_t)S * 4);
  save_device(out, "clip_gather.bin", gather2, (size_t)padded * pb);
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/clip.txt", out);
    FILE* f = fopen(path, "w");
    if (!f) die("cannot create", path);
    fprintf(f, "%u %.17g %.9g\n", h_flag, h_q, (double)h_c);
    fclose(f);
  }

  /* 3. the clipped step again, its first pass without a workspace */
  HIP_OK(hipMemset(g, 0xff, (size_t)S * 4));
  ZERO_OK_OR_DIE(zero_reduce_norm_noalloc(plan, c.rank, slices, c.ld, 0, ZERO_GRAD_SHARD,
                                          (zero_dtype_t)c.grad_dtype, c.inv_scale, g, 0.0, c.max_norm, flag,
                                          sumsq, coef, NULL, stream));
  zero_adam_args_t n = b;
  n.master_in = master_n;
  n.m_in = m_n;
  n.v_in = v_n;
  n.master_out = master_n;
  n.m_out = m_n;
  n.v_out = v_n;
  n.gather = gather3;
  ZERO_OK_OR_DIE(zero_adam_step(plan, &n, stream));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(&h_flag, flag, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&h_q, sumsq, 8, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&h_c, coef, 4, hipMemcpyDeviceToHost));
  save_device(out, "noalloc_master.bin", master_n, (size_t)S * 4);
  save_device(out, "noalloc_m.bin", m_n, (size_t)S * 4);
  save_device(out, "noalloc_v.bin", v_n, (size_t)S * 4);
  save_device(out, "noalloc_gather.bin", gather3, (size_t)padded * pb);
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/noalloc.txt", out);
    FILE* f = fopen(path, "w");
    if (!f) die("cannot create", path);
    fprintf(f, "%u %.17g %.9g\n", h_flag, h_q, (double)h_c);
    fclose(f);
  }

  void* bufs[] = {slices, master, m, v, gather, gather2, master_o, m_o, v_o, flag, g, ws, sumsq, coef,
                  master_n, m_n, v_n, gather3};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
  HIP_OK(hipStreamDestroy(stream));
  zero_plan_free(plan);
  free(c.numels);
  printf("ok\n");
  return 0;
}
