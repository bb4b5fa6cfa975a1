/*
 * zero_shard.h — C ABI of one rank's sharded mixed-precision Adam/AdamW step
 * (ZeRO-DP stage 1/2: optimizer states P_os, + gradients P_os+g) on MI355X.
 *
 * The operation (handbook chapter "ZeRO 与 FSDP：切分优化器状态、梯度与参数",
 * section "从零实现 ZeRO 的 Adam", zero_adam.py): parameters are flattened into
 * one zero-padded vector split into N equal contiguous shards; rank r receives
 * the SUM over ranks of the gradient of its shard (reduce-scatter), divides by
 * N, runs Adam on its fp32 master copy and moments, and the updated shards are
 * all-gathered back into full parameters.  Mixed precision ("PaddlePaddle
 * ZeRO优化…", section "混合精度才是最佳拍档"; "论文专题讲解：ZeRO…", section
 * "显存账") adds 16-bit gradients and parameters, loss-scale unscaling and a
 * skipped step when a gradient overflows.
 *
 * On one GPU the reduce-scatter's input is emulated by N gradient slices of the
 * rank's shard held in device memory (slice k = rank k's gradient of this shard);
 * the step writes the rank's new 16-bit parameters into its slots of the full
 * gather buffer, which is the payload an all-gather would move.
 *
 * Conventions shared by every call:
 *  - All functions return ZERO_OK (0) or a negative ZERO_E* code and never
 *    throw.  On an error nothing is enqueued and no memory is written; the
 *    message is available from zero_last_error() on the calling thread.
 *  - Device pointers are plain device addresses owned by the caller.  The
 *    library never allocates device memory.  The plan is host memory owned by
 *    the library (zero_plan ... zero_plan_free).
 *  - Device work is enqueued on the caller's stream `stream` (a hipStream_t;
 *    NULL = the null stream) and is asynchronous: flags, norms and coefficients
 *    land in device memory and are read by the caller after its own sync.
 *  - "Local" arrays have the rank's shard length S = zero_plan_shard_numel():
 *    the rank's pieces of every bucket, concatenated in bucket order.  They must
 *    be 16-byte aligned (ZERO_EALIGN otherwise).  The gather buffer needs only
 *    element alignment.
 *  - Floating point: every operation of the step is one IEEE fp32 rounding (no
 *    contraction into fused multiply-add, correctly rounded division and square
 *    root, denormals kept); 16-bit results are rounded to nearest, ties to even.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ZERO_OK = 0,
  ZERO_EINVAL = -1, /* bad argument: null pointer, range, dtype, aliasing, size */
  ZERO_EALIGN = -2, /* a local array or slice is not 16-byte aligned */
  ZERO_ENOMEM = -3, /* host allocation failed */
  ZERO_EHIP = -4,   /* the HIP runtime reported an error (code in the message) */
  ZERO_EIO = -5     /* a checkpoint file could not be written or read, or is corrupt */
};

typedef enum { ZERO_F32 = 0, ZERO_BF16 = 1, ZERO_F16 = 2 } zero_dtype_t;

/*
 * Layout of the fp32 optimizer state (master, m, v) of a rank's shard.
 *  ZERO_STATE_SEPARATE: three arrays of S elements.
 *  ZERO_STATE_TILED:    one buffer of ceil(S / 2048) tiles; tile t holds
 *                       master[2048 t .. 2048 t + 2047], then m, then v of the
 *                       same elements (6144 floats).  The three state streams
 *                       become one read and one write stream, which the HBM
 *                       serves measurably faster than six.  Positions past S
 *                       in the last tile are never read or written.
 */
typedef enum { ZERO_STATE_SEPARATE = 0, ZERO_STATE_TILED = 1 } zero_state_layout_t;
#define ZERO_STATE_TILE 2048

typedef struct zero_plan zero_plan_t;

/* ------------------------------------------------------------------------ */
/* Planner (host only, exact integer arithmetic)                               */
/* ------------------------------------------------------------------------ */

/*
 * Build the flat layout of `n_tensors` tensors of sizes numel[0..n_tensors-1]
 * (taken in list order) over `world` = N ranks (zero_adam.py: flatten, pad to
 * ceil(numel/N)*N, rank r owns [r*S, (r+1)*S)).
 *
 * bucket_cap <= 0: one bucket, exactly that flat vector.  bucket_cap > 0:
 * tensors are packed greedily in order into buckets (a bucket is closed when the
 * next tensor would take it past the cap; a tensor larger than the cap sits
 * alone), the constant-size buffers of ZeRO-R (C_B); each bucket b of B_b
 * elements is padded to P_b = N * S_b, S_b = ceil(B_b / N), and rank r's piece
 * of it sits at base_b + r * S_b in the gather buffer.
 *
 * numel: host array, each >= 0, sum > 0.  world >= 1.  *out receives the plan.
 * Errors: ZERO_EINVAL (bad sizes), ZERO_ENOMEM.
 */
int zero_plan(const int64_t* numel, int32_t n_tensors, int32_t world, int64_t bucket_cap,
              zero_plan_t** out);

/*
 * Per-parameter dim-0 layout (FSDP2 fully_shard: every parameter a tensor
 * split on its first dimension; handbook chapter "ZeRO 与 FSDP：切分优化器状态、
 * 梯度与参数", section "ZeRO-3 与 FSDP", where a (256, 64) weight on 2 ranks is
 * held as (128, 64) per rank).
 *
 * Parameter i has rows[i] rows of row_numel[i] elements (a 0-d parameter: one
 * row of one element).  Each parameter with elements is its own bucket: its
 * rows are padded to N * c_i, c_i = ceil(rows[i] / N), so S_b = c_i *
 * row_numel[i], P_b = N * S_b, rank r's piece holds rows [r*c_i, (r+1)*c_i),
 * and the bucket in the gather buffer is the padded parameter in row-major
 * order.  A parameter with no elements adds no bucket (it sits, empty, at the
 * end of the previous parameter's bucket, or at the start of the next one).
 * Every other call takes the plan as it takes a zero_plan() plan.
 *
 * rows, row_numel: host arrays, each >= 0, some parameter non-empty.  world >= 1.
 * Errors: ZERO_EINVAL (bad sizes), ZERO_ENOMEM.
 */
int zero_plan_dim0(const int64_t* rows, const int64_t* row_numel, int32_t n_tensors, int32_t world,
                   zero_plan_t** out);

/* Free a plan (NULL is ignored). */
void zero_plan_free(zero_plan_t* plan);

/* Scalars of a plan; -1 for a NULL plan. */
int64_t zero_plan_shard_numel(const zero_plan_t* plan);  /* S = sum_b S_b            */
int64_t zero_plan_total_numel(const zero_plan_t* plan);  /* Psi = sum of numel       */
int64_t zero_plan_padded_numel(const zero_plan_t* plan); /* gather length sum_b P_b  */
int32_t zero_plan_world(const zero_plan_t* plan);
int32_t zero_plan_num_buckets(const zero_plan_t* plan);
int32_t zero_plan_num_tensors(const zero_plan_t* plan);

/* Bucket b: flat base, element count B_b, padded length P_b, shard S_b, and
 * the tensors it holds (first index, count).  Any output pointer may be NULL. */
int zero_plan_bucket(const zero_plan_t* plan, int32_t b, int64_t* base, int64_t* numel,
                     int64_t* padded, int64_t* shard, int32_t* first_tensor, int32_t* n_tensors);

/* Tensor i: its bucket and the flat (gather-buffer) offset of its first element. */
int zero_plan_tensor(const zero_plan_t* plan, int32_t i, int32_t* bucket, int64_t* offset);

/*
 * Rank `rank`'s piece of bucket b: gather_off = base_b + rank*S_b (offset in the
 * gather buffer), local_off (offset in the rank's local arrays), valid =
 * clamp(B_b - rank*S_b, 0, S_b) leading non-padding elements.  Piece length is S_b.
 */
int zero_plan_rank_segment(const zero_plan_t* plan, int32_t rank, int32_t b, int64_t* gather_off,
                           int64_t* local_off, int64_t* valid);

/*
 * Per-device model-state bytes of mixed-precision Adam, K = 12 ("论文专题讲解：ZeRO…",
 * section "ZeRO-DP 三阶段"; handbook section "三个级别"):
 *   stage 0: 16 Psi (plain data parallel); 1: 4 Psi + 12 Psi/N; 2: 2 Psi + 14 Psi/N;
 *   3: 16 Psi / N.
 * formula_bytes gets the formula with the unpadded Psi; padded_bytes the same
 * with N*S for Psi and S for Psi/N (the bytes this layout really holds).
 * The pages' formulas fix 2-byte (fp16) parameters and gradients next to
 * 12 bytes of fp32 optimizer state per parameter, so the call takes no
 * parameter-byte argument: the accounting of other storage types is not on
 * the pages.
 */
int zero_plan_bytes(const zero_plan_t* plan, int32_t stage, double* formula_bytes,
                    int64_t* padded_bytes);

/* ------------------------------------------------------------------------ */
/* Device operations                                                          */
/* ------------------------------------------------------------------------ */

/*
 * fp32 elements of one state buffer in `layout`: S for ZERO_STATE_SEPARATE (per
 * array), 3 * 2048 * ceil(S / 2048) for ZERO_STATE_TILED (the whole buffer;
 * elements past S in the last tile are never read or written).  -1 for a NULL
 * plan or an unknown layout.
 */
int64_t zero_state_numel(const zero_plan_t* plan, int32_t layout);

/*
 * Bytes of device workspace that zero_reduce_shard / zero_shard_norm need: one
 * float64 partial sum and one overflow word per 2048 shard elements (about
 * 6 bytes per 1000 elements) plus 3 KiB for the finalize.  Caller-allocated,
 * 16-byte aligned, no initial content required.  0 for a NULL plan.
 */
size_t zero_workspace_bytes(const zero_plan_t* plan);

/*
 * Optional device piece table, for layouts with many gather pieces per rank
 * (the dim-0 layout of a model with hundreds or thousands of parameters).
 * Without it one launch of the update addresses at most 192 pieces (they
 * travel as kernel arguments), so such a layout takes one launch per 192
 * pieces, and zero_reduce_shard refuses a full-gradient layout with more
 * than 192 pieces inside one 2048-element tile.
 *
 * zero_plan_piece_table_bytes: device bytes of one rank's table, 16 per
 * piece (the plan's bucket count); 0 for a NULL plan.
 *
 * zero_plan_attach_piece_table: writes rank `rank`'s table into `table`
 * (caller-owned device memory, 16-byte aligned, at least `bytes` =
 * zero_plan_piece_table_bytes bytes; a synchronous copy from the host) and
 * attaches it to the plan.  From then on zero_adam_step and zero_reduce_shard
 * for that rank, on the device that was current at the attach, read the
 * pieces from the table: one launch covers the whole shard.  Calls for
 * another rank or device use the kernel-argument form.  The memory must stay
 * allocated and unchanged until the plan is freed or another attach replaces
 * it; table == NULL detaches.  Not thread-safe against concurrent calls that
 * use the same plan.  Errors: ZERO_EINVAL (plan, rank, size), ZERO_EALIGN,
 * ZERO_EHIP.
 */
int64_t zero_plan_piece_table_bytes(const zero_plan_t* plan);
int zero_plan_attach_piece_table(zero_plan_t* plan, int32_t rank, void* table, int64_t bytes);

/*
 * Where the gradient buffers a step reads come from.
 *
 * ZERO_GRAD_SHARD: each buffer is this rank's [S] shard, local index j.  With
 * N buffers they are the N ranks' contributions that the reduce-scatter sums
 * (the fused ZeRO-2 step; handbook chapter "ZeRO 与 FSDP：切分优化器状态、
 * 梯度与参数", section "从零实现 ZeRO 的 Adam", reduce_scatter with SUM); with
 * one buffer it is the stored reduce-scatter output, still the SUM over ranks
 * (ZeRO-2 with the collective run separately: a gradient partition of 2*Psi/N
 * bytes; "论文专题讲解：ZeRO…", section "ZeRO-DP 三阶段").
 * ZERO_GRAD_FULL: each buffer is a whole flat gradient of
 * zero_plan_padded_numel elements in the gather buffer's layout, and the rank
 * reads its pieces at the offsets of its gather slots.  With one buffer this
 * is ZeRO-1 (P_os): gradients all-reduced (SUM) in full on every rank, each
 * rank updating only its partition (the handbook chapter, section "三个级别";
 * "PaddlePaddle ZeRO优化…", section "第一层：只分片优化器状态（ZeRO-1）").
 */
typedef enum zero_grad_layout {
  ZERO_GRAD_SHARD = 0,
  ZERO_GRAD_FULL = 1
} zero_grad_layout_t;

/* Step control kept in device memory (defined with the loss-scale policy below). */
typedef struct zero_step_ctl zero_step_ctl_t;

/*
 * Gradient preparation, first pass of the clipped step (global-norm clipping
 * needs the norm of the whole gradient before any element is updated).
 * The reduction, average and unscale are those of the fused step: the SUM of
 * the reduce-scatter and g /= world of zero_adam.py (handbook chapter "ZeRO 与
 * FSDP：切分优化器状态、梯度与参数", section "从零实现 ZeRO 的 Adam") and
 * GradScaler's unscale ("PaddlePaddle ZeRO优化…", section "混合精度才是最佳
 * 拍档").  Global-norm clipping itself is not described on any of the pages:
 * the sum of squares written here and its use in zero_shard_norm are this
 * library's reading (textbook clipping by the global L2 norm).
 *
 * For every local element j < S, with C = grad_count (0 means N):
 *   acc = buf_0[j] + buf_1[j] + ... + buf_{C-1}[j]           (fp32, ascending k)
 *   g   = (acc / N) * inv_scale                              (zero_adam.py g /= world;
 *                                                             GradScaler unscale)
 * Buffer k starts at grad + k * grad_ld elements (dtype grad_dtype); the
 * stride matters only when C > 1 and must then be a 16-byte multiple at least
 * one buffer long.  grad_layout ZERO_GRAD_SHARD: [S] buffers, 16-byte aligned
 * (C == 1: a stored reduce-scatter output, already summed over the ranks).
 * ZERO_GRAD_FULL: whole flat gradients of zero_plan_padded_numel elements, read
 * at rank `rank`'s gather offsets (ZeRO-1), element aligned; the work is then
 * split into launches over runs of 2048-element tiles that touch at most 192
 * pieces, and a layout with more pieces inside one tile is refused -- unless
 * the rank's piece table is attached (zero_plan_attach_piece_table), which
 * makes it one launch for any layout.  `rank`
 * is used by the full layout only.  If g_out != NULL, g is stored there (fp32,
 * [S], 16-byte aligned).  Per 2048-element tile, an overflow word (any
 * non-finite g) and, if want_sumsq, the float64 sum of g^2 go to `ws`
 * (zero_workspace_bytes).  The partition of elements over tiles depends only
 * on S, so the sums are deterministic run to run (a shard of more than 2^26
 * elements is reduced in consecutive launches of at most 2^26 elements; the
 * partition over tiles is the same).
 * ctl (device zero_step_ctl_t, 8-byte aligned, or NULL): the loss scale is read
 * from it on the device, inv_scale = fp32(1 / ctl->scaler.scale), and the
 * argument inv_scale is ignored (a one-thread launch first writes ctl->k[4];
 * *ctl is not advanced here but by the zero_adam_step that follows).
 * Errors: ZERO_EINVAL (incl. C < 0), ZERO_EALIGN, ZERO_EHIP.
 */
int zero_reduce_shard(const zero_plan_t* plan, int32_t rank, const void* grad, int64_t grad_ld,
                      int32_t grad_count, int32_t grad_layout, zero_dtype_t grad_dtype, float inv_scale,
                      float* g_out, void* ws, int32_t want_sumsq, zero_step_ctl_t* ctl, void* stream);

/*
 * Second pass: finalize what zero_reduce_shard left in `ws` (two small launches:
 * 256 workgroups sum fixed ranges of the per-workgroup partials into `ws`, one
 * workgroup sums those in index order).  The overflow word is GradScaler's
 * inf/NaN check, on which the step is skipped ("PaddlePaddle ZeRO优化…",
 * section "混合精度才是最佳拍档").  The norm and the clip coefficient are not
 * on the pages (they never mention clipping): this is the textbook global-norm
 * clip, c = max_norm / ||g|| when ||g|| exceeds max_norm, with ||g|| taken over
 * the unclipped, unscaled gradient of every rank and the coefficient rounded
 * once to fp32 -- a reading, not a passage of the pages.
 *   overflow_out (device u32): 1 if any g was non-finite, else 0.
 *   q = sum of the partial sums in a fixed order; Q = q + other_ranks_sumsq (the
 *   other ranks' share of the global sum, 0 on one rank); norm = sqrt(Q) (fp64).
 *   sumsq_out (device f64, may be NULL): q.
 *   clip_coef_out (device f32, may be NULL): fp32(max_norm / norm) if
 *   max_norm > 0 and norm > max_norm, else 1.
 * Errors: ZERO_EINVAL, ZERO_EHIP.
 */
int zero_shard_norm(const zero_plan_t* plan, void* ws, double other_ranks_sumsq,
                    double max_norm, uint32_t* overflow_out, double* sumsq_out,
                    float* clip_coef_out, void* stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the two
 * calls above in one, with their workspace in a fixed array inside the
 * library instead of a caller buffer.  Equivalent to
 *   zero_reduce_shard(plan, rank, grad, grad_ld, grad_count, grad_layout,
 *                     grad_dtype, inv_scale, g_out, ws, 1, ctl, stream);
 *   zero_shard_norm(plan, ws, other_ranks_sumsq, max_norm, overflow_out,
 *                   sumsq_out, clip_coef_out, stream);
 * with every argument as documented there, and the same results bit for bit.
 * The array holds ZERO_NOALLOC_SCRATCH_BYTES (4 MiB) on every GPU the library
 * runs on, until the process ends: shards of at most
 * zero_noalloc_max_shard() elements (715,302,912); a larger plan is refused
 * with ZERO_EINVAL before anything is enqueued.  The call allocates no device
 * memory (its first call on a device looks up that device's array).  Every
 * call on one GPU uses that GPU's one array, so calls that overlap in time on
 * one GPU (on different streams, or from several threads) race and give
 * undefined results; calls ordered on one stream are safe.  Nothing in the
 * array needs to start at zero: every call writes each word it reads.
 * Errors: as the two calls, and ZERO_EINVAL for a shard beyond the limit.
 */
#define ZERO_NOALLOC_SCRATCH_BYTES (4 * 1024 * 1024)
int64_t zero_noalloc_max_shard(void);
int zero_reduce_norm_noalloc(const zero_plan_t* plan, int32_t rank, const void* grad, int64_t grad_ld,
                             int32_t grad_count, int32_t grad_layout, zero_dtype_t grad_dtype, float inv_scale,
                             float* g_out, double other_ranks_sumsq, double max_norm, uint32_t* overflow_out,
                             double* sumsq_out, float* clip_coef_out, zero_step_ctl_t* ctl, void* stream);

/* Arguments of zero_adam_step (host struct; pointers are device addresses). */
typedef struct zero_adam_args {
  int32_t rank;              /* 0 <= rank < N                                      */
  /* gradient source: either C gradient buffers summed in the step (fused) ... */
  const void* grad;          /* buffer k at grad + k*grad_ld elements              */
  int64_t grad_ld;           /* elements between buffers (unused when C == 1)     */
  zero_dtype_t grad_dtype;
  int32_t grad_count;        /* C: 0 = N (one per rank); 1 = an already summed one */
  int32_t grad_layout;       /* zero_grad_layout_t                                 */
  float inv_scale;           /* fp32(1 / loss scale); 1 without loss scaling       */
  /* ... or the fp32 gradient written by zero_reduce_shard (then grad is ignored) */
  const float* g_stash;
  const float* clip_coef;    /* device f32 multiplier of g_stash, or NULL (= 1)    */
  /* state (fp32).  ZERO_STATE_SEPARATE: three [S] arrays per side.
   * ZERO_STATE_TILED: master_in / master_out are the tiled buffers
   * (zero_state_numel elements) and m_in, v_in, m_out, v_out must be NULL.   */
  int32_t state_layout;      /* zero_state_layout_t                               */
  const float* master_in;
  const float* m_in;
  const float* v_in;
  float* master_out;
  float* m_out;
  float* v_out;
  /* output: full gather buffer (zero_plan_padded_numel elements); only this
   * rank's pieces are written, every element of them (padding too)          */
  void* gather;
  zero_dtype_t param_dtype;
  /* hyper-parameters (host doubles; rounded once to fp32 inside)               */
  double lr, beta1, beta2, eps, weight_decay;
  int64_t step;              /* 1-based index of this step (t after t += 1)       */
  /* flags (device u32)                                                         */
  const uint32_t* skip_in;   /* NULL, or: nonzero at run time -> state is not written   */
  uint32_t* overflow_out;    /* fused step: 1 if the step was not applied (a non-finite
                                g, or skip_in set), else 0                              */
  /* optional hipEvent_t pair recorded around the update launches only        */
  void* ev_begin;
  void* ev_end;
  /* optional step control in device memory: lr, step and inv_scale above are
   * then ignored and taken from *ctl, which the call advances (see below)      */
  zero_step_ctl_t* ctl;
} zero_adam_args_t;

/*
 * The AdamW update of the rank's shard and the write of its gather slots.
 *
 * Per element (zero_adam.py step() with decoupled weight decay; constants
 * computed in float64 and rounded once to fp32: b1, b2, 1-b1, 1-b2,
 * bc1 = 1-b1^step, bc2 = 1-b2^step, lr, eps, dec = 1-lr*wd):
 *   g      = fused: (sum_{k<C} buffer_k[piece(j)] / N) * inv_scale
 *            stash: g_stash * clip_coef
 *   m'     = b1*m + (1-b1)*g;     v' = b2*v + (1-b2)*(g*g)
 *   m_hat  = m'/bc1;  v_hat = v'/bc2;  u = (lr*m_hat) / (sqrt(v_hat) + eps)
 *   master'= dec*master - u;  gather[slot(j)] = round_to_nearest_even(master')
 *
 * Gradient buffers (zero_grad_layout_t): ZERO_GRAD_SHARD, [S] each, 16-byte
 * aligned, stride grad_ld >= S a 16-byte multiple when C > 1; ZERO_GRAD_FULL,
 * [zero_plan_padded_numel] each, element aligned, stride grad_ld >= that size
 * a 16-byte multiple when C > 1, read at the rank's gather offsets.  The sum
 * is always divided by N, the plan's world size.
 *
 * Overflow handling (GradScaler skips the optimizer step on inf/NaN):
 *  - fused mode: the flag is computed in the same pass over the slices.  The
 *    state outputs must not overlap the inputs (ping-pong buffers; the caller
 *    swaps them only when *overflow_out == 0 after the step).  If the flag is
 *    set, the rank's gather slots are rewritten from master_in before the call's
 *    work completes, so they keep their pre-step values.
 *    With overflow_out == NULL nothing is checked: the update is applied
 *    whatever g holds (non-finite values included), and the state outputs may
 *    then alias the inputs exactly (in place).
 *  - stash mode: the decision is known beforehand (skip_in = zero_shard_norm's
 *    overflow_out), so outputs may alias inputs (in place); overflow_out unused.
 *  - skip_in != NULL and *skip_in != 0 in either mode: the state outputs are
 *    not written; in fused mode with overflow_out, *overflow_out becomes 1 and
 *    the gather slots are rewritten from master_in (in stash mode they are not
 *    touched).
 * ev_begin/ev_end (hipEvent_t or NULL) are recorded on `stream` immediately
 * before and after the update's launches.  A shard of more than 2^26 elements
 * (2^23 with 64 16-bit gradient buffers in the shard layout) is updated in
 * consecutive launches of at most that many elements each, in order on
 * `stream` (large single grids stream measurably slower); the results are the
 * same as one launch's.
 * ctl != NULL (device zero_step_ctl_t, 8-byte aligned): lr, step and
 * inv_scale come from *ctl (t = ctl->step + 1).  The step's fp32 constants are
 * derived from it on the device before the update and it is advanced after the
 * update from the step's flag (overflow_out in fused mode, which is then
 * required; skip_in in stash mode, NULL meaning applied).  This adds no launch
 * to a fused step (the flag reset becomes the constants' launch, the restore
 * pass advances *ctl, and the one-workgroup form for small shards does both
 * itself) and two one-thread launches to a stash-mode step.  In fused mode a
 * step that is not applied also copies the input state to the output arrays,
 * so the output state is current after every call and the caller swaps the
 * buffers unconditionally, without reading the flag.
 * Errors: ZERO_EINVAL (incl. overlapping outputs in fused mode), ZERO_EALIGN,
 * ZERO_EHIP.
 */
int zero_adam_step(const zero_plan_t* plan, const zero_adam_args_t* args, void* stream);

/* ------------------------------------------------------------------------ */
/* Loss-scale policy and sharded checkpoints (host)                           */
/* ------------------------------------------------------------------------ */

/*
 * Dynamic loss scaling around the step.  The pages show GradScaler's
 * scale / step / update calls ("PaddlePaddle ZeRO优化…", section
 * "工程落地中的真实权衡", item "混合精度才是最佳拍档") and the step is
 * skipped on an overflow; the update rule is this library's reading:
 *   overflow:  scale = scale * backoff_factor, growth_tracker = 0
 *   clean:     growth_tracker += 1; when it reaches growth_interval,
 *              scale = scale * growth_factor (kept if that is not finite) and
 *              growth_tracker = 0
 * Products are single fp32 roundings.  The step takes inv_scale =
 * zero_scaler_inv_scale() = fp32(1 / scale).  Plain host struct, caller-owned.
 */
typedef struct zero_scaler {
  float scale;               /* current loss scale                              */
  int32_t growth_tracker;    /* clean steps since the scale last changed        */
  float growth_factor;       /* > 1 (2 by convention)                           */
  float backoff_factor;      /* in (0, 1) (0.5 by convention)                   */
  int32_t growth_interval;   /* >= 1 (2000 by convention)                       */
} zero_scaler_t;

/*
 * Step control in device memory (zero_adam_args_t.ctl; the ctl argument of
 * zero_reduce_shard).  It holds what changes from one step to the next -- the
 * step count, the learning rate and the loss scale -- so that a training loop
 * never waits for the device to learn whether a step was applied: the library
 * computes each step's fp32 constants from it on the device, exactly as the
 * host would (float64, rounded once; bc = 1 - beta^t with t = step + 1), and
 * after the update a one-thread kernel reads the step's flag and advances it
 * (step += 1 when applied, skipped += 1 otherwise, then the zero_scaler_update
 * rule above when `dynamic` is nonzero).  A captured pair of fused steps
 * (state A -> B, then B -> A) can then be replayed for every step of a loop.
 * Caller-owned device memory, 8-byte aligned.  The caller writes every field
 * but k before the first step and may rewrite any of them between steps in
 * stream order (lr for a schedule).  The device fields are not validated:
 * step < 0, a non-finite lr or a scale <= 0 give undefined numbers, never a
 * fault; a scale that has underflowed to 0 makes every step overflow.
 */
struct zero_step_ctl {
  int64_t step;              /* completed steps t; the next applied step uses t + 1 */
  int64_t skipped;           /* steps not applied                                   */
  double lr;                 /* learning rate of the next step                      */
  zero_scaler_t scaler;      /* loss scale (inv_scale = fp32(1 / scale))            */
  int32_t dynamic;           /* nonzero: update the scaler after every step         */
  float k[8];                /* written by the library: bc1, bc2, lr, dec = 1-lr*wd,
                                inv_scale of the last step begun; k[5..7] unused    */
};

/* Set *s to {init_scale, 0, growth_factor, backoff_factor, growth_interval}.
 * Errors: ZERO_EINVAL (NULL, init_scale not finite and > 0, growth_factor <= 1,
 * backoff_factor outside (0, 1), growth_interval < 1). */
int zero_scaler_init(zero_scaler_t* s, float init_scale, float growth_factor, float backoff_factor,
                     int32_t growth_interval);

/* Apply one update after a step whose flag was `overflow` (nonzero = the
 * step was skipped).  Errors: ZERO_EINVAL (NULL). */
int zero_scaler_update(zero_scaler_t* s, int32_t overflow);

/* fp32(1 / scale); 0 for NULL. */
float zero_scaler_inv_scale(const zero_scaler_t* s);

/*
 * 64-bit FNV-1a hash of a plan's layout: world size, the tensor sizes and
 * every bucket's size, shard and tensor count.  Two plans with the same hash
 * place every element at the same local and gather offsets.  0 for NULL.
 */
uint64_t zero_plan_hash(const zero_plan_t* plan);

/* Metadata saved with a shard. */
typedef struct zero_ckpt_meta {
  int64_t step;              /* optimizer steps completed (t)                   */
  zero_scaler_t scaler;      /* loss-scale state                                */
} zero_ckpt_meta_t;

/*
 * Sharded checkpoint: each rank writes only its own shard ("PaddlePaddle
 * ZeRO优化…", section "工程落地中的真实权衡", item 2: save sharded checkpoints,
 * every device its own part, and restore them shard by shard, instead of
 * gathering the full model first).
 *
 * File (little-endian): a 128-byte header, then master[S], m[S], v[S] as
 * fp32 in local order, whatever the device state layout.  Header: bytes 0-7
 * "ZEROSHD1"; u32 version = 1 at 8; u32 header bytes = 128 at 12; u64 plan
 * hash at 16; i32 world at 24; i32 rank at 28; i64 S at 32; i64 step at 40;
 * f32 scale at 48; i32 growth_tracker at 52; f32 growth_factor at 56; f32
 * backoff_factor at 60; i32 growth_interval at 64; u32 0 at 68; u64 FNV-1a
 * of the master, m and v bytes at 72, 80 and 88; zeros to 128.
 *
 * save: meta must be consistent (as checked on load, below).  The state
 * (device pointers, layout as for zero_adam_step: TILED takes
 * master only, m and v NULL) is copied to host on `stream` after the work
 * already queued there, in chunks through pinned host staging, and written to
 * `path` + ".tmp", which then replaces `path`.  Returns after the file is
 * complete.
 * load: checks the header against the plan (hash, world, S) and rank and its
 * step and loss-scale fields for consistency (step >= 0, scale finite and >=
 * 0, growth_factor > 1, backoff_factor in (0, 1), 0 <= growth_tracker <
 * growth_interval), then
 * verifies the three checksums in a read-only pass over the file; only then
 * copies the shard into the device state on `stream` and waits for it.  A
 * corrupt file is refused with ZERO_EIO before anything is copied, leaving the
 * device state as it was (if the file changes between the two passes, the
 * second pass's checksums catch it: ZERO_EIO, device state undefined).  With
 * the tiled layout, positions past S in the last tile are not written.
 * Errors: ZERO_EINVAL (arguments, or a file for another plan or rank),
 * ZERO_EALIGN, ZERO_EIO, ZERO_ENOMEM, ZERO_EHIP.
 */
int zero_checkpoint_save(const zero_plan_t* plan, int32_t rank, const char* path, int32_t state_layout,
                         const float* master, const float* m, const float* v, const zero_ckpt_meta_t* meta,
                         void* stream);
int zero_checkpoint_load(const zero_plan_t* plan, int32_t rank, const char* path, int32_t state_layout,
                         float* master, float* m, float* v, zero_ckpt_meta_t* meta, void* stream);

/*
 * A plain streaming copy of `bytes` bytes from src to dst (device pointers,
 * both 16-byte aligned, bytes a multiple of 16, no overlap), with the step's
 * own load and store forms (non-temporal 16-byte vectors, one-shot grid).  It
 * is the practical bandwidth ceiling the step's kernels are measured against
 * besides the published HBM peak: one read and one write stream, nothing
 * else.  Enqueued on `stream`.  Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_EHIP.
 */
int zero_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);

/* Message of the last error on this thread ("" if none). */
const char* zero_last_error(void);

/* Library version string. */
const char* zero_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
