/*
 * zero_shard.h - one data-parallel rank's sharded optimizer step (ZeRO stages 1/2) on MI355X.
 *
 * The operation: a flattened, padded parameter space is split evenly over Nd data-parallel ranks;
 * each rank keeps only its shard of the Adam state (fp32 parameter copy, m, v: 12 bytes per
 * parameter), reduces the gradient for its shard only, updates its own parameters, and hands the
 * 16-bit result to an all-gather that rebuilds the full parameter buffer on every rank.
 * Sources, cited by page title and section (P1..P3 below):
 *   P1 "ZeRO 优化器的三个阶段深度对比：显存节省与通信开销的量化分析" (wmrh.cn), sections 一 to 四;
 *   P2 "ZeRO 优化器：把显存“分”着用" (5688vip.com), ZeRO Stage 1 to 3 and ZeRO-Offload;
 *   P3 "ZeRO Optimization（零冗余优化）" (ai-master.cc glossary), core-operations and stages lists.
 * The pages print no update equations and say nothing about loss scaling, overflow or clipping;
 * the exact arithmetic below is this library's reading and is spelled out per entry point.
 *
 * Conventions for every entry point:
 *   - Plain C ABI: sizes are element counts (uint64_t); pointers named d_* or documented as device
 *     pointers must be device memory of the current HIP device; everything else is host memory.
 *   - Ownership: the caller allocates and frees every buffer. No entry point allocates memory except
 *     zero_arena_alloc, which exists to be asked for it; the library keeps no state except a
 *     thread-local error message.
 *   - Streams: device work is enqueued on `stream` (a hipStream_t, NULL = the null stream) and
 *     never synchronised, except where an entry point says otherwise; device outputs are valid once
 *     the stream reaches that point.
 *   - Errors: arguments are checked before any device work; on a bad argument nothing is launched
 *     and nothing is written. A failed launch returns ZERO_E_HIP. Details: zero_last_error().
 *   - n == 0 is valid and enqueues nothing (except where stated); arrays of length 0 may be NULL.
 *   - Results are deterministic: a given input and size always produces the same bits.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_MAX_REPLICAS 64   /* gradient replicas one call can sum */
#define ZERO_MAX_SHARDS 64     /* rank shards one gather can read */

typedef enum {
  ZERO_OK = 0,
  ZERO_E_INVAL = 1,       /* a null, out-of-range, aliased or inconsistent argument */
  ZERO_E_OVERFLOW = 2,    /* a size or byte count does not fit in 64 bits */
  ZERO_E_UNSUPPORTED = 3, /* a valid but unimplemented combination (e.g. fp32 parameter output) */
  ZERO_E_HIP = 4          /* the HIP runtime reported an error */
} zero_status;

typedef enum { ZERO_F32 = 0, ZERO_F16 = 1, ZERO_BF16 = 2 } zero_dtype;

typedef enum {
  ZERO_ADAMW = 0,   /* decoupled decay: p *= (1 - lr*wd) before the Adam step */
  ZERO_ADAM_L2 = 1  /* L2 decay: g += wd*p before the moments */
} zero_wd_mode;

/* Partition of N flat elements over nd ranks. */
typedef struct {
  uint64_t n;           /* real element count N */
  uint64_t padded_n;    /* P = shard_elems * nd */
  uint64_t shard_elems; /* S: elements per rank, padding included */
  uint64_t pad;         /* P - N, all at the tail of the flat space */
  uint32_t nd;          /* data-parallel degree */
  uint32_t align_elems; /* S is a multiple of this */
} zero_plan;

/* A gradient source: `count` equally typed device arrays, each at least n elements, summed in
 * ascending index order. `ptrs` is a host array of device pointers. Replicas may alias each other. */
typedef struct {
  const void* const* ptrs;
  uint32_t count;  /* 1 .. ZERO_MAX_REPLICAS */
  int32_t dtype;   /* zero_dtype */
} zero_grad_src;

/* Adam hyper-parameters, fp64 on the host; `step` is t >= 1 counting this step. */
typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
  int32_t wd_mode; /* zero_wd_mode */
  int32_t reserved;
  int64_t step;
} zero_adam_hparams;

/* fp32 step constants the kernels use, each rounded once from fp64 (see zero_adam_derive). */
typedef struct {
  float b1, b2;  /* beta1, beta2 */
  float c1, c2;  /* 1 - beta1, 1 - beta2 */
  float ss;      /* lr / (1 - beta1^t) */
  float bc;      /* sqrt(1 - beta2^t) */
  float e;       /* eps */
  float dec;     /* 1 - lr*wd */
  float w;       /* wd */
} zero_adam_scalars;

/* Even contiguous partition (P1 section 二; P3 stages list: each rank holds 1/Nd of the state).
 * S = align_elems * ceil(ceil(n/nd) / align_elems), P = S*nd, pad = P - n. Rank r owns the flat
 * range [r*S, (r+1)*S); padding sits at the tail; n < nd is allowed (trailing ranks own padding).
 * Host only. Errors: out == NULL, nd == 0 or align_elems == 0 -> ZERO_E_INVAL; P >= 2^64 ->
 * ZERO_E_OVERFLOW. */
zero_status zero_partition_plan(uint64_t n, uint32_t nd, uint32_t align_elems, zero_plan* out);

/* The range of rank `rank`: *begin = rank*S; *valid = min(S, max(0, n - begin)) real elements,
 * the rest of the shard is padding. Host only. Errors: NULL pointers, rank >= nd, or a plan whose
 * fields are inconsistent -> ZERO_E_INVAL. */
zero_status zero_shard_range(const zero_plan* p, uint32_t rank, uint64_t* begin, uint64_t* valid);

/* Per-rank model-state bytes of one stage (P1 sections 一/二: 16-bit parameters and gradients and
 * 12 bytes of Adam state per parameter; DP keeps all whole, ZeRO-1 shards the optimizer state,
 * ZeRO-2 also the gradients, ZeRO-3 also the parameters). A sharded component costs S elements,
 * a whole one N. out[0..3] = optimizer, gradient, parameter, total bytes. stage: 0 = DP, 1..3.
 * Host only. Errors: NULL, stage > 3 -> ZERO_E_INVAL; a byte count >= 2^64 -> ZERO_E_OVERFLOW. */
zero_status zero_stage_bytes(const zero_plan* p, uint32_t stage, uint32_t param_b, uint32_t grad_b,
                             uint32_t opt_b, uint64_t out[4]);

/* Bytes one rank sends per training step under one stage, the communication side of the trade
 * (P1 sections 一/二/三 and P3 stages list: ZeRO-1 and ZeRO-2 send as much as plain data
 * parallelism, about 2N; ZeRO-3 about 1.5 times that, from all-gathering the parameters for the
 * forward and again for the backward). Collectives are read as rings over the plan's padded
 * buffer: one reduce-scatter or all-gather sends (nd - 1) * S elements per rank, an all-reduce
 * twice that. DP all-reduces the gradients; ZeRO-1/2 reduce-scatter the gradients and all-gather
 * the parameters; ZeRO-3 reduce-scatters the gradients and all-gathers the parameters twice.
 * out[0..2] = gradient, parameter, total bytes. stage: 0 = DP, 1..3. Host only. Errors: NULL, an
 * inconsistent plan, stage > 3 -> ZERO_E_INVAL; a byte count >= 2^64 -> ZERO_E_OVERFLOW. */
zero_status zero_stage_comm_bytes(const zero_plan* p, uint32_t stage, uint32_t param_b,
                                  uint32_t grad_b, uint64_t out[3]);

/* The stage-choice rule of P1 section 四 (its decision tree: a card that can hold the whole model
 * takes ZeRO-1, one that can still hold parameters and gradients takes ZeRO-2, otherwise ZeRO-3 with
 * optimizer-state offload advised), read as: the smallest stage of 1..3 whose per-rank bytes
 * (zero_stage_bytes of this plan) are <= usable_bytes, the caller's budget after whatever it keeps
 * for activations and buffers; if none fits, stage 3 with offload_advised = 1. bytes[] is the chosen
 * stage's optimizer, gradient, parameter and total bytes. Host only. Errors: NULL, an inconsistent
 * plan -> ZERO_E_INVAL; a byte count >= 2^64 -> ZERO_E_OVERFLOW. */
typedef struct {
  uint32_t stage;           /* 1, 2 or 3 */
  uint32_t offload_advised; /* 1 when even ZeRO-3 does not fit the budget */
  uint64_t bytes[4];
} zero_stage_choice;

zero_status zero_choose_stage(const zero_plan* p, uint64_t usable_bytes, uint32_t param_b,
                              uint32_t grad_b, uint32_t opt_b, zero_stage_choice* out);

/* Placement of the arrays of one pass in a single device allocation (the "arena"), so that arrays
 * walked at the same element index do not start at addresses the memory interleave maps alike.
 * Not an operation of the pages: it places the rank's shard arrays (P1 section 二: each rank keeps
 * its own shard of parameters, gradients and optimizer state) for bandwidth on this GPU.
 * arrays[i]: bytes (the array's size), hot_offset (byte offset inside the array where the kernel's
 * walk starts, e.g. r*S*2 for rank r's slot inside a gathered 16-bit buffer; else 0), group (arrays
 * a kernel reads or writes at the same element index share a group id; ids are arbitrary) and
 * elem_bytes (2 or 4). Arrays are placed in the given order, each after the previous one ends. An
 * array's granule is its byte size rounded up to a power of two, at least ZERO_ARENA_MIN_GRANULE and
 * at most ZERO_ARENA_GRANULE; the k-th member of a group (counted in that order) gets its hot start
 * at a multiple of its granule plus k * ZERO_ARENA_STAGGER16 (16-bit) or k * ZERO_ARENA_STAGGER32
 * (fp32), modulo the granule.
 * offsets[i] (host, count entries) receives array i's byte offset from the arena start and
 * *total_bytes the size to allocate. Only offsets relative to one allocation matter: any
 * 256-byte-aligned allocation of total_bytes works, and every hot start is then 2 KiB aligned.
 * Host only. Errors: NULL, count 0 or > ZERO_ARENA_MAX_ARRAYS, elem_bytes not 2 or 4, hot_offset or
 * bytes not whole elements or hot_offset > bytes -> ZERO_E_INVAL; a total >= 2^64 ->
 * ZERO_E_OVERFLOW. */
#define ZERO_ARENA_MAX_ARRAYS 256
#define ZERO_ARENA_GRANULE (256ull << 20)
#define ZERO_ARENA_MIN_GRANULE (4ull << 20)
#define ZERO_ARENA_STAGGER16 2048ull
#define ZERO_ARENA_STAGGER32 12288ull
typedef struct {
  uint64_t bytes;
  uint64_t hot_offset;
  uint32_t group;
  uint32_t elem_bytes;
} zero_arena_array;

zero_status zero_arena_layout(const zero_arena_array* arrays, uint32_t count, uint64_t* offsets,
                              uint64_t* total_bytes);

/* Device memory for an arena: total_bytes from zero_arena_layout. Asks the device for physically
 * contiguous memory, so that the layout's offsets hold in physical addresses too; if it cannot
 * give that much contiguous memory, makes an ordinary device allocation instead.
 * *d_ptr receives the allocation (NULL for bytes == 0), *contiguous (nullable) 1 or 0 for which
 * kind it is. The caller owns it and releases it with zero_arena_free. These are the library's only
 * allocations; no step allocates. Host call on the current device. Errors: d_ptr NULL ->
 * ZERO_E_INVAL; no device memory of that size -> ZERO_E_HIP. */
zero_status zero_arena_alloc(uint64_t bytes, void** d_ptr, int32_t* contiguous);

/* Releases an allocation of zero_arena_alloc (NULL is a no-op). The device must have finished
 * with it (synchronise first). Errors: a HIP failure -> ZERO_E_HIP. */
zero_status zero_arena_free(void* d_ptr);

/* The fp32 constants of step hp->step of Adam with bias correction (Kingma and Ba's algorithm,
 * with AdamW's decoupled decay: the pages name Adam and its fp32 state, P1 sections 一/二 and P2
 * ZeRO Stage 1, but print no equations), each formed in fp64 and rounded once:
 * b1 = f32(beta1), b2 = f32(beta2), c1 = f32(1-beta1), c2 = f32(1-beta2),
 * ss = f32(lr / (1 - pow(beta1, t))), bc = f32(sqrt(1 - pow(beta2, t))), e = f32(eps),
 * dec = f32(1 - lr*wd), w = f32(wd). Host only. Errors: NULL, step < 1, beta outside [0, 1),
 * non-finite or negative lr/eps/wd, unknown wd_mode -> ZERO_E_INVAL. */
zero_status zero_adam_derive(const zero_adam_hparams* hp, zero_adam_scalars* out);

/* The constants of steps t = 1..count (the same algorithm as zero_adam_derive, whose passages it
 * follows): out[t-1] is zero_adam_derive's result for hp with step = t
 * (hp->step is ignored), bit for bit. A table for zero_adam_shard_step_dev_t, copied to the device
 * by the caller. Host only. Errors: NULL, count == 0, or hyper-parameters zero_adam_derive rejects
 * -> ZERO_E_INVAL. */
zero_status zero_adam_derive_table(const zero_adam_hparams* hp, uint32_t count,
                                   zero_adam_scalars* out);

/* Length, in doubles, of the squared-norm partials buffer for a shard of n elements:
 * ceil(n / 256) per-tile partials followed by 1024 second-level slots. Host only; never fails. */
uint64_t zero_sq_partials_len(uint64_t n);

/* Reduction half of the gradient reduce-scatter, done over local replicas (P1 section 二; P2 ZeRO
 * Stage 2): acc[i] = rep_0[i] + rep_1[i] + ... in ascending order, fp32 accumulator, each 16-bit
 * replica widened exactly. Optional outputs, any subset but at least one:
 *   out_grad      float[n]: acc. Device memory, or pinned host memory (hipHostMalloc), which the
 *                 kernel then writes over the host link (the offloaded step's direct staging);
 *                 never pageable host memory, which the kernel cannot write (not checked here).
 *   d_nonfinite   device int32: set to 1 if any acc[i] is +-inf or NaN, otherwise left as is
 *                 (so several calls OR into it; the caller zeroes it first).
 *   d_sq_partials device double[zero_sq_partials_len(n)]: entry t (t < ceil(n/256)) receives
 *                 sum over i in [256t, 256t+256) of (double(acc[i]) * sq_scale)^2, each in a fixed
 *                 order that does not depend on alignment; finish with zero_shard_sqnorm(NULL, n).
 * n == 0 enqueues nothing. Aliasing: out_grad and d_sq_partials must not overlap a replica or each
 * other, and d_nonfinite must not lie in a replica, out_grad or the partials. Alignment: every
 * array naturally aligned (fp32 and the flag on 4 bytes, 16-bit on 2, the partials on 8), at any
 * element offset; all take the vector path. Errors: bad source, no output, aliasing, an array not
 * naturally aligned -> ZERO_E_INVAL; n*8 >= 2^64 -> ZERO_E_OVERFLOW. */
zero_status zero_reduce_shard(const zero_grad_src* src, uint64_t n, float* out_grad,
                              int32_t* d_nonfinite, double* d_sq_partials, double sq_scale,
                              void* stream);

/* For callers that cannot allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): zero_reduce_shard with its squared-norm partials kept in a
 * scratch array the library owns, followed by the squared-norm finish of zero_shard_sqnorm, so the
 * caller passes only inputs and outputs. The result equals zero_reduce_shard(src, n, out_grad,
 * d_nonfinite, partials, sq_scale) then zero_shard_sqnorm(NULL, n, sq_scale, partials, d_sq) bit
 * for bit. out_grad (device float[n]) and d_nonfinite (device int32, OR-ed as there) are as in
 * zero_reduce_shard; d_sq (device double, nullable) receives the squared norm. At least one output.
 * The scratch is a static device array of ZERO_STATIC_SQ_PARTIALS doubles (32 MiB) on each GPU the
 * library runs on, held until the process ends; it needs no clearing (every call overwrites what it
 * reads). With d_sq, n may be at most ZERO_STATIC_MAX_ELEMS. It makes no allocation call: its
 * first call on a device looks up that device's copy of the array. All calls on one GPU share the
 * array, so calls that overlap in time on one GPU (other streams, other threads) race on it and
 * must be ordered by the caller. Errors: as zero_reduce_shard; n > ZERO_STATIC_MAX_ELEMS with d_sq,
 * d_sq overlapping a replica or out_grad -> ZERO_E_INVAL; the array's lookup failing -> ZERO_E_HIP. */
#define ZERO_STATIC_SQ_PARTIALS (4u << 20)
#define ZERO_STATIC_MAX_ELEMS (((uint64_t)ZERO_STATIC_SQ_PARTIALS - 1024u) * 256u)
zero_status zero_reduce_shard_static(const zero_grad_src* src, uint64_t n, float* out_grad,
                                     int32_t* d_nonfinite, double sq_scale, double* d_sq,
                                     void* stream);

/* Squared L2 norm of a shard in fp64, for gradient clipping. With d_grad != NULL, first writes the
 * per-tile partials of sum_i (double(d_grad[i]) * sq_scale)^2 into d_partials (as
 * zero_reduce_shard does); with d_grad == NULL, d_partials must already hold them from a
 * zero_reduce_shard call over the same n. Then sums them in a fixed two-level order (contiguous
 * chunks of ceil(tiles/1024) partials, then the chunk sums), using the buffer's last 1024 slots as
 * scratch, and writes the result to *d_out (device double; 0 for n == 0). d_partials holds
 * zero_sq_partials_len(n) doubles. Errors: d_partials or d_out NULL, d_out inside the partials or
 * the gradient, an array not naturally aligned -> ZERO_E_INVAL; n*8 >= 2^64 -> ZERO_E_OVERFLOW. */
zero_status zero_shard_sqnorm(const float* d_grad, uint64_t n, double sq_scale, double* d_partials,
                              double* d_out, void* stream);

/* One Adam/AdamW step on the rank's shard (P1 section 二: each rank updates only its own
 * parameter subset with its own optimizer state; P2 ZeRO Stage 1/2), fused with the gradient
 * reduction and the 16-bit cast into the rank's slot of the gathered buffer:
 *   acc = sum of src replicas (as zero_reduce_shard); g = acc * grad_scale
 *   [L2]    g = g + w*p
 *   m = b1*m + c1*g;  v = b2*v + c2*(g*g);  den = sqrt(v)/bc + e
 *   [AdamW] p = p*dec
 *   p = p - ss*(m/den)
 * every operation fp32, rounded to nearest even, no fused multiply-add, correctly rounded / and
 * sqrt, constants from zero_adam_derive(hp). master, m, v (device float[n]) are updated in place.
 * out_param (device, nullable): element i receives round-to-nearest-even(p[i]) as out_dtype
 * (ZERO_BF16 or ZERO_F16); pass the full gathered buffer plus r*S to write rank r's slot.
 * d_skip (device int32, nullable): when it holds a non-zero value at kernel start, nothing is
 * written (the overflow-skip path: the caller then does not advance t).
 * Aliasing: master, m, v, out_param must not overlap each other, any replica or d_skip.
 * Alignment: every array naturally aligned (fp32 and d_skip on 4 bytes, 16-bit on 2), at any
 * element offset: a slot at an odd element r*S of the gathered buffer (odd S) or replicas that are
 * slices of full-length gradient buffers take the same vector path as aligned ones.
 * Errors: NULLs, bad source, bad hparams, aliasing, an array not naturally aligned ->
 * ZERO_E_INVAL; out_dtype ZERO_F32 -> ZERO_E_UNSUPPORTED; n*8 >= 2^64 -> ZERO_E_OVERFLOW. */
zero_status zero_adam_shard_step(const zero_grad_src* src, uint64_t n, float grad_scale,
                                 float* master, float* m, float* v, const zero_adam_hparams* hp,
                                 void* out_param, int32_t out_dtype, const int32_t* d_skip,
                                 void* stream);

/* The step of zero_adam_shard_step (P1 section 二; P2 ZeRO Stage 1/2) with its grad scale read from
 * device memory: *d_grad_scale (device float) is read once per launch in place of a host
 * grad_scale, as zero_clip_scale writes it. With it the two-pass step (zero_reduce_shard,
 * zero_shard_sqnorm, zero_clip_scale, this call) is enqueued with nothing read back to the host
 * between its passes, and can be captured in a graph.
 * Everything else is as zero_adam_shard_step. Errors: as zero_adam_shard_step, plus d_grad_scale
 * NULL or overlapping master, m, v or out_param -> ZERO_E_INVAL. */
zero_status zero_adam_shard_step_dev_scale(const zero_grad_src* src, uint64_t n,
                                           const float* d_grad_scale, float* master, float* m,
                                           float* v, const zero_adam_hparams* hp, void* out_param,
                                           int32_t out_dtype, const int32_t* d_skip, void* stream);

/* Device status word of zero_adam_shard_step_dev_t: the device step t lay outside its constants
 * table, so the update wrote nothing and t did not advance. */
#define ZERO_DEV_T_OUT_OF_TABLE 1

/* The step of zero_adam_shard_step (P1 section 二; P2 ZeRO Stage 1/2) with its step counter also in
 * device memory, so that a whole training step can be enqueued, or captured in a graph and
 * replayed, without the host supplying t: each update block reads t = *d_step (device int64) and
 * takes its constants from d_table[t-1] (device zero_adam_scalars[table_len], e.g.
 * zero_adam_derive_table's) and the grad scale from *d_grad_scale. A t outside [1, table_len] has
 * no constants: then nothing is written (master, m, v and out_param keep their bits), t does not
 * advance and *d_status (device int32, zeroed by the caller; only ever set, so one check covers
 * many calls or graph replays) receives ZERO_DEV_T_OUT_OF_TABLE. After the update one
 * single-thread kernel on the same stream does that report, or advances *d_step by one, unless
 * d_skip is set (a skipped step does not count). With n == 0 only that kernel is enqueued. wd_mode
 * is the zero_wd_mode the table was derived for. Everything else as zero_adam_shard_step.
 * Errors: as zero_adam_shard_step; NULL d_grad_scale, d_table, d_step or d_status, table_len == 0,
 * an unknown wd_mode, d_step overlapping the table, the grad scale, the flag or a replica, d_status
 * overlapping any array or word of the call, or master, m, v or out_param overlapping any of them
 * -> ZERO_E_INVAL. */
zero_status zero_adam_shard_step_dev_t(const zero_grad_src* src, uint64_t n,
                                       const float* d_grad_scale, const zero_adam_scalars* d_table,
                                       uint32_t table_len, int64_t* d_step, int32_t* d_status,
                                       int32_t wd_mode, float* master, float* m, float* v,
                                       void* out_param, int32_t out_dtype, const int32_t* d_skip,
                                       void* stream);

/* Gradient-clipping scale for the two-pass step, formed on the device. The pages do not clip; this
 * is the usual global-norm rule, with the shard's squared norm standing for the global one:
 *   q = max_norm / (sqrt(*d_sq) + clip_eps)       fp64, each operation correctly rounded
 *   coef = q < 1 ? q : 1                           (a NaN q gives 1)
 *   *d_grad_scale = fp32_rne(coef * inv_loss_scale)
 * d_sq: device double, the squared norm of the unscaled gradient as zero_shard_sqnorm writes it;
 * d_grad_scale: device float, for zero_adam_shard_step_dev_scale. One single-thread kernel on
 * stream; nothing is read back. With the overflow flag set the norm is not finite and the scale
 * is meaningless, but the update it feeds is then skipped.
 * Errors: NULL or overlapping pointers; max_norm or inv_loss_scale not finite and > 0; clip_eps
 * not finite and >= 0 -> ZERO_E_INVAL. */
zero_status zero_clip_scale(const double* d_sq, double max_norm, double clip_eps,
                            double inv_loss_scale, float* d_grad_scale, void* stream);

/* ZeRO-3 parameter gather for one layer (P1 section 三; P2 ZeRO Stage 3; P3 core operations: with
 * parameters sharded, a layer's full parameters are rebuilt from every rank's shard before it runs
 * and the other ranks' parts are released afterwards). The gathered flat space is the nd shards of
 * shard_elems elements laid end to end in rank order (rank r holds [r*S, (r+1)*S), as
 * zero_partition_plan lays it out); d_out (device, count elements) receives its elements
 * [begin, begin + count). d_shards is a host array of nd device pointers, one per rank's shard of
 * elem_bytes-wide elements (2: 16-bit parameters, 4: fp32); only the shards the range touches are
 * read and must be non-NULL. On one GPU the shards are local buffers; across GPUs this is where an
 * all-gather would land. The bytes are copied unchanged. count == 0 enqueues nothing.
 * Errors: NULL array or out, nd outside 1..ZERO_MAX_SHARDS, elem_bytes not 2 or 4, a range past
 * nd*S, out overlapping a shard it reads -> ZERO_E_INVAL; sizes >= 2^64 -> ZERO_E_OVERFLOW. */
zero_status zero_gather_params(const void* const* d_shards, uint32_t nd, uint64_t shard_elems,
                               uint32_t elem_bytes, uint64_t begin, uint64_t count, void* d_out,
                               void* stream);

/* The host half of ZeRO-Offload (P2 ZeRO-Offload: the optimizer state lives in host memory and the
 * CPU updates it): one Adam/AdamW step on host arrays, with exactly the arithmetic, operation order
 * and rounding of zero_adam_shard_step (so both give the same bits), on the fp32 gradient grad
 * (host float[n]) times grad_scale; master, m, v (host float[n]) are updated in place and
 * out_param (host, nullable) receives the bf16/fp16 round-to-nearest-even parameters. threads: host
 * threads to split the range over (0 = all hardware threads). On CPUs with AVX2 and F16C the
 * results are written with streaming stores (to memory, not kept in the caches) when master, m and
 * v share one 32-byte phase (the fastest layout: all three 32-byte aligned). Synchronous; no HIP
 * calls.
 * Errors: NULLs, bad hparams, overlapping arrays -> ZERO_E_INVAL; out dtype fp32 ->
 * ZERO_E_UNSUPPORTED; n*8 >= 2^64 -> ZERO_E_OVERFLOW. */
zero_status zero_host_adam_step(const float* grad, uint64_t n, float grad_scale, float* master,
                                float* m, float* v, const zero_adam_hparams* hp, void* out_param,
                                int32_t out_dtype, uint32_t threads);

/* Staging for zero_offload_step, allocated by the caller. */
typedef struct {
  float* d_grad;        /* device float[2 * chunk_elems]: reduced-gradient chunks, or NULL: the
                           reduce kernel then writes each chunk straight into h_grad over the host
                           link, with no device staging and no copy (h_grad must then be pinned
                           and mapped for the device: checked, ZERO_E_INVAL otherwise) */
  float* h_grad;        /* pinned host float[2 * chunk_elems] (hipHostMalloc, so that the device can
                           write it): the chunks the host updates from */
  void* h_param;        /* pinned host 16-bit [2 * chunk_elems]: updated parameters */
  uint64_t chunk_elems; /* pipeline chunk, >= 1 */
  uint32_t threads;     /* host threads for the update (0 = all) */
  uint32_t reserved;
  void* h2d_stream;     /* stream for the parameter copies back to the GPU (NULL = `stream`) */
  void* events[4];      /* four distinct hipEvent_t made by the caller (timing may be disabled); the
                           call records and waits on them (two per staging buffer) and leaves them */
} zero_offload_buffers;

/* One rank's offloaded step (P2 ZeRO-Offload): for each chunk of the shard, the GPU sums the
 * gradient replicas (as zero_reduce_shard) and the chunk reaches pinned host memory (copied from
 * the device staging, or written there by the kernel when d_grad is NULL); the host
 * runs zero_host_adam_step on its part of h_master/h_m/h_v (host float[n], updated in place) and
 * the 16-bit parameters are copied into d_out_param (device, the rank's slot, out_dtype bf16 or
 * fp16). Chunks are double-buffered: the GPU reduces and copies chunk c+1 while the host updates
 * chunk c, and chunk c's parameters travel back on h2d_stream while the host works on the next.
 * Results equal zero_adam_shard_step's bit for bit. Host-synchronous: returns once every parameter
 * copy has landed. It allocates nothing and creates no HIP objects (the staging and the events are
 * the caller's); its host threads are started once per call and serve every chunk. Aliasing:
 * d_out_param, the staging d_grad and the replicas must not overlap. Errors: as zero_host_adam_step
 * and zero_reduce_shard, plus NULL or incomplete buffers (h_grad or h_param NULL, chunk_elems 0, a
 * NULL or repeated event) or device aliasing -> ZERO_E_INVAL and HIP failures -> ZERO_E_HIP (the state may then be partly updated). */
zero_status zero_offload_step(const zero_grad_src* src, uint64_t n, float grad_scale,
                              float* h_master, float* h_m, float* h_v, const zero_adam_hparams* hp,
                              void* d_out_param, int32_t out_dtype,
                              const zero_offload_buffers* buf, void* stream);

/* Static text for a status code (never NULL). */
const char* zero_status_str(zero_status s);

/* The detail of the last failing call on this thread ("" if none). */
const char* zero_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
