// Host-only entry points of libzero_shard: the partition plan, per-stage bytes, the fp32 Adam
// constants and the status/error strings. No device code and no HIP calls here.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "zero_fpenv.h"
#include "zero_internal.h"

namespace zero {

static thread_local char g_last_error[512];

zero_status fail(zero_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

zero_status ok() {
  g_last_error[0] = '\0';
  return ZERO_OK;
}

// a*b into *out, false on uint64 overflow.
static bool mul_u64(uint64_t a, uint64_t b, uint64_t* out) {
  return !__builtin_mul_overflow(a, b, out);
}

static bool add_u64(uint64_t a, uint64_t b, uint64_t* out) {
  return !__builtin_add_overflow(a, b, out);
}

static bool plan_consistent(const zero_plan* p) {
  uint64_t prod;
  return p->nd > 0 && p->align_elems > 0 && p->shard_elems % p->align_elems == 0 &&
         mul_u64(p->shard_elems, p->nd, &prod) && prod == p->padded_n && p->padded_n >= p->n &&
         p->pad == p->padded_n - p->n;
}

}  // namespace zero

using namespace zero;

extern "C" {

// Even contiguous split of the flat space: "ZeRO 优化器的三个阶段深度对比", section 二 (each rank
// holds 1/Nd of the state); tail padding and the alignment rounding are this library's reading.
zero_status zero_partition_plan(uint64_t n, uint32_t nd, uint32_t align_elems, zero_plan* out) {
  if (!out) return fail(ZERO_E_INVAL, "zero_partition_plan: out is NULL");
  if (nd == 0) return fail(ZERO_E_INVAL, "zero_partition_plan: nd must be >= 1");
  if (align_elems == 0) return fail(ZERO_E_INVAL, "zero_partition_plan: align_elems must be >= 1");
  // ceil(n / nd) without forming n + nd - 1 (which can wrap)
  const uint64_t per_rank = n / nd + (n % nd != 0);
  const uint64_t groups = per_rank / align_elems + (per_rank % align_elems != 0);
  uint64_t s, p;
  if (!mul_u64(groups, align_elems, &s) || !mul_u64(s, nd, &p))
    return fail(ZERO_E_OVERFLOW, "zero_partition_plan: padded length of n=%llu over nd=%u "
                "(align %u) does not fit in 64 bits", (unsigned long long)n, nd, align_elems);
  out->n = n;
  out->padded_n = p;
  out->shard_elems = s;
  out->pad = p - n;
  out->nd = nd;
  out->align_elems = align_elems;
  return ok();
}

zero_status zero_shard_range(const zero_plan* p, uint32_t rank, uint64_t* begin, uint64_t* valid) {
  if (!p || !begin || !valid) return fail(ZERO_E_INVAL, "zero_shard_range: NULL argument");
  if (!plan_consistent(p)) return fail(ZERO_E_INVAL, "zero_shard_range: inconsistent plan");
  if (rank >= p->nd)
    return fail(ZERO_E_INVAL, "zero_shard_range: rank %u >= nd %u", rank, p->nd);
  const uint64_t b = (uint64_t)rank * p->shard_elems;  // < padded_n, no overflow
  *begin = b;
  *valid = b >= p->n ? 0 : (p->n - b < p->shard_elems ? p->n - b : p->shard_elems);
  return ok();
}

// Per-stage model-state bytes: "ZeRO 优化器的三个阶段深度对比", sections 一 and 二 (16-bit params
// and grads, 12 bytes of Adam state; stage k shards the first k of optimizer state, gradients,
// parameters).
zero_status zero_stage_bytes(const zero_plan* p, uint32_t stage, uint32_t param_b, uint32_t grad_b,
                             uint32_t opt_b, uint64_t out[4]) {
  if (!p || !out) return fail(ZERO_E_INVAL, "zero_stage_bytes: NULL argument");
  if (!plan_consistent(p)) return fail(ZERO_E_INVAL, "zero_stage_bytes: inconsistent plan");
  if (stage > 3) return fail(ZERO_E_INVAL, "zero_stage_bytes: stage %u > 3", stage);
  const uint64_t opt_elems = stage >= 1 ? p->shard_elems : p->n;
  const uint64_t grad_elems = stage >= 2 ? p->shard_elems : p->n;
  const uint64_t param_elems = stage >= 3 ? p->shard_elems : p->n;
  uint64_t o, g, w, t;
  if (!mul_u64(opt_elems, opt_b, &o) || !mul_u64(grad_elems, grad_b, &g) ||
      !mul_u64(param_elems, param_b, &w) || !add_u64(o, g, &t) || !add_u64(t, w, &t))
    return fail(ZERO_E_OVERFLOW, "zero_stage_bytes: byte count does not fit in 64 bits");
  out[0] = o;
  out[1] = g;
  out[2] = w;
  out[3] = t;
  return ok();
}

// Bytes sent per rank per step: "ZeRO 优化器的三个阶段深度对比", sections 一 to 三, and "ZeRO
// Optimization", stages list (ZeRO-1/2 send as much as data parallelism, ZeRO-3 about 1.5 times).
// Ring collectives over the padded plan: one reduce-scatter or all-gather pass sends (nd-1)*S
// elements per rank; each stage is a count of such passes over gradients and parameters.
zero_status zero_stage_comm_bytes(const zero_plan* p, uint32_t stage, uint32_t param_b,
                                  uint32_t grad_b, uint64_t out[3]) {
  if (!p || !out) return fail(ZERO_E_INVAL, "zero_stage_comm_bytes: NULL argument");
  if (!plan_consistent(p)) return fail(ZERO_E_INVAL, "zero_stage_comm_bytes: inconsistent plan");
  if (stage > 3) return fail(ZERO_E_INVAL, "zero_stage_comm_bytes: stage %u > 3", stage);
  // (gradient passes, parameter passes): DP all-reduce = reduce-scatter + all-gather of the
  // gradients; ZeRO-1/2 reduce-scatter gradients, all-gather parameters; ZeRO-3 all-gathers the
  // parameters for the forward and again for the backward
  static const uint32_t kPasses[4][2] = {{2, 0}, {1, 1}, {1, 1}, {1, 2}};
  uint64_t one, g, w, t;
  if (!mul_u64((uint64_t)(p->nd - 1), p->shard_elems, &one) ||
      !mul_u64(one, (uint64_t)kPasses[stage][0] * grad_b, &g) ||
      !mul_u64(one, (uint64_t)kPasses[stage][1] * param_b, &w) || !add_u64(g, w, &t))
    return fail(ZERO_E_OVERFLOW, "zero_stage_comm_bytes: byte count does not fit in 64 bits");
  out[0] = g;
  out[1] = w;
  out[2] = t;
  return ok();
}

// Stage choice: "ZeRO 优化器的三个阶段深度对比", section 四 (the decision tree), read as the
// smallest stage whose per-rank bytes fit the caller's usable budget.
zero_status zero_choose_stage(const zero_plan* p, uint64_t usable_bytes, uint32_t param_b,
                              uint32_t grad_b, uint32_t opt_b, zero_stage_choice* out) {
  if (!p || !out) return fail(ZERO_E_INVAL, "zero_choose_stage: NULL argument");
  uint64_t b[4];
  for (uint32_t stage = 1; stage <= 3; ++stage) {
    const zero_status s = zero_stage_bytes(p, stage, param_b, grad_b, opt_b, b);
    if (s != ZERO_OK) return s;
    if (b[3] <= usable_bytes || stage == 3) {
      out->stage = stage;
      out->offload_advised = b[3] > usable_bytes ? 1u : 0u;
      for (int i = 0; i < 4; ++i) out->bytes[i] = b[i];
      return ok();
    }
  }
  return fail(ZERO_E_INVAL, "zero_choose_stage: unreachable");
}

// Placement of one pass's arrays in a single allocation. Not from the pages: a property of this
// GPU's memory system. Arrays that a kernel walks at the same element index ("lockstep") hit the same
// DRAM channels and banks when their starts agree in the address bits the interleave hashes; the
// fused step then loses up to 5% of its bandwidth. Here every hot start sits on a line of the
// array's granule (its size rounded up to a power of two, from 4 MiB to 256 MiB) past the arena
// start, plus a stagger of k * 2 KiB (16-bit arrays) or k * 12 KiB (fp32 arrays) for the k-th member
// of its lockstep group: the spacing that measured best on the step's kernels.
zero_status zero_arena_layout(const zero_arena_array* arrays, uint32_t count, uint64_t* offsets,
                              uint64_t* total_bytes) {
  const char* fn = "zero_arena_layout";
  if (!arrays || !offsets || !total_bytes) return fail(ZERO_E_INVAL, "%s: NULL argument", fn);
  if (count == 0 || count > ZERO_ARENA_MAX_ARRAYS)
    return fail(ZERO_E_INVAL, "%s: count %u outside 1..%d", fn, count, ZERO_ARENA_MAX_ARRAYS);
  uint32_t seen_group[ZERO_ARENA_MAX_ARRAYS], seen_count[ZERO_ARENA_MAX_ARRAYS];
  uint32_t ngroups = 0;
  uint64_t cursor = 0;
  for (uint32_t i = 0; i < count; ++i) {
    const zero_arena_array& a = arrays[i];
    if (a.elem_bytes != 2 && a.elem_bytes != 4)
      return fail(ZERO_E_INVAL, "%s: array %u: elem_bytes %u is not 2 or 4", fn, i, a.elem_bytes);
    if (a.hot_offset > a.bytes || a.hot_offset % a.elem_bytes != 0 || a.bytes % a.elem_bytes != 0)
      return fail(ZERO_E_INVAL, "%s: array %u: hot_offset %llu / bytes %llu not whole elements inside it",
                  fn, i, (unsigned long long)a.hot_offset, (unsigned long long)a.bytes);
    uint32_t g = 0;
    while (g < ngroups && seen_group[g] != a.group) ++g;
    if (g == ngroups) {
      seen_group[g] = a.group;
      seen_count[g] = 0;
      ++ngroups;
    }
    const uint64_t member = seen_count[g]++;
    uint64_t Q = ZERO_ARENA_MIN_GRANULE;      // the array's granule
    while (Q < a.bytes && Q < ZERO_ARENA_GRANULE) Q <<= 1;
    const uint64_t stagger = a.elem_bytes == 2 ? ZERO_ARENA_STAGGER16 : ZERO_ARENA_STAGGER32;
    const uint64_t delta = (member * stagger) % Q;
    // smallest base >= cursor with base + hot_offset == delta (mod Q)
    const uint64_t target = (delta + Q - a.hot_offset % Q) % Q;
    uint64_t base;
    if (!add_u64(cursor, (target + Q - cursor % Q) % Q, &base) || !add_u64(base, a.bytes, &cursor))
      return fail(ZERO_E_OVERFLOW, "%s: the arena exceeds 2^64 bytes", fn);
    offsets[i] = base;
  }
  *total_bytes = cursor;
  return ok();
}

// The fp32 constants of one Adam step, each rounded once from fp64 (Kingma-Ba bias correction;
// the pages name Adam and its state but print no equations).
zero_status zero_adam_derive(const zero_adam_hparams* hp, zero_adam_scalars* out) {
  if (!hp || !out) return fail(ZERO_E_INVAL, "zero_adam_derive: NULL argument");
  if (hp->step < 1) return fail(ZERO_E_INVAL, "zero_adam_derive: step %lld < 1", (long long)hp->step);
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return fail(ZERO_E_INVAL, "zero_adam_derive: betas must lie in [0, 1)");
  if (!isfinite(hp->lr) || !(hp->eps >= 0.0) || !isfinite(hp->eps) || !(hp->weight_decay >= 0.0) ||
      !isfinite(hp->weight_decay) || hp->lr < 0.0)
    return fail(ZERO_E_INVAL, "zero_adam_derive: lr, eps and weight_decay must be finite and >= 0");
  if (hp->wd_mode != ZERO_ADAMW && hp->wd_mode != ZERO_ADAM_L2)
    return fail(ZERO_E_INVAL, "zero_adam_derive: unknown wd_mode %d", hp->wd_mode);
  const zero::IeeeScope ieee;   // round to nearest, subnormals kept, whatever the caller's mode
  const double t = (double)hp->step;
  out->b1 = (float)hp->beta1;
  out->b2 = (float)hp->beta2;
  out->c1 = (float)(1.0 - hp->beta1);
  out->c2 = (float)(1.0 - hp->beta2);
  out->ss = (float)(hp->lr / (1.0 - pow(hp->beta1, t)));
  out->bc = (float)sqrt(1.0 - pow(hp->beta2, t));
  out->e = (float)hp->eps;
  out->dec = (float)(1.0 - hp->lr * hp->weight_decay);
  out->w = (float)hp->weight_decay;
  return ok();
}

// The constants of steps 1..count, each exactly as zero_adam_derive gives it for that step.
zero_status zero_adam_derive_table(const zero_adam_hparams* hp, uint32_t count,
                                   zero_adam_scalars* out) {
  if (!hp || !out) return fail(ZERO_E_INVAL, "zero_adam_derive_table: NULL argument");
  if (count == 0) return fail(ZERO_E_INVAL, "zero_adam_derive_table: count is 0");
  zero_adam_hparams h = *hp;
  for (uint32_t i = 0; i < count; ++i) {
    h.step = (int64_t)i + 1;
    const zero_status s = zero_adam_derive(&h, &out[i]);
    if (s != ZERO_OK) return s;
  }
  return ok();
}

const char* zero_status_str(zero_status s) {
  switch (s) {
    case ZERO_OK: return "ok";
    case ZERO_E_INVAL: return "invalid argument";
    case ZERO_E_OVERFLOW: return "size overflow";
    case ZERO_E_UNSUPPORTED: return "unsupported combination";
    case ZERO_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* zero_last_error(void) { return g_last_error; }

}  // extern "C"
