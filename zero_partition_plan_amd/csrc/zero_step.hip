// C-ABI entry points of the per-rank sharded optimizer step: argument checks, dispatch to the
// kernels of zero_step_kernels.hip, and the small kernels of the squared-norm finish, the clip scale
// and the device step counter.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "zero_internal.h"
#include "zero_step.h"

namespace {

using zero::step::AdamArgs;
using zero::step::DevCtl;
using zero::step::kBlock;
using zero::step::Phase;
using zero::step::ReduceArgs;
using zero::step::RepPtrs;
using zero::step::StepScalars;

constexpr int kWaves = kBlock / 64;
constexpr uint32_t kSqLevel1 = 1024;   // second-level partial slots

// The squared-norm partials of zero_reduce_shard_static, owned by the library: each GPU holds its
// own copy from the code object's load until the process ends. In host code this name is a host
// stand-in; device addresses come from hipGetSymbolAddress (static_scratch below).
static __device__ __align__(256) double scratch[ZERO_STATIC_SQ_PARTIALS];

// ---------------------------------------------------------------------------------------------
// squared-norm finish, clip scale, step counter

__device__ __forceinline__ double block_sum(double x, double* lds) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds[wave] = x;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
    s = lds[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += lds[w];
  }
  return s;  // meaningful in thread 0 only
}

// level 1: block b sums partials [b*chunk, min(ntiles, (b+1)*chunk)) into partials[ntiles + b]
__global__ __launch_bounds__(kBlock) void k_sq_level1(double* __restrict__ partials, uint64_t ntiles,
                                                      uint64_t chunk) {
  __shared__ double lds[kWaves];
  const uint64_t lo = (uint64_t)blockIdx.x * chunk;
  const uint64_t hi = lo + chunk < ntiles ? lo + chunk : ntiles;
  double s = 0.0;
  for (uint64_t i = lo + threadIdx.x; i < hi; i += kBlock) s += partials[i];
  s = block_sum(s, lds);
  if (threadIdx.x == 0) partials[ntiles + blockIdx.x] = s;
}

// level 2: one block sums the `count` level-1 values at `l1` into *out
__global__ __launch_bounds__(kBlock) void k_sq_finalize(const double* __restrict__ l1,
                                                        uint32_t count, double* __restrict__ out) {
  __shared__ double lds[kWaves];
  double s = 0.0;
  for (uint32_t i = threadIdx.x; i < count; i += kBlock) s += l1[i];
  s = block_sum(s, lds);
  if (threadIdx.x == 0) *out = s;
}

// clip scale: q = max_norm / (sqrt(sq) + eps) in fp64, coef = min(1, q) (1 for a NaN q), and the
// fp32 grad scale coef * inv_loss_scale rounded to nearest even. fp64 division and square root are
// correctly rounded in this build, as on the host.
__global__ __launch_bounds__(64) void k_clip_scale(const double* __restrict__ sq, double max_norm,
                                                   double eps, double inv_loss_scale,
                                                   float* __restrict__ gs) {
  if (threadIdx.x != 0) return;
  const double q = max_norm / (sqrt(*sq) + eps);
  const double coef = q < 1.0 ? q : 1.0;
  *gs = (float)(coef * inv_loss_scale);
}

// the step counter after an update: nothing on a skipped step; a t outside the constants table
// (the update then wrote nothing) is reported in *status and t stays; otherwise t advances
__global__ __launch_bounds__(64) void k_step_advance(int64_t* __restrict__ step,
                                                     const int32_t* __restrict__ skip,
                                                     int32_t* __restrict__ status,
                                                     uint32_t table_len) {
  if (threadIdx.x != 0) return;
  if (skip != nullptr && *skip != 0) return;
  const int64_t t = *step;
  if (t < 1 || t > (int64_t)table_len) *status = ZERO_DEV_T_OUT_OF_TABLE;
  else *step = t + 1;
}

// ---------------------------------------------------------------------------------------------
// host side

// ---------------------------------------------------------------------------------------------
// the library's scratch, per device

constexpr int kMaxDevices = 64;
std::atomic<double*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// the device address of `scratch` on the current device, looked up once per device
zero_status static_scratch(const char* fn, double** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return zero::fail(ZERO_E_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return zero::fail(ZERO_E_UNSUPPORTED, "%s: device index %d", fn, dev);
  double* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || addr == nullptr)
        return zero::fail(ZERO_E_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn,
                          hipGetErrorString(e));
      p = static_cast<double*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ZERO_OK;
}

zero_status launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return zero::fail(ZERO_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return zero::ok();
}

zero_status check_src(const char* fn, const zero_grad_src* src, uint64_t n) {
  if (!src || !src->ptrs) return zero::fail(ZERO_E_INVAL, "%s: gradient source is NULL", fn);
  if (src->count == 0 || src->count > ZERO_MAX_REPLICAS)
    return zero::fail(ZERO_E_INVAL, "%s: replica count %u outside 1..%d", fn, src->count,
                      ZERO_MAX_REPLICAS);
  if (!zero::dtype_valid(src->dtype))
    return zero::fail(ZERO_E_INVAL, "%s: unknown replica dtype %d", fn, src->dtype);
  for (uint32_t k = 0; k < src->count && n > 0; ++k)   // zero-length arrays may be NULL
    if (!src->ptrs[k]) return zero::fail(ZERO_E_INVAL, "%s: replica %u is NULL", fn, k);
  if (n > UINT64_MAX / 8) return zero::fail(ZERO_E_OVERFLOW, "%s: n = %llu too large", fn,
                                            (unsigned long long)n);
  return ZERO_OK;
}

// a word written by a call (flag, status, step) must not lie inside an array the call touches
zero_status word_clear(const char* fn, const char* word, const void* w, uint64_t wb,
                       const void* const* arr, const uint64_t* arr_b, const char* const* names,
                       int count) {
  for (int i = 0; i < count; ++i)
    if (zero::overlaps(w, wb, arr[i], arr_b[i]))
      return zero::fail(ZERO_E_INVAL, "%s: %s overlaps %s", fn, word, names[i]);
  return ZERO_OK;
}

zero_status word_clear_reps(const char* fn, const char* word, const void* w, uint64_t wb,
                            const zero_grad_src* src, uint64_t rb) {
  for (uint32_t k = 0; k < src->count; ++k)
    if (zero::overlaps(w, wb, src->ptrs[k], rb))
      return zero::fail(ZERO_E_INVAL, "%s: %s overlaps replica %u", fn, word, k);
  return ZERO_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// every replica naturally aligned (fp32 on 4 bytes, 16-bit on 2), as the kernels require
zero_status src_natural(const char* fn, const zero_grad_src* src) {
  const uintptr_t a = zero::dtype_bytes(src->dtype);
  for (uint32_t k = 0; k < src->count; ++k)
    if (!aligned(src->ptrs[k], a))
      return zero::fail(ZERO_E_INVAL, "%s: replica %u is not aligned to its %u-byte elements", fn, k,
                        (unsigned)a);
  return ZERO_OK;
}

// bit k set: 16-bit replica k starts at an odd element (2 bytes past a 4-byte word)
uint64_t rep_odd_mask(const zero_grad_src* src) {
  if (src->dtype == ZERO_F32) return 0;
  uint64_t m = 0;
  for (uint32_t k = 0; k < src->count; ++k)
    if (!aligned(src->ptrs[k], 4)) m |= 1ull << k;
  return m;
}

RepPtrs rep_ptrs(const zero_grad_src* src) {
  RepPtrs r{};
  for (uint32_t k = 0; k < src->count; ++k) r.p[k] = src->ptrs[k];
  return r;
}

// arguments already checked; n > 0
zero_status reduce_impl(const zero_grad_src* src, uint64_t n, float* G, int32_t* flag,
                        double* partials, double sq_scale, hipStream_t stream, const char* what) {
  const Phase ph{rep_odd_mask(src), 0};
  ReduceArgs a{rep_ptrs(src), (int)src->count, n, G, flag, partials, sq_scale, stream, ph};
  (void)hipGetLastError();
  switch (src->dtype) {
    case ZERO_F32: zero::step::launch_reduce<ZERO_F32>(a); break;
    case ZERO_F16: zero::step::launch_reduce<ZERO_F16>(a); break;
    default: zero::step::launch_reduce<ZERO_BF16>(a); break;
  }
  return launched(what);
}

zero_status sq_finish(uint64_t n, double* partials, double* out, hipStream_t stream, const char* what) {
  const uint64_t ntiles = zero::step::red_tiles(n);
  const uint32_t g1 = ntiles < kSqLevel1 ? (uint32_t)ntiles : kSqLevel1;
  (void)hipGetLastError();
  if (g1 > 0) {
    const uint64_t chunk = (ntiles + g1 - 1) / g1;
    hipLaunchKernelGGL(k_sq_level1, dim3(g1), dim3(kBlock), 0, stream, partials, ntiles, chunk);
  }
  hipLaunchKernelGGL(k_sq_finalize, dim3(1), dim3(kBlock), 0, stream, partials + ntiles, g1, out);
  return launched(what);
}

}  // namespace

extern "C" {

uint64_t zero_sq_partials_len(uint64_t n) { return zero::step::red_tiles(n) + kSqLevel1; }

zero_status zero_reduce_shard(const zero_grad_src* src, uint64_t n, float* out_grad,
                              int32_t* d_nonfinite, double* d_sq_partials, double sq_scale,
                              void* stream) {
  const char* fn = "zero_reduce_shard";
  zero_status s = check_src(fn, src, n);
  if (s != ZERO_OK) return s;
  if (!out_grad && !d_nonfinite && !d_sq_partials)
    return zero::fail(ZERO_E_INVAL, "%s: no output requested", fn);
  const uint64_t rb = n * zero::dtype_bytes(src->dtype), pb = zero_sq_partials_len(n) * 8;
  for (uint32_t k = 0; k < src->count; ++k) {
    if (out_grad && zero::overlaps(out_grad, n * 4, src->ptrs[k], rb))
      return zero::fail(ZERO_E_INVAL, "%s: out_grad overlaps replica %u", fn, k);
    if (d_sq_partials && zero::overlaps(d_sq_partials, pb, src->ptrs[k], rb))
      return zero::fail(ZERO_E_INVAL, "%s: partials overlap replica %u", fn, k);
  }
  if (d_sq_partials && out_grad && zero::overlaps(d_sq_partials, pb, out_grad, n * 4))
    return zero::fail(ZERO_E_INVAL, "%s: partials overlap out_grad", fn);
  if (d_nonfinite) {
    const void* arr[2] = {out_grad, d_sq_partials};
    const uint64_t arr_b[2] = {out_grad ? n * 4 : 0, d_sq_partials ? pb : 0};
    const char* names[2] = {"out_grad", "the partials"};
    s = word_clear(fn, "d_nonfinite", d_nonfinite, 4, arr, arr_b, names, 2);
    if (s == ZERO_OK) s = word_clear_reps(fn, "d_nonfinite", d_nonfinite, 4, src, rb);
    if (s != ZERO_OK) return s;
  }
  if (n == 0) return zero::ok();
  s = src_natural(fn, src);
  if (s != ZERO_OK) return s;
  if ((out_grad && !aligned(out_grad, 4)) || (d_nonfinite && !aligned(d_nonfinite, 4)) ||
      (d_sq_partials && !aligned(d_sq_partials, 8)))
    return zero::fail(ZERO_E_INVAL, "%s: out_grad, d_nonfinite or d_sq_partials is not aligned to "
                      "its elements", fn);
  return reduce_impl(src, n, out_grad, d_nonfinite, d_sq_partials, sq_scale,
                     static_cast<hipStream_t>(stream), fn);
}

zero_status zero_shard_sqnorm(const float* d_grad, uint64_t n, double sq_scale, double* d_partials,
                              double* d_out, void* stream) {
  const char* fn = "zero_shard_sqnorm";
  if (!d_partials || !d_out) return zero::fail(ZERO_E_INVAL, "%s: partials or out is NULL", fn);
  if (n > UINT64_MAX / 8)
    return zero::fail(ZERO_E_OVERFLOW, "%s: n = %llu too large", fn, (unsigned long long)n);
  const uint64_t pb = zero_sq_partials_len(n) * 8;
  if (zero::overlaps(d_partials, pb, d_out, 8))
    return zero::fail(ZERO_E_INVAL, "%s: out overlaps the partials", fn);
  if (!aligned(d_partials, 8) || !aligned(d_out, 8) || (d_grad && !aligned(d_grad, 4)))
    return zero::fail(ZERO_E_INVAL, "%s: an array is not aligned to its elements", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d_grad != nullptr) {
    const void* ptrs[1] = {d_grad};
    const zero_grad_src src{ptrs, 1, ZERO_F32};
    zero_status s = check_src(fn, &src, n);
    if (s != ZERO_OK) return s;
    if (zero::overlaps(d_partials, pb, d_grad, n * 4))
      return zero::fail(ZERO_E_INVAL, "%s: partials overlap the gradient", fn);
    if (zero::overlaps(d_out, 8, d_grad, n * 4))
      return zero::fail(ZERO_E_INVAL, "%s: out overlaps the gradient", fn);
    if (n > 0) {
      s = reduce_impl(&src, n, nullptr, nullptr, d_partials, sq_scale, st, fn);
      if (s != ZERO_OK) return s;
    }
  }
  return sq_finish(n, d_partials, d_out, st, fn);
}

zero_status zero_reduce_shard_static(const zero_grad_src* src, uint64_t n, float* out_grad,
                                     int32_t* d_nonfinite, double sq_scale, double* d_sq,
                                     void* stream) {
  const char* fn = "zero_reduce_shard_static";
  zero_status s = check_src(fn, src, n);
  if (s != ZERO_OK) return s;
  if (!out_grad && !d_nonfinite && !d_sq) return zero::fail(ZERO_E_INVAL, "%s: no output requested", fn);
  if (d_sq && n > ZERO_STATIC_MAX_ELEMS)
    return zero::fail(ZERO_E_INVAL, "%s: n = %llu exceeds the %llu elements the library's %u "
                      "squared-norm partials cover", fn, (unsigned long long)n,
                      (unsigned long long)ZERO_STATIC_MAX_ELEMS, (unsigned)ZERO_STATIC_SQ_PARTIALS);
  const uint64_t rb = n * zero::dtype_bytes(src->dtype);
  for (uint32_t k = 0; k < src->count; ++k) {
    if (out_grad && zero::overlaps(out_grad, n * 4, src->ptrs[k], rb))
      return zero::fail(ZERO_E_INVAL, "%s: out_grad overlaps replica %u", fn, k);
    if (d_sq && zero::overlaps(d_sq, 8, src->ptrs[k], rb))
      return zero::fail(ZERO_E_INVAL, "%s: d_sq overlaps replica %u", fn, k);
  }
  if (d_sq && out_grad && zero::overlaps(d_sq, 8, out_grad, n * 4))
    return zero::fail(ZERO_E_INVAL, "%s: d_sq overlaps out_grad", fn);
  if (d_nonfinite) {
    const void* arr[2] = {out_grad, d_sq};
    const uint64_t arr_b[2] = {out_grad ? n * 4 : 0, d_sq ? 8u : 0u};
    const char* names[2] = {"out_grad", "d_sq"};
    s = word_clear(fn, "d_nonfinite", d_nonfinite, 4, arr, arr_b, names, 2);
    if (s == ZERO_OK) s = word_clear_reps(fn, "d_nonfinite", d_nonfinite, 4, src, rb);
    if (s != ZERO_OK) return s;
  }
  s = src_natural(fn, src);
  if (s != ZERO_OK) return s;
  if ((out_grad && !aligned(out_grad, 4)) || (d_nonfinite && !aligned(d_nonfinite, 4)) ||
      (d_sq && !aligned(d_sq, 8)))
    return zero::fail(ZERO_E_INVAL, "%s: out_grad, d_nonfinite or d_sq is not aligned to its "
                      "elements", fn);
  double* partials = nullptr;
  if (d_sq) {
    s = static_scratch(fn, &partials);
    if (s != ZERO_OK) return s;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (n > 0) {
    s = reduce_impl(src, n, out_grad, d_nonfinite, partials, sq_scale, st, fn);
    if (s != ZERO_OK) return s;
  }
  return d_sq ? sq_finish(n, partials, d_sq, st, fn) : zero::ok();
}

}  // extern "C"

namespace {

// every step entry point: constants in sc0, or from device memory as dc says (dc.gs != NULL)
zero_status adam_step_impl(const char* fn, const zero_grad_src* src, uint64_t n,
                           const StepScalars& sc0, const DevCtl& dc, bool l2, float* master,
                           float* m, float* v, void* out_param, int32_t out_dtype,
                           const int32_t* d_skip, void* stream) {
  zero_status s = check_src(fn, src, n);
  if (s != ZERO_OK) return s;
  if (n > 0 && (!master || !m || !v))
    return zero::fail(ZERO_E_INVAL, "%s: master, m or v is NULL", fn);
  if (out_param) {
    if (out_dtype == ZERO_F32)
      return zero::fail(ZERO_E_UNSUPPORTED, "%s: fp32 parameter output is not supported", fn);
    if (out_dtype != ZERO_BF16 && out_dtype != ZERO_F16)
      return zero::fail(ZERO_E_INVAL, "%s: unknown out dtype %d", fn, out_dtype);
  }
  const uint64_t sb = n * 4, ob = out_param ? n * 2 : 0, rb = n * zero::dtype_bytes(src->dtype);
  const void* own[4] = {master, m, v, out_param};
  const uint64_t own_b[4] = {sb, sb, sb, ob};
  const char* own_names[4] = {"master", "m", "v", "out_param"};
  // device inputs the update reads (grad scale, constants table, step, skip flag) must not be
  // written by it
  const void* dev_in[4] = {dc.gs, dc.table, dc.step, d_skip};
  const uint64_t dev_in_b[4] = {dc.gs ? 4u : 0u,
                                dc.table ? (uint64_t)dc.table_len * sizeof(zero_adam_scalars) : 0u,
                                dc.step ? 8u : 0u, d_skip ? 4u : 0u};
  const char* dev_in_names[4] = {"the grad scale", "the constants table", "the step", "the skip flag"};
  for (int x = 0; x < 4; ++x) {
    for (int y = x + 1; y < 4; ++y)
      if (zero::overlaps(own[x], own_b[x], own[y], own_b[y]))
        return zero::fail(ZERO_E_INVAL, "%s: %s overlaps %s", fn, own_names[x], own_names[y]);
    for (uint32_t r = 0; r < src->count; ++r)
      if (zero::overlaps(own[x], own_b[x], src->ptrs[r], rb))
        return zero::fail(ZERO_E_INVAL, "%s: %s overlaps replica %u", fn, own_names[x], r);
    for (int d = 0; d < 4; ++d)
      if (zero::overlaps(own[x], own_b[x], dev_in[d], dev_in_b[d]))
        return zero::fail(ZERO_E_INVAL, "%s: %s overlaps %s", fn, own_names[x], dev_in_names[d]);
  }
  if (n == 0) return zero::ok();

  // every array naturally aligned: fp32 on 4 bytes, 16-bit on 2 (then any element offset works)
  s = src_natural(fn, src);
  if (s != ZERO_OK) return s;
  if (!aligned(master, 4) || !aligned(m, 4) || !aligned(v, 4) ||
      (out_param != nullptr && !aligned(out_param, 2)))
    return zero::fail(ZERO_E_INVAL, "%s: master, m, v or out_param is not aligned to its elements", fn);
  if ((dc.gs && !aligned(dc.gs, 4)) || (dc.table && !aligned(dc.table, 4)) ||
      (dc.step && !aligned(dc.step, 8)) || (d_skip && !aligned(d_skip, 4)))
    return zero::fail(ZERO_E_INVAL, "%s: a device scalar is not aligned to its size", fn);
  const uint64_t ntiles = n / zero::step::kAdamTile;
  const Phase ph{rep_odd_mask(src), out_param != nullptr && !aligned(out_param, 4)};
  AdamArgs a{rep_ptrs(src), (int)src->count, ntiles, n, sc0, master, m, v, out_param, d_skip, dc,
             static_cast<hipStream_t>(stream), n % zero::step::kAdamTile != 0, ph};
  const int odt = out_param ? out_dtype : ZERO_F32;
  (void)hipGetLastError();
  using zero::step::launch_adam;
#define ZERO_ADAM_OUT(RDT)                                                \
  switch (odt) {                                                          \
    case ZERO_BF16: launch_adam<RDT, ZERO_BF16>(a, l2); break;            \
    case ZERO_F16: launch_adam<RDT, ZERO_F16>(a, l2); break;              \
    default: launch_adam<RDT, ZERO_F32>(a, l2); break; /* no output */    \
  }
  switch (src->dtype) {
    case ZERO_F32: ZERO_ADAM_OUT(ZERO_F32) break;
    case ZERO_F16: ZERO_ADAM_OUT(ZERO_F16) break;
    default: ZERO_ADAM_OUT(ZERO_BF16) break;
  }
#undef ZERO_ADAM_OUT
  return launched(fn);
}

// the host-step entry points: constants derived from hp on the host
zero_status adam_step_host_t(const char* fn, const zero_grad_src* src, uint64_t n,
                             float grad_scale, const float* d_grad_scale, float* master, float* m,
                             float* v, const zero_adam_hparams* hp, void* out_param,
                             int32_t out_dtype, const int32_t* d_skip, void* stream) {
  zero_adam_scalars k;
  const zero_status s = zero_adam_derive(hp, &k);
  if (s != ZERO_OK) return s;
  const StepScalars sc{grad_scale, k.b1, k.b2, k.c1, k.c2, k.ss, k.bc, k.e, k.dec, k.w};
  const DevCtl dc{d_grad_scale, nullptr, nullptr, 0};
  return adam_step_impl(fn, src, n, sc, dc, hp->wd_mode == ZERO_ADAM_L2, master, m, v, out_param,
                        out_dtype, d_skip, stream);
}

}  // namespace

extern "C" {

zero_status zero_adam_shard_step(const zero_grad_src* src, uint64_t n, float grad_scale,
                                 float* master, float* m, float* v, const zero_adam_hparams* hp,
                                 void* out_param, int32_t out_dtype, const int32_t* d_skip,
                                 void* stream) {
  return adam_step_host_t("zero_adam_shard_step", src, n, grad_scale, nullptr, master, m, v, hp,
                          out_param, out_dtype, d_skip, stream);
}

zero_status zero_adam_shard_step_dev_scale(const zero_grad_src* src, uint64_t n,
                                           const float* d_grad_scale, float* master, float* m,
                                           float* v, const zero_adam_hparams* hp, void* out_param,
                                           int32_t out_dtype, const int32_t* d_skip,
                                           void* stream) {
  const char* fn = "zero_adam_shard_step_dev_scale";
  if (!d_grad_scale) return zero::fail(ZERO_E_INVAL, "%s: d_grad_scale is NULL", fn);
  return adam_step_host_t(fn, src, n, 1.0f, d_grad_scale, master, m, v, hp, out_param, out_dtype,
                          d_skip, stream);
}

zero_status zero_adam_shard_step_dev_t(const zero_grad_src* src, uint64_t n,
                                       const float* d_grad_scale, const zero_adam_scalars* d_table,
                                       uint32_t table_len, int64_t* d_step, int32_t* d_status,
                                       int32_t wd_mode, float* master, float* m, float* v,
                                       void* out_param, int32_t out_dtype, const int32_t* d_skip,
                                       void* stream) {
  const char* fn = "zero_adam_shard_step_dev_t";
  if (!d_grad_scale || !d_table || !d_step || !d_status)
    return zero::fail(ZERO_E_INVAL, "%s: d_grad_scale, d_table, d_step or d_status is NULL", fn);
  if (table_len == 0) return zero::fail(ZERO_E_INVAL, "%s: empty constants table", fn);
  if (wd_mode != ZERO_ADAMW && wd_mode != ZERO_ADAM_L2)
    return zero::fail(ZERO_E_INVAL, "%s: unknown wd_mode %d", fn, wd_mode);
  const uint64_t tb = (uint64_t)table_len * sizeof(zero_adam_scalars);
  if (zero::overlaps(d_step, 8, d_table, tb) || zero::overlaps(d_step, 8, d_grad_scale, 4) ||
      (d_skip && zero::overlaps(d_step, 8, d_skip, 4)))
    return zero::fail(ZERO_E_INVAL, "%s: d_step overlaps the table, the grad scale or the flag", fn);
  zero_status s = check_src(fn, src, n);
  if (s != ZERO_OK) return s;
  // the status word is written after the update: it must not lie in anything the step reads or
  // writes; nor may the step counter lie in a replica
  const uint64_t sb = n * 4, ob = out_param ? n * 2 : 0, rb = n * zero::dtype_bytes(src->dtype);
  const void* arr[8] = {master, m, v, out_param, d_table, d_grad_scale, d_step, d_skip};
  const uint64_t arr_b[8] = {sb, sb, sb, ob, tb, 4, 8, d_skip ? 4u : 0u};
  const char* names[8] = {"master", "m", "v", "out_param", "the constants table",
                          "the grad scale", "the step", "the skip flag"};
  s = word_clear(fn, "d_status", d_status, 4, arr, arr_b, names, 8);
  if (s == ZERO_OK) s = word_clear_reps(fn, "d_status", d_status, 4, src, rb);
  if (s == ZERO_OK) s = word_clear_reps(fn, "d_step", d_step, 8, src, rb);
  if (s != ZERO_OK) return s;
  const StepScalars sc{1.0f, 0, 0, 0, 0, 0, 0, 0, 0, 0};   // all read from the table
  const DevCtl dc{d_grad_scale, d_table, d_step, table_len};
  s = adam_step_impl(fn, src, n, sc, dc, wd_mode == ZERO_ADAM_L2, master, m, v,
                                 out_param, out_dtype, d_skip, stream);
  if (s != ZERO_OK) return s;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_step_advance, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), d_step,
                     d_skip, d_status, table_len);
  return launched(fn);
}

zero_status zero_clip_scale(const double* d_sq, double max_norm, double clip_eps,
                            double inv_loss_scale, float* d_grad_scale, void* stream) {
  const char* fn = "zero_clip_scale";
  if (!d_sq || !d_grad_scale) return zero::fail(ZERO_E_INVAL, "%s: d_sq or d_grad_scale is NULL", fn);
  if (zero::overlaps(d_sq, 8, d_grad_scale, 4))
    return zero::fail(ZERO_E_INVAL, "%s: d_grad_scale overlaps d_sq", fn);
  if (!(std::isfinite(max_norm) && max_norm > 0.0))
    return zero::fail(ZERO_E_INVAL, "%s: max_norm %g is not finite and positive", fn, max_norm);
  if (!(std::isfinite(clip_eps) && clip_eps >= 0.0))
    return zero::fail(ZERO_E_INVAL, "%s: clip_eps %g is not finite and non-negative", fn, clip_eps);
  if (!(std::isfinite(inv_loss_scale) && inv_loss_scale > 0.0))
    return zero::fail(ZERO_E_INVAL, "%s: inv_loss_scale %g is not finite and positive", fn,
                      inv_loss_scale);
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_clip_scale, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), d_sq,
                     max_norm, clip_eps, inv_loss_scale, d_grad_scale);
  return launched(fn);
}

}  // extern "C"
