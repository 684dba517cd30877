// Host half of ZeRO-Offload: the Adam/AdamW update on host-resident state ("ZeRO 优化器：把显存
// “分”着用", ZeRO-Offload: the CPU updates the optimizer state kept in host memory). The same fp32
// operation order as the GPU kernel, each operation rounded on its own (built with
// -ffp-contract=off; x86 division and square root are correctly rounded), so the two agree bit for
// bit. The range is split over host threads; an AVX2 build of the loop is used when the CPU has it.
// No HIP calls: this file also builds with a plain host compiler (and its sanitizers).
#include <math.h>
#include <string.h>

#include <thread>
#include <vector>

#include "zero_host_adam.h"

namespace {

// fp32 -> bf16, round to nearest even; a NaN keeps sign and top payload and becomes quiet.
inline uint16_t bf16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// fp32 -> IEEE binary16, round to nearest even, gradual underflow, overflow to infinity; a NaN
// keeps sign and top payload and becomes quiet.
inline uint16_t f16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  const uint32_t sign = (u >> 16) & 0x8000u, a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((a >> 13) & 0x3ffu));
  if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);        // >= 65520 (and inf) -> inf
  if (a >= 0x38800000u) {                                          // normal binary16 range
    uint32_t t = a - 0x38000000u;                                  // rebias 127 -> 15
    t = t + 0x0fffu + ((t >> 13) & 1u);
    return (uint16_t)(sign | (t >> 13));
  }
  if (a <= 0x33000000u) return (uint16_t)sign;                     // <= 2^-25 rounds to 0
  const uint32_t e = a >> 23, m = (a & 0x7fffffu) | 0x800000u;    // subnormal binary16
  const uint32_t shift = 126u - e;                                 // 14 .. 24
  uint32_t h = m >> shift;
  const uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1u);
  if (rem > half || (rem == half && (h & 1u))) ++h;
  return (uint16_t)(sign | h);
}

}  // namespace

namespace zero {
struct HostStep {
  const float* g;
  float gs;
  float *P, *M, *V;
  uint16_t* out;
  zero_adam_scalars k;
};
}  // namespace zero

namespace {

using zero::HostStep;

template <bool L2, int ODT>
inline __attribute__((always_inline)) void adam_range(const HostStep& s, uint64_t lo, uint64_t hi) {
  const zero_adam_scalars k = s.k;
  for (uint64_t i = lo; i < hi; ++i) {
    float g = s.g[i] * s.gs;
    float p = s.P[i], m = s.M[i], v = s.V[i];
    if (L2) g = g + k.w * p;
    m = k.b1 * m + k.c1 * g;
    v = k.b2 * v + k.c2 * (g * g);
    const float den = sqrtf(v) / k.bc + k.e;
    if (!L2) p = p * k.dec;
    p = p - k.ss * (m / den);
    s.P[i] = p;
    s.M[i] = m;
    s.V[i] = v;
    if (ODT == ZERO_BF16) s.out[i] = bf16_rne(p);
    else if (ODT == ZERO_F16) s.out[i] = f16_rne(p);
  }
}

template <bool L2, int ODT>
void range_base(const HostStep& s, uint64_t lo, uint64_t hi) {
  adam_range<L2, ODT>(s, lo, hi);
}

template <bool L2, int ODT>
__attribute__((target("avx2"))) void range_avx2(const HostStep& s, uint64_t lo, uint64_t hi) {
  adam_range<L2, ODT>(s, lo, hi);
}

typedef zero::HostRangeFn RangeFn;

template <bool L2>
RangeFn pick_odt(int odt, bool avx2) {
  if (odt == ZERO_BF16) return avx2 ? range_avx2<L2, ZERO_BF16> : range_base<L2, ZERO_BF16>;
  if (odt == ZERO_F16) return avx2 ? range_avx2<L2, ZERO_F16> : range_base<L2, ZERO_F16>;
  return avx2 ? range_avx2<L2, ZERO_F32> : range_base<L2, ZERO_F32>;
}

uint32_t hw_threads(uint32_t threads) {
  if (threads == 0) threads = std::thread::hardware_concurrency();
  return threads == 0 ? 1 : threads;
}

// threads actually used for n elements, and the length of each one's range
void split(uint64_t n, uint32_t& threads, uint64_t& per) {
  const uint64_t kGrain = 1u << 16;  // keep thread ranges at least this long
  if ((uint64_t)threads > (n + kGrain - 1) / kGrain) threads = (uint32_t)((n + kGrain - 1) / kGrain);
  if (threads < 1) threads = 1;
  per = ((n + threads - 1) / threads + 63) / 64 * 64;  // 256-byte aligned splits
}

void run_threads(RangeFn fn, const HostStep& s, uint64_t n, uint32_t threads) {
  threads = hw_threads(threads);
  uint64_t per = 0;
  split(n, threads, per);
  if (threads <= 1) {
    fn(s, 0, n);
    return;
  }
  // No exception may leave a C entry point: a range whose thread cannot be started (or whose
  // bookkeeping cannot be allocated) runs on the calling thread instead.
  std::vector<std::thread> pool;
  try {
    pool.reserve(threads - 1);
  } catch (...) {
    fn(s, 0, n);
    return;
  }
  for (uint32_t t = 1; t < threads; ++t) {
    const uint64_t lo = per * t, hi = lo + per < n ? lo + per : n;
    if (lo >= hi) continue;
    try {
      pool.emplace_back(fn, std::cref(s), lo, hi);
    } catch (...) {
      fn(s, lo, hi);
    }
  }
  fn(s, 0, per < n ? per : n);
  for (auto& th : pool) th.join();
}

bool have_avx2() {
  static const bool yes = __builtin_cpu_supports("avx2");
  return yes;
}

}  // namespace

namespace zero {

HostTeam::HostTeam(uint32_t threads) {
  threads = hw_threads(threads);
  try {
    workers_.reserve(threads - 1);
    for (uint32_t t = 1; t < threads; ++t) workers_.emplace_back(&HostTeam::work, this, t);
  } catch (...) {
    // fewer members: the ones that started serve; run() splits over size()
  }
}

HostTeam::~HostTeam() {
  {
    std::lock_guard<std::mutex> lock(mu_);
    stop_ = true;
  }
  go_.notify_all();
  for (auto& th : workers_) th.join();
}

void HostTeam::work(uint32_t member) {
  uint64_t seen = 0;
  for (;;) {
    HostRangeFn fn;
    const HostStep* s;
    uint64_t lo = 0, hi = 0;
    bool mine = false;
    {
      std::unique_lock<std::mutex> lock(mu_);
      go_.wait(lock, [&] { return stop_ || generation_ != seen; });
      if (stop_) return;
      seen = generation_;
      fn = fn_;
      s = step_;
      if (member < used_) {
        lo = per_ * member;
        hi = lo + per_ < n_ ? lo + per_ : n_;
        mine = lo < hi;
      }
    }
    if (mine) fn(*s, lo, hi);
    {
      std::lock_guard<std::mutex> lock(mu_);
      if (--pending_ == 0) done_.notify_one();
    }
  }
}

void HostTeam::run(HostRangeFn fn, const HostStep& s, uint64_t n) {
  uint32_t threads = size();
  uint64_t per = 0;
  split(n, threads, per);
  if (threads <= 1 || workers_.empty()) {
    fn(s, 0, n);
    return;
  }
  {
    std::lock_guard<std::mutex> lock(mu_);
    fn_ = fn;
    step_ = &s;
    n_ = n;
    per_ = per;
    used_ = threads;
    pending_ = (uint32_t)workers_.size();
    ++generation_;
  }
  go_.notify_all();
  fn(s, 0, per < n ? per : n);
  std::unique_lock<std::mutex> lock(mu_);
  done_.wait(lock, [&] { return pending_ == 0; });
}

zero_status host_step(const float* grad, uint64_t n, float grad_scale, float* master, float* m,
                      float* v, const zero_adam_scalars& k, bool l2, void* out, int out_dtype,
                      uint32_t threads, HostTeam* team) {
  HostStep s{grad, grad_scale, master, m, v, static_cast<uint16_t*>(out), k};
  const int odt = out ? out_dtype : ZERO_F32;
  const RangeFn fn = l2 ? pick_odt<true>(odt, have_avx2()) : pick_odt<false>(odt, have_avx2());
  if (team != nullptr) team->run(fn, s, n);
  else run_threads(fn, s, n, threads);
  return ZERO_OK;
}

zero_status check_host_args(const char* fn, bool need_grad, const float* grad, uint64_t n,
                            float* master, float* m, float* v, const zero_adam_hparams* hp,
                            void* out, int32_t out_dtype, zero_adam_scalars* k) {
  const zero_status s = zero_adam_derive(hp, k);
  if (s != ZERO_OK) return s;
  if (n > UINT64_MAX / 8) return zero::fail(ZERO_E_OVERFLOW, "%s: n too large", fn);
  if (out && out_dtype != ZERO_BF16 && out_dtype != ZERO_F16)
    return zero::fail(out_dtype == ZERO_F32 ? ZERO_E_UNSUPPORTED : ZERO_E_INVAL,
                      "%s: out dtype %d is not bf16 or fp16", fn, out_dtype);
  if (n == 0) return ZERO_OK;
  if ((need_grad && !grad) || !master || !m || !v)
    return zero::fail(ZERO_E_INVAL, "%s: NULL array", fn);
  const void* arr[4] = {master, m, v, out};
  const uint64_t bytes[4] = {n * 4, n * 4, n * 4, out ? n * 2 : 0};
  for (int a = 0; a < 4; ++a) {
    for (int b = a + 1; b < 4; ++b)
      if (zero::overlaps(arr[a], bytes[a], arr[b], bytes[b]))
        return zero::fail(ZERO_E_INVAL, "%s: arrays %d and %d overlap", fn, a, b);
    if (grad && zero::overlaps(arr[a], bytes[a], grad, n * 4))
      return zero::fail(ZERO_E_INVAL, "%s: array %d overlaps the gradient", fn, a);
  }
  return ZERO_OK;
}

}  // namespace zero

extern "C" {

zero_status zero_host_adam_step(const float* grad, uint64_t n, float grad_scale, float* master,
                                float* m, float* v, const zero_adam_hparams* hp, void* out_param,
                                int32_t out_dtype, uint32_t threads) {
  zero_adam_scalars k;
  const zero_status s = zero::check_host_args("zero_host_adam_step", true, grad, n, master, m, v,
                                              hp, out_param, out_dtype, &k);
  if (s != ZERO_OK || n == 0) return s == ZERO_OK ? zero::ok() : s;
  zero::host_step(grad, n, grad_scale, master, m, v, k, hp->wd_mode == ZERO_ADAM_L2, out_param,
                  out_dtype, threads);
  return zero::ok();
}

}  // extern "C"
