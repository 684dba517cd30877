// Host half of ZeRO-Offload: the Adam/AdamW update on host-resident state ("ZeRO 优化器：把显存
// “分”着用", ZeRO-Offload: the CPU updates the optimizer state kept in host memory). The same fp32
// operation order as the GPU kernel, each operation rounded on its own (built with
// -ffp-contract=off; x86 division and square root are correctly rounded; each thread's range runs
// in IEEE mode whatever the caller's), so the two agree bit for bit. The range is split over host threads. On CPUs with AVX2 and F16C the loop is written with
// vector intrinsics and streaming (non-temporal) stores: the state and the 16-bit parameters go
// straight to memory instead of being read for ownership into the caches, which the update, bound
// by host memory, turns into time. No HIP calls: this file also builds with a plain host compiler
// (and its sanitizers).
#include <immintrin.h>
#include <math.h>
#include <string.h>

#include <thread>
#include <vector>

#include "zero_fpenv.h"
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

using zero::IeeeScope;

template <bool L2, int ODT>
void range_base(const HostStep& s, uint64_t lo, uint64_t hi) {
  IeeeScope ieee;
  adam_range<L2, ODT>(s, lo, hi);
}

template <bool L2, int ODT>
__attribute__((target("avx2"))) void range_avx2(const HostStep& s, uint64_t lo, uint64_t hi) {
  IeeeScope ieee;
  adam_range<L2, ODT>(s, lo, hi);
}

// Eight elements of the update in AVX2, the same operations in the same order as adam_range (each
// IEEE-rounded on its own: vdivps and vsqrtps are correctly rounded, and nothing is contracted).
// Master, m and v are loaded from and streamed to 32-byte aligned addresses; the gradient may sit
// anywhere; the 16-bit parameters are streamed when OUT_NT (16-byte aligned) and stored plainly
// otherwise.
template <bool L2, int ODT, bool OUT_NT>
__attribute__((target("avx2,f16c"))) inline void adam8_stream(const HostStep& s, uint64_t i) {
  const zero_adam_scalars& k = s.k;
  __m256 g = _mm256_mul_ps(_mm256_loadu_ps(s.g + i), _mm256_set1_ps(s.gs));
  __m256 p = _mm256_load_ps(s.P + i), m = _mm256_load_ps(s.M + i), v = _mm256_load_ps(s.V + i);
  if (L2) g = _mm256_add_ps(g, _mm256_mul_ps(_mm256_set1_ps(k.w), p));
  m = _mm256_add_ps(_mm256_mul_ps(_mm256_set1_ps(k.b1), m), _mm256_mul_ps(_mm256_set1_ps(k.c1), g));
  v = _mm256_add_ps(_mm256_mul_ps(_mm256_set1_ps(k.b2), v),
                    _mm256_mul_ps(_mm256_set1_ps(k.c2), _mm256_mul_ps(g, g)));
  const __m256 den = _mm256_add_ps(_mm256_div_ps(_mm256_sqrt_ps(v), _mm256_set1_ps(k.bc)),
                                   _mm256_set1_ps(k.e));
  if (!L2) p = _mm256_mul_ps(p, _mm256_set1_ps(k.dec));
  p = _mm256_sub_ps(p, _mm256_mul_ps(_mm256_set1_ps(k.ss), _mm256_div_ps(m, den)));
  _mm256_stream_ps(s.P + i, p);
  _mm256_stream_ps(s.M + i, m);
  _mm256_stream_ps(s.V + i, v);
  if (ODT == ZERO_F32) return;
  __m128i h;
  if (ODT == ZERO_F16) {
    // the hardware binary16 conversion rounds to nearest even, keeps subnormals, overflows to
    // infinity and quiets a NaN keeping its top payload bits: f16_rne for every fp32 pattern
    h = _mm256_cvtps_ph(p, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
  } else {
    // bf16_rne on eight lanes: NaN -> top half with the quiet bit, else add 0x7fff + lsb, shift
    const __m256i u = _mm256_castps_si256(p);
    const __m256i nan = _mm256_cmpgt_epi32(_mm256_and_si256(u, _mm256_set1_epi32(0x7fffffff)),
                                           _mm256_set1_epi32(0x7f800000));
    const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(1));
    const __m256i rne = _mm256_srli_epi32(
        _mm256_add_epi32(u, _mm256_add_epi32(_mm256_set1_epi32(0x7fff), lsb)), 16);
    const __m256i qn = _mm256_or_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(0x40));
    const __m256i b = _mm256_blendv_epi8(rne, qn, nan);
    h = _mm_packus_epi32(_mm256_castsi256_si128(b), _mm256_extracti128_si256(b, 1));
  }
  if (OUT_NT) _mm_stream_si128(reinterpret_cast<__m128i*>(s.out + i), h);
  else _mm_storeu_si128(reinterpret_cast<__m128i*>(s.out + i), h);
}

template <bool L2, int ODT, bool OUT_NT>
__attribute__((target("avx2,f16c"))) void stream_body(const HostStep& s, uint64_t i, uint64_t hi) {
  for (; i + 8 <= hi; i += 8) adam8_stream<L2, ODT, OUT_NT>(s, i);
  adam_range<L2, ODT>(s, i, hi);
}

// The streaming form over [lo, hi): a scalar head up to master's first 32-byte boundary, the
// vector body, a scalar tail. When m or v does not share master's 32-byte phase the whole range
// takes the plain AVX2 loop. Ends with a store fence: streaming stores are weakly ordered, and
// the caller hands the results on (to another thread, or to a DMA copy) after this returns.
template <bool L2, int ODT>
__attribute__((target("avx2,f16c"))) void range_stream(const HostStep& s, uint64_t lo, uint64_t hi) {
  IeeeScope ieee;
  const auto phase = [](const void* p) { return reinterpret_cast<uintptr_t>(p) & 31u; };
  if (phase(s.M + lo) != phase(s.P + lo) || phase(s.V + lo) != phase(s.P + lo)) {
    adam_range<L2, ODT>(s, lo, hi);
    return;
  }
  uint64_t i = lo;
  while (i < hi && phase(s.P + i) != 0) ++i;
  adam_range<L2, ODT>(s, lo, i);
  if (ODT != ZERO_F32 && (reinterpret_cast<uintptr_t>(s.out + i) & 15u) == 0)
    stream_body<L2, ODT, true>(s, i, hi);
  else
    stream_body<L2, ODT, false>(s, i, hi);
  _mm_sfence();
}

typedef zero::HostRangeFn RangeFn;

enum class Isa { kBase, kAvx2, kStream };

template <bool L2, int ODT>
RangeFn pick_isa(Isa isa) {
  if (isa == Isa::kStream) return range_stream<L2, ODT>;
  return isa == Isa::kAvx2 ? range_avx2<L2, ODT> : range_base<L2, ODT>;
}

template <bool L2>
RangeFn pick_odt(int odt, Isa isa) {
  if (odt == ZERO_BF16) return pick_isa<L2, ZERO_BF16>(isa);
  if (odt == ZERO_F16) return pick_isa<L2, ZERO_F16>(isa);
  return pick_isa<L2, ZERO_F32>(isa);
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

Isa host_isa() {
  static const Isa isa = !__builtin_cpu_supports("avx2") ? Isa::kBase
                         : __builtin_cpu_supports("f16c") ? Isa::kStream
                                                          : Isa::kAvx2;
  return isa;
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
  const RangeFn fn = l2 ? pick_odt<true>(odt, host_isa()) : pick_odt<false>(odt, host_isa());
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
