// gfx950 kernels of the per-rank sharded optimizer step: the fused update (replica sum -> Adam ->
// 16-bit cast into the rank's slot) and the reduce pass (replica sum -> fp32 gradient, non-finite
// flag, fp64 squared-norm partials), with their launch dispatch.
//
// This file is compiled once per replica dtype / output dtype pair (-DZERO_STEP_RDT and
// -DZERO_STEP_ODT, each a zero_dtype; ZERO_STEP_ODT == ZERO_F32 means "no 16-bit output" and also
// carries the reduce pass), so that its many kernel variants build in parallel.
//
// Everything here is HBM-bound elementwise streaming (about 0.5 flop per byte), so nothing is
// shaped for MFMA. A tile is SUB groups of 4 consecutive elements per thread, the groups spaced
// block*4 elements apart, so every load instruction of a wave covers one contiguous 1 KiB (fp32)
// or 512 B (16-bit) run. Loads and stores are non-temporal: every byte is touched once per step.
// The Adam kernel runs one single-wave tile per block over the whole tiles of the shard, plus one
// block for a partial last tile.
// Measured on MI355X, one-wave blocks with one group per lane (a 256-element tile) moved this
// 15-stream read/write mix fastest: faster than 2 or 4 groups per lane, 128- or 256-thread blocks,
// grid-stride (persistent) launches and software-pipelined multi-tile blocks.
//
// Vector accesses need only 4-byte alignment: a 16-byte global access on a word boundary is one
// instruction (the hardware ignores the two low address bits of a dword-or-wider access, which is
// also why arrays must be naturally aligned). So fp32 arrays take the vector path at any element
// offset, and so do 16-bit arrays that start on a word. A 16-bit array that starts at an odd element is read as the three words around each
// 4-element group and realigned in registers, and a 16-bit output there is written as whole words
// built across neighbouring lanes (the MIS variants; see Phase in zero_step.h).
//
// Arithmetic is fp32 with every operation rounded on its own: the library is built with
// -ffp-contract=off and HIP's correctly rounded fp32 division and square root, so the results
// equal a plain IEEE evaluation of the same expression order bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "zero_device.h"
#include "zero_step.h"

#if !defined(ZERO_STEP_RDT) || !defined(ZERO_STEP_ODT)
#error "compile once per dtype pair: -DZERO_STEP_RDT=<zero_dtype> -DZERO_STEP_ODT=<zero_dtype>"
#endif

namespace zero {
namespace step {
namespace {

using zero::f32x2;
using zero::f32x4;
using zero::ld;
using zero::st;
using zero::u32x2;

// views that promise only word alignment (see the header comment); the loads and stores below
// take these pointer types directly, so the promise reaches the compiler unchanged
typedef f32x4 f32x4w __attribute__((aligned(4)));
typedef u32x2 u32x2w __attribute__((aligned(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef u32x3 u32x3w __attribute__((aligned(4)));

#if ZERO_NT
#define ZERO_LDW(p) __builtin_nontemporal_load(p)
#define ZERO_STW(p, v) __builtin_nontemporal_store((v), (p))
#else
#define ZERO_LDW(p) (*(p))
#define ZERO_STW(p, v) (*(p) = (v))
#endif
[[maybe_unused]] __device__ __forceinline__ f32x4 ldw4(const float* p) {
  return ZERO_LDW(reinterpret_cast<const f32x4w*>(p));
}
[[maybe_unused]] __device__ __forceinline__ void stw4(float* p, f32x4 v) { ZERO_STW(reinterpret_cast<f32x4w*>(p), v); }
[[maybe_unused]] __device__ __forceinline__ u32x2 ldw2(const uint16_t* p) {
  return ZERO_LDW(reinterpret_cast<const u32x2w*>(p));
}
[[maybe_unused]] __device__ __forceinline__ u32x3 ldw3(const uint16_t* p) {
  return ZERO_LDW(reinterpret_cast<const u32x3w*>(p));
}
[[maybe_unused]] __device__ __forceinline__ void stw2(uint16_t* p, u32x2 v) { ZERO_STW(reinterpret_cast<u32x2w*>(p), v); }

// f(0), f(1), ..., f(N-1) with compile-time indices and no loop in the code. A loop that runs
// once (N = 1) lets loop-invariant code motion promote its stores, and the promoted stores lose
// their non-temporal hint before the loop would be unrolled.
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// Grad scale and, with a table, the step constants from device memory. False when the device
// step t lies outside [1, table_len]: the caller then writes nothing.
__device__ __forceinline__ bool dev_scalars(const DevCtl& dc, StepScalars& sc) {
  sc.gs = *dc.gs;
  if (dc.table != nullptr) {
    const int64_t t = *dc.step;
    if (t < 1 || t > (int64_t)dc.table_len) return false;
    const zero_adam_scalars k = dc.table[t - 1];
    sc.b1 = k.b1;
    sc.b2 = k.b2;
    sc.c1 = k.c1;
    sc.c2 = k.c2;
    sc.ss = k.ss;
    sc.bc = k.bc;
    sc.e = k.e;
    sc.dec = k.dec;
    sc.w = k.w;
  }
  return true;
}

// ---------------------------------------------------------------------------------------------
// element conversions

[[maybe_unused]] __device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

[[maybe_unused]] __device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// fp32 -> 16-bit, round to nearest even, two values packed low-then-high. bf16 uses gfx950's
// v_cvt_pk_bf16_f32: checked against the integer rule (u + 0x7fff + ((u >> 16) & 1)) >> 16, with a
// NaN becoming (u >> 16) | 0x40, on all 2^32 fp32 patterns in the library's floating-point mode.
// binary16 uses the IEEE conversion in the default rounding mode.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int ODT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 x = {a, b};
  if constexpr (ODT == ZERO_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
}

template <int ODT>
__device__ __forceinline__ uint16_t to_out1(float x) {
  if constexpr (ODT == ZERO_BF16) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// two words of packed 16-bit elements -> 4 floats (exact)
template <int RDT>
__device__ __forceinline__ f32x4 widen4(uint32_t w0, uint32_t w1) {
  f32x4 r;
  if constexpr (RDT == ZERO_BF16) {
    r.x = __uint_as_float(w0 << 16);
    r.y = __uint_as_float(w0 & 0xffff0000u);
    r.z = __uint_as_float(w1 << 16);
    r.w = __uint_as_float(w1 & 0xffff0000u);
  } else {
    r.x = f16_to_f32(w0 & 0xffffu);
    r.y = f16_to_f32(w0 >> 16);
    r.z = f16_to_f32(w1 & 0xffffu);
    r.w = f16_to_f32(w1 >> 16);
  }
  return r;
}

// 4 consecutive replica elements starting at element i (i a multiple of 4; the array starts on a
// word)
template <int RDT>
__device__ __forceinline__ f32x4 ld_rep4(const void* base, uint64_t i) {
  if constexpr (RDT == ZERO_F32) {
    return ldw4(static_cast<const float*>(base) + i);
  } else {
    const u32x2 w = ldw2(static_cast<const uint16_t*>(base) + i);
    return widen4<RDT>(w.x, w.y);
  }
}

// The raw words holding 16-bit elements [i, i+4) of a replica: its two words when the array starts
// on a word, else the three words from element i-1 (the word holding i-1 and i also holds an
// element of the array, so it lies in the array's page). realign() then extracts the 4 elements.
[[maybe_unused]] __device__ __forceinline__ u32x3 ld_raw16(const void* base, uint64_t i, bool odd) {
  const uint16_t* b = static_cast<const uint16_t*>(base) + i;
  if (odd) return ldw3(b - 1);
  const u32x2 w = ldw2(b);
  return u32x3{w.x, w.y, 0u};
}

template <int RDT>
__device__ __forceinline__ f32x4 realign(const u32x3& r, uint32_t shift_bytes) {
  return widen4<RDT>(__builtin_amdgcn_alignbyte(r.y, r.x, shift_bytes),
                     __builtin_amdgcn_alignbyte(r.z, r.y, shift_bytes));
}

template <int RDT>
__device__ __forceinline__ float ld_rep1(const void* base, uint64_t i) {
  if constexpr (RDT == ZERO_F32) return static_cast<const float*>(base)[i];
  else if constexpr (RDT == ZERO_BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return f16_to_f32(static_cast<const uint16_t*>(base)[i]);
}

// ---------------------------------------------------------------------------------------------
// replica sum: acc = rep_0 + rep_1 + ... in ascending order (loads issued 8 replicas at a time)

template <int RDT, int RFIX, int SUB, bool MIS>
__device__ __forceinline__ void sum_reps4(const RepPtrs& reps, int nrep, uint64_t rep_odd,
                                          const uint64_t (&idx)[SUB], f32x4 (&acc)[SUB]) {
  constexpr int B = ZERO_REP_BATCH;   // replica loads in flight per lane before their adds
  const int R = RFIX ? RFIX : nrep;
  if constexpr (!MIS || RDT == ZERO_F32) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) acc[u] = ld_rep4<RDT>(reps.p[0], idx[u]);
    for (int k0 = 1; k0 < R; k0 += B) {
      f32x4 t[B][SUB];
#pragma unroll
      for (int j = 0; j < B; ++j)
        if (k0 + j < R) {
#pragma unroll
          for (int u = 0; u < SUB; ++u) t[j][u] = ld_rep4<RDT>(reps.p[k0 + j], idx[u]);
        }
#pragma unroll
      for (int j = 0; j < B; ++j)
        if (k0 + j < R) {
#pragma unroll
          for (int u = 0; u < SUB; ++u) acc[u] = acc[u] + t[j][u];
        }
    }
  } else {
    // 16-bit replicas, some starting at an odd element: every raw load of a batch is issued
    // before any is realigned, so the loads stay in flight together
    u32x3 r0[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) r0[u] = ld_raw16(reps.p[0], idx[u], rep_odd & 1u);
#pragma unroll
    for (int u = 0; u < SUB; ++u) acc[u] = realign<RDT>(r0[u], (uint32_t)(rep_odd & 1u) * 2u);
    for (int k0 = 1; k0 < R; k0 += B) {
      u32x3 t[B][SUB];
#pragma unroll
      for (int j = 0; j < B; ++j)
        if (k0 + j < R) {
          const bool odd = (rep_odd >> (k0 + j)) & 1u;
#pragma unroll
          for (int u = 0; u < SUB; ++u) t[j][u] = ld_raw16(reps.p[k0 + j], idx[u], odd);
        }
#pragma unroll
      for (int j = 0; j < B; ++j)
        if (k0 + j < R) {
          const uint32_t sh = (uint32_t)((rep_odd >> (k0 + j)) & 1u) * 2u;
#pragma unroll
          for (int u = 0; u < SUB; ++u) acc[u] = acc[u] + realign<RDT>(t[j][u], sh);
        }
    }
  }
}

template <int RDT>
__device__ __forceinline__ float sum_reps1(const RepPtrs& reps, int nrep, uint64_t i) {
  float a = ld_rep1<RDT>(reps.p[0], i);
  for (int k = 1; k < nrep; ++k) a = a + ld_rep1<RDT>(reps.p[k], i);
  return a;
}

// 16-bit output of elements [i, i+4). MIS (see k_adam_step) 1: the output starts at an odd
// element; 2: it may (out_odd says). Then the words are (i-1, i), (i+1, i+2) and (i+3, i+4): each
// lane but the first writes the 8 bytes (i-1, i, i+1, i+2) in one store, the element i-1 coming
// over from the lane before it by a shuffle, so a wave's stores cover one contiguous run and only
// the lines at its two ends are shared with the neighbouring waves. The first lane writes i as a
// 16-bit store and (i+1, i+2) as a word, and the last lane also writes i+3 as a 16-bit store, so
// no byte outside the wave's 256 elements is written.
template <int ODT, int MIS>
__device__ __forceinline__ void store_out4(void* out, uint64_t i, const f32x4& p, uint32_t out_odd) {
  const uint32_t lo = pack2<ODT>(p.x, p.y), hi = pack2<ODT>(p.z, p.w);
  uint16_t* o = static_cast<uint16_t*>(out) + i;
  if constexpr (MIS != 0) {
    if (MIS == 1 || out_odd) {
      const uint32_t left = (uint32_t)__shfl_up((int)hi, 1, 64);   // the previous lane's (i-2, i-1)
      const uint32_t mid = __builtin_amdgcn_alignbyte(hi, lo, 2);   // (i+1, i+2)
      const int lane = threadIdx.x & 63;
      // plain (write-back) stores here, not non-temporal ones: the pieces of a line shared with
      // the neighbouring waves then meet in L2 and go to memory as one line. Measured on MI355X
      // for the 7B step: 6.33 ms with non-temporal stores, 5.84 with plain stores at the ends only,
      // 5.61 with plain stores throughout, against 5.55 ms for an aligned slot.
      if (lane != 0) {
        *reinterpret_cast<u32x2w*>(o - 1) = u32x2{__builtin_amdgcn_alignbyte(lo, left, 2), mid};
      } else {
        *o = (uint16_t)(lo & 0xffffu);
        *reinterpret_cast<uint32_t*>(o + 1) = mid;
      }
      if (lane == 63) *(o + 3) = (uint16_t)(hi >> 16);
      return;
    }
  }
  stw2(o, u32x2{lo, hi});
}

// ---------------------------------------------------------------------------------------------
// one element of Adam / AdamW, every operation rounded on its own

template <bool L2>
__device__ __forceinline__ void adam1(float acc, float& p, float& m, float& v, const StepScalars& s) {
  float g = acc * s.gs;
  if (L2) g = g + s.w * p;
  m = s.b1 * m + s.c1 * g;
  v = s.b2 * v + s.c2 * (g * g);
  const float den = sqrtf(v) / s.bc + s.e;
  if (!L2) p = p * s.dec;
  p = p - s.ss * (m / den);
}

// ---------------------------------------------------------------------------------------------
// fused step: replica sum -> Adam/AdamW on master/m/v -> 16-bit cast into the rank's slot
//
// k_adam_step covers whole tiles with vector loads and stores, one tile per block. When the shard
// ends in a partial tile, the TAIL variant's grid has one block more, which walks that remainder
// (fewer than one tile) element by element, so a ragged shard still takes one launch.

// element i of the update: replica sum, Adam, 16-bit cast
template <int RDT, int ODT, bool L2>
__device__ __forceinline__ void adam_elem(const RepPtrs& reps, int nrep, uint64_t i,
                                          const StepScalars& sc, float* __restrict__ P,
                                          float* __restrict__ M, float* __restrict__ V,
                                          void* __restrict__ out) {
  const float a = sum_reps1<RDT>(reps, nrep, i);
  float p = P[i], m = M[i], v = V[i];
  adam1<L2>(a, p, m, v, sc);
  P[i] = p;
  M[i] = m;
  V[i] = v;
  if constexpr (ODT != ZERO_F32) static_cast<uint16_t*>(out)[i] = to_out1<ODT>(p);
}

// MIS 0: every 16-bit array starts on a 4-byte word; 1: the output starts at an odd element and
// the replicas on words; 2: replicas may start at odd elements (Phase.rep_odd) and so may the
// output (Phase.out_odd)
template <int RDT, int ODT, bool L2, int RFIX, bool SKIP, bool TAIL, bool DGS, int MIS>
__global__ __launch_bounds__(kAdamBlock) void k_adam_step(
    RepPtrs reps, int nrep, uint64_t first_tile, StepScalars sc, float* __restrict__ P,
    float* __restrict__ M, float* __restrict__ V, void* __restrict__ out,
    const int32_t* __restrict__ skip, DevCtl dc, uint64_t n, Phase ph) {
  // One tile per block and the grid is exactly the tile count (plus the remainder block with
  // TAIL): no loop bound and no per-block bound check to wait for, so a block's first loads issue
  // right after its arguments arrive.
  if constexpr (SKIP) {
    if (*skip != 0) return;
  }
  if constexpr (DGS) {   // grad scale (and step constants) from device memory
    if (!dev_scalars(dc, sc)) return;
  }
  constexpr uint64_t kTileElems = (uint64_t)kAdamBlock * 4 * ZERO_ADAM_SUB;
  if constexpr (TAIL) {
    if (blockIdx.x == gridDim.x - 1) {   // elements [tile start, n): fewer than one tile
#pragma unroll 1   // kept rolled: its registers must not raise the whole-tile path's budget
      for (uint64_t i = (first_tile + blockIdx.x) * kTileElems + threadIdx.x; i < n; i += kAdamBlock)
        adam_elem<RDT, ODT, L2>(reps, nrep, i, sc, P, M, V, out);
      return;
    }
  }
  constexpr int SUB = ZERO_ADAM_SUB;
  constexpr uint64_t kTile = (uint64_t)kAdamBlock * 4 * SUB;
  const uint64_t base = (first_tile + blockIdx.x) * kTile;
  uint64_t idx[SUB];
#pragma unroll
  for (int u = 0; u < SUB; ++u) idx[u] = base + (uint64_t)u * (kAdamBlock * 4) + threadIdx.x * 4u;
  f32x4 p[SUB], m[SUB], v[SUB], acc[SUB];
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    p[u] = ldw4(P + idx[u]);
    m[u] = ldw4(M + idx[u]);
    v[u] = ldw4(V + idx[u]);
  }
  sum_reps4<RDT, RFIX, SUB, MIS == 2>(reps, nrep, ph.rep_odd, idx, acc);
  unroll<SUB>([&](auto u) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float pq = p[u][q], mq = m[u][q], vq = v[u][q];
      adam1<L2>(acc[u][q], pq, mq, vq, sc);
      p[u][q] = pq;
      m[u][q] = mq;
      v[u][q] = vq;
    }
    stw4(P + idx[u], p[u]);
    stw4(M + idx[u], m[u]);
    stw4(V + idx[u], v[u]);
    if constexpr (ODT != ZERO_F32) store_out4<ODT, MIS>(out, idx[u], p[u], ph.out_odd);
  });
}

// ---------------------------------------------------------------------------------------------
// reduce pass: replica sum -> fp32 gradient, non-finite flag, fp64 squared-norm partials
//
// One single-wave block per tile of kRedTile = 256 elements, the Adam kernel's tile. Thread `lane`
// owns the elements base + lane*4 + q (q < 4) and adds their fp64 squares in that order; the 64
// lane sums are combined by a fixed xor butterfly and lane 0 writes partial[tile]. On MI355X one
// group per lane took 2.4% less time for the 16-replica reduce than two groups and 4.7% less than
// four, as it does for the Adam kernel. The vector path (whole tiles) and the per-element path
// (the ragged last tile) use the same element-to-lane map and order, so a partial depends only on
// the tile's elements. The finish is a fixed two-level sum (zero_shard_sqnorm),
// so the squared norm is bit-reproducible for a given input and n. No atomics: the flag is only
// ever set to 1 by plain stores.

[[maybe_unused]] __device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;  // lane 0's value is the fixed-order result
}

[[maybe_unused]] __device__ __forceinline__ bool nonfinite(float x) {
  return (__float_as_uint(x) & 0x7f800000u) == 0x7f800000u;
}

template <int RDT, int RFIX, bool VEC, bool MIS>
__device__ __forceinline__ void reduce_tile(const RepPtrs& reps, int nrep, uint64_t tile, uint64_t n,
                                            float* __restrict__ G, int32_t* __restrict__ flag,
                                            double* __restrict__ partials, double sq_scale,
                                            uint64_t rep_odd) {
  const uint64_t base = tile * kRedTile;
  double sq = 0.0;
  bool bad = false;
  if constexpr (VEC) {
    const uint64_t idx[1] = {base + threadIdx.x * 4u};
    f32x4 acc[1];
    sum_reps4<RDT, RFIX, 1, MIS>(reps, nrep, rep_odd, idx, acc);
    if (G != nullptr) stw4(G + idx[0], acc[0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bad |= nonfinite(acc[0][q]);
      const double d = (double)acc[0][q] * sq_scale;
      sq += d * d;
    }
  } else {
    for (int q = 0; q < 4; ++q) {
      const uint64_t i = base + threadIdx.x * 4u + q;
      if (i < n) {
        const float a = sum_reps1<RDT>(reps, nrep, i);
        if (G != nullptr) G[i] = a;
        bad |= nonfinite(a);
        const double d = (double)a * sq_scale;
        sq += d * d;
      }
    }
  }
  if (flag != nullptr && __ballot(bad) != 0 && threadIdx.x == 0) *flag = 1;
  if (partials != nullptr) {
    sq = wave_sum(sq);
    if (threadIdx.x == 0) partials[tile] = sq;
  }
}

// whole tiles with vector loads; with TAIL the grid has one block more, which takes the partial
// last tile element by element (same element order, so its partial is the same)
template <int RDT, int RFIX, bool TAIL, bool MIS>
__global__ __launch_bounds__(64) void k_reduce(RepPtrs reps, int nrep, uint64_t first_tile,
                                               uint64_t n, float* __restrict__ G,
                                               int32_t* __restrict__ flag,
                                               double* __restrict__ partials, double sq_scale,
                                               uint64_t rep_odd) {
  if constexpr (TAIL) {
    if (blockIdx.x == gridDim.x - 1) {
      reduce_tile<RDT, 0, false, false>(reps, nrep, first_tile + blockIdx.x, n, G, flag, partials,
                                        sq_scale, 0);
      return;
    }
  }
  reduce_tile<RDT, RFIX, true, MIS>(reps, nrep, first_tile + blockIdx.x, n, G, flag, partials,
                                    sq_scale, rep_odd);
}

// ---------------------------------------------------------------------------------------------
// Adam dispatch

template <int RDT, int ODT, bool L2, int RFIX, bool SKIP, bool TAIL, int MIS>
void launch_adam_grid(const AdamArgs& a, uint64_t t0, uint64_t blocks) {
  if (a.dc.gs != nullptr)
    hipLaunchKernelGGL((k_adam_step<RDT, ODT, L2, RFIX, SKIP, TAIL, true, MIS>),
                       dim3((unsigned)blocks), dim3(kAdamBlock), 0, a.stream, a.reps, a.nrep, t0,
                       a.sc, a.P, a.M, a.V, a.out, a.skip, a.dc, a.n, a.ph);
  else
    hipLaunchKernelGGL((k_adam_step<RDT, ODT, L2, RFIX, SKIP, TAIL, false, MIS>),
                       dim3((unsigned)blocks), dim3(kAdamBlock), 0, a.stream, a.reps, a.nrep, t0,
                       a.sc, a.P, a.M, a.V, a.out, a.skip, a.dc, a.n, a.ph);
}

template <int RDT, int ODT, bool L2, int RFIX, int MIS>
void launch_adam_tiles(const AdamArgs& a) {
  // Grids of at most kMaxGrid tiles, each told where its first tile is. A partial last tile
  // rides on the last grid as one extra block (TAIL); a shard shorter than one tile is then a
  // grid of that block alone.
  const bool tail = a.fused_tail;
  uint64_t t0 = 0;
  do {
    const uint64_t g = a.ntiles - t0 < kMaxGrid ? a.ntiles - t0 : kMaxGrid;
    const bool last = t0 + g == a.ntiles;
    if (last && tail) {
      if (a.skip != nullptr) launch_adam_grid<RDT, ODT, L2, RFIX, true, true, MIS>(a, t0, g + 1);
      else launch_adam_grid<RDT, ODT, L2, RFIX, false, true, MIS>(a, t0, g + 1);
    } else if (g > 0) {
      if (a.skip != nullptr) launch_adam_grid<RDT, ODT, L2, RFIX, true, false, MIS>(a, t0, g);
      else launch_adam_grid<RDT, ODT, L2, RFIX, false, false, MIS>(a, t0, g);
    }
    t0 += g;
  } while (t0 < a.ntiles);
}

template <int RDT, int ODT, bool L2, int MIS>
void launch_adam_by_count(const AdamArgs& a) {
  switch (a.nrep) {
    case 1: launch_adam_tiles<RDT, ODT, L2, 1, MIS>(a); break;
    case 8: launch_adam_tiles<RDT, ODT, L2, 8, MIS>(a); break;
    case 16: launch_adam_tiles<RDT, ODT, L2, 16, MIS>(a); break;
    case 64: launch_adam_tiles<RDT, ODT, L2, 64, MIS>(a); break;
    default: launch_adam_tiles<RDT, ODT, L2, 0, MIS>(a); break;
  }
}

template <int RDT, int ODT, bool L2>
void launch_adam_l2(const AdamArgs& a) {
  // only 16-bit replicas and a 16-bit output can start at an odd element
  if constexpr (RDT != ZERO_F32) {
    if (a.ph.rep_odd != 0) return launch_adam_by_count<RDT, ODT, L2, 2>(a);
  }
  if constexpr (ODT != ZERO_F32) {
    if (a.ph.out_odd != 0) return launch_adam_by_count<RDT, ODT, L2, 1>(a);
  }
  launch_adam_by_count<RDT, ODT, L2, 0>(a);
}

// ---------------------------------------------------------------------------------------------
// reduce dispatch

// whole tiles [0, full) as vector tiles in grids of at most kMaxGrid blocks; a partial last tile
// rides on the last grid as one extra block (a shard shorter than one tile is a grid of that block
// alone)
template <int RDT, int RFIX, bool MIS>
void launch_reduce_vec(const ReduceArgs& a, uint64_t full, bool tail) {
  uint64_t t = 0;
  do {
    const uint64_t g = full - t < kMaxGrid ? full - t : kMaxGrid;
    if (tail && t + g == full)
      hipLaunchKernelGGL((k_reduce<RDT, RFIX, true, MIS>), dim3((unsigned)(g + 1)), dim3(64), 0,
                         a.stream, a.reps, a.nrep, t, a.n, a.G, a.flag, a.partials, a.sq_scale,
                         a.ph.rep_odd);
    else if (g > 0)
      hipLaunchKernelGGL((k_reduce<RDT, RFIX, false, MIS>), dim3((unsigned)g), dim3(64), 0,
                         a.stream, a.reps, a.nrep, t, a.n, a.G, a.flag, a.partials, a.sq_scale,
                         a.ph.rep_odd);
    t += g;
  } while (t < full);
}

template <int RDT, bool MIS>
void launch_reduce_by_count(const ReduceArgs& a, uint64_t full, bool tail) {
  switch (a.nrep) {
    case 1: launch_reduce_vec<RDT, 1, MIS>(a, full, tail); break;
    case 8: launch_reduce_vec<RDT, 8, MIS>(a, full, tail); break;
    case 16: launch_reduce_vec<RDT, 16, MIS>(a, full, tail); break;
    case 64: launch_reduce_vec<RDT, 64, MIS>(a, full, tail); break;
    default: launch_reduce_vec<RDT, 0, MIS>(a, full, tail); break;
  }
}

}  // namespace

template <int RDT, int ODT>
void launch_adam(const AdamArgs& a, bool l2) {
  if (l2) launch_adam_l2<RDT, ODT, true>(a);
  else launch_adam_l2<RDT, ODT, false>(a);
}

template <int RDT>
void launch_reduce(const ReduceArgs& a) {
  const uint64_t all = red_tiles(a.n);
  const uint64_t full = a.n / kRedTile;
  const bool tail = all > full;
  if (RDT != ZERO_F32 && a.ph.rep_odd != 0) launch_reduce_by_count<RDT, RDT != ZERO_F32>(a, full, tail);
  else launch_reduce_by_count<RDT, false>(a, full, tail);
}

template void launch_adam<ZERO_STEP_RDT, ZERO_STEP_ODT>(const AdamArgs&, bool);
#if ZERO_STEP_ODT == ZERO_F32
template void launch_reduce<ZERO_STEP_RDT>(const ReduceArgs&);
#endif

}  // namespace step
}  // namespace zero
