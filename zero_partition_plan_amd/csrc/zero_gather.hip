// ZeRO-3 parameter gather on gfx950: rebuild one layer's contiguous parameters from the rank
// shards that hold them ("ZeRO 优化器的三个阶段深度对比", section 三; "ZeRO Optimization", core
// operations: before a layer runs, its full parameters are all-gathered from every rank's shard).
//
// The flat space is the nd shards of S elements laid end to end, so a layer's range [begin,
// begin + count) is at most nd contiguous segments, one per shard it touches. One launch copies
// them all: a table in the kernel arguments gives each segment's source, its offset in the output
// and its first tile, and every single-wave block copies one 2 KiB tile of one segment (two 16-byte
// non-temporal loads and stores per lane). A segment whose source or destination is not 16-byte
// aligned, and the ragged last tile of each segment, are copied element by element. Pure data
// movement: 2 x elem_bytes of HBM traffic per element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_device.h"
#include "zero_internal.h"

namespace {

using zero::ld;
using zero::st;
using zero::u32x4;

constexpr int kMaxShards = ZERO_MAX_SHARDS;
constexpr uint64_t kTileBytes = 64 * 16 * 2;   // per single-wave block
constexpr uint64_t kMaxGrid = 1u << 24;

struct Segs {
  const unsigned char* src[kMaxShards];
  uint64_t dst[kMaxShards + 1];    // output element where segment k starts; dst[nseg] = count
  uint64_t tile0[kMaxShards + 1];  // first tile of segment k; tile0[nseg] = total tiles
  uint32_t aligned[kMaxShards];    // 1: the segment's source and destination are 16-byte aligned
  uint32_t nseg;
};

template <int EB>
__global__ __launch_bounds__(64) void k_gather(Segs sg, uint64_t first_tile,
                                               unsigned char* __restrict__ out) {
  constexpr uint64_t kTileElems = kTileBytes / EB;
  const uint64_t t = first_tile + blockIdx.x;
  uint32_t k = 0;  // the segment holding tile t (uniform across the wave)
  while (k + 1 < sg.nseg && sg.tile0[k + 1] <= t) ++k;
  const uint64_t lt = t - sg.tile0[k];
  const uint64_t seg_len = sg.dst[k + 1] - sg.dst[k];
  const uint64_t e0 = lt * kTileElems;
  const uint64_t len = seg_len - e0 < kTileElems ? seg_len - e0 : kTileElems;
  const unsigned char* src = sg.src[k] + e0 * EB;
  unsigned char* dst = out + (sg.dst[k] + e0) * EB;
  if (sg.aligned[k] && len == kTileElems) {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    u32x4* d4 = reinterpret_cast<u32x4*>(dst);
    const u32x4 a = ld(s4 + threadIdx.x), b = ld(s4 + 64 + threadIdx.x);
    st(d4 + threadIdx.x, a);
    st(d4 + 64 + threadIdx.x, b);
  } else if constexpr (EB == 2) {
    const uint16_t* s = reinterpret_cast<const uint16_t*>(src);
    uint16_t* d = reinterpret_cast<uint16_t*>(dst);
    for (uint64_t i = threadIdx.x; i < len; i += 64) d[i] = s[i];
  } else {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);
    for (uint64_t i = threadIdx.x; i < len; i += 64) d[i] = s[i];
  }
}

}  // namespace

extern "C" {

zero_status zero_gather_params(const void* const* d_shards, uint32_t nd, uint64_t shard_elems,
                               uint32_t elem_bytes, uint64_t begin, uint64_t count, void* d_out,
                               void* stream) {
  const char* fn = "zero_gather_params";
  if (!d_shards) return zero::fail(ZERO_E_INVAL, "%s: shard array is NULL", fn);
  if (nd == 0 || nd > ZERO_MAX_SHARDS)
    return zero::fail(ZERO_E_INVAL, "%s: nd %u outside 1..%d", fn, nd, ZERO_MAX_SHARDS);
  if (elem_bytes != 2 && elem_bytes != 4)
    return zero::fail(ZERO_E_INVAL, "%s: elem_bytes %u is not 2 or 4", fn, elem_bytes);
  uint64_t total, end, bytes;
  if (__builtin_mul_overflow(shard_elems, (uint64_t)nd, &total) ||
      __builtin_add_overflow(begin, count, &end) ||
      __builtin_mul_overflow(total, (uint64_t)elem_bytes, &bytes))
    return zero::fail(ZERO_E_OVERFLOW, "%s: sizes do not fit in 64 bits", fn);
  if (end > total)
    return zero::fail(ZERO_E_INVAL, "%s: range [%llu, %llu) outside the %llu gathered elements", fn,
                      (unsigned long long)begin, (unsigned long long)end, (unsigned long long)total);
  if (count == 0) return zero::ok();
  if (!d_out) return zero::fail(ZERO_E_INVAL, "%s: out is NULL", fn);

  const uint64_t tile_elems = kTileBytes / elem_bytes;
  Segs sg{};
  const uint64_t S = shard_elems;
  const uint32_t r0 = (uint32_t)(begin / S), r1 = (uint32_t)((end - 1) / S);
  uint64_t tiles = 0;
  for (uint32_t r = r0; r <= r1; ++r) {
    if (!d_shards[r]) return zero::fail(ZERO_E_INVAL, "%s: shard %u is NULL", fn, r);
    const uint64_t lo = begin > (uint64_t)r * S ? begin : (uint64_t)r * S;
    const uint64_t hi = end < (uint64_t)(r + 1) * S ? end : (uint64_t)(r + 1) * S;
    const unsigned char* src =
        static_cast<const unsigned char*>(d_shards[r]) + (lo - (uint64_t)r * S) * elem_bytes;
    // the output must not overlap the part of any shard it reads
    if (zero::overlaps(d_out, count * elem_bytes, src, (hi - lo) * elem_bytes))
      return zero::fail(ZERO_E_INVAL, "%s: out overlaps shard %u", fn, r);
    const uint32_t k = r - r0;
    sg.src[k] = src;
    sg.dst[k] = lo - begin;
    sg.tile0[k] = tiles;
    const uintptr_t d = reinterpret_cast<uintptr_t>(d_out) + (lo - begin) * elem_bytes;
    sg.aligned[k] = ((reinterpret_cast<uintptr_t>(src) | d) & 15u) == 0;
    tiles += (hi - lo + tile_elems - 1) / tile_elems;
  }
  sg.nseg = r1 - r0 + 1;
  sg.dst[sg.nseg] = count;
  sg.tile0[sg.nseg] = tiles;

  hipStream_t strm = static_cast<hipStream_t>(stream);
  unsigned char* out = static_cast<unsigned char*>(d_out);
  (void)hipGetLastError();
  for (uint64_t t0 = 0; t0 < tiles; t0 += kMaxGrid) {
    const uint64_t g = tiles - t0 < kMaxGrid ? tiles - t0 : kMaxGrid;
    if (elem_bytes == 2)
      hipLaunchKernelGGL(k_gather<2>, dim3((unsigned)g), dim3(64), 0, strm, sg, t0, out);
    else
      hipLaunchKernelGGL(k_gather<4>, dim3((unsigned)g), dim3(64), 0, strm, sg, t0, out);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return zero::fail(ZERO_E_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return zero::ok();
}

}  // extern "C"
