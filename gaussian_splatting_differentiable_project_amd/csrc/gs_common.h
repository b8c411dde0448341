// Shared constants and wave64 helpers of the gfx950 kernels.
//
// The geometry constants live in one header because the visibility pass
// and the compaction pass must agree on them: both map bit b of the
// 64-bit mask word w to pair 64 w + b and both launch GS_MASK_GROUP lanes
// per work-group ([VRAM] "Bitmask compaction": the block size is a shared
// constant, otherwise the bit-to-word mapping silently shifts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gs.h"

namespace gs {

constexpr int kWave = 64;                  // CDNA wavefront width
constexpr int kMaskGroup = GS_MASK_GROUP;  // 128 pairs = 2 waves
constexpr int kTile = GS_TILE;             // 16 x 16 pixels
constexpr int kTilePix = kTile * kTile;
constexpr int kRow = GS_ROW;               // floats per screen row
constexpr float kNear = 0.01f;
constexpr double kBlur = 0.3;              // px^2 added to the 2D covariance (0.3 in the evaluating precision)
constexpr float kAlphaMax = 0.99f;
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kTStop = 1e-4f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kQ16 = 65535u;          // 16-bit box grid steps

// Radix sort geometry: 8-bit digits, 256 lanes, 16 keys per lane.
constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kSortThreads = 256;
constexpr int kSortChunks = 1024;  // count/scatter blocks per pass: 4 per CU, all resident
constexpr int kSortGroup = 32;                        // chunks per group total
constexpr int kSortGroups = kSortChunks / kSortGroup;

// Scan geometry (decoupled look-back): 256 lanes x 16 values.
constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanThreads * kScanItems;

// Look-back words: [63:62] status, [61:56] epoch tag, [55:0] value.
constexpr uint64_t kLbAgg = 1ull << 62;
constexpr uint64_t kLbPrefix = 2ull << 62;
constexpr uint64_t kLbValueMask = (1ull << 56) - 1;
constexpr uint32_t kSpinLimit = 1u << 24;  // bounded waits: a bug reports, never hangs

__device__ __forceinline__ uint64_t lb_word(uint64_t status, uint32_t tag, uint64_t v) {
  return status | (uint64_t(tag & 63u) << 56) | (v & kLbValueMask);
}
__device__ __forceinline__ uint32_t lb_tag(uint64_t w) { return uint32_t(w >> 56) & 63u; }
__device__ __forceinline__ uint64_t lb_status(uint64_t w) { return w & (3ull << 62); }

__device__ __forceinline__ void lb_store(uint64_t* p, uint64_t w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t lb_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix of everything before block `blk` for one counter of a
// decoupled look-back chain. `lb` is indexed [block * stride]. The block's
// own aggregate must already be published. Spins are bounded: on timeout
// *err is set and 0 is returned (the caller's output is then garbage but
// every wave still exits).
__device__ __forceinline__ uint64_t lookback_prefix(const uint64_t* lb, int64_t blk,
                                                    int64_t stride, uint32_t tag,
                                                    int* err) {
  uint64_t acc = 0;
  int64_t p = blk - 1;
  uint32_t spins = 0;
  while (p >= 0) {
    uint64_t w = lb_load(lb + p * stride);
    if (lb_tag(w) != tag || lb_status(w) == 0) {
      if (++spins > kSpinLimit) {
        atomicOr(err, 1);
        return 0;
      }
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    acc += w & kLbValueMask;
    if (lb_status(w) == kLbPrefix) break;
    --p;
  }
  return acc;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Non-temporal vector stores, for outputs written once and not read again
// by the kernel that writes them (the sorted list's lines, the gradient
// rows): they stream past the caches instead of taking lines from data
// the kernel still reads.
__device__ __forceinline__ void store_stream(uint32_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, p);
}
__device__ __forceinline__ void store_stream(float* p, float v) {
  __builtin_nontemporal_store(v, p);
}
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_stream(float4* p, float4 v) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Lane `src`'s value of a 64-bit register (src wave-uniform).
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int src) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), src));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), src));
  return (uint64_t(hi) << 32) | lo;
}

// Sum of a float over the 64 lanes; every lane gets the total.
// Row sums (16 lanes) by DPP row rotations, then the four row sums by
// readlane.
__device__ __forceinline__ float wave_sum(float v) {
  int x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false));  // row_ror:8
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false));  // row_ror:4
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false));  // row_ror:2
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false));  // row_ror:1
  x = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 48));
  return (r0 + r1) + (r2 + r3);
}

// Inclusive prefix sum of a uint64 over the 64 lanes (shuffle-based).
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  const int l = __lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint64_t t = __shfl_up(v, o, kWave);
    if (l >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  const int l = __lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t t = __shfl_up(v, o, kWave);
    if (l >= o) v += t;
  }
  return v;
}

// Exclusive prefix of everything before block `blk` for a single-counter
// decoupled look-back chain (lb[block]), computed by one whole wave: each
// step loads the 64 nearest unresolved predecessors at once, so a walk
// over d predecessors costs about d/64 round trips instead of d. Every
// lane of the wave must call it; all get the result. Spins are bounded
// (on timeout *err is set and 0 is returned).
__device__ __forceinline__ uint64_t lookback_prefix_wave(const uint64_t* lb, int64_t blk,
                                                         uint32_t tag, int* err) {
  const int lane = __lane_id();
  uint64_t acc = 0;
  int64_t p = blk - 1;  // nearest predecessor not yet summed
  uint32_t spins = 0;
  while (p >= 0) {
    const int64_t q = p - lane;
    const uint64_t w = q >= 0 ? lb_load(lb + q) : (kLbPrefix | (uint64_t(tag & 63u) << 56));
    const bool ready = lb_tag(w) == tag && lb_status(w) != 0;
    const bool pref = ready && lb_status(w) == kLbPrefix;
    const uint64_t not_ready = __ballot(!ready);
    const uint64_t prefixes = __ballot(pref);
    // lanes up to and including the nearest inclusive prefix
    const int first_pref = prefixes ? __builtin_ctzll(prefixes) : 64;
    const uint64_t upto = first_pref >= 63 ? ~0ull : ((2ull << first_pref) - 1);
    if (not_ready & upto) {
      // sum the ready run before the first gap, then wait on the gap
      const int gap = __builtin_ctzll(not_ready);
      const uint64_t take = gap == 0 ? 0ull : (~0ull >> (64 - gap));
      uint64_t v = ((take >> lane) & 1ull) ? (w & kLbValueMask) : 0ull;
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
      acc += v;
      p -= gap;
      if (gap == 0) {
        if (++spins > kSpinLimit) {
          if (lane == 0) atomicOr(err, 1);
          return 0;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      continue;
    }
    uint64_t v = ((upto >> lane) & 1ull) ? (w & kLbValueMask) : 0ull;
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    acc += v;
    if (prefixes) break;
    p -= 64;
  }
  return acc;
}

// Exclusive prefix over the 256 lanes of a 4-wave block; *total gets the
// block sum. s_w holds one word per wave. Every lane must call it; it
// synchronizes the block once.
__device__ __forceinline__ uint64_t block_excl_scan_u64(uint64_t v, uint64_t* s_w /*[4]*/,
                                                        uint64_t* total) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t incl = wave_incl_scan_u64(v);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  uint64_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint64_t t = s_w[w];
    off += (w < wave) ? t : 0ull;
    tot += t;
  }
  *total = tot;
  return off + incl - v;
}

__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* s_w, uint32_t* total) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t incl = wave_incl_scan_u32(v);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t t = s_w[w];
    off += (w < wave) ? t : 0u;
    tot += t;
  }
  *total = tot;
  return off + incl - v;
}

}  // namespace gs
