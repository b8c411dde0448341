// Tile intersection: count, emit, tile ranges.
//
// [VRAM] "The 4 GiB rule and the 2^31 limit": the exact number of
// (splat, tile) intersections is accumulated in 64 bits and checked on
// the host before anything is sized by it, the emit pass never writes
// past the real allocation, and every buffer whose length follows nnz or
// n_isects is addressed with 64-bit offsets. [VRAM] "16-bit packed AABB":
// the tile rectangle is decoded from the 16-bit box codes. [BWD] section 4:
// the tile offsets are kept for the backward.
//
// The sort is factored: slots are first sorted by their 32-bit depth key
// (nnz elements), intersections are then emitted in that order and sorted
// stably by tile id alone. Because each slot meets a tile at most once,
// the result is exactly the stable sort of (tile << 32) | depth keys in
// slot order, with a fraction of the bytes moved per intersection.
#include "gs_internal.h"

namespace gs {

namespace {

struct TileRect {
  uint32_t tx0, ty0, tx1, ty1;  // [tx0, tx1) x [ty0, ty1)
};

// Decoded edge = q * extent / 65535, so with 16-pixel tiles the first tile
// is floor(q0 * extent / (16 * 65535)) and the end is the ceiling of the
// same for q1: integer arithmetic only.
__device__ __forceinline__ TileRect rect_of(uint2 box, uint32_t W, uint32_t H) {
  constexpr uint64_t D = uint64_t(kTile) * kQ16;
  const uint64_t qx0 = box.x & 0xFFFFu, qy0 = box.x >> 16;
  const uint64_t qx1 = box.y & 0xFFFFu, qy1 = box.y >> 16;
  TileRect r;
  r.tx0 = uint32_t(qx0 * W / D);
  r.ty0 = uint32_t(qy0 * H / D);
  r.tx1 = uint32_t((qx1 * W + D - 1) / D);
  r.ty1 = uint32_t((qy1 * H + D - 1) / D);
  return r;
}

__device__ __forceinline__ uint32_t rect_count(const TileRect& r) {
  const uint32_t wx = r.tx1 > r.tx0 ? r.tx1 - r.tx0 : 0u;
  const uint32_t wy = r.ty1 > r.ty0 ? r.ty1 - r.ty0 : 0u;
  return wx * wy;
}

// Per slot: depth key bits and identity value for the depth sort, and
// the exact 64-bit total of tile counts (one atomic per work-group).
__global__ __launch_bounds__(256) void k_isect_prep(uint64_t nnz, const float* __restrict__ screen,
                                                   const uint2* __restrict__ aabb16, uint32_t W,
                                                   uint32_t H, uint32_t* __restrict__ dkeys,
                                                   uint32_t* __restrict__ dvals, uint64_t* total) {
  __shared__ uint64_t s_w[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint64_t n = 0;
  // grid-stride, so few blocks contend for the one 64-bit total
  const uint64_t stride = uint64_t(gridDim.x) * 256;
  for (uint64_t i = uint64_t(blockIdx.x) * 256 + tid; i < nnz; i += stride) {
    dkeys[i] = __float_as_uint(screen[i * kRow + 6]);
    dvals[i] = uint32_t(i);
    n += rect_count(rect_of(aabb16[i], W, H));
  }
  const uint64_t incl = wave_incl_scan_u64(n);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    const uint64_t b = s_w[0] + s_w[1] + s_w[2] + s_w[3];
    if (b) atomicAdd(reinterpret_cast<unsigned long long*>(total), (unsigned long long)b);
  }
}

// Intersections of the slots in depth order, with their offsets found on
// the way. Block b takes positions [b*512, (b+1)*512) of the depth order
// (position i holds slot order[i]); it counts their tiles, scans the
// counts, gets the number of entries of all earlier positions from a
// single-word decoupled look-back, and then writes its entries with
// consecutive lanes on consecutive entries: lane e finds its slot by a
// binary search over the block's offsets in LDS. Writes are clamped to
// `cap` entries. The look-back words and the ticket must start at zero.
constexpr int kEmitItems = 2;
constexpr int kEmitSlots = 256 * kEmitItems;

__global__ __launch_bounds__(256) void k_isect_emit(
    uint64_t nnz, const uint32_t* __restrict__ order, const uint2* __restrict__ aabb16,
    const int64_t* __restrict__ cam_off, int C, uint32_t W, uint32_t H, uint32_t tiles_x,
    uint32_t T, uint64_t cap, uint32_t* __restrict__ tkeys, uint32_t* __restrict__ tvals,
    uint64_t* lb, uint32_t* ticket, int* err) {
  __shared__ uint32_t s_blk;
  __shared__ uint64_t s_w[4];
  __shared__ uint64_t s_prefix;
  __shared__ uint64_t s_off[kEmitSlots + 1];  // block-local exclusive entry offsets
  __shared__ uint32_t s_slot[kEmitSlots];
  __shared__ uint32_t s_base[kEmitSlots];     // camera tile base + first tile of the rect
  __shared__ uint32_t s_wx[kEmitSlots];       // rect width in tiles
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid == 0) s_blk = atomicAdd(ticket, 1u);
  __syncthreads();
  const uint64_t blk = s_blk;
  const uint64_t base = blk * kEmitSlots;
  // slot data, read with consecutive lanes on consecutive positions
#pragma unroll
  for (int j = 0; j < kEmitItems; ++j) {
    const int li = j * 256 + tid;
    const uint64_t i = base + li;
    uint32_t k = 0, slot = 0, b0 = 0, wx = 0;
    if (i < nnz) {
      slot = order[i];
      // camera of the slot: cameras own consecutive slot ranges
      int lo = 0, hi = C - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (int64_t(slot) >= cam_off[mid]) lo = mid; else hi = mid - 1;
      }
      const TileRect r = rect_of(aabb16[slot], W, H);
      k = rect_count(r);
      wx = r.tx1 > r.tx0 ? r.tx1 - r.tx0 : 1u;
      b0 = uint32_t(lo) * T + r.ty0 * tiles_x + r.tx0;
    }
    s_slot[li] = slot;
    s_base[li] = b0;
    s_wx[li] = wx;
    s_off[li] = k;  // counts for now
  }
  __syncthreads();
  // exclusive scan of the 1024 counts: four consecutive ones per lane
  uint64_t c[kEmitItems], sum = 0;
#pragma unroll
  for (int j = 0; j < kEmitItems; ++j) {
    c[j] = s_off[tid * kEmitItems + j];
    sum += c[j];
  }
  const uint64_t incl = wave_incl_scan_u64(sum);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  uint64_t woff = 0, btot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    woff += (w < wave) ? s_w[w] : 0ull;
    btot += s_w[w];
  }
  uint64_t run = woff + incl - sum;
#pragma unroll
  for (int j = 0; j < kEmitItems; ++j) {
    s_off[tid * kEmitItems + j] = run;
    run += c[j];
  }
  if (wave == 0) {
    uint64_t prefix = 0;
    if (blk == 0) {
      if (lane == 0) lb_store(lb, lb_word(kLbPrefix, 1, btot));
    } else {
      if (lane == 0) lb_store(lb + blk, lb_word(kLbAgg, 1, btot));
      prefix = lookback_prefix_wave(lb, int64_t(blk), 1, err);
      if (lane == 0) lb_store(lb + blk, lb_word(kLbPrefix, 1, prefix + btot));
    }
    if (lane == 0) {
      s_off[kEmitSlots] = btot;
      s_prefix = prefix;
    }
  }
  __syncthreads();
  const uint64_t prefix = s_prefix;
  for (uint64_t e = tid; e < btot; e += 256) {
    // last position whose offset is <= e (a position with no entries has
    // the same offset as the next one, so the search lands on the owner)
    int lo = 0, hi = kEmitSlots - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= e) lo = mid; else hi = mid - 1;
    }
    const uint64_t o = prefix + e;
    if (o < cap) {
      const uint32_t k = uint32_t(e - s_off[lo]);
      const uint32_t wx = s_wx[lo];
      const uint32_t dy = k / wx, dx = k - dy * wx;
      tkeys[o] = s_base[lo] + dy * tiles_x + dx;
      tvals[o] = s_slot[lo];
    }
  }
}

// tile_offsets[t] = first sorted position whose tile id is >= t.
// Grid-stride over the n + 1 boundaries: a dispatch's work-item count is
// a 32-bit quantity, and n_isects can exceed 2^32.
__global__ __launch_bounds__(256) void k_tile_ranges(const uint32_t* __restrict__ tkeys,
                                                    uint64_t n, uint64_t n_tiles,
                                                    int64_t* __restrict__ toff) {
  const uint64_t stride = uint64_t(gridDim.x) * 256;
  for (uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x; i <= n; i += stride) {
    // ids are < n_tiles by construction; the clamps only keep the writes
    // inside toff[0..n_tiles] whatever the keys hold
    uint64_t cur = i < n ? tkeys[i] : n_tiles;
    cur = cur < n_tiles ? cur : n_tiles;
    int64_t prev = i > 0 ? int64_t(tkeys[i - 1]) : -1;
    prev = prev < int64_t(n_tiles) ? prev : int64_t(n_tiles);
    for (int64_t t = prev + 1; t <= int64_t(cur); ++t) toff[t] = int64_t(i);
  }
}

__global__ __launch_bounds__(256) void k_compose_keys(const uint32_t* __restrict__ tkeys,
                                                     const uint32_t* __restrict__ ids,
                                                     const float* __restrict__ screen, uint64_t n,
                                                     uint64_t* __restrict__ out) {
  const uint64_t stride = uint64_t(gridDim.x) * 256;
  for (uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
    const uint32_t s = ids[i];
    out[i] = (uint64_t(tkeys[i]) << 32) | __float_as_uint(screen[uint64_t(s) * kRow + 6]);
  }
}

// Keys for the raster launch order: tiles with more entries first (the
// key is 0xFFFF minus the entry count, saturated), values are tile ids.
__global__ __launch_bounds__(256) void k_tile_order_keys(const int64_t* __restrict__ toff,
                                                        uint64_t n_tiles,
                                                        uint32_t* __restrict__ keys,
                                                        uint32_t* __restrict__ vals) {
  const uint64_t stride = uint64_t(gridDim.x) * 256;
  for (uint64_t t = uint64_t(blockIdx.x) * 256 + threadIdx.x; t < n_tiles; t += stride) {
    const int64_t n = toff[t + 1] - toff[t];
    keys[t] = 0xFFFFu - uint32_t(n < 0xFFFF ? n : 0xFFFF);
    vals[t] = uint32_t(t);
  }
}

inline uint32_t grid_for(uint64_t n) { return uint32_t((n + 255) / 256); }
// Blocks for a grid-stride loop over n elements.
inline uint32_t grid_stride_blocks(uint64_t n) {
  const uint64_t b = (n + 255) / 256;
  return uint32_t(b < 65536 ? (b ? b : 1) : 65536);
}

}  // namespace

hipError_t launch_isect_prep(uint64_t nnz, const float* screen, const uint32_t* aabb16, int W,
                             int H, uint32_t* dkeys, uint32_t* dvals, uint64_t* total,
                             hipStream_t s) {
  if (nnz == 0) return hipSuccess;
  uint32_t blocks = grid_for(nnz);
  if (blocks > 1024) blocks = 1024;
  ProfScope prof("k_isect_prep", s);
  hipLaunchKernelGGL(k_isect_prep, dim3(blocks), dim3(256), 0, s, nnz, screen,
                     reinterpret_cast<const uint2*>(aabb16), uint32_t(W), uint32_t(H), dkeys,
                     dvals, total);
  return hipGetLastError();
}

hipError_t launch_isect_emit(uint64_t nnz, const uint32_t* order, const uint32_t* aabb16,
                             const int64_t* cam_off, int C, int W, int H, uint64_t cap,
                             uint32_t* tkeys, uint32_t* tvals, uint64_t* lb, uint32_t* ticket,
                             int* err, hipStream_t s) {
  if (nnz == 0) return hipSuccess;
  const uint64_t blocks = (nnz + kEmitSlots - 1) / kEmitSlots;
  if (!fits_dispatch(blocks, 256)) return hipErrorInvalidConfiguration;
  const uint32_t tiles_x = uint32_t((W + kTile - 1) / kTile);
  const uint32_t T = tiles_x * uint32_t((H + kTile - 1) / kTile);
  ProfScope prof("k_isect_emit", s);
  hipLaunchKernelGGL(k_isect_emit, dim3(uint32_t(blocks)), dim3(256), 0, s, nnz, order,
                     reinterpret_cast<const uint2*>(aabb16), cam_off, C, uint32_t(W),
                     uint32_t(H), tiles_x, T, cap, tkeys, tvals, lb, ticket, err);
  return hipGetLastError();
}

uint64_t isect_emit_lookback_words(uint64_t nnz) { return (nnz + kEmitSlots - 1) / kEmitSlots + 1; }

hipError_t launch_tile_ranges(const uint32_t* tkeys, uint64_t n, uint64_t n_tiles, int64_t* toff,
                              hipStream_t s) {
  ProfScope prof("k_tile_ranges", s);
  hipLaunchKernelGGL(k_tile_ranges, dim3(grid_stride_blocks(n + 1)), dim3(256), 0, s, tkeys, n, n_tiles,
                     toff);
  return hipGetLastError();
}

hipError_t launch_tile_order_keys(const int64_t* toff, uint64_t n_tiles, uint32_t* keys,
                                  uint32_t* vals, hipStream_t s) {
  if (n_tiles == 0) return hipSuccess;
  ProfScope prof("k_tile_order_keys", s);
  hipLaunchKernelGGL(k_tile_order_keys, dim3(grid_stride_blocks(n_tiles)), dim3(256), 0, s, toff,
                     n_tiles, keys, vals);
  return hipGetLastError();
}

hipError_t launch_compose_keys(const uint32_t* tkeys, const uint32_t* ids, const float* screen,
                               uint64_t n, uint64_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  ProfScope prof("k_compose_keys", s);
  hipLaunchKernelGGL(k_compose_keys, dim3(grid_stride_blocks(n)), dim3(256), 0, s, tkeys, ids, screen, n,
                     out);
  return hipGetLastError();
}

}  // namespace gs
