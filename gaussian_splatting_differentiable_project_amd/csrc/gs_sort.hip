// Device-wide scan and stable LSD radix sort for gfx950.
//
// [VRAM] "Bitmask compaction" scans the C*N/128 work-group counts;
// [VRAM] "The 4 GiB rule and the 2^31 limit" requires exact 64-bit totals
// and 64-bit addressing for buffers sized by n_isects. The sort orders the
// (tile_id << 32) | depth keys of the [VRAM] cost table (isect.ids_a/b).
//
// The scan is single-pass with a decoupled look-back: a block takes a
// ticket (so every block it waits on is already running), publishes its
// aggregate, then sums predecessors' aggregates until it meets an
// inclusive prefix. Each look-back word packs status, an epoch tag and a
// 56-bit value into one 64-bit atomic.
//
// The radix passes do not use a look-back. With 256 digit counters per
// block, a look-back walk moves 2 KB per predecessor through the
// cross-die coherent path, and on this chip that traffic and its latency
// cost about half of every pass. Each pass is reduce-then-scan instead:
// the keys are split into at most 1024 contiguous chunks (one resident
// block each); a counting kernel writes per-chunk digit counts and adds
// them into totals per group of 32 chunks; the scatter kernel derives its
// chunk's start per digit from at most 32 group totals and 31 chunk counts
// (no separate scan launch) and walks its chunk tile by tile with running
// per-digit cursors.
// Inside a tile, ranks come from eight ballots (lanes with equal digits),
// per-wave counters live in LDS, and the tile is reordered in LDS so each
// digit run is written contiguously. Stability: tiles are taken in order
// within a chunk and chunks in order within a digit.
#include "gs_internal.h"

namespace gs {

namespace {

__global__ void k_fill_u32(uint32_t* p, uint32_t v, uint64_t n) {
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// FROM_MASK: element e is the popcount of mask words 2e and 2e + 1 (one
// 128-pair group of the visibility bitmask), also written to counts[e].
template <bool FROM_MASK, bool OUT64>
__global__ __launch_bounds__(kScanThreads) void k_scan(const uint32_t* __restrict__ in,
                                                       const uint64_t* __restrict__ mask,
                                                       uint32_t* __restrict__ counts, uint64_t n,
                                                       uint32_t* __restrict__ out32,
                                                       uint64_t* __restrict__ out64,
                                                       uint64_t* total, uint64_t* lb,
                                                       uint32_t* ticket, int* err) {
  __shared__ uint32_t s_blk;
  __shared__ uint64_t s_wave[4];
  __shared__ uint64_t s_prefix;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid == 0) s_blk = atomicAdd(ticket, 1u);
  __syncthreads();
  const uint64_t blk = s_blk;
  const uint64_t base = blk * kScanTile + uint64_t(tid) * kScanItems;
  uint32_t v[kScanItems];
  uint64_t tsum = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const uint64_t e = base + i;
    uint32_t x = 0;
    if (e < n) {
      if (FROM_MASK) {
        x = uint32_t(__popcll(mask[2 * e]) + __popcll(mask[2 * e + 1]));
        counts[e] = x;
      } else {
        x = in[e];
      }
    }
    v[i] = x;
    tsum += x;
  }
  const uint64_t incl = wave_incl_scan_u64(tsum);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  uint64_t woff = 0, btot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    woff += (w < wave) ? s_wave[w] : 0ull;
    btot += s_wave[w];
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
      s_prefix = prefix;
      if ((blk + 1) * kScanTile >= n) *total = prefix + btot;
    }
  }
  __syncthreads();
  uint64_t run = s_prefix + woff + incl - tsum;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const uint64_t e = base + i;
    if (e < n) {
      if (OUT64)
        out64[e] = run;
      else
        out32[e] = uint32_t(run);
    }
    run += v[i];
  }
}

template <int ITEMS>
__global__ __launch_bounds__(kSortThreads) void k_radix_count(const uint32_t* __restrict__ keys, uint64_t n,
                                                    int shift, uint32_t dmask, uint64_t ct,
                                                    uint32_t* __restrict__ cnt,
                                                    uint64_t* __restrict__ grp) {
  constexpr uint64_t TILE = uint64_t(kSortThreads) * ITEMS;
  __shared__ uint32_t s_h[4][256];
  const int tid = threadIdx.x, wave = tid >> 6;
#pragma unroll
  for (int w = 0; w < 4; ++w) s_h[w][tid] = 0;
  __syncthreads();
  const uint64_t e0 = uint64_t(blockIdx.x) * ct * TILE;
  uint64_t e1 = e0 + ct * TILE;
  if (e1 > n) e1 = n;
  for (uint64_t b = e0; b < e1; b += TILE) {
    uint32_t k[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint64_t e = b + uint64_t(i) * kSortThreads + tid;
      k[i] = e < e1 ? keys[e] : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint64_t e = b + uint64_t(i) * kSortThreads + tid;
      if (e < e1) atomicAdd(&s_h[wave][(k[i] >> shift) & dmask], 1u);
    }
  }
  __syncthreads();
  const uint32_t c = s_h[0][tid] + s_h[1][tid] + s_h[2][tid] + s_h[3][tid];
  cnt[uint64_t(blockIdx.x) * 256 + tid] = c;
  if (c) atomicAdd(reinterpret_cast<unsigned long long*>(grp + (blockIdx.x / kSortGroup) * 256 + tid),
                   (unsigned long long)c);
}

// The lanes (among those where `valid` holds) whose digit, the low DB bits
// of d, equals this lane's: one ballot per digit bit. For each bit the set
// keeps the lanes whose ballot bit matches this lane's, p &= ~(ballot ^ m)
// with m all ones when this lane's bit is set; written per 32-bit half so
// each bit costs one three-input bitwise op per half (scatter time per step
// 15M 5-camera 0.805 -> 0.786 ms, 3M 5-camera 0.896 -> 0.875 ms).
template <int DB>
__device__ __forceinline__ uint64_t wave_digit_peers(uint32_t d, bool valid) {
  const uint64_t v = __ballot(valid);
  uint32_t lo = uint32_t(v), hi = uint32_t(v >> 32);
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    const uint32_t m = uint32_t(int32_t(d << (31 - b)) >> 31);
    const uint64_t bb = __ballot(m != 0u);
    lo &= ~(uint32_t(bb) ^ m);
    hi &= ~(uint32_t(bb >> 32) ^ m);
  }
  return (uint64_t(hi) << 32) | lo;
}

// DB: ballots per key, the digit's width rounded up to 6, 7 or 8 (bits of
// the digit above its width are zero, so ballots on them add nothing).
template <int ITEMS, int DB>
__global__ __launch_bounds__(kSortThreads) void k_radix_scatter(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out, uint64_t n, int shift,
    uint32_t dmask, uint64_t ct, const uint32_t* __restrict__ cnt, const uint64_t* __restrict__ grp,
    uint64_t* __restrict__ grp_next) {
  constexpr int TILE = kSortThreads * ITEMS;
  __shared__ int64_t s_gstart[256];
  __shared__ uint32_t s_whist[4][256];
  __shared__ uint32_t s_lstart[256];
  __shared__ uint64_t s_w64[4];
  __shared__ uint32_t s_w32[4];
  __shared__ uint32_t s_keys[TILE];
  __shared__ uint32_t s_vals[TILE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // Start of this chunk's run of digit tid: the keys of all smaller
  // digits, plus this digit's keys in earlier chunk groups (group totals)
  // and in earlier chunks of this group.
  // Every load is issued unconditionally (clamped row, result selected)
  // so that all of them are in flight together.
  const uint32_t g = blockIdx.x / kSortGroup;
  const uint32_t G = (gridDim.x + kSortGroup - 1) / kSortGroup;
  uint64_t tot_d = 0, before = 0;
#pragma unroll 8
  for (uint32_t i = 0; i < uint32_t(kSortGroups); ++i) {
    const uint64_t v = grp[(i < G ? i : G - 1) * 256 + tid];
    tot_d += i < G ? v : 0ull;
    before += i < g ? v : 0ull;
  }
  const uint32_t q0 = g * kSortGroup;
#pragma unroll 8
  for (uint32_t i = 0; i + 1 < uint32_t(kSortGroup); ++i) {
    const uint32_t q = q0 + i;
    const uint32_t v = cnt[uint64_t(q < blockIdx.x ? q : blockIdx.x) * 256 + tid];
    before += q < blockIdx.x ? v : 0u;
  }
  uint64_t run;  // next output position of digit tid
  {
    uint64_t tot;
    run = block_excl_scan_u64(tot_d, s_w64, &tot) + before;
  }
  // the next pass's group totals start from zero
  for (uint32_t r = blockIdx.x; r < uint32_t(kSortGroups); r += gridDim.x) grp_next[r * 256 + tid] = 0;
  const uint64_t lt = lanemask_lt();
  const uint64_t e0 = uint64_t(blockIdx.x) * ct * TILE;
  uint64_t e1 = e0 + ct * uint64_t(TILE);
  if (e1 > n) e1 = n;
  // Each lane reads items i * 64 past its own first key of a tile: one
  // base pointer per lane, the item offsets are immediates.
  const uint64_t lane0 = uint64_t(wave) * (ITEMS * kWave) + lane;
  uint32_t key[ITEMS], val[ITEMS];
  {
    const uint32_t* kp = keys_in + e0 + lane0;
    const uint32_t* vp = vals_in + e0 + lane0;
    const int64_t left = int64_t(e1) - int64_t(e0 + lane0);  // keys from this lane's first on
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      key[i] = i * kWave < left ? kp[i * kWave] : 0u;
      val[i] = i * kWave < left ? vp[i * kWave] : 0u;
    }
  }
  for (uint64_t base = e0; base < e1; base += TILE) {
#pragma unroll
    for (int w = 0; w < 4; ++w) s_whist[w][tid] = 0;
    __syncthreads();
    uint32_t rank[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint64_t e = base + uint64_t(wave) * (ITEMS * kWave) + i * kWave + lane;
      const bool valid = e < e1;
      const uint32_t d = (key[i] >> shift) & dmask;
      const uint64_t peers = wave_digit_peers<DB>(d, valid);
      const uint32_t before = s_whist[wave][d];
      const uint32_t r = uint32_t(__popcll(peers & lt));
      if (valid && r == 0) s_whist[wave][d] = before + uint32_t(__popcll(peers));
      rank[i] = before + r;
    }
    __syncthreads();
    const uint32_t c0 = s_whist[0][tid], c1 = s_whist[1][tid], c2 = s_whist[2][tid],
                   c3 = s_whist[3][tid];
    const uint32_t cnt = c0 + c1 + c2 + c3;
    s_whist[0][tid] = 0;
    s_whist[1][tid] = c0;
    s_whist[2][tid] = c0 + c1;
    s_whist[3][tid] = c0 + c1 + c2;
    uint32_t tot;
    const uint32_t lstart = block_excl_scan_u32(cnt, s_w32, &tot);
    s_lstart[tid] = lstart;
    s_gstart[tid] = int64_t(run) - int64_t(lstart);
    run += cnt;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint64_t e = base + uint64_t(wave) * (ITEMS * kWave) + i * kWave + lane;
      if (e < e1) {
        const uint32_t d = (key[i] >> shift) & dmask;
        const uint32_t pos = s_lstart[d] + s_whist[wave][d] + rank[i];
        s_keys[pos] = key[i];
        s_vals[pos] = val[i];
      }
    }
    __syncthreads();
    // the next tile's loads overlap this tile's scatter
    {
      const uint64_t nb = base + TILE;
      const uint32_t* kp = keys_in + nb + lane0;
      const uint32_t* vp = vals_in + nb + lane0;
      const int64_t left = int64_t(e1) - int64_t(nb + lane0);
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        key[i] = i * kWave < left ? kp[i * kWave] : 0u;
        val[i] = i * kWave < left ? vp[i * kWave] : 0u;
      }
    }
    const uint64_t cnt_blk = (e1 - base) < uint64_t(TILE) ? (e1 - base) : uint64_t(TILE);
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const uint32_t li = uint32_t(j * kSortThreads + tid);
      if (li < cnt_blk) {
        const uint32_t k = s_keys[li];
        const uint32_t d = (k >> shift) & dmask;
        const uint64_t g = uint64_t(s_gstart[d] + int64_t(li));
        keys_out[g] = k;
        vals_out[g] = s_vals[li];
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_fill_u32(void* p, uint32_t v, uint64_t n_words, hipStream_t s) {
  if (n_words == 0) return hipSuccess;
  uint64_t blocks = (n_words + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  ProfScope prof("k_fill_u32", s);
  hipLaunchKernelGGL(k_fill_u32, dim3(uint32_t(blocks)), dim3(256), 0, s,
                     static_cast<uint32_t*>(p), v, n_words);
  return hipGetLastError();
}

hipError_t launch_scan_u32(const uint32_t* in, const uint64_t* mask, uint32_t* counts,
                           uint64_t n, uint32_t* out32, uint64_t* out64, uint64_t* total,
                           uint64_t* lookback, uint32_t* ticket, int* err, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint64_t blocks = (n + kScanTile - 1) / kScanTile;
  if (!fits_dispatch(blocks, kScanThreads)) return hipErrorInvalidConfiguration;
  const dim3 grid{uint32_t(blocks)}, block{uint32_t(kScanThreads)};
  ProfScope prof("k_scan", s);
  if (mask) {
    if (out64)
      hipLaunchKernelGGL((k_scan<true, true>), grid, block, 0, s, in, mask, counts, n, out32, out64, total, lookback, ticket, err);
    else
      hipLaunchKernelGGL((k_scan<true, false>), grid, block, 0, s, in, mask, counts, n, out32, out64, total, lookback, ticket, err);
  } else {
    if (out64)
      hipLaunchKernelGGL((k_scan<false, true>), grid, block, 0, s, in, mask, counts, n, out32, out64, total, lookback, ticket, err);
    else
      hipLaunchKernelGGL((k_scan<false, false>), grid, block, 0, s, in, mask, counts, n, out32, out64, total, lookback, ticket, err);
  }
  return hipGetLastError();
}

int sort_passes(int bits) { return bits <= 0 ? 1 : (bits + kRadixBits - 1) / kRadixBits; }

namespace {

struct SortPlan {
  int items;       // keys per lane per tile
  uint64_t ct;     // tiles per chunk
  uint32_t P;      // chunks (= blocks of the count and scatter kernels)
};

// Small inputs (under 256K keys) take 1024-key tiles so that enough
// blocks run; larger ones take 2048-key tiles (measured: a 1M-key pass is
// faster with half the blocks, each doing twice the work), and from 32M
// keys 4096-key tiles; there are at most kSortChunks chunks.
SortPlan sort_plan(uint64_t n) {
  SortPlan p{};
  p.items = n < (uint64_t(1) << 18) ? 4 : n < (uint64_t(1) << 25) ? 8 : 16;
  const uint64_t tile = uint64_t(kSortThreads) * p.items;
  const uint64_t tiles = (n + tile - 1) / tile;
  p.ct = (tiles + kSortChunks - 1) / kSortChunks;
  p.P = uint32_t((tiles + p.ct - 1) / p.ct);
  return p;
}

template <int ITEMS>
void launch_pass(const SortPlan& pl, const uint32_t* ki, const uint32_t* vi, uint32_t* ko,
                 uint32_t* vo, uint64_t n, int shift, uint32_t dmask, SortScratch& sc,
                 hipStream_t s) {
  uint64_t* grp = sc.grp + sc.parity * (kSortGroups * kRadix);
  uint64_t* grp_next = sc.grp + (sc.parity ^ 1) * (kSortGroups * kRadix);
  {
    ProfScope prof("k_radix_count", s);
    hipLaunchKernelGGL(k_radix_count<ITEMS>, dim3(pl.P), dim3(kSortThreads), 0, s, ki, n, shift,
                       dmask, pl.ct, sc.cnt, grp);
  }
  {
    ProfScope prof("k_radix_scatter", s);
    const int width = 32 - __builtin_clz(dmask | 1u);
#define GS_SCATTER(DB)                                                                            \
  hipLaunchKernelGGL((k_radix_scatter<ITEMS, DB>), dim3(pl.P), dim3(kSortThreads), 0, s, ki, vi, \
                     ko, vo, n, shift, dmask, pl.ct, sc.cnt, grp, grp_next)
    if (width <= 6)
      GS_SCATTER(6);
    else if (width == 7)
      GS_SCATTER(7);
    else
      GS_SCATTER(8);
#undef GS_SCATTER
  }
  sc.parity ^= 1;
}

}  // namespace

uint64_t sort_counts_bytes() { return uint64_t(kSortChunks) * kRadix * sizeof(uint32_t); }

uint64_t sort_groups_bytes() { return 2ull * kSortGroups * kRadix * sizeof(uint64_t); }

hipError_t launch_sort_passes(uint32_t* keys_a, uint32_t* vals_a, uint32_t* keys_b,
                              uint32_t* vals_b, uint64_t n, int bit0, int bits,
                              SortScratch& sc, bool* in_b, hipStream_t s) {
  const int passes = sort_passes(bits);
  *in_b = (passes & 1) != 0;
  if (n == 0) return hipSuccess;
  const SortPlan pl = sort_plan(n);
  uint32_t *ki = keys_a, *vi = vals_a, *ko = keys_b, *vo = vals_b;
  // the bits are split evenly over the passes: fewer digit values per
  // pass make longer runs of equal digits, so the scattered writes coalesce
  const int width = bits <= 0 ? 1 : (bits + passes - 1) / passes;
  for (int p = 0; p < passes; ++p) {
    const int shift = bit0 + width * p;
    const uint32_t dmask = (1u << width) - 1u;
    if (pl.items == 4)
      launch_pass<4>(pl, ki, vi, ko, vo, n, shift, dmask, sc, s);
    else if (pl.items == 8)
      launch_pass<8>(pl, ki, vi, ko, vo, n, shift, dmask, sc, s);
    else
      launch_pass<16>(pl, ki, vi, ko, vo, n, shift, dmask, sc, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint32_t* t = ki;
    ki = ko;
    ko = t;
    t = vi;
    vi = vo;
    vo = t;
  }
  return hipSuccess;
}

}  // namespace gs
