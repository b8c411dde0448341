// Device-wide scan and stable LSD radix sort for gfx950.
//
// [VRAM] "Bitmask compaction" scans the C*N/128 work-group counts;
// [VRAM] "The 4 GiB rule and the 2^31 limit" requires exact 64-bit totals
// and 64-bit addressing for buffers sized by n_isects. The sort orders the
// (tile_id << 32) | depth keys of the [VRAM] cost table (isect.ids_a/b).
//
// Both use a single-pass decoupled look-back: a block takes a ticket (so
// every block it waits on is already running), publishes its aggregate,
// then sums predecessors' aggregates until it meets an inclusive prefix.
// Each look-back word packs status, an epoch tag and a 56-bit value into
// one 64-bit atomic, so stale words from an earlier pass are never read as
// ready and one zero-fill per call serves every pass.
//
// The radix pass follows the one-sweep scheme: one 8-bit digit per pass,
// 4096 keys per 256-lane block. Ranks inside a wave come from eight
// ballots (lanes with equal digits), per-wave counters live in LDS, the
// block reorders its keys in LDS and writes each digit run contiguously.
#include "gs_internal.h"

namespace gs {

namespace {

__global__ void k_fill_u32(uint32_t* p, uint32_t v, uint64_t n) {
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// Exclusive block scan of one uint32 per lane over 256 lanes.
__device__ __forceinline__ uint32_t block_excl_scan_256(uint32_t v, uint32_t* s_tmp /*[4]*/,
                                                        uint32_t* total) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t incl = wave_incl_scan_u32(v);
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t t = s_tmp[w];
    off += (w < wave) ? t : 0u;
    tot += t;
  }
  *total = tot;
  return off + incl - v;
}

template <bool GATHER, bool OUT64>
__global__ __launch_bounds__(kScanThreads) void k_scan(const uint32_t* __restrict__ in,
                                                       const uint32_t* __restrict__ idx, uint64_t n,
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
    if (e < n) x = GATHER ? in[idx[e]] : in[e];
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
  if (tid == 0) {
    uint64_t prefix = 0;
    if (blk == 0) {
      lb_store(lb, lb_word(kLbPrefix, 1, btot));
    } else {
      lb_store(lb + blk, lb_word(kLbAgg, 1, btot));
      prefix = lookback_prefix(lb, int64_t(blk), 1, 1, err);
      lb_store(lb + blk, lb_word(kLbPrefix, 1, prefix + btot));
    }
    s_prefix = prefix;
    if ((blk + 1) * kScanTile >= n) *total = prefix + btot;
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

// Histograms of `passes` consecutive 8-bit digits starting at bit0.
__global__ __launch_bounds__(256) void k_sort_hist(const uint32_t* __restrict__ keys, uint64_t n,
                                                   int bit0, int passes, uint64_t* hist) {
  __shared__ uint32_t s_h[4][kRadix];
  const int tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) s_h[p][tid] = 0;
  __syncthreads();
  const uint64_t stride = uint64_t(gridDim.x) * 256;
  for (uint64_t e = uint64_t(blockIdx.x) * 256 + tid; e < n; e += stride) {
    const uint32_t k = keys[e];
    for (int p = 0; p < passes; ++p) atomicAdd(&s_h[p][(k >> (bit0 + kRadixBits * p)) & 255u], 1u);
  }
  __syncthreads();
  for (int p = 0; p < passes; ++p)
    if (s_h[p][tid]) atomicAdd(reinterpret_cast<unsigned long long*>(hist + p * kRadix + tid),
                               (unsigned long long)s_h[p][tid]);
}

// In place: hist[p][d] -> exclusive prefix over d (start of digit d).
__global__ __launch_bounds__(256) void k_digit_base(uint64_t* hist) {
  __shared__ uint64_t s_w[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint64_t* h = hist + blockIdx.x * kRadix;
  const uint64_t v = h[tid];
  const uint64_t incl = wave_incl_scan_u64(v);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  uint64_t off = 0;
  for (int w = 0; w < wave; ++w) off += s_w[w];
  h[tid] = off + incl - v;
}

__global__ __launch_bounds__(kSortThreads) void k_onesweep(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out, uint64_t n, int shift,
    const uint64_t* __restrict__ digit_base, uint64_t* lb, uint32_t* ticket, uint32_t tag,
    int* err) {
  __shared__ uint32_t s_blk;
  __shared__ uint32_t s_whist[4][kRadix];
  __shared__ uint32_t s_lstart[kRadix];
  __shared__ int64_t s_gstart[kRadix];
  __shared__ uint32_t s_tmp[4];
  __shared__ uint32_t s_keys[kSortTile];
  __shared__ uint32_t s_vals[kSortTile];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int w = 0; w < 4; ++w) s_whist[w][tid] = 0;
  if (tid == 0) s_blk = atomicAdd(ticket, 1u);
  __syncthreads();
  const uint64_t blk = s_blk;
  const uint64_t base = blk * kSortTile;
  const uint64_t lt = lanemask_lt();

  uint32_t key[kSortItems], val[kSortItems], rank[kSortItems];
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint64_t e = base + uint64_t(wave) * (kSortItems * kWave) + i * kWave + lane;
    const bool valid = e < n;
    key[i] = valid ? keys_in[e] : 0u;
    val[i] = valid ? vals_in[e] : 0u;
    const uint32_t d = (key[i] >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < kRadixBits; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const uint32_t before = s_whist[wave][d];
    const uint32_t r = uint32_t(__popcll(peers & lt));
    if (valid && r == 0) s_whist[wave][d] = before + uint32_t(__popcll(peers));
    rank[i] = before + r;
  }
  __syncthreads();

  // lane tid owns digit tid: wave offsets, block total, look-back, starts
  const uint32_t c0 = s_whist[0][tid], c1 = s_whist[1][tid], c2 = s_whist[2][tid],
                 c3 = s_whist[3][tid];
  const uint32_t cnt = c0 + c1 + c2 + c3;
  s_whist[0][tid] = 0;
  s_whist[1][tid] = c0;
  s_whist[2][tid] = c0 + c1;
  s_whist[3][tid] = c0 + c1 + c2;
  uint64_t prefix = 0;
  uint64_t* my_lb = lb + blk * kRadix + tid;
  if (blk == 0) {
    lb_store(my_lb, lb_word(kLbPrefix, tag, cnt));
  } else {
    lb_store(my_lb, lb_word(kLbAgg, tag, cnt));
    prefix = lookback_prefix(lb + tid, int64_t(blk), kRadix, tag, err);
    lb_store(my_lb, lb_word(kLbPrefix, tag, prefix + cnt));
  }
  uint32_t tot;
  const uint32_t lstart = block_excl_scan_256(cnt, s_tmp, &tot);
  s_lstart[tid] = lstart;
  s_gstart[tid] = int64_t(digit_base[tid] + prefix) - int64_t(lstart);
  __syncthreads();

#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint64_t e = base + uint64_t(wave) * (kSortItems * kWave) + i * kWave + lane;
    if (e < n) {
      const uint32_t d = (key[i] >> shift) & 255u;
      const uint32_t pos = s_lstart[d] + s_whist[wave][d] + rank[i];
      s_keys[pos] = key[i];
      s_vals[pos] = val[i];
    }
  }
  __syncthreads();
  const uint64_t cnt_blk = (n - base) < uint64_t(kSortTile) ? (n - base) : uint64_t(kSortTile);
#pragma unroll
  for (int j = 0; j < kSortItems; ++j) {
    const uint32_t li = uint32_t(j * kSortThreads + tid);
    if (li < cnt_blk) {
      const uint32_t k = s_keys[li];
      const uint32_t d = (k >> shift) & 255u;
      const uint64_t g = uint64_t(s_gstart[d] + int64_t(li));
      keys_out[g] = k;
      vals_out[g] = s_vals[li];
    }
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

hipError_t launch_scan_u32(const uint32_t* in, const uint32_t* idx, uint64_t n, uint32_t* out32,
                           uint64_t* out64, uint64_t* total, uint64_t* lookback,
                           uint32_t* ticket, int* err, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint64_t blocks = (n + kScanTile - 1) / kScanTile;
  if (!fits_dispatch(blocks, kScanThreads)) return hipErrorInvalidConfiguration;
  const dim3 grid{uint32_t(blocks)}, block{uint32_t(kScanThreads)};
  ProfScope prof("k_scan", s);
  if (idx) {
    if (out64)
      hipLaunchKernelGGL((k_scan<true, true>), grid, block, 0, s, in, idx, n, out32, out64, total, lookback, ticket, err);
    else
      hipLaunchKernelGGL((k_scan<true, false>), grid, block, 0, s, in, idx, n, out32, out64, total, lookback, ticket, err);
  } else {
    if (out64)
      hipLaunchKernelGGL((k_scan<false, true>), grid, block, 0, s, in, idx, n, out32, out64, total, lookback, ticket, err);
    else
      hipLaunchKernelGGL((k_scan<false, false>), grid, block, 0, s, in, idx, n, out32, out64, total, lookback, ticket, err);
  }
  return hipGetLastError();
}

int sort_passes(int bits) { return bits <= 0 ? 1 : (bits + kRadixBits - 1) / kRadixBits; }

uint64_t sort_blocks(uint64_t n) { return (n + kSortTile - 1) / kSortTile; }

hipError_t launch_sort_histogram(const uint32_t* keys, uint64_t n, int bit0, int bits,
                                 const SortScratch& sc, hipStream_t s) {
  if (n == 0) return hipSuccess;
  uint64_t blocks = (n + 256 * 16 - 1) / (256 * 16);
  if (blocks > 512) blocks = 512;  // few blocks: fewer global atomics per bin
  ProfScope prof("k_sort_hist", s);
  hipLaunchKernelGGL(k_sort_hist, dim3(uint32_t(blocks)), dim3(256), 0, s, keys, n, bit0,
                     sort_passes(bits), sc.hist);
  return hipGetLastError();
}

hipError_t launch_sort_passes(uint32_t* keys_a, uint32_t* vals_a, uint32_t* keys_b,
                              uint32_t* vals_b, uint64_t n, int bit0, int bits,
                              const SortScratch& sc, uint32_t tag0, bool* in_b,
                              hipStream_t s) {
  const int passes = sort_passes(bits);
  *in_b = (passes & 1) != 0;
  if (n == 0) return hipSuccess;
  {
    ProfScope prof("k_digit_base", s);
    hipLaunchKernelGGL(k_digit_base, dim3(passes), dim3(256), 0, s, sc.hist);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint64_t blocks = sort_blocks(n);
  if (!fits_dispatch(blocks, kSortThreads)) return hipErrorInvalidConfiguration;
  uint32_t *ki = keys_a, *vi = vals_a, *ko = keys_b, *vo = vals_b;
  for (int p = 0; p < passes; ++p) {
    ProfScope prof("k_onesweep", s);
    hipLaunchKernelGGL(k_onesweep, dim3(uint32_t(blocks)), dim3(kSortThreads), 0, s, ki, vi, ko,
                       vo, n, bit0 + kRadixBits * p, sc.hist + p * kRadix, sc.lookback,
                       sc.tickets + p, tag0 + uint32_t(p), sc.err);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint32_t* t = ki; ki = ko; ko = t;
    t = vi; vi = vo; vo = t;
  }
  return hipSuccess;
}

}  // namespace gs
