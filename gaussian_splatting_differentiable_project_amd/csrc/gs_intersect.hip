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
#include <cstdlib>

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

// Inclusive running maximum over the 64 lanes.
// All ones when bit b of x is set, else zero (a signed one-bit extract,
// kept opaque so that a test of it stays one compare).
__device__ __forceinline__ uint32_t bit_as_mask(uint32_t x, int b) {
  uint32_t r;
  asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(r) : "v"(x), "i"(b));
  return r;
}

__device__ __forceinline__ uint32_t wave_incl_max_u32(uint32_t v) {
  const int l = __lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, kWave);
    if (l >= o) v = t > v ? t : v;
  }
  return v;
}

// Per slot: depth key bits and identity value for the depth sort, and
// the exact 64-bit totals of tile counts (total[0]) and of segment counts
// (total[1 + kPrepBlocks]: rectangle rows times the 64-tile windows each
// row meets), one atomic each per work-group.
// total[1 + b] receives block b's largest key (high word) and the
// complement of its smallest key (low word): the host reduces them and
// skips the depth passes over digits that every key shares. Words of
// blocks that are not launched stay zero, which neither maximum notices.
__global__ __launch_bounds__(256) void k_isect_prep(uint64_t nnz, const float* __restrict__ screen,
                                                   const uint2* __restrict__ aabb16, uint32_t W,
                                                   uint32_t H, uint32_t* __restrict__ dkeys,
                                                   uint32_t* __restrict__ dvals, uint64_t* total) {
  __shared__ uint64_t s_w[4], s_wr[4];
  __shared__ uint32_t s_max[4], s_nmin[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint64_t n = 0, nr = 0;
  uint32_t kmax = 0, knmin = 0;
  // grid-stride, so few blocks contend for the one 64-bit total
  const uint64_t stride = uint64_t(gridDim.x) * 256;
  for (uint64_t i = uint64_t(blockIdx.x) * 256 + tid; i < nnz; i += stride) {
    const uint32_t k = __float_as_uint(screen[i * kRow + 6]);
    dkeys[i] = k;
    dvals[i] = uint32_t(i);
    kmax = k > kmax ? k : kmax;
    knmin = ~k > knmin ? ~k : knmin;
    const TileRect r = rect_of(aabb16[i], W, H);
    const uint32_t c = rect_count(r);
    n += c;
    nr += c ? (r.ty1 - r.ty0) * (((r.tx1 - 1u) >> 6) - (r.tx0 >> 6) + 1u) : 0u;
  }
  const uint64_t incl = wave_incl_scan_u64(n);
  const uint64_t incl_r = wave_incl_scan_u64(nr);
  const uint32_t wmax = wave_incl_max_u32(kmax), wnmin = wave_incl_max_u32(knmin);
  if (lane == 63) {
    s_w[wave] = incl;
    s_wr[wave] = incl_r;
    s_max[wave] = wmax;
    s_nmin[wave] = wnmin;
  }
  __syncthreads();
  if (tid == 0) {
    const uint64_t b = s_w[0] + s_w[1] + s_w[2] + s_w[3];
    if (b) atomicAdd(reinterpret_cast<unsigned long long*>(total), (unsigned long long)b);
    const uint64_t br = s_wr[0] + s_wr[1] + s_wr[2] + s_wr[3];
    if (br)
      atomicAdd(reinterpret_cast<unsigned long long*>(total + 1 + kPrepBlocks),
                (unsigned long long)br);
    uint32_t m = 0, nm = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      m = s_max[w] > m ? s_max[w] : m;
      nm = s_nmin[w] > nm ? s_nmin[w] : nm;
    }
    total[1 + blockIdx.x] = (uint64_t(m) << 32) | nm;
  }
}

// Emission of the intersections, fused with the first digit pass of the
// stable LSD sort by tile id. Block b owns a contiguous range of
// depth-order positions (position i holds slot order[i]), walked in
// sub-batches of 512. A pass of an LSD radix sort over the emitted
// sequence would place the entries of digit d after every entry of a
// smaller digit, and among equal digits in emission order. The digit is the low `bits` (at most 8) bits of the
// tile id. That placement is computed here without ever writing the
// unsorted sequence:
//   k_emit_count  counts, per block, its entries of every digit (from the
//                 tile rectangles alone: each rectangle row is a run of
//                 consecutive tile ids, i.e. a cyclic run of digits);
//   a scan of the [digit][block] count matrix in that order gives each
//                 block the first output position of each of its digit runs;
//   k_emit_write  enumerates the block's entries in emission order, ranks
//                 them within their digit stably, and writes each digit run
//                 of a round contiguously.
// Each slot meets a tile at most once, so the entries of one tile are in
// depth order (then slot order) exactly as the stable sort of
// (tile << 32) | depth keys leaves them.
constexpr int kEmitBits = 8;
constexpr uint32_t kEmitRadix = 1u << kEmitBits;
constexpr int kEmitSlots = 512;      // positions per sub-batch
constexpr uint64_t kEmitBlocks = 8192;  // target block count (32 per CU; measured against 2048 and 16384)

struct EmitGeom {
  uint32_t W, H, tiles_x, tiles_y, T;
  uint32_t pitch;         // key step between rectangle rows: tiles_x, or windows per row
  int C;
  uint32_t bits;          // digit width, 1..kEmitBits
  uint64_t nnz, per_blk;  // positions per block (a multiple of kEmitSlots)
  // Row mode: the entries are segments, the part of a pair's tile row
  // that falls in one window of 64 tiles, instead of (tile, pair) entries.
  // Their key is the window id (c * tiles_y + ty) * nwin + tx / 64 in bits
  // [0, rb), with the pair's first tile on the row in the next xb bits and
  // its width minus one above those (rb + 2 xb <= 32).
  int rows;
  uint32_t rb, xb, nwin;
};

// Depth-order position i: its slot, the global id of the first tile of
// its rectangle (camera tile base included) and the rectangle's size.
// In row mode the rectangle is that of its windows (rows by windows per
// row): the base is the segment key of its first one.
__device__ __forceinline__ void emit_slot(uint64_t i, const uint32_t* __restrict__ order,
                                          const uint2* __restrict__ aabb16,
                                          const int64_t* __restrict__ cam_off,
                                          const EmitGeom& g, uint32_t& slot, uint32_t& b0,
                                          uint32_t& wx, uint32_t& wy) {
  slot = order[i];
  // camera of the slot: cameras own consecutive slot ranges
  int lo = 0, hi = g.C - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (int64_t(slot) >= cam_off[mid]) lo = mid; else hi = mid - 1;
  }
  const TileRect r = rect_of(aabb16[slot], g.W, g.H);
  wx = r.tx1 > r.tx0 ? r.tx1 - r.tx0 : 0u;
  wy = r.ty1 > r.ty0 ? r.ty1 - r.ty0 : 0u;
  if (g.rows) {
    const bool any = wx != 0u && wy != 0u;
    const uint32_t w0 = r.tx0 >> 6;
    b0 = any ? ((uint32_t(lo) * g.tiles_y + r.ty0) * g.nwin + w0) |
                   ((r.tx0 | ((wx - 1u) << g.xb)) << g.rb)
             : 0u;
    wx = any ? ((r.tx1 - 1u) >> 6) - w0 + 1u : 0u;
  } else {
    b0 = uint32_t(lo) * g.T + r.ty0 * g.tiles_x + r.tx0;
  }
}

// mat[d * nblk + b] = entries of block b whose tile id has low digit d
// (rows d >= 2^bits are zero); rec[i] = (first tile id, wx | wy << 16) of
// position i, so the write kernel reads its rectangles without the
// dependent gathers. A rectangle row of wx tiles starting at
// tile id s covers every digit floor(wx / R) times plus the cyclic run
// [s, s + wx mod R), R = 2^bits; the runs are added to a difference array
// in LDS and summed once.
__global__ __launch_bounds__(256) void k_emit_count(const uint32_t* __restrict__ order,
                                                   const uint2* __restrict__ aabb16,
                                                   const int64_t* __restrict__ cam_off,
                                                   EmitGeom g, uint64_t nblk,
                                                   uint32_t* __restrict__ mat,
                                                   uint2* __restrict__ rec) {
  const uint32_t R = 1u << g.bits, M = R - 1;
  __shared__ uint32_t s_diff[kEmitRadix];
  __shared__ uint32_t s_full;
  __shared__ uint32_t s_w[4];
  const int tid = threadIdx.x;
  s_diff[tid] = 0;
  if (tid == 0) s_full = 0;
  __syncthreads();
  uint32_t full = 0;
  const uint64_t i0 = uint64_t(blockIdx.x) * g.per_blk;
  const uint64_t i1 = i0 + g.per_blk < g.nnz ? i0 + g.per_blk : g.nnz;
  for (uint64_t i = i0 + tid; i < i1; i += 256) {
    uint32_t slot, b0, wx, wy;
    emit_slot(i, order, aabb16, cam_off, g, slot, b0, wx, wy);
    rec[i] = make_uint2(b0, wx | (wy << 16));  // both at most 4096
    if (wx == 0 || wy == 0) continue;
    full += (wx >> g.bits) * wy;
    const uint32_t rem = wx & M;
    if (rem == 0) continue;
    for (uint32_t dy = 0; dy < wy; ++dy) {
      const uint32_t s = (b0 + dy * g.pitch) & M;
      const uint32_t e = s + rem;
      atomicAdd(&s_diff[s], 1u);
      if (e < R) {
        atomicAdd(&s_diff[e], 0xFFFFFFFFu);
      } else {  // the run wraps: [s, R) and [0, e - R)
        atomicAdd(&s_diff[0], 1u);
        atomicAdd(&s_diff[e - R], 0xFFFFFFFFu);
      }
    }
  }
  if (full) atomicAdd(&s_full, full);
  __syncthreads();
  // counts = inclusive prefix of the differences (modulo 2^32, exact for
  // the true counts) plus the whole-round part
  const uint32_t v = s_diff[tid];
  uint32_t tot;
  const uint32_t run = block_excl_scan_u32(v, s_w, &tot) + v + s_full;
  mat[uint64_t(tid) * nblk + blockIdx.x] = uint32_t(tid) < R ? run : 0u;
}

// mat_off: exclusive scan of mat in [digit][block] order. Writes are
// clamped to `cap` entries.
// The block's entries are walked in emission order in rounds of up to
// 256 * ITEMS. Slot data lives in a window of two sub-batch halves: a
// sub-batch is loaded into the half whose previous occupant has no entry
// left at or after the round's start, so rounds run across sub-batch
// boundaries and are full unless the window runs dry. The position owning
// each entry of a round comes from an owner map in LDS: every position
// whose first entry falls in the round marks that entry with its block-
// relative index, and a running maximum over the round (started from the
// previous round's last owner) fills the rest. Ranks within a digit come
// from one ballot per digit bit and per-wave digit counters; each digit
// run of the round is then gathered in LDS and written contiguously. DB is
// the number of those ballots: the digit width rounded up to 6, 7 or 8.
template <int ITEMS, int DB>
__global__ __launch_bounds__(256) void k_emit_write(
    const uint32_t* __restrict__ order, const uint2* __restrict__ rec, EmitGeom g, uint64_t nblk,
    const uint64_t* __restrict__ mat_off, uint64_t cap, uint32_t* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out) {
  const uint32_t M = (1u << g.bits) - 1;
  constexpr int TILE = 256 * ITEMS;
  constexpr int OWN = TILE / 256;        // owner-map entries per thread
  constexpr int WIN = 2 * kEmitSlots;    // window of two halves
  constexpr int PT = kEmitSlots / 256;   // positions per thread in a half
  static_assert(64 * ITEMS < 65536, "per-wave digit counters are 16-bit");
  __shared__ uint64_t s_off[WIN];             // block entry offset of each position's first entry
  __shared__ uint64_t s_end[2];               // block entry offset where each half's sub-batch ends
  __shared__ uint32_t s_slot[WIN];
  __shared__ uint32_t s_base[WIN];            // global id of the rectangle's first tile
  __shared__ uint32_t s_wx[WIN];              // rectangle width in tiles
  __shared__ int64_t s_gstart[kEmitRadix];    // output position of digit run d, minus its LDS start
  __shared__ uint16_t s_whist[4][kEmitRadix]; // per-wave digit counts, then LDS starts
  __shared__ uint32_t s_own[TILE];            // block-relative position owning each entry
  __shared__ uint64_t s_w64[4];
  __shared__ uint32_t s_w32[4];
  __shared__ uint32_t s_keys[TILE];
  __shared__ uint32_t s_vals[TILE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t blk = blockIdx.x;
  // first output position of this block's run of digit tid
  uint64_t run = mat_off[uint64_t(tid) * nblk + blk];
  const uint64_t lt = lanemask_lt();
  const uint64_t i0 = blk * g.per_blk;
  const uint64_t i1 = i0 + g.per_blk < g.nnz ? i0 + g.per_blk : g.nnz;
  const uint64_t n_sb = (i1 - i0 + kEmitSlots - 1) / kEmitSlots;
  // slot data of the next sub-batch, two positions per thread, loaded
  // ahead of its use
  uint2 nrec[PT];
  uint32_t nslot[PT];
  auto fetch = [&](uint64_t sb) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const uint64_t i = i0 + sb * kEmitSlots + j * 256 + tid;
      nrec[j] = i < i1 ? rec[i] : make_uint2(0u, 1u);  // width 1, height 0: no entries
      nslot[j] = i < i1 ? order[i] : 0u;
    }
  };
  uint64_t loaded = 0;  // sub-batches loaded so far (uniform)
  uint64_t e_end = 0;   // block entry offset after the last loaded one (uniform)
  // Loads sub-batch `loaded` into half (loaded & 1). The caller has
  // synchronized, so no lane still reads that half.
  auto load = [&]() {
    const int h = int(loaded & 1) * kEmitSlots;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int li = h + j * 256 + tid;
      const uint32_t wx = nrec[j].y & 0xFFFFu, wy = nrec[j].y >> 16;
      s_slot[li] = nslot[j];
      s_base[li] = nrec[j].x;
      s_wx[li] = wx ? wx : 1u;
      s_off[li] = uint64_t(wx) * wy;  // counts for now
    }
    if (loaded + 1 < n_sb) fetch(loaded + 1);
    __syncthreads();
    uint64_t c[PT], sum = 0;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      c[j] = s_off[h + tid * PT + j];
      sum += c[j];
    }
    uint64_t btot;
    uint64_t o = e_end + block_excl_scan_u64(sum, s_w64, &btot);
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      s_off[h + tid * PT + j] = o;
      o += c[j];
    }
    e_end += btot;
    if (tid == 0) s_end[loaded & 1] = e_end;
    ++loaded;
  };
  fetch(0);
  uint64_t rb = 0;
  uint32_t carry = 0;  // owner of the last entry of the previous round
  while (true) {
    // fill the window while the round is not covered and the half to
    // refill holds no entry at or after rb
    while (loaded < n_sb && e_end < rb + TILE) {
      if (loaded >= 2) {
        __syncthreads();
        if (s_end[loaded & 1] > rb) break;
      }
      __syncthreads();
      load();
    }
    __syncthreads();
    if (rb >= e_end) break;  // nothing loaded is left, and nothing more to load
    const uint32_t n_here = uint32_t(e_end - rb < uint64_t(TILE) ? e_end - rb : uint64_t(TILE));
    // block-relative index of the sub-batch in each half
    const uint64_t sb_new = loaded - 1, sb_old = loaded >= 2 ? loaded - 2 : loaded - 1;
#pragma unroll
    for (int w = 0; w < 4; ++w) s_whist[w][tid] = 0;
#pragma unroll
    for (int q = 0; q < OWN; ++q) s_own[q * 256 + tid] = 0;
    __syncthreads();
    // positions whose first entry lies in this round mark it
#pragma unroll
    for (int j = 0; j < WIN / 256; ++j) {
      const int wpos = j * 256 + tid;
      const int h = wpos / kEmitSlots, li = wpos % kEmitSlots;
      // a half is live once a sub-batch has been loaded into it
      const bool live = loaded >= 2 || uint64_t(h) == (sb_new & 1);
      const uint64_t first = s_off[wpos];
      const uint64_t end = li + 1 < kEmitSlots ? s_off[wpos + 1] : s_end[h];
      const uint64_t sb = (sb_new & 1) == uint64_t(h) ? sb_new : sb_old;
      if (live && end > first && first >= rb && first - rb < uint64_t(n_here))
        s_own[first - rb] = uint32_t(sb * kEmitSlots + li);
    }
    __syncthreads();
    {  // running maximum over the round, OWN consecutive entries per thread
      uint32_t m = 0;
      uint32_t loc[OWN];
#pragma unroll
      for (int q = 0; q < OWN; ++q) {
        const uint32_t x = s_own[tid * OWN + q];
        m = x > m ? x : m;
        loc[q] = m;
      }
      const uint32_t incl = wave_incl_max_u32(m);
      if (lane == 63) s_w32[wave] = incl;
      __syncthreads();
      uint32_t before = carry;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = s_w32[w];
        before = (w < wave && x > before) ? x : before;
      }
      const uint32_t prev = __shfl_up(incl, 1, kWave);
      if (lane > 0 && prev > before) before = prev;
#pragma unroll
      for (int q = 0; q < OWN; ++q) s_own[tid * OWN + q] = loc[q] > before ? loc[q] : before;
    }
    __syncthreads();
    carry = s_own[n_here - 1];
    uint32_t key[ITEMS], val[ITEMS], rank[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint32_t le = uint32_t(wave * (ITEMS * kWave) + i * kWave + lane);
      const bool valid = le < n_here;
      // straight-line for every lane (an entry past the round's end reads
      // some loaded position's data and is dropped), so the loads overlap
      const uint32_t own = s_own[le] % WIN;  // window slot of the owner
      const uint32_t k = uint32_t(rb + le - s_off[own]);
      const uint32_t w = s_wx[own];
      // k < w * wy with w, wy <= 4096: k / w is below 4096 and the fp32
      // estimate (exact operands, reciprocal and product within 2^-22
      // relative) is within 2^-10 of it, so its truncation is within one
      // of floor(k / w); one correction each way makes it exact. Every
      // product here is of values below 2^24 and stays below 2^32.
      uint32_t dy = uint32_t(float(k) * __builtin_amdgcn_rcpf(float(w)));
      uint32_t dw = __umul24(dy, w);
      const bool over = dw > k, under = dw + w <= k;
      dy = over ? dy - 1 : under ? dy + 1 : dy;
      dw = over ? dw - w : under ? dw + w : dw;
      const uint32_t t = valid ? s_base[own] + __umul24(dy, g.pitch) + (k - dw) : 0u;
      key[i] = t;
      val[i] = s_slot[own];
      // rank among the wave's earlier entries with the same digit (digits
      // are below 2^bits, so the ballots of higher bits agree everywhere)
      const uint32_t d = t & M;
      const uint64_t vb = __ballot(valid);
      uint32_t plo = uint32_t(vb), phi = uint32_t(vb >> 32);
      // per bit, all ones where this lane's bit is set, else zero: a lane
      // keeps the peers whose ballot bit equals its own (all ballots first,
      // so the compares do not wait on each other's results)
      uint32_t sm[DB];
      uint64_t bb[DB];
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        sm[b] = bit_as_mask(d, b);
        bb[b] = __ballot(sm[b] != 0u);
      }
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        plo &= ~(uint32_t(bb[b]) ^ sm[b]);
        phi &= ~(uint32_t(bb[b] >> 32) ^ sm[b]);
      }
      const uint64_t peers = (uint64_t(phi) << 32) | plo;
      const uint32_t before = s_whist[wave][d];
      const uint32_t r = uint32_t(__popcll(peers & lt));
      if (valid && r == 0) s_whist[wave][d] = uint16_t(before + uint32_t(__popcll(peers)));
      rank[i] = before + r;
    }
    __syncthreads();
    // digit tid: its LDS start plus the earlier waves' counts, and the
    // output position of its run
    uint32_t cw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) cw[w] = s_whist[w][tid];
    const uint32_t cnt = cw[0] + cw[1] + cw[2] + cw[3];
    uint32_t ttot;
    const uint32_t ls = block_excl_scan_u32(cnt, s_w32, &ttot);
    {
      uint32_t x = ls;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s_whist[w][tid] = uint16_t(x);
        x += cw[w];
      }
    }
    s_gstart[tid] = int64_t(run) - int64_t(ls);
    run += cnt;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint32_t le = uint32_t(wave * (ITEMS * kWave) + i * kWave + lane);
      if (le < n_here) {
        const uint32_t pos = uint32_t(s_whist[wave][key[i] & M]) + rank[i];
        s_keys[pos] = key[i];
        s_vals[pos] = val[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const uint32_t li = uint32_t(j * 256 + tid);
      if (li < n_here) {
        const uint32_t k = s_keys[li];
        const uint64_t gpos = uint64_t(s_gstart[k & M] + int64_t(li));
        if (gpos < cap) {
          keys_out[gpos] = k;
          vals_out[gpos] = s_vals[li];
        }
      }
    }
    rb += n_here;
  }
}

// tile_offsets[t] = first sorted position whose tile id (key & kmask) is
// >= t. Each lane takes four consecutive boundaries with one 16-byte load;
// the key before its first one comes from the lane below (or, for lane 0,
// one more load). Grid-stride over the n + 1 boundaries: a dispatch's
// work-item count is a 32-bit quantity, and n_isects can exceed 2^32.
__global__ __launch_bounds__(256) void k_tile_ranges(const uint32_t* __restrict__ tkeys,
                                                    uint64_t n, uint64_t n_tiles, uint32_t kmask,
                                                    int64_t* __restrict__ toff) {
  const uint64_t groups = (n + 4) / 4;  // boundaries 0..n, four per lane
  const uint64_t stride = uint64_t(gridDim.x) * 256;
  const int lane = threadIdx.x & 63;
  // ids are < n_tiles by construction; the clamps only keep the writes
  // inside toff[0..n_tiles] whatever the keys hold
  const uint32_t cap = n_tiles < 0xFFFFFFFFull ? uint32_t(n_tiles) : 0xFFFFFFFFu;
  for (uint64_t q = uint64_t(blockIdx.x) * 256 + threadIdx.x; q < groups; q += stride) {
    const uint64_t i0 = q * 4;
    uint32_t k[4];
    if (i0 + 3 < n) {
      const uint4 v = *reinterpret_cast<const uint4*>(tkeys + i0);
      k[0] = v.x & kmask, k[1] = v.y & kmask, k[2] = v.z & kmask, k[3] = v.w & kmask;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) k[j] = i0 + j < n ? (tkeys[i0 + j] & kmask) : cap;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = k[j] < cap ? k[j] : cap;
    // lanes leave the loop from the top, so the lane below is still in it
    const uint32_t below = __shfl_up(k[3], 1, kWave);
    int64_t prev = -1;
    if (i0 > 0) {
      const uint32_t p = lane == 0 ? (tkeys[i0 - 1] & kmask) : below;
      prev = int64_t(p < cap ? p : cap);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t i = i0 + j;
      if (i > n) break;
      const int64_t cur = i < n ? int64_t(k[j]) : int64_t(cap);
      for (int64_t t = prev + 1; t <= cur; ++t) toff[t] = int64_t(i);
      prev = cur;
    }
  }
}

// ---- The sort by tile through window segments ----
// A pair's entries on one tile row are a run of consecutive tiles. Rows
// are cut into windows of 64 tiles, and the sorted list is built from
// segments, the part of a pair's row inside one window, instead of
// (tile, pair) entries. The segments are emitted in depth order and sorted
// stably by window id (the emit and radix passes above, on segment keys);
// every window's segment list is then in depth order. Each list is cut
// into chunks of K segments. Per chunk, a difference array over the
// window's tiles counts the segments covering every tile (k_row_count); an
// exclusive scan of those counts over the window's chunks, per tile, gives
// each chunk its first rank in every tile's list and the tile's total
// (k_row_colscan); a scan of the totals gives the tile offsets.
// k_row_expand then walks each chunk in order, one wave per chunk, one
// lane per tile of the window: each segment covering a lane's tile is that
// tile's next entry. Within a tile the entries so come in segment order,
// i.e. in depth order, which is the stable sort of (tile << 32) | depth
// keys in slot order.
struct RowGeom {
  uint32_t tiles_x, nwin, R;  // tiles per row, windows per row, windows (C * tiles_y * nwin)
  uint32_t rb, xb;            // segment key layout (see EmitGeom), rb < 32
  uint32_t K;                 // segments per chunk
};

// [x0, x1) of the pair's run on the row for segment key k, clamped to the
// row.
__device__ __forceinline__ void row_span(uint32_t k, const RowGeom& g, uint32_t& x0,
                                         uint32_t& x1) {
  const uint32_t xm = (1u << g.xb) - 1u;
  const uint32_t a = (k >> g.rb) & xm;
  const uint32_t b = a + ((k >> (g.rb + g.xb)) & xm) + 1u;
  x0 = a < g.tiles_x ? a : g.tiles_x;
  x1 = b < g.tiles_x ? b : g.tiles_x;
}

// Bits [a, b) of a 64-bit word, 0 <= a < b <= 64.
__device__ __forceinline__ uint64_t bit_range(uint32_t a, uint32_t b) {
  const uint64_t upto = b >= 64 ? ~0ull : (1ull << b) - 1ull;
  return upto & ~((1ull << a) - 1ull);
}

// The segment's tiles inside window w as bits of the window (tile
// 64 w + i is bit i); zero for a key outside the window.
__device__ __forceinline__ uint64_t segment_bits(uint32_t k, const RowGeom& g, uint32_t w) {
  uint32_t a, b;
  row_span(k, g, a, b);
  const uint32_t lo = w * 64, hi = lo + 64;
  a = a > lo ? a : lo;
  b = b < hi ? b : hi;
  return a < b ? bit_range(a - lo, b - lo) : 0ull;
}

// Window of chunk q: the largest r < R with cq[r] <= q (cq is the
// exclusive scan of the per-window chunk counts, so that window's chunks
// include q).
__device__ __forceinline__ uint32_t chunk_row(const uint64_t* __restrict__ cq, uint32_t R,
                                              uint64_t q) {
  uint32_t lo = 0, hi = R - 1;
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) >> 1;
    if (cq[mid] <= q) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void k_row_chunks(const int64_t* __restrict__ roff, RowGeom g,
                                                   uint32_t* __restrict__ cc) {
  const uint32_t stride = gridDim.x * 256;
  for (uint32_t r = blockIdx.x * 256 + threadIdx.x; r < g.R; r += stride) {
    const int64_t len = roff[r + 1] - roff[r];
    cc[r] = len > 0 ? uint32_t((uint64_t(len) + g.K - 1) / g.K) : 0u;
  }
}

// cm[q][i] = segments of chunk q covering tile i of its window. One wave
// per chunk (the grid is an upper bound; waves past the last chunk
// leave): every lane adds its segments into 64 per-tile counters kept as
// a difference array in LDS. Only interior bounds go through LDS atomics:
// a segment ending at the window's end needs no decrement (the counts
// stop at tile 63), and those starting at the window's first tile, which
// would all hit one word, are counted in a register and added once.
__global__ __launch_bounds__(256) void k_row_count(const uint32_t* __restrict__ rkeys,
                                                  const int64_t* __restrict__ roff,
                                                  const uint64_t* __restrict__ cq, RowGeom g,
                                                  uint64_t qmax, uint32_t* __restrict__ cm) {
  __shared__ uint32_t s_d[4][64];
  const int lane = threadIdx.x & 63;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t q = uint64_t(blockIdx.x) * 4 + wv;
  const uint64_t Q = cq[g.R] < qmax ? cq[g.R] : qmax;
  if (q >= Q) return;  // the whole wave
  uint32_t* d = s_d[wv];
  const uint32_t rw = chunk_row(cq, g.R, q);
  const uint32_t w = rw % g.nwin;
  const uint64_t s0 = uint64_t(roff[rw]) + (q - cq[rw]) * g.K;
  const uint64_t e = uint64_t(roff[rw + 1]);
  const uint64_t s1 = s0 + g.K < e ? s0 + g.K : e;
  d[lane] = 0;
  uint32_t nf = 0;  // this lane's segments starting at tile 0 of the window
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // eight keys per lane in flight, then their counts
  constexpr int kLoads = 8;
  for (uint64_t i0 = s0 + lane; i0 < s1; i0 += 64 * kLoads) {
    uint32_t kk[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const uint64_t i = i0 + uint64_t(j) * 64;
      kk[j] = i < s1 ? rkeys[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      if (i0 + uint64_t(j) * 64 >= s1) break;
      uint32_t a, b;
      row_span(kk[j], g, a, b);
      const uint32_t lo = w * 64, hi = lo + 64;
      a = a > lo ? a : lo;
      b = b < hi ? b : hi;
      if (a < b) {
        if (a > lo) atomicAdd(&d[a - lo], 1u);
        else ++nf;
        if (b < hi) atomicAdd(&d[b - lo], 0xFFFFFFFFu);
      }
    }
  }
  const uint32_t n_first = __builtin_amdgcn_readlane(wave_incl_scan_u32(nf), 63);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // counts = inclusive prefix of the differences (modulo 2^32, exact for
  // the true counts)
  cm[q * 64 + lane] = wave_incl_scan_u32(d[lane] + (lane == 0 ? n_first : 0u));
}

// Per (window, tile): the exclusive scan of cm over the window's chunks,
// in place (each chunk's first rank in the tile's list), and the tile's
// entry count.
__global__ __launch_bounds__(256) void k_row_colscan(const uint64_t* __restrict__ cq, RowGeom g,
                                                    uint64_t qmax, uint32_t* __restrict__ cm,
                                                    uint32_t* __restrict__ tcount) {
  const uint64_t n = uint64_t(g.R) * 64;
  const uint64_t stride = uint64_t(gridDim.x) * 256;
  for (uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
    const uint32_t rw = uint32_t(i >> 6), l = uint32_t(i & 63);
    const uint32_t w = rw % g.nwin, row = rw / g.nwin;
    const uint32_t x = w * 64 + l;
    const uint64_t q0 = cq[rw];
    const uint64_t q1 = cq[rw + 1] < qmax ? cq[rw + 1] : qmax;
    uint32_t run = 0;
    uint64_t q = q0;
    // eight loads in flight, then their stores
    for (; q + 8 <= q1; q += 8) {
      uint32_t c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = cm[(q + j) * 64 + l];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        cm[(q + j) * 64 + l] = run;
        run += c[j];
      }
    }
    for (; q < q1; ++q) {
      const uint32_t c = cm[q * 64 + l];
      cm[q * 64 + l] = run;
      run += c;
    }
    if (x < g.tiles_x) tcount[uint64_t(row) * g.tiles_x + x] = run;
  }
}

// One wave per chunk, one lane per tile of the chunk's window. The chunk's
// segments are read 64 at a time, one per lane, as 64-bit masks of the
// window tiles they cover; the wave transposes the 64 x 64 bit matrix
// (segment x tile) so that each lane holds the set of those segments
// covering its tile, and takes them lowest first (up to four per step) as
// its tile's next entries. A lane stages its entries in LDS, in a ring of
// 32 consecutive output positions (slot = position mod 32), slot-major
// (slot s of lane l at word s * 64 + l, so the lanes' writes of one step
// fall in distinct banks whatever their slots); completed aligned groups of
// GROUP positions are written out, GROUP / 4 lanes with one 16-byte store
// each per group, 64 / (GROUP / 4) groups per store instruction. The
// groups at the two ends of a lane's range are written in part, word by
// word. Writes are clamped to `cap` entries; ids must be 16-byte aligned.
// GROUP is 16 (64 bytes, two groups in the ring, completed groups written
// every flush_every<16>() steps) or 32 (a whole 128-byte line, one group
// filling the ring, written in the step that completes it): 32 halves the
// write requests where a chunk's run per tile is long, 16 writes fewer
// partial groups where it is short.
constexpr int kRing = 32;  // staged entries per lane
constexpr int kTake = 4;   // entries a lane takes per step
// slots per lane: the ring, then kTake overflow slots (a step writes its
// entries to consecutive slots from its first; entries past the ring's
// end belong to the group after any completed one and move to the ring's
// start after that group is written)
constexpr int kRingSlots = kRing + kTake;
// steps between flushes of the completed groups: with two groups in the
// ring a lane's writes reach a completed group's slots again only after
// GROUP - kTake + 1 more entries; with one, the group goes in its step
template <int GROUP>
__host__ __device__ constexpr uint32_t flush_every() {
  return GROUP >= kRing ? 1u : uint32_t(GROUP - kTake) / kTake;
}
static_assert(flush_every<16>() >= 1 && flush_every<32>() == 1, "");

// Index of the lowest set bit of x, 0xFFFFFFFF for x == 0 (the hardware
// instruction, without a clamp to 32).
__device__ __forceinline__ uint32_t lowest_bit(uint32_t x) {
  uint32_t r;
  asm("v_ffbl_b32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

__device__ __forceinline__ void wave_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lane l reads lane l ^ J's value (all lanes active). DPP inside rows of
// 16 (J = 8 and 4 compose two of its fixed permutations), a swizzle
// across the two 16-lane rows of each half, a permute across halves.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  const int v = int(x);
  if constexpr (J == 1) return uint32_t(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, true));
  if constexpr (J == 2) return uint32_t(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, true));
  if constexpr (J == 4) {  // l ^ 7 (half-row mirror), then l ^ 3 (quad_perm [3,2,1,0])
    const int y = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, true);
    return uint32_t(__builtin_amdgcn_update_dpp(0, y, 0x1B, 0xf, 0xf, true));
  }
  if constexpr (J == 8) {  // l ^ 15 (row mirror), then l ^ 7 (half-row mirror)
    const int y = __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, true);
    return uint32_t(__builtin_amdgcn_update_dpp(0, y, 0x141, 0xf, 0xf, true));
  }
  if constexpr (J == 16) return uint32_t(__builtin_amdgcn_ds_swizzle(v, 0x401F));
  return uint32_t(__shfl_xor(v, 32, kWave));
}

// The 64 x 64 bit-matrix transpose across the wave: lane l holds row l
// (bit b is element (l, b)); afterwards lane l holds column l. At each
// scale J the lanes l and l ^ J swap their off-diagonal J x J blocks: the
// lane with bit J clear keeps its bits b with (b & J) == 0 and sends the
// others moved down by J; its partner keeps those others and sends its
// bits with (b & J) == 0 moved up by J. For J <= 16 a moved bit stays in
// its 2J-bit block, so inside one 32-bit word the move is a rotation, and
// the bits received fill exactly the positions sent. `out[k]` and `rot[k]`
// are the lane's sent bits and rotation for J = 16 >> k.
struct TransposeLane {
  uint32_t out[5], rot[5];
};

__device__ __forceinline__ TransposeLane transpose_lane(int lane) {
  constexpr uint32_t kLow[5] = {0x0000FFFFu, 0x00FF00FFu, 0x0F0F0F0Fu, 0x33333333u, 0x55555555u};
  TransposeLane c;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const uint32_t J = 16u >> k;
    const bool up = (uint32_t(lane) & J) != 0u;
    c.out[k] = up ? kLow[k] : ~kLow[k];
    c.rot[k] = up ? 32u - J : J;  // rotate right: up by J, or down by J
  }
  return c;
}

template <int J, int K>
__device__ __forceinline__ uint32_t transpose_word(uint32_t w, const TransposeLane& c) {
  const uint32_t sent = w & c.out[K];
  const uint32_t got = lane_xor<J>(__builtin_amdgcn_alignbit(sent, sent, c.rot[K]));
  return (w & ~c.out[K]) | got;
}

__device__ __forceinline__ void wave_transpose64(uint32_t& lo, uint32_t& hi,
                                                 const TransposeLane& c) {
  // J = 32: the lower half's high words trade with the upper half's low words
  const bool up = __lane_id() >= 32;
  const uint32_t got = lane_xor<32>(up ? lo : hi);
  lo = up ? got : lo;
  hi = up ? hi : got;
  lo = transpose_word<16, 0>(lo, c);
  hi = transpose_word<16, 0>(hi, c);
  lo = transpose_word<8, 1>(lo, c);
  hi = transpose_word<8, 1>(hi, c);
  lo = transpose_word<4, 2>(lo, c);
  hi = transpose_word<4, 2>(hi, c);
  lo = transpose_word<2, 3>(lo, c);
  hi = transpose_word<2, 3>(hi, c);
  lo = transpose_word<1, 4>(lo, c);
  hi = transpose_word<1, 4>(hi, c);
}

// Writes the groups of the lanes in `lanes`: lane l's group covers output
// positions G_l + j, j in [vlo_l, vhi_l), staged in its ring slots
// (G_l + j) mod kRing (word slot * 64 + l). Each such lane posts (G, vlo | vhi << 8, lane) in
// LDS in lane order; four lanes then write each posted group, 16 bytes
// each (word by word for a partial group); with `stream` (uniform) as
// non-temporal stores.
template <int GROUP>
__device__ __forceinline__ void flush_groups(uint64_t lanes, const uint32_t* buf, uint4* desc,
                                             uint64_t G, uint32_t vlohi, uint64_t cap,
                                             uint32_t* __restrict__ ids, bool stream) {
  if (!lanes) return;
  const int lane = __lane_id();
  if ((lanes >> lane) & 1ull) {
    const uint32_t rank = uint32_t(__popcll(lanes & lanemask_lt()));
    desc[rank] = make_uint4(uint32_t(G), uint32_t(G >> 32), vlohi, uint32_t(lane));
  }
  wave_order();
  constexpr uint32_t kLanesPerGroup = GROUP / 4, kGroupsPerStore = kWave / kLanesPerGroup;
  const uint32_t n = uint32_t(__popcll(lanes));
  const uint32_t sub = uint32_t(lane) % kLanesPerGroup;
  for (uint32_t g0 = 0; g0 < n; g0 += kGroupsPerStore) {
    const uint32_t gi = g0 + uint32_t(lane) / kLanesPerGroup;
    if (gi < n) {
      const uint4 d = desc[gi];
      const uint64_t gs = (uint64_t(d.y) << 32) | d.x;
      const uint32_t vlo = d.z & 0xFFu, vhi = d.z >> 8;
      const uint32_t j0 = 4 * sub;
      const uint32_t* src = buf + d.w;
      const uint32_t s0 = (d.x + j0) & (kRing - 1);  // four slots, no wrap (s0 % 4 == 0)
      const uint4 v = make_uint4(src[(s0 + 0) * kWave], src[(s0 + 1) * kWave],
                                 src[(s0 + 2) * kWave], src[(s0 + 3) * kWave]);
      const uint64_t p = gs + j0;
      if (vlo == 0 && vhi == uint32_t(GROUP) && p + 3 < cap) {
        if (stream)
          store_stream(reinterpret_cast<uint4*>(ids + p), v);
        else
          *reinterpret_cast<uint4*>(ids + p) = v;
      } else {
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (uint32_t u = 0; u < 4; ++u)
          if (j0 + u >= vlo && j0 + u < vhi && p + u < cap) {
            if (stream)
              store_stream(ids + p + u, vv[u]);
            else
              ids[p + u] = vv[u];
          }
      }
    }
  }
  wave_order();
}

template <bool KEYS, int GROUP>
__global__ __launch_bounds__(256) void k_row_expand(
    const uint32_t* __restrict__ rkeys, const uint32_t* __restrict__ rvals,
    const int64_t* __restrict__ roff, const uint64_t* __restrict__ cq,
    const uint32_t* __restrict__ cm, const int64_t* __restrict__ toff, RowGeom g, uint64_t qmax,
    uint64_t cap, const float* __restrict__ screen, uint64_t nnz, uint32_t* __restrict__ ids,
    uint64_t* __restrict__ keys_out, bool stream) {
  __shared__ uint32_t s_buf[4][kRingSlots * kWave];
  __shared__ uint4 s_desc[4][kWave];
  const int lane = threadIdx.x & 63;
  // wave-uniform: the chunk walk below runs on scalar registers
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t q = uint64_t(blockIdx.x) * 4 + wv;
  const uint64_t Q = cq[g.R] < qmax ? cq[g.R] : qmax;
  if (q >= Q) return;  // the whole wave
  uint32_t* buf = s_buf[wv];
  uint32_t* mine = buf + lane;  // slot s at mine[s * kWave]
  uint4* desc = s_desc[wv];
  const uint32_t rw = chunk_row(cq, g.R, q);
  const uint32_t w = rw % g.nwin, row = rw / g.nwin;
  const uint64_t s0 = uint64_t(roff[rw]) + (q - cq[rw]) * g.K;
  const uint64_t e = uint64_t(roff[rw + 1]);
  const uint64_t s1 = s0 + g.K < e ? s0 + g.K : e;
  const uint32_t x = w * 64 + uint32_t(lane);
  const uint32_t t = row * g.tiles_x + x;  // global tile id (c * T + ty * tiles_x + x)
  const uint64_t base = x < g.tiles_x ? uint64_t(toff[t]) + cm[q * 64 + lane] : 0ull;
  uint32_t sp = uint32_t(base);  // low word of the next output position
  uint32_t off = 0;              // entries taken

  // Takes the segments of one 32-bit word of the transposed set (segment
  // indices i0 + bit) in order, kTake per step.
  // a completed group awaits writing: at most one per lane between
  // flushes, so it is the group before the one holding the lane's next
  // position
  bool pend = false;
  uint32_t steps = 0;     // steps since the last flush (uniform)
  auto flush_pending = [&]() {
    const uint64_t lanes = __ballot(pend);
    if (lanes) {
      const uint64_t pend_g = ((base + off) & ~uint64_t(GROUP - 1)) - GROUP;
      const uint32_t vlo = pend_g < base ? uint32_t(base - pend_g) : 0u;
      wave_order();
      flush_groups<GROUP>(lanes, buf, desc, pend_g, vlo | (uint32_t(GROUP) << 8), cap, ids, stream);
    }
    pend = false;
    steps = 0;
  };

  auto take = [&](uint32_t cw, int i0, uint32_t val) {
    while (__ballot(cw != 0u)) {
      // up to kTake entries into consecutive slots from this step's first
      // one; slots past the k taken ones receive values that later entries
      // overwrite before any group holding them is written out
      const uint32_t slot0 = sp & (kRing - 1);
      uint32_t* wp = mine + slot0 * kWave;
      const uint32_t n = uint32_t(__popc(cw));
      const uint32_t k = n < uint32_t(kTake) ? n : uint32_t(kTake);
#pragma unroll
      for (int u = 0; u < kTake; ++u) {
        // the lowest remaining segment, its pair read from its lane (once
        // none remain, the lane below i0, a slot value later entries
        // overwrite)
        const int i = i0 + int(lowest_bit(cw));
        const uint32_t v = uint32_t(__builtin_amdgcn_ds_bpermute(i * 4, int(val)));
        wp[u * kWave] = v;
        cw &= cw - 1u;
        if (KEYS && uint32_t(u) < k) {
          const uint64_t p = base + off + u;
          if (p < cap && v < nnz)
            keys_out[p] = (uint64_t(t) << 32) | __float_as_uint(screen[uint64_t(v) * kRow + 6]);
        }
      }
      const uint32_t sp2 = sp + k;
      // at most one group boundary is crossed per step: the group of the
      // GROUP positions before it is complete, and waits for the next flush
      pend = pend || ((sp2 ^ sp) & ~uint32_t(GROUP - 1)) != 0u;
      sp = sp2;
      off += k;
      // A lane writes at most kTake entries, kTake - 1 slots ahead, per
      // step, so a completed group's slots stay untouched for
      // flush_every() more steps; a lane completes at most one group
      // between flushes. Entries in the overflow slots belong to the group
      // after any completed one, so they move to the ring's start after
      // the flush.
      if (++steps == flush_every<GROUP>()) flush_pending();
      if (slot0 + k > uint32_t(kRing)) {  // wrapped: the overflow slots belong at the ring's start
#pragma unroll
        for (int u = 0; u < kTake; ++u) mine[u * kWave] = mine[(kRing + u) * kWave];
      }
    }
  };

  const TransposeLane tl = transpose_lane(lane);
  // Segments are loaded kAhead batches of 64 at a time, the next group
  // while the current one is walked: a wait for loads also waits for every
  // store issued before it, so it comes once per group of batches.
  constexpr int kAhead = 4;
  uint32_t nk[kAhead], nv[kAhead];
#pragma unroll
  for (int j = 0; j < kAhead; ++j) {
    const uint64_t i = s0 + j * 64 + lane;
    nk[j] = i < s1 ? rkeys[i] : 0u;
    nv[j] = i < s1 ? rvals[i] : 0u;
  }
  for (uint64_t sg = s0; sg < s1; sg += kAhead * 64) {
    uint32_t ck[kAhead], cv[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      ck[j] = nk[j];
      cv[j] = nv[j];
      const uint64_t i = sg + (kAhead + j) * 64 + lane;
      nk[j] = i < s1 ? rkeys[i] : 0u;
      nv[j] = i < s1 ? rvals[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      if (sg + j * 64 >= s1) break;  // uniform
      const bool in = sg + j * 64 + lane < s1;
      const uint64_t m = in ? segment_bits(ck[j], g, w) : 0ull;
      // lane i now holds the set of this batch's segments covering tile i
      uint32_t clo = uint32_t(m), chi = uint32_t(m >> 32);
      wave_transpose64(clo, chi, tl);
      take(clo, 0, cv[j]);
      take(chi, 32, cv[j]);
    }
  }
  flush_pending();
  // the partial last groups
  const uint64_t pos = base + off;
  const bool part = off != 0 && (uint32_t(pos) & (GROUP - 1)) != 0u;
  const uint64_t G = pos & ~uint64_t(GROUP - 1);
  const uint32_t vlo = G < base ? uint32_t(base - G) : 0u;
  const uint64_t rest = __ballot(part);
  wave_order();
  flush_groups<GROUP>(rest, buf, desc, G, vlo | ((uint32_t(pos) & (GROUP - 1)) << 8), cap, ids,
                      stream);
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

// The launch order for at most kOrderSmall tiles without a radix sort. The
// key (0xFFFF - saturated count) << 16 | tile id is unique per tile, so the
// position of tile i in the stable heavy-first order is the number of keys
// below its own. A block ranks 64 tiles (one per lane); its sixteen waves
// split the other keys, built in LDS a chunk at a time from the offsets
// (all of a thread's loads issued before the first is used) and read back
// as 16-byte broadcasts.
constexpr uint32_t kOrderSmall = 16384;
constexpr uint32_t kOrderChunk = 4096;
constexpr uint32_t kOrderThreads = 1024;
constexpr uint32_t kOrderLoads = (kOrderChunk + kOrderThreads) / kOrderThreads;  // covers len + 1

__device__ __forceinline__ uint32_t order_key(int64_t n, uint32_t t) {
  return ((0xFFFFu - uint32_t(n < 0xFFFF ? n : 0xFFFF)) << 16) | t;
}

__global__ __launch_bounds__(kOrderThreads) void k_tile_order_rank(
    const int64_t* __restrict__ toff, uint32_t n_tiles, uint32_t* __restrict__ order) {
  __shared__ int64_t s_off[kOrderChunk + 1];
  __shared__ uint4 s_k[kOrderChunk / 4];
  __shared__ uint32_t s_part[kOrderThreads / 64][64];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr uint32_t kWaves = kOrderThreads / 64;
  const uint32_t i = blockIdx.x * 64 + lane;
  const uint32_t ic = min(i, n_tiles - 1);
  const int64_t o0 = toff[ic], o1 = toff[ic + 1];
  // ids stay below 2^15, so a real key is never 0xFFFFFFFF: padding ranks
  // after every tile and a lane past the end writes nothing
  const uint32_t v = i < n_tiles ? order_key(o1 - o0, i) : 0xFFFFFFFFu;
  uint32_t cnt = 0;
  uint32_t* s_flat = reinterpret_cast<uint32_t*>(s_k);
  for (uint32_t c0 = 0; c0 < n_tiles; c0 += kOrderChunk) {
    const uint32_t len = min(kOrderChunk, n_tiles - c0);
    int64_t r[kOrderLoads];
#pragma unroll
    for (uint32_t q = 0; q < kOrderLoads; ++q)
      r[q] = toff[min(c0 + tid + q * kOrderThreads, n_tiles)];  // toff has n_tiles + 1 values
#pragma unroll
    for (uint32_t q = 0; q < kOrderLoads; ++q) {
      const uint32_t t = tid + q * kOrderThreads;
      if (t <= len) s_off[t] = r[q];
    }
    __syncthreads();
#pragma unroll
    for (uint32_t q = 0; q < kOrderChunk / kOrderThreads; ++q) {
      const uint32_t t = tid + q * kOrderThreads;
      s_flat[t] = t < len ? order_key(s_off[t + 1] - s_off[t], c0 + t) : 0xFFFFFFFFu;
    }
    __syncthreads();
    const uint32_t groups = (len + 3) >> 2;
#pragma unroll 4
    for (uint32_t g = wave; g < groups; g += kWaves) {
      const uint4 k = s_k[g];
      cnt += uint32_t(k.x < v) + uint32_t(k.y < v) + uint32_t(k.z < v) + uint32_t(k.w < v);
    }
    __syncthreads();
  }
  s_part[wave][lane] = cnt;
  __syncthreads();
  if (wave == 0 && i < n_tiles) {
    uint32_t rank = 0;
#pragma unroll
    for (uint32_t w = 0; w < kWaves; ++w) rank += s_part[w][lane];
    order[rank] = i;
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
  if (blocks > kPrepBlocks) blocks = kPrepBlocks;
  ProfScope prof("k_isect_prep", s);
  hipLaunchKernelGGL(k_isect_prep, dim3(blocks), dim3(256), 0, s, nnz, screen,
                     reinterpret_cast<const uint2*>(aabb16), uint32_t(W), uint32_t(H), dkeys,
                     dvals, total);
  return hipGetLastError();
}

// The digit widths of the whole sort by tile id are balanced: P passes
// in all (P = ceil(bits / 8), at least one, the emit's included), the
// emit's digit ceil(bits / P) wide. Narrower digits make longer runs of
// equal digits, so the scattered writes coalesce better.
int emit_digit_bits(int tile_bits) {
  const int passes = tile_bits <= kEmitBits ? 1 : (tile_bits + kEmitBits - 1) / kEmitBits;
  const int b = (tile_bits + passes - 1) / passes;
  return b < 1 ? 1 : b;
}

namespace {

// Positions per emit block: whole sub-batches, about kEmitBlocks blocks.
uint64_t emit_per_block(uint64_t nnz) {
  const uint64_t subs = (nnz + kEmitSlots - 1) / kEmitSlots;
  return ((subs + kEmitBlocks - 1) / kEmitBlocks) * kEmitSlots;
}

uint64_t emit_blocks(uint64_t nnz) {
  return nnz ? (nnz + emit_per_block(nnz) - 1) / emit_per_block(nnz) : 0;
}

}  // namespace

// Sized by min(sub-batches, kEmitBlocks), which bounds emit_blocks and,
// unlike it, never decreases as nnz grows, so a workspace sized for a
// capacity also fits every smaller count.
uint64_t emit_matrix_len(uint64_t nnz) {
  const uint64_t subs = (nnz + kEmitSlots - 1) / kEmitSlots;
  return (subs < kEmitBlocks ? subs : kEmitBlocks) * kEmitRadix;
}

hipError_t launch_isect_emit(uint64_t nnz, const uint32_t* order, const uint32_t* aabb16,
                             const int64_t* cam_off, int C, int W, int H, int bits,
                             const RowKeys* rows, uint64_t cap, uint32_t* mat, uint32_t* rec,
                             uint64_t* mat_off, uint64_t* mat_total,
                             uint64_t* lb, uint32_t* ticket, int* err, uint32_t* tkeys,
                             uint32_t* tvals, hipStream_t s) {
  if (nnz == 0) return hipSuccess;
  EmitGeom g;
  g.W = uint32_t(W);
  g.H = uint32_t(H);
  g.tiles_x = uint32_t((W + kTile - 1) / kTile);
  g.tiles_y = uint32_t((H + kTile - 1) / kTile);
  g.T = g.tiles_x * g.tiles_y;
  g.C = C;
  g.rows = rows != nullptr;
  g.rb = rows ? uint32_t(rows->rb) : 0u;
  g.xb = rows ? uint32_t(rows->xb) : 0u;
  g.nwin = (g.tiles_x + 63) / 64;
  g.pitch = rows ? g.nwin : g.tiles_x;
  g.bits = uint32_t(bits < 1 ? 1 : bits > kEmitBits ? kEmitBits : bits);
  g.nnz = nnz;
  g.per_blk = emit_per_block(nnz);
  const uint64_t nblk = emit_blocks(nnz);
  const uint2* box = reinterpret_cast<const uint2*>(aabb16);
  {
    ProfScope prof("k_emit_count", s);
    hipLaunchKernelGGL(k_emit_count, dim3(uint32_t(nblk)), dim3(256), 0, s, order, box, cam_off,
                       g, nblk, mat, reinterpret_cast<uint2*>(rec));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_scan_u32(mat, nullptr, nullptr, nblk * kEmitRadix, nullptr, mat_off, mat_total, lb,
                      ticket,
                      err, s);
  if (e != hipSuccess) return e;
  // 2048-entry rounds: four blocks per CU stay resident (4096-entry rounds
  // fit two). Measured against 4096 with about 8192 blocks: emit per step
  // 13M-sh3-7680px 24.9 -> 21.4 ms, 15M 5-camera 0.59 -> 0.55 ms, 3M
  // 5-camera 0.73 -> 0.77 ms.
  ProfScope prof("k_emit_write", s);
#define GS_EMIT(DB)                                                                          \
  hipLaunchKernelGGL((k_emit_write<8, DB>), dim3(uint32_t(nblk)), dim3(256), 0, s, order,    \
                     reinterpret_cast<const uint2*>(rec), g, nblk, mat_off, cap, tkeys, tvals)
  if (g.bits <= 6)
    GS_EMIT(6);
  else if (g.bits == 7)
    GS_EMIT(7);
  else
    GS_EMIT(8);
#undef GS_EMIT
  return hipGetLastError();
}

hipError_t launch_tile_ranges(const uint32_t* tkeys, uint64_t n, uint64_t n_tiles, int64_t* toff,
                              hipStream_t s, uint32_t kmask) {
  ProfScope prof("k_tile_ranges", s);
  hipLaunchKernelGGL(k_tile_ranges, dim3(grid_stride_blocks((n + 4) / 4)), dim3(256), 0, s, tkeys, n,
                     n_tiles, kmask, toff);
  return hipGetLastError();
}

bool row_keys_fit(int C, int W, int H, RowKeys* out) {
  const uint64_t tx = uint64_t((W + kTile - 1) / kTile), ty = uint64_t((H + kTile - 1) / kTile);
  const uint64_t R = uint64_t(C) * ty * ((tx + 63) / 64);
  int rb = 0, xb = 0;
  while (rb < 64 && ((R - 1) >> rb)) ++rb;
  while (xb < 64 && ((tx - 1) >> xb)) ++xb;
  if (rb > 30 || rb + 2 * xb > 32) return false;
  out->rb = rb;
  out->xb = xb;
  return true;
}

uint64_t row_windows(int C, int W, int H) {
  const uint64_t tx = uint64_t((W + kTile - 1) / kTile), ty = uint64_t((H + kTile - 1) / kTile);
  return uint64_t(C) * ty * ((tx + 63) / 64);
}

namespace {

// Chunk length: about 16K chunks (one wave each) for the count of
// segments, between 256 and 4096 segments, so that the count matrix (64
// words per chunk) stays under a quarter of the segment count plus one
// chunk per window.
uint32_t row_chunk(uint64_t n_segments) {
  uint64_t k = 256;
  while (k < 4096 && k * 16384 < n_segments) k <<= 1;
  return uint32_t(k);
}

uint64_t row_chunks_max(uint64_t n_segments, uint64_t R, uint32_t K) {
  return (n_segments + K - 1) / K + R;
}

}  // namespace

hipError_t launch_row_sort(const uint32_t* rkeys, const uint32_t* rvals, uint64_t n_segments,
                           int C, int W, int H, const RowKeys& rk, const RowScratch& w,
                           int* err, const float* screen, uint64_t nnz, uint64_t cap,
                           uint32_t* ids, int64_t* toff, uint64_t* keys_out, hipStream_t s) {
  RowGeom g;
  g.tiles_x = uint32_t((W + kTile - 1) / kTile);
  g.nwin = (g.tiles_x + 63) / 64;
  g.R = uint32_t(row_windows(C, W, H));
  g.rb = uint32_t(rk.rb);
  g.xb = uint32_t(rk.xb);
  g.K = row_chunk(n_segments);
  const uint64_t n_tiles = uint64_t(C) * uint64_t((H + kTile - 1) / kTile) * g.tiles_x;
  const uint64_t qmax = row_chunks_max(n_segments, g.R, g.K);
  if (!fits_dispatch((qmax + 3) / 4, 256)) return hipErrorInvalidConfiguration;
  // window offsets of the sorted segment keys, then chunks per window and
  // their scan
  hipError_t e = launch_tile_ranges(rkeys, n_segments, g.R, w.roff, s,
                                    g.rb ? (1u << g.rb) - 1u : 0u);
  if (e != hipSuccess) return e;
  {
    ProfScope prof("k_row_chunks", s);
    hipLaunchKernelGGL(k_row_chunks, dim3(grid_stride_blocks(g.R)), dim3(256), 0, s, w.roff, g,
                       w.cc);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_scan_u32(w.cc, nullptr, nullptr, g.R, nullptr, w.cq, w.cq + g.R, w.lb_c, w.ticket_c,
                      err, s);
  if (e != hipSuccess) return e;
  const dim3 grid{uint32_t((qmax + 3) / 4)};
  {
    ProfScope prof("k_row_count", s);
    hipLaunchKernelGGL(k_row_count, grid, dim3(256), 0, s, rkeys, w.roff, w.cq, g, qmax, w.cm);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope prof("k_row_colscan", s);
    hipLaunchKernelGGL(k_row_colscan, dim3(grid_stride_blocks(uint64_t(g.R) * 64)), dim3(256), 0,
                       s, w.cq, g, qmax, w.cm, w.tcount);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // tile offsets: the exclusive scan of the tile counts, total at the end
  e = launch_scan_u32(w.tcount, nullptr, nullptr, n_tiles, nullptr,
                      reinterpret_cast<uint64_t*>(toff), reinterpret_cast<uint64_t*>(toff + n_tiles),
                      w.lb_t, w.ticket_t, err, s);
  if (e != hipSuccess) return e;
  // 128-byte groups where a chunk's run per tile averages at least
  // kLongRun entries (cap is the entry count here); GS_EXPAND_GROUP (16
  // or 32, read at each call) overrides the choice for sweeps and tests
  const char* genv = std::getenv("GS_EXPAND_GROUP");
  const int group_env = genv && (std::atoi(genv) == 16 || std::atoi(genv) == 32) ? std::atoi(genv) : 0;
  constexpr uint64_t kLongRun = 512;
  const bool wide = group_env ? group_env == 32 : cap >= kLongRun * 64 * qmax;
  // non-temporal group stores for a list the caches cannot hold anyway
  // (measured: 7.87 -> 7.3 ms for a 19 GB list; a 25 MB list, which the
  // rasterizer then finds in cache, is slower with them)
  constexpr uint64_t kStreamBytes = uint64_t(128) << 20;
  const bool stream = cap * sizeof(uint32_t) >= kStreamBytes;
  ProfScope prof("k_row_expand", s);
#define GS_EXPAND(KEYS, GRP)                                                                    \
  hipLaunchKernelGGL((k_row_expand<KEYS, GRP>), grid, dim3(256), 0, s, rkeys, rvals, w.roff,    \
                     w.cq, w.cm, toff, g, qmax, cap, screen, nnz, ids, keys_out, stream)
  if (keys_out) {
    if (wide) GS_EXPAND(true, 32); else GS_EXPAND(true, 16);
  } else {
    if (wide) GS_EXPAND(false, 32); else GS_EXPAND(false, 16);
  }
#undef GS_EXPAND
  return hipGetLastError();
}

uint64_t row_matrix_len(uint64_t n_segments, int C, int W, int H, bool bound) {
  // the bound takes the shortest chunk any segment count can get
  const uint32_t K = bound ? row_chunk(0) : row_chunk(n_segments);
  return row_chunks_max(n_segments, row_windows(C, W, H), K) * 64;
}

bool tile_order_small(uint64_t n_tiles) { return n_tiles > 0 && n_tiles <= kOrderSmall; }

hipError_t launch_tile_order_small(const int64_t* toff, uint64_t n_tiles, uint32_t* order,
                                   hipStream_t s) {
  if (!tile_order_small(n_tiles)) return hipErrorInvalidValue;
  ProfScope prof("k_tile_order_rank", s);
  hipLaunchKernelGGL(k_tile_order_rank, dim3(uint32_t((n_tiles + 63) / 64)), dim3(kOrderThreads), 0, s, toff,
                     uint32_t(n_tiles), order);
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
