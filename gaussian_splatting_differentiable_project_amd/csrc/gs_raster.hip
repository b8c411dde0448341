// Per-tile rasterization, forward and backward.
//
// [PROF] names the forward kernel rasterize_fwd; [BWD] section 4 describes
// the backward (rasterize_to_pixels_3dgs_bwd): it reuses the forward's
// tile offsets, flattened intersection list, per-pixel last contributing
// entry and final transmittance, splits each pixel's gradient over the
// Gaussians on it along the blend order, and adds the per-pixel terms
// into fp32 screen-space gradients with atomics. The pages give no
// per-pixel formula; the rule is the textbook one fixed in gs.h.
//
// Optional outputs ([BWD] sections 2-3: the per-pixel gradients of the
// colour, depth and transmittance images, and the background hook that
// adds into the transmittance gradient): a depth image composited like a
// colour channel whose value is the entry's depth, D = sum z alpha T, and
// a per-camera background colour blended as C + T_final bg.
//
// gfx950 mapping: one work-group per 16x16 tile; PPT pixels per lane, so
// a 256-pixel tile is 256/PPT lanes. Screen rows of a batch of the tile's
// list are staged in LDS (gathered through the flattened ids) and read
// back as wave-uniform broadcasts. The backward sums each entry's
// gradient over the PPT pixels of a lane, then over the wave with DPP row
// rotations, and issues one fp32 atomic per field per wave -- and only
// for waves where some pixel actually composited the entry.
#include <cstdlib>

#include "gs_internal.h"

namespace gs {

namespace {

// Per-entry constants staged in LDS. The conic's diagonal is stored
// halved and the opacity as log2, so that
//   sigma = a' dx^2 + c' dy^2 + b dx dy   (a' = a/2, c' = c/2)
//   raw   = exp2(log2(o) - sigma log2(e)) = o exp(-sigma)
// costs six multiply/adds and one exponential per pixel. The forward and
// the backward evaluate exactly the same expressions (explicit fused
// operations, no contraction freedom), so they take the same skip
// decisions on every (pixel, entry).
struct Staged {
  float4 a;  // u, v, a', c'
  float4 b;  // b, log2(o), r, g
  float2 c;  // blue, 1/o
  float z;   // depth (used only with a depth image)
};

__device__ __forceinline__ Staged stage_row(const float* __restrict__ screen, uint32_t s) {
  const float2* r = reinterpret_cast<const float2*>(screen + int64_t(s) * kRow);
  const float2 r0 = r[0], r1 = r[1], r2 = r[2], r3 = r[3], r4 = r[4];
  Staged e;
  e.a = make_float4(r0.x, r0.y, 0.5f * r1.x, 0.5f * r2.x);
  e.b = make_float4(r1.y, __builtin_amdgcn_logf(r2.y), r3.y, r4.x);
  e.c = make_float2(r4.y, __builtin_amdgcn_rcpf(r2.y));
  e.z = r3.x;
  return e;
}

// sigma = a' dx^2 + (c' dy + b dx) dy with dx = u - px, dy = v - py (a', c'
// the halved conic). A lane's pixels share their column, so the dx terms
// are formed once per entry and lane; both raster kernels evaluate sigma
// in this same order, so they take the same alpha decisions bit for bit.
struct ColTerms {
  float dx, bdx, adxx;  // dx, b dx, a' dx^2
};

__device__ __forceinline__ ColTerms col_terms(const float4& A, const float4& Bv, float px) {
  ColTerms t;
  t.dx = A.x - px;
  t.bdx = Bv.x * t.dx;
  t.adxx = (A.z * t.dx) * t.dx;
  return t;
}

struct Eval {
  float dy, raw, alpha;
};

__device__ __forceinline__ Eval eval_splat(const ColTerms& t, const float4& A, const float4& Bv,
                                           float py) {
  Eval e;
  e.dy = A.y - py;
  const float sig = fmaf(fmaf(A.w, e.dy, t.bdx), e.dy, t.adxx);
  e.raw = __builtin_amdgcn_exp2f(fmaf(-sig, kLog2e, Bv.y));
  e.alpha = fminf(kAlphaMax, e.raw);
  return e;
}

// Minimum of the entry's sigma over the rectangle [x0,x1] x [y0,y1] of
// pixel centres: sigma is a convex quadratic in the pixel position, so the
// minimum is 0 if the splat centre is inside, else the least of the four
// edge minima (a 1-D quadratic clamped to the edge).
__device__ __forceinline__ float rect_min_sigma(const Staged& e, float x0, float x1, float y0,
                                                float y1) {
  const float u = e.a.x, v = e.a.y, ha = e.a.z, hc = e.a.w, b = e.b.x;
  if (u >= x0 && u <= x1 && v >= y0 && v <= y1) return 0.f;
  // sigma(dx, dy) = ha dx^2 + hc dy^2 + b dx dy with dx = u - px, dy = v - py
  auto q = [&](float dx, float dy) { return fmaf(ha * dx, dx, fmaf(hc * dy, dy, b * dx * dy)); };
  const float ia = 0.5f / ha, ic = 0.5f / hc;
  const float dxa = u - x0, dxb = u - x1;
  const float dya_v = fminf(fmaxf(-b * dxa * ic, v - y1), v - y0);
  const float dyb_v = fminf(fmaxf(-b * dxb * ic, v - y1), v - y0);
  const float dya = v - y0, dyb = v - y1;
  const float dxa_h = fminf(fmaxf(-b * dya * ia, u - x1), u - x0);
  const float dxb_h = fminf(fmaxf(-b * dyb * ia, u - x1), u - x0);
  return fminf(fminf(q(dxa, dya_v), q(dxb, dyb_v)), fminf(q(dxa_h, dya), q(dxb_h, dyb)));
}

// Largest sigma at which the entry still reaches alpha >= 1/255:
// alpha >= 1/255  <=>  sigma <= ln(255 o). The margin (1e-3 plus 1e-4
// relative) is far above the rounding on either side of the comparison,
// so a test against it never skips anything a pixel would composite.
__device__ __forceinline__ float reach_limit(const Staged& e) {
  const float cut = (e.b.y + 7.99435343f) * 0.69314718f;  // ln(255 o)
  return cut + 1e-3f + 1e-4f * fabsf(cut);
}

// Can the entry reach alpha >= 1/255 anywhere in the tile?
__device__ __forceinline__ bool reaches_tile(const Staged& e, float x0, float x1, float y0,
                                             float ylast) {
  return rect_min_sigma(e, x0, x1, y0, fminf(y0 + 15.f, ylast)) <= reach_limit(e);
}

// Which 4-row strips of the tile can the entry reach (bit k = rows
// 4k..4k+3)? Entries and strips that fail are skipped.
__device__ __forceinline__ uint32_t reach_mask(const Staged& e, float x0, float x1, float y0,
                                               float ylast) {
  const float lim = reach_limit(e);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float s0 = y0 + 4.f * k;
    if (s0 <= ylast && rect_min_sigma(e, x0, x1, s0, fminf(s0 + 3.f, ylast)) <= lim) m |= 1u << k;
  }
  return m;
}

// Order-preserving compaction of a batch staged by all NT lanes: lanes with
// keep write their entry to the next free LDS slot. Returns the count.
template <int NT>
__device__ __forceinline__ int compact_slot(bool keep, int* s_wcnt, int* pos) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t bal = __ballot(keep);
  const int mine = __popcll(bal & lanemask_lt());
  if constexpr (NT <= kWave) {
    *pos = mine;
    return __popcll(bal);
  } else {
    if (lane == 0) s_wcnt[wave] = __popcll(bal);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
      const int c = s_wcnt[w];
      off += w < wave ? c : 0;
      tot += c;
    }
    *pos = off + mine;
    return tot;
  }
}

template <int PPT, bool DEPTH>
__global__ __launch_bounds__(kTilePix / PPT) void k_raster_fwd(
    const float* __restrict__ screen, const uint32_t* __restrict__ ids,
    const int64_t* __restrict__ toff, const uint32_t* __restrict__ order, int W, int H,
    int tiles_x, int T, const float* __restrict__ background, float* __restrict__ out_rgb,
    float* __restrict__ out_T, float* __restrict__ out_depth, int32_t* __restrict__ last_ids) {
  constexpr int NT = kTilePix / PPT;
  static_assert(NT % kTile == 0, "a lane's pixels share one column");
  constexpr int B = NT;
  __shared__ float4 s_a[B];
  __shared__ float4 s_b[B];
  __shared__ float s_c[B];
  __shared__ float s_z[DEPTH ? B : 1];
  __shared__ int s_lid[B];
  __shared__ uint32_t s_reach[B];
  __shared__ int s_wcnt[NT / kWave];
  const int tid = threadIdx.x;
  const int64_t t = order ? int64_t(order[blockIdx.x]) : int64_t(blockIdx.x);
  const int c = int(t / T);
  const int tl = int(t - int64_t(c) * T);
  const int ty = tl / tiles_x, tx = tl - ty * tiles_x;
  const int64_t start = toff[t], end = toff[t + 1];

  float px[PPT], py[PPT], Tr[PPT], cr[PPT], cg[PPT], cb[PPT], cd[PPT];
  int last[PPT];
  bool live[PPT];
  bool inside[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int p = tid + k * NT;
    const int X = tx * kTile + (p & 15), Yp = ty * kTile + (p >> 4);
    inside[k] = X < W && Yp < H;
    live[k] = inside[k];
    px[k] = float(X) + 0.5f;
    py[k] = float(Yp) + 0.5f;
    Tr[k] = 1.f;
    cr[k] = cg[k] = cb[k] = cd[k] = 0.f;
    last[k] = -1;
  }

  const float tx0 = float(tx * kTile) + 0.5f, ty0 = float(ty * kTile) + 0.5f;
  const float tx1 = fminf(tx0 + 15.f, float(W) - 0.5f), ylast = float(H) - 0.5f;
  const int wave = tid >> 6;
  const uint32_t wave_u = __builtin_amdgcn_readfirstlane(uint32_t(wave));
  for (int64_t b0 = start; b0 < end; b0 += B) {
    bool any_live = false;
#pragma unroll
    for (int k = 0; k < PPT; ++k) any_live |= live[k];
    if (__syncthreads_count(any_live) == 0) break;
    Staged e;
    uint32_t reach = 0;
    if (b0 + tid < end) {
      e = stage_row(screen, ids[b0 + tid]);
      reach = reach_mask(e, tx0, tx1, ty0, ylast);
    }
    int pos;
    const int nb = compact_slot<NT>(reach != 0, s_wcnt, &pos);
    if (reach) {
      s_a[pos] = e.a;
      s_b[pos] = e.b;
      s_c[pos] = e.c.x;
      if (DEPTH) s_z[pos] = e.z;
      s_lid[pos] = int(b0 - start) + tid;
      s_reach[pos] = reach;
    }
    __syncthreads();
    for (int j = 0; j < nb; ++j) {
      // the entry's strips, the same for every lane: tested on the scalar unit
      const uint32_t rm = __builtin_amdgcn_readfirstlane(s_reach[j]);
      const float4 A = s_a[j], Bv = s_b[j];
      const float cblue = s_c[j];
      const float zj = DEPTH ? s_z[j] : 0.f;
      const int lid = s_lid[j];
      const ColTerms ct = col_terms(A, Bv, px[0]);  // the lane's pixels share px
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        // pixel k of this wave lies in strip wave + k * (waves per tile)
        if (!((rm >> (wave_u + k * (NT / kWave))) & 1u)) continue;
        const Eval e = eval_splat(ct, A, Bv, py[k]);
        const float Tn = Tr[k] * (1.f - e.alpha);
        const bool use = live[k] && e.alpha >= kAlphaMin;
        const bool stop = use && Tn < kTStop;
        if (stop) live[k] = false;
        if (use && !stop) {
          const float w = e.alpha * Tr[k];
          cr[k] = fmaf(Bv.z, w, cr[k]);
          cg[k] = fmaf(Bv.w, w, cg[k]);
          cb[k] = fmaf(cblue, w, cb[k]);
          if (DEPTH) cd[k] = fmaf(zj, w, cd[k]);
          Tr[k] = Tn;
          last[k] = lid;
        }
      }
    }
  }
  float bg0 = 0.f, bg1 = 0.f, bg2 = 0.f;
  if (background) {
    bg0 = background[3 * c + 0];
    bg1 = background[3 * c + 1];
    bg2 = background[3 * c + 2];
  }
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    if (!inside[k]) continue;
    const int p = tid + k * NT;
    const int64_t pix = (int64_t(c) * H + ty * kTile + (p >> 4)) * W + tx * kTile + (p & 15);
    out_rgb[3 * pix + 0] = fmaf(Tr[k], bg0, cr[k]);
    out_rgb[3 * pix + 1] = fmaf(Tr[k], bg1, cg[k]);
    out_rgb[3 * pix + 2] = fmaf(Tr[k], bg2, cb[k]);
    out_T[pix] = Tr[k];
    if (DEPTH) out_depth[pix] = cd[k];
    last_ids[pix] = last[k];
  }
}

// DPP lane permutations inside 16-lane rows (all lanes active, every
// source lane valid, so no old value is needed).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
constexpr int kDppRowMirror = 0x140;      // lane reads 15 - l within its row
constexpr int kDppRowHalfMirror = 0x141;  // lane reads 7 - l within its half-row
constexpr int kDppXor2 = 0x4E;            // quad_perm [2,3,0,1]
constexpr int kDppXor1 = 0xB1;            // quad_perm [1,0,3,2]

// Sum nine (or, with the depth term, ten) per-lane values over the wave
// and add the totals to dst[field] with one atomic instruction. Transposed
// reduction: at each step a lane pairs with a partner differing in one
// lane bit and keeps the sums of half of the remaining values
// (9|10 -> 5 -> 3 -> 2 -> 1), so a lane ends with one value summed over
// its 16-lane row; two exchanges across rows finish the sum. Lanes 0..15
// then hold: lane -> value index 0,1,2,-,3,4,-,-,5,6,7,-,8,9,-,- (value
// index -> screen field 0,1,2,3,4,5,7,8,9, then 6). Must be called with
// all 64 lanes active.
template <int NV>
__device__ __forceinline__ void wave_reduce_atomic(const float (&v)[NV], float* dst) {
  static_assert(NV == 9 || NV == 10, "nine or ten fields");
  // Every DPP read is evaluated by all lanes before any select: a DPP
  // inside a conditional would read lanes that are switched off.
  const int lane = __lane_id();
  bool hi = (lane & 8) != 0;
  float w1[5];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo_s = v[k] + dpp<kDppRowMirror>(v[k]);
    const float hi_s = v[5 + k] + dpp<kDppRowMirror>(v[5 + k]);
    w1[k] = hi ? hi_s : lo_s;
  }
  {
    const float lo_s = v[4] + dpp<kDppRowMirror>(v[4]);
    const float hi_s = NV == 10 ? v[NV - 1] + dpp<kDppRowMirror>(v[NV - 1]) : 0.f;
    w1[4] = hi ? hi_s : lo_s;
  }
  hi = (lane & 4) != 0;
  float w2[3];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float lo_s = w1[k] + dpp<kDppRowHalfMirror>(w1[k]);
    const float hi_s = w1[3 + k] + dpp<kDppRowHalfMirror>(w1[3 + k]);
    w2[k] = hi ? hi_s : lo_s;
  }
  {
    const float lo_s = w1[2] + dpp<kDppRowHalfMirror>(w1[2]);
    w2[2] = hi ? 0.f : lo_s;
  }
  hi = (lane & 2) != 0;
  const float s30 = w2[0] + dpp<kDppXor2>(w2[0]);
  const float s31 = w2[1] + dpp<kDppXor2>(w2[1]);
  const float s32 = w2[2] + dpp<kDppXor2>(w2[2]);
  const float w3_0 = hi ? s32 : s30;
  const float w3_1 = hi ? 0.f : s31;
  hi = (lane & 1) != 0;
  const float s40 = w3_0 + dpp<kDppXor1>(w3_0);
  const float s41 = w3_1 + dpp<kDppXor1>(w3_1);
  float w4 = hi ? s41 : s40;
  w4 += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, w4), 0x401F));
  w4 += __shfl_xor(w4, 32, kWave);
  constexpr uint64_t kFieldPlus1 =
      NV == 10 ? 0x7a098600540321ull : 0xa098600540321ull;  // 4 bits per lane 0..15
  const int f = lane < 16 ? int((kFieldPlus1 >> (4 * lane)) & 15u) - 1 : -1;
  if (f >= 0) atomicAdd(dst + f, w4);
}

template <int PPT, bool DEPTH>
__global__ __launch_bounds__(kTilePix / PPT) void k_raster_bwd(
    const float* __restrict__ screen, const uint32_t* __restrict__ ids,
    const int64_t* __restrict__ toff, const uint32_t* __restrict__ order, int W, int H,
    int tiles_x, int T, const float* __restrict__ background, const float* __restrict__ out_T,
    const int32_t* __restrict__ last_ids, const float* __restrict__ v_rgb,
    const float* __restrict__ v_T, const float* __restrict__ v_depth,
    float* __restrict__ v_screen, float* __restrict__ v_background) {
  constexpr int NT = kTilePix / PPT;
  static_assert(NT % kTile == 0, "a lane's pixels share one column");
  constexpr int B = NT;
  __shared__ float4 s_a[B];
  __shared__ float4 s_b[B];
  __shared__ float2 s_c[B];
  __shared__ float s_z[DEPTH ? B : 1];
  __shared__ uint32_t s_id[B];
  __shared__ int s_lid[B];
  __shared__ int s_wcnt[NT / kWave];
  __shared__ int s_max;
  const int tid = threadIdx.x;
  const int64_t t = order ? int64_t(order[blockIdx.x]) : int64_t(blockIdx.x);
  const int c = int(t / T);
  const int tl = int(t - int64_t(c) * T);
  const int ty = tl / tiles_x, tx = tl - ty * tiles_x;
  const int64_t start = toff[t], end = toff[t + 1];
  if (tid == 0) s_max = -1;

  // Per pixel: current transmittance (walking back to front), the running
  // dot product P = g . sum_{later} colour alpha T (depth included as a
  // fourth channel), the upstream colour and depth gradients g, gD, and
  // the T gradient term (g_T + g . bg) T_final (the background hook).
  float px[PPT], py[PPT], Tc[PPT], Pd[PPT], g0[PPT], g1[PPT], g2[PPT], gD[PPT], gTT[PPT];
  int last[PPT];
  int my_max = -1;
  float bg0 = 0.f, bg1 = 0.f, bg2 = 0.f;
  if (background) {
    bg0 = background[3 * c + 0];
    bg1 = background[3 * c + 1];
    bg2 = background[3 * c + 2];
  }
  float vb0 = 0.f, vb1 = 0.f, vb2 = 0.f;  // this lane's share of dL/dbg
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int p = tid + k * NT;
    const int X = tx * kTile + (p & 15), Yp = ty * kTile + (p >> 4);
    const bool in = X < W && Yp < H;
    px[k] = float(X) + 0.5f;
    py[k] = float(Yp) + 0.5f;
    Pd[k] = 0.f;
    if (in) {
      const int64_t pix = (int64_t(c) * H + Yp) * W + X;
      Tc[k] = out_T[pix];
      last[k] = last_ids[pix];
      g0[k] = v_rgb[3 * pix + 0];
      g1[k] = v_rgb[3 * pix + 1];
      g2[k] = v_rgb[3 * pix + 2];
      gD[k] = DEPTH ? v_depth[pix] : 0.f;
      const float gT = (v_T ? v_T[pix] : 0.f) + fmaf(g2[k], bg2, fmaf(g1[k], bg1, g0[k] * bg0));
      gTT[k] = gT * Tc[k];
      vb0 = fmaf(g0[k], Tc[k], vb0);
      vb1 = fmaf(g1[k], Tc[k], vb1);
      vb2 = fmaf(g2[k], Tc[k], vb2);
    } else {
      Tc[k] = 1.f;
      last[k] = -1;
      g0[k] = g1[k] = g2[k] = gD[k] = gTT[k] = 0.f;
    }
    my_max = max(my_max, last[k]);
  }
  if (v_background) {
    // dL/dbg = sum over the camera's pixels of v_rgb T_final
    vb0 = wave_sum(vb0);
    vb1 = wave_sum(vb1);
    vb2 = wave_sum(vb2);
    if ((tid & (kWave - 1)) == 0) {
      atomicAdd(v_background + 3 * c + 0, vb0);
      atomicAdd(v_background + 3 * c + 1, vb1);
      atomicAdd(v_background + 3 * c + 2, vb2);
    }
  }
  __syncthreads();
  if (my_max >= 0) atomicMax(&s_max, my_max);
  __syncthreads();
  const int n_used = s_max + 1;
  if (n_used <= 0 || end <= start) return;
  const int64_t stop_at = start + n_used;

  const float tx0 = float(tx * kTile) + 0.5f, ty0 = float(ty * kTile) + 0.5f;
  const float tx1 = fminf(tx0 + 15.f, float(W) - 0.5f), ylast = float(H) - 0.5f;
  for (int64_t b_end = stop_at; b_end > start; b_end -= B) {
    const int64_t b_start = (b_end - start) > B ? b_end - B : start;
    const int n_in = int(b_end - b_start);
    __syncthreads();
    Staged e;
    uint32_t sid = 0;
    bool keep = false;
    if (tid < n_in) {
      sid = ids[b_start + tid];
      e = stage_row(screen, sid);
      keep = reaches_tile(e, tx0, tx1, ty0, ylast);
    }
    int pos;
    const int nb = compact_slot<NT>(keep, s_wcnt, &pos);
    if (keep) {
      s_a[pos] = e.a;
      s_b[pos] = e.b;
      s_c[pos] = e.c;
      if (DEPTH) s_z[pos] = e.z;
      s_id[pos] = sid;
      s_lid[pos] = int(b_start - start) + tid;
    }
    __syncthreads();
    for (int j = nb - 1; j >= 0; --j) {
      const float4 A = s_a[j], Bv = s_b[j];
      const float2 Cv = s_c[j];
      const float zj = DEPTH ? s_z[j] : 0.f;
      const int lid = s_lid[j];
      // per-lane sums over its pixels, which share dx: the weights
      // dL/dsigma and their first and second moments in dy (the dx moments
      // follow from dx), sum of dL/dalpha raw, colour and depth grads
      const ColTerms ct = col_terms(A, Bv, px[0]);
      float s0 = 0.f, sy = 0.f, syy = 0.f, mo = 0.f;
      float gr = 0.f, gg = 0.f, gbl = 0.f, gz = 0.f;
      bool any = false;
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const Eval e = eval_splat(ct, A, Bv, py[k]);
        if (lid <= last[k] && e.alpha >= kAlphaMin) {
          any = true;
          const float om = __builtin_amdgcn_rcpf(1.f - e.alpha);
          const float Ti = Tc[k] * om;
          const float w = e.alpha * Ti;
          gr = fmaf(w, g0[k], gr);
          gg = fmaf(w, g1[k], gg);
          gbl = fmaf(w, g2[k], gbl);
          if (DEPTH) gz = fmaf(w, gD[k], gz);
          float gc = fmaf(g2[k], Cv.x, fmaf(g1[k], Bv.w, g0[k] * Bv.z));
          if (DEPTH) gc = fmaf(gD[k], zj, gc);
          const float va = fmaf(Ti, gc, -(Pd[k] + gTT[k]) * om);
          Pd[k] = fmaf(w, gc, Pd[k]);
          Tc[k] = Ti;
          if (e.raw <= kAlphaMax) {
            const float vs = -va * e.alpha;
            mo = fmaf(va, e.raw, mo);
            const float vy = vs * e.dy;
            s0 += vs;
            sy += vy;
            syy = fmaf(vy, e.dy, syy);
          }
        }
      }
      if (__ballot(any) != 0ull) {
        const float mx = ct.dx * s0, my = sy, mxx = (ct.dx * ct.dx) * s0, mxy = ct.dx * sy,
                    myy = syy;
        // dsigma/du = a dx + b dy, dsigma/dv = b dx + c dy, dsigma/da = dx^2/2,
        // dsigma/db = dx dy, dsigma/dc = dy^2/2, dalpha/do = exp(-sigma)
        const float a2 = A.z + A.z, c2 = A.w + A.w;
        float* dst = v_screen + int64_t(s_id[j]) * kRow;
        if (DEPTH) {
          const float vals[10] = {fmaf(a2, mx, Bv.x * my), fmaf(Bv.x, mx, c2 * my), 0.5f * mxx,
                                  mxy, 0.5f * myy, mo * Cv.y, gr, gg, gbl, gz};
          wave_reduce_atomic<10>(vals, dst);
        } else {
          const float vals[9] = {fmaf(a2, mx, Bv.x * my), fmaf(Bv.x, mx, c2 * my), 0.5f * mxx,
                                 mxy, 0.5f * myy, mo * Cv.y, gr, gg, gbl};
          wave_reduce_atomic<9>(vals, dst);
        }
      }
    }
  }
}

}  // namespace

// Pixels per lane of the forward and backward tiles (1, 2 or 4, i.e. 4, 2
// or 1 wave per tile). GS_RASTER_PPT_FWD / GS_RASTER_PPT_BWD override the
// defaults for launch-shape sweeps (0 = the default).
int ppt_from_env(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v) return dflt;
  const int p = std::atoi(v);
  return (p == 1 || p == 2 || p == 4) ? p : dflt;
}

// Forward: four waves per tile while tiles are few, then two (two pixels
// per lane, half the staging and barrier work per pixel), then one. Measured
// (ms at 1 / 2 / 4 pixels per lane): 640x480, 1,200 tiles, 0.106 / 0.110 /
// 0.166; 1024x512, 2,048 tiles, 0.105 / 0.096 / 0.117; 1920x1080, 8,160
// tiles, 0.234 / 0.192 / 0.196; 5-camera 1600x1064, 33,500 tiles, 1.09 /
// 0.76 / 0.70; 15M 5-camera, 21,730 tiles, 0.72 / 0.49 / 0.45; 7680x7680,
// 230,400 tiles, 3.81 / 2.85 / 2.38.
inline int fwd_ppt(int64_t tiles) { return tiles >= 16384 ? 4 : tiles >= 2048 ? 2 : 1; }

// Backward: one wave per tile (four pixels per lane: the per-entry
// reduction and atomics are paid once per 256 pixels) once there are
// enough tiles to fill the chip; with few tiles, more waves per tile.
// Measured: 1920x1080 (8,160 tiles) 0.43 ms at four pixels per lane, 0.49
// at two, 0.59 at one; 128x128 (64 tiles) 0.50, 0.37, 0.25 ms.
inline int bwd_ppt(int64_t tiles) { return tiles >= 2048 ? 4 : tiles >= 512 ? 2 : 1; }

hipError_t launch_raster_fwd(int C, int W, int H, const float* screen, const uint32_t* ids,
                             const int64_t* toff, const uint32_t* order, const float* background,
                             float* out_rgb, float* out_T, float* out_depth, int32_t* last_ids,
                             hipStream_t s) {
  const int ppt_env = ppt_from_env("GS_RASTER_PPT_FWD", 0);
  const int tiles_x = (W + kTile - 1) / kTile, tiles_y = (H + kTile - 1) / kTile;
  const int T = tiles_x * tiles_y;
  const int64_t blocks = int64_t(C) * T;
  if (blocks == 0) return hipSuccess;
  const int ppt = ppt_env ? ppt_env : fwd_ppt(blocks);
  if (!fits_dispatch(uint64_t(blocks), kTilePix)) return hipErrorInvalidConfiguration;
  const dim3 grid{uint32_t(blocks)};
#define GS_FWD(P, D)                                                                           \
  hipLaunchKernelGGL((k_raster_fwd<P, D>), grid, dim3(kTilePix / P), 0, s, screen, ids, toff,  \
                     order, W, H, tiles_x, T, background, out_rgb, out_T, out_depth, last_ids)
  ProfScope prof("k_raster_fwd", s);
  if (out_depth) {
    if (ppt == 4) GS_FWD(4, true); else if (ppt == 2) GS_FWD(2, true); else GS_FWD(1, true);
  } else {
    if (ppt == 4) GS_FWD(4, false); else if (ppt == 2) GS_FWD(2, false); else GS_FWD(1, false);
  }
#undef GS_FWD
  return hipGetLastError();
}

hipError_t launch_raster_bwd(int C, int W, int H, const float* screen, const uint32_t* ids,
                             const int64_t* toff, const uint32_t* order, const float* background,
                             const float* out_T, const int32_t* last_ids, const float* v_rgb,
                             const float* v_T, const float* v_depth, float* v_screen,
                             float* v_background, hipStream_t s) {
  const int ppt_env = ppt_from_env("GS_RASTER_PPT_BWD", 0);
  const int tiles_x = (W + kTile - 1) / kTile, tiles_y = (H + kTile - 1) / kTile;
  const int T = tiles_x * tiles_y;
  const int64_t blocks = int64_t(C) * T;
  if (blocks == 0) return hipSuccess;
  const int ppt = ppt_env ? ppt_env : bwd_ppt(blocks);
  if (!fits_dispatch(uint64_t(blocks), kTilePix)) return hipErrorInvalidConfiguration;
  const dim3 grid{uint32_t(blocks)};
#define GS_BWD(P, D)                                                                           \
  hipLaunchKernelGGL((k_raster_bwd<P, D>), grid, dim3(kTilePix / P), 0, s, screen, ids, toff,  \
                     order, W, H, tiles_x, T, background, out_T, last_ids, v_rgb, v_T, v_depth, \
                     v_screen, v_background)
  ProfScope prof("k_raster_bwd", s);
  if (v_depth) {
    if (ppt == 4) GS_BWD(4, true); else if (ppt == 2) GS_BWD(2, true); else GS_BWD(1, true);
  } else {
    if (ppt == 4) GS_BWD(4, false); else if (ppt == 2) GS_BWD(2, false); else GS_BWD(1, false);
  }
#undef GS_BWD
  return hipGetLastError();
}

}  // namespace gs
