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
// gfx950 mapping: one work-group per 16x16 tile; PPT pixels per lane, so
// a 256-pixel tile is 256/PPT lanes. Screen rows of a batch of the tile's
// list are staged in LDS (gathered through the flattened ids) and read
// back as wave-uniform broadcasts. The backward sums each entry's
// gradient over the PPT pixels of a lane, then over the wave with DPP row
// rotations, and issues one fp32 atomic per field per wave -- and only
// for waves where some pixel actually composited the entry.
#include "gs_internal.h"

namespace gs {

namespace {

__device__ __forceinline__ float fast_exp_neg(float s) {
  // exp(-s) through the hardware base-2 exponential
  return __builtin_amdgcn_exp2f(-s * kLog2e);
}

// sigma = (a dx^2 + c dy^2) / 2 + b dx dy, written with explicit fused
// operations only, so the forward and the backward (separate kernels)
// round it identically and take the same skip decisions.
__device__ __forceinline__ float splat_sigma(float a, float b, float c, float dx, float dy) {
  return fmaf(b * dx, dy, 0.5f * fmaf(a, dx * dx, c * (dy * dy)));
}

template <int PPT>
__global__ __launch_bounds__(kTilePix / PPT) void k_raster_fwd(
    const float* __restrict__ screen, const uint32_t* __restrict__ ids,
    const int64_t* __restrict__ toff, int W, int H, int tiles_x, int T,
    float* __restrict__ out_rgb, float* __restrict__ out_T, int32_t* __restrict__ last_ids) {
  constexpr int NT = kTilePix / PPT;
  constexpr int B = NT;
  __shared__ float4 s_a[B];  // u, v, conic a, conic b
  __shared__ float4 s_b[B];  // conic c, opacity, r, g
  __shared__ float s_c[B];   // b
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int c = int(t / T);
  const int tl = int(t - int64_t(c) * T);
  const int ty = tl / tiles_x, tx = tl - ty * tiles_x;
  const int64_t start = toff[t], end = toff[t + 1];

  float px[PPT], py[PPT], Tr[PPT], cr[PPT], cg[PPT], cb[PPT];
  int last[PPT];
  bool live[PPT];
  int64_t pix[PPT];
  bool inside[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int p = tid + k * NT;
    const int X = tx * kTile + (p & 15), Yp = ty * kTile + (p >> 4);
    inside[k] = X < W && Yp < H;
    live[k] = inside[k];
    px[k] = float(X) + 0.5f;
    py[k] = float(Yp) + 0.5f;
    pix[k] = (int64_t(c) * H + Yp) * W + X;
    Tr[k] = 1.f;
    cr[k] = cg[k] = cb[k] = 0.f;
    last[k] = -1;
  }

  for (int64_t b0 = start; b0 < end; b0 += B) {
    bool any_live = false;
#pragma unroll
    for (int k = 0; k < PPT; ++k) any_live |= live[k];
    if (__syncthreads_count(any_live) == 0) break;
    if (b0 + tid < end) {
      const uint32_t s = ids[b0 + tid];
      const float2* r = reinterpret_cast<const float2*>(screen + int64_t(s) * kRow);
      const float2 r0 = r[0], r1 = r[1], r2 = r[2], r3 = r[3], r4 = r[4];
      s_a[tid] = make_float4(r0.x, r0.y, r1.x, r1.y);
      s_b[tid] = make_float4(r2.x, r2.y, r3.y, r4.x);
      s_c[tid] = r4.y;
    }
    __syncthreads();
    const int nb = int((end - b0) < B ? (end - b0) : B);
    for (int j = 0; j < nb; ++j) {
      const float4 A = s_a[j], Bv = s_b[j];
      const float cblue = s_c[j];
      const int lid = int(b0 - start) + j;
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const float dx = A.x - px[k], dy = A.y - py[k];
        const float sig = splat_sigma(A.z, A.w, Bv.x, dx, dy);
        const float alpha = fminf(kAlphaMax, Bv.y * fast_exp_neg(sig));
        const float Tn = Tr[k] * (1.f - alpha);
        const bool use = live[k] && sig >= 0.f && alpha >= kAlphaMin;
        const bool stop = use && Tn < kTStop;
        if (stop) live[k] = false;
        if (use && !stop) {
          const float w = alpha * Tr[k];
          cr[k] = fmaf(Bv.z, w, cr[k]);
          cg[k] = fmaf(Bv.w, w, cg[k]);
          cb[k] = fmaf(cblue, w, cb[k]);
          Tr[k] = Tn;
          last[k] = lid;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    if (!inside[k]) continue;
    out_rgb[3 * pix[k] + 0] = cr[k];
    out_rgb[3 * pix[k] + 1] = cg[k];
    out_rgb[3 * pix[k] + 2] = cb[k];
    out_T[pix[k]] = Tr[k];
    last_ids[pix[k]] = last[k];
  }
}

template <int PPT>
__global__ __launch_bounds__(kTilePix / PPT) void k_raster_bwd(
    const float* __restrict__ screen, const uint32_t* __restrict__ ids,
    const int64_t* __restrict__ toff, int W, int H, int tiles_x, int T,
    const float* __restrict__ out_T, const int32_t* __restrict__ last_ids,
    const float* __restrict__ v_rgb, const float* __restrict__ v_T, float* __restrict__ v_screen) {
  constexpr int NT = kTilePix / PPT;
  constexpr int B = NT;
  __shared__ float4 s_a[B];  // u, v, conic a, conic b
  __shared__ float4 s_b[B];  // conic c, opacity, r, g
  __shared__ float s_c[B];   // b
  __shared__ uint32_t s_id[B];
  __shared__ int s_max;
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int c = int(t / T);
  const int tl = int(t - int64_t(c) * T);
  const int ty = tl / tiles_x, tx = tl - ty * tiles_x;
  const int64_t start = toff[t], end = toff[t + 1];
  if (tid == 0) s_max = -1;

  float px[PPT], py[PPT], Tc[PPT], S0[PPT], S1[PPT], S2[PPT], g0[PPT], g1[PPT], g2[PPT],
      gTT[PPT];
  int last[PPT];
  int my_max = -1;
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int p = tid + k * NT;
    const int X = tx * kTile + (p & 15), Yp = ty * kTile + (p >> 4);
    const bool in = X < W && Yp < H;
    px[k] = float(X) + 0.5f;
    py[k] = float(Yp) + 0.5f;
    S0[k] = S1[k] = S2[k] = 0.f;
    if (in) {
      const int64_t pix = (int64_t(c) * H + Yp) * W + X;
      Tc[k] = out_T[pix];
      last[k] = last_ids[pix];
      g0[k] = v_rgb[3 * pix + 0];
      g1[k] = v_rgb[3 * pix + 1];
      g2[k] = v_rgb[3 * pix + 2];
      gTT[k] = (v_T ? v_T[pix] : 0.f) * Tc[k];
    } else {
      Tc[k] = 1.f;
      last[k] = -1;
      g0[k] = g1[k] = g2[k] = gTT[k] = 0.f;
    }
    my_max = max(my_max, last[k]);
  }
  __syncthreads();
  if (my_max >= 0) atomicMax(&s_max, my_max);
  __syncthreads();
  const int n_used = s_max + 1;
  if (n_used <= 0 || end <= start) return;
  const int64_t stop_at = start + n_used;

  for (int64_t b_end = stop_at; b_end > start; b_end -= B) {
    const int64_t b_start = (b_end - start) > B ? b_end - B : start;
    const int nb = int(b_end - b_start);
    __syncthreads();
    if (tid < nb) {
      const uint32_t s = ids[b_start + tid];
      const float2* r = reinterpret_cast<const float2*>(screen + int64_t(s) * kRow);
      const float2 r0 = r[0], r1 = r[1], r2 = r[2], r3 = r[3], r4 = r[4];
      s_a[tid] = make_float4(r0.x, r0.y, r1.x, r1.y);
      s_b[tid] = make_float4(r2.x, r2.y, r3.y, r4.x);
      s_c[tid] = r4.y;
      s_id[tid] = s;
    }
    __syncthreads();
    for (int j = nb - 1; j >= 0; --j) {
      const float4 A = s_a[j], Bv = s_b[j];
      const float cblue = s_c[j];
      const int lid = int(b_start - start) + j;
      float gu = 0.f, gv = 0.f, ga = 0.f, gb = 0.f, gc = 0.f, go = 0.f, gr = 0.f, gg = 0.f,
            gbl = 0.f;
      bool any = false;
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const float dx = A.x - px[k], dy = A.y - py[k];
        const float sig = splat_sigma(A.z, A.w, Bv.x, dx, dy);
        const float ex = fast_exp_neg(sig);
        const float raw = Bv.y * ex;
        const float alpha = fminf(kAlphaMax, raw);
        const bool use = lid <= last[k] && sig >= 0.f && alpha >= kAlphaMin;
        if (use) {
          any = true;
          const float om = 1.f / (1.f - alpha);
          const float Ti = Tc[k] * om;
          const float w = alpha * Ti;
          gr = fmaf(w, g0[k], gr);
          gg = fmaf(w, g1[k], gg);
          gbl = fmaf(w, g2[k], gbl);
          const float va = g0[k] * (Bv.z * Ti - S0[k] * om) + g1[k] * (Bv.w * Ti - S1[k] * om) +
                           g2[k] * (cblue * Ti - S2[k] * om) - gTT[k] * om;
          S0[k] = fmaf(Bv.z, w, S0[k]);
          S1[k] = fmaf(Bv.w, w, S1[k]);
          S2[k] = fmaf(cblue, w, S2[k]);
          Tc[k] = Ti;
          if (raw <= kAlphaMax) {
            const float vs = -va * alpha;
            go = fmaf(va, ex, go);
            gu = fmaf(vs, A.z * dx + A.w * dy, gu);
            gv = fmaf(vs, A.w * dx + Bv.x * dy, gv);
            ga = fmaf(vs, 0.5f * dx * dx, ga);
            gb = fmaf(vs, dx * dy, gb);
            gc = fmaf(vs, 0.5f * dy * dy, gc);
          }
        }
      }
      if (__ballot(any) != 0ull) {
        gu = wave_sum(gu);
        gv = wave_sum(gv);
        ga = wave_sum(ga);
        gb = wave_sum(gb);
        gc = wave_sum(gc);
        go = wave_sum(go);
        gr = wave_sum(gr);
        gg = wave_sum(gg);
        gbl = wave_sum(gbl);
        if ((tid & 63) == 0) {
          float* dst = v_screen + int64_t(s_id[j]) * kRow;
          atomicAdd(dst + 0, gu);
          atomicAdd(dst + 1, gv);
          atomicAdd(dst + 2, ga);
          atomicAdd(dst + 3, gb);
          atomicAdd(dst + 4, gc);
          atomicAdd(dst + 5, go);
          atomicAdd(dst + 7, gr);
          atomicAdd(dst + 8, gg);
          atomicAdd(dst + 9, gbl);
        }
      }
    }
  }
}

}  // namespace

constexpr int kFwdPPT = 1;
constexpr int kBwdPPT = 1;

hipError_t launch_raster_fwd(int C, int W, int H, const float* screen, const uint32_t* ids,
                             const int64_t* toff, float* out_rgb, float* out_T, int32_t* last_ids,
                             hipStream_t s) {
  const int tiles_x = (W + kTile - 1) / kTile, tiles_y = (H + kTile - 1) / kTile;
  const int T = tiles_x * tiles_y;
  const int64_t blocks = int64_t(C) * T;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_raster_fwd<kFwdPPT>, dim3(uint32_t(blocks)), dim3(kTilePix / kFwdPPT), 0, s,
                     screen, ids, toff, W, H, tiles_x, T, out_rgb, out_T, last_ids);
  return hipGetLastError();
}

hipError_t launch_raster_bwd(int C, int W, int H, const float* screen, const uint32_t* ids,
                             const int64_t* toff, const float* out_T, const int32_t* last_ids,
                             const float* v_rgb, const float* v_T, float* v_screen,
                             hipStream_t s) {
  const int tiles_x = (W + kTile - 1) / kTile, tiles_y = (H + kTile - 1) / kTile;
  const int T = tiles_x * tiles_y;
  const int64_t blocks = int64_t(C) * T;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_raster_bwd<kBwdPPT>, dim3(uint32_t(blocks)), dim3(kTilePix / kBwdPPT), 0, s,
                     screen, ids, toff, W, H, tiles_x, T, out_T, last_ids, v_rgb, v_T, v_screen);
  return hipGetLastError();
}

}  // namespace gs
