// Projection backward: screen-row gradients -> parameter gradients.
//
// [BWD] section 5 (projection_3dgs_backward): the chain rule through the
// intrinsics and extrinsics sends each visible pair's screen gradient to
// the Gaussian's position, rotation, scale, opacity and SH coefficients,
// all in fp32. [BWD] section 6: only the first sub-batch zeroes the
// accumulators (our `accumulate` flag).
//
// [BWD] section 6 (fused projection backward + optimizer): the fused
// variant folds each Gaussian's gradient straight into an Adam step of its
// parameters and moments, so no gradient buffer is written.
//
// gfx950 mapping: the same Gaussian-major, 128-lane geometry as the
// projection passes. A lane owns one Gaussian, walks the cameras whose
// mask bit is set, recovers the pair's slot from the scan and the mask
// words exactly as the compaction pass assigned it, and keeps every
// per-Gaussian gradient in registers, so each output is written once and
// no atomics are needed across cameras.
#include "gs_internal.h"

namespace gs {

namespace {

// One Adam step of n consecutive parameter elements (bias corrections
// precomputed). The three arrays never overlap, and the restrict-qualified
// parameters say so: every load is issued before the first store, instead
// of one load-update-store round trip per element. Elements below
// n_first take lr_first, the others lr_rest.
template <int n>
__device__ __forceinline__ void adam_run(float* __restrict__ p, float* __restrict__ m,
                                         float* __restrict__ v, const float* g, int n_first,
                                         float lr_first, float lr_rest, const AdamArgs& ad) {
  float pp[n], mm[n], vv[n];
#pragma unroll
  for (int i = 0; i < n; ++i) {
    pp[i] = p[i];
    mm[i] = m[i];
    vv[i] = v[i];
  }
#pragma unroll
  for (int i = 0; i < n; ++i) {
    mm[i] = fmaf(ad.beta1, mm[i], (1.f - ad.beta1) * g[i]);
    vv[i] = fmaf(ad.beta2, vv[i], (1.f - ad.beta2) * g[i] * g[i]);
    const float lr = i < n_first ? lr_first : lr_rest;
    pp[i] -= lr * (mm[i] * ad.inv_bc1) / (sqrtf(vv[i] * ad.inv_bc2) + ad.eps);
  }
#pragma unroll
  for (int i = 0; i < n; ++i) {
    p[i] = pp[i];
    m[i] = mm[i];
    v[i] = vv[i];
  }
}

// View direction d = (mu - cc) / |mu - cc| (inv = 1 / |mu - cc|) and the
// SH basis there.
template <int DEG>
__device__ __forceinline__ void sh_dir_basis(const ShNorm& norm, const float* mu, const float* cc,
                                             float* d, float& inv, float* Y) {
  d[0] = mu[0] - cc[0], d[1] = mu[1] - cc[1], d[2] = mu[2] - cc[2];
  inv = 1.f / sqrtf(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
  d[0] *= inv, d[1] *= inv, d[2] *= inv;
  sh_basis<DEG>(norm, d[0], d[1], d[2], Y);
}

// The colour clamp: dL/draw = dL/drgb where the raw colour
// sum_k sh_k Y_k + 0.5 is positive, else 0.
template <int DEG>
__device__ __forceinline__ void sh_clamp_grad(const float* Y, const float* shc, const float* vrgb,
                                              float* vraw) {
  constexpr int K = (DEG + 1) * (DEG + 1);
#pragma unroll
  for (int ch = 0; ch < 3; ++ch) {
    float acc = 0.5f;
#pragma unroll
    for (int kk = 0; kk < K; ++kk) acc = fmaf(Y[kk], shc[3 * kk + ch], acc);
    vraw[ch] = acc > 0.f ? vrgb[ch] : 0.f;
  }
}

// dL/dsh_k += Y_k dL/draw.
template <int DEG>
__device__ __forceinline__ void sh_accumulate(const float* Y, const float* vraw, float* gsh) {
  constexpr int K = (DEG + 1) * (DEG + 1);
#pragma unroll
  for (int kk = 0; kk < K; ++kk) {
    gsh[3 * kk + 0] = fmaf(Y[kk], vraw[0], gsh[3 * kk + 0]);
    gsh[3 * kk + 1] = fmaf(Y[kk], vraw[1], gsh[3 * kk + 1]);
    gsh[3 * kk + 2] = fmaf(Y[kk], vraw[2], gsh[3 * kk + 2]);
  }
}

// The view direction's share of dL/dmu: through the basis at d, then
// through the normalisation d = (mu - cc) / |mu - cc|.
template <int DEG>
__device__ __forceinline__ void sh_dir_grad(const ShNorm& norm, const float* d, float inv,
                                            const float* shc, const float* vraw, float* gmu) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  if constexpr (DEG > 0) {
    float wY[K];
#pragma unroll
    for (int kk = 0; kk < K; ++kk)
      wY[kk] = shc[3 * kk] * vraw[0] + shc[3 * kk + 1] * vraw[1] + shc[3 * kk + 2] * vraw[2];
    float gd[3] = {0.f, 0.f, 0.f};
    sh_basis_vjp<DEG>(norm, d[0], d[1], d[2], wY, gd);
    const float dot = gd[0] * d[0] + gd[1] * d[1] + gd[2] * d[2];
    gmu[0] += (gd[0] - d[0] * dot) * inv;
    gmu[1] += (gd[1] - d[1] * dot) * inv;
    gmu[2] += (gd[2] - d[2] * dot) * inv;
  }
}

// The SH colour's part of one pair's backward: colour = max(0, sum_k
// sh_k Y_k(d) + 0.5) with d = (mu - cc) / |mu - cc| toward the camera
// centre cc. Adds dL/dsh into gsh and the view direction's share of dL/dmu
// into gmu.
template <int DEG>
__device__ __forceinline__ void pair_bwd_sh(const ShNorm& norm, const float* mu, const float* cc,
                                            const float* shc, const float* vrgb, float* gsh,
                                            float* gmu) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  float d[3], inv, Y[K], vraw[3];
  sh_dir_basis<DEG>(norm, mu, cc, d, inv, Y);
  sh_clamp_grad<DEG>(Y, shc, vrgb, vraw);
  sh_accumulate<DEG>(Y, vraw, gsh);
  sh_dir_grad<DEG>(norm, d, inv, shc, vraw, gmu);
}

// The geometric part of one pair's backward, from the pair's forward
// quantities P: the opacity logit, dL/dM (M = Rq diag(s)) through the conic,
// the EWA covariance and the camera rotation, and dL/dmu through the
// Jacobian's dependence on the camera-space point, (u, v) and the depth.
__device__ __forceinline__ void pair_bwd_geom(const Camera& k, const PairFwd<float>& P, float o,
                                              float vu, float vv, float va, float vb, float vc,
                                              float vo, float vz, float* gmu, float* gM,
                                              float& glogit) {
  // opacity = sigmoid(logit)
  glogit = fmaf(vo, o * (1.f - o), glogit);

  // conic = inverse of S: dL/dS = -A V A with V = [[va, vb/2], [vb/2, vc]]
  const float hb = 0.5f * vb;
  const float av00 = P.ca * va + P.cb * hb, av01 = P.ca * hb + P.cb * vc;
  const float av10 = P.cb * va + P.cc * hb, av11 = P.cb * hb + P.cc * vc;
  const float vS00 = -(av00 * P.ca + av01 * P.cb);
  const float vS01 = -(av00 * P.cb + av01 * P.cc);
  const float vS11 = -(av10 * P.cb + av11 * P.cc);

  // S = TM TM^T + blur  ->  dL/dTM = 2 vS TM
  float vT0[3], vT1[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    vT0[j] = 2.f * (vS00 * P.TM[j] + vS01 * P.TM[3 + j]);
    vT1[j] = 2.f * (vS01 * P.TM[j] + vS11 * P.TM[3 + j]);
  }
  // TM = J Wm with J = [[j00, 0, j02], [0, j11, j12]]
  const float z = P.z, iz = 1.f / z, iz2 = iz * iz;
  const float j00 = k.fx * iz, j02 = -k.fx * P.x * iz2;
  const float j11 = k.fy * iz, j12 = -k.fy * P.y * iz2;
  float vj00 = 0.f, vj02 = 0.f, vj11 = 0.f, vj12 = 0.f;
  float vW[9];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    vj00 += vT0[j] * P.Wm[j];
    vj02 += vT0[j] * P.Wm[6 + j];
    vj11 += vT1[j] * P.Wm[3 + j];
    vj12 += vT1[j] * P.Wm[6 + j];
    vW[j] = j00 * vT0[j];
    vW[3 + j] = j11 * vT1[j];
    vW[6 + j] = j02 * vT0[j] + j12 * vT1[j];
  }
  // Wm = Rcam M  ->  dL/dM += Rcam^T vW
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      gM[3 * i + j] += k.R[i] * vW[j] + k.R[3 + i] * vW[3 + j] + k.R[6 + i] * vW[6 + j];

  // camera-space point: through J, (u, v) and the depth column
  const float iz3 = iz2 * iz;
  const float vx = vj02 * (-k.fx * iz2) + vu * k.fx * iz;
  const float vy = vj12 * (-k.fy * iz2) + vv * k.fy * iz;
  const float vzz = vj00 * (-k.fx * iz2) + vj02 * (2.f * k.fx * P.x * iz3) +
                    vj11 * (-k.fy * iz2) + vj12 * (2.f * k.fy * P.y * iz3) -
                    vu * k.fx * P.x * iz2 - vv * k.fy * P.y * iz2 + vz;
  // p = Rcam mu + t
#pragma unroll
  for (int j = 0; j < 3; ++j) gmu[j] += k.R[j] * vx + k.R[3 + j] * vy + k.R[6 + j] * vzz;
}

// The per-Gaussian end of the backward but for the SH coefficients (see
// store_sh_rows): the rotation and scale gradients from dL/dM, then the
// gradients written (or added), or folded into one Adam step. `any` says
// whether a camera sees the Gaussian; without one every gradient is zero.
template <int DEG, bool ADAM>
__device__ __forceinline__ void finish_gaussian(int64_t g, bool any, const GaussLocal<float>& G,
                                                const float* gmu, const float* gM, float glogit,
                                                const float* gsh, float* __restrict__ v_means,
                                                float* __restrict__ v_quats,
                                                float* __restrict__ v_log_scales,
                                                float* __restrict__ v_opacity_logits,
                                                float* __restrict__ v_sh, int accumulate,
                                                const AdamArgs& ad) {
  // M = Rq diag(s): dRq = dM diag(s), ds_j = sum_i dM_ij Rq_ij
  float gq[4] = {0.f, 0.f, 0.f, 0.f};
  float gls[3] = {0.f, 0.f, 0.f};
  if (any) {
    float gR[9];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        gR[3 * i + j] = gM[3 * i + j] * G.s[j];
        gls[j] += gM[3 * i + j] * G.Rq[3 * i + j];
      }
#pragma unroll
    for (int j = 0; j < 3; ++j) gls[j] *= G.s[j];
    const float w = G.qh[0], x = G.qh[1], y = G.qh[2], z = G.qh[3];
    // d/d(w,x,y,z) of the rotation-matrix entries contracted with gR
    float vw = 2.f * (z * (gR[3] - gR[1]) + y * (gR[2] - gR[6]) + x * (gR[7] - gR[5]));
    float vx = 2.f * (y * (gR[1] + gR[3]) + z * (gR[2] + gR[6]) + w * (gR[7] - gR[5])) -
               4.f * x * (gR[4] + gR[8]);
    float vy = 2.f * (x * (gR[1] + gR[3]) + w * (gR[2] - gR[6]) + z * (gR[5] + gR[7])) -
               4.f * y * (gR[0] + gR[8]);
    float vz = 2.f * (w * (gR[3] - gR[1]) + x * (gR[2] + gR[6]) + y * (gR[5] + gR[7])) -
               4.f * z * (gR[0] + gR[4]);
    // through q / |q|
    const float dot = vw * w + vx * x + vy * y + vz * z;
    const float iqn = 1.f / G.qn;
    gq[0] = (vw - w * dot) * iqn;
    gq[1] = (vx - x * dot) * iqn;
    gq[2] = (vy - y * dot) * iqn;
    gq[3] = (vz - z * dot) * iqn;
  }

  if (ADAM) {
    // every element steps, a zero gradient included (as Adam would on
    // gradient buffers); each lane touches only its own Gaussian, so the
    // in-place parameter update cannot race with another lane's reads
    adam_run<3>(ad.p[0] + 3 * g, ad.m[0] + 3 * g, ad.v[0] + 3 * g, gmu, 3, ad.lr[0], ad.lr[0], ad);
    adam_run<4>(ad.p[1] + 4 * g, ad.m[1] + 4 * g, ad.v[1] + 4 * g, gq, 4, ad.lr[1], ad.lr[1], ad);
    adam_run<3>(ad.p[2] + 3 * g, ad.m[2] + 3 * g, ad.v[2] + 3 * g, gls, 3, ad.lr[2], ad.lr[2], ad);
    adam_run<1>(ad.p[3] + g, ad.m[3] + g, ad.v[3] + g, &glogit, 1, ad.lr[3], ad.lr[3], ad);
  } else if (accumulate) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      v_means[3 * g + j] += gmu[j];
      v_log_scales[3 * g + j] += gls[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) v_quats[4 * g + j] += gq[j];
    v_opacity_logits[g] += glogit;
  } else {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      store_stream(v_means + 3 * g + j, gmu[j]);
      store_stream(v_log_scales + 3 * g + j, gls[j]);
    }
    store_stream(reinterpret_cast<float4*>(v_quats) + g, make_float4(gq[0], gq[1], gq[2], gq[3]));
    store_stream(v_opacity_logits + g, glogit);
  }
}

// The SH part of the end of the backward for a wave's 64 consecutive
// Gaussians g0 .. g0 + 63 (lane l holds Gaussian g0 + l's 3K values in
// gsh): written as contiguous float4s, staged through LDS 32 rows at a
// time, so every store instruction covers 1 KB of consecutive memory
// instead of 64 scattered 16-byte pieces at the row stride. With ADAM the
// same walk applies one Adam step to the SH parameters and moments
// (coefficient 0, the first 3 values of a row, is DC). Rows past N are
// left alone. Every lane of the wave must call it; `stage` holds
// 32 * sh_stage_stride<DEG>() floats of this wave's LDS, free on entry and
// on exit.
// Row stride of the SH staging (floats): with 3K a multiple of 4, an odd
// number of 16-byte groups, so rows start 16-byte aligned and eight
// consecutive rows cover all 32 banks with their 4-word pieces; otherwise
// odd, so single-word accesses of 32 rows fall in 32 different banks.
template <int DEG>
constexpr int sh_stage_stride() {
  constexpr int R = 3 * (DEG + 1) * (DEG + 1);
  return R % 4 == 0 ? ((R / 4) % 2 == 1 ? R : R + 4) : (R % 2 == 1 ? R : R + 1);
}

template <int DEG, bool ADAM>
__device__ __forceinline__ void store_sh_rows(float* stage, const float* gsh, int64_t g0,
                                              int64_t N, float* __restrict__ v_sh,
                                              int accumulate, const AdamArgs& ad) {
  constexpr int R = 3 * (DEG + 1) * (DEG + 1);
  constexpr int S = sh_stage_stride<DEG>();
  const int lane = __lane_id();
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    const int r0 = h * 32;
    if (lane >= r0 && lane < r0 + 32) {
      float* dst = stage + (lane - r0) * S;
#pragma unroll
      for (int i = 0; i < R; ++i) dst[i] = gsh[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const int64_t rows = N - (g0 + r0) < 32 ? N - (g0 + r0) : 32;
    if (rows > 0) {
      const int n = int(rows) * R;   // floats of this half
      const int64_t e0 = (g0 + r0) * R;
      if (ADAM) {
        float* __restrict__ p = ad.p[4] + e0;
        float* __restrict__ m = ad.m[4] + e0;
        float* __restrict__ v = ad.v[4] + e0;
        for (int i = lane; i < n; i += kWave) {
          const int row = i / R, col = i - row * R;
          const float gr = stage[row * S + col];
          const float lr = col < 3 ? ad.lr[4] : ad.lr[5];
          const float mm = fmaf(ad.beta1, m[i], (1.f - ad.beta1) * gr);
          const float vv = fmaf(ad.beta2, v[i], (1.f - ad.beta2) * gr * gr);
          p[i] -= lr * (mm * ad.inv_bc1) / (sqrtf(vv * ad.inv_bc2) + ad.eps);
          m[i] = mm;
          v[i] = vv;
        }
      } else {
        if constexpr (R % 4 == 0) {
          // e0 * 4 bytes is a multiple of 128: float4 from an aligned base
          float4* __restrict__ dst = reinterpret_cast<float4*>(v_sh + e0);
          constexpr int R4 = R / 4;
          const int n4 = n >> 2;
          for (int q = lane; q < n4; q += kWave) {
            const int row = q / R4, col = q - row * R4;
            float4 x = *reinterpret_cast<const float4*>(stage + row * S + 4 * col);
            if (accumulate) {
              const float4 y = dst[q];
              x.x += y.x, x.y += y.y, x.z += y.z, x.w += y.w;
              dst[q] = x;
            } else {
              store_stream(dst + q, x);
            }
          }
        } else {
          for (int i = lane; i < n; i += kWave) {
            const int row = i / R, col = i - row * R;
            const float x = stage[row * S + col];
            v_sh[e0 + i] = accumulate ? v_sh[e0 + i] + x : x;
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
}

template <int DEG, bool ADAM>
__global__ __launch_bounds__(kMaskGroup) void k_project_bwd(
    ProjectArgs a, const uint64_t* __restrict__ mask, const uint32_t* __restrict__ wg_scan,
    const float* __restrict__ v_screen, float* __restrict__ v_means, float* __restrict__ v_quats,
    float* __restrict__ v_log_scales, float* __restrict__ v_opacity_logits,
    float* __restrict__ v_sh, int accumulate, AdamArgs ad) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  __shared__ __align__(16) float s_stage[2][32 * sh_stage_stride<DEG>()];  // per wave: SH staging
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t g = int64_t(blockIdx.x) * kMaskGroup + tid;
  const bool valid = g < a.N;
  const uint64_t lt = lanemask_lt();

  float gmu[3] = {0.f, 0.f, 0.f};
  float gM[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) gM[i] = 0.f;
  float glogit = 0.f;
  float gsh[K * 3];
#pragma unroll
  for (int i = 0; i < K * 3; ++i) gsh[i] = 0.f;

  bool any = false;   // padding lanes have no bits set
  for (int c = 0; c < a.C; ++c) {
    const int64_t p0 = int64_t(c) * a.N_pad + int64_t(blockIdx.x) * kMaskGroup;
    any |= ((mask[p0 / 64 + wave] >> lane) & 1ull) != 0;
  }

  GaussLocal<float> G;
  float o = 0.f;
  if (any) {
    gauss_local(a.means, a.quats, a.log_scales, g, G);
    o = 1.f / (1.f + expf(-a.opacity_logits[g]));
    float shc[K * 3];
    const float* shg = a.sh + g * (K * 3);
#pragma unroll
    for (int i = 0; i < K * 3; ++i) shc[i] = shg[i];
    const float Wf = float(a.W), Hf = float(a.H);

    for (int c = 0; c < a.C; ++c) {
      const int64_t p0 = int64_t(c) * a.N_pad + int64_t(blockIdx.x) * kMaskGroup;
      const uint64_t w0 = mask[p0 / 64], w1 = mask[p0 / 64 + 1];
      const uint64_t mine = wave ? w1 : w0;
      if (!((mine >> lane) & 1ull)) continue;
      const int64_t slot = int64_t(wg_scan[p0 / kMaskGroup]) + (wave ? __popcll(w0) : 0) +
                           __popcll(mine & lt);
      const float2* vr = reinterpret_cast<const float2*>(v_screen + slot * kRow);
      const float2 r0 = vr[0], r1 = vr[1], r2 = vr[2], r3 = vr[3], r4 = vr[4];
      const float vu = r0.x, vv = r0.y, va = r1.x, vb = r1.y, vc = r2.x, vo = r2.y, vz = r3.x;
      const float vrgb[3] = {r3.y, r4.x, r4.y};

      const Camera k = load_camera(a.viewmats, a.Ks, c);
      PairFwd<float> P;
      pair_fwd<float>(k, G, Wf, Hf, P);

      pair_bwd_sh<DEG>(a.norm, G.mu, k.cc, shc, vrgb, gsh, gmu);
      pair_bwd_geom(k, P, o, vu, vv, va, vb, vc, vo, vz, gmu, gM, glogit);
    }
  }

  store_sh_rows<DEG, ADAM>(s_stage[wave], gsh, int64_t(blockIdx.x) * kMaskGroup + wave * kWave,
                           a.N, v_sh, accumulate, ad);
  if (!valid) return;
  finish_gaussian<DEG, ADAM>(g, any, G, gmu, gM, glogit, gsh, v_means, v_quats, v_log_scales,
                             v_opacity_logits, v_sh, accumulate, ad);
}


// Pair-queue variant for scenes of 2 to kPbMaxCams cameras. Walking every
// camera in every lane runs the per-pair arithmetic with only the lanes of
// visible pairs active: about one in five in a five-camera scene. Here one
// wave owns 64 Gaussians (half a mask group):
//  1. it lists the wave's visible pairs in LDS Gaussian by Gaussian (each
//     lane's pairs contiguous, cameras ascending), and puts the
//     camera-independent data of its Gaussians (position, M, opacity) and
//     the cameras in LDS;
//  2. then, 64 listed pairs at a time, one lane per pair (all lanes busy)
//     runs the geometric backward and the view direction's share of the SH
//     colour's backward, reading the pair's SH coefficients from memory
//     (each Gaussian's row is shared by its few visible cameras and stays in
//     cache), and leaves its 13 sums (dL/dmu, dL/dM, dL/dlogit) and its
//     clamped colour gradient in LDS;
//  3. and each lane adds the results of its own pairs in that batch (a
//     contiguous run: no atomics, no two lanes on one row).
// After the last batch each lane accumulates dL/dsh = sum over its cameras
// of Y(d) dL/draw in registers and finishes its Gaussian as the
// camera-walking kernel does (recomputing the Gaussian's local frame, which
// keeps it out of the registers live across the batches).
constexpr int kPbMaxCams = 8;
constexpr int kPbRes = 13;  // per pair: dL/dmu (3), dL/dM (9), dL/dlogit
constexpr int kPbCam = 20;  // floats per staged camera: R, t, fx, fy, cx, cy, cc, pad

__host__ __device__ constexpr size_t pb_queue_bytes(int C) {
  return size_t(kWave) * size_t(C) * (sizeof(uint32_t) + 3 * sizeof(float));
}

__device__ __forceinline__ Camera camera_from(const float* sc) {
  Camera k;
#pragma unroll
  for (int i = 0; i < 9; ++i) k.R[i] = sc[i];
#pragma unroll
  for (int i = 0; i < 3; ++i) k.t[i] = sc[9 + i];
  k.fx = sc[12], k.fy = sc[13], k.cx = sc[14], k.cy = sc[15];
#pragma unroll
  for (int i = 0; i < 3; ++i) k.cc[i] = sc[16 + i];
  return k;
}

template <int DEG, bool ADAM>
__global__ __launch_bounds__(kWave) void k_project_bwd_pairs(
    ProjectArgs a, const uint64_t* __restrict__ mask, const uint32_t* __restrict__ wg_scan,
    const float* __restrict__ v_screen, float* __restrict__ v_means, float* __restrict__ v_quats,
    float* __restrict__ v_log_scales, float* __restrict__ v_opacity_logits,
    float* __restrict__ v_sh, int accumulate, AdamArgs ad) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  // per-Gaussian data and per-pair results; at the end, the SH staging
  constexpr int kStage = 32 * sh_stage_stride<DEG>();
  constexpr int kPool = (13 + kPbRes) * kWave > kStage ? (13 + kPbRes) * kWave : kStage;
  __shared__ __align__(16) float s_pool[kPool];
  float(*s_mu)[kWave] = reinterpret_cast<float(*)[kWave]>(s_pool);
  float(*s_M)[kWave] = reinterpret_cast<float(*)[kWave]>(s_pool + 3 * kWave);
  float* s_o = s_pool + 12 * kWave;
  float(*s_res)[kWave] = reinterpret_cast<float(*)[kWave]>(s_pool + 13 * kWave);
  __shared__ float s_cam[kPbMaxCams * kPbCam];
  __shared__ uint32_t s_base[kPbMaxCams];  // slot of each camera's first pair of the wave
  __shared__ uint64_t s_mine[kPbMaxCams];  // each camera's visible lanes
  extern __shared__ uint32_t s_dyn[];
  const int lane = threadIdx.x;
  const int C = a.C;
  uint32_t* s_who = s_dyn;                                       // [64 C] camera << 6 | lane
  float* s_vraw = reinterpret_cast<float*>(s_dyn + kWave * C);   // [3][64 C] dL/draw
  const int qcap = kWave * C;

  const int64_t blk = blockIdx.x;
  const int64_t grp = blk >> 1;
  const int half = int(blk & 1);
  const int64_t g = blk * kWave + lane;

  // 1. which cameras see each lane's Gaussian; the list offsets
  const CamWords cw = load_cam_words(mask, wg_scan, a.N_pad, grp, 0, C);
  uint32_t vmask = 0;  // cameras that see this lane's Gaussian
  for (int c = 0; c < C; ++c) {
    const uint64_t w0 = cam_w0(cw, c), w1 = cam_w1(cw, c);
    const uint64_t mine = half ? w1 : w0;
    if (lane == 0) {
      s_mine[c] = mine;
      s_base[c] = cam_base(cw, c) + (half ? uint32_t(__popcll(w0)) : 0u);
    }
    vmask |= uint32_t((mine >> lane) & 1ull) << c;
  }
  const int cnt = __popc(vmask);
  const int off = int(wave_incl_scan_u32(uint32_t(cnt))) - cnt;  // first list entry
  const int qn = __builtin_amdgcn_readlane(off + cnt, 63);      // wave-uniform
  const bool any = cnt != 0;
  float gmu[3] = {0.f, 0.f, 0.f}, gM[9], glogit = 0.f, gsh[K * 3];
#pragma unroll
  for (int i = 0; i < 9; ++i) gM[i] = 0.f;
#pragma unroll
  for (int i = 0; i < K * 3; ++i) gsh[i] = 0.f;

  if (qn > 0) {  // wave-uniform
    {
      uint32_t vm = vmask;
      for (int j = off; vm; ++j) {
        const int c = __builtin_ctz(vm);
        vm &= vm - 1u;
        s_who[j] = (uint32_t(c) << 6) | uint32_t(lane);
      }
    }
    if (any) {
      GaussLocal<float> G;
      gauss_local(a.means, a.quats, a.log_scales, g, G);
#pragma unroll
      for (int i = 0; i < 3; ++i) s_mu[i][lane] = G.mu[i];
#pragma unroll
      for (int i = 0; i < 9; ++i) s_M[i][lane] = G.M[i];
      s_o[lane] = 1.f / (1.f + expf(-a.opacity_logits[g]));
    }
    if (lane < C) {
      const Camera k = load_camera(a.viewmats, a.Ks, lane);
      float* sc = s_cam + lane * kPbCam;
#pragma unroll
      for (int i = 0; i < 9; ++i) sc[i] = k.R[i];
#pragma unroll
      for (int i = 0; i < 3; ++i) sc[9 + i] = k.t[i];
      sc[12] = k.fx, sc[13] = k.fy, sc[14] = k.cx, sc[15] = k.cy;
#pragma unroll
      for (int i = 0; i < 3; ++i) sc[16 + i] = k.cc[i];
    }
    __syncthreads();

    const float Wf = float(a.W), Hf = float(a.H);
    for (int b = 0; b < qn; b += kWave) {
      // 2. one lane per listed pair
      const int e = b + lane;
      if (e < qn) {
        const uint32_t who = s_who[e];
        const int c = int(who >> 6), gl = int(who & 63u);
        // a camera's visible lanes take consecutive slots
        const int64_t slot = int64_t(s_base[c]) + __popcll(s_mine[c] & ((1ull << gl) - 1ull));
        const float2* vr = reinterpret_cast<const float2*>(v_screen + slot * kRow);
        const float2 r0 = vr[0], r1 = vr[1], r2 = vr[2], r3 = vr[3], r4 = vr[4];
        float shc[K * 3];
        const float* shg = a.sh + (blk * kWave + gl) * (K * 3);
#pragma unroll
        for (int i = 0; i < K * 3; ++i) shc[i] = shg[i];
        const Camera k = camera_from(s_cam + c * kPbCam);
        GaussLocal<float> Gp;
#pragma unroll
        for (int i = 0; i < 3; ++i) Gp.mu[i] = s_mu[i][gl];
#pragma unroll
        for (int i = 0; i < 9; ++i) Gp.M[i] = s_M[i][gl];
        PairFwd<float> P;
        pair_fwd<float>(k, Gp, Wf, Hf, P);
        float pmu[3] = {0.f, 0.f, 0.f}, pM[9], plogit = 0.f;
#pragma unroll
        for (int i = 0; i < 9; ++i) pM[i] = 0.f;
        pair_bwd_geom(k, P, s_o[gl], r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, pmu, pM, plogit);
        float d[3], inv, Y[K], vraw[3];
        const float vrgb[3] = {r3.y, r4.x, r4.y};
        sh_dir_basis<DEG>(a.norm, Gp.mu, k.cc, d, inv, Y);
        sh_clamp_grad<DEG>(Y, shc, vrgb, vraw);
        sh_dir_grad<DEG>(a.norm, d, inv, shc, vraw, pmu);
#pragma unroll
        for (int j = 0; j < 3; ++j) s_res[j][lane] = pmu[j];
#pragma unroll
        for (int j = 0; j < 9; ++j) s_res[3 + j][lane] = pM[j];
        s_res[12][lane] = plogit;
#pragma unroll
        for (int j = 0; j < 3; ++j) s_vraw[j * qcap + e] = vraw[j];
      }
      __syncthreads();
      // 3. each lane: its own pairs of this batch
      const int j1 = min(off + cnt, b + kWave);
      for (int j = max(off, b); j < j1; ++j) {
        const int r = j - b;
#pragma unroll
        for (int i = 0; i < 3; ++i) gmu[i] += s_res[i][r];
#pragma unroll
        for (int i = 0; i < 9; ++i) gM[i] += s_res[3 + i][r];
        glogit += s_res[12][r];
      }
      __syncthreads();
    }
    // dL/dsh over this lane's cameras (its list entries, cameras ascending)
    if (any) {
      const float mu[3] = {s_mu[0][lane], s_mu[1][lane], s_mu[2][lane]};
      uint32_t vm = vmask;
      for (int j = off; vm; ++j) {
        const int c = __builtin_ctz(vm);
        vm &= vm - 1u;
        const float vraw[3] = {s_vraw[j], s_vraw[qcap + j], s_vraw[2 * qcap + j]};
        float d[3], inv, Y[K];
        sh_dir_basis<DEG>(a.norm, mu, s_cam + c * kPbCam + 16, d, inv, Y);
        sh_accumulate<DEG>(Y, vraw, gsh);
      }
    }
  }
  store_sh_rows<DEG, ADAM>(s_pool, gsh, blk * kWave, a.N, v_sh, accumulate, ad);
  if (g >= a.N) return;
  GaussLocal<float> G;
  if (any) gauss_local(a.means, a.quats, a.log_scales, g, G);
  finish_gaussian<DEG, ADAM>(g, any, G, gmu, gM, glogit, gsh, v_means, v_quats, v_log_scales,
                             v_opacity_logits, v_sh, accumulate, ad);
}

}  // namespace

hipError_t launch_project_bwd(const ProjectArgs& a, const uint64_t* mask,
                              const uint32_t* wg_scan, const float* v_screen, float* v_means,
                              float* v_quats, float* v_log_scales, float* v_opacity_logits,
                              float* v_sh, int accumulate, const AdamArgs* adam, hipStream_t s) {
  const int64_t blocks = a.N_pad / kMaskGroup;
  if (blocks == 0) return hipSuccess;
  if (!fits_dispatch(uint64_t(blocks), kMaskGroup)) return hipErrorInvalidConfiguration;
  const AdamArgs ad = adam ? *adam : AdamArgs{};
  ProfScope prof(adam ? "k_project_bwd_adam" : "k_project_bwd", s);
  if (a.C >= 2 && a.C <= kPbMaxCams) {
    // pair queue: one wave per 64 Gaussians
    const dim3 grid{uint32_t(2 * blocks)}, block{uint32_t(kWave)};
    const size_t shm = pb_queue_bytes(a.C);
#define GS_LAUNCH_PBQ(D, A)                                                                    \
  hipLaunchKernelGGL((k_project_bwd_pairs<D, A>), grid, block, shm, s, a, mask, wg_scan,         \
                     v_screen, v_means, v_quats, v_log_scales, v_opacity_logits, v_sh,           \
                     accumulate, ad)
    if (adam) {
      switch (a.deg) {
        case 0: GS_LAUNCH_PBQ(0, true); break;
        case 1: GS_LAUNCH_PBQ(1, true); break;
        case 2: GS_LAUNCH_PBQ(2, true); break;
        default: GS_LAUNCH_PBQ(3, true); break;
      }
    } else {
      switch (a.deg) {
        case 0: GS_LAUNCH_PBQ(0, false); break;
        case 1: GS_LAUNCH_PBQ(1, false); break;
        case 2: GS_LAUNCH_PBQ(2, false); break;
        default: GS_LAUNCH_PBQ(3, false); break;
      }
    }
#undef GS_LAUNCH_PBQ
    return hipGetLastError();
  }
  const dim3 grid{uint32_t(blocks)}, block{uint32_t(kMaskGroup)};
#define GS_LAUNCH_PB(D, A)                                                                    \
  hipLaunchKernelGGL((k_project_bwd<D, A>), grid, block, 0, s, a, mask, wg_scan, v_screen,      \
                     v_means, v_quats, v_log_scales, v_opacity_logits, v_sh, accumulate, ad)
  if (adam) {
    switch (a.deg) {
      case 0: GS_LAUNCH_PB(0, true); break;
      case 1: GS_LAUNCH_PB(1, true); break;
      case 2: GS_LAUNCH_PB(2, true); break;
      default: GS_LAUNCH_PB(3, true); break;
    }
  } else {
    switch (a.deg) {
      case 0: GS_LAUNCH_PB(0, false); break;
      case 1: GS_LAUNCH_PB(1, false); break;
      case 2: GS_LAUNCH_PB(2, false); break;
      default: GS_LAUNCH_PB(3, false); break;
    }
  }
#undef GS_LAUNCH_PB
  return hipGetLastError();
}

}  // namespace gs
