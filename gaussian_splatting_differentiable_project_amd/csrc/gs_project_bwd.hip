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

template <int DEG, bool ADAM>
__global__ __launch_bounds__(kMaskGroup) void k_project_bwd(
    ProjectArgs a, const uint64_t* __restrict__ mask, const uint32_t* __restrict__ wg_scan,
    const float* __restrict__ v_screen, float* __restrict__ v_means, float* __restrict__ v_quats,
    float* __restrict__ v_log_scales, float* __restrict__ v_opacity_logits,
    float* __restrict__ v_sh, int accumulate, AdamArgs ad) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t g = int64_t(blockIdx.x) * kMaskGroup + tid;
  if (g >= a.N) return;
  const uint64_t lt = lanemask_lt();

  float gmu[3] = {0.f, 0.f, 0.f};
  float gM[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) gM[i] = 0.f;
  float glogit = 0.f;
  float gsh[K * 3];
#pragma unroll
  for (int i = 0; i < K * 3; ++i) gsh[i] = 0.f;

  bool any = false;
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

      // colour = max(0, sum_k sh_k Y_k(d) + 0.5), d = (mu - cc) / |mu - cc|
      float dx = G.mu[0] - k.cc[0], dy = G.mu[1] - k.cc[1], dz = G.mu[2] - k.cc[2];
      const float inv = 1.f / sqrtf(dx * dx + dy * dy + dz * dz);
      dx *= inv, dy *= inv, dz *= inv;
      float Y[K];
      sh_basis<DEG>(a.norm, dx, dy, dz, Y);
      float vraw[3];
#pragma unroll
      for (int ch = 0; ch < 3; ++ch) {
        float acc = 0.5f;
#pragma unroll
        for (int kk = 0; kk < K; ++kk) acc = fmaf(Y[kk], shc[3 * kk + ch], acc);
        vraw[ch] = acc > 0.f ? vrgb[ch] : 0.f;
      }
      float wY[K];
#pragma unroll
      for (int kk = 0; kk < K; ++kk) {
        gsh[3 * kk + 0] = fmaf(Y[kk], vraw[0], gsh[3 * kk + 0]);
        gsh[3 * kk + 1] = fmaf(Y[kk], vraw[1], gsh[3 * kk + 1]);
        gsh[3 * kk + 2] = fmaf(Y[kk], vraw[2], gsh[3 * kk + 2]);
        wY[kk] = shc[3 * kk] * vraw[0] + shc[3 * kk + 1] * vraw[1] + shc[3 * kk + 2] * vraw[2];
      }
      if constexpr (DEG > 0) {
        float gd[3] = {0.f, 0.f, 0.f};
        sh_basis_vjp<DEG>(a.norm, dx, dy, dz, wY, gd);
        const float dot = gd[0] * dx + gd[1] * dy + gd[2] * dz;
        gmu[0] += (gd[0] - dx * dot) * inv;
        gmu[1] += (gd[1] - dy * dot) * inv;
        gmu[2] += (gd[2] - dz * dot) * inv;
      }

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
  }

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
    // SH in runs of at most 12 values that divide the 3K values exactly
    // (3, 12, 9, 12 for degrees 0-3), to bound the registers held at once;
    // coefficient 0 (the first 3 values) is DC
    constexpr int kRun = (K * 3) % 12 == 0 ? 12 : ((K * 3) % 9 == 0 ? 9 : K * 3);
    static_assert((K * 3) % kRun == 0, "runs must tile the SH values");
    const int64_t e0 = g * (K * 3);
#pragma unroll
    for (int r = 0; r < K * 3; r += kRun)
      adam_run<kRun>(ad.p[4] + e0 + r, ad.m[4] + e0 + r, ad.v[4] + e0 + r, gsh + r, r == 0 ? 3 : 0,
                     ad.lr[4], ad.lr[5], ad);
  } else if (accumulate) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      v_means[3 * g + j] += gmu[j];
      v_log_scales[3 * g + j] += gls[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) v_quats[4 * g + j] += gq[j];
    v_opacity_logits[g] += glogit;
    float* out = v_sh + g * (K * 3);
#pragma unroll
    for (int i = 0; i < K * 3; ++i) out[i] += gsh[i];
  } else {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      v_means[3 * g + j] = gmu[j];
      v_log_scales[3 * g + j] = gls[j];
    }
    reinterpret_cast<float4*>(v_quats)[g] = make_float4(gq[0], gq[1], gq[2], gq[3]);
    v_opacity_logits[g] = glogit;
    float* out = v_sh + g * (K * 3);
#pragma unroll
    for (int i = 0; i < K * 3; ++i) out[i] = gsh[i];
  }
}

}  // namespace

hipError_t launch_project_bwd(const ProjectArgs& a, const uint64_t* mask,
                              const uint32_t* wg_scan, const float* v_screen, float* v_means,
                              float* v_quats, float* v_log_scales, float* v_opacity_logits,
                              float* v_sh, int accumulate, const AdamArgs* adam, hipStream_t s) {
  const int64_t blocks = a.N_pad / kMaskGroup;
  if (blocks == 0) return hipSuccess;
  if (!fits_dispatch(uint64_t(blocks), kMaskGroup)) return hipErrorInvalidConfiguration;
  const dim3 grid{uint32_t(blocks)}, block{uint32_t(kMaskGroup)};
  const AdamArgs ad = adam ? *adam : AdamArgs{};
#define GS_LAUNCH_PB(D, A)                                                                    \
  hipLaunchKernelGGL((k_project_bwd<D, A>), grid, block, 0, s, a, mask, wg_scan, v_screen,      \
                     v_means, v_quats, v_log_scales, v_opacity_logits, v_sh, accumulate, ad)
  ProfScope prof(adam ? "k_project_bwd_adam" : "k_project_bwd", s);
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
