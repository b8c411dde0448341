// Per-pair projection arithmetic shared by the compaction pass and the
// projection backward (both recompute it from the raw parameters).
//
// The pages print no projection formula; this is the textbook EWA
// splatting the trainer's projection and projection backward
// ([BWD] section 5) work with: camera point p = R mu + t, 3D covariance
// M M^T with M = R(q/|q|) diag(exp(log_scale)), 2D covariance
// J W W^T J^T + 0.3 I with W = R M and J the perspective Jacobian at p,
// 3-sigma radius from the larger eigenvalue, opacity = sigmoid(logit),
// colour = max(0, SH(view direction) + 0.5).
#pragma once

#include "gs_common.h"

namespace gs {

// Real SH normalisation constants N_{l,|m|} (sqrt(2) folded in for m != 0),
// order: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3).
// Filled on the host from sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!).
struct ShNorm {
  double n[10];
};

struct Camera {
  float R[9];  // world -> camera rotation, row-major
  float t[3];
  float fx, fy, cx, cy;
  float cc[3];  // camera centre -R^T t
};

__device__ __forceinline__ Camera load_camera(const float* __restrict__ viewmats,
                                              const float* __restrict__ Ks, int c) {
  Camera k;
  const float* V = viewmats + 16 * c;
  const float* Kc = Ks + 9 * c;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
#pragma unroll
    for (int j = 0; j < 3; ++j) k.R[3 * i + j] = V[4 * i + j];
    k.t[i] = V[4 * i + 3];
  }
  k.fx = Kc[0];
  k.fy = Kc[4];
  k.cx = Kc[2];
  k.cy = Kc[5];
#pragma unroll
  for (int j = 0; j < 3; ++j)
    k.cc[j] = -(k.R[j] * k.t[0] + k.R[3 + j] * k.t[1] + k.R[6 + j] * k.t[2]);
  return k;
}

// Depth in fp32 with every product and sum rounded separately, in the
// order ((R20 x + R21 y) + R22 z) + t2: its bits become the sort key, so
// its evaluation order is part of the result. Contraction into fused
// multiply-adds is switched off for this function.
__device__ __forceinline__ float depth_z32(const Camera& k, float mx, float my, float mz) {
#pragma clang fp contract(off)
  float z = k.R[6] * mx;
  z = z + k.R[7] * my;
  z = z + k.R[8] * mz;
  return z + k.t[2];
}

__device__ __forceinline__ float t_sqrt(float x) { return sqrtf(x); }
__device__ __forceinline__ double t_sqrt(double x) { return sqrt(x); }
__device__ __forceinline__ float t_exp(float x) { return expf(x); }
__device__ __forceinline__ double t_exp(double x) { return exp(x); }

// The mask words and group slot base of up to 64 cameras for one 128-pair
// mask group, loaded at once: lane j holds camera c0 + j's two words (the
// group's two waves) and the first slot of its group (zeros past C). A
// camera loop then takes them with readlanes instead of one dependent
// memory round trip per camera.
struct CamWords {
  uint64_t w0, w1;
  uint32_t base;
};

__device__ __forceinline__ CamWords load_cam_words(const uint64_t* __restrict__ mask,
                                                   const uint32_t* __restrict__ wg_scan,
                                                   int64_t N_pad, int64_t grp, int c0, int C) {
  CamWords cw{0, 0, 0};
  const int c = c0 + int(__lane_id());
  if (c < C) {
    const int64_t p0 = int64_t(c) * N_pad + grp * kMaskGroup;
    cw.w0 = mask[p0 / 64];
    cw.w1 = mask[p0 / 64 + 1];
    cw.base = wg_scan[p0 / kMaskGroup];
  }
  return cw;
}

// Camera c0 + j's words from a CamWords (j wave-uniform).
__device__ __forceinline__ uint64_t cam_w0(const CamWords& cw, int j) { return readlane_u64(cw.w0, j); }
__device__ __forceinline__ uint64_t cam_w1(const CamWords& cw, int j) { return readlane_u64(cw.w1, j); }
__device__ __forceinline__ uint32_t cam_base(const CamWords& cw, int j) {
  return uint32_t(__builtin_amdgcn_readlane(int(cw.base), j));
}

// Rotation matrix of the unit quaternion (w, x, y, z), row-major.
template <typename T>
__device__ __forceinline__ void quat_rotmat(T w, T x, T y, T z, T* R) {
  R[0] = T(1) - T(2) * (y * y + z * z);
  R[1] = T(2) * (x * y - w * z);
  R[2] = T(2) * (x * z + w * y);
  R[3] = T(2) * (x * y + w * z);
  R[4] = T(1) - T(2) * (x * x + z * z);
  R[5] = T(2) * (y * z - w * x);
  R[6] = T(2) * (x * z - w * y);
  R[7] = T(2) * (y * z + w * x);
  R[8] = T(1) - T(2) * (x * x + y * y);
}

// Quantities of one Gaussian that do not depend on the camera.
template <typename T>
struct GaussLocal {
  float mu[3];   // the stored position (fp32 input)
  T qn;          // |q|
  T qh[4];       // q / |q|
  T Rq[9];
  T s[3];        // exp(log_scale)
  T M[9];        // Rq diag(s)
};

template <typename T>
__device__ __forceinline__ void gauss_local(const float* __restrict__ means,
                                            const float* __restrict__ quats,
                                            const float* __restrict__ log_scales, int64_t g,
                                            GaussLocal<T>& G) {
  G.mu[0] = means[3 * g + 0];
  G.mu[1] = means[3 * g + 1];
  G.mu[2] = means[3 * g + 2];
  const float4 q = reinterpret_cast<const float4*>(quats)[g];
  const T qw = q.x, qx = q.y, qy = q.z, qz = q.w;
  G.qn = t_sqrt(qw * qw + qx * qx + qy * qy + qz * qz);
  const T inv = T(1) / G.qn;
  G.qh[0] = qw * inv;
  G.qh[1] = qx * inv;
  G.qh[2] = qy * inv;
  G.qh[3] = qz * inv;
  quat_rotmat<T>(G.qh[0], G.qh[1], G.qh[2], G.qh[3], G.Rq);
#pragma unroll
  for (int j = 0; j < 3; ++j) G.s[j] = t_exp(T(log_scales[3 * g + j]));
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) G.M[3 * i + j] = G.Rq[3 * i + j] * G.s[j];
}

// Screen-space quantities of one (camera, Gaussian) pair.
template <typename T>
struct PairFwd {
  T x, y, z;        // camera-space point
  float z32;        // the fp32 key depth (near test and sort key)
  T Wm[9];          // R_cam M
  T TM[6];          // J W, two rows
  T S00, S01, S11;  // 2D covariance incl. blur
  T det;
  T ca, cb, cc;     // conic = inverse 2D covariance
  T u, v, r;
  bool visible;
  T x0, x1, y0, y1;  // box clamped to the image
};

template <typename T>
__device__ __forceinline__ void pair_fwd(const Camera& k, const GaussLocal<T>& G, T Wimg,
                                         T Himg, PairFwd<T>& P) {
  const T mx = G.mu[0], my = G.mu[1], mz = G.mu[2];
  P.x = fma(T(k.R[0]), mx, fma(T(k.R[1]), my, fma(T(k.R[2]), mz, T(k.t[0]))));
  P.y = fma(T(k.R[3]), mx, fma(T(k.R[4]), my, fma(T(k.R[5]), mz, T(k.t[1]))));
  P.z = fma(T(k.R[6]), mx, fma(T(k.R[7]), my, fma(T(k.R[8]), mz, T(k.t[2]))));
  P.z32 = depth_z32(k, G.mu[0], G.mu[1], G.mu[2]);
  const T iz = T(1) / P.z;
  P.u = fma(T(k.fx), P.x * iz, T(k.cx));
  P.v = fma(T(k.fy), P.y * iz, T(k.cy));
  // W = R_cam M
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      P.Wm[3 * i + j] = T(k.R[3 * i + 0]) * G.M[0 + j] + T(k.R[3 * i + 1]) * G.M[3 + j] +
                        T(k.R[3 * i + 2]) * G.M[6 + j];
  const T j00 = T(k.fx) * iz, j02 = -T(k.fx) * P.x * iz * iz;
  const T j11 = T(k.fy) * iz, j12 = -T(k.fy) * P.y * iz * iz;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    P.TM[j] = j00 * P.Wm[j] + j02 * P.Wm[6 + j];
    P.TM[3 + j] = j11 * P.Wm[3 + j] + j12 * P.Wm[6 + j];
  }
  P.S00 = P.TM[0] * P.TM[0] + P.TM[1] * P.TM[1] + P.TM[2] * P.TM[2] + T(kBlur);
  P.S01 = P.TM[0] * P.TM[3] + P.TM[1] * P.TM[4] + P.TM[2] * P.TM[5];
  P.S11 = P.TM[3] * P.TM[3] + P.TM[4] * P.TM[4] + P.TM[5] * P.TM[5] + T(kBlur);
  P.det = P.S00 * P.S11 - P.S01 * P.S01;
  const T idet = T(1) / P.det;
  P.ca = P.S11 * idet;
  P.cb = -P.S01 * idet;
  P.cc = P.S00 * idet;
  const T mid = T(0.5) * (P.S00 + P.S11);
  const T lam = mid + t_sqrt(fmax(T(0), mid * mid - P.det));
  P.r = T(3) * t_sqrt(lam);
  P.x0 = fmax(P.u - P.r, T(0));
  P.x1 = fmin(P.u + P.r, Wimg);
  P.y0 = fmax(P.v - P.r, T(0));
  P.y1 = fmin(P.v + P.r, Himg);
  P.visible = (P.z32 > kNear) && (P.x1 > P.x0) && (P.y1 > P.y0);
}

// Real SH basis up to degree DEG at unit direction (x, y, z), in the
// polynomial form N_{l|m|} (-1)^|m| P_l^{(|m|)}(z) {Re,Im}((x+iy)^|m|),
// where P_l^{(m)} is the m-th derivative of the Legendre polynomial.
template <int DEG, typename T>
__device__ __forceinline__ void sh_basis(const ShNorm& N, T x, T y, T z, T* Y) {
  Y[0] = T(N.n[0]);
  if constexpr (DEG >= 1) {
    Y[1] = -T(N.n[2]) * y;
    Y[2] = T(N.n[1]) * z;
    Y[3] = -T(N.n[2]) * x;
  }
  if constexpr (DEG >= 2) {
    const T xx = x * x, yy = y * y, zz = z * z;
    Y[4] = T(N.n[5]) * 6.f * x * y;
    Y[5] = -T(N.n[4]) * 3.f * y * z;
    Y[6] = T(N.n[3]) * (T(1.5) * zz - T(0.5));
    Y[7] = -T(N.n[4]) * 3.f * x * z;
    Y[8] = T(N.n[5]) * 3.f * (xx - yy);
    if constexpr (DEG >= 3) {
      const T f = T(7.5) * zz - T(1.5);  // P_3'(z)
      Y[9] = -T(N.n[9]) * 15.f * (3.f * xx * y - yy * y);
      Y[10] = T(N.n[8]) * 30.f * x * y * z;
      Y[11] = -T(N.n[7]) * f * y;
      Y[12] = T(N.n[6]) * (T(2.5) * zz * z - T(1.5) * z);
      Y[13] = -T(N.n[7]) * f * x;
      Y[14] = T(N.n[8]) * 15.f * z * (xx - yy);
      Y[15] = -T(N.n[9]) * 15.f * (xx * x - 3.f * x * yy);
    }
  }
}

// d/d(x,y,z) of the same polynomials (not yet projected on the sphere).
// Adds sum_k w[k] * grad Y_k into g.
template <int DEG, typename T>
__device__ __forceinline__ void sh_basis_vjp(const ShNorm& N, T x, T y, T z, const T* w, T* g) {
  if constexpr (DEG >= 1) {
    g[1] += -T(N.n[2]) * w[1];
    g[2] += T(N.n[1]) * w[2];
    g[0] += -T(N.n[2]) * w[3];
  }
  if constexpr (DEG >= 2) {
    const T a4 = T(N.n[5]) * 6.f * w[4];
    g[0] += a4 * y;
    g[1] += a4 * x;
    const T a5 = -T(N.n[4]) * 3.f * w[5];
    g[1] += a5 * z;
    g[2] += a5 * y;
    g[2] += T(N.n[3]) * 3.f * z * w[6];
    const T a7 = -T(N.n[4]) * 3.f * w[7];
    g[0] += a7 * z;
    g[2] += a7 * x;
    const T a8 = T(N.n[5]) * 6.f * w[8];
    g[0] += a8 * x;
    g[1] -= a8 * y;
    if constexpr (DEG >= 3) {
      const T xx = x * x, yy = y * y, zz = z * z;
      const T a9 = -T(N.n[9]) * 15.f * w[9];
      g[0] += a9 * 6.f * x * y;
      g[1] += a9 * 3.f * (xx - yy);
      const T a10 = T(N.n[8]) * 30.f * w[10];
      g[0] += a10 * y * z;
      g[1] += a10 * x * z;
      g[2] += a10 * x * y;
      const T f = T(7.5) * zz - T(1.5), fp = 15.f * z;
      const T a11 = -T(N.n[7]) * w[11];
      g[1] += a11 * f;
      g[2] += a11 * fp * y;
      g[2] += T(N.n[6]) * (T(7.5) * zz - T(1.5)) * w[12];
      const T a13 = -T(N.n[7]) * w[13];
      g[0] += a13 * f;
      g[2] += a13 * fp * x;
      const T a14 = T(N.n[8]) * 15.f * w[14];
      g[0] += a14 * 2.f * x * z;
      g[1] -= a14 * 2.f * y * z;
      g[2] += a14 * (xx - yy);
      const T a15 = -T(N.n[9]) * 15.f * w[15];
      g[0] += a15 * 3.f * (xx - yy);
      g[1] -= a15 * 6.f * x * y;
    }
  }
}

}  // namespace gs
