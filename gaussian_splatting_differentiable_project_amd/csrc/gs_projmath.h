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
  float n[10];
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
// its evaluation order is part of the result.
__device__ __forceinline__ float depth_z32(const Camera& k, float mx, float my, float mz) {
  float z = __fmul_rn(k.R[6], mx);
  z = __fadd_rn(z, __fmul_rn(k.R[7], my));
  z = __fadd_rn(z, __fmul_rn(k.R[8], mz));
  return __fadd_rn(z, k.t[2]);
}

// Rotation matrix of the unit quaternion (w, x, y, z), row-major.
__device__ __forceinline__ void quat_rotmat(float w, float x, float y, float z, float* R) {
  R[0] = 1.f - 2.f * (y * y + z * z);
  R[1] = 2.f * (x * y - w * z);
  R[2] = 2.f * (x * z + w * y);
  R[3] = 2.f * (x * y + w * z);
  R[4] = 1.f - 2.f * (x * x + z * z);
  R[5] = 2.f * (y * z - w * x);
  R[6] = 2.f * (x * z - w * y);
  R[7] = 2.f * (y * z + w * x);
  R[8] = 1.f - 2.f * (x * x + y * y);
}

// Quantities of one Gaussian that do not depend on the camera.
struct GaussLocal {
  float mu[3];
  float qn;      // |q|
  float qh[4];   // q / |q|
  float Rq[9];
  float s[3];    // exp(log_scale)
  float M[9];    // Rq diag(s)
};

__device__ __forceinline__ void gauss_local(const float* __restrict__ means,
                                            const float* __restrict__ quats,
                                            const float* __restrict__ log_scales, int64_t g,
                                            GaussLocal& G) {
  G.mu[0] = means[3 * g + 0];
  G.mu[1] = means[3 * g + 1];
  G.mu[2] = means[3 * g + 2];
  const float4 q = reinterpret_cast<const float4*>(quats)[g];
  G.qn = sqrtf(q.x * q.x + q.y * q.y + q.z * q.z + q.w * q.w);
  const float inv = 1.f / G.qn;
  G.qh[0] = q.x * inv;
  G.qh[1] = q.y * inv;
  G.qh[2] = q.z * inv;
  G.qh[3] = q.w * inv;
  quat_rotmat(G.qh[0], G.qh[1], G.qh[2], G.qh[3], G.Rq);
#pragma unroll
  for (int j = 0; j < 3; ++j) G.s[j] = expf(log_scales[3 * g + j]);
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) G.M[3 * i + j] = G.Rq[3 * i + j] * G.s[j];
}

// Screen-space quantities of one (camera, Gaussian) pair.
struct PairFwd {
  float x, y, z;    // camera-space point (z is the fp32 key depth)
  float Wm[9];      // R_cam M
  float TM[6];      // J W, two rows
  float S00, S01, S11;  // 2D covariance incl. blur
  float det;
  float ca, cb, cc;     // conic = inverse 2D covariance
  float u, v, r;
  bool visible;
  float x0, x1, y0, y1;  // box clamped to the image
};

__device__ __forceinline__ void pair_fwd(const Camera& k, const GaussLocal& G, float Wimg,
                                         float Himg, PairFwd& P) {
  const float mx = G.mu[0], my = G.mu[1], mz = G.mu[2];
  // The screen position is computed in fp64 and rounded once: the 40-byte
  // row stores it in fp32, and an fp32 evaluation of fx x / z + cx would
  // add several ulps at the image edges (about 5e-4 px at 1000 px).
  const double dmx = mx, dmy = my, dmz = mz;
  const double xd = fma(double(k.R[0]), dmx, fma(double(k.R[1]), dmy, fma(double(k.R[2]), dmz, double(k.t[0]))));
  const double yd = fma(double(k.R[3]), dmx, fma(double(k.R[4]), dmy, fma(double(k.R[5]), dmz, double(k.t[1]))));
  const double zd = fma(double(k.R[6]), dmx, fma(double(k.R[7]), dmy, fma(double(k.R[8]), dmz, double(k.t[2]))));
  const double izd = 1.0 / zd;
  P.u = float(fma(double(k.fx), xd * izd, double(k.cx)));
  P.v = float(fma(double(k.fy), yd * izd, double(k.cy)));
  P.x = float(xd);
  P.y = float(yd);
  P.z = depth_z32(k, mx, my, mz);
  const float z = P.z;
  const float iz = 1.f / z;
  // W = R_cam M
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      P.Wm[3 * i + j] = k.R[3 * i + 0] * G.M[0 + j] + k.R[3 * i + 1] * G.M[3 + j] +
                        k.R[3 * i + 2] * G.M[6 + j];
  const float j00 = k.fx * iz, j02 = -k.fx * P.x * iz * iz;
  const float j11 = k.fy * iz, j12 = -k.fy * P.y * iz * iz;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    P.TM[j] = j00 * P.Wm[j] + j02 * P.Wm[6 + j];
    P.TM[3 + j] = j11 * P.Wm[3 + j] + j12 * P.Wm[6 + j];
  }
  P.S00 = P.TM[0] * P.TM[0] + P.TM[1] * P.TM[1] + P.TM[2] * P.TM[2] + kBlur;
  P.S01 = P.TM[0] * P.TM[3] + P.TM[1] * P.TM[4] + P.TM[2] * P.TM[5];
  P.S11 = P.TM[3] * P.TM[3] + P.TM[4] * P.TM[4] + P.TM[5] * P.TM[5] + kBlur;
  P.det = P.S00 * P.S11 - P.S01 * P.S01;
  const float idet = 1.f / P.det;
  P.ca = P.S11 * idet;
  P.cb = -P.S01 * idet;
  P.cc = P.S00 * idet;
  const float mid = 0.5f * (P.S00 + P.S11);
  const float lam = mid + sqrtf(fmaxf(0.f, mid * mid - P.det));
  P.r = 3.f * sqrtf(lam);
  P.x0 = fmaxf(P.u - P.r, 0.f);
  P.x1 = fminf(P.u + P.r, Wimg);
  P.y0 = fmaxf(P.v - P.r, 0.f);
  P.y1 = fminf(P.v + P.r, Himg);
  P.visible = (z > kNear) && (P.x1 > P.x0) && (P.y1 > P.y0);
}

// Real SH basis up to degree DEG at unit direction (x, y, z), in the
// polynomial form N_{l|m|} (-1)^|m| P_l^{(|m|)}(z) {Re,Im}((x+iy)^|m|),
// where P_l^{(m)} is the m-th derivative of the Legendre polynomial.
template <int DEG>
__device__ __forceinline__ void sh_basis(const ShNorm& N, float x, float y, float z, float* Y) {
  Y[0] = N.n[0];
  if constexpr (DEG >= 1) {
    Y[1] = -N.n[2] * y;
    Y[2] = N.n[1] * z;
    Y[3] = -N.n[2] * x;
  }
  if constexpr (DEG >= 2) {
    const float xx = x * x, yy = y * y, zz = z * z;
    Y[4] = N.n[5] * 6.f * x * y;
    Y[5] = -N.n[4] * 3.f * y * z;
    Y[6] = N.n[3] * (1.5f * zz - 0.5f);
    Y[7] = -N.n[4] * 3.f * x * z;
    Y[8] = N.n[5] * 3.f * (xx - yy);
    if constexpr (DEG >= 3) {
      const float f = 7.5f * zz - 1.5f;  // P_3'(z)
      Y[9] = -N.n[9] * 15.f * (3.f * xx * y - yy * y);
      Y[10] = N.n[8] * 30.f * x * y * z;
      Y[11] = -N.n[7] * f * y;
      Y[12] = N.n[6] * (2.5f * zz * z - 1.5f * z);
      Y[13] = -N.n[7] * f * x;
      Y[14] = N.n[8] * 15.f * z * (xx - yy);
      Y[15] = -N.n[9] * 15.f * (xx * x - 3.f * x * yy);
    }
  }
}

// d/d(x,y,z) of the same polynomials (not yet projected on the sphere).
// Adds sum_k w[k] * grad Y_k into g.
template <int DEG>
__device__ __forceinline__ void sh_basis_vjp(const ShNorm& N, float x, float y, float z,
                                             const float* w, float* g) {
  if constexpr (DEG >= 1) {
    g[1] += -N.n[2] * w[1];
    g[2] += N.n[1] * w[2];
    g[0] += -N.n[2] * w[3];
  }
  if constexpr (DEG >= 2) {
    const float a4 = N.n[5] * 6.f * w[4];
    g[0] += a4 * y;
    g[1] += a4 * x;
    const float a5 = -N.n[4] * 3.f * w[5];
    g[1] += a5 * z;
    g[2] += a5 * y;
    g[2] += N.n[3] * 3.f * z * w[6];
    const float a7 = -N.n[4] * 3.f * w[7];
    g[0] += a7 * z;
    g[2] += a7 * x;
    const float a8 = N.n[5] * 6.f * w[8];
    g[0] += a8 * x;
    g[1] -= a8 * y;
    if constexpr (DEG >= 3) {
      const float xx = x * x, yy = y * y, zz = z * z;
      const float a9 = -N.n[9] * 15.f * w[9];
      g[0] += a9 * 6.f * x * y;
      g[1] += a9 * 3.f * (xx - yy);
      const float a10 = N.n[8] * 30.f * w[10];
      g[0] += a10 * y * z;
      g[1] += a10 * x * z;
      g[2] += a10 * x * y;
      const float f = 7.5f * zz - 1.5f, fp = 15.f * z;
      const float a11 = -N.n[7] * w[11];
      g[1] += a11 * f;
      g[2] += a11 * fp * y;
      g[2] += N.n[6] * (7.5f * zz - 1.5f) * w[12];
      const float a13 = -N.n[7] * w[13];
      g[0] += a13 * f;
      g[2] += a13 * fp * x;
      const float a14 = N.n[8] * 15.f * w[14];
      g[0] += a14 * 2.f * x * z;
      g[1] -= a14 * 2.f * y * z;
      g[2] += a14 * (xx - yy);
      const float a15 = -N.n[9] * 15.f * w[15];
      g[0] += a15 * 3.f * (xx - yy);
      g[1] -= a15 * 6.f * x * y;
    }
  }
}

}  // namespace gs
