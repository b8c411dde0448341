// Packed projection: visibility bitmask pass and compaction pass.
//
// [VRAM] "Bitmask compaction": the first pass projects every (camera,
// Gaussian) pair and ORs the visibility predicate into work-group bit
// words, writing one popcount per work-group; a scan over the C*N/128
// counts follows; the second pass re-projects only the survivors and
// recovers each one's exact output slot as (scanned count of earlier
// work-groups) + (set bits before this lane).
//
// gfx950 mapping: a 128-lane work-group is two wave64s; each wave's
// ballot *is* one 64-bit mask word, so the bit words need no shared
// memory at all. Threads are Gaussian-major (lane = Gaussian, loop over
// cameras), so the parameters are read once per Gaussian, not C times.
#include <cmath>

#include "gs_internal.h"

namespace gs {

namespace {

template <typename T>
__device__ __forceinline__ void zero_local(GaussLocal<T>& G) {
#pragma unroll
  for (int i = 0; i < 3; ++i) G.mu[i] = 0.f, G.s[i] = T(1);
  G.qn = T(1);
  G.qh[0] = T(1), G.qh[1] = G.qh[2] = G.qh[3] = T(0);
#pragma unroll
  for (int i = 0; i < 9; ++i) G.Rq[i] = G.M[i] = (i % 4 == 0) ? T(1) : T(0);
}

// Visibility of one pair: the depth test on the fp32 key depth (exact by
// definition) and the four margins of the clamped box, u + r > 0,
// u - r < W, v + r > 0, v - r < H. They are first evaluated in fp32; a
// margin within a bound of zero leaves the pair "unsure", and only then is
// it evaluated again in fp64 as the compaction pass evaluates it. The
// bound has two parts: 4e-5 of the coordinate scale (1 + |u| + |u - cx|),
// against a measured fp32 error of the centre below 1.2e-6 of it, and
// 6e-4 of r, against the radius' worst case: sqrt(m^2 - det) cancels for
// nearly isotropic covariances, leaving a relative error of about
// 2^-12 in lambda_max and 1.7e-4 in r.
__device__ __forceinline__ bool visible_fp32(const PairFwd<float>& P, float cx, float cy,
                                             float W, float H, bool* unsure) {
  *unsure = false;
  if (!(P.z32 > kNear)) return false;
  const float tx = 4e-5f * (1.f + fabsf(P.u) + fabsf(P.u - cx)) + 6e-4f * P.r;
  const float ty = 4e-5f * (1.f + fabsf(P.v) + fabsf(P.v - cy)) + 6e-4f * P.r;
  const float m0 = P.u + P.r, m1 = W - (P.u - P.r), m2 = P.v + P.r, m3 = H - (P.v - P.r);
  if (!(fabsf(m0) < 3e38f && fabsf(m1) < 3e38f && fabsf(m2) < 3e38f && fabsf(m3) < 3e38f &&
        tx < 3e38f && ty < 3e38f)) {
    *unsure = true;
    return false;
  }
  if (m0 < -tx || m1 < -tx || m2 < -ty || m3 < -ty) return false;
  if (m0 > tx && m1 > tx && m2 > ty && m3 > ty) return true;
  *unsure = true;
  return false;
}

__global__ __launch_bounds__(kMaskGroup) void k_project_mask(ProjectArgs a, uint64_t* mask) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t g = int64_t(blockIdx.x) * kMaskGroup + tid;
  const bool valid = g < a.N;
  // The decision is the fp64 projection's (the compaction pass computes
  // the rows in fp64 and the two must agree); fp32 settles every pair not
  // close to an edge of the decision, and fp64 runs only for the others.
  GaussLocal<float> Gf;
  if (valid)
    gauss_local(a.means, a.quats, a.log_scales, g, Gf);
  else
    zero_local(Gf);
  GaussLocal<double> G;
  bool have_g64 = false;
  const float Wf = float(a.W), Hf = float(a.H);
  Camera kn = load_camera(a.viewmats, a.Ks, 0);
  for (int c = 0; c < a.C; ++c) {
    const Camera k = kn;
    // the next camera's parameters load while this one is projected
    if (c + 1 < a.C) kn = load_camera(a.viewmats, a.Ks, c + 1);
    PairFwd<float> Pf;
    pair_fwd(k, Gf, Wf, Hf, Pf);
    bool unsure;
    bool vis = visible_fp32(Pf, float(k.cx), float(k.cy), Wf, Hf, &unsure);
    unsure = unsure && valid;
    if (__ballot(unsure)) {
      if (unsure) {
        if (!have_g64) {
          gauss_local(a.means, a.quats, a.log_scales, g, G);
          have_g64 = true;
        }
        PairFwd<double> P;
        pair_fwd(k, G, double(a.W), double(a.H), P);
        vis = P.visible;
      }
    }
    const uint64_t word = __ballot(valid && vis);
    const int64_t p0 = int64_t(c) * a.N_pad + int64_t(blockIdx.x) * kMaskGroup;
    if (lane == 0) mask[p0 / 64 + wave] = word;
  }
}

// Mask pass for 2 to kMaskFastCams cameras. A bound test settles most
// pairs in fp32 from the Gaussian's position and largest scale alone;
// only the others run the full projection of k_project_mask, queued per
// block so that every lane of a pass has a pair. (With one camera there is
// nothing to share the Gaussian's loads across, and the camera-walking
// kernel is faster.)
//
// The bounds are those of the fp64 projection, for any input:
//  - each fp64 camera-space coordinate lies within e = 2^-21 (max|R|
//    (|mx| + |my| + |mz|) + max|t|) of its fp32 value (three fused
//    roundings, each at most 2^-24 of that sum);
//  - for z > e the fp64 ratio x / z lies within da = e (z + |x|) /
//    (z (z - e)) of the fp32 one (plus that ratio's own rounding), so the
//    fp64 centre lies within tu = |fx| da (plus rounding margins) of the
//    fp32 centre u;
//  - the radius is 3 sqrt(lambda_max) and lambda_max is at most the trace
//    of the 2D covariance, |J R_cam M|_F^2 + 2 blur, with |J R_cam M|_F at
//    most |J R_cam|_F max(s); the rows of J R_cam are (f / z) (R_i - (x /
//    z) R_2), bounded through the row norms with |x / z| <= |x / z| + da
//    and 1 / z <= 1 / (z - e).
// A pair past the near test is visible in fp64 when its centre is inside
// the image: the radius is then positive, and a radius that is not finite
// also leaves the clamped box non-empty. It is invisible when the centre
// lies farther outside than the bounded radius, which is taken only when
// the fp64 radius is sure to be finite: a finite, non-zero squared
// quaternion norm and finite scales in fp32 (no log scale NaN). The
// largest scale is exp of the largest log scale (exp is monotonic; the
// fp32 value is within 2 ulp). All other pairs are queued.
constexpr int kMaskFastCams = 64;
constexpr int kMaskCam = 24;  // floats per staged camera: R, t, fx, fy, cx, cy, 2^-21 max|R|,
                              // 2^-21 max|t|, row norms of R, fx^2, fy^2, pad

size_t mask_fast_lds(int C) {
  return size_t(C) * (2 * sizeof(uint64_t) + kMaskCam * sizeof(float) +
                      kMaskGroup * sizeof(uint16_t));
}

__device__ __forceinline__ Camera mask_camera(const float* sc) {
  Camera k;
#pragma unroll
  for (int i = 0; i < 9; ++i) k.R[i] = sc[i];
#pragma unroll
  for (int i = 0; i < 3; ++i) k.t[i] = sc[9 + i];
  k.fx = sc[12], k.fy = sc[13], k.cx = sc[14], k.cy = sc[15];
  k.cc[0] = k.cc[1] = k.cc[2] = 0.f;  // not read by the projection
  return k;
}

__global__ __launch_bounds__(kMaskGroup) void k_project_mask_fast(ProjectArgs a, uint64_t* mask) {
  extern __shared__ __align__(16) uint64_t s_mdyn[];
  const int C = a.C;
  uint64_t* s_vis = s_mdyn;                                           // [C][2] mask words
  float* s_cam = reinterpret_cast<float*>(s_mdyn + 2 * C);            // [C][kMaskCam]
  uint16_t* s_q = reinterpret_cast<uint16_t*>(s_cam + kMaskCam * C);  // queued camera << 7 | lane
  __shared__ uint32_t s_qn;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t g = int64_t(blockIdx.x) * kMaskGroup + tid;
  const bool valid = g < a.N;
  if (tid < C) {
    const Camera k = load_camera(a.viewmats, a.Ks, tid);
    float* sc = s_cam + tid * kMaskCam;
    float rm = 0.f, tm = 0.f;
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      sc[i] = k.R[i];
      rm = fmaxf(rm, fabsf(k.R[i]));
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      sc[9 + i] = k.t[i];
      tm = fmaxf(tm, fabsf(k.t[i]));
      sc[18 + i] = sqrtf(k.R[3 * i] * k.R[3 * i] + k.R[3 * i + 1] * k.R[3 * i + 1] +
                         k.R[3 * i + 2] * k.R[3 * i + 2]) * (1.f + 1e-6f);
    }
    sc[12] = k.fx, sc[13] = k.fy, sc[14] = k.cx, sc[15] = k.cy;
    sc[16] = 0x1p-21f * rm;
    sc[17] = 0x1p-21f * tm;
    sc[21] = k.fx * k.fx, sc[22] = k.fy * k.fy, sc[23] = 0.f;
  }
  if (tid == 0) s_qn = 0;
  float mx = 0.f, my = 0.f, mz = 0.f, smax2 = 0.f;
  bool finite_r = false;
  if (valid) {
    mx = a.means[3 * g + 0], my = a.means[3 * g + 1], mz = a.means[3 * g + 2];
    const float4 q = reinterpret_cast<const float4*>(a.quats)[g];
    const float l0 = a.log_scales[3 * g + 0], l1 = a.log_scales[3 * g + 1],
                l2 = a.log_scales[3 * g + 2];
    const float smax = expf(fmaxf(fmaxf(l0, l1), l2));
    smax2 = smax * smax;
    const float qn2 = q.x * q.x + q.y * q.y + q.z * q.z + q.w * q.w;
    const float lsum = l0 + l1 + l2;
    finite_r = qn2 > 0.f && qn2 < 3e38f && smax2 < 3e38f && lsum == lsum;
  }
  const float m1 = fabsf(mx) + fabsf(my) + fabsf(mz);
  const float Wf = float(a.W), Hf = float(a.H);
  const uint64_t lt = lanemask_lt();
  __syncthreads();

  for (int c = 0; c < C; ++c) {
    const float* sc = s_cam + c * kMaskCam;
    const Camera k = mask_camera(sc);
    const float ra = sc[16], ta = sc[17], n0 = sc[18], n1 = sc[19], n2 = sc[20];
    const float fx2 = sc[21], fy2 = sc[22];
    const float z32 = depth_z32(k, mx, my, mz);
    bool sure_vis = false, need = false;
    if (valid && z32 > kNear) {
      const float x = fmaf(k.R[0], mx, fmaf(k.R[1], my, fmaf(k.R[2], mz, k.t[0])));
      const float y = fmaf(k.R[3], mx, fmaf(k.R[4], my, fmaf(k.R[5], mz, k.t[1])));
      const float z = fmaf(k.R[6], mx, fmaf(k.R[7], my, fmaf(k.R[8], mz, k.t[2])));
      const float e = fmaf(ra, m1, ta);
      const float zl = z - e;
      bool sure_inv = false;
      if (zl > 0.f) {
        const float iz = __builtin_amdgcn_rcpf(z), izl = __builtin_amdgcn_rcpf(zl);
        const float q = e * iz * izl;
        const float ax = x * iz, ay = y * iz;
        const float dax = fmaf(q, z + fabsf(x), 2.5e-7f * fabsf(ax)) * 1.01f;
        const float day = fmaf(q, z + fabsf(y), 2.5e-7f * fabsf(ay)) * 1.01f;
        const float u = fmaf(k.fx, ax, k.cx), v = fmaf(k.fy, ay, k.cy);
        const float tu = fmaf(fabsf(k.fx), dax, 1e-6f * (fabsf(u) + fabsf(k.cx) + 1.f));
        const float tv = fmaf(fabsf(k.fy), day, 1e-6f * (fabsf(v) + fabsf(k.cy) + 1.f));
        sure_vis = u - tu > 0.f && u + tu < Wf && v - tv > 0.f && v + tv < Hf;
        const float r0 = fmaf(fabsf(ax) + dax, n2, n0), r1 = fmaf(fabsf(ay) + day, n2, n1);
        const float j2 = (fx2 * r0 * r0 + fy2 * r1 * r1) * (izl * izl);
        const float rup = 3.f * __builtin_amdgcn_sqrtf(fmaf(j2, smax2, 0.6f) * 1.01f);
        sure_inv = finite_r && (u + tu + rup < 0.f || u - tu - rup > Wf || v + tv + rup < 0.f ||
                                v - tv - rup > Hf);
      }
      need = !(sure_vis || sure_inv);
    }
    const uint64_t nb = __ballot(need);
    if (nb) {  // wave-uniform
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&s_qn, uint32_t(__popcll(nb)));
      base = __builtin_amdgcn_readfirstlane(base);
      if (need) s_q[base + uint32_t(__popcll(nb & lt))] = uint16_t((c << 7) | tid);
    }
    const uint64_t word = __ballot(sure_vis);
    if (lane == 0) s_vis[2 * c + wave] = word;
  }
  __syncthreads();

  // the queued pairs, one per lane: the camera-walking kernel's test
  const uint32_t qn = s_qn;
  for (uint32_t i = uint32_t(tid); i < qn; i += kMaskGroup) {
    const uint32_t it = s_q[i];
    const int c = int(it >> 7), t = int(it & 127u);
    const int64_t gt = int64_t(blockIdx.x) * kMaskGroup + t;
    GaussLocal<float> G1;
    gauss_local(a.means, a.quats, a.log_scales, gt, G1);
    const Camera k = mask_camera(s_cam + c * kMaskCam);
    PairFwd<float> Pf;
    pair_fwd(k, G1, Wf, Hf, Pf);
    bool unsure;
    bool vis = visible_fp32(Pf, k.cx, k.cy, Wf, Hf, &unsure);
    if (unsure) {
      GaussLocal<double> G;
      gauss_local(a.means, a.quats, a.log_scales, gt, G);
      PairFwd<double> P;
      pair_fwd(k, G, double(a.W), double(a.H), P);
      vis = P.visible;
    }
    if (vis)
      atomicOr(reinterpret_cast<unsigned long long*>(&s_vis[2 * c + (t >> 6)]),
               1ull << (t & 63));
  }
  __syncthreads();
  for (int i = tid; i < 2 * C; i += kMaskGroup) {
    const int64_t p0 = int64_t(i >> 1) * a.N_pad + int64_t(blockIdx.x) * kMaskGroup;
    mask[p0 / 64 + (i & 1)] = s_vis[i];
  }
}

// One visible pair: its fp32 screen row and 16-bit box at slot `slot`.
// fp64 arithmetic, rounded once into the fp32 row (see the mask pass).
// G carries the Gaussian's position and M = Rq diag(s), the only parts
// the pair's projection reads.
template <int DEG>
__device__ __forceinline__ void compact_pair(const ProjectArgs& a, const GaussLocal<double>& G,
                                             float opac, const float* shg, const Camera& k,
                                             int64_t slot, float* __restrict__ screen,
                                             uint32_t* __restrict__ aabb16) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  PairFwd<double> P;
  pair_fwd(k, G, double(a.W), double(a.H), P);
  // colour toward the camera centre
  double dx = double(G.mu[0]) - k.cc[0], dy = double(G.mu[1]) - k.cc[1],
         dz = double(G.mu[2]) - k.cc[2];
  const double inv = 1.0 / sqrt(dx * dx + dy * dy + dz * dz);
  dx *= inv, dy *= inv, dz *= inv;
  double Y[K];
  sh_basis<DEG>(a.norm, dx, dy, dz, Y);
  float rgb[3];
#pragma unroll
  for (int ch = 0; ch < 3; ++ch) {
    double acc = 0.5;
#pragma unroll
    for (int kk = 0; kk < K; ++kk) acc = fma(Y[kk], double(shg[3 * kk + ch]), acc);
    rgb[ch] = float(fmax(acc, 0.0));
  }
  float2* row = reinterpret_cast<float2*>(screen + slot * kRow);
  row[0] = make_float2(float(P.u), float(P.v));
  row[1] = make_float2(float(P.ca), float(P.cb));
  row[2] = make_float2(float(P.cc), opac);
  row[3] = make_float2(P.z32, rgb[0]);
  row[4] = make_float2(rgb[1], rgb[2]);
  // 16-bit box: min edges round down, max edges round up, on the grid
  // of 65535 steps over [0, extent]; the edge is taken in fp32 and scaled
  // in fp32 (a float deciding an integer code: one fixed precision).
  const float fx0 = fminf(fmaxf(floorf(float(P.x0) * a.qsx), 0.f), 65535.f);
  const float fy0 = fminf(fmaxf(floorf(float(P.y0) * a.qsy), 0.f), 65535.f);
  const float fx1 = fminf(fmaxf(ceilf(float(P.x1) * a.qsx), 0.f), 65535.f);
  const float fy1 = fminf(fmaxf(ceilf(float(P.y1) * a.qsy), 0.f), 65535.f);
  uint2 box;
  box.x = uint32_t(fx0) | (uint32_t(fy0) << 16);
  box.y = uint32_t(fx1) | (uint32_t(fy1) << 16);
  reinterpret_cast<uint2*>(aabb16)[slot] = box;
}

// The dense compaction of the wave slot w (Gaussians 64 w .. 64 w + 63,
// half w & 1 of mask group w >> 1): each lane walks the cameras for its
// own Gaussian, the camera uniform across the wave, its SH coefficients
// read once into registers. Every lane of the wave calls it, and every
// lane stays through the camera walk: lane j loads camera c0 + j's mask
// words, which the others read.
template <int DEG>
__device__ __forceinline__ void compact_dense_wave(const ProjectArgs& a,
                                                   const uint64_t* __restrict__ mask,
                                                   const uint32_t* __restrict__ wg_scan,
                                                   float* __restrict__ screen,
                                                   uint32_t* __restrict__ aabb16, int64_t w) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  const int lane = int(__lane_id());
  const int half = int(w & 1);
  const int64_t grp = w >> 1;
  const int64_t gw = w * kWave;
  const uint64_t lt = lanemask_lt();
  CamWords cw = load_cam_words(mask, wg_scan, a.N_pad, grp, 0, a.C);
  bool any = false;
  for (int c = 0; c < a.C; ++c) {
    if ((c & 63) == 0 && c > 0) cw = load_cam_words(mask, wg_scan, a.N_pad, grp, c, a.C);
    const uint64_t mine = half ? cam_w1(cw, c & 63) : cam_w0(cw, c & 63);
    any |= ((mine >> lane) & 1ull) != 0;
  }
  if (__ballot(any) == 0ull) return;  // the whole wave
  GaussLocal<double> G;
  float opac = 0.f;
  float shc[K * 3];
#pragma unroll
  for (int i = 0; i < K * 3; ++i) shc[i] = 0.f;
  if (any) {
    gauss_local(a.means, a.quats, a.log_scales, gw + lane, G);
    opac = float(1.0 / (1.0 + exp(-double(a.opacity_logits[gw + lane]))));
    const float* shg = a.sh + (gw + lane) * (K * 3);
#pragma unroll
    for (int i = 0; i < K * 3; ++i) shc[i] = shg[i];
  }
  if (a.C > 64) cw = load_cam_words(mask, wg_scan, a.N_pad, grp, 0, a.C);
  for (int c = 0; c < a.C; ++c) {
    if ((c & 63) == 0 && c > 0) cw = load_cam_words(mask, wg_scan, a.N_pad, grp, c, a.C);
    const uint64_t w0 = cam_w0(cw, c & 63), w1 = cam_w1(cw, c & 63);
    const uint64_t mine = half ? w1 : w0;
    if (!((mine >> lane) & 1ull)) continue;
    const int64_t slot = int64_t(cam_base(cw, c & 63)) + (half ? __popcll(w0) : 0) +
                         __popcll(mine & lt);
    if (slot < a.cap)
      compact_pair<DEG>(a, G, opac, shc, load_camera(a.viewmats, a.Ks, c), slot, screen, aabb16);
  }
}

// Compaction, one wave per 64 Gaussians (half a mask group), in one of
// two ways chosen per wave:
//  - dense (the wave's visible pairs are at least half of 64 per camera):
//    compact_dense_wave;
//  - sparse (many cameras, each seeing a small part of the scene): such a
//    walk would run every camera's fp64 projection with only the visible
//    lanes active -- about one in five in a five-camera scene -- so the
//    wave instead gathers its visible pairs camera by camera into an LDS
//    queue, in slot order, and computes them 64 at a time, one pair per
//    lane; the camera-independent part of each Gaussian is computed once
//    by its own lane and shared through LDS.
// A pair past the caller's capacity is counted by the scan, not written.
template <int DEG>
__global__ __launch_bounds__(kWave) void k_project_compact(ProjectArgs a,
                                                           const uint64_t* __restrict__ mask,
                                                           const uint32_t* __restrict__ wg_scan,
                                                           float* __restrict__ screen,
                                                           uint32_t* __restrict__ aabb16) {
  __shared__ uint32_t s_cl[2 * kWave];  // camera << 6 | lane of the Gaussian
  __shared__ int64_t s_slot[2 * kWave];
  __shared__ double s_M[9][kWave];
  __shared__ float s_mu[3][kWave];
  __shared__ float s_op[kWave];
  constexpr int K = (DEG + 1) * (DEG + 1);
  const int lane = threadIdx.x;
  const int half = int(blockIdx.x & 1);
  const int64_t grp = int64_t(blockIdx.x >> 1);
  const int64_t gw = int64_t(blockIdx.x) * kWave;  // this wave's first Gaussian
  const uint64_t lt = lanemask_lt();
  // Which cameras see this lane's Gaussian (mask words are wave-uniform
  // loads; the bits of padding lanes are clear).
  // Cameras are taken 64 at a time: lane j loads camera c0 + j's words.
  bool any = false;
  int npairs = 0;  // the wave's visible pairs (wave-uniform)
  CamWords cw{};
  for (int c = 0; c < a.C; ++c) {
    if ((c & 63) == 0) cw = load_cam_words(mask, wg_scan, a.N_pad, grp, c, a.C);
    const uint64_t mine = half ? cam_w1(cw, c & 63) : cam_w0(cw, c & 63);
    any |= ((mine >> lane) & 1ull) != 0;
    npairs += __popcll(mine);
  }
  if (npairs == 0) return;
  if (2 * npairs >= a.C * kWave) {
    compact_dense_wave<DEG>(a, mask, wg_scan, screen, aabb16, int64_t(blockIdx.x));
    return;
  }
  GaussLocal<double> G;
  float opac = 0.f;
  if (any) {
    gauss_local(a.means, a.quats, a.log_scales, gw + lane, G);
    opac = float(1.0 / (1.0 + exp(-double(a.opacity_logits[gw + lane]))));
  }
  if (any) {
#pragma unroll
    for (int i = 0; i < 9; ++i) s_M[i][lane] = G.M[i];
#pragma unroll
    for (int i = 0; i < 3; ++i) s_mu[i][lane] = G.mu[i];
    s_op[lane] = opac;
  }
  auto run = [&](uint32_t cl, int64_t slot) {
    if (slot >= a.cap) return;
    const int src = int(cl & 63u);
    GaussLocal<double> Gs;
#pragma unroll
    for (int i = 0; i < 9; ++i) Gs.M[i] = s_M[i][src];
#pragma unroll
    for (int i = 0; i < 3; ++i) Gs.mu[i] = s_mu[i][src];
    compact_pair<DEG>(a, Gs, s_op[src], a.sh + (gw + src) * (K * 3),
                      load_camera(a.viewmats, a.Ks, int(cl >> 6)), slot, screen, aabb16);
  };
  int qn = 0;  // queued pairs (wave-uniform)
  // the count above left the last 64-camera block loaded
  if (a.C > 64) cw = load_cam_words(mask, wg_scan, a.N_pad, grp, 0, a.C);
  for (int c = 0; c < a.C; ++c) {
    if ((c & 63) == 0 && c > 0) cw = load_cam_words(mask, wg_scan, a.N_pad, grp, c, a.C);
    const uint64_t w0 = cam_w0(cw, c & 63), w1 = cam_w1(cw, c & 63);
    const uint64_t mine = half ? w1 : w0;
    if (mine == 0) continue;
    const int64_t base = int64_t(cam_base(cw, c & 63)) + (half ? __popcll(w0) : 0);
    if ((mine >> lane) & 1ull) {
      const int r = __popcll(mine & lt);
      s_cl[qn + r] = (uint32_t(c) << 6) | uint32_t(lane);
      s_slot[qn + r] = base + r;
    }
    qn += __popcll(mine);
    if (qn >= kWave) {
      __syncthreads();
      const uint32_t cl = s_cl[lane];
      const int64_t slot = s_slot[lane];
      // move the entries past the first 64 to the front
      const bool mv = lane < qn - kWave;
      uint32_t t_cl = 0;
      int64_t t_slot = 0;
      if (mv) {
        t_cl = s_cl[kWave + lane];
        t_slot = s_slot[kWave + lane];
      }
      __syncthreads();
      if (mv) {
        s_cl[lane] = t_cl;
        s_slot[lane] = t_slot;
      }
      qn -= kWave;
      run(cl, slot);
    }
  }
  __syncthreads();
  if (lane < qn) run(s_cl[lane], s_slot[lane]);
}

// The dense wave slots for 2 to kCpMaxCams cameras (the sparse ones are
// k_project_compact_pairs'). A wave checks kDenseSpan slots at once, lane
// j slot kDenseSpan b + j: its visible pairs are the popcounts of its mask
// words over the cameras, and it is dense when they are at least half of
// 64 per camera. The wave then runs each dense slot in turn. Where cameras
// see small parts of the scene few slots are dense and most waves only
// check; where most are dense, a wave runs kDenseSpan of them.
// Compaction per step, 3M 5-camera (mostly dense) / 15M 5-camera (mostly
// sparse) scenes, by span: 1 (a wave per slot) 0.36 / 0.95 ms, 4 0.36 /
// 0.80, 8 0.37 / 0.77, 16 0.39 / 0.76, 64 0.70 / 0.73.
constexpr int kDenseSpan = 8;
static_assert(kDenseSpan >= 1 && kDenseSpan <= 64, "one slot per checking lane");
template <int DEG>
__global__ __launch_bounds__(kWave) void k_project_compact_dense(ProjectArgs a,
                                                                 const uint64_t* __restrict__ mask,
                                                                 const uint32_t* __restrict__ wg_scan,
                                                                 float* __restrict__ screen,
                                                                 uint32_t* __restrict__ aabb16,
                                                                 int64_t n_slots) {
  const int64_t w = int64_t(blockIdx.x) * kDenseSpan + threadIdx.x;
  const bool mine = threadIdx.x < unsigned(kDenseSpan) && w < n_slots;
  const int64_t words = a.N_pad / 64;  // mask words per camera
  int np = 0;
  if (mine)
    for (int c = 0; c < a.C; ++c) np += __popcll(mask[int64_t(c) * words + w]);
  uint64_t dense = __ballot(mine && 2 * np >= a.C * kWave);
  while (dense) {
    const int j = __builtin_ctzll(dense);
    dense &= dense - 1;
    compact_dense_wave<DEG>(a, mask, wg_scan, screen, aabb16,
                            int64_t(blockIdx.x) * kDenseSpan + j);
  }
}

// Compaction of the sparse waves for 2 to kCpMaxCams cameras (the dense
// ones run in k_project_compact_dense, launched beside it): the
// pair-list form of the sparse path above, in a kernel of its own so that
// it does not carry the dense path's registers (the SH row held across the
// camera walk): the wave lists its visible pairs in LDS Gaussian by Gaussian, puts
// each Gaussian's position, M (fp64) and opacity and the cameras in LDS,
// then computes the listed pairs 64 at a time, one per lane, each reading
// its Gaussian's SH row from memory.
constexpr int kCpMaxCams = 32;

template <int DEG>
__global__ __launch_bounds__(kWave, 4) void k_project_compact_pairs(
    ProjectArgs a, const uint64_t* __restrict__ mask, const uint32_t* __restrict__ wg_scan,
    float* __restrict__ screen, uint32_t* __restrict__ aabb16) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  __shared__ double s_M[9][kWave];
  __shared__ float s_mu[3][kWave];
  __shared__ float s_op[kWave];
  __shared__ uint32_t s_base[kCpMaxCams];
  __shared__ uint64_t s_mine[kCpMaxCams];
  __shared__ Camera s_cam[kCpMaxCams];
  extern __shared__ uint32_t s_who[];  // [64 C] camera << 6 | lane, Gaussian-major
  const int lane = threadIdx.x;
  const int C = a.C;
  const int half = int(blockIdx.x & 1);
  const int64_t grp = int64_t(blockIdx.x >> 1);
  const int64_t gw = int64_t(blockIdx.x) * kWave;  // this wave's first Gaussian

  const CamWords cw = load_cam_words(mask, wg_scan, a.N_pad, grp, 0, C);
  uint32_t vmask = 0;
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
  const int off = int(wave_incl_scan_u32(uint32_t(cnt))) - cnt;
  const int qn = __builtin_amdgcn_readlane(off + cnt, 63);  // wave-uniform
  // dense waves (at least half of 64 per camera) are k_project_compact's
  if (qn == 0 || 2 * qn >= C * kWave) return;
  {
    uint32_t vm = vmask;
    for (int j = off; vm; ++j) {
      const int c = __builtin_ctz(vm);
      vm &= vm - 1u;
      s_who[j] = (uint32_t(c) << 6) | uint32_t(lane);
    }
  }
  if (cnt) {
    GaussLocal<double> G;
    gauss_local(a.means, a.quats, a.log_scales, gw + lane, G);
#pragma unroll
    for (int i = 0; i < 9; ++i) s_M[i][lane] = G.M[i];
#pragma unroll
    for (int i = 0; i < 3; ++i) s_mu[i][lane] = G.mu[i];
    s_op[lane] = float(1.0 / (1.0 + exp(-double(a.opacity_logits[gw + lane]))));
  }
  if (lane < C) s_cam[lane] = load_camera(a.viewmats, a.Ks, lane);
  __syncthreads();
  for (int b = 0; b < qn; b += kWave) {
    const int e = b + lane;
    if (e >= qn) break;
    const uint32_t who = s_who[e];
    const int c = int(who >> 6), gl = int(who & 63u);
    const int64_t slot = int64_t(s_base[c]) + __popcll(s_mine[c] & ((1ull << gl) - 1ull));
    if (slot >= a.cap) continue;
    GaussLocal<double> Gs;
#pragma unroll
    for (int i = 0; i < 9; ++i) Gs.M[i] = s_M[i][gl];
#pragma unroll
    for (int i = 0; i < 3; ++i) Gs.mu[i] = s_mu[i][gl];
    compact_pair<DEG>(a, Gs, s_op[gl], a.sh + (gw + gl) * (K * 3), s_cam[c], slot, screen,
                      aabb16);
  }
}

__global__ void k_cam_offsets(const uint32_t* __restrict__ wg_scan, int64_t groups_per_cam, int C,
                              const uint64_t* __restrict__ total, int64_t* __restrict__ out) {
  const int c = threadIdx.x + blockIdx.x * blockDim.x;
  if (c > C) return;
  if (c == C || groups_per_cam == 0)
    out[c] = c == 0 ? 0 : int64_t(*total);
  else
    out[c] = int64_t(wg_scan[int64_t(c) * groups_per_cam]);
}

}  // namespace

hipError_t launch_cam_offsets(const uint32_t* wg_scan, int64_t groups_per_cam, int C,
                              const uint64_t* total, int64_t* out, hipStream_t s) {
  const int n = C + 1;
  ProfScope prof("k_cam_offsets", s);
  hipLaunchKernelGGL(k_cam_offsets, dim3((n + 255) / 256), dim3(256), 0, s, wg_scan,
                     groups_per_cam, C, total, out);
  return hipGetLastError();
}

ShNorm sh_norm_table() {
  // N_{l,m} = sqrt((2l+1)/(4 pi) * (l-m)!/(l+m)!), times sqrt(2) if m > 0.
  const double pi = 3.14159265358979323846;
  auto fact = [](int n) {
    double f = 1.0;
    for (int i = 2; i <= n; ++i) f *= i;
    return f;
  };
  ShNorm t{};
  int idx = 0;
  for (int l = 0; l <= 3; ++l)
    for (int m = 0; m <= l; ++m) {
      double v = std::sqrt((2.0 * l + 1.0) / (4.0 * pi) * fact(l - m) / fact(l + m));
      if (m > 0) v *= std::sqrt(2.0);
      t.n[idx++] = v;
    }
  return t;
}

hipError_t launch_project_mask(const ProjectArgs& a, uint64_t* mask, hipStream_t s) {
  const int64_t blocks = a.N_pad / kMaskGroup;
  if (blocks == 0) return hipSuccess;
  if (!fits_dispatch(uint64_t(blocks), kMaskGroup)) return hipErrorInvalidConfiguration;
  ProfScope prof("k_project_mask", s);
  if (a.C >= 2 && a.C <= kMaskFastCams)
    hipLaunchKernelGGL(k_project_mask_fast, dim3(uint32_t(blocks)), dim3(kMaskGroup),
                       mask_fast_lds(a.C), s, a, mask);
  else
    hipLaunchKernelGGL(k_project_mask, dim3(uint32_t(blocks)), dim3(kMaskGroup), 0, s, a, mask);
  return hipGetLastError();
}

hipError_t launch_project_compact(const ProjectArgs& a, const uint64_t* mask,
                                  const uint32_t* wg_scan, float* screen, uint32_t* aabb16,
                                  hipStream_t s) {
  const int64_t blocks = a.N_pad / kWave;  // one wave per half mask group
  if (blocks == 0) return hipSuccess;
  if (!fits_dispatch(uint64_t(blocks), kWave)) return hipErrorInvalidConfiguration;
  const dim3 grid{uint32_t(blocks)}, block{uint32_t(kWave)};
  ProfScope prof("k_project_compact", s);
  if (a.C >= 2 && a.C <= kCpMaxCams) {
    const size_t shm = size_t(kWave) * size_t(a.C) * sizeof(uint32_t);
    const dim3 dgrid{uint32_t((blocks + kDenseSpan - 1) / kDenseSpan)};  // kDenseSpan slots per wave
#define GS_LAUNCH_CP(D)                                                                         \
  hipLaunchKernelGGL(k_project_compact_pairs<D>, grid, block, shm, s, a, mask, wg_scan, screen, \
                     aabb16)
#define GS_LAUNCH_CD(D)                                                                        \
  hipLaunchKernelGGL(k_project_compact_dense<D>, dgrid, block, 0, s, a, mask, wg_scan, screen,  \
                     aabb16, blocks)
    switch (a.deg) {
      case 0: GS_LAUNCH_CP(0); GS_LAUNCH_CD(0); break;
      case 1: GS_LAUNCH_CP(1); GS_LAUNCH_CD(1); break;
      case 2: GS_LAUNCH_CP(2); GS_LAUNCH_CD(2); break;
      default: GS_LAUNCH_CP(3); GS_LAUNCH_CD(3); break;
    }
#undef GS_LAUNCH_CP
#undef GS_LAUNCH_CD
    return hipGetLastError();
  }
#define GS_LAUNCH_C(D)                                                                          \
  hipLaunchKernelGGL(k_project_compact<D>, grid, block, 0, s, a, mask, wg_scan, screen,          \
                     aabb16)
  switch (a.deg) {
    case 0: GS_LAUNCH_C(0); break;
    case 1: GS_LAUNCH_C(1); break;
    case 2: GS_LAUNCH_C(2); break;
    default: GS_LAUNCH_C(3); break;
  }
#undef GS_LAUNCH_C
  return hipGetLastError();
}

}  // namespace gs
