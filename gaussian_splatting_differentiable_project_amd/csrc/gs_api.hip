// C ABI of libgs: argument checks, workspace layout and the host-side
// sequencing of the kernels on the caller's stream.
//
// Error protocol ([VRAM] "The 4 GiB rule and the 2^31 limit"): totals
// are computed exactly in 64 bits on the device and read back once per
// call; the host checks them against the caller's capacities before it
// queues any kernel whose size depends on them, and returns the required
// size instead of writing past an allocation. Kernels queued before the
// check (the compaction) clamp their writes to the capacity themselves.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gs_internal.h"

using namespace gs;

// Device scratch of gs_project_noalloc: the projection workspace (totals,
// error flag, ticket, camera offsets, look-back words of the group-count
// scan) lives here instead of in a caller buffer. Every device the library
// runs on holds its own copy until the process ends. Host code reaches it
// only through the address hipGetSymbolAddress returns on that device.
constexpr uint64_t kNoAllocScratchBytes = 64 * 1024;
constexpr int kNoAllocMaxCams = 256;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr uint64_t kAlign = 256;

inline uint64_t align_up(uint64_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t tiles_x_of(int W) { return (W + kTile - 1) / kTile; }
int64_t tiles_y_of(int H) { return (H + kTile - 1) / kTile; }

int bits_for(uint64_t n_values) {  // bits needed to hold values 0..n_values-1
  int b = 0;
  while (b < 64 && (n_values - 1) >> b) ++b;
  return b;
}

// Bump layout of a workspace: offsets are computed the same way for
// sizing (base == nullptr) and for carving.
struct Carver {
  char* base;
  uint64_t off = 0;
  template <typename T>
  T* take(uint64_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + count * sizeof(T));
    return p;
  }
};

// ---- gs_project workspace ----
struct ProjectWs {
  uint64_t* total;
  int* err;
  uint32_t* ticket;
  int64_t* cam_off;   // [C+1]
  uint64_t* lookback;  // scan of the group counts
  uint64_t bytes;
};

ProjectWs carve_project(void* base, int64_t n_groups, int32_t C) {
  Carver cv{static_cast<char*>(base)};
  ProjectWs w{};
  w.total = cv.take<uint64_t>(1);
  w.err = cv.take<int>(1);
  w.ticket = cv.take<uint32_t>(1);
  w.cam_off = cv.take<int64_t>(uint64_t(C) + 1);
  w.lookback = cv.take<uint64_t>((uint64_t(n_groups) + kScanTile - 1) / kScanTile + 1);
  w.bytes = cv.off;
  return w;
}

// ---- gs_intersect workspace ----
// Layout: the words that must start at zero come first (one fill), then
// every array the first phase needs (sized by nnz and the tile count),
// then the arrays sized by n_isects (tile entries) or by the segment
// count (row segments), whichever way the geometry sorts.
struct IsectWs {
  uint64_t* total;      // [2 + kPrepBlocks]: n_isects, per-block depth key ranges, segments
  int* err;
  uint32_t* ticket;     // scan of the emit count matrix
  uint64_t* scan_lb;    // its look-back words
  uint64_t* sort_grp;   // radix sort group totals
  uint32_t *ticket_c, *ticket_t;  // row path: scans of the chunk and tile counts
  uint64_t *lb_c, *lb_t;
  uint64_t zero_words;  // u32 words to clear, from the start
  int64_t* cam_off;     // [C+1]
  uint32_t *dkeys_a, *dkeys_b, *dvals_a, *dvals_b;
  uint32_t *ord_keys_a, *ord_keys_b, *ord_vals_b;  // launch-order sort of the tiles
  uint32_t* sort_cnt;   // radix sort chunk counts (fixed size)
  uint32_t* emit_cnt;   // [digit][emit block] entry counts
  uint32_t* emit_rec;   // [nnz][2] rectangle of each depth-order position
  uint64_t* emit_off;   // their exclusive scan: first output position of each run
  uint64_t* emit_total;
  uint64_t phase1_bytes;  // enough to count (I still unknown)
  uint32_t *tkeys_a, *tkeys_b, *tvals;  // tile path
  uint32_t *rkeys_a, *rkeys_b, *rvals;  // row path
  RowScratch rows;
  uint64_t bytes;
};

// n_segments < 0: size the row path for every segment count up to
// n_isects (a pair's segments never outnumber its entries).
IsectWs carve_isect(void* base, int32_t C, int32_t W, int32_t H, int64_t nnz, int64_t n_isects,
                    int64_t n_segments) {
  Carver cv{static_cast<char*>(base)};
  IsectWs w{};
  const uint64_t n = uint64_t(nnz);
  const uint64_t mat = emit_matrix_len(n);
  const uint64_t n_tiles = uint64_t(C) * uint64_t(tiles_x_of(W) * tiles_y_of(H));
  const uint64_t R = row_windows(C, W, H);  // segment lists of the row path
  RowKeys rk{};
  const bool rows = row_keys_fit(C, W, H, &rk);
  w.total = cv.take<uint64_t>(2 + kPrepBlocks);
  w.err = cv.take<int>(1);
  w.ticket = cv.take<uint32_t>(1);
  w.scan_lb = cv.take<uint64_t>((mat + kScanTile - 1) / kScanTile + 1);
  w.sort_grp = cv.take<uint64_t>(sort_groups_bytes() / sizeof(uint64_t));
  if (rows) {
    w.rows.ticket_c = cv.take<uint32_t>(1);
    w.rows.ticket_t = cv.take<uint32_t>(1);
    w.rows.lb_c = cv.take<uint64_t>((R + kScanTile - 1) / kScanTile + 1);
    w.rows.lb_t = cv.take<uint64_t>((n_tiles + kScanTile - 1) / kScanTile + 1);
  }
  w.zero_words = cv.off / 4;
  w.cam_off = cv.take<int64_t>(uint64_t(C) + 1);
  w.dkeys_a = cv.take<uint32_t>(n);
  w.dkeys_b = cv.take<uint32_t>(n);
  w.dvals_a = cv.take<uint32_t>(n);
  w.dvals_b = cv.take<uint32_t>(n);
  w.ord_keys_a = cv.take<uint32_t>(n_tiles);
  w.ord_keys_b = cv.take<uint32_t>(n_tiles);
  w.ord_vals_b = cv.take<uint32_t>(n_tiles);
  w.sort_cnt = cv.take<uint32_t>(sort_counts_bytes() / sizeof(uint32_t));
  w.emit_cnt = cv.take<uint32_t>(mat);
  w.emit_rec = cv.take<uint32_t>(2 * n);
  w.emit_off = cv.take<uint64_t>(mat);
  w.emit_total = cv.take<uint64_t>(1);
  w.phase1_bytes = cv.off;
  const uint64_t I = n_isects > 0 ? uint64_t(n_isects) : 0;
  if (rows) {
    const bool bound = n_segments < 0;
    const uint64_t S = bound ? I : uint64_t(n_segments);
    w.rkeys_a = cv.take<uint32_t>(S);
    w.rkeys_b = cv.take<uint32_t>(S);
    w.rvals = cv.take<uint32_t>(S);
    w.rows.roff = cv.take<int64_t>(R + 1);
    w.rows.cc = cv.take<uint32_t>(R);
    w.rows.cq = cv.take<uint64_t>(R + 1);
    w.rows.cm = cv.take<uint32_t>(row_matrix_len(S, C, W, H, bound));
    w.rows.tcount = cv.take<uint32_t>(n_tiles);
  } else {
    w.tkeys_a = cv.take<uint32_t>(I);
    w.tkeys_b = cv.take<uint32_t>(I);
    w.tvals = cv.take<uint32_t>(I);
  }
  w.bytes = cv.off;
  return w;
}

// Page-locked host words for the device-to-host readback of each call,
// one set per thread and device (never freed: the process owns them).
// A call records an event after the copy and waits on that event only,
// so the kernels queued behind the copy keep the device busy while the
// host checks the totals.
struct HostStage {
  int64_t* buf = nullptr;
  uint64_t words = 0;
  hipEvent_t ev = nullptr;
};
constexpr int kMaxDevices = 64;
thread_local HostStage tl_stage[kMaxDevices];

hipError_t host_stage(uint64_t words, HostStage** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  HostStage& h = tl_stage[dev];
  if (!h.ev) {
    e = hipEventCreateWithFlags(&h.ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  if (h.words < words) {
    if (h.buf) {
      e = hipHostFree(h.buf);
      if (e != hipSuccess) return e;
      h.buf = nullptr;
      h.words = 0;
    }
    void* p = nullptr;
    e = hipHostMalloc(&p, words * sizeof(int64_t), hipHostMallocDefault);
    if (e != hipSuccess) return e;
    h.buf = static_cast<int64_t*>(p);
    h.words = words;
  }
  *out = &h;
  return hipSuccess;
}

// The device address of `scratch` on the current device, looked up once
// per device (with that device current) and kept.
void* g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GS_OK : GS_E_HIP; }

#define GS_TRY(expr)                            \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return GS_E_HIP;      \
  } while (0)

bool valid_image(int32_t C, int32_t W, int32_t H) {
  return C >= 1 && W >= 1 && H >= 1 && W <= 65535 && H <= 65535;
}

ProjectArgs project_args(int64_t N, int32_t C, int32_t W, int32_t H, int32_t deg,
                         const float* means, const float* quats, const float* log_scales,
                         const float* opacity_logits, const float* sh, const float* viewmats,
                         const float* Ks) {
  ProjectArgs a{};
  a.N = N, a.N_pad = gs_pad_n(N), a.C = C, a.W = W, a.H = H, a.deg = deg;
  a.means = means, a.quats = quats, a.log_scales = log_scales, a.opacity_logits = opacity_logits;
  a.sh = sh, a.viewmats = viewmats, a.Ks = Ks;
  a.norm = sh_norm_table();
  a.qsx = float(kQ16) / float(W);
  a.qsy = float(kQ16) / float(H);
  return a;
}

}  // namespace

extern "C" {

const char* gs_status_str(int status) {
  switch (status) {
    case GS_OK: return "ok";
    case GS_E_INVALID: return "invalid argument";
    case GS_E_CAPACITY: return "output capacity too small";
    case GS_E_WORKSPACE: return "workspace too small";
    case GS_E_OVERFLOW: return "count exceeds its storage type";
    case GS_E_HIP: return "HIP runtime error";
    case GS_E_DEVICE: return "kernel reported an internal error";
    default: return "unknown status";
  }
}

int gs_version(void) { return 200; }

int gs_readback_status(int32_t device_flag, int64_t count, int64_t count_limit,
                       int64_t capacity) {
  if (device_flag != 0) return GS_E_DEVICE;  // the count itself is then unreliable
  if (count < 0 || count >= count_limit) return GS_E_OVERFLOW;
  if (count > capacity) return GS_E_CAPACITY;
  return GS_OK;
}

int gs_tile_offsets_check(const int64_t* tile_offsets, uint64_t n_tiles) {
  if (!tile_offsets) return GS_E_INVALID;
  if (tile_offsets[0] != 0) return GS_E_INVALID;
  int overflow = 0;
  for (uint64_t t = 0; t < n_tiles; ++t) {
    const int64_t a = tile_offsets[t], b = tile_offsets[t + 1];
    if (b < a) return GS_E_INVALID;
    if (b - a >= (int64_t(1) << 31)) overflow = 1;
  }
  return overflow ? GS_E_OVERFLOW : GS_OK;
}

int64_t gs_pad_n(int64_t N) { return N <= 0 ? 0 : ((N + kMaskGroup - 1) / kMaskGroup) * kMaskGroup; }

uint64_t gs_project_workspace_bytes(int64_t N, int32_t C) {
  if (N < 0 || C < 1) return 0;
  return carve_project(nullptr, int64_t(C) * gs_pad_n(N) / kMaskGroup, C).bytes;
}

uint64_t gs_intersect_workspace_bytes(int32_t C, int32_t W, int32_t H, int64_t nnz,
                                      int64_t n_isects) {
  if (C < 1 || nnz < 0 || W < 1 || H < 1) return 0;
  return carve_isect(nullptr, C, W, H, nnz, n_isects, -1).bytes;
}

}  // extern "C"

namespace {

// Argument checks and kernel sequence shared by gs_project and
// gs_project_noalloc, up to (not including) the readback of the totals:
// the zero fill of the workspace, the visibility pass, the scan of the
// group counts and the camera offsets, then the compaction. `ws` is the
// carved workspace; `before_compact` runs after the offsets are queued and
// before the compaction (gs_project puts its readback there).
template <typename F>
int project_queue(hipStream_t s, const ProjectArgs& a, uint64_t* mask, uint32_t* wg_count,
                  uint32_t* wg_scan, float* screen, uint32_t* aabb16, const ProjectWs& ws,
                  void* ws_base, F&& before_compact) {
  const int64_t n_groups = int64_t(a.C) * a.N_pad / kMaskGroup;
  GS_TRY(launch_fill_u32(ws_base, 0u, ws.bytes / 4, s));
  GS_TRY(launch_project_mask(a, mask, s));
  // the group counts are the popcounts of the mask words; the scan takes
  // them from the words and writes them out on the way
  GS_TRY(launch_scan_u32(nullptr, mask, wg_count, uint64_t(n_groups), wg_scan, nullptr, ws.total,
                         ws.lookback, ws.ticket, ws.err, s));
  GS_TRY(launch_cam_offsets(wg_scan, a.N_pad / kMaskGroup, a.C, ws.total, ws.cam_off, s));
  GS_TRY(before_compact());
  // The compaction needs no host decision: slots at or past the capacity
  // are not written, so it is queued before the host reads the count.
  GS_TRY(launch_project_compact(a, mask, wg_scan, screen, aabb16, s));
  return GS_OK;
}

int project_check(int64_t N, int32_t C, int32_t W, int32_t H, int32_t sh_degree,
                  const float* means, const float* quats, const float* log_scales,
                  const float* opacity_logits, const float* sh, const float* viewmats,
                  const float* Ks, const uint64_t* mask, const uint32_t* wg_count,
                  const uint32_t* wg_scan, const float* screen, const uint32_t* aabb16,
                  int64_t screen_capacity, const int64_t* nnz_out) {
  if (N < 0 || !valid_image(C, W, H) || sh_degree < 0 || sh_degree > 3 || !nnz_out ||
      screen_capacity < 0)
    return GS_E_INVALID;
  if (N > 0 && (!means || !quats || !log_scales || !opacity_logits || !sh || !viewmats || !Ks ||
                !mask || !wg_count || !wg_scan))
    return GS_E_INVALID;
  if (!aligned(quats, 16) || !aligned(screen, 8) || !aligned(aabb16, 8) || !aligned(mask, 8))
    return GS_E_INVALID;
  if (screen_capacity > 0 && (!screen || !aabb16)) return GS_E_INVALID;
  return GS_OK;
}

}  // namespace

extern "C" {

int gs_project(void* stream, int64_t N, int32_t C, int32_t W, int32_t H, int32_t sh_degree,
               const float* means, const float* quats, const float* log_scales,
               const float* opacity_logits, const float* sh, const float* viewmats,
               const float* Ks, uint64_t* mask, uint32_t* wg_count, uint32_t* wg_scan,
               float* screen, uint32_t* aabb16, int64_t screen_capacity, void* workspace,
               uint64_t workspace_bytes, int64_t* nnz_out, int64_t* cam_offsets_out) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = project_check(N, C, W, H, sh_degree, means, quats, log_scales, opacity_logits, sh,
                         viewmats, Ks, mask, wg_count, wg_scan, screen, aabb16, screen_capacity,
                         nnz_out);
  if (st != GS_OK) return st;
  if ((N > 0 && !workspace) || !aligned(workspace, kAlign)) return GS_E_INVALID;
  const ProjectArgs a = [&] {
    ProjectArgs r = project_args(N, C, W, H, sh_degree, means, quats, log_scales, opacity_logits,
                                 sh, viewmats, Ks);
    r.cap = screen_capacity;
    return r;
  }();
  const int64_t n_groups = int64_t(C) * a.N_pad / kMaskGroup;
  const ProjectWs ws = carve_project(workspace, n_groups, C);
  if (!workspace || workspace_bytes < ws.bytes) return GS_E_WORKSPACE;

  HostStage* hs = nullptr;
  GS_TRY(host_stage(uint64_t(C) + 2, &hs));
  hs->buf[C + 1] = 0;  // receives the 4-byte error flag in its low half
  st = project_queue(s, a, mask, wg_count, wg_scan, screen, aabb16, ws, workspace, [&] {
    hipError_t e = hipMemcpyAsync(hs->buf, ws.cam_off, sizeof(int64_t) * (C + 1),
                                  hipMemcpyDeviceToHost, s);
    // the scan's bounded look-back raises this flag if a wait timed out;
    // the slots and nnz are then wrong, so it is checked before them
    if (e == hipSuccess)
      e = hipMemcpyAsync(hs->buf + C + 1, ws.err, sizeof(int), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipEventRecord(hs->ev, s);
    return e;
  });
  // wait even after an error: the copy into the staging words must land
  const hipError_t e2 = hipEventSynchronize(hs->ev);
  if (st != GS_OK) return st;
  if (e2 != hipSuccess) return GS_E_HIP;
  const int64_t nnz = hs->buf[C];
  int flag = 0;
  std::memcpy(&flag, hs->buf + C + 1, sizeof(int));
  *nnz_out = nnz;
  if (cam_offsets_out) std::memcpy(cam_offsets_out, hs->buf, sizeof(int64_t) * (C + 1));
  return gs_readback_status(flag, nnz, int64_t(1) << 31, screen_capacity);
}

int gs_project_noalloc(void* stream, int64_t N, int32_t C, int32_t W, int32_t H,
                       int32_t sh_degree, const float* means, const float* quats,
                       const float* log_scales, const float* opacity_logits, const float* sh,
                       const float* viewmats, const float* Ks, uint64_t* mask,
                       uint32_t* wg_count, uint32_t* wg_scan, float* screen, uint32_t* aabb16,
                       int64_t screen_capacity, int64_t* nnz_out, int64_t* cam_offsets_out) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = project_check(N, C, W, H, sh_degree, means, quats, log_scales, opacity_logits, sh,
                         viewmats, Ks, mask, wg_count, wg_scan, screen, aabb16, screen_capacity,
                         nnz_out);
  if (st != GS_OK) return st;
  // sizes past the static scratch (or the host words below) are refused
  // before any device work
  const int64_t n_groups = int64_t(C) * gs_pad_n(N) / kMaskGroup;
  if (C > kNoAllocMaxCams || carve_project(nullptr, n_groups, C).bytes > kNoAllocScratchBytes)
    return GS_E_WORKSPACE;
  void* base = nullptr;
  GS_TRY(scratch_address(&base));
  const ProjectWs ws = carve_project(base, n_groups, C);
  ProjectArgs a = project_args(N, C, W, H, sh_degree, means, quats, log_scales, opacity_logits, sh,
                               viewmats, Ks);
  a.cap = screen_capacity;
  st = project_queue(s, a, mask, wg_count, wg_scan, screen, aabb16, ws, base,
                     [] { return hipSuccess; });
  if (st != GS_OK) return st;
  // the totals land in words on this thread's stack: no page-locked
  // staging, so the host waits for the whole call here
  int64_t words[kNoAllocMaxCams + 1];
  int flag = 0;
  GS_TRY(hipMemcpyAsync(words, ws.cam_off, sizeof(int64_t) * (C + 1), hipMemcpyDeviceToHost, s));
  GS_TRY(hipMemcpyAsync(&flag, ws.err, sizeof(int), hipMemcpyDeviceToHost, s));
  GS_TRY(hipStreamSynchronize(s));
  const int64_t nnz = words[C];
  *nnz_out = nnz;
  if (cam_offsets_out) std::memcpy(cam_offsets_out, words, sizeof(int64_t) * (C + 1));
  return gs_readback_status(flag, nnz, int64_t(1) << 31, screen_capacity);
}

int gs_intersect(void* stream, int32_t C, int32_t W, int32_t H, int64_t nnz, const float* screen,
                 const uint32_t* aabb16, const int64_t* cam_offsets, void* workspace,
                 uint64_t workspace_bytes, uint32_t* flatten_ids, int64_t isect_capacity,
                 int64_t* tile_offsets, uint64_t* sorted_keys, uint32_t* tile_order,
                 int64_t* n_isects_out, uint64_t* workspace_needed_out) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!valid_image(C, W, H) || nnz < 0 || !n_isects_out || !workspace_needed_out ||
      !tile_offsets || !cam_offsets || isect_capacity < 0)
    return GS_E_INVALID;
  if (nnz > 0 && (!screen || !aabb16)) return GS_E_INVALID;
  if (!aligned(aabb16, 8) || !aligned(workspace, kAlign) || !aligned(flatten_ids, 16))
    return GS_E_INVALID;
  *n_isects_out = -1;
  if (nnz >= (int64_t(1) << 31)) return GS_E_OVERFLOW;
  int64_t widest = 0;  // most pairs of any one camera
  for (int c = 0; c < C; ++c) {
    if (cam_offsets[c] < 0 || cam_offsets[c] > cam_offsets[c + 1]) return GS_E_INVALID;
    widest = cam_offsets[c + 1] - cam_offsets[c] > widest ? cam_offsets[c + 1] - cam_offsets[c]
                                                          : widest;
  }
  if (cam_offsets[0] != 0 || cam_offsets[C] != nnz) return GS_E_INVALID;
  // A pair meets each tile of its camera at most once, so no tile list is
  // longer than its camera's pair count; the raster calls index a list
  // with 32-bit local ids (last_ids), which this bound keeps below 2^31.
  if (widest >= (int64_t(1) << 31)) return GS_E_OVERFLOW;
  const uint64_t n_tiles = uint64_t(C) * uint64_t(tiles_x_of(W) * tiles_y_of(H));
  if (n_tiles >= (uint64_t(1) << 32)) return GS_E_OVERFLOW;

  RowKeys rk{};
  const bool rows = row_keys_fit(C, W, H, &rk);
  IsectWs ws = carve_isect(workspace, C, W, H, nnz, 0, 0);
  *workspace_needed_out = ws.phase1_bytes;
  if (!workspace || workspace_bytes < ws.phase1_bytes) return GS_E_WORKSPACE;
  SortScratch sc;
  sc.cnt = ws.sort_cnt;
  sc.grp = ws.sort_grp;
  HostStage* hs = nullptr;
  GS_TRY(host_stage(3 + kPrepBlocks, &hs));
  hs->buf[2 + kPrepBlocks] = 0;  // receives the scans' error flag

  // Phase 1: depth keys, per-slot tile counts and their exact 64-bit total.
  GS_TRY(launch_fill_u32(workspace, 0u, ws.zero_words, s));
  GS_TRY(hipMemcpyAsync(ws.cam_off, cam_offsets, sizeof(int64_t) * (C + 1),
                        hipMemcpyHostToDevice, s));
  GS_TRY(launch_isect_prep(uint64_t(nnz), screen, aabb16, W, H, ws.dkeys_a, ws.dvals_a, ws.total,
                           s));
  GS_TRY(hipMemcpyAsync(hs->buf, ws.total, (2 + kPrepBlocks) * sizeof(uint64_t),
                        hipMemcpyDeviceToHost, s));
  GS_TRY(hipEventRecord(hs->ev, s));
  // Phase 2 needs only nnz-sized memory, so it is queued before the host
  // waits for the total: a stable sort of the slots by depth, low 24 bits
  // first (three passes, ending in the b buffers).
  bool in_b = false;
  const hipError_t e = launch_sort_passes(ws.dkeys_a, ws.dvals_a, ws.dkeys_b, ws.dvals_b,
                                          uint64_t(nnz), 0, 24, sc, &in_b, s);
  // wait even after an error: the copy into the staging words must land
  const hipError_t e2 = hipEventSynchronize(hs->ev);
  if (e != hipSuccess || e2 != hipSuccess) return GS_E_HIP;
  // The top 8 bits need a pass only when the keys differ there: every key
  // lies between the smallest and the largest, so when those two agree
  // above bit 24, all keys do (positive depths order like their bits).
  uint32_t kmax = 0, knmin = 0;
  for (uint32_t b = 0; b < kPrepBlocks; ++b) {
    const uint64_t w = uint64_t(hs->buf[1 + b]);
    const uint32_t m = uint32_t(w >> 32), nm = uint32_t(w);
    kmax = m > kmax ? m : kmax;
    knmin = nm > knmin ? nm : knmin;
  }
  const uint32_t kmin = ~knmin;
  if (nnz > 0 && ((kmin ^ kmax) >> 24) != 0) {
    bool in_b2 = false;
    GS_TRY(launch_sort_passes(ws.dkeys_b, ws.dvals_b, ws.dkeys_a, ws.dvals_a, uint64_t(nnz), 24,
                              8, sc, &in_b2, s));
    in_b = !in_b2;  // one pass: from b back into a
  }
  const uint32_t* order = in_b ? ws.dvals_b : ws.dvals_a;
  const uint64_t I = uint64_t(hs->buf[0]);
  const uint64_t S = uint64_t(hs->buf[1 + kPrepBlocks]);  // tile-row segments
  bool flag_pending = false;
  *n_isects_out = int64_t(I);
  if (I >= (uint64_t(1) << 62)) return GS_E_OVERFLOW;
  ws = carve_isect(workspace, C, W, H, nnz, int64_t(I), int64_t(S));
  *workspace_needed_out = ws.bytes;
  if (int64_t(I) > isect_capacity) return GS_E_CAPACITY;
  if (workspace_bytes < ws.bytes) return GS_E_WORKSPACE;
  if (I > 0 && !flatten_ids) return GS_E_INVALID;

  if (I == 0) {
    GS_TRY(launch_fill_u32(tile_offsets, 0u, 2 * (n_tiles + 1), s));
  } else if (rows) {
    // Phase 3: (tile row, pair) segments in depth order, written already
    // partitioned by the low digit of their row id (the first pass of a
    // stable sort by row id); phase 4: the remaining digits. The pair ids
    // start in flatten_ids when the pass count is odd, so that they end in
    // the workspace, which the expansion reads while writing flatten_ids.
    const int b1 = emit_digit_bits(rk.rb);
    const int rest = rk.rb > b1 ? rk.rb - b1 : 0;
    const int passes = rest ? sort_passes(rest) : 0;
    uint32_t* v_first = (passes & 1) ? flatten_ids : ws.rvals;
    uint32_t* v_second = (passes & 1) ? ws.rvals : flatten_ids;
    GS_TRY(launch_isect_emit(uint64_t(nnz), order, aabb16, ws.cam_off, C, W, H, b1, &rk, S,
                             ws.emit_cnt, ws.emit_rec, ws.emit_off, ws.emit_total, ws.scan_lb,
                             ws.ticket, ws.err, ws.rkeys_a, v_first, s));
    in_b = false;
    if (passes)
      GS_TRY(launch_sort_passes(ws.rkeys_a, v_first, ws.rkeys_b, v_second, S, b1, rest, sc,
                                &in_b, s));
    // Phase 5: tile offsets from the segments' counts, then the entries.
    GS_TRY(launch_row_sort(in_b ? ws.rkeys_b : ws.rkeys_a, ws.rvals, S, C, W, H, rk, ws.rows,
                           ws.err, screen, uint64_t(nnz), I, flatten_ids, tile_offsets,
                           sorted_keys, s));
  } else {
    // Phase 3: (tile id, slot) entries in depth order, written already
    // partitioned by the low digit of the tile id (the first sort pass).
    const int tbits = bits_for(n_tiles);
    const int b1 = emit_digit_bits(tbits);
    const int rest = tbits > b1 ? tbits - b1 : 0;
    const int passes = rest ? sort_passes(rest) : 0;
    // the final pass must land its values in flatten_ids
    uint32_t* v_first = (passes & 1) ? ws.tvals : flatten_ids;
    uint32_t* v_second = (passes & 1) ? flatten_ids : ws.tvals;
    GS_TRY(launch_isect_emit(uint64_t(nnz), order, aabb16, ws.cam_off, C, W, H, b1, nullptr, I,
                             ws.emit_cnt, ws.emit_rec, ws.emit_off, ws.emit_total, ws.scan_lb,
                             ws.ticket,
                             ws.err, ws.tkeys_a, v_first, s));
    // Phase 4: the remaining digits of the stable sort by tile id.
    in_b = false;
    if (passes)
      GS_TRY(launch_sort_passes(ws.tkeys_a, v_first, ws.tkeys_b, v_second, I, b1, rest, sc,
                                &in_b, s));
    const uint32_t* tkeys = in_b ? ws.tkeys_b : ws.tkeys_a;
    // Phase 5: per-tile ranges (and the composed 64-bit keys on request).
    GS_TRY(launch_tile_ranges(tkeys, I, n_tiles, tile_offsets, s));
    if (sorted_keys) GS_TRY(launch_compose_keys(tkeys, flatten_ids, screen, I, sorted_keys, s));
  }
  if (I > 0) {
    // The scans above wait on predecessors with a bounded spin and raise
    // ws.err when a wait times out (their offsets are then wrong). The
    // flag is copied here, and the host waits for that copy only after
    // the launch-order kernels have been queued, so the device stays busy
    // meanwhile.
    GS_TRY(hipMemcpyAsync(hs->buf + 2 + kPrepBlocks, ws.err, sizeof(int), hipMemcpyDeviceToHost,
                          s));
    GS_TRY(hipEventRecord(hs->ev, s));
    flag_pending = true;
  }
  // Phase 6: launch order for the raster calls, longest tiles first (a
  // stable sort of 16-bit inverted counts): ranks of unique keys for small
  // tile counts, else two radix passes that end in tile_order.
  if (tile_order) {
    if (tile_order_small(n_tiles)) {
      GS_TRY(launch_tile_order_small(tile_offsets, n_tiles, tile_order, s));
    } else {
      GS_TRY(launch_tile_order_keys(tile_offsets, n_tiles, ws.ord_keys_a, tile_order, s));
      GS_TRY(launch_sort_passes(ws.ord_keys_a, tile_order, ws.ord_keys_b, ws.ord_vals_b, n_tiles,
                                0, 16, sc, &in_b, s));
    }
  }
  if (!flag_pending) return GS_OK;
  GS_TRY(hipEventSynchronize(hs->ev));
  int flag = 0;
  std::memcpy(&flag, hs->buf + 2 + kPrepBlocks, sizeof(int));
  return flag ? GS_E_DEVICE : GS_OK;
}

int gs_rasterize_fwd(void* stream, int32_t C, int32_t W, int32_t H, const float* screen,
                     const uint32_t* flatten_ids, const int64_t* tile_offsets,
                     const uint32_t* tile_order, const float* background, float* out_rgb,
                     float* out_T, float* out_depth, int32_t* last_ids) {
  if (!valid_image(C, W, H) || !tile_offsets || !out_rgb || !out_T || !last_ids)
    return GS_E_INVALID;
  if (!aligned(screen, 8)) return GS_E_INVALID;
  return hip_status(launch_raster_fwd(C, W, H, screen, flatten_ids, tile_offsets, tile_order,
                                      background, out_rgb, out_T, out_depth, last_ids,
                                      static_cast<hipStream_t>(stream)));
}

int gs_rasterize_bwd(void* stream, int32_t C, int32_t W, int32_t H, int64_t nnz,
                     const float* screen, const uint32_t* flatten_ids, const int64_t* tile_offsets,
                     const uint32_t* tile_order, const float* background, const float* out_T,
                     const int32_t* last_ids, const float* v_rgb, const float* v_T,
                     const float* v_depth, float* v_screen, float* v_background) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!valid_image(C, W, H) || nnz < 0 || !tile_offsets || !out_T || !last_ids || !v_rgb)
    return GS_E_INVALID;
  if (nnz > 0 && !v_screen) return GS_E_INVALID;
  if (!aligned(screen, 8)) return GS_E_INVALID;
  GS_TRY(launch_fill_u32(v_screen, 0u, uint64_t(nnz) * kRow, s));
  if (v_background) GS_TRY(launch_fill_u32(v_background, 0u, 3ull * uint64_t(C), s));
  return hip_status(launch_raster_bwd(C, W, H, screen, flatten_ids, tile_offsets, tile_order,
                                      background, out_T, last_ids, v_rgb, v_T, v_depth, v_screen,
                                      v_background, s));
}

int gs_project_bwd(void* stream, int64_t N, int32_t C, int32_t W, int32_t H, int32_t sh_degree,
                   const float* means, const float* quats, const float* log_scales,
                   const float* opacity_logits, const float* sh, const float* viewmats,
                   const float* Ks, const uint64_t* mask, const uint32_t* wg_scan,
                   const float* v_screen, float* v_means, float* v_quats, float* v_log_scales,
                   float* v_opacity_logits, float* v_sh, int32_t accumulate) {
  if (N < 0 || !valid_image(C, W, H) || sh_degree < 0 || sh_degree > 3) return GS_E_INVALID;
  if (N == 0) return GS_OK;
  if (!means || !quats || !log_scales || !opacity_logits || !sh || !viewmats || !Ks || !mask ||
      !wg_scan || !v_means || !v_quats || !v_log_scales || !v_opacity_logits || !v_sh)
    return GS_E_INVALID;
  if (!aligned(quats, 16) || !aligned(v_quats, 16) || !aligned(v_sh, 16) || !aligned(v_screen, 8))
    return GS_E_INVALID;
  const ProjectArgs a = project_args(N, C, W, H, sh_degree, means, quats, log_scales,
                                     opacity_logits, sh, viewmats, Ks);
  return hip_status(launch_project_bwd(a, mask, wg_scan, v_screen, v_means, v_quats, v_log_scales,
                                       v_opacity_logits, v_sh, accumulate, nullptr,
                                       static_cast<hipStream_t>(stream)));
}

int gs_project_bwd_adam(void* stream, int64_t N, int32_t C, int32_t W, int32_t H,
                        int32_t sh_degree, float* means, float* quats, float* log_scales,
                        float* opacity_logits, float* sh, const float* viewmats, const float* Ks,
                        const uint64_t* mask, const uint32_t* wg_scan, const float* v_screen,
                        float* const* adam_m, float* const* adam_v, const float* lr, float beta1,
                        float beta2, float eps, int32_t step) {
  if (N < 0 || !valid_image(C, W, H) || sh_degree < 0 || sh_degree > 3) return GS_E_INVALID;
  if (!adam_m || !adam_v || !lr || step < 1 || !(beta1 >= 0.f && beta1 < 1.f) ||
      !(beta2 >= 0.f && beta2 < 1.f) || !(eps > 0.f))
    return GS_E_INVALID;
  if (N == 0) return GS_OK;
  if (!means || !quats || !log_scales || !opacity_logits || !sh || !viewmats || !Ks || !mask ||
      !wg_scan)
    return GS_E_INVALID;
  for (int i = 0; i < 5; ++i)
    if (!adam_m[i] || !adam_v[i]) return GS_E_INVALID;
  if (!aligned(quats, 16) || !aligned(v_screen, 8)) return GS_E_INVALID;
  const ProjectArgs a = project_args(N, C, W, H, sh_degree, means, quats, log_scales,
                                     opacity_logits, sh, viewmats, Ks);
  AdamArgs ad{};
  float* const params[5] = {means, quats, log_scales, opacity_logits, sh};
  for (int i = 0; i < 5; ++i) {
    ad.p[i] = params[i];
    ad.m[i] = adam_m[i];
    ad.v[i] = adam_v[i];
  }
  for (int i = 0; i < 6; ++i) ad.lr[i] = lr[i];
  ad.beta1 = beta1;
  ad.beta2 = beta2;
  ad.eps = eps;
  // bias corrections in double, then rounded once
  ad.inv_bc1 = float(1.0 / (1.0 - std::pow(double(beta1), double(step))));
  ad.inv_bc2 = float(1.0 / (1.0 - std::pow(double(beta2), double(step))));
  return hip_status(launch_project_bwd(a, mask, wg_scan, v_screen, nullptr, nullptr, nullptr,
                                       nullptr, nullptr, 0, &ad,
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"
