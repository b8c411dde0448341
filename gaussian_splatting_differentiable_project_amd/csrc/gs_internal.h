// Host-side launchers shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gs_projmath.h"

namespace gs {

// Records a HIP event pair around one kernel launch on stream s when
// gs_profile_enable() is on and the name matches its filter.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_{}, b_{};
  bool on_ = false;
};

// A dispatch's work-item count per dimension is 32-bit: a grid of
// blocks x threads >= 2^32 would silently wrap. Launchers that size their
// grid by the data check it with this before launching.
inline bool fits_dispatch(uint64_t blocks, uint64_t threads_per_block) {
  return blocks * (threads_per_block ? threads_per_block : 256) < (uint64_t(1) << 32);
}

struct ProjectArgs {
  int64_t N, N_pad;
  int32_t C, W, H, deg;
  const float *means, *quats, *log_scales, *opacity_logits, *sh, *viewmats, *Ks;
  ShNorm norm;
  float qsx, qsy;  // 65535 / W, 65535 / H in fp32
  int64_t cap;     // compaction: slots at or past this are not written
};

ShNorm sh_norm_table();

hipError_t launch_project_mask(const ProjectArgs& a, uint64_t* mask, hipStream_t s);
hipError_t launch_project_compact(const ProjectArgs& a, const uint64_t* mask,
                                  const uint32_t* wg_scan, float* screen, uint32_t* aabb16,
                                  hipStream_t s);
// Adam state for the fused projection backward: parameter, first and
// second moment pointers for means, quats, log_scales, opacity_logits, sh
// (updated in place), learning rates of the six groups (means, quats,
// log_scales, opacity_logits, SH coefficient 0, higher SH), betas, eps and
// the inverse bias corrections 1 / (1 - beta^t).
struct AdamArgs {
  float* p[5];
  float* m[5];
  float* v[5];
  float lr[6];
  float beta1, beta2, eps, inv_bc1, inv_bc2;
};

// adam == nullptr: write (or add) the gradients; else fold them into one
// Adam step and write no gradient (the v_* pointers are then unused).
hipError_t launch_project_bwd(const ProjectArgs& a, const uint64_t* mask,
                              const uint32_t* wg_scan, const float* v_screen, float* v_means,
                              float* v_quats, float* v_log_scales, float* v_opacity_logits,
                              float* v_sh, int accumulate, const AdamArgs* adam, hipStream_t s);

// Exclusive scan of n uint32 values into uint32 or uint64 outputs; the
// total is written to *total (device). With `mask` non-null the values are
// the popcounts of mask word pairs (2e, 2e + 1), also written to counts[e],
// and `in` is unused. Scratch: lookback[ceil(n / kScanTile)] + one ticket;
// both must be zero.
hipError_t launch_scan_u32(const uint32_t* in, const uint64_t* mask, uint32_t* counts,
                           uint64_t n, uint32_t* out32, uint64_t* out64, uint64_t* total,
                           uint64_t* lookback, uint32_t* ticket, int* err, hipStream_t s);

hipError_t launch_fill_u32(void* p, uint32_t v, uint64_t n_words, hipStream_t s);

// Stable LSD radix sort, one 8-bit digit per pass, of uint32 keys with
// uint32 values, over the bit range [bit0, bit0 + bits). The scratch has
// fixed sizes whatever n is. The group totals must be zero before the
// first pass of the first sort that uses a scratch; each pass clears the
// buffer the next one fills, so consecutive sorts on one stream can share
// it (parity tracks which buffer is live).
struct SortScratch {
  uint32_t* cnt;   // [kSortChunks][256] per-chunk digit counts (sort_counts_bytes)
  uint64_t* grp;   // [2][kSortGroups][256] group totals (sort_groups_bytes), zeroed
  int parity = 0;
};
int sort_passes(int bits);
uint64_t sort_counts_bytes();
uint64_t sort_groups_bytes();
// Runs all passes; the result ends in (keys_a, vals_a) when the pass count
// is even, else in (keys_b, vals_b), which *in_b reports.
hipError_t launch_sort_passes(uint32_t* keys_a, uint32_t* vals_a, uint32_t* keys_b,
                              uint32_t* vals_b, uint64_t n, int bit0, int bits,
                              SortScratch& sc, bool* in_b, hipStream_t s);

// Intersection stages (gs_intersect.hip).
// total[2 + kPrepBlocks] (zeroed): total[0] = intersection count; for
// each block b, total[1 + b] = (largest depth key << 32) | complement of
// its smallest depth key; total[1 + kPrepBlocks] = segment count (the
// sum over pairs of their rectangles' rows times the 64-tile windows each
// row meets).
constexpr uint32_t kPrepBlocks = 1024;
hipError_t launch_isect_prep(uint64_t nnz, const float* screen, const uint32_t* aabb16, int W,
                             int H, uint32_t* dkeys, uint32_t* dvals, uint64_t* total,
                             hipStream_t s);
// Entries of the slots in depth order, written already stably
// partitioned by the low `bits` = emit_digit_bits(tile_bits) bits of their
// tile id (the first pass of the LSD sort by tile id). Scratch: a count matrix
// mat[emit_matrix_len(nnz)] (uint32), per-position rectangle records
// rec[2 * nnz] (uint32), the matrix scan mat_off (uint64) and its total,
// and the scan's look-back words (ceil(emit_matrix_len / kScanTile)) and
// ticket, which must be zero. Writes are clamped to `cap` entries.
// With `rows` set, the emit writes segments instead: the part of a pair's
// tile row inside one window of 64 tiles, keyed by the window id
// (c * tiles_y + ty) * ceil(tiles_x / 64) + tx / 64 in bits [0, rb), the
// pair's first tile on the row in the next xb bits, its width - 1 above;
// `bits` then splits the window id.
struct RowKeys {
  int rb, xb;
};
// Whether the segment keys of this geometry fit 32 bits (rb + 2 xb <= 32).
bool row_keys_fit(int C, int W, int H, RowKeys* out);
int emit_digit_bits(int tile_bits);
uint64_t emit_matrix_len(uint64_t nnz);
hipError_t launch_isect_emit(uint64_t nnz, const uint32_t* order, const uint32_t* aabb16,
                             const int64_t* cam_off, int C, int W, int H, int bits,
                             const RowKeys* rows, uint64_t cap, uint32_t* mat, uint32_t* rec,
                             uint64_t* mat_off, uint64_t* mat_total,
                             uint64_t* lb, uint32_t* ticket, int* err, uint32_t* tkeys,
                             uint32_t* tvals, hipStream_t s);
// Ranges of keys & kmask in a list sorted by them.
hipError_t launch_tile_ranges(const uint32_t* tkeys, uint64_t n, uint64_t n_tiles, int64_t* toff,
                              hipStream_t s, uint32_t kmask = 0xFFFFFFFFu);
// The sorted list from the segments sorted by window id (keys rkeys, pairs
// rvals): tile offsets toff[C*T + 1], ids[n_isects] and, when keys_out is
// not null, the 64-bit keys. Scratch (R = C * tiles_y * ceil(tiles_x / 64)
// windows, row_windows()): roff[R + 1], cc[R], cq[R + 1], the count matrix
// cm[row_matrix_len], tcount[C*T], and two scans' look-back words and
// tickets (zeroed): lb_c for R values, lb_t for C*T values. Writes are
// clamped to `cap` entries.
struct RowScratch {
  int64_t* roff;
  uint32_t* cc;
  uint64_t* cq;
  uint32_t* cm;
  uint32_t* tcount;
  uint64_t *lb_c, *lb_t;
  uint32_t *ticket_c, *ticket_t;
};
// Count-matrix words for n_segments segments; with `bound`, an upper
// bound valid for every smaller segment count.
uint64_t row_matrix_len(uint64_t n_segments, int C, int W, int H, bool bound);
uint64_t row_windows(int C, int W, int H);
hipError_t launch_row_sort(const uint32_t* rkeys, const uint32_t* rvals, uint64_t n_segments,
                           int C, int W, int H, const RowKeys& rk, const RowScratch& w,
                           int* err, const float* screen, uint64_t nnz, uint64_t cap,
                           uint32_t* ids, int64_t* toff, uint64_t* keys_out, hipStream_t s);
// Heavy-first launch order in one kernel for small tile counts.
bool tile_order_small(uint64_t n_tiles);
hipError_t launch_tile_order_small(const int64_t* toff, uint64_t n_tiles, uint32_t* order,
                                   hipStream_t s);
hipError_t launch_tile_order_keys(const int64_t* toff, uint64_t n_tiles, uint32_t* keys,
                                  uint32_t* vals, hipStream_t s);
hipError_t launch_compose_keys(const uint32_t* tkeys, const uint32_t* ids, const float* screen,
                               uint64_t n, uint64_t* out, hipStream_t s);

// Rasterization (gs_raster.hip).
hipError_t launch_raster_fwd(int C, int W, int H, const float* screen, const uint32_t* ids,
                             const int64_t* toff, const uint32_t* order, const float* background,
                             float* out_rgb, float* out_T, float* out_depth, int32_t* last_ids,
                             hipStream_t s);
hipError_t launch_raster_bwd(int C, int W, int H, const float* screen, const uint32_t* ids,
                             const int64_t* toff, const uint32_t* order, const float* background,
                             const float* out_T, const int32_t* last_ids, const float* v_rgb,
                             const float* v_T, const float* v_depth, float* v_screen,
                             float* v_background, hipStream_t s);

// First slot of every camera from the group scan (gs_project.hip).
hipError_t launch_cam_offsets(const uint32_t* wg_scan, int64_t groups_per_cam, int C,
                              const uint64_t* total, int64_t* out, hipStream_t s);

}  // namespace gs
