// Phase arena planner ([VRAM] "Phase Arena"): buffers whose lives never
// overlap share bytes of one allocation. The pages' example is the pair
// of intersection sort buffers, which live only inside the intersection
// phase, and the screen-row gradients, which exist only from the
// rasterize backward on. Each buffer of one step is declared with the
// first and last phase in which its bytes are valid; a packing pass places
// every buffer at the lowest offset that overlaps no placed buffer whose
// phases intersect its own. Without aliasing every buffer gets bytes of its
// own, which is the same layout a caller gets with separate allocations.
// Host arithmetic only: no device work, no allocation.
#include <algorithm>

#include "gs_internal.h"

using gs::kMaskGroup;
using gs::kTile;

namespace {

constexpr uint64_t kArenaAlign = 256;

struct Slot {
  uint64_t bytes;
  int first, last;  // phases 0 project, 1 intersect, 2 raster fwd, 3 raster bwd, 4 project bwd
};

uint64_t up(uint64_t x) { return (x + kArenaAlign - 1) & ~(kArenaAlign - 1); }

}  // namespace

extern "C" int gs_arena_plan(int64_t N, int32_t C, int32_t W, int32_t H, int64_t nnz,
                             int64_t n_isects, uint64_t isect_ws_bytes, int32_t alias,
                             uint64_t* offsets, uint64_t* sizes, uint64_t* arena_bytes) {
  if (N < 0 || C < 1 || W < 1 || H < 1 || W > 65535 || H > 65535 || nnz < 0 || n_isects < 0 ||
      !offsets || !sizes || !arena_bytes)
    return GS_E_INVALID;
  const uint64_t Np = uint64_t(gs_pad_n(N));
  const uint64_t pairs = uint64_t(C) * Np;
  const uint64_t tiles = uint64_t(C) * uint64_t((W + kTile - 1) / kTile) *
                         uint64_t((H + kTile - 1) / kTile);
  const uint64_t px = uint64_t(C) * uint64_t(W) * uint64_t(H);
  const uint64_t n = uint64_t(nnz), I = uint64_t(n_isects);
  Slot s[GS_ARENA_SLOTS];
  s[GS_SLOT_MASK] = {pairs / 8, 0, 4};
  s[GS_SLOT_WG_COUNT] = {4 * (pairs / kMaskGroup), 0, 0};
  s[GS_SLOT_WG_SCAN] = {4 * (pairs / kMaskGroup), 0, 4};
  s[GS_SLOT_PROJECT_WS] = {gs_project_workspace_bytes(N, C), 0, 0};
  s[GS_SLOT_SCREEN] = {40 * n, 0, 3};
  s[GS_SLOT_AABB16] = {8 * n, 0, 1};
  s[GS_SLOT_ISECT_WS] = {isect_ws_bytes ? isect_ws_bytes
                                        : gs_intersect_workspace_bytes(C, W, H, nnz, n_isects),
                         1, 1};
  s[GS_SLOT_FLATTEN_IDS] = {4 * I, 1, 3};
  s[GS_SLOT_TILE_OFFSETS] = {8 * (tiles + 1), 1, 3};
  s[GS_SLOT_TILE_ORDER] = {4 * tiles, 1, 3};
  s[GS_SLOT_OUT_RGB] = {12 * px, 2, 4};
  s[GS_SLOT_OUT_T] = {4 * px, 2, 4};
  s[GS_SLOT_LAST_IDS] = {4 * px, 2, 3};
  s[GS_SLOT_V_SCREEN] = {40 * n, 3, 4};
  for (int i = 0; i < GS_ARENA_SLOTS; ++i) sizes[i] = s[i].bytes;

  uint64_t total = 0;
  if (!alias) {
    for (int i = 0; i < GS_ARENA_SLOTS; ++i) {
      offsets[i] = total;
      total += up(s[i].bytes);
    }
    *arena_bytes = total;
    return GS_OK;
  }
  // largest first; each at the lowest offset clear of every placed buffer
  // that is alive in one of its phases
  int order[GS_ARENA_SLOTS];
  for (int i = 0; i < GS_ARENA_SLOTS; ++i) order[i] = i;
  std::stable_sort(order, order + GS_ARENA_SLOTS,
                   [&](int a, int b) { return s[a].bytes > s[b].bytes; });
  bool placed[GS_ARENA_SLOTS] = {};
  for (int k = 0; k < GS_ARENA_SLOTS; ++k) {
    const int i = order[k];
    const uint64_t len = up(s[i].bytes);
    uint64_t off = 0;
    for (bool moved = true; moved;) {
      moved = false;
      for (int j = 0; j < GS_ARENA_SLOTS; ++j) {
        if (!placed[j] || s[j].last < s[i].first || s[i].last < s[j].first) continue;
        const uint64_t lo = offsets[j], hi = offsets[j] + up(s[j].bytes);
        if (off < hi && lo < off + len) {
          off = hi;
          moved = true;
        }
      }
    }
    offsets[i] = off;
    placed[i] = true;
    total = std::max(total, off + len);
  }
  *arena_bytes = total;
  return GS_OK;
}
