/*
 * gs.h -- C ABI of libgs, a differentiable 16x16-tile Gaussian rasterizer
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages on a 3D Gaussian Splatting trainer):
 *  [VRAM]  "Spirula Studio VRAM deep dive: the splat x img category and
 *          bitmask compaction, training ten million Gaussians in 8 GB"
 *  [BWD]   "How Spirula Studio's backward pass sends image gradients back
 *          to every Gaussian"
 *  [PROF]  "3D Gaussian Splatting profiling guide: reading every step of
 *          Spirula Studio with SS_PROFILE=1"
 *  [GSPLAT] a deployment blog on the gsplat CUDA library, section 2.3
 *          (a C API over caller-owned device pointers loaded by ctypes).
 *
 * Conventions shared by every entry point
 *  - Every pointer is a DEVICE pointer unless its comment says (host).
 *  - Every buffer is owned by the caller; the library allocates no device
 *    memory and keeps no device state between calls ([GSPLAT] 2.3: memory
 *    lifetimes belong to the caller).
 *  - `stream` is a hipStream_t passed as void*; all work is enqueued on it.
 *    gs_project and gs_intersect block the host on an event recorded
 *    after the copy of a 64-bit total, for the host-side check of
 *    [VRAM] "The 4 GiB rule and the 2^31 limit"; work that does not depend
 *    on that total is queued before the wait, and work sized by it after.
 *    The other calls return without waiting. The stream must belong to
 *    the current device. Each calling thread keeps a few page-locked
 *    host words and one event per device for these reads (held until the
 *    process ends).
 *  - Inputs are fp32, structure-of-arrays:
 *      means[N][3], quats[N][4] as (w,x,y,z) (need not be unit length),
 *      log_scales[N][3], opacity_logits[N], sh[N][K][3] with
 *      K = (sh_degree+1)^2 ordered l = 0..deg, m = -l..l,
 *      viewmats[C][4][4] row-major world->camera (x right, y down,
 *      z forward), Ks[C][3][3] pinhole intrinsics. All C cameras share one
 *      W x H image size.
 *  - Pair index p = c * N_pad + g (camera-major), N_pad = N rounded up to
 *    GS_MASK_GROUP. A "slot" is the rank of a visible pair in p order.
 *  - A screen row ([VRAM] per-element cost table, proj.screen, 40 bytes) is
 *    10 floats: u, v, conic_a, conic_b, conic_c, opacity, depth z, r, g, b.
 *  - Returns GS_OK (0) or a negative status; no call aborts or prints.
 *    On an error nothing is written past any stated capacity; what lies
 *    within a capacity is then unspecified.
 */
#ifndef GS_H
#define GS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  GS_OK = 0,
  GS_E_INVALID = -1,   /* null required pointer or out-of-range argument */
  GS_E_CAPACITY = -2,  /* an output is too small; required count returned */
  GS_E_WORKSPACE = -3, /* workspace too small; required bytes returned */
  GS_E_OVERFLOW = -4,  /* a count exceeds the width of its storage type */
  GS_E_HIP = -5,       /* HIP runtime error (launch, copy, sync) */
  GS_E_DEVICE = -6     /* a kernel reported an internal error */
};

#define GS_TILE 16        /* tiles are 16 x 16 pixels */
#define GS_MASK_GROUP 128 /* pairs per visibility work-group ([VRAM]
                             "Bitmask compaction": one popcount per
                             128-lane work-group) */
#define GS_ROW 10         /* floats per screen row */

/* Text of a status code (static storage). */
const char* gs_status_str(int status);
/* Library version, major * 10000 + minor * 100 + patch. */
int gs_version(void);

/* ---------------------------------------------------------------------
 * Host-side checks (host only, no GPU work).
 *
 * gs_readback_status -- the decision gs_project applies to the words it
 * reads back ([VRAM] "The 4 GiB rule and the 2^31 limit": an exact total is
 * checked on the host against the storage it must fit before it is
 * trusted). device_flag is the error word of the call's kernels: a
 * look-back scan whose bounded wait for a predecessor timed out sets it,
 * and the total and slots are then wrong. Returns GS_E_DEVICE if
 * device_flag != 0 (checked first, since the count is then unreliable),
 * GS_E_OVERFLOW if count < 0 or count >= count_limit, GS_E_CAPACITY if
 * count > capacity, else GS_OK. gs_intersect maps the same flag of its
 * emit scan to GS_E_DEVICE.
 *
 * gs_tile_offsets_check -- validates (host) tile_offsets[n_tiles + 1]
 * before it is handed to the raster calls: GS_E_INVALID if
 * tile_offsets[0] != 0 or a range is negative (null pointer included),
 * GS_E_OVERFLOW if any tile's list holds 2^31 entries or more (the raster
 * calls index a tile's list with the 32-bit local ids of last_ids;
 * [VRAM] "The 4 GiB rule and the 2^31 limit" is about exactly such a
 * silent wrap), else GS_OK. gs_intersect's output always passes: a pair
 * meets each tile of its camera at most once, so a list is no longer than
 * its camera's pair count, which gs_intersect checks below 2^31.
 * ------------------------------------------------------------------- */
int gs_readback_status(int32_t device_flag, int64_t count, int64_t count_limit,
                       int64_t capacity);
int gs_tile_offsets_check(const int64_t* tile_offsets, uint64_t n_tiles);

/* ---------------------------------------------------------------------
 * Buffer sizes (host only, no GPU work).
 *
 * gs_pad_n: N_pad = ceil(N / 128) * 128.
 * Sizes for gs_project, counted in elements:
 *   mask      uint64[C * N_pad / 64]    (bit p%64 of word p/64 = pair p)
 *   wg_count  uint32[C * N_pad / 128]   (popcount of each 128-pair group)
 *   wg_scan   uint32[C * N_pad / 128]   (its exclusive prefix sum)
 * These are the [VRAM] cost-table rows proj.mask (C*N/8 bytes) and
 * proj.block_count / proj.scan (C*N/32 bytes each).
 * gs_project_workspace_bytes: device scratch needed by gs_project.
 * gs_intersect_workspace_bytes: device scratch needed by gs_intersect for
 * nnz visible pairs producing n_isects (tile, pair) intersections.
 * ------------------------------------------------------------------- */
int64_t gs_pad_n(int64_t N);
uint64_t gs_project_workspace_bytes(int64_t N, int32_t C);
uint64_t gs_intersect_workspace_bytes(int32_t C, int32_t W, int32_t H,
                                      int64_t nnz, int64_t n_isects);

/* ---------------------------------------------------------------------
 * gs_project -- packed projection of C cameras x N Gaussians.
 * [VRAM] "Bitmask compaction" and "16-bit packed AABB".
 *
 * Pass 1 tests every (camera, Gaussian) pair for visibility (depth beyond
 * the near plane and a 3-sigma screen box that overlaps the image), ORs
 * the predicate into bit-words with wavefront ballots and writes one
 * popcount per 128-pair group. A scan of those counts gives each group's
 * first slot and nnz. Pass 2 re-projects only visible pairs and writes
 * screen row `slot` = scan of earlier groups + set bits before the pair:
 *   screen[nnz][10] fp32: u, v, conic (a,b,c) of the inverse 2D covariance
 *     (EWA projection plus 0.3 px blur), sigmoid(opacity_logit), camera
 *     depth z, RGB from the SH coefficients toward the camera centre
 *     (max(0, sum + 0.5)).
 *   aabb16[nnz][2] uint32: the 3-sigma box clamped to the image on a
 *     uniform 65535-step grid over [0, W] x [0, H], min edges rounded
 *     down and max edges rounded up: word0 = qx0 | qy0 << 16,
 *     word1 = qx1 | qy1 << 16.
 *
 * Outputs: mask, wg_count, wg_scan (sizes above); screen and aabb16 with
 * room for screen_capacity rows; (host) *nnz_out; (host, nullable)
 * cam_offsets_out[C+1]: first slot of each camera, cam_offsets_out[C]=nnz.
 * workspace: device scratch of gs_project_workspace_bytes(N, C) bytes.
 * Errors: GS_E_INVALID for N < 0, C < 1, W or H outside [1, 65535],
 * sh_degree outside [0, 3], or a null required pointer. GS_E_DEVICE when
 * the scan of the group counts reports a timed-out wait (the host reads
 * its error word with nnz; see gs_readback_status).
 * GS_E_CAPACITY when nnz > screen_capacity: *nnz_out, cam_offsets_out and
 * mask, wg_count, wg_scan are valid; rows at slots below the capacity may
 * have been written, nothing at or past it (the compaction runs before
 * the host sees nnz and skips slots >= screen_capacity). GS_E_OVERFLOW
 * when nnz >= 2^31 (slots are 31-bit).
 * ------------------------------------------------------------------- */
int gs_project(void* stream, int64_t N, int32_t C, int32_t W, int32_t H,
               int32_t sh_degree, const float* means, const float* quats,
               const float* log_scales, const float* opacity_logits,
               const float* sh, const float* viewmats, const float* Ks,
               uint64_t* mask, uint32_t* wg_count, uint32_t* wg_scan,
               float* screen, uint32_t* aabb16, int64_t screen_capacity,
               void* workspace, uint64_t workspace_bytes,
               int64_t* nnz_out, int64_t* cam_offsets_out);

/* ---------------------------------------------------------------------
 * gs_project_noalloc -- gs_project for callers that cannot allocate
 * memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.
 *
 * Same arguments, results and errors as gs_project, without the workspace:
 * the projection workspace lives in a fixed 64 KiB device array inside the
 * library (one per device, held until the process ends), and the totals
 * are read back into host stack words, so the call allocates nothing
 * (no device, page-locked or heap memory). Limits: C <= 256 and
 * gs_project_workspace_bytes(N, C) <= 65536, which holds up to about
 * 4e9 camera-Gaussian pairs; past them it returns GS_E_WORKSPACE before
 * any device work. It blocks the host until its kernels finish (the
 * readback is not overlapped with the compaction as in gs_project). Every
 * call on one device shares that array: calls that overlap on a device
 * (two host threads, or two streams) race and must be serialized by the
 * caller. Each call clears what must start at zero.
 * ------------------------------------------------------------------- */
int gs_project_noalloc(void* stream, int64_t N, int32_t C, int32_t W, int32_t H,
                       int32_t sh_degree, const float* means, const float* quats,
                       const float* log_scales, const float* opacity_logits,
                       const float* sh, const float* viewmats, const float* Ks,
                       uint64_t* mask, uint32_t* wg_count, uint32_t* wg_scan,
                       float* screen, uint32_t* aabb16, int64_t screen_capacity,
                       int64_t* nnz_out, int64_t* cam_offsets_out);

/* ---------------------------------------------------------------------
 * gs_intersect -- (tile, pair) intersections, sorted per tile by depth.
 * [VRAM] "The 4 GiB rule and the 2^31 limit" (exact 64-bit total checked
 * on the host before anything is sized by it; 64-bit addressing for every
 * buffer sized by nnz or n_isects), the cost-table row isect.ids_a/b
 * (keys (tile_id << 32) | depth); [BWD] section 4 (tile offsets and the
 * flattened intersection list kept for the backward).
 *
 * A pair's tile rectangle comes from its aabb16 words with integer
 * arithmetic: tx0 = floor(qx0*W / (16*65535)), tx1 = ceil(qx1*W /
 * (16*65535)) (exclusive), same for y with H. Its key for tile
 * (tx, ty) of camera c is (c*T + ty*ceil(W/16) + tx) << 32 | bits(z) with
 * T = ceil(W/16)*ceil(H/16) and z the fp32 depth of its screen row. The
 * result equals a stable sort of those 64-bit keys emitted slot by slot:
 * within a tile, entries are ordered by depth, then by slot.
 *
 * Inputs: screen[nnz][10], aabb16[nnz][2] from gs_project, and (host)
 * cam_offsets[C+1] (first slot of every camera).
 * Outputs: flatten_ids[n_isects] (uint32 slot of every sorted entry,
 * capacity isect_capacity, 16-byte aligned); tile_offsets[C*T+1] int64 (entries of global
 * tile t are flatten_ids[tile_offsets[t] .. tile_offsets[t+1]));
 * sorted_keys[n_isects] (nullable: the sorted 64-bit keys);
 * tile_order[C*T] (nullable: every global tile id once, ordered by
 * decreasing entry count, ties by tile id -- a launch order for the
 * raster calls so that the longest tiles start first);
 * (host) *n_isects_out; (host) *workspace_needed_out.
 * Errors: GS_E_INVALID as for gs_project or nnz < 0;
 * GS_E_OVERFLOW if nnz >= 2^31; GS_E_CAPACITY if n_isects >
 * isect_capacity (flatten_ids, tile_offsets, sorted_keys and tile_order
 * are then not written); GS_E_OVERFLOW also if one camera holds 2^31
 * pairs or more (its tiles' lists could then pass the 32-bit local ids of
 * the raster calls); GS_E_DEVICE if the scan of the emit's per-block
 * counts reports a timed-out wait (the host reads that flag after queuing
 * every kernel of the call, so this call waits twice: once for the total,
 * once for the flag); GS_E_WORKSPACE if workspace_bytes is short (the
 * bytes needed are returned; before the count is known this is the lower
 * bound for counting, after it the full amount). Call again after growing.
 * ------------------------------------------------------------------- */
int gs_intersect(void* stream, int32_t C, int32_t W, int32_t H, int64_t nnz,
                 const float* screen, const uint32_t* aabb16,
                 const int64_t* cam_offsets, void* workspace,
                 uint64_t workspace_bytes, uint32_t* flatten_ids,
                 int64_t isect_capacity, int64_t* tile_offsets,
                 uint64_t* sorted_keys, uint32_t* tile_order,
                 int64_t* n_isects_out, uint64_t* workspace_needed_out);

/* ---------------------------------------------------------------------
 * gs_rasterize_fwd -- per-tile front-to-back alpha compositing.
 * [PROF] kernel rasterize_fwd; [BWD] section 4 (what the forward saves).
 *
 * For every pixel (centre (j+0.5, i+0.5)) of camera c, over the entries of
 * its tile in sorted order: d = (u - px, v - py),
 * sigma = (a dx^2 + c dy^2)/2 + b dx dy (>= 0: the conic is positive
 * definite), alpha = min(0.99, o exp(-sigma)); entries with
 * alpha < 1/255 are skipped; if T*(1-alpha) < 1e-4 the walk stops before
 * that entry; otherwise rgb += colour*alpha*T and T *= 1-alpha.
 * tile_order (nullable) is the order in which tiles are launched (from
 * gs_intersect; null = tile id order); it changes no result.
 * background (nullable) is one RGB colour per camera, background[C][3],
 * blended in as rgb + T_final * background[c] (null = no blend).
 * Outputs (all C x H x W, row-major): out_rgb[C][H][W][3] (premultiplied,
 * plus the background term), out_T[C][H][W] final transmittance,
 * out_depth[C][H][W] (nullable) the depth composited like a colour
 * channel, sum of z*alpha*T with z the row's depth (not normalised),
 * last_ids[C][H][W] local index (within the tile's list) of the last
 * composited entry, -1 if none. [BWD] sections 2-3 name the depth image
 * among the rendered outputs and the background blend among the image
 * corrections. Errors: GS_E_INVALID.
 * ------------------------------------------------------------------- */
int gs_rasterize_fwd(void* stream, int32_t C, int32_t W, int32_t H,
                     const float* screen, const uint32_t* flatten_ids,
                     const int64_t* tile_offsets, const uint32_t* tile_order,
                     const float* background, float* out_rgb, float* out_T,
                     float* out_depth, int32_t* last_ids);

/* ---------------------------------------------------------------------
 * gs_rasterize_bwd -- gradient of L = <v_rgb, out_rgb> + <v_T, out_T>
 * + <v_depth, out_depth> with respect to every screen row. [BWD] section 4
 * (rasterize_to_pixels_3dgs_bwd: the pixel gradient is split over the
 * Gaussians on that pixel in proportion to their alpha contribution, in
 * blend order, and summed with atomics into the fp32 screen gradients)
 * and sections 2-3 (the depth image's gradient v_render_depth; the
 * background hook adds its transmittance gradient into v_render_Ts).
 *
 * Walks each pixel's entries back to front from last_ids, recovering the
 * transmittance before entry i as T_{i+1} / (1 - alpha_i). Writes
 * v_screen[nnz][10] fp32 (zeroed by this call first; the depth column is
 * the depth image's gradient, 0 when v_depth is null). v_T and v_depth may
 * be null (taken as zero). background: the forward's (nullable); with it,
 * v_T is taken as v_T + v_rgb . background[c]. v_background[C][3]
 * (nullable) receives dL/dbackground = sum over each camera's pixels of
 * v_rgb * out_T (overwritten). Entries whose alpha hit the 0.99 clamp get
 * no opacity or position/conic gradient. tile_order as for
 * gs_rasterize_fwd. Summation order is not fixed (float atomics), so
 * results vary in the last bits run to run.
 * ------------------------------------------------------------------- */
int gs_rasterize_bwd(void* stream, int32_t C, int32_t W, int32_t H,
                     int64_t nnz, const float* screen,
                     const uint32_t* flatten_ids, const int64_t* tile_offsets,
                     const uint32_t* tile_order, const float* background,
                     const float* out_T, const int32_t* last_ids,
                     const float* v_rgb, const float* v_T, const float* v_depth,
                     float* v_screen, float* v_background);

/* ---------------------------------------------------------------------
 * gs_project_bwd -- screen-row gradients to parameter gradients.
 * [BWD] section 5 (projection_3dgs_backward: the chain rule through the
 * intrinsics and extrinsics; gradients are fp32) and section 6 (only the
 * first sub-batch zeroes the accumulators).
 *
 * For each Gaussian, over every camera whose mask bit is set, reads
 * v_screen[slot] (slot from wg_scan and the mask, as gs_project assigned
 * it) and applies the exact chain rule of the projection: means (camera
 * transform, the Jacobian's dependence on the camera-space point and the
 * SH view direction, and the row's depth z, whose gradient is the depth
 * column of v_screen), raw quaternions (through normalisation), log-scales,
 * opacity logits and SH coefficients (zero where the colour clamp at 0 is
 * active). Nothing flows through the radius, box or visibility test.
 * Outputs v_means[N][3], v_quats[N][4], v_log_scales[N][3],
 * v_opacity_logits[N], v_sh[N][K][3]: overwritten when accumulate == 0
 * (zeros for Gaussians visible nowhere), added to when accumulate != 0.
 * quats, v_quats and v_sh must be 16-byte aligned (GS_E_INVALID).
 * ------------------------------------------------------------------- */
int gs_project_bwd(void* stream, int64_t N, int32_t C, int32_t W, int32_t H,
                   int32_t sh_degree, const float* means, const float* quats,
                   const float* log_scales, const float* opacity_logits,
                   const float* sh, const float* viewmats, const float* Ks,
                   const uint64_t* mask, const uint32_t* wg_scan,
                   const float* v_screen, float* v_means, float* v_quats,
                   float* v_log_scales, float* v_opacity_logits, float* v_sh,
                   int32_t accumulate);

/* ---------------------------------------------------------------------
 * gs_project_bwd_adam -- projection backward fused with one Adam step.
 * [BWD] section 6 (the fused projection backward + optimizer: the
 * world-space gradients are folded straight into the Adam optimizer and
 * no fp32 gradient buffer is allocated).
 *
 * Computes exactly the gradients gs_project_bwd would write (same inputs,
 * accumulate = 0) and, instead of writing them, applies one bias-corrected
 * Adam step to every element of every Gaussian, a zero gradient included:
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2;
 *   p -= lr * (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps).
 * means, quats, log_scales, opacity_logits and sh are read for the
 * backward and then updated in place. adam_m[5] and adam_v[5] (host
 * arrays of device pointers, in the order means, quats, log_scales,
 * opacity_logits, sh, each shaped like its parameter) are the moments,
 * updated in place. lr[6] (host): learning rates of means, quats,
 * log_scales, opacity_logits, SH coefficient 0 (DC colour) and the higher
 * SH coefficients. step >= 1 is the step number after this update.
 * Each Gaussian is touched by one lane only. Errors: GS_E_INVALID (also
 * for beta outside [0, 1), eps <= 0 or step < 1).
 * ------------------------------------------------------------------- */
int gs_project_bwd_adam(void* stream, int64_t N, int32_t C, int32_t W, int32_t H,
                        int32_t sh_degree, float* means, float* quats,
                        float* log_scales, float* opacity_logits, float* sh,
                        const float* viewmats, const float* Ks,
                        const uint64_t* mask, const uint32_t* wg_scan,
                        const float* v_screen, float* const* adam_m,
                        float* const* adam_v, const float* lr, float beta1,
                        float beta2, float eps, int32_t step);

/* ---------------------------------------------------------------------
 * gs_arena_plan -- one allocation for every buffer of a step, with the
 * buffers whose lives never overlap sharing bytes ([VRAM] "Phase Arena":
 * the intersection sort buffers live only inside the intersection phase
 * and the screen-row gradients only from the rasterize backward on, so
 * they can share one allocation; the arena then costs its largest phase,
 * not the sum; SS_POOL_ALIAS=0 there turns the sharing off).
 *
 * Host arithmetic only. For a step with N Gaussians, C cameras of W x H,
 * capacities nnz (visible pairs) and n_isects (intersections), and an
 * intersection workspace of isect_ws_bytes (0 = the bound
 * gs_intersect_workspace_bytes(C, W, H, nnz, n_isects), which holds for any
 * scene of those capacities; a caller that has seen the bytes gs_intersect
 * reports as needed may pass those, with a margin, instead), writes for
 * each slot below (host arrays of GS_ARENA_SLOTS) its byte offset in the
 * arena (256-byte aligned) and its size, and (host) *arena_bytes. Phases:
 * 0 gs_project, 1 gs_intersect, 2 gs_rasterize_fwd, 3 gs_rasterize_bwd,
 * 4 gs_project_bwd; a slot's bytes are valid from its first to its last
 * phase, and another slot may reuse them outside that range:
 *   MASK 0-4, WG_COUNT 0, WG_SCAN 0-4, PROJECT_WS 0, SCREEN 0-3,
 *   AABB16 0-1, ISECT_WS 1, FLATTEN_IDS 1-3, TILE_OFFSETS 1-3,
 *   TILE_ORDER 1-3, OUT_RGB 2-4, OUT_T 2-4, LAST_IDS 2-3, V_SCREEN 3-4.
 * alias = 0 gives every slot bytes of its own. Calls on one stream keep
 * the phases apart; parameters, gradients and optimizer state are not in
 * the arena. Errors: GS_E_INVALID.
 * ------------------------------------------------------------------- */
#define GS_ARENA_SLOTS 14
#define GS_SLOT_MASK 0
#define GS_SLOT_WG_COUNT 1
#define GS_SLOT_WG_SCAN 2
#define GS_SLOT_PROJECT_WS 3
#define GS_SLOT_SCREEN 4
#define GS_SLOT_AABB16 5
#define GS_SLOT_ISECT_WS 6
#define GS_SLOT_FLATTEN_IDS 7
#define GS_SLOT_TILE_OFFSETS 8
#define GS_SLOT_TILE_ORDER 9
#define GS_SLOT_OUT_RGB 10
#define GS_SLOT_OUT_T 11
#define GS_SLOT_LAST_IDS 12
#define GS_SLOT_V_SCREEN 13
int gs_arena_plan(int64_t N, int32_t C, int32_t W, int32_t H, int64_t nnz,
                  int64_t n_isects, uint64_t isect_ws_bytes, int32_t alias,
                  uint64_t* offsets, uint64_t* sizes, uint64_t* arena_bytes);

/* ---------------------------------------------------------------------
 * Per-kernel timing (opt-in; a HIP event pair around each launch of a
 * kernel whose name contains `filter`, on the stream it runs on).
 * [PROF] sections 3-4 describe the trainer's own per-kernel GPU timing
 * report; this is the library's counterpart for benchmarks.
 *
 * gs_profile_enable: start recording (filter NULL or "" = every kernel).
 * gs_profile_disable: stop recording (recorded events are kept).
 * gs_profile_reset: wait for and release every recorded event.
 * gs_profile_query: for the kernel named exactly `kernel` (e.g.
 *   "k_raster_bwd"), wait for its recorded launches and return their
 *   count and summed duration in milliseconds (host out-params).
 * Kernel names: k_project_mask, k_scan, k_cam_offsets, k_project_compact,
 * k_fill_u32, k_isect_prep, k_radix_count, k_radix_scatter, k_emit_count,
 * k_emit_write, k_tile_ranges, k_row_chunks, k_row_count, k_row_colscan,
 * k_row_expand, k_tile_order_keys, k_tile_order_rank, k_compose_keys,
 * k_raster_fwd, k_raster_bwd, k_project_bwd, k_project_bwd_adam.
 * Recording adds host overhead per launch
 * and is not meant to stay on in production.
 * ------------------------------------------------------------------- */
int gs_profile_enable(const char* filter);
/* gs_valu_probe: a throughput probe of the fp32 vector unit, for sizing the
 * raster kernels' roofline on the machine at hand (not part of a step).
 * Launches `blocks` blocks of 256 lanes on `stream`; each lane runs
 * `iters` rounds of eight independent chains of one instruction: kind 0 a
 * plain fp32 fused multiply-add, kind 1 the hardware base-2 exponential.
 * out[blocks * 256] (device) receives each lane's sum. Work per launch:
 * blocks * 256 * iters * 8 instructions (an FMA counts 2 flops). The
 * caller times it. Errors: GS_E_INVALID, GS_E_HIP. */
int gs_valu_probe(void* stream, int32_t kind, int32_t blocks, int32_t iters, float* out);
int gs_profile_disable(void);
int gs_profile_reset(void);
int gs_profile_query(const char* kernel, int64_t* launches, double* total_ms);

/* ---------------------------------------------------------------------
 * Launch-shape overrides for sweeps (environment; unset or any other
 * value keeps the library's choice; results are the same either way):
 *   GS_RASTER_PPT_FWD, GS_RASTER_PPT_BWD = 1, 2 or 4 (read at each
 *     raster call): pixels per lane of the raster kernels (4, 2 or 1
 *     waves per tile). By default the forward takes 1 below 2,048 tiles,
 *     2 below 16,384, else 4; the backward 1 below 512 tiles, 2 below
 *     2,048, else 4.
 *   GS_EXPAND_GROUP = 16 or 32 (read at each gs_intersect call): entries
 *     per group the list expansion writes at once (64 or 128 bytes); by
 *     default 32 where a chunk's run per tile averages at least 512
 *     entries.
 * ------------------------------------------------------------------- */

#ifdef __cplusplus
}
#endif

#endif /* GS_H */
