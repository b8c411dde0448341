"""Benchmark: fwd+bwd rasterizer steps/s on one MI355X.

A step is one pass of the whole path on one seeded synthetic scene:
gs_project -> gs_intersect -> gs_rasterize_fwd -> gs_rasterize_bwd ->
gs_project_bwd, with fixed upstream image gradients and every input
resident in HBM before the timed region starts. Prints one JSON line.

The headline workload is the large five-camera scene (15M Gaussians, SH
degree 3, 5 cameras of 1297x840: 75M camera-Gaussian pairs), the stand-in
for the pages' own scene ([VRAM] "Three key numbers"). The same line
carries, as extra keys, the high-resolution scene (13M Gaussians at
7680x7680, about 4.8e9 intersections), run after the headline scene's
buffers are freed.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4]
       [--extra-config 5 | --no-extra] [--no-cpu-baseline]
       [--calibrate-copy MIB] [--calibrate-valu]

--calibrate-copy runs only a plain device-to-device copy of MIB MiB (for
scaling the FETCH_SIZE / WRITE_SIZE hardware counters to bytes).
--calibrate-valu runs only the library's fp32 FMA and exp throughput
loops and prints the measured rates.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
# ALU peak for the raster kernels: MI355X's published fp32 vector rate,
# 157.3 TFLOP/s = 256 CUs x 4 SIMDs x 32 lanes x 2 (FMA) x 2.4 GHz.
# `--calibrate-valu` measures what plain (unpacked) fp32 FMAs and exps
# reach on the box with the library's own throughput loops.
ALU_PEAK_TFLOPS = 157.3
# What plain fp32 FMAs reach on the chip (`--calibrate-valu`: 37.4e12
# lane-ops/s, a wave64 VALU instruction every 4 clocks per SIMD), the
# ceiling for code without packed fp32 instructions.
MEASURED_FMA_TFLOPS = 74.9
CSRC = os.path.join(ROOT, "gaussian_splatting_differentiable_project_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

KERNELS = ["k_project_mask", "k_scan", "k_cam_offsets", "k_project_compact", "k_fill_u32",
           "k_isect_prep", "k_radix_count", "k_radix_scatter", "k_emit_count", "k_emit_write",
           "k_tile_ranges", "k_row_chunks", "k_row_count", "k_row_colscan", "k_row_expand",
           "k_tile_order_keys", "k_tile_order_rank", "k_raster_fwd", "k_raster_bwd", "k_project_bwd",
           "k_project_bwd_adam"]
KERNEL_SOURCE = {"k_raster_fwd": "gs_raster.hip", "k_raster_bwd": "gs_raster.hip",
                 "k_project_mask": "gs_project.hip", "k_project_compact": "gs_project.hip",
                 "k_project_bwd": "gs_project_bwd.hip", "k_radix_scatter": "gs_sort.hip",
                 "k_emit_write": "gs_intersect.hip", "k_row_expand": "gs_intersect.hip"}

# Flops of one (pixel, entry) evaluation in the raster kernels: the alpha
# test every evaluation needs (dx, dy, three products, the quadratic form,
# the exponent, the clamp: 14), plus the compositing (forward: 9) or the
# gradient terms (backward: 35) of an entry that is composited. The
# method's evaluations are those up to each pixel's last composited entry,
# sum over pixels of (last_id + 1); each is counted with the composited
# cost, an upper bound (entries skipped below 1/255 cost only the test).
FLOPS_EVAL = 14
FLOPS_FWD_COMPOSITE = 9
FLOPS_BWD_COMPOSITE = 35


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--extra-config", type=int, default=5,
                    help="a second scene reported as extra keys of the same line "
                         "(train mode, default run only)")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--calibrate-valu", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle's raster sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    ap.add_argument("--adam", action="store_true",
                    help="train mode: fold the projection backward into one Adam step "
                         "(gs_project_bwd_adam) instead of writing gradients")
    ap.add_argument("--arena", action="store_true",
                    help="train mode: carve every per-step buffer from one phase arena "
                         "(GS_POOL_ALIAS=0 turns the aliasing off)")
    ap.add_argument("--mode", choices=("train", "render"), default="train",
                    help="train: the whole fwd+bwd step (the headline metric); render: "
                         "projection, intersection and forward only, in frames/s")
    return ap.parse_args()


def source_sha(kernel: str) -> str | None:
    f = KERNEL_SOURCE.get(kernel)
    if f is None:
        return None
    h = hashlib.sha256()
    for name in (f, "gs_common.h", "gs_projmath.h", "gs_internal.h"):
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def _bits(n_values: int) -> int:
    return max(0, int(n_values - 1).bit_length())


def _emit_digit_bits(bits: int) -> int:
    total = 1 if bits <= 8 else (bits + 7) // 8
    return max(1, (bits + total - 1) // total)


def sort_model(spec, aabb16, n_isects):
    """How the library sorts the entries by tile for this geometry, and the
    elements its passes move: through window segments (the part of a
    pair's tile row inside one window of 64 tiles; the emit's first digit
    and radix passes over the segments, then the expansion writes the
    entries) when the segment key fits 32 bits, else the entries
    themselves sorted by tile id."""
    import torch
    tx = (spec.width + 15) // 16
    ty = (spec.height + 15) // 16
    windows = spec.n_cams * ty * ((tx + 63) // 64)
    rb, xb = _bits(windows), _bits(tx)
    if rb <= 30 and rb + 2 * xb <= 32:
        b = aabb16.to(torch.int64)
        D = 16 * 65535
        x0 = (b[:, 0] & 0xFFFF) * spec.width // D
        y0 = ((b[:, 0] >> 16) & 0xFFFF) * spec.height // D
        x1 = ((b[:, 1] & 0xFFFF) * spec.width + D - 1) // D
        y1 = (((b[:, 1] >> 16) & 0xFFFF) * spec.height + D - 1) // D
        ok = (x1 > x0) & (y1 > y0)
        segs = ((y1 - y0) * (((x1 - 1) >> 6) - (x0 >> 6) + 1)).clamp(min=0)
        S = int(segs[ok].sum().item()) if b.numel() else 0
        b1 = _emit_digit_bits(rb)
        rest = max(0, rb - b1)
        return {"rows": True, "segments": S, "passes": (rest + 7) // 8 if rest else 0,
                "elems": S}
    bits = _bits(spec.n_cams * tx * ty)
    b1 = _emit_digit_bits(bits)
    rest = max(0, bits - b1)
    return {"rows": False, "segments": None, "passes": (rest + 7) // 8 if rest else 0,
            "elems": n_isects}


def order_passes(spec):
    """Radix passes of the heavy-first launch order, as the library chooses
    them: none up to 16,384 tiles (one rank kernel), else two 8-bit passes."""
    n_tiles = spec.n_cams * ((spec.width + 15) // 16) * ((spec.height + 15) // 16)
    return 0 if 0 < n_tiles <= 16384 else 2


def hbm_bytes(kernel, spec, nnz, n_isects, V, sm, depth_passes=4):
    """Algorithmic HBM bytes of one launch of an HBM-bound kernel; sm is
    sort_model()."""
    N, C, K = spec.n, spec.n_cams, spec.K
    Np = ((N + 127) // 128) * 128
    pairs = C * Np
    if kernel == "k_project_mask":   # 40 B of geometry per Gaussian; mask bits + counts
        return 40 * N + pairs / 8 + 4 * pairs / 128
    if kernel == "k_project_compact":  # mask + scan; params + SH of visible; 48 B out per pair
        return pairs / 8 + 4 * pairs / 128 + (44 + 12 * K) * V + 48 * nnz
    if kernel == "k_project_bwd":    # params + SH read and grads written per Gaussian
        return (44 + 12 * K) * (V + N) + 40 * nnz + pairs / 8 + 4 * pairs / 128
    if kernel == "k_project_bwd_adam":  # params, first and second moments read and written
        return 6 * (44 + 12 * K) * N + 40 * nnz + pairs / 8 + 4 * pairs / 128
    if kernel == "k_radix_scatter":  # mean over the step's passes: 8 B read + 8 B written per key
        tiles = C * ((spec.width + 15) // 16) * ((spec.height + 15) // 16)
        op = order_passes(spec)
        return (16 * (depth_passes * nnz + sm["passes"] * sm["elems"] + op * tiles)
                / (depth_passes + sm["passes"] + op))
    if kernel == "k_emit_write":     # order + rectangle per pair; 8 B per entry or segment
        return 12 * nnz + 8 * sm["elems"]
    if kernel == "k_row_expand":     # 8 B per segment read, 4 B per entry written
        return 8 * sm["segments"] + 4 * n_isects if sm["rows"] else None
    return None


_T0 = time.perf_counter()


def note(msg: str) -> None:
    """A progress line on stderr (stdout carries only the JSON line)."""
    print(f"[bench {time.perf_counter() - _T0:6.1f}s] {msg}", file=sys.stderr, flush=True)


def raster_evals(last_ids):
    """The method's raster evaluations: every pixel walks its entries up to
    and including its last composited one, sum over pixels of (last + 1)."""
    import torch
    return int((last_ids.to(torch.int64) + 1).sum().item())


def host_cores() -> int:
    """Worker processes for the oracle baseline: the host cores this process
    may run on, at most 16 (a one-GPU share of the box)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


# ---- oracle baseline workers (spawned processes; they never touch the GPU)

def _w_init():
    from threadpoolctl import threadpool_limits
    global _LIMIT
    _LIMIT = threadpool_limits(limits=1)   # one BLAS thread per worker process


def _w_noop(x):
    import oracle  # noqa: F401  (warm the import)
    return x


def _w_project(args):
    import oracle
    from oracle.project import screen_rows
    means, quats, ls, logits, sh, vm, K, W, H, deg = args
    pc = oracle.project_camera(means, quats, ls, logits, sh, vm, K, W, H, deg)
    idx = np.flatnonzero(pc["visible"])
    rows = screen_rows(pc, idx).astype(np.float32)
    w0 = (pc["qx0"][idx] | (pc["qy0"][idx] << 16)).astype(np.uint32)
    w1 = (pc["qx1"][idx] | (pc["qy1"][idx] << 16)).astype(np.uint32)
    return idx, rows, np.stack([w0, w1], 1)


def _w_raster(args):
    """Forward and backward of one tile as a one-tile image of its own (the
    rows' centres shifted by the tile origin, a whole number of pixels, so
    every pixel offset is as in the full image); returns its seconds."""
    import oracle
    x0, y0, w, h, rows, vr, vT, bwd = args
    rows = rows.astype(np.float64)
    rows[:, 0] -= x0
    rows[:, 1] -= y0
    n = rows.shape[0]
    ids = np.arange(n, dtype=np.uint32)
    offs = np.array([0, n], np.int64)
    t0 = time.perf_counter()
    oracle.rasterize_fwd(rows, ids, offs, 1, w, h)
    if bwd:
        oracle.rasterize_bwd(rows, ids, offs, 1, w, h, vr[None], vT[None])
    return time.perf_counter() - t0


def _w_project_bwd(args):
    import oracle
    from oracle.project import Projection
    sub, cam, gauss = args
    t0 = time.perf_counter()
    oracle.project_bwd(sub, Projection(cam=cam, gauss=gauss), np.zeros((cam.size, 10)))
    return time.perf_counter() - t0


def cpu_baseline(sc, spec, seconds, render_only=False, isect_sample=4_000_000,
                 pbwd_sample=400_000):
    """The fp64 oracle, unmodified, on the host cores (one worker process
    per core, at most 16), on a bounded sample of the same scene:
    projection of every pair (parallel over Gaussian chunks and cameras);
    intersection and stable sort on a seeded subset of pairs, scaled to all
    entries (one process: the oracle's sort); raster forward + backward on
    seeded random tiles (parallel over tiles), scaled to all tiles;
    projection backward on seeded random visible pairs (parallel), scaled
    to all pairs. Wall-clock seconds per stage, summed."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    from oracle.intersect import intersect as o_intersect, tile_rects_from_aabb16
    rng = np.random.default_rng(0)
    N, C, W, H, deg = sc["N"], sc["C"], sc["W"], sc["H"], sc["sh_degree"]
    tiles_x, tiles_y = (W + 15) // 16, (H + 15) // 16
    T = tiles_x * tiles_y
    cores = host_cores()
    with mp.get_context("spawn").Pool(cores, initializer=_w_init) as pool, \
            threadpool_limits(limits=1):
        pool.map(_w_noop, range(cores))
        note(f"oracle baseline: {cores} worker processes up")
        # projection of every pair
        chunk = 1 << 17
        tasks = [(sc["means"][g0:g0 + chunk], sc["quats"][g0:g0 + chunk],
                  sc["log_scales"][g0:g0 + chunk], sc["opacity_logits"][g0:g0 + chunk],
                  sc["sh"][g0:g0 + chunk], sc["viewmats"][c], sc["Ks"][c], W, H, deg)
                 for c in range(C) for g0 in range(0, N, chunk)]
        t0 = time.perf_counter()
        res = pool.map(_w_project, tasks, chunksize=1)
        t_proj = time.perf_counter() - t0
        note(f"oracle baseline: projection of all pairs {t_proj:.1f} s")
        del tasks
        gidx, cam = [], []
        for k, (idx, _, _) in enumerate(res):
            c, g0 = divmod(k, (N + chunk - 1) // chunk)
            gidx.append(idx + g0 * chunk)
            cam.append(np.full(idx.size, c, np.int64))
        gidx, cam = np.concatenate(gidx), np.concatenate(cam)
        rows = np.concatenate([r[1] for r in res])
        aabb = np.concatenate([r[2] for r in res])
        del res
        nnz = rows.shape[0]
        tx0, ty0, tx1, ty1 = tile_rects_from_aabb16(aabb, W, H)
        counts = (tx1 - tx0) * (ty1 - ty0)
        n_is = int(counts.sum())
        # intersection and sort on a seeded subset of pairs
        perm = rng.permutation(nnz)
        take = np.sort(perm[: int(np.searchsorted(np.cumsum(counts[perm]), isect_sample)) + 1])

        class _Sub:
            pass
        sub = _Sub()
        sub.C, sub.aabb16, sub.cam, sub.z32 = C, aabb[take], cam[take], rows[take, 6]
        n_sub = int(counts[take].sum())
        t0 = time.perf_counter()
        o_intersect(sub, W, H)
        t_isect = (time.perf_counter() - t0) * n_is / max(n_sub, 1)
        note(f"oracle baseline: intersect + sort of {n_sub} entries, scaled {t_isect:.1f} s")
        del sub, perm
        # raster on seeded random tiles: random (camera, tile row) lines,
        # random tiles on each; lists from the rectangles, one pass over the
        # pairs per line (untimed)
        zb = rows[:, 6].view(np.uint32)
        lines = rng.choice(C * tiles_y, size=min(32, C * tiles_y), replace=False)

        def line_tasks(ln):
            c, ty = divmod(int(ln), tiles_y)
            cand = np.flatnonzero((cam == c) & (ty0 <= ty) & (ty < ty1))
            cx0, cx1 = tx0[cand], tx1[cand]
            out = []
            for tx in np.sort(rng.choice(tiles_x, size=min(64, tiles_x), replace=False)):
                sel = cand[(cx0 <= tx) & (tx < cx1)]
                lst = sel[np.lexsort((sel, zb[sel]))]
                x0, y0 = int(tx) * 16, ty * 16
                w, h = min(16, W - x0), min(16, H - y0)
                out.append((x0, y0, w, h, rows[lst], sc["v_rgb"][c, y0:y0 + h, x0:x0 + w],
                            sc["v_T"][c, y0:y0 + h, x0:x0 + w], not render_only))
            return out

        done, t_raster = 0, 0.0
        for k, ln in enumerate(lines):
            batch = line_tasks(ln)
            t0 = time.perf_counter()
            pool.map(_w_raster, batch, chunksize=1)
            t_raster += time.perf_counter() - t0
            done += len(batch)
            if k % 8 == 0:
                note(f"oracle baseline: raster on {done} tiles {t_raster:.1f} s")
            if t_raster > seconds:
                break
        t_raster_all = t_raster * (C * T) / done
        # projection backward on seeded random visible pairs
        t_pbwd, n_pb = 0.0, 0
        if not render_only and nnz:
            n_pb = min(nnz, pbwd_sample)
            pick = np.sort(rng.choice(nnz, n_pb, replace=False))
            parts = np.array_split(pick, 4 * cores)
            jobs = []
            for part in parts:
                g_u, g_local = np.unique(gidx[part], return_inverse=True)
                sub_sc = {k: sc[k][g_u] for k in ("means", "quats", "log_scales",
                                                   "opacity_logits", "sh")}
                sub_sc.update(N=int(g_u.size), C=C, W=W, H=H, sh_degree=deg,
                              viewmats=sc["viewmats"], Ks=sc["Ks"])
                jobs.append((sub_sc, cam[part], g_local))
            t0 = time.perf_counter()
            pool.map(_w_project_bwd, jobs, chunksize=1)
            t_pbwd = (time.perf_counter() - t0) * nnz / n_pb
            note(f"oracle baseline: projection backward on {n_pb} pairs, scaled {t_pbwd:.1f} s")
    est = t_proj + t_isect + t_raster_all + t_pbwd
    return dict(value=1.0 / est, unit="frames/s" if render_only else "steps/s", cores=cores,
                kind="oracle",
                sample=(f"fp64 NumPy oracle in {cores} worker processes: projection of all "
                        f"{C * N} pairs ({t_proj:.1f} s); intersect + stable sort on {take.size} "
                        f"seeded random pairs ({n_sub} of {n_is} entries, one process) scaled to "
                        f"all ({t_isect:.1f} s); raster {'fwd' if render_only else 'fwd+bwd'} on "
                        f"{done} of {C * T} seeded random tiles on {k + 1} random tile rows "
                        f"({t_raster:.1f} s) scaled to all "
                        f"({t_raster_all:.0f} s)"
                        + (f"; projection backward on {n_pb} of {nnz} seeded random visible "
                           f"pairs scaled to all ({t_pbwd:.1f} s)" if not render_only else "")
                        + f"; est. {est:.0f} s/step"))


def calibrate_copy(mib):
    import torch
    n = mib * 2**20 // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4,
                      "copies": 3}))


def calibrate_valu():
    """Throughput of plain fp32 FMAs and of the hardware exp, from the
    library's probe kernels (256-lane blocks, eight independent chains per
    lane), timed with events on the launching stream."""
    import torch

    import gaussian_splatting_differentiable_project_amd as gsd
    blocks, iters = 256 * 64, 4096
    out = torch.empty(blocks * 256, device="cuda")
    res = {}
    for kind, name in ((0, "fma"), (1, "exp")):
        gsd.valu_probe(kind, blocks, iters, out)   # warm-up
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        reps = 5
        for _ in range(reps):
            gsd.valu_probe(kind, blocks, iters, out)
        ev1.record()
        torch.cuda.synchronize()
        sec = ev0.elapsed_time(ev1) * 1e-3 / reps
        ops = blocks * 256 * iters * 8
        res[name] = {"lane_ops_per_s": ops / sec, "launch_ms": sec * 1e3}
    res["fma"]["tflops"] = 2 * res["fma"]["lane_ops_per_s"] / 1e12
    res["fma"]["frac_of_157.3"] = res["fma"]["tflops"] / ALU_PEAK_TFLOPS
    print(json.dumps({"valu_probe": res, "blocks": blocks, "iters": iters, "chains": 8}))


def run_config(cid, a, cpu_baseline_on, mode="train"):
    """One scene: warm-up, a per-kernel breakdown pass, then K timed steps
    with events around the dominant kernel only. Returns the JSON dict."""
    import torch

    import gaussian_splatting_differentiable_project_amd as gsd
    spec = workloads.CONFIGS[cid]
    note(f"{spec.name}: drawing the scene")
    sc = workloads.make_scene(spec)
    s = gsd.Scene.from_numpy(sc, "cuda")
    note(f"{spec.name}: scene resident on the GPU")
    v_rgb = torch.from_numpy(sc["v_rgb"]).cuda()
    v_T = torch.from_numpy(sc["v_T"]).cuda()
    r = gsd.Rasterizer("cuda")
    stream = torch.cuda.current_stream()
    render = mode == "render"
    adam = gsd.AdamState.zeros_like(s) if (a.adam and not render) else None
    arena = gsd.PhaseArena() if (a.arena and not render) else None
    stages = ["project", "intersect", "raster_fwd"] + ([] if render else ["raster_bwd",
                                                                          "project_bwd"])

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        if arena is not None:   # one call: the stage split is not recorded
            mark(0)
            out = r.step_arena(s, v_rgb, v_T, arena)
            for i in range(1, len(stages) + 1):
                mark(i)
            return out["proj"], out["isect"], out["last"]
        mark(0)
        p = r.project(s)
        mark(1)
        it = r.intersect(s, p)
        mark(2)
        rgb, T, last = r.rasterize_fwd(s, p, it)
        mark(3)
        if not render:
            vs = r.rasterize_bwd(s, p, it, T, last, v_rgb, v_T)
            mark(4)
            if adam is not None:
                r.project_bwd_adam(s, p, vs, adam)
            else:
                r.project_bwd(s, p, vs)
            mark(5)
        return p, it, last

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    note(f"{spec.name}: {a.warmup} warm-up steps done")

    # per-kernel breakdown (not the headline timing): every kernel timed
    n_bd = 3
    gsd.profile_reset()
    gsd.profile_enable(None)
    bd_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
             for _ in range(n_bd)]
    for k in range(n_bd):
        step(bd_ev[k])
    torch.cuda.synchronize()
    gsd.profile_disable()
    kernel_ms = {}
    for kn in KERNELS:
        n, ms = gsd.profile_query(kn)
        if n:
            kernel_ms[kn] = ms / n_bd
    stage_ms = {st: float(np.mean([bd_ev[k][i].elapsed_time(bd_ev[k][i + 1]) for k in range(n_bd)]))
                for i, st in enumerate(stages)}
    dom = max(kernel_ms, key=kernel_ms.get)
    gsd.profile_reset()
    note(f"{spec.name}: per-kernel breakdown done; dominant kernel {dom}")

    # timed region: events only around the dominant kernel, on its stream
    gsd.profile_enable(dom)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        p, it, last = step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    note(f"{spec.name}: {a.steps} timed steps, {wall * 1e3 / a.steps:.3f} ms/step")
    peak_mib = torch.cuda.max_memory_allocated() / 2**20
    gsd.profile_disable()
    n_dom, dom_ms_total = gsd.profile_query(dom)
    gsd.profile_reset()
    dom_ms = dom_ms_total / max(n_dom, 1)
    launches_per_step = n_dom / a.steps

    ms_per_step = wall * 1e3 / a.steps
    steps_s = a.steps / wall
    nnz, n_is = p.nnz, it.n_isects
    vis = np.unpackbits(p.mask.cpu().numpy().view(np.uint8), bitorder="little").astype(bool)
    Np = gsd.pad_n(spec.n)
    V = int(vis[: spec.n_cams * Np].reshape(spec.n_cams, Np).any(0).sum())
    del vis
    tx, ty = gsd.tiles(spec.width, spec.height)
    sm = sort_model(spec, p.aabb16[:nnz] if p.aabb16 is not None else
                    torch.empty(0, 2, dtype=torch.int32, device="cuda"), it.n_isects)
    # the depth sort runs its top 8-bit pass only when the keys differ there
    depth_passes = 3
    if nnz:
        kb = p.screen[:nnz, 6].contiguous().view(torch.int32).to(torch.int64)
        depth_passes += int(((int(kb.min()) ^ int(kb.max())) >> 24) != 0)
        del kb
    evals = raster_evals(last)

    if dom in ("k_raster_bwd", "k_raster_fwd"):
        per_comp = FLOPS_BWD_COMPOSITE if dom == "k_raster_bwd" else FLOPS_FWD_COMPOSITE
        work = (FLOPS_EVAL + per_comp) * evals
        achieved = work / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "alu", "kernel": dom, "achieved": achieved, "peak": ALU_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / ALU_PEAK_TFLOPS,
                "frac_of_measured_fma": achieved / MEASURED_FMA_TFLOPS,
                "flops_per_launch": work, "evaluations": evals,
                "flops_per_evaluation": FLOPS_EVAL + per_comp, "launch_ms": dom_ms}
    else:
        byt = hbm_bytes(dom, spec, nnz, n_is, V, sm, depth_passes)
        achieved = byt / (dom_ms * 1e-3) / 1e9 if byt else None
        roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
                "bytes_per_launch": byt, "launch_ms": dom_ms}
    roof["traffic"] = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        ent = tr.get(f"{dom}@{spec.name}") or tr.get(dom)
        if ent and ent.get("workload") == spec.name and ent.get("source_sha") == source_sha(dom):
            roof["traffic"] = ent["hbm_bytes_per_launch"]

    out = {
        "metric": ("render frames/s (projection, intersection, forward) at 1 MI355X" if render else
                   "fwd+bwd rasterizer steps/s and M visible pairs/s at 1 MI355X; % HBM peak"),
        "value": steps_s,
        "unit": "frames/s" if render else "steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name + ("-render" if render else "-adam" if adam else
                                           "-arena" if arena else ""),
                   "N": spec.n,
                   "sh_degree": spec.sh_degree,
                   "cameras": spec.n_cams, "width": spec.width, "height": spec.height,
                   "focal": spec.focal, "seed": spec.seed},
        "m_visible_pairs_per_s": nnz * steps_s / 1e6,
        "nnz": nnz,
        "n_isects": n_is,
        "segments": sm["segments"],
        "visible_gaussians": V,
        "raster_evaluations": evals,
        "stage_ms": stage_ms,
        "kernel_ms_per_step": kernel_ms,
        "dominant_launches_per_step": launches_per_step,
        "roofline": roof,
        "peak_device_MiB": peak_mib,
    }
    if arena is not None:
        out["arena"] = {"alias": arena.alias, "MiB": arena.buf.numel() / 2**20}
    hb = {}
    for kn, ms in kernel_ms.items():
        byt = hbm_bytes(kn, spec, nnz, n_is, V, sm, depth_passes)
        if byt:
            if kn == "k_radix_scatter":   # per-launch mean; ms is the step's sum
                byt *= depth_passes + sm["passes"] + order_passes(spec)
            hb[kn] = byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    # the whole sort (depth passes over the pairs, tile passes over the
    # entries, launch-order passes over the tiles if any; each pass reads and
    # writes a 4 B key and a 4 B value per element) against the time of all
    # its kernels: counting and scatter
    sort_ms = sum(kernel_ms.get(k, 0.0) for k in ("k_radix_count", "k_radix_scatter"))
    sort_bytes = 16 * (depth_passes * nnz + sm["passes"] * sm["elems"]
                       + order_passes(spec) * spec.n_cams * tx * ty)
    if sort_ms > 0:
        hb["sort (all radix kernels)"] = sort_bytes / (sort_ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    out["hbm_frac_by_kernel"] = hb
    # raster kernels against the fp32 vector peak, by the method's evaluations
    for kn, per_comp in (("k_raster_fwd", FLOPS_FWD_COMPOSITE), ("k_raster_bwd", FLOPS_BWD_COMPOSITE)):
        if kn in kernel_ms:
            tf = (FLOPS_EVAL + per_comp) * evals / (kernel_ms[kn] * 1e-3) / 1e12
            out.setdefault("alu_frac_by_kernel", {})[kn] = tf / ALU_PEAK_TFLOPS
            out.setdefault("alu_frac_of_measured_fma", {})[kn] = tf / MEASURED_FMA_TFLOPS
    if render:
        out["ms_per_frame"] = out.pop("ms_per_step")
    del p, it, last, r, s, v_rgb, v_T, adam, arena
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu_baseline_on:
        out["cpu_baseline"] = cpu_baseline(sc, spec, a.cpu_sample_seconds, render_only=render)
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "one GPU only: the library has no multi-GPU path; use --gpus 1"}))
        sys.exit(2)
    import torch

    import gaussian_splatting_differentiable_project_amd as gsd
    gsd.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.calibrate_copy:
        calibrate_copy(a.calibrate_copy)
        return
    if a.calibrate_valu:
        calibrate_valu()
        return
    out = run_config(a.config, a, not a.no_cpu_baseline, a.mode)
    extra = (not a.no_extra and a.mode == "train" and not a.adam and not a.arena
             and a.extra_config != a.config)
    if extra:
        # the second scene after the first one's buffers are freed; a few
        # steps only (one step moves about 0.2 TB)
        import copy
        b = copy.copy(a)
        b.steps, b.warmup = min(a.steps, 5), min(a.warmup, 2)
        ex = run_config(a.extra_config, b, False, "train")
        out[f"config{a.extra_config}"] = {
            k: ex[k] for k in ("config", "value", "unit", "steps", "warmup", "ms_per_step",
                               "m_visible_pairs_per_s", "nnz", "n_isects", "roofline",
                               "hbm_frac_by_kernel", "alu_frac_by_kernel",
                               "kernel_ms_per_step", "peak_device_MiB") if k in ex}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
