"""Full-size parity: the HIP path on a whole benchmark scene against the
oracle on everything the oracle can afford, and on seeded samples of the
rest.

* Projection: every (camera, Gaussian) pair, chunk by chunk in the oracle:
  mask bits bit-exact outside fragile pairs, every visible pair's screen
  row and 16-bit box.
* Intersection and sort: exact per-tile lists (oracle order: depth bits,
  then slot) on sampled tiles, compared as sequences of pair ids with
  fragile pairs removed; over the whole list, the order property of a
  stable key sort and per-tile counts against a 2-D difference count of
  the GPU's own box codes.
* Images: sampled tiles, oracle walk over the oracle's own list and rows.
* Gradients: sampled Gaussians whose tiles are all rasterized by the
  oracle, so their screen gradients are complete; then the oracle's
  projection backward for exactly those Gaussians.

Every expected value comes from the oracle on the seeded inputs; GPU
outputs are only compared, never fed to the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import raster as oraster
from oracle.intersect import TILE, tile_rects_from_aabb16
from oracle.project import NEAR, Projection, quantize_aabb16, screen_rows
from tests import parity as P

Q16 = 65535


def chunk_fragile(pc, W, H):
    """Fragile pairs of one projected chunk (see parity.fragile_pairs)."""
    u, v, r, z = pc["u"], pc["v"], pc["r"], pc["z"]
    f = np.abs(z - NEAR) <= 1e-5 * NEAR
    with np.errstate(invalid="ignore"):
        for a, ext in ((u, W), (v, H)):
            t = P.tau_px(np.abs(a) + r)
            f |= np.abs(a + r) <= t
            f |= np.abs(a - r - ext) <= t
            lo = np.maximum(a - r, 0.0)
            hi = np.minimum(a + r, float(ext))
            vis = pc["visible"]
            f |= vis & P._tile_fragile_edge(lo, ext, True, t)
            f |= vis & P._tile_fragile_edge(hi, ext, False, t)
    f |= ~np.isfinite(u) | ~np.isfinite(v)
    return f & (z > 0)


def _project_chunk(args):
    """One (camera, Gaussian range) task of OracleScene (runs in a worker)."""
    means, quats, log_scales, logits, sh, viewmat, K, W, H, deg = args
    pc = oracle.project_camera(means, quats, log_scales, logits, sh, viewmat, K, W, H, deg)
    idx = np.flatnonzero(pc["visible"])
    rows = screen_rows(pc, idx).astype(np.float32)
    w0 = (pc["qx0"][idx] | (pc["qy0"][idx] << 16)).astype(np.uint32)
    w1 = (pc["qx1"][idx] | (pc["qy1"][idx] << 16)).astype(np.uint32)
    return pc["visible"], chunk_fragile(pc, W, H), rows, np.stack([w0, w1], 1)


class OracleScene:
    """The oracle's projection of a whole scene, pair by pair, kept compact:
    visible flags, fragility, and fp32-stored rows / boxes / depth bits of
    the visible pairs in slot order. Chunks run in `workers` fresh
    processes (spawned, so they never touch the GPU of this process)."""

    def __init__(self, sc, chunk=1 << 18, workers=0):
        import multiprocessing as mp
        import os
        N, C, W, H = sc["N"], sc["C"], sc["W"], sc["H"]
        self.N, self.C, self.W, self.H = N, C, W, H
        self.Np = ((N + 127) // 128) * 128
        self.vis = np.zeros(C * self.Np, bool)
        self.frag = np.zeros(C * self.Np, bool)
        tasks, where = [], []
        for c in range(C):
            for g0 in range(0, N, chunk):
                g1 = min(N, g0 + chunk)
                tasks.append((sc["means"][g0:g1], sc["quats"][g0:g1], sc["log_scales"][g0:g1],
                              sc["opacity_logits"][g0:g1], sc["sh"][g0:g1], sc["viewmats"][c],
                              sc["Ks"][c], W, H, sc["sh_degree"]))
                where.append(c * self.Np + g0)
        if workers == 0:
            workers = min(16, os.cpu_count() or 1, len(tasks))
        if workers > 1:
            with mp.get_context("spawn").Pool(workers) as pool:
                results = pool.map(_project_chunk, tasks, chunksize=1)
        else:
            results = [_project_chunk(t) for t in tasks]
        rows, boxes = [], []
        for base, (vis, frag, rw, bx) in zip(where, results):
            self.vis[base: base + vis.size] = vis
            self.frag[base: base + vis.size] = frag
            rows.append(rw)
            boxes.append(bx)
        del results, tasks
        self.pairs = np.flatnonzero(self.vis)
        self.nnz = self.pairs.size
        self.rows = np.concatenate(rows) if rows else np.zeros((0, 10), np.float32)
        self.aabb = np.concatenate(boxes) if boxes else np.zeros((0, 2), np.uint32)
        self.cam = self.pairs // self.Np
        self.gauss = self.pairs % self.Np
        self.tiles_x = (W + TILE - 1) // TILE
        self.tiles_y = (H + TILE - 1) // TILE
        self.T = self.tiles_x * self.tiles_y
        self.rect = np.stack(tile_rects_from_aabb16(self.aabb, W, H), 1)  # tx0, ty0, tx1, ty1
        self.zbits = self.rows[:, 6].view(np.uint32)

    def tile_list(self, t):
        """Oracle slots of global tile t in sorted order (depth bits, slot)."""
        c, tl = divmod(int(t), self.T)
        ty, tx = divmod(tl, self.tiles_x)
        r = self.rect
        sel = np.flatnonzero((self.cam == c) & (r[:, 0] <= tx) & (tx < r[:, 2]) &
                             (r[:, 1] <= ty) & (ty < r[:, 3]))
        return sel[np.lexsort((sel, self.zbits[sel]))]

    def tiles_of_slot(self, s):
        tx0, ty0, tx1, ty1 = (int(v) for v in self.rect[s])
        c = int(self.cam[s])
        return [c * self.T + ty * self.tiles_x + tx for ty in range(ty0, ty1) for tx in range(tx0, tx1)]


def gpu_pairs_from_mask(mask_words, n_pairs):
    vis = np.unpackbits(np.ascontiguousarray(mask_words).view(np.uint8), bitorder="little")
    return np.flatnonzero(vis[:n_pairs])


def compare_projection(o: OracleScene, gmask, gscreen, gaabb):
    """Mask bits and every common visible pair's row and box; returns a
    report dict and the GPU's visible pair ids."""
    n_pairs = o.C * o.Np
    gp = gpu_pairs_from_mask(gmask, n_pairs)
    gvis = np.zeros(n_pairs, bool)
    gvis[gp] = True
    diff = gvis != o.vis
    bad = diff & ~o.frag
    assert not bad.any(), f"{int(bad.sum())} non-fragile mask mismatches, e.g. {np.flatnonzero(bad)[:5]}"
    both = np.intersect1d(gp, o.pairs, assume_unique=True)
    gi = np.searchsorted(gp, both)
    oi = np.searchsorted(o.pairs, both)
    rg = gscreen[gi].astype(np.float64)
    ro = o.rows[oi].astype(np.float64)
    ulps = P.compare_rows(rg, ro)
    ag = gaabb[gi].astype(np.int64)
    ao = o.aabb[oi].astype(np.int64)
    for w in range(2):
        for sh in (0, 16):
            dq = np.abs(((ag[:, w] >> sh) & 0xFFFF) - ((ao[:, w] >> sh) & 0xFFFF))
            assert dq.max(initial=0) <= 1
    rgr = np.stack(tile_rects_from_aabb16(ag.astype(np.uint32), o.W, o.H), 1)
    rbad = (rgr != o.rect[oi]).any(1) & ~o.frag[both]
    assert not rbad.any(), both[rbad][:5]
    return dict(nnz_gpu=int(gp.size), nnz_oracle=o.nnz, fragile=int(o.frag.sum()),
                mask_diffs=int(diff.sum()), row_ulps=ulps), gp


def check_sort_order(toff, ids, screen_dev, chunk=1 << 27):
    """Whole-list order property (on the GPU, chunked): entry keys
    (tile << 32 | depth bits) never decrease and equal keys keep
    increasing slots -- the result of a stable sort of slot-ordered keys."""
    dev = ids.device
    I = ids.numel()
    zb = screen_dev[:, 6].contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    bounds = toff[1:-1].contiguous()
    prev = None
    for e0 in range(0, I, chunk):
        e1 = min(I, e0 + chunk)
        pos = torch.arange(e0, e1, device=dev, dtype=torch.int64)
        tile = torch.searchsorted(bounds, pos, right=True)
        slot = ids[e0:e1].to(torch.int64) & 0xFFFFFFFF
        key = (tile << 32) | zb[slot]
        ok = bool(((key[1:] > key[:-1]) | ((key[1:] == key[:-1]) & (slot[1:] > slot[:-1]))).all())
        assert ok, f"order violated in [{e0}, {e1})"
        k0, s0 = int(key[0]), int(slot[0])
        if prev is not None:
            assert k0 > prev[0] or (k0 == prev[0] and s0 > prev[1]), f"order violated at {e0}"
        prev = (int(key[-1]), int(slot[-1]))
        del pos, tile, slot, key


def check_launch_order(order, toff):
    """The heavy-first launch order, by its defining properties (which fix
    it uniquely): a permutation of the tile ids along which the saturated
    entry count never increases and equal counts keep increasing ids."""
    n = toff.numel() - 1
    o = order.to(torch.int64) & 0xFFFFFFFF
    assert o.numel() == n
    assert torch.equal(torch.sort(o).values, torch.arange(n, device=o.device)), "not a permutation"
    cnt = torch.diff(toff).clamp(max=0xFFFF)[o]
    ok = (cnt[1:] < cnt[:-1]) | ((cnt[1:] == cnt[:-1]) & (o[1:] > o[:-1]))
    assert bool(ok.all()), "launch order violated"


def gpu_tile_counts_from_boxes(aabb_dev, cam_offsets, C, W, H):
    """Per-tile entry counts implied by the GPU's own 16-bit boxes: each
    slot adds one to every tile of its rectangle (2-D difference array)."""
    dev = aabb_dev.device
    tiles_x, tiles_y = (W + TILE - 1) // TILE, (H + TILE - 1) // TILE
    a = aabb_dev.contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    D = TILE * Q16
    tx0 = ((a[:, 0] & 0xFFFF) * W) // D
    ty0 = ((a[:, 0] >> 16) * H) // D
    tx1 = ((a[:, 1] & 0xFFFF) * W + D - 1) // D
    ty1 = ((a[:, 1] >> 16) * H + D - 1) // D
    sizes = torch.tensor(np.diff(np.asarray(cam_offsets, np.int64)), device=dev)
    cam = torch.repeat_interleave(torch.arange(C, device=dev), sizes)
    ok = (tx1 > tx0) & (ty1 > ty0)
    cam, tx0, tx1, ty0, ty1 = cam[ok], tx0[ok], tx1[ok], ty0[ok], ty1[ok]
    grid = torch.zeros(C * (tiles_y + 1) * (tiles_x + 1), dtype=torch.int64, device=dev)
    base = cam * ((tiles_y + 1) * (tiles_x + 1))
    one = torch.ones_like(tx0)
    for yy, xx, sgn in ((ty0, tx0, 1), (ty0, tx1, -1), (ty1, tx0, -1), (ty1, tx1, 1)):
        grid.index_add_(0, base + yy * (tiles_x + 1) + xx, sgn * one)
    cnt = grid.view(C, tiles_y + 1, tiles_x + 1).cumsum(1).cumsum(2)[:, :tiles_y, :tiles_x]
    return cnt.reshape(-1)


def raster_tiles(o: OracleScene, tiles, sc, with_bwd=False):
    """Oracle raster over the given global tiles using compact lists.

    Returns (tiles, rgb, T, last, fragile pixel mask, screen gradients,
    composited slots): images are full-size arrays, NaN outside the tiles;
    the gradients (with_bwd) map every slot on those tiles to its row;
    composited slots are those the oracle's walk composites at >= 1 pixel.
    """
    C, W, H = o.C, o.W, o.H
    order = sorted(int(t) for t in tiles)
    lists = {t: o.tile_list(t) for t in order}
    uniq = np.unique(np.concatenate([lists[t] for t in order] + [np.zeros(0, np.int64)]))
    local = {int(s): k for k, s in enumerate(uniq)}
    rows = o.rows[uniq].astype(np.float64)
    rgb = np.full((C, H, W, 3), np.nan)
    Tm = np.full((C, H, W), np.nan)
    last = np.full((C, H, W), -2, np.int64)
    frag_px = np.zeros((C, H, W), bool)
    composited = set()
    for t in order:
        c, tl = divmod(t, o.T)
        ii, jj = oraster._tile_pixels(tl, o.tiles_x, W, H)
        ids = np.array([local[int(s)] for s in lists[t]], np.int64)
        if ids.size == 0:
            rgb[c, ii, jj] = 0.0
            Tm[c, ii, jj] = 1.0
            last[c, ii, jj] = -1
            continue
        Cc, Tt, ll, _, rec = oraster._walk_tile(rows[ids], jj + 0.5, ii + 0.5, record=True)
        rgb[c, ii, jj] = Cc[:, :3]
        Tm[c, ii, jj] = Tt
        last[c, ii, jj] = ll
        a = rec["alpha"]
        Tn = rec["Tb"] * (1.0 - a)
        stops = (a >= oraster.ALPHA_MIN) & (Tn < oraster.T_STOP) & ~rec["comp"]
        first = np.where(stops.any(1), stops.argmax(1), a.shape[1])
        reached = np.arange(a.shape[1])[None, :] <= first[:, None]
        bad = reached & (np.abs(a - oraster.ALPHA_MIN) <= P.ALPHA_WIN * oraster.ALPHA_MIN)
        bad |= reached & (a >= oraster.ALPHA_MIN) & \
            (np.abs(Tn - oraster.T_STOP) <= P.T_WIN * oraster.T_STOP)
        fp = bad.any(1)
        # pixels a fragile pair reaches with alpha >= 1/255
        for k, s in enumerate(lists[t]):
            if o.frag[o.pairs[s]]:
                fp |= reached[:, k] & (a[:, k] >= oraster.ALPHA_MIN * (1 - 1e-3))
        frag_px[c, ii, jj] = fp
        composited.update(int(s) for s in lists[t][rec["comp"].any(0)])
    vs = None
    if with_bwd:
        n_tiles = C * o.T
        counts = np.zeros(n_tiles, np.int64)
        for t in order:
            counts[t] = lists[t].size
        offs = np.zeros(n_tiles + 1, np.int64)
        offs[1:] = np.cumsum(counts)
        flat = np.zeros(int(offs[-1]), np.int64)
        for t in order:
            flat[offs[t]:offs[t + 1]] = [local[int(s)] for s in lists[t]]
        g = oracle.rasterize_bwd(rows, flat, offs, C, W, H, sc["v_rgb"], sc["v_T"], tiles=order)
        vs = {int(s): g[local[int(s)]] for s in uniq}
    return order, rgb, Tm, last, frag_px, vs, composited
