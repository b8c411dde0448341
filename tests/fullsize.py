"""Full-size parity: the HIP path on a whole benchmark scene against the
oracle on everything the oracle can afford, and on seeded samples of the
rest.

* Projection: every (camera, Gaussian) pair, chunk by chunk in the oracle:
  mask bits bit-exact outside fragile pairs, every visible pair's screen
  row, and its 16-bit box codes exactly outside code-fragile pairs (an
  edge whose fp32 scaled value lies within the fragility window of an
  integer code).
* Intersection and sort: on scenes the oracle can sort whole (up to a few
  1e8 entries), the whole sorted list of (tile, pair) entries from
  ``oracle.intersect``, compared bit-exactly once fragile pairs' entries
  are removed from both sides; on the larger scene, exact per-tile lists
  on sampled tiles, and over the whole list the order property of a
  stable key sort and per-tile counts against a 2-D difference count of
  the GPU's own box codes.
* Images: sampled tiles (at least 1% of the scene's tiles), each tile
  composited by the oracle as a one-tile image of its own in a worker
  process.
* Gradients: sampled Gaussians, small and large (up to 256 tiles), whose
  tiles are all rasterized backward by the oracle, so their screen
  gradients are complete; then the oracle's projection backward for
  exactly those Gaussians.

Every expected value comes from the oracle on the seeded inputs; GPU
outputs are only compared, never fed to the oracle.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np
import torch

import oracle
from oracle import raster as oraster
from oracle.intersect import TILE, tile_rects_from_aabb16
from oracle.project import NEAR, screen_rows
from tests import parity as P

Q16 = 65535


def pool_size(n_tasks: int) -> int:
    """Worker processes: the host cores this process may use, at most 16."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(16, cores, n_tasks))


def _code_fragile_edge(e, extent, is_min, tau):
    """Does moving edge e by +-tau change its 16-bit code?"""
    s = np.float32(Q16) / np.float32(extent)
    lo = (np.asarray(e - tau, np.float64)).astype(np.float32) * s
    hi = (np.asarray(e + tau, np.float64)).astype(np.float32) * s
    f = np.floor if is_min else np.ceil
    return np.clip(f(lo), 0, Q16) != np.clip(f(hi), 0, Q16)


def chunk_fragile(pc, W, H):
    """(fragile, code-fragile) pairs of one projected chunk (see
    parity.fragile_pairs): fragile pairs may differ in visibility, tile
    rectangle or key; code-fragile pairs may differ in a 16-bit code.

    Both sides take a code as floor or ceil of fp32(edge) * fp32(65535 /
    extent), from an fp64 edge that each side evaluates with its own
    operation order (relative differences near 1e-15). A code can differ
    only where the fp64 edges straddle an fp32 rounding point that moves
    the product across an integer: the window is a relative 1e-9 of the
    coordinate, far above those differences."""
    u, v, r, z = pc["u"], pc["v"], pc["r"], pc["z"]
    f = np.abs(z - NEAR) <= 1e-5 * NEAR
    cf = np.zeros_like(f)
    vis = pc["visible"]
    with np.errstate(invalid="ignore"):
        for a, ext in ((u, W), (v, H)):
            t = P.tau_px(np.abs(a) + r)
            f |= np.abs(a + r) <= t
            f |= np.abs(a - r - ext) <= t
            lo = np.maximum(a - r, 0.0)
            hi = np.minimum(a + r, float(ext))
            f |= vis & P._tile_fragile_edge(lo, ext, True, t)
            f |= vis & P._tile_fragile_edge(hi, ext, False, t)
            tc = 1e-9 * np.maximum(1.0, np.abs(a) + r)
            cf |= vis & _code_fragile_edge(lo, ext, True, tc)
            cf |= vis & _code_fragile_edge(hi, ext, False, tc)
    f |= ~np.isfinite(u) | ~np.isfinite(v)
    f &= z > 0
    return f, cf | f


def _project_chunk(args):
    """One (camera, Gaussian range) task of OracleScene (runs in a worker)."""
    means, quats, log_scales, logits, sh, viewmat, K, W, H, deg = args
    pc = oracle.project_camera(means, quats, log_scales, logits, sh, viewmat, K, W, H, deg)
    idx = np.flatnonzero(pc["visible"])
    rows = screen_rows(pc, idx).astype(np.float32)
    w0 = (pc["qx0"][idx] | (pc["qy0"][idx] << 16)).astype(np.uint32)
    w1 = (pc["qx1"][idx] | (pc["qy1"][idx] << 16)).astype(np.uint32)
    frag, code_frag = chunk_fragile(pc, W, H)
    return pc["visible"], frag, code_frag, rows, np.stack([w0, w1], 1)


class _ProjView:
    """The fields of an oracle Projection that ``oracle.intersect`` reads."""

    def __init__(self, C, aabb16, cam, z32):
        self.C, self.aabb16, self.cam, self.z32 = C, aabb16, cam, z32


class OracleScene:
    """The oracle's projection of a whole scene, pair by pair, kept compact:
    visible flags, fragility, and fp32-stored rows / boxes / depth bits of
    the visible pairs in slot order. Chunks run in worker processes
    (spawned, so they never touch the GPU of this process)."""

    def __init__(self, sc, chunk=1 << 18, workers=0):
        N, C, W, H = sc["N"], sc["C"], sc["W"], sc["H"]
        self.N, self.C, self.W, self.H = N, C, W, H
        self.Np = ((N + 127) // 128) * 128
        self.vis = np.zeros(C * self.Np, bool)
        self.frag = np.zeros(C * self.Np, bool)
        self.code_frag = np.zeros(C * self.Np, bool)
        tasks, where = [], []
        for c in range(C):
            for g0 in range(0, N, chunk):
                g1 = min(N, g0 + chunk)
                tasks.append((sc["means"][g0:g1], sc["quats"][g0:g1], sc["log_scales"][g0:g1],
                              sc["opacity_logits"][g0:g1], sc["sh"][g0:g1], sc["viewmats"][c],
                              sc["Ks"][c], W, H, sc["sh_degree"]))
                where.append(c * self.Np + g0)
        workers = workers or pool_size(len(tasks))
        if workers > 1:
            with mp.get_context("spawn").Pool(workers) as pool:
                results = pool.map(_project_chunk, tasks, chunksize=1)
        else:
            results = [_project_chunk(t) for t in tasks]
        rows, boxes = [], []
        for base, (vis, frag, cfrag, rw, bx) in zip(where, results):
            self.vis[base: base + vis.size] = vis
            self.frag[base: base + vis.size] = frag
            self.code_frag[base: base + vis.size] = cfrag
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
        self.tx0, self.ty0, self.tx1, self.ty1 = (np.ascontiguousarray(self.rect[:, k])
                                                  for k in range(4))
        self.zbits = self.rows[:, 6].view(np.uint32)
        self.n_isects = int(((self.rect[:, 2] - self.rect[:, 0]) *
                             (self.rect[:, 3] - self.rect[:, 1])).sum())

    def intersect(self):
        """``oracle.intersect`` on the whole scene."""
        pv = _ProjView(self.C, self.aabb, self.cam, self.rows[:, 6].astype(np.float32))
        return oracle.intersect(pv, self.W, self.H)

    def tile_lists(self, tiles):
        """{global tile: oracle slots in sorted order (depth bits, slot)} for
        the given tiles. Pairs are bucketed by (camera, first tile row), so
        a row's candidates are the buckets of the rows above it that a box
        can span."""
        if not hasattr(self, "_by_row"):
            key = self.cam * (self.tiles_y + 1) + self.ty0
            order = np.argsort(key, kind="stable")
            self._by_row = (order, np.searchsorted(key[order],
                                                   np.arange(self.C * (self.tiles_y + 1) + 1)))
            self._hmax = int((self.ty1 - self.ty0).max(initial=1))
        order, starts = self._by_row
        rows = {}
        for t in tiles:
            c, tl = divmod(int(t), self.T)
            rows.setdefault((c, tl // self.tiles_x), []).append(int(t))
        out = {}
        for (c, ty), ts in rows.items():
            b0 = c * (self.tiles_y + 1) + max(0, ty - self._hmax + 1)
            b1 = c * (self.tiles_y + 1) + ty + 1
            cand = order[starts[b0]:starts[b1]]
            cand = cand[self.ty1[cand] > ty]
            cx0, cx1 = self.tx0[cand], self.tx1[cand]
            for t in ts:
                tx = (t - c * self.T) % self.tiles_x
                sel = np.sort(cand[(cx0 <= tx) & (tx < cx1)])
                out[t] = sel[np.lexsort((sel, self.zbits[sel]))]
        return out

    def tiles_of_slot(self, s):
        tx0, ty0, tx1, ty1 = (int(v) for v in self.rect[s])
        c = int(self.cam[s])
        return [c * self.T + ty * self.tiles_x + tx for ty in range(ty0, ty1) for tx in range(tx0, tx1)]


def gpu_pairs_from_mask(mask_words, n_pairs):
    vis = np.unpackbits(np.ascontiguousarray(mask_words).view(np.uint8), bitorder="little")
    return np.flatnonzero(vis[:n_pairs])


def compare_projection(o: OracleScene, gmask, gscreen, gaabb):
    """Mask bits, and every common visible pair's row and box codes; returns
    a report dict and the GPU's visible pair ids."""
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
    code_ok = ~o.code_frag[both]
    code_diffs = int((ag != ao).any(1).sum())
    assert np.array_equal(ag[code_ok], ao[code_ok]), \
        f"16-bit codes differ on {int(((ag != ao).any(1) & code_ok).sum())} non-code-fragile pairs"
    for w in range(2):   # code-fragile pairs still agree to one grid step
        for sh in (0, 16):
            dq = np.abs(((ag[:, w] >> sh) & 0xFFFF) - ((ao[:, w] >> sh) & 0xFFFF))
            assert dq.max(initial=0) <= 1
    rgr = np.stack(tile_rects_from_aabb16(ag.astype(np.uint32), o.W, o.H), 1)
    rbad = (rgr != o.rect[oi]).any(1) & ~o.frag[both]
    assert not rbad.any(), both[rbad][:5]
    return dict(nnz_gpu=int(gp.size), nnz_oracle=o.nnz, fragile=int(o.frag.sum()),
                code_fragile=int(o.code_frag.sum()), code_diffs=code_diffs,
                mask_diffs=int(diff.sum()), row_ulps=ulps), gp


def compare_whole_lists(o: OracleScene, gp, toff, ids):
    """The whole sorted list, as (tile, pair) entries, against
    ``oracle.intersect`` on the same scene, with every entry of a fragile
    pair removed from both sides. Returns (entries compared, entries
    removed on the oracle side, the tiles whose full lists differ)."""
    iso = o.intersect()
    toff_o = iso.tile_offsets
    t_o = np.repeat(np.arange(toff_o.size - 1, dtype=np.int64), np.diff(toff_o))
    p_o = o.pairs[iso.flatten_ids.astype(np.int64)]
    del iso
    # tiles whose lists differ with fragile pairs kept: count differs, or
    # some entry differs among tiles of equal counts
    same_cnt = np.diff(toff) == np.diff(toff_o)
    differ = set(np.flatnonzero(~same_cnt).tolist())
    sel_g = np.repeat(same_cnt, np.diff(toff))
    sel_o = np.repeat(same_cnt, np.diff(toff_o))
    pg_same = gp[ids[sel_g].astype(np.int64)]
    bad = pg_same != p_o[sel_o]
    differ.update(np.unique(t_o[sel_o][bad]).tolist())
    del sel_g, sel_o, pg_same, bad
    keep = ~o.frag[p_o]
    t_o, p_o = t_o[keep], p_o[keep]
    removed = int((~keep).sum())
    del keep
    t_g = np.repeat(np.arange(toff.size - 1, dtype=np.int64), np.diff(toff))
    p_g = gp[ids.astype(np.int64)]
    keep = ~o.frag[p_g]
    t_g, p_g = t_g[keep], p_g[keep]
    assert t_g.size == t_o.size, (t_g.size, t_o.size)
    np.testing.assert_array_equal(t_g, t_o, err_msg="tile of a sorted entry")
    np.testing.assert_array_equal(p_g, p_o, err_msg="pair of a sorted entry")
    return int(t_g.size), removed, differ


def gpu_tile_pairs(gp, toff, ids_dev, t):
    """The GPU's list of global tile t as pair ids."""
    g = ids_dev[int(toff[t]):int(toff[t + 1])].cpu().numpy().view(np.uint32)
    return gp[g.astype(np.int64)]


def differing_tiles(o: OracleScene, gp, toff, ids_dev, tiles, lists):
    """The tiles among ``tiles`` whose GPU list, as pair ids, is not the
    oracle's list entry for entry (a fragile pair placed differently)."""
    return {int(t) for t in tiles
            if not np.array_equal(gpu_tile_pairs(gp, toff, ids_dev, t), o.pairs[lists[t]])}


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


def _raster_tile_task(args):
    """Composite one tile with the oracle as a one-tile image of its own (in
    a worker process). The rows' centres are shifted by the tile origin, a
    whole number of pixels, which leaves every pixel offset dx, dy exactly
    as in the full image. Returns the tile's colour, T, last ids, fragile
    pixels, which list entries were composited and, with ``with_bwd``, the
    screen-row gradients of the list entries."""
    t, x0, y0, w, h, rows, vr, vT, with_bwd = args
    rows = rows.astype(np.float64)
    rows[:, 0] -= x0
    rows[:, 1] -= y0
    n = rows.shape[0]
    ids = np.arange(n, dtype=np.uint32)
    offs = np.array([0, n], np.int64)
    rgb, T, last, _ = oracle.rasterize_fwd(rows, ids, offs, 1, w, h)
    rgb, T, last = rgb[0].reshape(-1, 3), T[0].reshape(-1), last[0].reshape(-1)
    fp = np.zeros(w * h, bool)
    comp = np.zeros(n, bool)
    if n:
        ii, jj = oraster._tile_pixels(0, 1, w, h)
        _, _, _, evals, _ = oraster._walk_tile(rows, jj + 0.5, ii + 0.5, record=False)
        reach = int(evals.max())
        _, _, _, _, rec = oraster._walk_tile(rows[:reach], jj + 0.5, ii + 0.5, record=True)
        a = rec["alpha"]
        Tn = rec["Tb"] * (1.0 - a)
        stops = (a >= oraster.ALPHA_MIN) & (Tn < oraster.T_STOP) & ~rec["comp"]
        first = np.where(stops.any(1), stops.argmax(1), a.shape[1])
        reached = np.arange(a.shape[1])[None, :] <= first[:, None]
        bad = reached & (np.abs(a - oraster.ALPHA_MIN) <= P.ALPHA_WIN * oraster.ALPHA_MIN)
        bad |= reached & (a >= oraster.ALPHA_MIN) & \
            (np.abs(Tn - oraster.T_STOP) <= P.T_WIN * oraster.T_STOP)
        fp = bad.any(1)
        comp[:reach] = rec["comp"].any(0)
    g = None
    if with_bwd and n:
        g = oracle.rasterize_bwd(rows, ids, offs, 1, w, h, vr[None], vT[None])
        used = np.flatnonzero(np.any(g != 0.0, axis=1))
        g = (used, g[used])
    return t, rgb, T, last, fp, comp, g


def raster_tiles(o: OracleScene, tiles, sc, with_bwd=False, lists=None):
    """Oracle raster over the given global tiles, in worker processes.

    Returns (tiles, rgb, T, last, fragile pixel mask, screen gradients,
    composited slots): images are full-size arrays, NaN outside the tiles;
    fragile pixels are those whose walk meets an alpha or stop decision
    inside the fragility window (tiles whose GPU list differs from the
    oracle's are the caller's to exclude); the gradients (with_bwd) map
    every slot with a nonzero gradient on those tiles to its summed row;
    composited slots are those the oracle's walk composites at >= 1 pixel.
    """
    C, W, H = o.C, o.W, o.H
    order = sorted(int(t) for t in tiles)
    lists = lists if lists is not None else o.tile_lists(order)
    rgb = np.full((C, H, W, 3), np.nan)
    Tm = np.full((C, H, W), np.nan)
    last = np.full((C, H, W), -2, np.int64)
    frag_px = np.zeros((C, H, W), bool)
    composited = set()
    vs = {} if with_bwd else None

    def tasks():
        for t in order:
            c, tl = divmod(t, o.T)
            ty, tx = divmod(tl, o.tiles_x)
            x0, y0 = tx * TILE, ty * TILE
            w, h = min(TILE, W - x0), min(TILE, H - y0)
            sl = lists[t]
            vr = sc["v_rgb"][c, y0:y0 + h, x0:x0 + w] if with_bwd else None
            vT = sc["v_T"][c, y0:y0 + h, x0:x0 + w] if with_bwd else None
            yield (t, x0, y0, w, h, o.rows[sl], vr, vT, with_bwd)

    workers = pool_size(len(order))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers) as pool:
        for t, r_, T_, l_, fp, comp, g in pool.imap_unordered(_raster_tile_task, tasks(),
                                                              chunksize=4):
            c, tl = divmod(t, o.T)
            ii, jj = oraster._tile_pixels(tl, o.tiles_x, W, H)
            rgb[c, ii, jj] = r_
            Tm[c, ii, jj] = T_
            last[c, ii, jj] = l_
            frag_px[c, ii, jj] = fp
            sl = lists[t]
            composited.update(int(s) for s in sl[comp])
            if g is not None:
                for k, row in zip(*g):
                    s = int(sl[k])
                    vs[s] = vs[s] + row if s in vs else row.copy()
    return order, rgb, Tm, last, frag_px, vs, composited
