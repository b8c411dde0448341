"""Parity helpers: run the HIP path through its C ABI and compare with the
oracle, excluding the decisions an fp32 kernel cannot reproduce from an
fp64 reference ("fragile" items, decided from the oracle's own values).

Tolerances (the pages' rasterizer targets):
* mask, nnz, per-tile counts and sorted order: bit-exact on non-fragile
  pairs and pixels;
* images: max-abs 1e-4 on non-fragile pixels;
* gradients: relative L2 1e-3 per tensor.

Fragility windows (readings): a pair is fragile if, in fp64, its depth is
within a relative 1e-5 of the near plane, a box edge is within TAU_PX of
the image border it is tested against, or a box edge scaled to the 16-bit
grid lies within TAU_PX (in codes) of a grid point that decides a tile
crossing. TAU_PX = max(1e-5 px, 8 ulp32 of the coordinate) -- the
literal 1e-5 px is below fp32 resolution past 128 px. A pixel is fragile
if any entry it reaches has alpha within a relative 2e-5 of 1/255 (the
fp32 error of sigma near the threshold is a few 1e-6), if its stop test
is within a relative 1e-4 of 1e-4 (T is a product of up to hundreds of
rounded factors), or if its tile is touched by a fragile pair.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import raster as oraster
from oracle.intersect import TILE
from oracle.project import NEAR

IMG_TOL = 1e-4
GRAD_TOL = 1e-3
ALPHA_WIN = 2e-5   # relative window around alpha = 1/255
T_WIN = 1e-4       # relative window around the T = 1e-4 stop
Q16 = 65535


def ulp32(x):
    x = np.abs(np.asarray(x, np.float64)).astype(np.float32)
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


def tau_px(coord):
    return np.maximum(1e-5, 8.0 * ulp32(np.maximum(np.abs(coord), 1.0)))


def rel_l2(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def compare_rows(rg, ro):
    """GPU screen rows vs the oracle's fp32-stored rows of the same pairs.
    Both sides evaluate the projection in fp64 and round once, so every
    value agrees to within one fp32 ulp (of the conic's scale for the
    conic, of max(|x|, 0.5) for colours); depth bits are exact. Returns
    the largest differences in ulps."""
    rg = np.asarray(rg, np.float64)
    ro = np.asarray(ro, np.float64)
    out = {}
    for j, name in ((0, "u"), (1, "v"), (5, "opacity")):
        d = np.abs(rg[:, j] - ro[:, j]) / ulp32(ro[:, j])
        out[name] = float(d.max(initial=0))
    cs = ulp32(np.maximum(np.abs(ro[:, 2]), np.abs(ro[:, 4])))
    out["conic"] = float((np.abs(rg[:, 2:5] - ro[:, 2:5]) / cs[:, None]).max(initial=0))
    out["rgb"] = float((np.abs(rg[:, 7:] - ro[:, 7:]) / ulp32(np.maximum(np.abs(ro[:, 7:]), 0.5))).max(initial=0))
    np.testing.assert_array_equal(rg[:, 6].astype(np.float32).view(np.uint32),
                                  ro[:, 6].astype(np.float32).view(np.uint32))
    assert out["u"] <= 1 and out["v"] <= 1 and out["opacity"] <= 1, out
    assert out["conic"] <= 2 and out["rgb"] <= 1, out
    return out


def unpack_mask(words: np.ndarray, n_pairs: int) -> np.ndarray:
    w = np.asarray(words).view(np.uint64)
    bits = (w[:, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)
    return bits.astype(bool).ravel()[:n_pairs]


def _tile_fragile_edge(e, extent, is_min, tau):
    """Does moving edge e by +-tau change the tile its 16-bit code decides?"""
    s = np.float32(Q16) / np.float32(extent)
    lo = (np.asarray(e - tau, np.float64)).astype(np.float32) * s
    hi = (np.asarray(e + tau, np.float64)).astype(np.float32) * s
    f = np.floor if is_min else np.ceil
    qlo = np.clip(f(lo), 0, Q16).astype(np.int64)
    qhi = np.clip(f(hi), 0, Q16).astype(np.int64)
    D = TILE * Q16
    if is_min:
        return (qlo * extent) // D != (qhi * extent) // D
    return -((-(qlo * extent)) // D) != -((-(qhi * extent)) // D)


def fragile_pairs(scene: dict, proj) -> np.ndarray:
    """Boolean [C * N_pad]: pairs whose visibility, tile rect or key an fp32
    kernel may decide differently from the fp64 oracle."""
    N, C, W, H, Np = scene["N"], scene["C"], scene["W"], scene["H"], proj.N_pad
    frag = np.zeros(C * Np, bool)
    for c in range(C):
        pc = oracle.project_camera(scene["means"], scene["quats"], scene["log_scales"],
                                   scene["opacity_logits"], scene["sh"], scene["viewmats"][c],
                                   scene["Ks"][c], W, H, scene["sh_degree"])
        u, v, r, z = pc["u"], pc["v"], pc["r"], pc["z"]
        f = np.abs(z - NEAR) <= 1e-5 * NEAR
        with np.errstate(invalid="ignore"):
            for a, ext in ((u, W), (v, H)):
                t = tau_px(np.abs(a) + r)
                f |= np.abs(a + r) <= t          # box max edge vs 0
                f |= np.abs(a - r - ext) <= t    # box min edge vs extent
                lo = np.maximum(a - r, 0.0)
                hi = np.minimum(a + r, float(ext))
                vis = pc["visible"]
                f |= vis & _tile_fragile_edge(lo, ext, True, t)
                f |= vis & _tile_fragile_edge(hi, ext, False, t)
        f |= ~np.isfinite(u) | ~np.isfinite(v)
        frag[c * Np: c * Np + N] = f & (z > 0)
    return frag


def fragile_pixels(screen, flatten_ids, tile_offsets, C, W, H, tiles_touched=None):
    """Boolean [C, H, W]: pixels whose composite crosses a threshold within
    the fragility window (evaluated by the oracle's own walk)."""
    tiles_x = (W + TILE - 1) // TILE
    T_per = tiles_x * ((H + TILE - 1) // TILE)
    out = np.zeros((C, H, W), bool)
    screen = np.asarray(screen, np.float64)
    for t in range(C * T_per):
        c, tl = divmod(t, T_per)
        ii, jj = oraster._tile_pixels(tl, tiles_x, W, H)
        if tiles_touched is not None and tiles_touched[t]:
            out[c, ii, jj] = True
            continue
        ids = np.asarray(flatten_ids[int(tile_offsets[t]):int(tile_offsets[t + 1])], np.int64)
        if ids.size == 0:
            continue
        rows = screen[ids]
        _, _, _, _, rec = oraster._walk_tile(rows, jj + 0.5, ii + 0.5, record=True)
        a = rec["alpha"]
        Tn = rec["Tb"] * (1.0 - a)
        # entries a pixel reaches: up to and including the one that stops it
        stops = (a >= oraster.ALPHA_MIN) & (Tn < oraster.T_STOP) & ~rec["comp"]
        first = np.where(stops.any(1), stops.argmax(1), a.shape[1])
        reached = np.arange(a.shape[1])[None, :] <= first[:, None]
        bad = reached & (np.abs(a - oraster.ALPHA_MIN) <= ALPHA_WIN * oraster.ALPHA_MIN)
        bad |= reached & (a >= oraster.ALPHA_MIN) & \
            (np.abs(Tn - oraster.T_STOP) <= T_WIN * oraster.T_STOP)
        out[c, ii, jj] = bad.any(axis=1)
    return out


def to_dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def u32_as_i32(a):
    return np.ascontiguousarray(np.asarray(a, np.uint32)).view(np.int32)


def check_step(sc, out, grads_o, ref, label=""):
    """A whole GPU step (``Rasterizer.step``-shaped dict) against the oracle
    step (``oracle.loss_and_grads(sc, rows32=True)``): nnz and the mask
    bit-exact outside fragile pairs; the sorted lists bit-exact as pair
    ids once fragile pairs' entries are removed; images max-abs 1e-4 and
    last_ids exact outside fragile pixels; gradients relative L2 1e-3.
    Returns a report dict."""
    proj, isect = ref["proj"], ref["isect"]
    C, W, H = sc["C"], sc["W"], sc["H"]
    frag = fragile_pairs(sc, proj)
    p, it = out["proj"], out["isect"]
    n_pairs = C * proj.N_pad
    gvis = unpack_mask(p.mask.cpu().numpy(), n_pairs)
    ovis = np.zeros(n_pairs, bool)
    ovis[proj.pairs] = True
    assert not ((gvis != ovis) & ~frag).any(), "mask differs on a non-fragile pair"
    gp = np.flatnonzero(gvis)
    ids_g = it.flatten_ids.cpu().numpy().view(np.uint32).astype(np.int64)
    lists_g = gp[ids_g]
    lists_o = proj.pairs[isect.flatten_ids.astype(np.int64)]
    np.testing.assert_array_equal(lists_g[~frag[lists_g]], lists_o[~frag[lists_o]])
    # tiles whose full lists (fragile pairs kept) differ are left out whole
    toff_g = it.tile_offsets.cpu().numpy()
    tiles_touched = np.zeros(isect.tile_offsets.size - 1, bool)
    for t in range(tiles_touched.size):
        a = gp[ids_g[toff_g[t]:toff_g[t + 1]]]
        o0, o1 = isect.tile_offsets[t], isect.tile_offsets[t + 1]
        b = proj.pairs[isect.flatten_ids[o0:o1].astype(np.int64)]
        tiles_touched[t] = not np.array_equal(a, b)
    if not frag.any():
        np.testing.assert_array_equal(toff_g, isect.tile_offsets)
    fpx = fragile_pixels(proj.screen, isect.flatten_ids, isect.tile_offsets, C, W, H,
                         tiles_touched)
    ok = ~fpx
    e_rgb = float(np.abs(out["rgb"].cpu().numpy() - ref["rgb"])[ok].max(initial=0))
    e_T = float(np.abs(out["T"].cpu().numpy() - ref["T"])[ok].max(initial=0))
    last_bad = int((out["last"].cpu().numpy() != ref["last"])[ok].sum())
    errs = {k: rel_l2(out["grads"][k].cpu().numpy(), grads_o[k]) for k in grads_o}
    rep = dict(nnz=p.nnz, n_isects=it.n_isects, oracle_nnz=proj.nnz,
               oracle_isects=isect.n_isects, fragile_pairs=int(frag.sum()),
               tiles_differing=int(tiles_touched.sum()), fragile_px=int(fpx.sum()),
               rgb_err=e_rgb, T_err=e_T, last_ids_diff=last_bad, grads=errs)
    print(f"{label}: {rep}")
    assert e_rgb <= IMG_TOL and e_T <= IMG_TOL, rep
    assert last_bad == 0, rep
    assert max(errs.values()) <= GRAD_TOL, rep
    # the exclusions stay small: below 0.5% of pixels, 0.1% of pairs
    assert fpx.sum() <= 0.005 * fpx.size + 4, rep
    assert frag.sum() <= 0.001 * proj.nnz + 4, rep
    return rep
