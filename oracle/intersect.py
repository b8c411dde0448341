"""Tile intersection, key sort and tile ranges (oracle).

[VRAM] "The 4 GiB rule and the 2^31 limit": the number of (splat, tile)
intersections is counted exactly in 64 bits before anything is sized by
it; [VRAM] per-element buffer cost table: each intersection carries an
8-byte key (tile_id << 32) | depth. [BWD] section 4: the forward keeps the
tile offsets and the flattened intersection list for the backward.

Readings:
* tile rectangle of a visible pair, from its 16-bit box codes with
  integer arithmetic only: the decoded edge is q * extent / 65535, so with
  16-pixel tiles tx0 = floor(qx0 W / (16 * 65535)) and the exclusive end
  tx1 = ceil(qx1 W / (16 * 65535)); the same for y with H.
* emission order: slots in increasing order, each slot's tiles row-major.
* key = (c * T + ty * tiles_x + tx) << 32 | bits(z32), T = tiles per camera.
  Positive float32 depths order like their bit patterns.
* sort: a stable sort of the keys (a stable LSD radix sort has this
  result); equal keys keep emission order, i.e. increasing slot.
* tile_offsets[t] = first sorted position whose tile id is >= t, for
  t = 0..C*T (so diff() gives per-tile counts and the last entry is the
  total).
"""
from __future__ import annotations

import numpy as np

__all__ = ["TILE", "tile_rects_from_aabb16", "intersect", "Intersection"]

TILE = 16
Q16 = 65535


def tile_rects_from_aabb16(aabb16: np.ndarray, W: int, H: int):
    """(tx0, ty0, tx1, ty1) int64 per slot; tx1/ty1 exclusive."""
    w = np.asarray(aabb16).astype(np.int64)
    qx0, qy0 = w[:, 0] & 0xFFFF, w[:, 0] >> 16
    qx1, qy1 = w[:, 1] & 0xFFFF, w[:, 1] >> 16
    D = TILE * Q16
    tx0 = (qx0 * W) // D
    ty0 = (qy0 * H) // D
    tx1 = -((-(qx1 * W)) // D)
    ty1 = -((-(qy1 * H)) // D)
    return tx0, ty0, tx1, ty1


class Intersection:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def intersect(proj, W: int, H: int) -> Intersection:
    """Counts, keys, stable sort and tile ranges for a ``Projection``."""
    C = proj.C
    ntx, nty = (W + TILE - 1) // TILE, (H + TILE - 1) // TILE
    T = ntx * nty
    tx0, ty0, tx1, ty1 = tile_rects_from_aabb16(proj.aabb16, W, H)
    wx = np.maximum(tx1 - tx0, 0)
    wy = np.maximum(ty1 - ty0, 0)
    counts = wx * wy
    n_isects = int(counts.sum())
    nnz = counts.size
    slot = np.repeat(np.arange(nnz, dtype=np.int64), counts)
    first = np.cumsum(counts) - counts
    k = np.arange(n_isects, dtype=np.int64) - np.repeat(first, counts)
    wxs = np.repeat(wx, counts)
    ty = np.repeat(ty0, counts) + k // np.maximum(wxs, 1)
    tx = np.repeat(tx0, counts) + k % np.maximum(wxs, 1)
    tile = np.repeat(proj.cam.astype(np.int64), counts) * T + ty * ntx + tx
    zbits = proj.z32.view(np.uint32).astype(np.uint64)
    keys = (tile.astype(np.uint64) << np.uint64(32)) | zbits[slot]
    order = np.argsort(keys, kind="stable")
    sorted_keys = keys[order]
    flatten_ids = slot[order].astype(np.uint32)
    tile_offsets = np.searchsorted(sorted_keys >> np.uint64(32),
                                   np.arange(C * T + 1, dtype=np.uint64), side="left").astype(np.int64)
    return Intersection(counts=counts, n_isects=n_isects, keys=keys,
                        sorted_keys=sorted_keys, flatten_ids=flatten_ids,
                        tile_offsets=tile_offsets, tiles_x=ntx, tiles_y=nty, T=T,
                        rects=(tx0, ty0, tx1, ty1))
