"""Pins for the oracle's tile intersection, key sort and tile ranges:
brute-force tile coverage from the decoded boxes, sort invariants and
per-tile counts."""
import numpy as np
import pytest

import oracle
import workloads
from oracle.intersect import tile_rects_from_aabb16


def _decoded_overlap_bruteforce(q0, q1, extent, n_tiles):
    """Tiles [16 t, 16 t + 16) met by the decoded box [q0 e/65535, q1 e/65535],
    by exact integer comparison per tile (no floor/ceil)."""
    t = np.arange(n_tiles)
    return (q0 * extent < 16 * (t + 1) * 65535) & (q1 * extent > 16 * t * 65535)


@pytest.mark.parametrize("W,H", [(128, 128), (97, 61), (1920, 1080), (7680, 7680), (65535, 17)])
def test_tile_rect_matches_bruteforce(W, H):
    rng = np.random.default_rng(W + H)
    n = 3000
    qx0 = rng.integers(0, 65535, n)
    qx1 = np.minimum(65535, qx0 + 1 + rng.integers(0, 4000, n))
    qy0 = rng.integers(0, 65535, n)
    qy1 = np.minimum(65535, qy0 + 1 + rng.integers(0, 4000, n))
    # edge cases: boxes on exact tile boundaries and the code range ends
    qx0[:4] = [0, 0, 65535 - 1, (16 * 65535) // W]
    qx1[:4] = [1, 65535, 65535, qx0[3] + 1]
    aabb = np.stack([(qx0 | (qy0 << 16)), (qx1 | (qy1 << 16))], 1).astype(np.uint32)
    tx0, ty0, tx1, ty1 = tile_rects_from_aabb16(aabb, W, H)
    ntx, nty = (W + 15) // 16, (H + 15) // 16
    for i in range(n):
        bx = np.flatnonzero(_decoded_overlap_bruteforce(qx0[i], qx1[i], W, ntx))
        by = np.flatnonzero(_decoded_overlap_bruteforce(qy0[i], qy1[i], H, nty))
        assert (bx.min(), bx.max() + 1) == (tx0[i], tx1[i]), i
        assert (by.min(), by.max() + 1) == (ty0[i], ty1[i]), i
        assert tx1[i] - tx0[i] >= 1 and ty1[i] - ty0[i] >= 1


@pytest.mark.parametrize("name", ["tiny", "multicam", "sh1-odd-n", "sh3-ragged"])
def test_sort_invariants_and_ranges(name):
    sc = workloads.make_scene(workloads.SMALL[name])
    pr = oracle.project(sc)
    it = oracle.intersect(pr, sc["W"], sc["H"])
    keys, ids, offs = it.sorted_keys, it.flatten_ids.astype(np.int64), it.tile_offsets
    assert it.n_isects == keys.size == ids.size == int(offs[-1])
    assert np.all(keys[1:] >= keys[:-1])
    # within equal keys, slots strictly ascending (stable: emission order)
    same = keys[1:] == keys[:-1]
    assert np.all(ids[1:][same] > ids[:-1][same])
    # the sorted (key, slot) pairs are a permutation of the emitted ones
    assert np.array_equal(np.sort(it.keys), keys)
    emitted_slots = np.repeat(np.arange(pr.nnz), it.counts)
    assert np.array_equal(np.sort(ids), emitted_slots)
    # low word = the slot's depth bits; high word = the tile containing it
    zb = pr.z32.view(np.uint32)
    assert np.array_equal((keys & np.uint64(0xFFFFFFFF)).astype(np.uint32), zb[ids])
    tile_of_pos = np.repeat(np.arange(offs.size - 1), np.diff(offs))
    assert np.array_equal((keys >> np.uint64(32)).astype(np.int64), tile_of_pos)
    # per-tile counts from the rectangles, tile by tile (brute force)
    tx0, ty0, tx1, ty1 = it.rects
    T = it.T
    counts = np.zeros(pr.C * T, np.int64)
    for s in range(pr.nnz):
        c = int(pr.cam[s])
        for ty in range(ty0[s], ty1[s]):
            for tx in range(tx0[s], tx1[s]):
                counts[c * T + ty * it.tiles_x + tx] += 1
    assert np.array_equal(np.diff(offs), counts)
    # each tile's list is exactly its covering slots, sorted by (depth, slot)
    for t in range(0, pr.C * T, max(1, pr.C * T // 13)):
        c, tl = divmod(t, T)
        ty, tx = divmod(tl, it.tiles_x)
        cover = np.flatnonzero((pr.cam == c) & (tx0 <= tx) & (tx < tx1) & (ty0 <= ty) & (ty < ty1))
        order = cover[np.lexsort((cover, zb[cover]))]
        assert np.array_equal(ids[offs[t]:offs[t + 1]], order)
