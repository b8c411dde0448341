"""HIP path vs the fp64 oracle, stage by stage and end to end, through the
C ABI (libgs.so). Scenes: the small seeded workloads (several tiles, a
ragged tile tail, 1-3 cameras, SH degrees 0-3)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import fullsize as F
from tests import parity as P

pytestmark = pytest.mark.gpu

gsd = pytest.importorskip("gaussian_splatting_differentiable_project_amd")

SCENES = list(workloads.SMALL.keys())

# More than 64 cameras: the compaction reads the mask words 64 cameras at a
# time. A wide view (every pair visible: dense waves, each lane walking the
# cameras) and a narrow one (about a quarter visible: sparse waves, pairs
# queued camera by camera). 64 cameras: the most the bound-test mask pass
# takes (its queue entries hold the camera in 6 bits).
MANY_CAMS = {
    "ring-64cam-narrow": workloads.SceneSpec("sh1-3000-64cam-40x32-narrow", 3000, 1, 64, 40, 32,
                                             120.0, 2.0, -3.0, 0.4, 5.0, seed=2008),
    "ring-70cam-wide": workloads.SceneSpec("sh1-1500-70cam-40x32-wide", 1500, 1, 70, 40, 32, 30.0,
                                           1.0, -2.8, 0.4, 5.0, seed=2006),
    "ring-70cam-narrow": workloads.SceneSpec("sh1-3000-70cam-40x32-narrow", 3000, 1, 70, 40, 32,
                                             120.0, 2.0, -3.0, 0.4, 5.0, seed=2007),
}


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return gsd.load()


_cache = {}


def reference(name):
    """Oracle results for one small scene (computed once per session), with
    the screen rows stored in fp32 as the method stores them."""
    if name not in _cache:
        sc = workloads.make_scene(workloads.SMALL[name] if name in workloads.SMALL
                                  else MANY_CAMS[name])
        L, grads, ref = oracle.loss_and_grads(sc, rows32=True)
        _cache[name] = (sc, grads, ref)
    return _cache[name]


def gpu_scene(sc):
    return gsd.Scene.from_numpy(sc, "cuda")


@pytest.mark.parametrize("name", SCENES + list(MANY_CAMS))
def test_project_mask_and_rows(lib, name):
    sc, _, ref = reference(name)
    proj = ref["proj"]
    r = gsd.Rasterizer()
    p = r.project(gpu_scene(sc))
    torch.cuda.synchronize()
    n_pairs = sc["C"] * proj.N_pad
    vis_gpu = P.unpack_mask(p.mask.cpu().numpy(), n_pairs)
    frag = P.fragile_pairs(sc, proj)
    diff = vis_gpu != proj.visible_pairs
    print(f"{name}: nnz gpu={p.nnz} oracle={proj.nnz} fragile={int(frag.sum())} "
          f"mask diffs={int(diff.sum())} (fragile among them={int((diff & frag).sum())})")
    assert not (diff & ~frag).any(), np.flatnonzero(diff & ~frag)[:10]
    if not diff.any():
        assert p.nnz == proj.nnz
        np.testing.assert_array_equal(p.wg_count.cpu().numpy().view(np.uint32), proj.wg_count)
        np.testing.assert_array_equal(p.wg_scan.cpu().numpy().view(np.uint32), proj.wg_scan)
    # work-group counts are the popcounts of the GPU's own mask; the scan is their prefix
    wgc = p.wg_count.cpu().numpy().view(np.uint32).astype(np.int64)
    np.testing.assert_array_equal(wgc, vis_gpu.reshape(-1, 128).sum(1))
    np.testing.assert_array_equal(p.wg_scan.cpu().numpy().view(np.uint32).astype(np.int64),
                                  np.cumsum(wgc) - wgc)
    assert p.nnz == int(vis_gpu.sum())
    assert p.cam_offsets[-1] == p.nnz
    # screen rows of pairs visible on both sides
    gpu_pairs = np.flatnonzero(vis_gpu)
    both = np.intersect1d(gpu_pairs, proj.pairs)
    gi = np.searchsorted(gpu_pairs, both)
    oi = np.searchsorted(proj.pairs, both)
    rows_g = p.screen.cpu().numpy().astype(np.float64)[gi]
    rows_o = proj.screen[oi]
    errs = P.compare_rows(rows_g, rows_o)
    print(f"{name}: row errors in ulps {errs}")
    # AABB16 codes: exact outside code-fragile pairs (whose fp32 product
    # lies within a relative 1e-9 of an integer), never more than one code
    # apart; tile rectangles equal off fragile pairs
    ag = p.aabb16.cpu().numpy().view(np.uint32)[gi].astype(np.int64)
    ao = proj.aabb16[oi].astype(np.int64)
    code_frag = F.OracleScene(sc, workers=1).code_frag[both]
    for w in range(2):
        for sh in (0, 16):
            d = np.abs(((ag[:, w] >> sh) & 0xFFFF) - ((ao[:, w] >> sh) & 0xFFFF))
            assert d.max(initial=0) <= 1
            assert not (d[~code_frag] != 0).any(), both[(d != 0) & ~code_frag][:10]
    print(f"{name}: code-fragile pairs {int(code_frag.sum())} of {both.size}")
    rg = np.stack(tile_rects(ag, sc["W"], sc["H"]), 1)
    ro = np.stack(tile_rects(ao, sc["W"], sc["H"]), 1)
    bad = (rg != ro).any(1) & ~frag[both]
    assert not bad.any(), both[bad][:10]


def tile_rects(a, W, H):
    return oracle.tile_rects_from_aabb16(a.astype(np.uint32), W, H)


@pytest.mark.parametrize("name", SCENES)
def test_intersect_sort_bit_exact(lib, name):
    """Stage-isolated: the oracle's own fp32 rows and box codes go in, so
    counts, keys, order and tile ranges must match bit for bit."""
    sc, _, ref = reference(name)
    check_intersect(sc, ref["proj"], ref["isect"])


@pytest.mark.parametrize("with_keys", [False, True], ids=["ids", "ids+keys"])
@pytest.mark.parametrize("group", [16, 32])
@pytest.mark.parametrize("name", ["sh2-dense", "wide-2cam-4096px"])
def test_intersect_expand_groups(lib, name, group, with_keys, monkeypatch):
    """Both group sizes of the list expansion (64- and 128-byte groups;
    the library takes 128 only for long runs per chunk and tile, which
    only scenes of over 8M segments reach), forced through its override,
    with and without the 64-bit keys: the same lists as the oracle."""
    if name in WIDE:
        sc = workloads.make_scene(WIDE[name])
        proj = oracle.project(sc)
        proj.screen = proj.screen.astype(np.float32).astype(np.float64)
        isect = oracle.intersect(proj, sc["W"], sc["H"])
    else:
        sc, _, ref = reference(name)
        proj, isect = ref["proj"], ref["isect"]
    monkeypatch.setenv("GS_EXPAND_GROUP", str(group))
    check_intersect(sc, proj, isect, with_keys=with_keys)


# Scenes with many tiles (over 2^16 tile ids), so that the sort by tile id
# takes its wider first digit and, past 2^18 tiles, more than one further
# pass. Only projection and intersection are compared. The 65520-pixel-wide
# one has tile rows too long for a 32-bit (row, first tile, width) segment
# key, so its entries are sorted by tile id directly; the others go through
# tile-row segments.
WIDE = {
    "wide-tilepath-2cam-65520x4096": workloads.SceneSpec("sh0-2000-2cam-65520x4096", 2000, 0,
                                                         2, 65520, 4096, 3547.0, 2.0, -3.5,
                                                         0.5, 5.0, seed=2103),
    "wide-2cam-4096px": workloads.SceneSpec("sh0-3000-2cam-4096px", 3000, 0, 2, 4096, 4096,
                                            3547.0, 2.0, -3.5, 0.5, 5.0, seed=2101),
    "wide-5cam-4096x4000": workloads.SceneSpec("sh0-2000-5cam-4096x4000", 2000, 0, 5, 4096,
                                               4000, 3547.0, 2.0, -3.5, 0.5, 5.0, seed=2102),
}


@pytest.mark.parametrize("name", list(WIDE))
def test_intersect_sort_many_tiles(lib, name):
    sc = workloads.make_scene(WIDE[name])
    proj = oracle.project(sc)
    proj.screen = proj.screen.astype(np.float32).astype(np.float64)
    isect = oracle.intersect(proj, sc["W"], sc["H"])
    n_tiles = isect.tile_offsets.size - 1
    print(f"{name}: tiles={n_tiles} nnz={proj.nnz} n_isects={isect.n_isects}")
    assert n_tiles > (1 << 16)
    check_intersect(sc, proj, isect)


# About 9.2M visible pairs: past 8192 emit blocks of one 512-pair
# sub-batch, so each emit block walks three sub-batches and its rounds
# cross sub-batch boundaries (the smaller scenes give every block a single
# sub-batch). About 60M entries; the oracle needs about 30 s and 8 GB.
MULTI = workloads.SceneSpec("sh0-9.5M-1080p", 9_500_000, 0, 1, 1920, 1080, 1100.0, 2.0, -4.5, 0.5,
                            5.0, seed=2105)


def test_intersect_sort_multi_subbatch(lib):
    sc = workloads.make_scene(MULTI)
    proj = oracle.project(sc)
    proj.screen = proj.screen.astype(np.float32).astype(np.float64)
    isect = oracle.intersect(proj, sc["W"], sc["H"])
    print(f"nnz={proj.nnz} n_isects={isect.n_isects}")
    assert proj.nnz > 8192 * 512 * 2
    check_intersect(sc, proj, isect)


# Depths from about 2 to 10 (across 8.0, where the fp32 exponent and the
# key's top byte change), so the depth sort needs its fourth pass; the
# other small scenes keep every depth within [2, 8) and skip it.
DEEP = workloads.SceneSpec("sh1-3000-2cam-200x150-deep", 3000, 1, 2, 200, 150, 180.0, 4.0,
                           -3.0, 0.5, 6.0, seed=2103)


def test_intersect_sort_wide_depth_range(lib):
    sc = workloads.make_scene(DEEP)
    proj = oracle.project(sc)
    proj.screen = proj.screen.astype(np.float32).astype(np.float64)
    isect = oracle.intersect(proj, sc["W"], sc["H"])
    bits = proj.screen[:, 6].astype(np.float32).view(np.uint32)
    print(f"depth keys {bits.min():#x}..{bits.max():#x} nnz={proj.nnz} n_isects={isect.n_isects}")
    assert (int(bits.min()) ^ int(bits.max())) >> 24 != 0
    check_intersect(sc, proj, isect)


# Tile counts around the limits of the rank-based launch order (one chunk of
# 4,096 keys, several chunks, exactly 16,384 tiles) and just past it, where
# the order comes from two radix passes instead. Most tiles are empty, so
# ties (kept in increasing tile id) dominate.
ORDER_SIZES = {
    "tiles-4096": workloads.SceneSpec("sh0-3000-1024px", 3000, 0, 1, 1024, 1024, 887.0, 2.0,
                                      -3.5, 0.5, 5.0, seed=2107),
    "tiles-4160": workloads.SceneSpec("sh0-3000-1024x1040", 3000, 0, 1, 1024, 1040, 887.0, 2.0,
                                      -3.5, 0.5, 5.0, seed=2108),
    "tiles-16384": workloads.SceneSpec("sh0-3000-2048px", 3000, 0, 1, 2048, 2048, 1773.0, 2.0,
                                       -3.5, 0.5, 5.0, seed=2109),
    "tiles-16512": workloads.SceneSpec("sh0-3000-2064x2048", 3000, 0, 1, 2064, 2048, 1773.0,
                                       2.0, -3.5, 0.5, 5.0, seed=2110),
}


@pytest.mark.parametrize("name", list(ORDER_SIZES))
def test_intersect_launch_order_sizes(lib, name):
    sc = workloads.make_scene(ORDER_SIZES[name])
    proj = oracle.project(sc)
    proj.screen = proj.screen.astype(np.float32).astype(np.float64)
    isect = oracle.intersect(proj, sc["W"], sc["H"])
    n_tiles = isect.tile_offsets.size - 1
    assert n_tiles == int(name.split("-")[1])
    print(f"{name}: nnz={proj.nnz} n_isects={isect.n_isects}")
    check_intersect(sc, proj, isect)


def check_intersect(sc, proj, isect, with_keys=True):
    screen = P.to_dev(proj.screen.astype(np.float32))
    aabb = P.to_dev(P.u32_as_i32(proj.aabb16))
    cam = [0] + [int(np.searchsorted(proj.cam, c)) for c in range(1, sc["C"])] + [proj.nnz]
    C, W, H = sc["C"], sc["W"], sc["H"]
    n_tiles = isect.tile_offsets.size - 1
    ws_bytes = gsd.load().gs_intersect_workspace_bytes(C, W, H, proj.nnz, isect.n_isects)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ids = torch.empty(max(isect.n_isects, 1), dtype=torch.int32, device="cuda")
    keys = torch.empty(max(isect.n_isects, 1), dtype=torch.int64, device="cuda")
    toff = torch.empty(n_tiles + 1, dtype=torch.int64, device="cuda")
    order = torch.empty(n_tiles, dtype=torch.int32, device="cuda")
    st, n_is, need = gsd.gs_intersect(C, W, H, proj.nnz, screen, aabb, cam, ws, ws_bytes, ids,
                                      ids.numel(), toff, keys if with_keys else None, order)
    torch.cuda.synchronize()
    assert st == 0, gsd.status_str(st)
    assert n_is == isect.n_isects
    np.testing.assert_array_equal(toff.cpu().numpy(), isect.tile_offsets)
    np.testing.assert_array_equal(ids.cpu().numpy()[:n_is].view(np.uint32), isect.flatten_ids)
    if with_keys:
        np.testing.assert_array_equal(keys.cpu().numpy()[:n_is].view(np.uint64), isect.sorted_keys)
    np.testing.assert_array_equal(order.cpu().numpy(), launch_order(isect.tile_offsets))


def launch_order(tile_offsets):
    """The raster launch order the library documents: tiles by decreasing
    entry count (saturated at 65535), ties by increasing tile id."""
    cnt = np.minimum(np.diff(tile_offsets), 0xFFFF)
    return np.argsort(-cnt, kind="stable").astype(np.int32)


@pytest.mark.parametrize("ordered", [False, True], ids=["id-order", "heavy-first"])
@pytest.mark.parametrize("name", SCENES)
def test_raster_fwd_stage(lib, name, ordered):
    """Stage-isolated forward: oracle rows (fp32) and oracle tile lists in,
    tiles launched in id order or in the heavy-first order."""
    check_raster_fwd(name, ordered)


# Every width of the forward kernel (these scenes alone take one pixel per
# lane).
@pytest.mark.parametrize("ppt", [1, 2, 4])
@pytest.mark.parametrize("name", ["tiny", "multicam", "sh2-dense"])
def test_raster_fwd_widths(lib, name, ppt, monkeypatch):
    monkeypatch.setenv("GS_RASTER_PPT_FWD", str(ppt))
    check_raster_fwd(name, True)


def check_raster_fwd(name, ordered):
    sc, _, ref = reference(name)
    proj, isect = ref["proj"], ref["isect"]
    C, W, H = sc["C"], sc["W"], sc["H"]
    rows32 = proj.screen.astype(np.float32)
    rgb_o, T_o, last_o, _ = oracle.rasterize_fwd(rows32.astype(np.float64), isect.flatten_ids,
                                                 isect.tile_offsets, C, W, H)
    rgb = torch.empty(C, H, W, 3, device="cuda")
    T = torch.empty(C, H, W, device="cuda")
    last = torch.empty(C, H, W, dtype=torch.int32, device="cuda")
    order = P.to_dev(launch_order(isect.tile_offsets)) if ordered else None
    st = gsd.gs_rasterize_fwd(C, W, H, P.to_dev(rows32), P.to_dev(P.u32_as_i32(isect.flatten_ids)),
                              P.to_dev(isect.tile_offsets), order, None, rgb, T, None, last)
    torch.cuda.synchronize()
    assert st == 0
    frag = P.fragile_pixels(rows32, isect.flatten_ids, isect.tile_offsets, C, W, H)
    ok = ~frag
    e_rgb = np.abs(rgb.cpu().numpy() - rgb_o)[ok].max()
    e_T = np.abs(T.cpu().numpy() - T_o)[ok].max()
    lg = last.cpu().numpy()
    print(f"{name}: fragile px={int(frag.sum())}/{frag.size} rgb err={e_rgb:.2e} T err={e_T:.2e} "
          f"last mismatches={int((lg != last_o)[ok].sum())}")
    assert e_rgb <= P.IMG_TOL and e_T <= P.IMG_TOL
    np.testing.assert_array_equal(lg[ok], last_o[ok])


# 32,768 tiles: past the tile count from which the forward runs four pixels
# per lane (one wave per tile).
MANY_TILES = workloads.SceneSpec("sh0-4000-2cam-2048px", 4000, 0, 2, 2048, 2048, 1773.0, 2.0,
                                 -3.5, 0.5, 5.0, seed=2106)


def test_raster_fwd_stage_many_tiles(lib):
    sc = workloads.make_scene(MANY_TILES)
    proj = oracle.project(sc)
    rows32 = proj.screen.astype(np.float32)
    proj.screen = rows32.astype(np.float64)
    isect = oracle.intersect(proj, sc["W"], sc["H"])
    C, W, H = sc["C"], sc["W"], sc["H"]
    assert isect.tile_offsets.size - 1 >= 16384
    rgb_o, T_o, last_o, _ = oracle.rasterize_fwd(proj.screen, isect.flatten_ids,
                                                 isect.tile_offsets, C, W, H)
    rgb = torch.empty(C, H, W, 3, device="cuda")
    T = torch.empty(C, H, W, device="cuda")
    last = torch.empty(C, H, W, dtype=torch.int32, device="cuda")
    order = P.to_dev(launch_order(isect.tile_offsets))
    st = gsd.gs_rasterize_fwd(C, W, H, P.to_dev(rows32), P.to_dev(P.u32_as_i32(isect.flatten_ids)),
                              P.to_dev(isect.tile_offsets), order, None, rgb, T, None, last)
    torch.cuda.synchronize()
    assert st == 0
    frag = P.fragile_pixels(rows32, isect.flatten_ids, isect.tile_offsets, C, W, H)
    ok = ~frag
    e_rgb = np.abs(rgb.cpu().numpy() - rgb_o)[ok].max()
    e_T = np.abs(T.cpu().numpy() - T_o)[ok].max()
    lg = last.cpu().numpy()
    print(f"fragile px={int(frag.sum())}/{frag.size} rgb err={e_rgb:.2e} T err={e_T:.2e}")
    assert e_rgb <= P.IMG_TOL and e_T <= P.IMG_TOL
    np.testing.assert_array_equal(lg[ok], last_o[ok])


@pytest.mark.parametrize("ordered", [False, True], ids=["id-order", "heavy-first"])
@pytest.mark.parametrize("name", SCENES)
def test_raster_bwd_stage(lib, name, ordered):
    check_raster_bwd(name, ordered)


# Every width of the backward kernel (the library picks one by tile count:
# these scenes alone would only reach one pixel per lane).
@pytest.mark.parametrize("ppt", [1, 2, 4])
@pytest.mark.parametrize("name", ["tiny", "multicam", "sh2-dense"])
def test_raster_bwd_widths(lib, name, ppt, monkeypatch):
    monkeypatch.setenv("GS_RASTER_PPT_BWD", str(ppt))
    check_raster_bwd(name, True)


def check_raster_bwd(name, ordered):
    sc, _, ref = reference(name)
    proj, isect = ref["proj"], ref["isect"]
    C, W, H = sc["C"], sc["W"], sc["H"]
    rows32 = proj.screen.astype(np.float32)
    rows64 = rows32.astype(np.float64)
    _, T_o, last_o, _ = oracle.rasterize_fwd(rows64, isect.flatten_ids, isect.tile_offsets, C, W, H)
    vs_o = oracle.rasterize_bwd(rows64, isect.flatten_ids, isect.tile_offsets, C, W, H,
                                sc["v_rgb"], sc["v_T"])
    # forward state from the GPU's own forward on the same inputs
    d_rows = P.to_dev(rows32)
    d_ids = P.to_dev(P.u32_as_i32(isect.flatten_ids))
    d_toff = P.to_dev(isect.tile_offsets)
    rgb = torch.empty(C, H, W, 3, device="cuda")
    T = torch.empty(C, H, W, device="cuda")
    last = torch.empty(C, H, W, dtype=torch.int32, device="cuda")
    order = P.to_dev(launch_order(isect.tile_offsets)) if ordered else None
    assert gsd.gs_rasterize_fwd(C, W, H, d_rows, d_ids, d_toff, order, None, rgb, T, None, last) == 0
    v_screen = torch.empty(proj.nnz, 10, device="cuda")
    st = gsd.gs_rasterize_bwd(C, W, H, proj.nnz, d_rows, d_ids, d_toff, order, None, T, last,
                              P.to_dev(sc["v_rgb"]), P.to_dev(sc["v_T"]), None, v_screen, None)
    torch.cuda.synchronize()
    assert st == 0
    vg = v_screen.cpu().numpy()
    errs = {j: P.rel_l2(vg[:, j], vs_o[:, j]) for j in (0, 1, 2, 3, 4, 5, 7, 8, 9)}
    print(f"{name}: v_screen rel L2 per column {errs}")
    assert max(errs.values()) <= P.GRAD_TOL
    assert np.all(vg[:, 6] == 0)


@pytest.mark.parametrize("name", SCENES)
def test_project_bwd_stage(lib, name):
    """Stage-isolated: the oracle's mask/scan and its v_screen (fp32) in."""
    sc, grads_unused, ref = reference(name)
    proj = ref["proj"]
    vs32 = ref["v_screen"].astype(np.float32)
    g_o = oracle.project_bwd(sc, proj, vs32.astype(np.float64))
    s = gpu_scene(sc)
    r = gsd.Rasterizer()
    p = gsd.Projected(proj.nnz, [], P.to_dev(proj.mask.view(np.int64)),
                      P.to_dev(proj.wg_count.view(np.int32)), P.to_dev(proj.wg_scan.view(np.int32)),
                      None, None)
    g = r.project_bwd(s, p, P.to_dev(vs32))
    torch.cuda.synchronize()
    errs = {k: P.rel_l2(g[k].cpu().numpy(), g_o[k]) for k in g_o}
    print(f"{name}: grad rel L2 {errs}")
    assert max(errs.values()) <= P.GRAD_TOL
    # accumulate: a second call adds the same gradients
    g2 = r.project_bwd(s, p, P.to_dev(vs32), grads={k: v.clone() for k, v in g.items()},
                       accumulate=True)
    torch.cuda.synchronize()
    for k in g:
        np.testing.assert_allclose(g2[k].cpu().numpy(), 2 * g[k].cpu().numpy(), rtol=1e-6,
                                   atol=1e-30)


@pytest.mark.parametrize("name", SCENES + list(MANY_CAMS))
def test_end_to_end(lib, name):
    """Whole step on the GPU vs the whole oracle step."""
    sc, grads_o, ref = reference(name)
    r = gsd.Rasterizer()
    s = gpu_scene(sc)
    out = r.step(s, P.to_dev(sc["v_rgb"]), P.to_dev(sc["v_T"]))
    torch.cuda.synchronize()
    P.check_step(sc, out, grads_o, ref, name)
