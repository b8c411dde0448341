"""The C-ABI library loads on the CPU host and exports what include/gs.h
declares; host-only entry points (sizes, status text) behave as stated.
No kernel is launched here."""
from __future__ import annotations

import ctypes
import json
import os
import re

import numpy as np
import pytest

import gaussian_splatting_differentiable_project_amd as gsd
from gaussian_splatting_differentiable_project_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gs.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gs_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    try:
        return gsd.load()
    except ImportError as e:
        pytest.fail(f"libgs.so must be built before the tests: {e}")


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == {"gs_status_str", "gs_version", "gs_readback_status",
                          "gs_tile_offsets_check", "gs_pad_n", "gs_project_workspace_bytes",
                          "gs_intersect_workspace_bytes", "gs_project", "gs_project_noalloc",
                          "gs_intersect",
                          "gs_rasterize_fwd", "gs_rasterize_bwd", "gs_project_bwd",
                          "gs_project_bwd_adam", "gs_arena_plan", "gs_profile_enable",
                          "gs_profile_disable",
                          "gs_profile_reset",
                          "gs_profile_query", "gs_valu_probe"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(_lib.EXPORTS) == set(names)


def test_status_strings_and_version(lib):
    assert lib.gs_version() >= 100
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert gsd.status_str(st) and gsd.status_str(st) != "unknown status"
    assert gsd.status_str(-99) == "unknown status"


def test_pad_n(lib):
    assert [gsd.pad_n(n) for n in (0, 1, 127, 128, 129, 4096, 3001)] == \
        [0, 128, 128, 128, 256, 4096, 3072]


def test_workspace_sizes_monotone(lib):
    f = lib.gs_intersect_workspace_bytes
    a = f(1, 128, 128, 1000, 0)
    b = f(1, 128, 128, 1000, 10_000)
    c = f(1, 128, 128, 2000, 10_000)
    assert 0 < a < b < c
    # 64-bit sizes: 5e9 intersections need > 4 GiB of key storage
    assert f(1, 7680, 7680, 13_000_000, 5_000_000_000) > 3 * 4 * 5_000_000_000
    assert lib.gs_project_workspace_bytes(15_000_000, 5) > 0
    assert lib.gs_intersect_workspace_bytes(0, 10, 10, 1, 1) == 0  # C < 1


def test_intersect_workspace_never_shrinks_as_nnz_grows(lib):
    """A workspace sized for a capacity (the growth-only buffers, the phase
    arena) must fit every smaller pair count: the size may not dip where the
    emit's block layout changes (every 2048 sub-batches of 512 pairs)."""
    f = lib.gs_intersect_workspace_bytes
    edges = [512 * 2048 * k + d for k in (1, 2, 3) for d in (-513, -1, 0, 1, 511, 512, 513)]
    rng = np.random.default_rng(7)
    pts = sorted(set(edges + [int(x) for x in rng.integers(1, 40_000_000, 200)] + [971_385, 1_068_524]))
    for C, W, H in ((1, 1920, 1080), (5, 1297, 840)):
        sizes = [f(C, W, H, n, 1_000_000) for n in pts]
        bad = [(pts[i], pts[i + 1]) for i in range(len(pts) - 1) if sizes[i + 1] < sizes[i]]
        assert not bad, bad[:5]


def test_invalid_arguments_need_no_gpu(lib):
    """Argument checks run before any HIP call."""
    nnz = ctypes.c_int64(7)
    cam = (ctypes.c_int64 * 2)()
    # W = 0 is invalid
    st = lib.gs_project(None, 10, 1, 0, 10, 0, *([None] * 7), None, None, None, None, None, 0,
                        None, 0, ctypes.byref(nnz), cam)
    assert st == gsd.GS_E_INVALID
    # SH degree 4 is invalid
    st = lib.gs_project(None, 10, 1, 10, 10, 4, *([None] * 7), None, None, None, None, None, 0,
                        None, 0, ctypes.byref(nnz), cam)
    assert st == gsd.GS_E_INVALID
    assert lib.gs_rasterize_fwd(None, 0, 10, 10, None, None, None, None, None, None, None, None,
                                None) == \
        gsd.GS_E_INVALID
    n_is = ctypes.c_int64(0)
    need = ctypes.c_uint64(0)
    # nnz >= 2^31 overflows the 31-bit slot ids
    cam2 = (ctypes.c_int64 * 2)(0, 1 << 31)
    st = lib.gs_intersect(None, 1, 16, 16, 1 << 31, 8, 8, cam2, None, 0, None, 0, 8, None, None,
                          ctypes.byref(n_is), ctypes.byref(need))
    assert st == gsd.GS_E_OVERFLOW


def test_readback_status_protocol(lib):
    """The host decision on the words read back after the visibility scan:
    a raised device flag wins over everything (the count is then garbage),
    then a count past its storage type, then a short capacity."""
    f = lib.gs_readback_status
    lim = 1 << 31
    assert f(0, 0, lim, 0) == gsd.GS_OK
    assert f(0, 100, lim, 100) == gsd.GS_OK
    assert f(0, 101, lim, 100) == gsd.GS_E_CAPACITY
    assert f(0, lim - 1, lim, lim) == gsd.GS_OK
    assert f(0, lim, lim, 1 << 40) == gsd.GS_E_OVERFLOW
    assert f(0, -1, lim, 10) == gsd.GS_E_OVERFLOW
    # the flag is checked first: a timed-out scan leaves any count behind
    for count, cap in ((5, 10), (101, 100), (lim, 1 << 40)):
        assert f(1, count, lim, cap) == gsd.GS_E_DEVICE
    assert f(-7, 0, lim, 0) == gsd.GS_E_DEVICE


def test_tile_offsets_check(lib):
    """Tile ranges the raster calls can index with 32-bit local ids:
    ranges of 2^31 entries or more are an overflow ([VRAM] 'The 4 GiB rule
    and the 2^31 limit'); a decreasing or shifted offset table is invalid."""
    def check(offs):
        a = np.ascontiguousarray(np.asarray(offs, np.int64))
        return lib.gs_tile_offsets_check(a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                         a.size - 1)
    big = 1 << 31
    assert check([0]) == gsd.GS_OK                       # no tiles
    assert check([0, 0, 5, 5, 9]) == gsd.GS_OK
    assert check([0, big - 1, big - 1 + 3]) == gsd.GS_OK  # 2^31 - 1 still fits
    assert check([0, 3, 3 + big]) == gsd.GS_E_OVERFLOW   # one list of exactly 2^31
    assert check([0, 4_000_000_000, 4_000_000_001]) == gsd.GS_E_OVERFLOW
    assert check([0, 5, 4]) == gsd.GS_E_INVALID           # negative range
    assert check([1, 5]) == gsd.GS_E_INVALID              # must start at 0
    assert lib.gs_tile_offsets_check(None, 3) == gsd.GS_E_INVALID
    # past 2^32 entries in total, every list short: fine (the high-res scene)
    offs = np.arange(0, 230_401, dtype=np.int64) * 20_700
    assert offs[-1] > 1 << 32 and check(offs) == gsd.GS_OK


def test_intersect_checks_cam_offsets(lib):
    """gs_intersect validates the host cam_offsets before any GPU work: they
    bound each tile list (a pair meets a tile of its camera at most once),
    so they must be a non-decreasing table from 0 to nnz."""
    n_is = ctypes.c_int64(0)
    need = ctypes.c_uint64(0)
    cam = (ctypes.c_int64 * 3)(0, 5, 10)
    st = lib.gs_intersect(None, 2, 16, 16, 10, 8, 8, cam, None, 0, None, 0, None, None, None,
                          ctypes.byref(n_is), ctypes.byref(need))
    assert st == gsd.GS_E_INVALID   # tile_offsets is required
    bad = (ctypes.c_int64 * 3)(0, 6, 10)
    st = lib.gs_intersect(None, 2, 16, 16, 11, 8, 8, bad, None, 0, None, 0, 8, None, None,
                          ctypes.byref(n_is), ctypes.byref(need))
    assert st == gsd.GS_E_INVALID   # cam_offsets[C] must equal nnz


def test_buffer_formulas_reproduce_pages_numbers():
    """Sizes of the mask, group counts and scan follow the pages' cost table
    (VRAM deep dive, per-element buffer cost table and 'Bitmask
    compaction'): at C x N = 5 x 15M the bitmask path is 13.42 MiB where
    the old int32 mask + int32 scan was 572.20 MiB."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_numbers.json")))
    C, N = g["three_key_numbers"]["cameras"], g["three_key_numbers"]["gaussians"]
    Np = gsd.pad_n(N)
    mask_bytes = C * Np // 64 * 8
    groups = C * Np // 128
    new_mib = (mask_bytes + 2 * groups * 4) / 2**20
    old_mib = C * N * g["mask_compaction"]["old_bytes_per_pair"] / 2**20
    assert abs(new_mib - g["mask_compaction"]["new_mib"]) < 0.02
    assert abs(old_mib - g["mask_compaction"]["old_mib"]) < 0.01
    # screen rows and box codes: 40 and 8 bytes per visible pair
    assert gsd.load and _lib.ROW * 4 == 40


def test_fused_adam_argument_checks(lib):
    """Invalid optimizer settings are refused before any GPU work."""
    m = (ctypes.c_void_p * 5)()
    lr = (ctypes.c_float * 6)(*([1e-3] * 6))
    base = [None, 10, 1, 16, 16, 0] + [None] * 10
    assert lib.gs_project_bwd_adam(*base, m, m, lr, 0.9, 0.999, 1e-8, 0) == gsd.GS_E_INVALID  # step
    assert lib.gs_project_bwd_adam(*base, m, m, lr, 1.0, 0.999, 1e-8, 1) == gsd.GS_E_INVALID  # beta1
    assert lib.gs_project_bwd_adam(*base, m, m, lr, 0.9, 0.999, 0.0, 1) == gsd.GS_E_INVALID   # eps
    assert lib.gs_project_bwd_adam(*base, None, m, lr, 0.9, 0.999, 1e-8, 1) == gsd.GS_E_INVALID
    # null moments for N = 10 Gaussians
    assert lib.gs_project_bwd_adam(*base, m, m, lr, 0.9, 0.999, 1e-8, 1) == gsd.GS_E_INVALID


PHASES = {"mask": (0, 4), "wg_count": (0, 0), "wg_scan": (0, 4), "project_ws": (0, 0),
          "screen": (0, 3), "aabb16": (0, 1), "isect_ws": (1, 1), "flatten_ids": (1, 3),
          "tile_offsets": (1, 3), "tile_order": (1, 3), "out_rgb": (2, 4), "out_T": (2, 4),
          "last_ids": (2, 3), "v_screen": (3, 4)}


@pytest.mark.parametrize("shape", [(1_000_000, 1, 1920, 1080, 971_385, 6_284_871),
                                   (15_000_000, 5, 1297, 840, 14_840_666, 78_674_028),
                                   (4096, 1, 128, 128, 4096, 10_358), (1, 1, 1, 1, 0, 0)])
def test_arena_plan_properties(lib, shape):
    """Phase arena ([VRAM] "Phase Arena"): every slot lies inside the arena;
    with aliasing, slots alive in a common phase never share a byte; the
    aliased arena is never larger than the plain one, whose size is the sum;
    the pages' pair (intersection sort buffers, screen-row gradients) shares."""
    N, C, W, H, nnz, I = shape
    st0, plain, tot0 = gsd.gs_arena_plan(N, C, W, H, nnz, I, alias=False)
    st1, al, tot1 = gsd.gs_arena_plan(N, C, W, H, nnz, I, alias=True)
    assert st0 == st1 == gsd.GS_OK
    up = lambda b: (b + 255) // 256 * 256
    assert tot0 == sum(up(b) for _, b in plain.values())
    assert tot1 <= tot0
    for plan, tot in ((plain, tot0), (al, tot1)):
        for k, (o, b) in plan.items():
            assert o % 256 == 0 and o + b <= tot, k
    for a in al:
        for b in al:
            if a >= b:
                continue
            (fa, la), (fb, lb) = PHASES[a], PHASES[b]
            if la < fb or lb < fa:
                continue
            (oa, sa), (ob, sb) = al[a], al[b]
            assert oa + sa <= ob or ob + sb <= oa, (a, b)
    # sizes follow the documented formulas
    Np = (N + 127) // 128 * 128
    assert plain["mask"][1] == C * Np // 8 and plain["v_screen"][1] == 40 * nnz
    assert plain["isect_ws"][1] == lib.gs_intersect_workspace_bytes(C, W, H, nnz, I)
    # an explicit intersection workspace (the need a call reported) replaces the bound
    st2, given, _ = gsd.gs_arena_plan(N, C, W, H, nnz, I, alias=True, isect_ws_bytes=123_457)
    assert st2 == gsd.GS_OK and given["isect_ws"][1] == 123_457
    if nnz > 1000:
        o_i, s_i = al["isect_ws"]
        o_v, s_v = al["v_screen"]
        assert o_i < o_v + s_v and o_v < o_i + s_i   # they share bytes
    assert lib.gs_arena_plan(-1, 1, 1, 1, 0, 0, 0, 1, None, None, None) == gsd.GS_E_INVALID
