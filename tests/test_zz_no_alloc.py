"""gs_project_noalloc (the projection with its workspace in the library's
static device scratch, for callers that cannot allocate) against
gs_project on the same inputs: two calls in a row, the second on a
smaller scene, every output bit-identical (the same kernels run; only
where the workspace lives differs). Sizes past the scratch are refused
before any device work."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

gsd = pytest.importorskip("gaussian_splatting_differentiable_project_amd")


def _buffers(s, cap):
    Np = gsd.pad_n(s.N)
    return dict(mask=torch.full((max(s.C * Np // 64, 1),), -1, dtype=torch.int64, device="cuda"),
                wg_count=torch.full((max(s.C * Np // 128, 1),), -1, dtype=torch.int32, device="cuda"),
                wg_scan=torch.full((max(s.C * Np // 128, 1),), -1, dtype=torch.int32, device="cuda"),
                screen=torch.full((max(cap, 1) * 10,), float("nan"), device="cuda"),
                aabb=torch.full((max(cap, 1) * 2,), -1, dtype=torch.int32, device="cuda"))


def _inputs(s):
    return (s.N, s.C, s.W, s.H, s.sh_degree, s.means, s.quats, s.log_scales, s.opacity_logits,
            s.sh, s.viewmats, s.Ks)


def test_noalloc_matches_gs_project_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gsd.load()
    # a larger scene first, then a smaller one: the second call must not see
    # anything the first left in the shared scratch
    for name in ("multicam", "sh1-odd-n"):
        sc = workloads.make_scene(workloads.SMALL[name])
        s = gsd.Scene.from_numpy(sc, "cuda")
        ref = gsd.Rasterizer().project(s)
        cap = ref.nnz + 17
        b = _buffers(s, cap)
        print(f"{name}: N={s.N} C={s.C} nnz={ref.nnz}", flush=True)
        st, nnz, cam = gsd.gs_project_noalloc(*_inputs(s), b["mask"], b["wg_count"], b["wg_scan"],
                                              b["screen"], b["aabb"], cap)
        torch.cuda.synchronize()
        assert st == gsd.GS_OK, gsd.status_str(st)
        assert nnz == ref.nnz and cam == ref.cam_offsets
        assert torch.equal(b["mask"], ref.mask)
        assert torch.equal(b["wg_count"], ref.wg_count)
        assert torch.equal(b["wg_scan"], ref.wg_scan)
        assert torch.equal(b["screen"][: nnz * 10].view(nnz, 10), ref.screen)
        assert torch.equal(b["aabb"][: nnz * 2].view(nnz, 2), ref.aabb16)
        # nothing written past the visible rows
        assert torch.isnan(b["screen"][nnz * 10:]).all()
        assert (b["aabb"][nnz * 2:] == -1).all()


def test_noalloc_capacity_protocol():
    """A capacity below nnz: GS_E_CAPACITY with nnz returned, nothing
    written at or past the capacity (as gs_project)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sc = workloads.make_scene(workloads.SMALL["sh3-ragged"])
    s = gsd.Scene.from_numpy(sc, "cuda")
    ref = gsd.Rasterizer().project(s)
    cap = ref.nnz // 2
    b = _buffers(s, ref.nnz)
    st, nnz, _ = gsd.gs_project_noalloc(*_inputs(s), b["mask"], b["wg_count"], b["wg_scan"],
                                        b["screen"], b["aabb"], cap)
    torch.cuda.synchronize()
    assert st == gsd.GS_E_CAPACITY and nnz == ref.nnz
    assert torch.equal(b["screen"][: cap * 10].view(cap, 10), ref.screen[:cap])
    assert torch.isnan(b["screen"][cap * 10:]).all()


def test_noalloc_refuses_sizes_past_the_scratch():
    """More cameras than the host words hold, or a workspace past 64 KiB:
    GS_E_WORKSPACE before any device work (host check only)."""
    lib = gsd.load()
    nnz = ctypes.c_int64(-1)
    cam = (ctypes.c_int64 * 300)()
    p = 256  # any aligned non-null address: nothing is dereferenced
    args = [p] * 7 + [p] * 5
    st = lib.gs_project_noalloc(None, 1000, 257, 64, 64, 0, *args, 0, ctypes.byref(nnz), cam)
    assert st == gsd.GS_E_WORKSPACE
    assert lib.gs_project_workspace_bytes(40_000_000_000, 256) > 65536
    st = lib.gs_project_noalloc(None, 40_000_000_000, 256, 64, 64, 0, *args, 0,
                                ctypes.byref(nnz), cam)
    assert st == gsd.GS_E_WORKSPACE
