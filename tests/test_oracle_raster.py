"""Pins for the oracle's compositing: the single-Gaussian closed form, a
hand-computed three-splat stack with early stop, and a tile-free per-pixel
brute force over all visible pairs."""
import math

import numpy as np
import pytest

import oracle
import workloads
from oracle.raster import ALPHA_MIN
from tests.helpers import make_scene_from, intrinsics

Y00 = 1.0 / (2.0 * math.sqrt(math.pi))


@pytest.mark.parametrize("opacity", [0.3, 0.995])
def test_single_isotropic_gaussian_image(opacity):
    W, H, f, depth, s = 64, 48, 80.0, 4.0, 0.06
    logit = math.log(opacity / (1 - opacity))
    rgb = np.array([0.2, 0.6, 0.9])
    sc = make_scene_from([[0.0, 0.0, 0.0]], [[1.0, 0, 0, 0]], [[math.log(s)] * 3], [logit],
                         ((rgb - 0.5) / Y00)[None, None], workloads.lookat_viewmat((0, 0, depth)),
                         intrinsics(f, f, W, H), W, H, 0)
    proj, isect, out, T, last, _ = oracle.render(sc)
    s32 = math.exp(float(np.float32(math.log(s))))
    var = (f * s32 / depth) ** 2 + 0.3
    o = 1 / (1 + math.exp(-float(np.float32(logit))))
    jj, ii = np.meshgrid(np.arange(W) + 0.5, np.arange(H) + 0.5)
    rho2 = (jj - W / 2) ** 2 + (ii - H / 2) ** 2
    alpha = np.minimum(0.99, o * np.exp(-0.5 * rho2 / var))
    # pixels in tiles the box covers
    tx0, ty0, tx1, ty1 = (int(v[0]) for v in isect.rects)
    covered = np.zeros((H, W), bool)
    covered[ty0 * 16:ty1 * 16, tx0 * 16:tx1 * 16] = True
    alpha = np.where(covered & (alpha >= ALPHA_MIN), alpha, 0.0)
    np.testing.assert_allclose(out[0], alpha[..., None] * rgb, atol=1e-6)   # rgb is fp32-stored
    np.testing.assert_allclose(T[0], 1 - alpha, atol=1e-12)
    assert np.array_equal(last[0], np.where(alpha > 0, 0, -1))
    assert proj.screen[0, 7:10] == pytest.approx(rgb, abs=1e-6)
    if opacity < 0.353:   # o e^-4.5 < 1/255: nothing beyond the 3-sigma box counts
        assert not np.any((out[0].sum(-1) > 0) & ~covered)


def test_three_splat_stack_early_stop():
    """alphas 0.99, 0.9, 0.95 at one pixel: T goes 1 -> 0.01 -> 0.001, and the
    third would leave T = 5e-5 < 1e-4, so it stops there without compositing."""
    rows = np.zeros((3, 10))
    rows[:, 0:2] = [0.5, 0.5]           # centred on pixel (0, 0)
    rows[:, 2] = rows[:, 4] = 1.0
    rows[:, 5] = [0.999, 0.9, 0.95]
    rows[:, 6] = [1.0, 2.0, 3.0]
    rows[:, 7:10] = [[1, 0, 0], [0, 1, 0], [0, 0, 1]]
    fids = np.array([0, 1, 2], np.uint32)
    offs = np.array([0, 3])
    out, T, last, ev = oracle.rasterize_fwd(rows, fids, offs, 1, 1, 1)
    np.testing.assert_allclose(out[0, 0, 0], [0.99, 0.9 * 0.01, 0.0], atol=1e-15)
    assert T[0, 0, 0] == pytest.approx(0.001, rel=1e-12)
    assert last[0, 0, 0] == 1 and ev[0, 0, 0] == 3


def _bruteforce_image(proj, sc):
    """Per pixel, every visible pair of that camera, ordered by (depth bits,
    slot), composited with the same per-pixel rules -- no tiles at all."""
    C, W, H = sc["C"], sc["W"], sc["H"]
    out = np.zeros((C, H, W, 3))
    Tout = np.ones((C, H, W))
    zb = proj.z32.view(np.uint32)
    for c in range(C):
        slots = np.flatnonzero(proj.cam == c)
        slots = slots[np.lexsort((slots, zb[slots]))]
        u, v, a, b, cc, o = (proj.screen[slots, k] for k in range(6))
        rgb = proj.screen[slots, 7:10]
        for i in range(H):
            for j in range(W):
                dx, dy = u - (j + 0.5), v - (i + 0.5)
                sig = 0.5 * (a * dx * dx + cc * dy * dy) + b * dx * dy
                al = np.minimum(0.99, o * np.exp(-sig))
                T, acc = 1.0, np.zeros(3)
                for k in np.flatnonzero((sig >= 0) & (al >= ALPHA_MIN)):
                    Tn = T * (1 - al[k])
                    if Tn < 1e-4:
                        break
                    acc += rgb[k] * al[k] * T
                    T = Tn
                out[c, i, j], Tout[c, i, j] = acc, T
    return out, Tout


@pytest.mark.parametrize("name,n", [("sh2-dense", 1500), ("multicam", 900)])
def test_tiles_equal_tile_free_bruteforce(name, n):
    spec = workloads.SMALL[name]
    spec = workloads.SceneSpec(spec.name, n, spec.sh_degree, spec.n_cams, 48, 40,
                               spec.focal * 48 / spec.width, spec.mean_half_extent,
                               spec.log_scale_mu, spec.log_scale_sigma, spec.cam_radius,
                               seed=spec.seed)
    sc = workloads.make_scene(spec)
    # every opacity below e^4.5/255 = 0.353: alpha beyond the 3-sigma box < 1/255,
    # so dropping the tiles a box does not cover changes nothing
    o = 0.02 + 0.33 * np.random.default_rng(1).uniform(size=n)
    sc["opacity_logits"] = np.log(o / (1 - o)).astype(np.float32)
    proj, isect, out, T, last, _ = oracle.render(sc)
    assert float(proj.screen[:, 5].max()) < 0.353
    ref, Tref = _bruteforce_image(proj, sc)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    np.testing.assert_allclose(T, Tref, atol=1e-12)
    assert (T < 0.5).mean() > 0.05     # the scene is dense enough to exercise compositing
