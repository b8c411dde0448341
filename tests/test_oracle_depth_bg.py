"""Pins for the oracle's depth channel and background blend.

[BWD] section 2 lists the per-pixel output gradients as v_render_rgb,
v_render_depth and v_render_Ts; section 3's background hook adds the
background's transmittance gradient into v_render_Ts. Readings (oracle
raster docstring): D = sum z alpha T like a colour channel; C_out =
C + T_final bg with one RGB colour per camera.

Pins: the single-Gaussian closed form (D = z alpha, C_out = rgb alpha +
(1 - alpha) bg), the hand-computed three-splat stack, and central finite
differences of every screen-row column with a depth loss and a
background, of the background itself, of the depth column's path to the
means (through the exact fp64 camera depth), and, through the whole
path, of the other parameter tensors.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from oracle.raster import ALPHA_MIN, decision_signature
from tests.helpers import fd_scene, intrinsics, make_scene_from

Y00 = 1.0 / (2.0 * math.sqrt(math.pi))
REL = 1e-6


def _close(fd, an, scale):
    return abs(fd - an) <= REL * max(abs(an), 1e-3 * scale) + 1e-10


def test_single_gaussian_depth_and_background_closed_form():
    W, H, f, depth, s, opacity = 64, 48, 80.0, 4.0, 0.06, 0.3
    logit = math.log(opacity / (1 - opacity))
    rgb = np.array([0.2, 0.6, 0.9])
    bg = np.array([[0.05, 0.5, 0.25]])
    sc = make_scene_from([[0.0, 0.0, 0.0]], [[1.0, 0, 0, 0]], [[math.log(s)] * 3], [logit],
                         ((rgb - 0.5) / Y00)[None, None], workloads.lookat_viewmat((0, 0, depth)),
                         intrinsics(f, f, W, H), W, H, 0)
    proj, isect, out, T, last, _, D = oracle.render(sc, background=bg, depth=True)
    s32 = math.exp(float(np.float32(math.log(s))))
    var = (f * s32 / depth) ** 2 + 0.3
    o = 1 / (1 + math.exp(-float(np.float32(logit))))
    jj, ii = np.meshgrid(np.arange(W) + 0.5, np.arange(H) + 0.5)
    rho2 = (jj - W / 2) ** 2 + (ii - H / 2) ** 2
    alpha = np.minimum(0.99, o * np.exp(-0.5 * rho2 / var))
    tx0, ty0, tx1, ty1 = (int(v[0]) for v in isect.rects)
    covered = np.zeros((H, W), bool)
    covered[ty0 * 16:ty1 * 16, tx0 * 16:tx1 * 16] = True
    alpha = np.where(covered & (alpha >= ALPHA_MIN), alpha, 0.0)
    np.testing.assert_allclose(D[0], depth * alpha, atol=1e-12)     # the mean is at camera depth 4
    np.testing.assert_allclose(out[0], alpha[..., None] * rgb + (1 - alpha)[..., None] * bg[0],
                               atol=1e-6)                            # rgb is fp32-stored
    np.testing.assert_allclose(T[0], 1 - alpha, atol=1e-12)


def test_three_splat_stack_depth_and_background():
    """alphas 0.99, 0.9 composited at depths 1 and 2, the third stops:
    D = 1 * 0.99 + 2 * 0.9 * 0.01 and C_out = C + 0.001 bg."""
    rows = np.zeros((3, 10))
    rows[:, 0:2] = [0.5, 0.5]
    rows[:, 2] = rows[:, 4] = 1.0
    rows[:, 5] = [0.999, 0.9, 0.95]
    rows[:, 6] = [1.0, 2.0, 3.0]
    rows[:, 7:10] = [[1, 0, 0], [0, 1, 0], [0, 0, 1]]
    fids = np.array([0, 1, 2], np.uint32)
    offs = np.array([0, 3])
    bg = np.array([[0.2, 0.3, 0.4]])
    out, T, last, ev, D = oracle.rasterize_fwd(rows, fids, offs, 1, 1, 1, background=bg, depth=True)
    assert D[0, 0, 0] == pytest.approx(0.99 + 2 * 0.9 * 0.01, rel=1e-13)
    np.testing.assert_allclose(out[0, 0, 0], [0.99, 0.9 * 0.01, 0.0] + 0.001 * bg[0], atol=1e-15)


@pytest.fixture(scope="module")
def case():
    sc = fd_scene(seed=33, N=40, C=2, W=40, H=36, deg=1)
    sc["opacity_logits"][:6] = 6.0
    rng = np.random.default_rng(7)
    v_depth = rng.normal(size=(sc["C"], sc["H"], sc["W"]))
    bg = rng.uniform(0, 1, (sc["C"], 3))
    proj, isect, *_ = oracle.render(sc)
    return sc, proj, isect, v_depth, bg


def _loss(sc, isect, screen, v_depth, bg):
    rgb, T, _, _, D = oracle.rasterize_fwd(screen, isect.flatten_ids, isect.tile_offsets, sc["C"],
                                           sc["W"], sc["H"], background=bg, depth=True)
    return float((sc["v_rgb"].astype(np.float64) * rgb).sum() + (sc["v_T"].astype(np.float64) * T).sum()
                 + (v_depth * D).sum())


def _sig(sc, isect, screen):
    return decision_signature(screen, isect.flatten_ids, isect.tile_offsets, sc["C"], sc["W"], sc["H"])


@pytest.mark.parametrize("cols", [[0, 1], [2, 3, 4], [5], [6], [7, 8, 9]],
                         ids=["uv", "conic", "opacity", "depth", "rgb"])
def test_raster_bwd_with_depth_and_background_fd(case, cols):
    sc, proj, isect, v_depth, bg = case
    screen = proj.screen.copy()
    g = oracle.rasterize_bwd(screen, isect.flatten_ids, isect.tile_offsets, sc["C"], sc["W"], sc["H"],
                             sc["v_rgb"], sc["v_T"], v_depth=v_depth, background=bg)
    gnorm = np.linalg.norm(g[:, cols])
    assert gnorm > 0
    rng = np.random.default_rng(100 + sum(cols))
    probes = []
    for _ in range(16):
        d = np.zeros_like(screen)
        d[:, cols] = rng.normal(size=(screen.shape[0], len(cols)))
        probes.append(d / np.linalg.norm(d))
    for _ in range(48):
        d = np.zeros_like(screen)
        d[rng.integers(screen.shape[0]), cols[rng.integers(len(cols))]] = 1.0
        probes.append(d)
    used = 0
    for d in probes:
        h = 1e-6 * max(1.0, float(np.abs(screen[:, cols]).max()))
        sp, sm = screen + h * d, screen - h * d
        if _sig(sc, isect, sp) != _sig(sc, isect, sm):
            continue
        fd = (_loss(sc, isect, sp, v_depth, bg) - _loss(sc, isect, sm, v_depth, bg)) / (2 * h)
        an = float((g * d).sum())
        assert _close(fd, an, gnorm), (fd, an)
        used += 1
    assert used >= 0.75 * len(probes)


def test_background_gradient_fd(case):
    sc, proj, isect, v_depth, bg = case
    screen = proj.screen
    _, T, _, _ = oracle.rasterize_fwd(screen, isect.flatten_ids, isect.tile_offsets, sc["C"], sc["W"],
                                      sc["H"])
    g = oracle.background_grad(T, sc["v_rgb"])
    h = 1e-6
    for c in range(sc["C"]):
        for k in range(3):
            d = np.zeros_like(bg)
            d[c, k] = h
            fd = (_loss(sc, isect, screen, v_depth, bg + d) - _loss(sc, isect, screen, v_depth, bg - d)) / (2 * h)
            assert _close(fd, g[c, k], np.linalg.norm(g)), (c, k, fd, g[c, k])


def test_depth_gradient_is_zero_without_depth_loss(case):
    sc, proj, isect, _, bg = case
    g = oracle.rasterize_bwd(proj.screen, isect.flatten_ids, isect.tile_offsets, sc["C"], sc["W"],
                             sc["H"], sc["v_rgb"], sc["v_T"], background=bg)
    assert np.all(g[:, 6] == 0)


@pytest.fixture(scope="module")
def path_case():
    sc = fd_scene(seed=12, N=36, C=2, W=40, H=36, deg=2)
    for k in ("means", "quats", "log_scales", "opacity_logits", "sh"):
        sc[k] = sc[k].astype(np.float64)
    sc["opacity_logits"][:4] = 5.5
    rng = np.random.default_rng(9)
    v_depth = rng.normal(size=(sc["C"], sc["H"], sc["W"]))
    bg = rng.uniform(0, 1, (sc["C"], 3))
    L, grads, aux = oracle.loss_and_grads(sc, v_depth=v_depth, background=bg)
    return sc, grads, v_depth, bg


def _path_eval(sc, v_depth, bg):
    proj, isect, rgb, T, last, _, D = oracle.render(sc, background=bg, depth=True)
    L = float((sc["v_rgb"].astype(np.float64) * rgb).sum() + (sc["v_T"].astype(np.float64) * T).sum()
              + (v_depth * D).sum())
    sig = (proj.pairs.tobytes(), (proj.screen[:, 7:10] == 0).tobytes(),
           decision_signature(proj.screen, isect.flatten_ids, isect.tile_offsets, sc["C"], sc["W"], sc["H"]))
    return L, sig


# The screen row stores the fp32 depth z32 (the sort key's value), a
# staircase in the means at the finite-difference step; the means are
# pinned through the exact fp64 camera depth below instead.
@pytest.mark.parametrize("name,gname", [("opacity_logits", "v_opacity_logits"), ("quats", "v_quats"),
                                        ("log_scales", "v_log_scales"), ("sh", "v_sh")])
def test_path_with_depth_and_background_fd(path_case, name, gname):
    sc, grads, v_depth, bg = path_case
    g = grads[gname]
    theta = sc[name]
    gnorm = np.linalg.norm(g)
    assert gnorm > 0
    rng = np.random.default_rng(len(name) + 50)
    probes = []
    for _ in range(12):
        d = rng.normal(size=theta.shape)
        probes.append(d / np.linalg.norm(d))
    flat_nz = np.flatnonzero(g.ravel() != 0)
    for _ in range(24):
        d = np.zeros(theta.size)
        d[flat_nz[rng.integers(flat_nz.size)]] = 1.0
        probes.append(d.reshape(theta.shape))
    used = 0
    for d in probes:
        h = 1e-6 * max(1.0, float(np.abs(theta).max()))
        sp, sm = dict(sc), dict(sc)
        sp[name] = theta + h * d
        sm[name] = theta - h * d
        Lp, sig_p = _path_eval(sp, v_depth, bg)
        Lm, sig_m = _path_eval(sm, v_depth, bg)
        if sig_p != sig_m:
            continue
        fd = (Lp - Lm) / (2 * h)
        an = float((g * d).sum())
        assert _close(fd, an, gnorm), (name, fd, an)
        used += 1
    assert used >= 0.75 * len(probes)


def test_depth_row_gradient_reaches_means_fd():
    """A gradient on the rows' depth column flows to the means through the
    camera depth z = (R mu + t)_z: finite differences of sum vz * z, with z
    the exact fp64 camera depth of each visible pair."""
    sc = fd_scene(seed=44, N=30, C=2, W=40, H=36, deg=1)
    sc["means"] = sc["means"].astype(np.float64)
    proj = oracle.project(sc)
    rng = np.random.default_rng(3)
    vz = rng.normal(size=proj.nnz)
    v_screen = np.zeros((proj.nnz, 10))
    v_screen[:, 6] = vz
    g = oracle.project_bwd(sc, proj, v_screen)["v_means"]

    def L(means):
        tot = 0.0
        for c in range(sc["C"]):
            pc = oracle.project_camera(means, sc["quats"], sc["log_scales"], sc["opacity_logits"],
                                       sc["sh"], sc["viewmats"][c], sc["Ks"][c], sc["W"], sc["H"],
                                       sc["sh_degree"])
            sel = proj.cam == c
            tot += float((vz[sel] * pc["z"][proj.gauss[sel]]).sum())
        return tot

    h = 1e-6
    for _ in range(24):
        d = rng.normal(size=sc["means"].shape)
        d /= np.linalg.norm(d)
        fd = (L(sc["means"] + h * d) - L(sc["means"] - h * d)) / (2 * h)
        an = float((g * d).sum())
        assert _close(fd, an, np.linalg.norm(g)), (fd, an)
