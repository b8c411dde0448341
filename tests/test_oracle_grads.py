"""Pins for the oracle's gradients: central finite differences in fp64.

L = <v_rgb, out_rgb> + <v_T, out_T>. For every gradient tensor: 16 random
directions restricted to that tensor and 64 sampled coordinates. A probe
is skipped when any discrete decision differs between theta + h and
theta - h (visible set, tile lists, per-pixel composited sets, 0.99-clamp
flags, colour clamp); at least 3/4 of the probes must be usable.
"""
import numpy as np
import pytest

import oracle
from oracle.raster import decision_signature
from tests.helpers import fd_scene

REL = 1e-6


def _close(fd, an, scale):
    return abs(fd - an) <= REL * max(abs(an), 1e-3 * scale) + 1e-10


# ---------------------------------------------------------------- raster only

@pytest.fixture(scope="module")
def raster_case():
    sc = fd_scene(seed=21, N=40, C=1, W=40, H=36, deg=1)
    sc["opacity_logits"][:6] = 6.0            # alpha hits the 0.99 clamp near centres
    proj, isect, *_ = oracle.render(sc)
    return sc, proj, isect


def _raster_loss(sc, isect, screen):
    rgb, T, _, _ = oracle.rasterize_fwd(screen, isect.flatten_ids, isect.tile_offsets,
                                        sc["C"], sc["W"], sc["H"])
    return float((sc["v_rgb"].astype(np.float64) * rgb).sum() + (sc["v_T"].astype(np.float64) * T).sum())


def _raster_sig(sc, isect, screen):
    return decision_signature(screen, isect.flatten_ids, isect.tile_offsets, sc["C"], sc["W"], sc["H"])


@pytest.mark.parametrize("cols", [[0, 1], [2, 3, 4], [5], [7, 8, 9]], ids=["uv", "conic", "opacity", "rgb"])
def test_raster_bwd_finite_differences(raster_case, cols):
    sc, proj, isect = raster_case
    screen = proj.screen.copy()
    g = oracle.rasterize_bwd(screen, isect.flatten_ids, isect.tile_offsets, sc["C"], sc["W"], sc["H"],
                             sc["v_rgb"], sc["v_T"])
    assert np.all(g[:, 6] == 0)
    rng = np.random.default_rng(sum(cols))
    gnorm = np.linalg.norm(g[:, cols])
    assert gnorm > 0
    probes, used = [], 0
    for _ in range(16):
        d = np.zeros_like(screen)
        d[:, cols] = rng.normal(size=(screen.shape[0], len(cols)))
        d /= np.linalg.norm(d)
        probes.append(d)
    for _ in range(64):
        d = np.zeros_like(screen)
        d[rng.integers(screen.shape[0]), cols[rng.integers(len(cols))]] = 1.0
        probes.append(d)
    for d in probes:
        h = 1e-6 * max(1.0, float(np.abs(screen[:, cols]).max()))
        sp, sm = screen + h * d, screen - h * d
        if _raster_sig(sc, isect, sp) != _raster_sig(sc, isect, sm):
            continue
        fd = (_raster_loss(sc, isect, sp) - _raster_loss(sc, isect, sm)) / (2 * h)
        an = float((g * d).sum())
        assert _close(fd, an, gnorm), (fd, an)
        used += 1
    assert used >= 0.75 * len(probes)


# ---------------------------------------------------------------- whole path

@pytest.fixture(scope="module")
def path_case():
    sc = fd_scene(seed=5, N=36, C=2, W=40, H=36, deg=3)
    for k in ("means", "quats", "log_scales", "opacity_logits", "sh"):
        sc[k] = sc[k].astype(np.float64)
    sc["opacity_logits"][:4] = 5.5
    L, grads, aux = oracle.loss_and_grads(sc)
    return sc, L, grads, aux


def _path_eval(sc):
    proj, isect, rgb, T, last, _ = oracle.render(sc)
    L = float((sc["v_rgb"].astype(np.float64) * rgb).sum() + (sc["v_T"].astype(np.float64) * T).sum())
    sig = (proj.pairs.tobytes(), (proj.screen[:, 7:10] == 0).tobytes(),
           decision_signature(proj.screen, isect.flatten_ids, isect.tile_offsets, sc["C"], sc["W"], sc["H"]))
    return L, sig


@pytest.mark.parametrize("name,gname", [("means", "v_means"), ("quats", "v_quats"),
                                        ("log_scales", "v_log_scales"),
                                        ("opacity_logits", "v_opacity_logits"), ("sh", "v_sh")])
def test_path_finite_differences(path_case, name, gname):
    sc, L0, grads, aux = path_case
    g = grads[gname]
    theta = sc[name]
    gnorm = np.linalg.norm(g)
    assert gnorm > 0
    rng = np.random.default_rng(len(name))
    probes = []
    for _ in range(16):
        d = rng.normal(size=theta.shape)
        probes.append(d / np.linalg.norm(d))
    flat_nz = np.flatnonzero(g.ravel() != 0)
    for _ in range(64):
        d = np.zeros(theta.size)
        d[flat_nz[rng.integers(flat_nz.size)] if rng.uniform() < 0.8 else rng.integers(theta.size)] = 1.0
        probes.append(d.reshape(theta.shape))
    used = 0
    for d in probes:
        h = 1e-6 * max(1.0, float(np.abs(theta).max()))
        sp, sm = dict(sc), dict(sc)
        sp[name] = theta + h * d
        sm[name] = theta - h * d
        Lp, sig_p = _path_eval(sp)
        Lm, sig_m = _path_eval(sm)
        if sig_p != sig_m:
            continue
        fd = (Lp - Lm) / (2 * h)
        an = float((g * d).sum())
        assert _close(fd, an, gnorm), (name, fd, an)
        used += 1
    assert used >= 0.75 * len(probes)


def test_invisible_gaussians_get_zero_grads(path_case):
    sc, _, grads, aux = path_case
    proj = aux["proj"]
    seen = np.zeros(sc["N"], bool)
    seen[proj.gauss[proj.gauss < sc["N"]]] = True
    for k, g in grads.items():
        assert np.all(g[~seen] == 0), k
