"""Seeded synthetic scenes for the differentiable tile rasterizer.

This module only *draws inputs*. It holds none of the rasterizer's
arithmetic: no projection, no compositing, no gradients. Both the fp64
oracle (``oracle/``) and the HIP path's tests and benchmark take their
inputs from here, so the two sides see byte-identical fp32 arrays.

Input conventions (the pages give no formula for them; these are the
readings used throughout):

* ``means[N,3]``, ``quats[N,4]`` stored as (w, x, y, z), ``log_scales[N,3]``,
  ``opacity_logits[N]``, ``sh[N,K,3]`` with K = (degree+1)^2 and the
  coefficients ordered l = 0..degree, m = -l..l -- all fp32, SoA.
* ``viewmats[C,4,4]``: row-major world->camera, OpenCV axes (x right,
  y down, z forward). Cameras are built by a look-at with world up +y:
  forward f = normalize(target - eye), right = normalize(f x up),
  down = f x right, rotation rows (right, down, f), t = -R eye.
* ``Ks[C,3,3]``: pinhole intrinsics with the principal point at the image
  centre (W/2, H/2).
* Ring rigs put camera k at r (sin 2 pi k/C, 0, cos 2 pi k/C) looking at the
  origin, so camera 0 sits at (0, 0, r).
* Colours are drawn as RGB ~ U[0,1] and stored as the degree-0 coefficient
  (rgb - 0.5) / Y00 with Y00 = 1 / (2 sqrt(pi)), the constant value of the
  l = 0 real spherical harmonic; higher coefficients ~ N(0, sigma).
* "N(mu, s)" means standard deviation s.

Draw order (fixed, so a seed names one scene): means, log_scales, quats
(N(0, I4) then normalised), opacity_logits, rgb, sh_rest, v_rgb, v_T.
Every draw is made in float64 and cast to float32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["SceneSpec", "CONFIGS", "SMALL", "make_scene", "lookat_viewmat",
           "camera_rig", "n_pad", "tiles_x", "tiles_y"]

TILE = 16          # 16x16 pixel tiles
MASK_GROUP = 128   # Gaussians per visibility work-group


@dataclasses.dataclass(frozen=True)
class SceneSpec:
    name: str
    n: int                   # Gaussians
    sh_degree: int
    n_cams: int
    width: int
    height: int
    focal: float             # fx = fy
    mean_half_extent: float  # means ~ U[-e, e]^3
    log_scale_mu: float
    log_scale_sigma: float
    cam_radius: float        # distance of every camera from the origin
    sh_rest_sigma: float = 0.1
    with_v_T: bool = True    # draw dL/dT ~ N(0,1); otherwise zero
    seed: int = 0

    @property
    def K(self) -> int:
        return (self.sh_degree + 1) ** 2


# The five workloads of the benchmark suite (ids 1..5); seed = 1000 + id.
CONFIGS = {
    1: SceneSpec("tiny-4k-128px", 4096, 0, 1, 128, 128, 111.0, 1.0, -3.0, 0.3,
                 5.0, 0.0, with_v_T=False, seed=1001),
    2: SceneSpec("1M-sh3-1080p", 1_000_000, 3, 1, 1920, 1080, 1100.0, 2.0,
                 -4.5, 0.5, 5.0, seed=1002),
    3: SceneSpec("3M-sh3-5cam-1600x1064", 3_000_000, 3, 5, 1600, 1064, 1386.0,
                 2.0, -4.5, 0.5, 5.0, seed=1003),
    4: SceneSpec("15M-sh3-5cam-1297x840", 15_000_000, 3, 5, 1297, 840, 1950.0,
                 4.0, -5.0, 0.6, 6.0, seed=1004),
    5: SceneSpec("13M-sh3-7680px", 13_000_000, 3, 1, 7680, 7680, 6650.0, 2.0,
                 -4.0, 0.6, 5.0, seed=1005),
}

# Small scenes with the same distributions, sized so the oracle finishes in
# seconds while still spanning several tiles and a ragged tile tail.
SMALL = {
    "tiny": CONFIGS[1],
    "sh3-ragged": SceneSpec("sh3-20k-200x120", 20_000, 3, 1, 200, 120, 115.0,
                            2.0, -3.2, 0.5, 5.0, seed=2001),
    "multicam": SceneSpec("sh3-8k-3cam-150x100", 8_000, 3, 3, 150, 100, 130.0,
                          2.0, -3.0, 0.5, 5.0, seed=2002),
    "sh1-odd-n": SceneSpec("sh1-3001-97x61", 3001, 1, 2, 97, 61, 85.0, 1.5,
                           -2.8, 0.4, 5.0, seed=2003),
    "sh2-dense": SceneSpec("sh2-12k-64x48", 12_000, 2, 1, 64, 48, 60.0, 1.5,
                           -2.5, 0.4, 5.0, seed=2004),
    # six narrow cameras, each seeing a few percent of the Gaussians: most
    # (camera, Gaussian) pairs are invisible
    "sparse-6cam": SceneSpec("sh2-9001-6cam-80x60-narrow", 9001, 2, 6, 80, 60, 320.0,
                             2.0, -3.0, 0.5, 5.0, seed=2005),
}


def n_pad(n: int) -> int:
    """N rounded up to a whole visibility work-group (128 Gaussians)."""
    return ((n + MASK_GROUP - 1) // MASK_GROUP) * MASK_GROUP


def tiles_x(width: int) -> int:
    return (width + TILE - 1) // TILE


def tiles_y(height: int) -> int:
    return (height + TILE - 1) // TILE


def lookat_viewmat(eye, target=(0.0, 0.0, 0.0), up=(0.0, 1.0, 0.0)) -> np.ndarray:
    """World->camera 4x4 (OpenCV axes) for a camera at ``eye`` facing ``target``."""
    eye = np.asarray(eye, np.float64)
    f = np.asarray(target, np.float64) - eye
    f /= np.linalg.norm(f)
    right = np.cross(f, np.asarray(up, np.float64))
    right /= np.linalg.norm(right)
    down = np.cross(f, right)
    R = np.stack([right, down, f])
    V = np.eye(4)
    V[:3, :3] = R
    V[:3, 3] = -R @ eye
    return V


def camera_rig(spec: SceneSpec):
    """(viewmats[C,4,4], Ks[C,3,3]) as float32 for the spec's camera ring."""
    C = spec.n_cams
    vms = []
    for k in range(C):
        a = 2.0 * math.pi * k / C
        eye = spec.cam_radius * np.array([math.sin(a), 0.0, math.cos(a)])
        vms.append(lookat_viewmat(eye))
    K = np.array([[spec.focal, 0.0, spec.width / 2.0],
                  [0.0, spec.focal, spec.height / 2.0],
                  [0.0, 0.0, 1.0]])
    Ks = np.repeat(K[None], C, axis=0)
    return np.stack(vms).astype(np.float32), Ks.astype(np.float32)


def make_scene(spec: SceneSpec, seed: int | None = None) -> dict:
    """Draw one scene plus its fixed upstream image gradients."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    N, K = spec.n, spec.K
    e = spec.mean_half_extent
    means = rng.uniform(-e, e, size=(N, 3))
    log_scales = rng.normal(spec.log_scale_mu, spec.log_scale_sigma, size=(N, 3))
    quats = rng.normal(0.0, 1.0, size=(N, 4))
    quats /= np.linalg.norm(quats, axis=1, keepdims=True)
    opacity_logits = rng.normal(0.0, 1.0, size=N)
    rgb = rng.uniform(0.0, 1.0, size=(N, 3))
    sh = np.zeros((N, K, 3), np.float32)
    sh[:, 0, :] = ((rgb - 0.5) * (2.0 * math.sqrt(math.pi))).astype(np.float32)
    del rgb
    if K > 1:
        sh[:, 1:, :] = rng.normal(0.0, spec.sh_rest_sigma, size=(N, K - 1, 3)).astype(np.float32)
    viewmats, Ks = camera_rig(spec)
    C, H, W = spec.n_cams, spec.height, spec.width
    v_rgb = rng.normal(0.0, 1.0, size=(C, H, W, 3)).astype(np.float32)
    if spec.with_v_T:
        v_T = rng.normal(0.0, 1.0, size=(C, H, W)).astype(np.float32)
    else:
        v_T = np.zeros((C, H, W), np.float32)
    return dict(
        spec=spec, N=N, C=C, W=W, H=H, sh_degree=spec.sh_degree,
        means=means.astype(np.float32),
        quats=quats.astype(np.float32),
        log_scales=log_scales.astype(np.float32),
        opacity_logits=opacity_logits.astype(np.float32),
        sh=sh, viewmats=viewmats, Ks=Ks, v_rgb=v_rgb, v_T=v_T,
    )
