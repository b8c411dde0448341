"""One whole step of the path in the oracle: project -> intersect -> raster
forward -> raster backward -> projection backward ([BWD] sections 4-5).

Row storage. [VRAM]'s per-element buffer cost table gives proj.screen as
40 bytes per visible pair for (xy, conic, opacity, depth, rgb): ten
4-byte floats. With ``rows32=True`` the rasterizer stages consume the
screen rows rounded to float32, as stored by the method; the projection
itself and every gradient stay fp64. With ``rows32=False`` (the default,
used by the finite-difference pins) the rows stay fp64, so the whole step
is one smooth fp64 function of the inputs.
"""
from __future__ import annotations

import numpy as np

from .project import project
from .intersect import intersect
from .raster import rasterize_fwd, rasterize_bwd
from .project_bwd import project_bwd

__all__ = ["render", "loss_and_grads"]


def render(scene: dict, rows32: bool = False):
    proj = project(scene)
    if rows32:
        proj.screen = proj.screen.astype(np.float32).astype(np.float64)
    isect = intersect(proj, scene["W"], scene["H"])
    rgb, T, last, evals = rasterize_fwd(proj.screen, isect.flatten_ids, isect.tile_offsets,
                                        scene["C"], scene["W"], scene["H"])
    return proj, isect, rgb, T, last, evals


def loss_and_grads(scene: dict, v_rgb=None, v_T=None, rows32: bool = False):
    """L = <v_rgb, out_rgb> + <v_T, out_T> and its parameter gradients."""
    v_rgb = scene["v_rgb"] if v_rgb is None else v_rgb
    v_T = scene["v_T"] if v_T is None else v_T
    proj, isect, rgb, T, last, _ = render(scene, rows32=rows32)
    L = float((np.asarray(v_rgb, np.float64) * rgb).sum() + (np.asarray(v_T, np.float64) * T).sum())
    v_screen = rasterize_bwd(proj.screen, isect.flatten_ids, isect.tile_offsets,
                             scene["C"], scene["W"], scene["H"], v_rgb, v_T)
    grads = project_bwd(scene, proj, v_screen)
    return L, grads, dict(proj=proj, isect=isect, rgb=rgb, T=T, last=last, v_screen=v_screen)
