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
from .raster import rasterize_fwd, rasterize_bwd, background_grad
from .project_bwd import project_bwd

__all__ = ["render", "loss_and_grads"]


def render(scene: dict, rows32: bool = False, background=None, depth: bool = False):
    """(proj, isect, rgb, T, last, evals), plus the depth image last when
    ``depth`` is set; ``background`` is an optional [C, 3] colour."""
    proj = project(scene)
    if rows32:
        proj.screen = proj.screen.astype(np.float32).astype(np.float64)
    isect = intersect(proj, scene["W"], scene["H"])
    out = rasterize_fwd(proj.screen, isect.flatten_ids, isect.tile_offsets,
                        scene["C"], scene["W"], scene["H"], background=background, depth=depth)
    return (proj, isect) + tuple(out)


def loss_and_grads(scene: dict, v_rgb=None, v_T=None, rows32: bool = False, v_depth=None,
                   background=None):
    """L = <v_rgb, out_rgb> + <v_T, out_T> (+ <v_depth, out_depth>) and its
    parameter gradients; with a background, out_rgb is the blended image
    and aux["v_background"] holds dL/dbg."""
    v_rgb = scene["v_rgb"] if v_rgb is None else v_rgb
    v_T = scene["v_T"] if v_T is None else v_T
    proj, isect, rgb, T, last, _, D = render(scene, rows32=rows32, background=background,
                                             depth=True)
    L = float((np.asarray(v_rgb, np.float64) * rgb).sum() + (np.asarray(v_T, np.float64) * T).sum())
    if v_depth is not None:
        L += float((np.asarray(v_depth, np.float64) * D).sum())
    v_screen = rasterize_bwd(proj.screen, isect.flatten_ids, isect.tile_offsets,
                             scene["C"], scene["W"], scene["H"], v_rgb, v_T, v_depth=v_depth,
                             background=background)
    grads = project_bwd(scene, proj, v_screen)
    aux = dict(proj=proj, isect=isect, rgb=rgb, T=T, last=last, depth=D, v_screen=v_screen)
    if background is not None:
        aux["v_background"] = background_grad(T, v_rgb)
    return L, grads, aux
