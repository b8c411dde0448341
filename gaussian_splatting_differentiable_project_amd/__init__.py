"""Differentiable 16x16-tile Gaussian rasterizer for MI355X (gfx950).

The compute path is the HIP library ``libgs.so`` (C ABI in include/gs.h);
this package is its thin ctypes binding plus the build script.
"""
from ._lib import (GS_OK, GS_E_INVALID, GS_E_CAPACITY, GS_E_WORKSPACE, GS_E_OVERFLOW, GS_E_HIP,
                   GS_E_DEVICE, EXPORTS, GsError, Rasterizer, Scene, Projected, Intersected,
                   AdamState, PhaseArena, ARENA_SLOTS, load, status_str, pad_n, tiles, gs_project,
                   gs_project_noalloc, gs_intersect, gs_rasterize_fwd, gs_rasterize_bwd, gs_project_bwd,
                   gs_project_bwd_adam, gs_arena_plan,
                   profile_enable, profile_disable, profile_reset, profile_query, valu_probe)

__all__ = ["GS_OK", "GS_E_INVALID", "GS_E_CAPACITY", "GS_E_WORKSPACE", "GS_E_OVERFLOW",
           "GS_E_HIP", "GS_E_DEVICE", "EXPORTS", "GsError", "Rasterizer", "Scene", "Projected",
           "Intersected", "AdamState", "PhaseArena", "ARENA_SLOTS", "load", "status_str", "pad_n",
           "tiles", "gs_project", "gs_project_noalloc", "gs_arena_plan",
           "gs_intersect", "gs_rasterize_fwd", "gs_rasterize_bwd", "gs_project_bwd",
           "gs_project_bwd_adam",
           "profile_enable", "profile_disable", "profile_reset", "profile_query", "valu_probe"]
