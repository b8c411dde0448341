"""Plain fp64 CPU oracle for the differentiable 16x16-tile Gaussian rasterizer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package. The HIP library never calls it, and
this package imports nothing from the HIP path or its Python binding: the
two share only the seeded input generator in ``workloads``.

Sources. The pages this follows are four web pages about a 3D Gaussian
Splatting trainer:

* [VRAM] "Spirula Studio VRAM deep dive: the splat x img category and
  bitmask compaction" -- sections "Three key numbers" (C x N, nnz,
  n_isects), the per-element buffer cost table, "Bitmask compaction",
  "16-bit packed AABB" and "The 4 GiB rule and the 2^31 limit".
* [BWD] "How Spirula Studio's backward pass sends image gradients back to
  every Gaussian" -- sections 2-3 (the per-pixel output gradients of the
  colour, depth and transmittance images; the background hook), 4
  (rasterize backward), 5 (projection backward) and 6 (the fused
  projection backward + Adam).
* [PROFILE] "Performance profiling guide: reading every step with
  SS_PROFILE=1" (kernel names only).
* [GSPLAT] a deployment blog about a CUDA splatting library (C API over
  caller-owned device pointers).

The pages print no projection or compositing formula. Everything below
that is not quoted from them is the textbook 3D Gaussian Splatting
pipeline (EWA splatting of a 3D covariance, 3-sigma screen radius,
alpha = opacity * exp(-1/2 d^T Sigma^-1 d) clamped to 0.99, skipped
below 1/255, front-to-back compositing stopping once T < 1e-4), with the
open points fixed by the readings listed in each function.

Every function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, brute force, invariants, SciPy, the pages' printed numbers
or central finite differences. No function is "parity unpinned".

Floating point: all arithmetic is float64, except the two places where a
float decides an integer and the pages' method fixes the kernel's
precision (the fp32 depth bits in the sort key and the fp32 scaling in
the 16-bit box quantization); there the oracle takes the decision in
float32, exactly as the rasterizer must.
"""
from .sh import sh_basis, sh_basis_grad, num_sh
from .project import project, project_camera, quat_to_rotmat
from .intersect import intersect, tile_rects_from_aabb16
from .raster import rasterize_fwd, rasterize_bwd, background_grad
from .project_bwd import project_bwd
from .pipeline import render, loss_and_grads
from .adam import adam_step, LR_KEYS

__all__ = [
    "sh_basis", "sh_basis_grad", "num_sh", "project", "project_camera",
    "quat_to_rotmat", "intersect", "tile_rects_from_aabb16", "rasterize_fwd",
    "rasterize_bwd", "background_grad", "project_bwd", "render", "loss_and_grads",
    "adam_step", "LR_KEYS",
]
