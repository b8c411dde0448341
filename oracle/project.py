"""Packed projection of C cameras x N Gaussians (fp64 oracle).

Follows [VRAM] "Bitmask compaction": a mask over all C x N (camera,
Gaussian) pairs, one popcount per 128-pair work-group, an exclusive scan
of those counts, and a compacted list of visible pairs whose output slot
is (scan of earlier work-groups) + (set bits before this pair). The
plain definition of that scheme is a stable filter: slots enumerate the
visible pairs in increasing pair index p = c * N_pad + g, where
N_pad = ceil(N / 128) * 128 (padding pairs are never visible).

Per pair, the screen row is the pages' (xy, conic, opacity, depth, rgb)
([VRAM] per-element buffer cost table, "proj.screen"), 10 values:
(u, v, conic_a, conic_b, conic_c, opacity, z, r, g, b), and the box is the
16-bit AABB of [VRAM] "16-bit packed AABB".

Readings (the pages state no formula):
* camera: p = R mu + t from the row-major world->camera matrix (OpenCV
  axes); intrinsics fx = K00, fy = K11, cx = K02, cy = K12;
  pixel (i, j) has its centre at (j + 0.5, i + 0.5).
* near plane 0.01, no far plane, no field-of-view clamp in the Jacobian.
* covariance: q^ = q / |q| with q = (w, x, y, z); M = R(q^) diag(exp(s));
  Sigma3 = M M^T; EWA: J = [[fx/z, 0, -fx x/z^2], [0, fy/z, -fy y/z^2]],
  Sigma2 = J Rc Sigma3 Rc^T J^T + 0.3 I (the 0.3 px blur); the conic
  (a, b, c) holds entries (00, 01, 11) of Sigma2^-1.
* radius r = 3 sqrt(lambda_max(Sigma2)) (no rounding); box
  [u-r, u+r] x [v-r, v+r] intersected with [0, W] x [0, H]; a pair is
  visible iff its depth passes the near test and that box has positive
  width and height. No opacity cull.
* opacity = sigmoid(logit); colour from SH toward the camera centre
  -R^T t (see ``sh``).
* depth: the near test and the sort key both use z32, the camera-space
  depth evaluated in float32 as ((R20 x + R21 y) + R22 z) + t2 with every
  product and sum rounded to float32 (no fused multiply-add). The key
  needs the depth's exact bits, so the oracle computes them in the same
  precision and order as the kernel must.
* AABB16 ([VRAM] "16-bit packed AABB"): each edge is quantized on a
  uniform grid of 65535 steps over [0, extent]; the minimum edge rounds
  down, the maximum edge rounds up, both clamped to [0, 65535]. The
  scale 65535/extent and the product edge * scale are float32 (a float
  deciding an integer code: same precision as the kernel). Packing:
  word 0 = qx0 | qy0 << 16, word 1 = qx1 | qy1 << 16.
"""
from __future__ import annotations

import numpy as np

from .sh import sh_basis, num_sh

__all__ = ["quat_to_rotmat", "project_camera", "project", "depth32",
           "Projection", "NEAR", "BLUR", "MASK_GROUP"]

NEAR = 0.01
BLUR = 0.3
MASK_GROUP = 128
Q16 = 65535


def quat_to_rotmat(q: np.ndarray) -> np.ndarray:
    """Rotation matrix of unit quaternions q[..., 4] = (w, x, y, z)."""
    w, x, y, z = (q[..., i] for i in range(4))
    R = np.empty(q.shape[:-1] + (3, 3), np.float64)
    R[..., 0, 0] = 1 - 2 * (y * y + z * z)
    R[..., 0, 1] = 2 * (x * y - w * z)
    R[..., 0, 2] = 2 * (x * z + w * y)
    R[..., 1, 0] = 2 * (x * y + w * z)
    R[..., 1, 1] = 1 - 2 * (x * x + z * z)
    R[..., 1, 2] = 2 * (y * z - w * x)
    R[..., 2, 0] = 2 * (x * z - w * y)
    R[..., 2, 1] = 2 * (y * z + w * x)
    R[..., 2, 2] = 1 - 2 * (x * x + y * y)
    return R


def depth32(means: np.ndarray, viewmat: np.ndarray) -> np.ndarray:
    """Camera-space depth in float32, rounded after every operation."""
    m = np.asarray(means).astype(np.float32)
    R = np.asarray(viewmat).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        z = R[2, 0] * m[:, 0]
        z = z + R[2, 1] * m[:, 1]
        z = z + R[2, 2] * m[:, 2]
        z = z + R[2, 3]
    return z.astype(np.float32)


def quantize_aabb16(x0, x1, y0, y1, W: int, H: int):
    """(qx0, qy0, qx1, qy1) int64 codes of float box edges."""
    sx = np.float32(Q16) / np.float32(W)
    sy = np.float32(Q16) / np.float32(H)
    with np.errstate(invalid="ignore", over="ignore"):
        X0 = np.asarray(x0).astype(np.float32) * sx
        X1 = np.asarray(x1).astype(np.float32) * sx
        Y0 = np.asarray(y0).astype(np.float32) * sy
        Y1 = np.asarray(y1).astype(np.float32) * sy
        q = [np.clip(np.nan_to_num(f(v), nan=0.0), 0, Q16).astype(np.int64)
             for f, v in ((np.floor, X0), (np.floor, Y0), (np.ceil, X1), (np.ceil, Y1))]
    return q[0], q[1], q[2], q[3]


def project_camera(means, quats, log_scales, opacity_logits, sh, viewmat, K,
                   W: int, H: int, sh_degree: int) -> dict:
    """All per-pair quantities of one camera for the given Gaussians (fp64)."""
    mu = np.asarray(means, np.float64)
    V = np.asarray(viewmat, np.float64)
    K = np.asarray(K, np.float64)
    Rc, t = V[:3, :3], V[:3, 3]
    fx, fy, cx, cy = K[0, 0], K[1, 1], K[0, 2], K[1, 2]
    n = mu.shape[0]
    out = {}
    with np.errstate(all="ignore"):
        p = mu @ Rc.T + t
        x, y, z = p[:, 0], p[:, 1], p[:, 2]
        z32 = depth32(means, viewmat)
        q = np.asarray(quats, np.float64)
        qn = np.linalg.norm(q, axis=1)
        qh = q / qn[:, None]
        Rq = quat_to_rotmat(qh)
        s = np.exp(np.asarray(log_scales, np.float64))
        M = Rq * s[:, None, :]
        S3 = M @ np.swapaxes(M, 1, 2)
        Sc = Rc @ S3 @ Rc.T
        J = np.zeros((n, 2, 3))
        J[:, 0, 0] = fx / z
        J[:, 0, 2] = -fx * x / (z * z)
        J[:, 1, 1] = fy / z
        J[:, 1, 2] = -fy * y / (z * z)
        S2 = J @ Sc @ np.swapaxes(J, 1, 2)
        S2[:, 0, 0] += BLUR
        S2[:, 1, 1] += BLUR
        det = S2[:, 0, 0] * S2[:, 1, 1] - S2[:, 0, 1] * S2[:, 1, 0]
        conic_a = S2[:, 1, 1] / det
        conic_b = -S2[:, 0, 1] / det
        conic_c = S2[:, 0, 0] / det
        u = fx * x / z + cx
        v = fy * y / z + cy
        mid = 0.5 * (S2[:, 0, 0] + S2[:, 1, 1])
        lam = mid + np.sqrt(np.maximum(0.0, mid * mid - det))
        r = 3.0 * np.sqrt(lam)
        x0 = np.maximum(u - r, 0.0)
        x1 = np.minimum(u + r, float(W))
        y0 = np.maximum(v - r, 0.0)
        y1 = np.minimum(v + r, float(H))
        visible = (z32 > np.float32(NEAR)) & (x1 > x0) & (y1 > y0)
        opac = 1.0 / (1.0 + np.exp(-np.asarray(opacity_logits, np.float64)))
        cam_center = -Rc.T @ t
        dvec = mu - cam_center
        dnorm = np.linalg.norm(dvec, axis=1)
        d = dvec / dnorm[:, None]
        Y = sh_basis(sh_degree, d)
        shc = np.asarray(sh, np.float64).reshape(n, num_sh(sh_degree), 3)
        raw = np.einsum("nk,nkc->nc", Y, shc) + 0.5
        rgb = np.maximum(raw, 0.0)
    qx0, qy0, qx1, qy1 = quantize_aabb16(x0, x1, y0, y1, W, H)
    out.update(p=p, x=x, y=y, z=z, z32=z32, qn=qn, qh=qh, Rq=Rq, s=s, M=M,
               S3=S3, Sc=Sc, J=J, S2=S2, det=det, conic=np.stack([conic_a, conic_b, conic_c], 1),
               u=u, v=v, r=r, x0=x0, x1=x1, y0=y0, y1=y1, visible=visible,
               opacity=opac, dvec=dvec, dnorm=dnorm, d=d, Y=Y, raw=raw, rgb=rgb,
               qx0=qx0, qy0=qy0, qx1=qx1, qy1=qy1, Rc=Rc, fx=fx, fy=fy)
    return out


def screen_rows(pc: dict, idx: np.ndarray) -> np.ndarray:
    """The 10-value screen rows of the pairs ``idx`` of one camera."""
    return np.column_stack([
        pc["u"][idx], pc["v"][idx], pc["conic"][idx, 0], pc["conic"][idx, 1],
        pc["conic"][idx, 2], pc["opacity"][idx], pc["z32"][idx].astype(np.float64),
        pc["rgb"][idx, 0], pc["rgb"][idx, 1], pc["rgb"][idx, 2]])


class Projection:
    """Output of ``project``: the compacted visible-pair list and its mask."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def project(scene: dict, chunk: int = 1 << 18, keep_camera_data: bool = False) -> Projection:
    """Project every (camera, Gaussian) pair of ``scene`` (the inputs of gs_project).

    Returns mask words (uint64, bit b of word w = pair 64 w + b), per-128
    work-group counts and their exclusive scan (uint32), nnz, the pair index
    of every slot, screen rows [nnz, 10] (fp64; the depth column holds z32),
    AABB16 words [nnz, 2] (uint32) and the per-slot tile-relevant data
    (camera index, z32).
    """
    N, C, W, H = scene["N"], scene["C"], scene["W"], scene["H"]
    deg = scene["sh_degree"]
    Np = ((N + MASK_GROUP - 1) // MASK_GROUP) * MASK_GROUP
    vis = np.zeros(C * Np, bool)
    rows, aabb, zbits, cams = [], [], [], []
    per_cam = []
    for c in range(C):
        cam_rows, cam_aabb, cam_z = [], [], []
        for g0 in range(0, N, chunk):
            g1 = min(N, g0 + chunk)
            pc = project_camera(scene["means"][g0:g1], scene["quats"][g0:g1],
                                scene["log_scales"][g0:g1], scene["opacity_logits"][g0:g1],
                                scene["sh"][g0:g1], scene["viewmats"][c], scene["Ks"][c],
                                W, H, deg)
            if keep_camera_data:
                per_cam.append((c, g0, pc))
            idx = np.flatnonzero(pc["visible"])
            vis[c * Np + g0 + idx] = True
            cam_rows.append(screen_rows(pc, idx))
            w0 = (pc["qx0"][idx] | (pc["qy0"][idx] << 16)).astype(np.uint32)
            w1 = (pc["qx1"][idx] | (pc["qy1"][idx] << 16)).astype(np.uint32)
            cam_aabb.append(np.stack([w0, w1], 1))
            cam_z.append(pc["z32"][idx])
        rows += cam_rows
        aabb += cam_aabb
        zbits += cam_z
    pairs = np.flatnonzero(vis)
    bits = vis.reshape(-1, 64).astype(np.uint64)
    mask = (bits << np.arange(64, dtype=np.uint64)).sum(axis=1, dtype=np.uint64)
    wg_count = vis.reshape(-1, MASK_GROUP).sum(axis=1).astype(np.uint32)
    wg_scan = (np.cumsum(wg_count.astype(np.int64)) - wg_count).astype(np.uint32)
    screen = np.concatenate(rows) if rows else np.zeros((0, 10))
    aabb = np.concatenate(aabb) if aabb else np.zeros((0, 2), np.uint32)
    z32 = np.concatenate(zbits) if zbits else np.zeros(0, np.float32)
    return Projection(N=N, C=C, W=W, H=H, N_pad=Np, visible_pairs=vis, pairs=pairs,
                      nnz=int(pairs.size), mask=mask, wg_count=wg_count,
                      wg_scan=wg_scan, screen=screen, aabb16=aabb,
                      z32=z32.astype(np.float32), cam=pairs // Np, gauss=pairs % Np,
                      per_cam=per_cam)
