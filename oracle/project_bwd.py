"""Projection backward (oracle): screen-row gradients -> parameter gradients.

[BWD] section 5 (``projection_3dgs_backward``): the chain rule through the
camera intrinsics and extrinsics turns each Gaussian's screen-space
gradient into gradients of its position, rotation, scale, opacity, DC
colour and higher SH coefficients; the gradients are float32 buffers.
[BWD] section 6: only the first sub-batch zeroes the accumulators, later
ones add into them (the ``accumulate`` flag of the library).

This is the exact chain rule of ``project.project_camera`` w.r.t. the raw
inputs, summed over every camera in which the Gaussian is visible:
means (camera transform, Jacobian's dependence on the camera-space point,
and the SH view direction), raw quaternions (through normalisation),
log-scales (through exp), opacity logits (through the sigmoid) and SH
coefficients (zero where the colour clamp at 0 is active). No gradient
flows through the radius, the box, the tile rectangle or the visibility
test, which are piecewise constant.
"""
from __future__ import annotations

import numpy as np

from .project import project_camera
from .sh import sh_basis_grad, num_sh

__all__ = ["project_bwd", "rotmat_grad"]


def rotmat_grad(q: np.ndarray) -> np.ndarray:
    """dR/dq for R = quat_to_rotmat(q): shape [..., 4, 3, 3], q = (w, x, y, z)."""
    w, x, y, z = (q[..., i] for i in range(4))
    G = np.zeros(q.shape[:-1] + (4, 3, 3))
    # d/dw
    G[..., 0, 0, 1] = -2 * z; G[..., 0, 0, 2] = 2 * y
    G[..., 0, 1, 0] = 2 * z;  G[..., 0, 1, 2] = -2 * x
    G[..., 0, 2, 0] = -2 * y; G[..., 0, 2, 1] = 2 * x
    # d/dx
    G[..., 1, 0, 1] = 2 * y;  G[..., 1, 0, 2] = 2 * z
    G[..., 1, 1, 0] = 2 * y;  G[..., 1, 1, 1] = -4 * x; G[..., 1, 1, 2] = -2 * w
    G[..., 1, 2, 0] = 2 * z;  G[..., 1, 2, 1] = 2 * w;  G[..., 1, 2, 2] = -4 * x
    # d/dy
    G[..., 2, 0, 0] = -4 * y; G[..., 2, 0, 1] = 2 * x;  G[..., 2, 0, 2] = 2 * w
    G[..., 2, 1, 0] = 2 * x;  G[..., 2, 1, 2] = 2 * z
    G[..., 2, 2, 0] = -2 * w; G[..., 2, 2, 1] = 2 * z;  G[..., 2, 2, 2] = -4 * y
    # d/dz
    G[..., 3, 0, 0] = -4 * z; G[..., 3, 0, 1] = -2 * w; G[..., 3, 0, 2] = 2 * x
    G[..., 3, 1, 0] = 2 * w;  G[..., 3, 1, 1] = -4 * z; G[..., 3, 1, 2] = 2 * y
    G[..., 3, 2, 0] = 2 * x;  G[..., 3, 2, 1] = 2 * y
    return G


def project_bwd(scene: dict, proj, v_screen: np.ndarray) -> dict:
    """Parameter gradients from screen-row gradients ``v_screen[nnz, 10]``."""
    N, C, W, H, deg = scene["N"], scene["C"], scene["W"], scene["H"], scene["sh_degree"]
    K = num_sh(deg)
    g_means = np.zeros((N, 3))
    g_quats = np.zeros((N, 4))
    g_ls = np.zeros((N, 3))
    g_op = np.zeros(N)
    g_sh = np.zeros((N, K, 3))
    v_screen = np.asarray(v_screen, np.float64)
    for c in range(C):
        sel = np.flatnonzero(proj.cam == c)
        if sel.size == 0:
            continue
        g = proj.gauss[sel].astype(np.int64)
        vs = v_screen[sel]
        pc = project_camera(scene["means"][g], scene["quats"][g], scene["log_scales"][g],
                            scene["opacity_logits"][g], scene["sh"][g], scene["viewmats"][c],
                            scene["Ks"][c], W, H, deg)
        vu, vv, va, vb, vc, vo, vz = (vs[:, i] for i in range(7))
        v_rgb = vs[:, 7:10]
        # colour: rgb = max(0, sum_k sh_k Y_k(d) + 0.5), d = (mu - cam) / |mu - cam|
        v_raw = v_rgb * (pc["raw"] > 0.0)
        g_sh[g] += pc["Y"][:, :, None] * v_raw[:, None, :]
        shc = np.asarray(scene["sh"][g], np.float64).reshape(-1, K, 3)
        v_Y = np.einsum("nkc,nc->nk", shc, v_raw)
        v_d = np.einsum("nk,nkj->nj", v_Y, sh_basis_grad(deg, pc["d"]))
        d = pc["d"]
        v_mu = (v_d - d * (d * v_d).sum(1, keepdims=True)) / pc["dnorm"][:, None]
        # opacity = sigmoid(logit)
        o = pc["opacity"]
        g_op[g] += vo * o * (1.0 - o)
        # conic = Sigma2^-1
        A = np.zeros((sel.size, 2, 2))
        A[:, 0, 0] = pc["conic"][:, 0]; A[:, 0, 1] = A[:, 1, 0] = pc["conic"][:, 1]
        A[:, 1, 1] = pc["conic"][:, 2]
        V = np.zeros((sel.size, 2, 2))
        V[:, 0, 0] = va; V[:, 0, 1] = V[:, 1, 0] = 0.5 * vb; V[:, 1, 1] = vc
        vS2 = -A @ V @ A
        # Sigma2 = J Sc J^T + blur
        J, Sc = pc["J"], pc["Sc"]
        vJ = 2.0 * vS2 @ J @ Sc
        vSc = np.swapaxes(J, 1, 2) @ vS2 @ J
        # camera-space point p = (x, y, z): Jacobian entries, (u, v) and depth
        x, y, z = pc["x"], pc["y"], pc["z"]
        fx, fy = pc["fx"], pc["fy"]
        vx = vJ[:, 0, 2] * (-fx / z**2) + vu * fx / z
        vy = vJ[:, 1, 2] * (-fy / z**2) + vv * fy / z
        vzz = (vJ[:, 0, 0] * (-fx / z**2) + vJ[:, 0, 2] * (2.0 * fx * x / z**3)
               + vJ[:, 1, 1] * (-fy / z**2) + vJ[:, 1, 2] * (2.0 * fy * y / z**3)
               - vu * fx * x / z**2 - vv * fy * y / z**2 + vz)
        vp = np.stack([vx, vy, vzz], 1)
        Rc = pc["Rc"]
        v_mu += vp @ Rc
        g_means[g] += v_mu
        # Sc = Rc Sigma3 Rc^T; Sigma3 = M M^T; M = Rq diag(s)
        vS3 = Rc.T @ vSc @ Rc
        M, Rq, s = pc["M"], pc["Rq"], pc["s"]
        vM = 2.0 * vS3 @ M
        vRq = vM * s[:, None, :]
        vs_ = (vM * Rq).sum(1)
        g_ls[g] += vs_ * s
        qh, qn = pc["qh"], pc["qn"]
        vqh = np.einsum("nij,nkij->nk", vRq, rotmat_grad(qh))
        g_quats[g] += (vqh - qh * (qh * vqh).sum(1, keepdims=True)) / qn[:, None]
    return dict(v_means=g_means, v_quats=g_quats, v_log_scales=g_ls,
                v_opacity_logits=g_op, v_sh=g_sh)
