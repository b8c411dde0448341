"""Shared test helpers: hand-built scenes and independent reference maths."""
import numpy as np

import workloads


def make_scene_from(means, quats, log_scales, logits, sh, viewmats, Ks, W, H, deg,
                    v_rgb=None, v_T=None):
    means = np.asarray(means, np.float32).reshape(-1, 3)
    N = means.shape[0]
    viewmats = np.asarray(viewmats, np.float32).reshape(-1, 4, 4)
    C = viewmats.shape[0]
    K = (deg + 1) ** 2
    rng = np.random.default_rng(123)
    return dict(
        N=N, C=C, W=W, H=H, sh_degree=deg,
        means=means,
        quats=np.asarray(quats, np.float32).reshape(N, 4),
        log_scales=np.asarray(log_scales, np.float32).reshape(N, 3),
        opacity_logits=np.asarray(logits, np.float32).reshape(N),
        sh=np.asarray(sh, np.float32).reshape(N, K, 3),
        viewmats=viewmats,
        Ks=np.asarray(Ks, np.float32).reshape(C, 3, 3),
        v_rgb=(rng.normal(size=(C, H, W, 3)).astype(np.float32) if v_rgb is None else v_rgb),
        v_T=(rng.normal(size=(C, H, W)).astype(np.float32) if v_T is None else v_T),
    )


def intrinsics(fx, fy, W, H):
    return np.array([[fx, 0, W / 2], [0, fy, H / 2], [0, 0, 1]], np.float32)


def hamilton(p, q):
    """Quaternion product p q, (w, x, y, z) order."""
    pw, px, py, pz = p
    qw, qx, qy, qz = q
    return np.array([pw * qw - px * qx - py * qy - pz * qz,
                     pw * qx + px * qw + py * qz - pz * qy,
                     pw * qy - px * qz + py * qw + pz * qx,
                     pw * qz + px * qy - py * qx + pz * qw])


def rotate_by_quat(q, v):
    q = np.asarray(q, np.float64) / np.linalg.norm(q)
    qc = q * np.array([1, -1, -1, -1])
    return hamilton(hamilton(q, np.concatenate([[0.0], v])), qc)[1:]


def fd_scene(seed=7, N=30, C=2, W=40, H=36, deg=3, focal=50.0, ls_mu=-1.8):
    """A tiny scene for finite differences: big splats, unnormalised quats."""
    spec = workloads.SceneSpec("fd", N, deg, C, W, H, focal, 1.0, ls_mu, 0.3, 5.0,
                               sh_rest_sigma=0.3, seed=seed)
    sc = workloads.make_scene(spec)
    rng = np.random.default_rng(seed + 1)
    sc["quats"] = (sc["quats"] * rng.uniform(0.5, 2.0, size=(N, 1))).astype(np.float32)
    return sc
