"""Adam update of the Gaussian parameters (oracle), the optimizer that the
fused projection backward folds its gradients into.

[BWD] section 6, "fused projection backward + optimizer (FPBO)": with it
enabled, the world-space gradient accumulation is folded straight into the
Adam optimizer's registers and the fp32 gradient buffers are never
allocated. The pages name the optimizer but print no formula, so this is
Adam as Kingma and Ba define it (bias-corrected moments):

  m <- b1 m + (1 - b1) g,   v <- b2 v + (1 - b2) g^2,
  theta <- theta - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)

for step t >= 1, applied to every element, including Gaussians with a zero
gradient (the fused update must equal "write the gradients, then Adam").
Readings: one learning rate per attribute of [BWD] section 5's list --
means, quats, scales (log_scales here), opacities (logits), DC colour
(SH coefficient 0) and the higher SH coefficients.
"""
from __future__ import annotations

import numpy as np

__all__ = ["adam_step", "LR_KEYS"]

# the six learning-rate groups, in the order the library takes them
LR_KEYS = ("means", "quats", "log_scales", "opacity_logits", "sh_dc", "sh_rest")

_GRAD = {"means": "v_means", "quats": "v_quats", "log_scales": "v_log_scales",
         "opacity_logits": "v_opacity_logits", "sh": "v_sh"}


def _lr_array(name: str, shape, lr: dict) -> np.ndarray:
    if name != "sh":
        return np.full(shape, float(lr[name]))
    a = np.full(shape, float(lr["sh_rest"]))
    a[:, 0, :] = float(lr["sh_dc"])
    return a


def adam_step(params: dict, grads: dict, m: dict, v: dict, lr: dict, beta1: float,
              beta2: float, eps: float, step: int):
    """One Adam step (fp64) on the five parameter tensors.

    params / m / v: dicts keyed means, quats, log_scales, opacity_logits, sh;
    grads: keyed v_means, ... as ``project_bwd`` returns them; lr: keyed by
    LR_KEYS. Returns (new params, new m, new v); inputs are not modified.
    """
    assert step >= 1
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    out_p, out_m, out_v = {}, {}, {}
    for name, gname in _GRAD.items():
        p = np.asarray(params[name], np.float64)
        g = np.asarray(grads[gname], np.float64).reshape(p.shape)
        mm = beta1 * np.asarray(m[name], np.float64) + (1.0 - beta1) * g
        vv = beta2 * np.asarray(v[name], np.float64) + (1.0 - beta2) * g * g
        out_p[name] = p - _lr_array(name, p.shape, lr) * (mm / bc1) / (np.sqrt(vv / bc2) + eps)
        out_m[name] = mm
        out_v[name] = vv
    return out_p, out_m, out_v
