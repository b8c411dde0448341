"""Pins for the oracle's Adam step (the optimizer of the fused projection
backward): the closed form of a constant gradient (every bias-corrected
step moves by lr g / (|g| + eps)), zero-gradient decay, the per-group
learning rates, and agreement with PyTorch's own Adam (an independent
library implementation) over several steps of random gradients."""
import numpy as np
import pytest
import torch

import oracle

NAMES = ("means", "quats", "log_scales", "opacity_logits", "sh")
SHAPES = {"means": (7, 3), "quats": (7, 4), "log_scales": (7, 3), "opacity_logits": (7,),
          "sh": (7, 9, 3)}
LR = {"means": 1.6e-4, "quats": 1e-3, "log_scales": 5e-3, "opacity_logits": 5e-2, "sh_dc": 2.5e-3,
      "sh_rest": 1.25e-4}


def _zeros():
    return {k: np.zeros(SHAPES[k]) for k in NAMES}


def _grads(rng):
    return {"v_" + k: rng.normal(size=SHAPES[k]) for k in NAMES}


def test_constant_gradient_closed_form():
    rng = np.random.default_rng(0)
    p0 = {k: rng.normal(size=SHAPES[k]) for k in NAMES}
    g = _grads(rng)
    p, m, v = p0, _zeros(), _zeros()
    b1, b2, eps = 0.9, 0.999, 1e-8
    for t in range(1, 6):
        p, m, v = oracle.adam_step(p, g, m, v, LR, b1, b2, eps, t)
    for k in NAMES:
        gk = g["v_" + k]
        lr = np.full(SHAPES[k], LR[k] if k != "sh" else LR["sh_rest"])
        if k == "sh":
            lr[:, 0, :] = LR["sh_dc"]
        np.testing.assert_allclose(p[k], p0[k] - 5 * lr * gk / (np.abs(gk) + eps), rtol=0, atol=1e-12)


def test_zero_gradient_only_decays_moments():
    rng = np.random.default_rng(1)
    p0 = {k: rng.normal(size=SHAPES[k]) for k in NAMES}
    m0 = {k: rng.normal(size=SHAPES[k]) for k in NAMES}
    v0 = {k: rng.uniform(0.1, 1, SHAPES[k]) for k in NAMES}
    g = {"v_" + k: np.zeros(SHAPES[k]) for k in NAMES}
    p, m, v = oracle.adam_step(p0, g, m0, v0, LR, 0.9, 0.999, 1e-8, 3)
    for k in NAMES:
        np.testing.assert_allclose(m[k], 0.9 * m0[k], rtol=1e-15)
        np.testing.assert_allclose(v[k], 0.999 * v0[k], rtol=1e-15)
        assert np.all(np.sign(p0[k] - p[k]) == np.sign(m0[k]))   # momentum keeps moving


@pytest.mark.parametrize("eps", [1e-8, 1e-15])
def test_matches_torch_adam(eps):
    rng = np.random.default_rng(2)
    p0 = {k: rng.normal(size=SHAPES[k]) for k in NAMES}
    b1, b2 = 0.9, 0.999
    # torch.optim.Adam with one parameter group per learning rate
    tp = {k: torch.tensor(p0[k], dtype=torch.float64, requires_grad=True) for k in NAMES}
    sh_dc = torch.tensor(p0["sh"][:, :1], dtype=torch.float64, requires_grad=True)
    sh_rest = torch.tensor(p0["sh"][:, 1:], dtype=torch.float64, requires_grad=True)
    groups = [{"params": [tp[k]], "lr": LR[k]} for k in NAMES if k != "sh"]
    groups += [{"params": [sh_dc], "lr": LR["sh_dc"]}, {"params": [sh_rest], "lr": LR["sh_rest"]}]
    opt = torch.optim.Adam(groups, betas=(b1, b2), eps=eps)
    p, m, v = p0, _zeros(), _zeros()
    for t in range(1, 8):
        g = _grads(rng)
        for k in NAMES:
            if k != "sh":
                tp[k].grad = torch.tensor(g["v_" + k])
        sh_dc.grad = torch.tensor(g["v_sh"][:, :1])
        sh_rest.grad = torch.tensor(g["v_sh"][:, 1:])
        opt.step()
        p, m, v = oracle.adam_step(p, g, m, v, LR, b1, b2, eps, t)
    for k in NAMES:
        ref = (torch.cat([sh_dc, sh_rest], 1) if k == "sh" else tp[k]).detach().numpy()
        np.testing.assert_allclose(p[k], ref, rtol=1e-12, atol=1e-14)
