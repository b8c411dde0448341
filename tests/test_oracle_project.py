"""Pins for the oracle's projection: closed forms, Monte Carlo, invariants,
the 16-bit box quantization and the pages' printed quantization steps."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads
from oracle.project import project_camera, quantize_aabb16, depth32
from tests.helpers import make_scene_from, intrinsics, rotate_by_quat

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_rotation_matches_hamilton_product():
    rng = np.random.default_rng(3)
    for _ in range(20):
        q = rng.normal(size=4)
        v = rng.normal(size=3)
        R = oracle.quat_to_rotmat(q / np.linalg.norm(q))
        np.testing.assert_allclose(R @ v, rotate_by_quat(q, v), atol=1e-12)
        np.testing.assert_allclose(R @ R.T, np.eye(3), atol=1e-12)
        assert np.linalg.det(R) == pytest.approx(1.0, abs=1e-12)


@pytest.mark.parametrize("fx,fy,depth,ls", [(111.0, 111.0, 5.0, -3.0), (300.0, 170.0, 2.5, -1.0)])
def test_isotropic_on_axis_closed_form(fx, fy, depth, ls):
    W, H = 128, 96
    vm = workloads.lookat_viewmat((0, 0, depth))
    q = np.array([0.3, -0.5, 0.7, 0.1])      # rotation must not matter
    pc = project_camera(np.zeros((1, 3)), q[None], np.full((1, 3), ls), np.zeros(1),
                        np.zeros((1, 1, 3)), vm, intrinsics(fx, fy, W, H), W, H, 0)
    s = math.exp(float(np.float32(ls)))
    vx = (fx * s / depth) ** 2 + 0.3
    vy = (fy * s / depth) ** 2 + 0.3
    np.testing.assert_allclose(pc["conic"][0], [1 / vx, 0.0, 1 / vy], rtol=1e-12, atol=1e-15)
    assert pc["u"][0] == pytest.approx(W / 2) and pc["v"][0] == pytest.approx(H / 2)
    assert pc["r"][0] == pytest.approx(3 * math.sqrt(max(vx, vy)), rel=1e-12)
    assert pc["z"][0] == pytest.approx(depth)


def test_isotropic_off_axis_closed_form():
    fx, fy, W, H = 200.0, 150.0, 320, 240
    vm = np.eye(4)                             # world == camera
    x, y, z = 0.7, -0.4, 3.0
    s = 0.05
    pc = project_camera(np.array([[x, y, z]]), np.array([[1.0, 0, 0, 0]]),
                        np.full((1, 3), math.log(s)), np.zeros(1), np.zeros((1, 1, 3)),
                        vm, intrinsics(fx, fy, W, H), W, H, 0)
    s2 = s ** 2
    Sxx = s2 * (fx / z) ** 2 * (1 + (x / z) ** 2) + 0.3
    Syy = s2 * (fy / z) ** 2 * (1 + (y / z) ** 2) + 0.3
    Sxy = s2 * fx * fy * x * y / z**4
    det = Sxx * Syy - Sxy**2
    np.testing.assert_allclose(pc["conic"][0], [Syy / det, -Sxy / det, Sxx / det], rtol=1e-12)
    assert pc["u"][0] == pytest.approx(fx * x / z + W / 2)
    assert pc["v"][0] == pytest.approx(fy * y / z + H / 2)


def test_monte_carlo_projected_covariance():
    """Empirical covariance of projected 3D samples -> J W Sigma3 W^T J^T."""
    rng = np.random.default_rng(11)
    fx, fy, W, H = 400.0, 380.0, 640, 480
    vm = workloads.lookat_viewmat((2.0, 1.0, 6.0), target=(0.3, -0.2, 0.0))
    mu = np.array([0.9, -0.6, 0.4])
    q = np.array([0.8, 0.3, -0.5, 0.2])
    scales = np.array([0.012, 0.004, 0.007])
    axes = np.stack([rotate_by_quat(q, e) for e in np.eye(3)])      # rows: rotated axes
    n = 2_000_000
    xi = rng.normal(size=(n, 3)) * scales
    X = mu + xi @ axes
    P = X @ vm[:3, :3].T + vm[:3, 3]
    uv = np.stack([fx * P[:, 0] / P[:, 2] + W / 2, fy * P[:, 1] / P[:, 2] + H / 2], 1)
    emp = np.cov(uv.T)
    pc = project_camera(mu[None], q[None], np.log(scales)[None], np.zeros(1),
                        np.zeros((1, 1, 3)), vm, intrinsics(fx, fy, W, H), W, H, 0)
    S2 = pc["S2"][0] - 0.3 * np.eye(2)
    scale = np.abs(S2).max()
    assert np.abs(emp - S2).max() < 0.01 * scale
    np.testing.assert_allclose(uv.mean(0), [pc["u"][0], pc["v"][0]], atol=0.02)


def test_visibility_cases():
    W, H, f = 100, 80, 90.0
    vm = np.eye(4)
    means = np.array([
        [0.0, 0.0, 3.0],      # centre: visible
        [0.0, 0.0, -3.0],     # behind: invisible
        [0.0, 0.0, 0.005],    # in front of the near plane: invisible
        [50.0, 0.0, 3.0],     # far right: invisible
        [0.0, 0.0, 0.02],     # just past the near plane, on axis: visible
    ])
    n = len(means)
    pc = project_camera(means, np.tile([1.0, 0, 0, 0], (n, 1)), np.full((n, 3), -3.0),
                        np.zeros(n), np.zeros((n, 1, 3)), vm, intrinsics(f, f, W, H), W, H, 0)
    assert pc["visible"].tolist() == [True, False, False, False, True]
    # box touching the right border from outside: u - r == W is not visible
    x = 3.0 * (W / 2 + 3.0) / f   # u = W + 3 px
    s = 0.01
    pc = project_camera(np.array([[x, 0, 3.0]]), np.array([[1.0, 0, 0, 0]]),
                        np.full((1, 3), math.log(s)), np.zeros(1), np.zeros((1, 1, 3)), vm,
                        intrinsics(f, f, W, H), W, H, 0)
    assert (pc["u"][0] - pc["r"][0] < W) == bool(pc["visible"][0])


def test_radius_bound_and_centre_rule():
    """Two facts a visibility test may use to settle pairs early, checked on
    the fp64 projection: the screen radius 3 sqrt(lambda_max) is at most
    3 sqrt(|J R_cam|_F^2 max(s)^2 + 2 blur) (lambda_max is at most the 2D
    covariance's trace, |J R_cam M|_F^2 + 2 blur, and |J R_cam M|_F is at
    most |J R_cam|_F |M|_2 with |M|_2 = max(s) for a rotation times a
    diagonal), including for a camera matrix that is not a rotation; and a
    pair past the near plane whose centre lies inside the image is visible
    whatever its size."""
    rng = np.random.default_rng(11)
    W, H = 160, 120
    n = 20000
    for skew in (False, True):
        vm = workloads.lookat_viewmat((0.3, -0.2, 4.0))
        if skew:
            vm[:3, :3] *= 1.7
            vm[0, 1] += 0.6
            vm[2, 0] -= 0.3
        means = rng.uniform(-3, 3, (n, 3))
        quats = rng.normal(size=(n, 4)) * (10.0 ** rng.uniform(-6, 6, n))[:, None]
        ls = rng.uniform(-9, 2, (n, 3))
        K = intrinsics(rng.uniform(60, 400), rng.uniform(60, 400), W, H)
        pc = project_camera(means, quats, ls, np.zeros(n), np.zeros((n, 1, 3)), vm, K, W, H, 0)
        front = pc["z"] > 0.05
        R = np.asarray(vm, np.float64)[:3, :3]
        x, y, z = pc["x"], pc["y"], pc["z"]
        JR0 = (K[0, 0] / z)[:, None] * (R[0][None, :] - (x / z)[:, None] * R[2][None, :])
        JR1 = (K[1, 1] / z)[:, None] * (R[1][None, :] - (y / z)[:, None] * R[2][None, :])
        jr2 = (JR0 ** 2).sum(1) + (JR1 ** 2).sum(1)
        smax = np.exp(np.asarray(ls, np.float64).max(1))
        bound = 3.0 * np.sqrt(jr2 * smax ** 2 + 2 * 0.3)
        r = pc["r"]
        assert np.all(r[front] <= bound[front] * (1 + 1e-12)), np.max(r[front] / bound[front])
        # the bound is not vacuous: within a factor 3 for most pairs
        assert np.median(bound[front] / r[front]) < 3.0
        inside = front & (pc["z32"] > 0.01) & (pc["u"] > 0) & (pc["u"] < W) & (pc["v"] > 0) & (pc["v"] < H)
        assert inside.sum() > 1000 and np.all(pc["visible"][inside])



@pytest.mark.parametrize("name", ["tiny", "multicam", "sh1-odd-n"])
def test_compaction_invariants(name):
    sc = workloads.make_scene(workloads.SMALL[name])
    pr = oracle.project(sc)
    pop = sum(bin(int(w)).count("1") for w in pr.mask)
    assert pr.nnz == pop == int(pr.wg_count.sum())
    assert np.array_equal(pr.wg_scan[1:], np.cumsum(pr.wg_count)[:-1].astype(np.uint32))
    assert pr.wg_scan[0] == 0
    # slots enumerate the visible pairs in increasing pair index (brute force)
    slot = 0
    for c in range(pr.C):
        pc = project_camera(sc["means"], sc["quats"], sc["log_scales"], sc["opacity_logits"],
                            sc["sh"], sc["viewmats"][c], sc["Ks"][c], sc["W"], sc["H"],
                            sc["sh_degree"])
        for g in range(pr.N_pad):
            vis = g < sc["N"] and bool(pc["visible"][g])
            word, bit = divmod(c * pr.N_pad + g, 64)
            assert bool((int(pr.mask[word]) >> bit) & 1) == vis
            if vis:
                assert pr.pairs[slot] == c * pr.N_pad + g
                assert pr.screen[slot, 0] == pc["u"][g]
                slot += 1
    assert slot == pr.nnz
    # the per-work-group count is the popcount of its two 64-bit words
    for w in range(len(pr.wg_count)):
        bits = bin(int(pr.mask[2 * w])).count("1") + bin(int(pr.mask[2 * w + 1])).count("1")
        assert bits == pr.wg_count[w]


def test_depth32_bits():
    rng = np.random.default_rng(5)
    m = rng.uniform(-2, 2, size=(1000, 3)).astype(np.float32)
    vm = workloads.lookat_viewmat((0, 0, 5)).astype(np.float32)
    # axis-aligned camera: the row (0, 0, -1, 5) leaves one rounding, 5 - z
    assert np.array_equal(depth32(m, vm), np.float32(5.0) - m[:, 2])
    vm2 = workloads.camera_rig(workloads.CONFIGS[3])[0][1]
    z64 = m.astype(np.float64) @ vm2[2, :3].astype(np.float64) + float(vm2[2, 3])
    z32 = depth32(m, vm2).astype(np.float64)
    assert np.all(np.abs(z32 - z64) <= 4 * np.spacing(np.float32(8.0)))


def test_aabb16_contains_box_and_step():
    rng = np.random.default_rng(9)
    for W in (97, 608, 1920, 6000):
        x0 = rng.uniform(0, W, 20000)
        x1 = np.minimum(W, x0 + rng.uniform(0, 30, 20000))
        qx0, _, qx1, _ = quantize_aabb16(x0, x1, np.zeros_like(x0), np.ones_like(x0), W, 1)
        step = W / 65535.0
        slack = 2 * np.spacing(np.float32(65535.0)) * step   # fp32 rounding of the scaled edge
        lo, hi = qx0 * step, qx1 * step
        assert np.all(lo <= x0 + slack) and np.all(hi >= x1 - slack)
        assert np.all(x0 - lo < step + slack) and np.all(hi - x1 < step + slack)
        xs = np.sort(x0)
        q_sorted, _, _, _ = quantize_aabb16(xs, xs, xs * 0, xs * 0 + 1, W, 1)
        assert np.all(np.diff(q_sorted) >= 0)
        # clamps to the code range
        q = quantize_aabb16(np.array([0.0]), np.array([float(W)]), np.zeros(1), np.ones(1), W, 1)
        assert q[0][0] == 0 and q[2][0] == 65535


def test_pages_quantization_steps():
    """[VRAM] "16-bit packed AABB": the step is extent/65535, printed as
    0.009 px at 608 px and 0.09 px at 6000 px."""
    with open(os.path.join(GOLDEN, "pages_numbers.json")) as f:
        g = json.load(f)["aabb16_step"]
    for case in g["cases"]:
        W = case["extent_px"]
        xs = np.linspace(0, W, 2_000_001)
        q, _, _, _ = quantize_aabb16(xs, xs, xs * 0, xs * 0 + 1, W, 1)
        change = xs[1:][np.diff(q) > 0]
        step = (change[-1] - change[0]) / (change.size - 1)   # mean code width
        assert round(step, case["digits"]) == case["printed_step_px"]
        assert step == pytest.approx(W / 65535, rel=2e-3)


def test_sh_colour_uses_view_direction_from_camera_centre():
    """Colour = max(0, sum_k sh_k Y_k(d) + 0.5) with d the unit vector from the
    camera's position (the look-at eye, not the translation column) to the mean."""
    rng = np.random.default_rng(17)
    eye = np.array([1.5, -2.0, 4.0])
    vm = workloads.lookat_viewmat(eye, target=(0.2, 0.1, -0.3))
    mu = rng.uniform(-0.5, 0.5, size=(8, 3))
    sh = rng.normal(0, 0.6, size=(8, 16, 3))
    pc = project_camera(mu, np.tile([1.0, 0, 0, 0], (8, 1)), np.full((8, 3), -3.0), np.zeros(8),
                        sh, vm, intrinsics(300, 300, 256, 256), 256, 256, 3)
    d = (mu - eye) / np.linalg.norm(mu - eye, axis=1, keepdims=True)
    Y = oracle.sh_basis(3, d)
    raw = np.einsum("nk,nkc->nc", Y, sh) + 0.5
    np.testing.assert_allclose(pc["rgb"], np.maximum(raw, 0.0), atol=1e-12)
    assert np.any(raw < 0)          # the clamp is exercised
