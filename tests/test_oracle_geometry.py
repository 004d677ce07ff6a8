"""Pins of the oracle's projection (steps 1-7) against mathematics.

Nothing here is checked against the oracle itself: rotations against the
Hamilton-product action of a quaternion, covariances against their
eigen-decomposition, the EWA 2D covariance against a closed form on the
optical axis and against a numerically differentiated pinhole projection off
axis, the radius against a library eigen-solver, and the tile rect against a
brute-force interval test of every tile.
"""
import numpy as np
import pytest

import oracle
from differentiable_rasterization_amd import scenes


def hamilton(a, b):
    w1, x1, y1, z1 = a
    w2, x2, y2, z2 = b
    return np.array([w1 * w2 - x1 * x2 - y1 * y2 - z1 * z2,
                     w1 * x2 + x1 * w2 + y1 * z2 - z1 * y2,
                     w1 * y2 - x1 * z2 + y1 * w2 + z1 * x2,
                     w1 * z2 + x1 * y2 - y1 * x2 + z1 * w2])


def rotate_by_quat(q, v):
    q = np.asarray(q, float) / np.linalg.norm(q)
    qc = q * np.array([1, -1, -1, -1])
    return hamilton(hamilton(q, np.concatenate([[0.0], v])), qc)[1:]


def test_rotation_is_quaternion_action():
    rng = np.random.default_rng(0)
    for _ in range(200):
        q = rng.normal(size=4) * rng.uniform(0.1, 10)  # any non-zero norm
        R = oracle.rotation(q)
        np.testing.assert_allclose(R @ R.T, np.eye(3), atol=1e-12)
        assert abs(np.linalg.det(R) - 1.0) < 1e-12
        for _ in range(3):
            v = rng.normal(size=3)
            np.testing.assert_allclose(R @ v, rotate_by_quat(q, v), atol=1e-12)


def test_identity_quaternion():
    # identity initialisation [1,0,0,0] of the gsplat guide §3.3
    np.testing.assert_array_equal(oracle.rotation([1, 0, 0, 0]), np.eye(3))
    S = oracle.cov3d([1, 0, 0, 0], [0.01, 0.01, 0.01])
    np.testing.assert_allclose(S, 1e-4 * np.eye(3), rtol=1e-14)


def test_cov3d_isotropic_and_principal_axes():
    rng = np.random.default_rng(1)
    for _ in range(100):
        q = rng.normal(size=4)
        s = float(rng.uniform(0.01, 2.0))
        np.testing.assert_allclose(oracle.cov3d(q, [s, s, s]), s * s * np.eye(3), atol=1e-13)
        sc = rng.uniform(0.01, 2.0, size=3)
        S = oracle.cov3d(q, sc)
        np.testing.assert_allclose(S, S.T, atol=1e-15)
        np.testing.assert_allclose(np.linalg.eigvalsh(S), np.sort(sc ** 2), rtol=1e-10)
        for j in range(3):  # axis j of the Gaussian is q e_j q*, with variance s_j^2
            e = np.zeros(3)
            e[j] = 1.0
            a = rotate_by_quat(q, e)
            np.testing.assert_allclose(S @ a, sc[j] ** 2 * a, atol=1e-12)


def _single(mean, scale, quat=(1, 0, 0, 0), deg=0):
    K = (deg + 1) ** 2
    return (np.array([mean], float), np.array([scale], float), np.array([quat], float),
            np.zeros((1, K, 3)))


@pytest.mark.parametrize("eps2d", [0.0, 0.3])
def test_ewa_on_axis_closed_form(eps2d):
    cam = scenes.identity_camera(64, 48, 64.0, 50.0)
    for z, s in [(2.0, 0.05), (4.0, 0.1), (7.5, 0.3)]:
        q = np.random.default_rng(int(z * 10)).normal(size=4)  # isotropic: rotation irrelevant
        m, sc, qq, sh = _single([0.0, 0.0, z], [s, s, s], q)
        p = oracle.project(m, sc, qq, sh, 0, cam, dict(eps2d=eps2d), oracle.MODE_F64)
        a, b, c = p["cov2d"][0]
        e = float(np.float32(eps2d))  # the method's constants are fp32 values
        np.testing.assert_allclose(a, (64.0 * s / z) ** 2 + e, rtol=1e-12)
        np.testing.assert_allclose(c, (50.0 * s / z) ** 2 + e, rtol=1e-12)
        assert abs(b) < 1e-12
        np.testing.assert_allclose(p["means2d"][0], [32.0, 24.0], atol=1e-12)
        assert p["depths"][0] == z


def _pinhole(cam, t):
    return np.array([cam.fx * t[0] / t[2] + cam.cx, cam.fy * t[1] / t[2] + cam.cy])


def test_ewa_off_axis_against_numerical_jacobian():
    """Sigma2D = J W Sigma W^T J^T with J the Jacobian of the pinhole map,
    here obtained by central differences of the map itself (the form of the
    2D covariance stated for the projection step)."""
    rng = np.random.default_rng(2)
    cams = scenes.sphere_poses(3, 6.0, 7, 320, 200, 180.0)
    for cam in cams:
        W = np.asarray(cam.R, float)
        tc = np.asarray(cam.t, float)
        for _ in range(20):
            # a point in view: pick camera-space t then map back to world
            t = np.array([rng.uniform(-1, 1), rng.uniform(-0.6, 0.6), 1.0]) * rng.uniform(2, 8)
            mean = np.linalg.solve(W, t - tc)  # W is orthonormal only to fp32 accuracy
            sc = rng.uniform(0.02, 0.3, size=3)
            q = rng.normal(size=4)
            m, s_, qq, sh = _single(mean, sc, q)
            for eps2d in (0.0, 0.3):
                p = oracle.project(m, s_, qq, sh, 0, cam, dict(eps2d=eps2d), oracle.MODE_F64)
                assert p["radii"][0] > 0
                h = 1e-6
                J = np.zeros((2, 3))
                for k in range(3):
                    e = np.zeros(3)
                    e[k] = h
                    J[:, k] = (_pinhole(cam, t + e) - _pinhole(cam, t - e)) / (2 * h)
                Sig = oracle.cov3d(q, sc)
                S2 = J @ W @ Sig @ W.T @ J.T + float(np.float32(eps2d)) * np.eye(2)
                a, b, c = p["cov2d"][0]
                np.testing.assert_allclose([a, b, c], [S2[0, 0], S2[0, 1], S2[1, 1]],
                                           rtol=2e-6, atol=2e-6 * abs(S2).max())
                A, B, Cc = p["conics"][0]
                np.testing.assert_allclose(np.array([[A, B], [B, Cc]]) @ np.array([[a, b], [b, c]]),
                                           np.eye(2), atol=1e-10)
                # the completed square's factor: L L^T is the same inverse
                l11, l21, l22 = p["chol"][0]
                L = np.array([[l11, 0.0], [l21, l22]])
                np.testing.assert_allclose(L @ L.T @ np.array([[a, b], [b, c]]), np.eye(2),
                                           atol=1e-10)
                np.testing.assert_allclose(p["means2d"][0], _pinhole(cam, t), rtol=1e-12)
                np.testing.assert_allclose(p["depths"][0], t[2], rtol=1e-12)


def test_radius_is_three_sigma_of_largest_eigenvalue():
    scene, cam = scenes.tiny_scene()
    p = oracle.project(scene.means, scene.scales, scene.quats, scene.sh, 0, cam,
                       mode=oracle.MODE_F64)
    vis = p["radii"] > 0
    assert vis.sum() > 1000
    for (a, b, c), r in zip(p["cov2d"][vis], p["radii"][vis]):
        lam = np.linalg.eigvalsh(np.array([[a, b], [b, c]]))[-1]
        assert r == int(np.ceil(3.0 * np.sqrt(lam)))


def test_f32_key_path_close_to_f64():
    scene, cam = scenes.box_scene(n=20000, width=480, height=270, fx=275.0)
    p32 = oracle.project(scene.means, scene.scales, scene.quats, scene.sh, 3, cam,
                         mode=oracle.MODE_F32KEY)
    p64 = oracle.project(scene.means, scene.scales, scene.quats, scene.sh, 3, cam,
                         mode=oracle.MODE_F64)
    both = (p32["radii"] > 0) & (p64["radii"] > 0)
    assert both.sum() > 0.8 * max((p64["radii"] > 0).sum(), 1)
    assert (p32["radii"] > 0).sum() == (p64["radii"] > 0).sum()
    np.testing.assert_allclose(p32["means2d"][both], p64["means2d"][both], rtol=1e-6, atol=1e-4)
    np.testing.assert_allclose(p32["depths"][both], p64["depths"][both], rtol=1e-6)
    np.testing.assert_allclose(p32["cov2d"][both], p64["cov2d"][both], rtol=1e-4, atol=1e-4)
    assert np.abs(p32["radii"][both] - p64["radii"][both]).max() <= 1
    # fp32 outputs really are fp32 values
    for k in ("means2d", "conics", "depths", "cov2d"):
        np.testing.assert_array_equal(p32[k], p32[k].astype(np.float32).astype(np.float64))


def brute_force_tiles(u, v, r, width, height):
    """Every tile whose pixel square [16tx, 16tx+16) x [16ty, 16ty+16)
    intersects the closed square [u-r, u+r] x [v-r, v+r], with the square's
    edges rounded to fp32 as the key path computes them."""
    f = np.float32
    lo_x, hi_x = float(f(u) - f(r)), float(f(u) + f(r))
    lo_y, hi_y = float(f(v) - f(r)), float(f(v) + f(r))
    gx, gy = (width + 15) // 16, (height + 15) // 16
    out = []
    for ty in range(gy):
        for tx in range(gx):
            if 16 * tx <= hi_x and 16 * tx + 16 > lo_x and 16 * ty <= hi_y and 16 * ty + 16 > lo_y:
                out.append(ty * gx + tx)
    return out


def test_tile_rect_brute_force():
    scene, cam = scenes.tiny_scene()
    # add a few Gaussians straddling the image border and one off-screen
    p = oracle.project(scene.means, scene.scales, scene.quats, scene.sh, 0, cam)
    gx = (cam.width + 15) // 16
    for i in range(scene.n):
        r = p["radii"][i]
        if r == 0:
            continue
        u, v = p["means2d"][i]
        bf = brute_force_tiles(u, v, r, cam.width, cam.height)
        x0, x1, y0, y1 = p["rect"][i]
        rect = [ty * gx + tx for ty in range(y0, y1) for tx in range(x0, x1)]
        assert rect == bf, i
        assert p["tiles"][i] == len(bf)


def test_culling_rules():
    cam = scenes.identity_camera(64, 64, 64.0)
    means = np.array([[0, 0, 3.0], [0, 0, -1.0], [0, 0, 0.005], [np.nan, 0, 3], [0, 0, 3],
                      [0, 0, 3], [500.0, 0, 3.0], [0, 0, 3]])
    scales = np.full((8, 3), 0.05)
    scales[4, 0] = np.inf
    quats = np.tile([1.0, 0, 0, 0], (8, 1))
    quats[5] = 0.0
    quats[7] = [2.0, 0, 0, 0]  # any non-zero norm is accepted
    p = oracle.project(means, scales, quats, np.zeros((8, 1, 3)), 0, cam)
    # in front / behind / inside near plane / NaN mean / inf scale / zero quat / off-screen / ok
    np.testing.assert_array_equal(p["radii"] > 0, [1, 0, 0, 0, 0, 0, 0, 1])
    assert np.all(p["conics"][p["radii"] == 0] == 0)
    np.testing.assert_array_equal(p["tiles"][p["radii"] == 0], 0)


def test_completed_square_factor_on_fp32_key_path():
    """In fp32, L11 = sqrt(A), L21 = B / L11, L22 = 1 / sqrt(c) reproduce the
    conic to a few roundings per entry, including needle-like splats whose
    conic is nearly singular (heavy-tailed scales)."""
    scene = scenes.heavy_tail_scene(n=20000, seed=9)
    cam = scenes.sphere_poses(1, 6.0, 51, 256, 256, scenes.focal_for(256))[0]
    p = oracle.project(scene.means, scene.scales, scene.quats, scene.sh, 3, cam)
    vis = p["radii"] > 0
    A, B, C = p["conics"][vis].T
    l11, l21, l22 = p["chol"][vis].T
    a, b, c = p["cov2d"][vis].T
    kappa = (a + c) ** 2 / (a * c - b * b)  # >= condition number of the 2D covariance
    assert kappa.max() > 1e3  # needles are present
    u = 2.0 ** -24
    assert np.all(np.abs(l11 * l11 - A) <= 4 * u * A)
    assert np.all(np.abs(l11 * l21 - B) <= 4 * u * np.abs(B))
    assert np.all(np.abs(l21 * l21 + l22 * l22 - C) <= 8 * u * C)
    np.testing.assert_array_equal(l22, (np.float32(1) / np.sqrt(c.astype(np.float32))))


def test_completed_square_evaluates_needles_stably():
    """Why the quadratic form is evaluated as a completed square: far along a
    needle the expanded A dx^2 + 2B dx dy + C dy^2 cancels terms of order 1e5
    down to q ~ 1, so its fp32 evaluation is off by ~1e-2, while the
    completed square's fp32 evaluation stays within a few 1e-5 of the value
    the same fp32 factors define."""
    f32 = np.float32
    # 2D covariance of a needle: sigma 300 px along (1,1)/sqrt2, 0.6 px across
    R = np.array([[1.0, -1.0], [1.0, 1.0]]) / np.sqrt(2.0)
    S = R @ np.diag([300.0 ** 2, 0.6 ** 2]) @ R.T
    a, b, c = f32(S[0, 0]), f32(S[0, 1]), f32(S[1, 1])
    det = f32(a * c - b * b)
    A, B, C = f32(c / det), f32(-(b / det)), f32(a / det)
    l11 = f32(np.sqrt(A))
    l21 = f32(B / l11)
    l22 = f32(1) / f32(np.sqrt(c))
    t = np.linspace(-600.0, 600.0, 41)
    dx = (t / np.sqrt(2.0) + 0.3).astype(f32)
    dy = (t / np.sqrt(2.0) - 0.2).astype(f32)
    q_ref = (float(l11) * dx.astype(float) + float(l21) * dy.astype(float)) ** 2 + \
        (float(l22) * dy.astype(float)) ** 2
    e1 = l11 * dx + l21 * dy
    e2 = l22 * dy
    q_sq = e1 * e1 + e2 * e2                                   # fp32
    q_ex = A * dx * dx + f32(2) * B * dx * dy + C * dy * dy    # fp32
    assert np.abs(q_sq - q_ref).max() < 1e-4
    assert np.abs(q_ex - (float(A) * dx.astype(float) ** 2 + 2 * float(B) * dx.astype(float) *
                          dy.astype(float) + float(C) * dy.astype(float) ** 2)).max() > 1e-3
