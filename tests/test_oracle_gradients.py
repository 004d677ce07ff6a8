"""Pins of the oracle's analytic backward (step 13).

(i) Dual-number directional derivatives: for random directions v over every
parameter, <grad L, v> from the analytic backward must equal dL(x + e v)/de
computed exactly by forward-mode dual numbers through the whole fp64 forward.
(ii) Central finite differences on individual parameters (every parameter
kind, on the 1,024-Gaussian SH0 scene and a 100-Gaussian SH3 scene), with
steps that cross a discrete decision (visibility, tile sets, skipped or
stopped pairs, clamps) detected by the forward's decision signature and
excluded; the count of excluded steps is asserted to be small.
"""
import numpy as np
import pytest

import oracle
from differentiable_rasterization_amd import scenes

PARAMS = ("means", "scales", "quats", "opacities", "sh")


def _as64(scene):
    return {k: getattr(scene, k).astype(np.float64) for k in PARAMS}


def _analytic(scene, cam, target, loss_kind, bg):
    f = oracle.render_f64(scene, cam, None, bg)
    g_img = oracle.loss_grad_image(f["raster"]["image"], target, loss_kind)
    g = oracle.backward(scene, cam, f, g_img, None, bg)
    return dict(means=g["g3"]["means"], scales=g["g3"]["scales"], quats=g["g3"]["quats"],
                opacities=g["g2"]["opacities"], sh=g["g3"]["sh"]), f


def _scene64(scene):
    p = _as64(scene)
    return scenes.Scene(p["means"], p["scales"], p["quats"], p["opacities"], p["sh"],
                        scene.sh_degree)


def coverage_scene():
    """100 SH3 Gaussians that exercise every branch of the backward: culled
    ones (behind the camera, far off-screen), ones beyond the field-of-view
    clamp of the Jacobian whose footprint still reaches the image, pairs whose
    alpha is clamped at alpha_max, colours clamped at zero, and quaternions of
    non-unit norm."""
    s, cam = scenes.box_scene(n=100, seed=7, width=96, height=64, fx=40.0)
    rng = np.random.default_rng(8)
    s.quats *= rng.uniform(0.5, 2.0, size=(100, 1)).astype(np.float32)
    # camera: R = I, t = (0,0,8), so world = camera - (0,0,8)
    s.means[:3] = [[0, 0, -9.0], [0, 0, -8.5], [60.0, 0, 0]]
    s.means[3] = [1.8 * 5.0, 0.2, 5.0 - 8.0]
    s.means[4] = [-1.9 * 5.0, -1.0, 5.0 - 8.0]
    s.means[5] = [0.3, 2.2 * 4.0, 4.0 - 8.0]
    s.scales[3:6] = 1.5
    s.opacities[6:12] = 0.9999
    s.scales[6:12] = 0.4
    s.sh[12:20, 0, :] = -1.2  # dark DC: the clamp at zero engages for some views
    return s, cam


def _cases():
    s1, c1 = scenes.tiny_scene()
    s2, c2 = coverage_scene()
    return [(s1, c1, oracle.LOSS_L2), (s2, c2, oracle.LOSS_L2), (s2, c2, oracle.LOSS_L1)]


def test_coverage_scene_exercises_every_branch():
    s, cam = coverage_scene()
    s = _scene64(s)
    f = oracle.render_f64(s, cam)
    p = f["proj"]
    assert np.sum(p["radii"][:3] == 0) == 3
    W = cam.width
    lim = 1.3 * (0.5 * W / cam.fx)
    for i in (3, 4):  # beyond the fov clamp yet visible
        assert p["radii"][i] > 0
        assert abs(p["means2d"][i][0] - cam.cx) / cam.fx > lim
    assert p["radii"][5] > 0 and abs(p["means2d"][5][1] - cam.cy) / cam.fy > 1.3 * (0.5 * cam.height / cam.fy)
    assert p["clamped"][p["radii"] > 0].sum() > 0
    # some pixel of the clamped-opacity Gaussians has o * G > alpha_max
    img = f["raster"]
    m = oracle.composite(cam.width, cam.height, f["bins"]["ranges"], f["bins"]["ids"], p["means2d"],
                         p["chol"], s.opacities, p["colors"], p["depths"], with_margin=True)
    assert np.any(img["last"] > 0)
    hits = 0
    for i in range(6, 12):
        if p["radii"][i] == 0:
            continue
        u, v = p["means2d"][i]
        A, B, C = p["conics"][i]
        for py in range(cam.height):
            for px in range(cam.width):
                dx, dy = px + 0.5 - u, py + 0.5 - v
                if 0.9999 * np.exp(-0.5 * (A * dx * dx + 2 * B * dx * dy + C * dy * dy)) > 0.99:
                    hits += 1
    assert hits > 0
    assert np.all(np.abs(np.linalg.norm(s.quats, axis=1) - 1) > 1e-3)


@pytest.mark.parametrize("case", [0, 1, 2])
def test_jvp_matches_analytic_gradient(case):
    scene, cam, loss_kind = _cases()[case]
    scene = _scene64(scene)
    target = scenes.target_image(cam, 1).astype(np.float64)
    bg = (0.1, 0.2, 0.3)
    grad, f = _analytic(scene, cam, target, loss_kind, bg)
    culled = f["proj"]["radii"] == 0
    for k in ("means", "scales", "quats", "sh"):
        assert np.all(grad[k][culled] == 0)
    rng = np.random.default_rng(100 + case)
    for trial in range(3):
        v = {k: rng.normal(size=getattr(scene, k).shape) for k in PARAMS}
        L, dL, sig, M = oracle.loss_jvp(scene.means, scene.scales, scene.quats, scene.opacities,
                                        scene.sh, scene.sh_degree, cam, target, loss_kind, bg,
                                        direction=v)
        ip = sum(float(np.sum(grad[k] * v[k])) for k in PARAMS)
        assert M == f["bins"]["M"]
        np.testing.assert_allclose(ip, dL, rtol=1e-9)
        # each parameter group on its own, so one group cannot mask another
        for k in PARAMS:
            vk = {k: v[k]}
            _, dLk, _, _ = oracle.loss_jvp(scene.means, scene.scales, scene.quats,
                                           scene.opacities, scene.sh, scene.sh_degree, cam,
                                           target, loss_kind, bg, direction=vk)
            ipk = float(np.sum(grad[k] * v[k]))
            np.testing.assert_allclose(ipk, dLk, rtol=1e-8, atol=1e-10 * abs(dL), err_msg=k)


def _image(scene, cam, target, loss_kind, bg):
    _, _, sig, _, img = oracle.loss_jvp(scene.means, scene.scales, scene.quats, scene.opacities,
                                        scene.sh, scene.sh_degree, cam, target, loss_kind, bg,
                                        return_image=True)
    return img, sig


def _pixel_loss(img, target, loss_kind):
    r = img - target
    return r * r if loss_kind == oracle.LOSS_L2 else np.abs(r)


@pytest.mark.parametrize("case", [0, 1])
def test_central_finite_differences(case):
    scene, cam, loss_kind = _cases()[case]
    scene = _scene64(scene)
    target = scenes.target_image(cam, 1).astype(np.float64)
    bg = (0.1, 0.2, 0.3)
    grad, f = _analytic(scene, cam, target, loss_kind, bg)
    _, sig0 = _image(scene, cam, target, loss_kind, bg)
    rng = np.random.default_rng(7 + case)
    vis = np.nonzero(f["proj"]["radii"] > 0)[0]
    picks = rng.choice(vis, size=min(len(vis), 24), replace=False)
    checked = flipped = 0
    worst = 0.0
    for i in picks:
        for k in PARAMS:
            arr = getattr(scene, k)
            for idx in np.ndindex(arr.shape[1:]):
                full = (i,) + idx
                x = arr[full]
                h = 1e-6 * max(1.0, abs(x))
                arr[full] = x + h
                Ip, sp = _image(scene, cam, target, loss_kind, bg)
                arr[full] = x - h
                Im, sm = _image(scene, cam, target, loss_kind, bg)
                arr[full] = x
                if sp != sig0 or sm != sig0:
                    flipped += 1
                    continue
                # difference taken per pixel before summing: pixels the step
                # does not reach cancel exactly, so no large-sum rounding floor
                dpix = _pixel_loss(Ip, target, loss_kind) - _pixel_loss(Im, target, loss_kind)
                fd = float(np.sum(dpix)) / (2 * h)
                g = grad[k][full]
                # FD truncation O(h^2) and per-pixel rounding ~1e-16/h per touched pixel
                tol = 2e-6 * abs(g) + 1e-8 * np.count_nonzero(dpix) ** 0.5 + 1e-9
                err = abs(fd - g)
                worst = max(worst, err / tol)
                assert err <= tol, (k, full, fd, g)
                checked += 1
    print("FD worst err/tol %.3g, checked %d, flipped %d" % (worst, checked, flipped))
    assert checked > 300
    assert flipped <= 0.05 * (checked + flipped)


def needle_scene(n=12_000, seed=11):
    """Gaussians in front of an identity camera (1920x1080, fx = 1100): a
    third of them needles (one axis e^-2.5..1, the other two e^-9..e^-6), the
    rest log-scales N(-3, 0.5), random rotations, SH3, plus random 2D
    gradients with magnitudes spread over four decades."""
    rng = np.random.default_rng(seed)
    z = rng.uniform(2.0, 8.0, n)
    means = np.stack([rng.uniform(-0.8, 0.8, n) * z, rng.uniform(-0.45, 0.45, n) * z, z], 1)
    logs = rng.normal(-3.0, 0.5, (n, 3))
    nd = rng.random(n) < 0.35
    logs[nd, 0] = rng.uniform(-2.5, 0.0, nd.sum())
    logs[nd, 1:] = rng.uniform(-9.0, -6.0, (nd.sum(), 2))
    q = rng.normal(size=(n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    sh = rng.normal(0.0, 0.2, (n, 16, 3))
    sh[:, 0, :] = (rng.random((n, 3)) - 0.5) / scenes.Y00
    f = lambda a: np.asarray(a, np.float32).astype(np.float64)
    scene = scenes.Scene(f(means), f(np.exp(logs)), f(q), f(rng.uniform(0.1, 1.0, n)), f(sh), 3)
    cam = scenes.identity_camera(1920, 1080, 1100.0)
    g2 = (rng.normal(size=(n, 2)), rng.normal(size=(n, 3)) * 10.0 ** rng.uniform(-2, 2, (n, 1)),
          rng.normal(size=(n, 3)))
    return scene, cam, g2


def _kappa(proj):
    a, b, c = proj["cov2d"].T
    half_tr = 0.5 * (a + c)
    lmax = half_tr + np.sqrt(np.maximum(half_tr * half_tr - (a * c - b * b), 0.0))
    return lmax / ((a * c - b * b) / lmax)


def _pbwd(scene, cam, radii, g2):
    return oracle.project_bwd(scene.means, scene.scales, scene.quats, scene.sh, 3, cam, radii,
                              *g2)


def _flat(d, n):
    return np.concatenate([d[k].reshape(n, -1) for k in ("means", "scales", "quats", "sh")], 1)


def test_projection_backward_is_linear_in_its_2d_gradients():
    """The bound below rests on linearity: with the discrete decisions fixed by
    the parameters, f(a x + b y) = a f(x) + b f(y)."""
    scene, cam, g2 = needle_scene()
    radii = oracle.project(scene.means, scene.scales, scene.quats, scene.sh, 3, cam)["radii"]
    assert (radii > 0).mean() > 0.99
    rng = np.random.default_rng(5)
    y = tuple(rng.normal(size=x.shape) for x in g2)
    a, b = 0.75, -2.5
    n = scene.n
    fx, fy = _flat(_pbwd(scene, cam, radii, g2), n), _flat(_pbwd(scene, cam, radii, y), n)
    fxy = _flat(_pbwd(scene, cam, radii, tuple(a * u + b * v for u, v in zip(g2, y))), n)
    scale = np.abs(a * fx) + np.abs(b * fy)
    # fp64 rounding of the chain, relative to the Gaussian's largest output
    tol = 1e-9 * scale.max(axis=1, keepdims=True) + 1e-300
    assert np.all(np.abs(fxy - (a * fx + b * fy)) <= tol)


def test_projection_bound_is_sound_under_input_perturbations():
    """12,000 Gaussians (needles up to a 2D condition number above 1e5): for
    random perturbations d of the 2D gradients on the corners of the box
    |d_k| <= s_k, every output moves by at most the bound e."""
    scene, cam, g2 = needle_scene()
    proj = oracle.project(scene.means, scene.scales, scene.quats, scene.sh, 3, cam)
    radii, kappa = proj["radii"], _kappa(proj)
    vis = radii > 0
    assert kappa[vis].max() > 1e5 and (kappa[vis] > 1e4).sum() > 500
    rng = np.random.default_rng(6)
    s = tuple(np.abs(x) * 10.0 ** rng.uniform(-3, 0, x.shape) for x in g2)
    n = scene.n
    e = _flat(oracle.project_bwd_bound(scene.means, scene.scales, scene.quats, scene.sh, 3, cam,
                                       radii, *s), n)
    f0 = _flat(_pbwd(scene, cam, radii, g2), n)
    worst = 0.0
    for trial in range(6):
        d = tuple(si * rng.choice([-1.0, 1.0], si.shape) for si in s)
        f1 = _flat(_pbwd(scene, cam, radii, tuple(x + di for x, di in zip(g2, d))), n)
        slack = 1e-9 * np.maximum(np.abs(f0), np.abs(f1)).max(axis=1, keepdims=True)
        moved = np.abs(f1 - f0)
        assert np.all(moved <= e * (1 + 1e-9) + slack), trial
        worst = max(worst, float((moved[vis] / np.maximum(e[vis], 1e-300)).max()))
    # random corners come close to the worst case somewhere
    assert worst > 0.99, worst


def test_projection_bound_equals_the_worst_corner_by_brute_force():
    """On 1,500 Gaussians (a third needles) the bound equals, output by
    output, the largest |f(d)| over all 256 corners d = (+-s_0, ..., +-s_7)
    of the input box, found by evaluating every corner: a dropped Jacobian
    term, a wrong factor or a wrong sign rule would change it."""
    scene, cam, g2 = needle_scene(n=1500, seed=12)
    radii = oracle.project(scene.means, scene.scales, scene.quats, scene.sh, 3, cam)["radii"]
    rng = np.random.default_rng(9)
    s = tuple(np.abs(x) * 10.0 ** rng.uniform(-3, 0, x.shape) for x in g2)
    s[1][::7, 1] = 0.0  # an input known exactly contributes nothing
    n = scene.n
    e = _flat(oracle.project_bwd_bound(scene.means, scene.scales, scene.quats, scene.sh, 3, cam,
                                       radii, *s), n)
    best = np.zeros_like(e)
    cols = np.concatenate(s, 1)
    for corner in range(256):
        signs = np.array([1.0 if (corner >> k) & 1 else -1.0 for k in range(8)])
        d = cols * signs
        f = _flat(_pbwd(scene, cam, radii, (d[:, 0:2], d[:, 2:5], d[:, 5:8])), n)
        best = np.maximum(best, np.abs(f))
    scale = e.max(axis=1, keepdims=True)
    assert np.all(np.abs(best - e) <= 1e-9 * scale + 1e-300)
    assert np.all(e[radii <= 0] == 0)
