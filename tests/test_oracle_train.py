"""Pins of the oracle's training-step pieces: the mean-L1 + 0.2 D-SSIM image
loss of the gsplat guide (lmnt.cn/news/262699) §4.1 training loop, with the
standard SSIM index as its ssim() (Wang et al. 2004: 11 x 11 Gaussian window,
sigma 1.5, zero padding, C1 = 0.01^2, C2 = 0.03^2), and the per-group Adam
step of §4.2 with the activation chain rule."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _imgs(h, w, seed, c=3):
    rng = np.random.default_rng(seed)
    return rng.random((h, w, c)), rng.random((h, w, c))


def test_window_closed_form():
    w = oracle.ssim_window_1d()
    assert len(w) == 11
    assert abs(w.sum() - 1.0) < 1e-15
    np.testing.assert_allclose(w, w[::-1], rtol=0, atol=0)
    for k in range(1, 6):
        # Gaussian of standard deviation 1.5: w[5+k] / w[5] = exp(-k^2 / 4.5)
        assert abs(w[5 + k] / w[5] - np.exp(-k * k / 4.5)) < 1e-15


def test_window_sum_is_zero_padded_correlation():
    from scipy import ndimage
    rng = np.random.default_rng(3)
    plane = rng.random((23, 31))
    w = oracle.ssim_window_1d()
    ref = ndimage.correlate(plane, np.outer(w, w), mode="constant", cval=0.0)
    np.testing.assert_allclose(oracle.window_sum(plane), ref, rtol=0, atol=1e-14)
    # smaller than the window in one direction
    plane = rng.random((4, 19))
    ref = ndimage.correlate(plane, np.outer(w, w), mode="constant", cval=0.0)
    np.testing.assert_allclose(oracle.window_sum(plane), ref, rtol=0, atol=1e-14)


def test_identical_images():
    x, _ = _imgs(17, 13, 4)
    np.testing.assert_allclose(oracle.ssim_map(x, x), 1.0, rtol=0, atol=1e-12)
    loss, g, _ = oracle.l1_dssim_loss_grad(x, x)
    assert abs(loss) < 1e-12
    # x = y maximises the index (s <= 1), and sign(0) = 0
    assert np.abs(g).max() < 1e-15


def test_constant_images_interior():
    a, b = 0.3, 0.8
    x = np.full((30, 30, 3), a)
    y = np.full((30, 30, 3), b)
    s = oracle.ssim_map(x, y)
    want = (2 * a * b + oracle.SSIM_C1) / (a * a + b * b + oracle.SSIM_C1)
    # a full window inside: zero variance and covariance
    np.testing.assert_allclose(s[5:25, 5:25], want, rtol=1e-12)


def test_map_equals_direct_centred_definition():
    x, y = _imgs(9, 12, 5)
    H, W, C = x.shape
    w = oracle.ssim_window_1d()
    w2 = np.outer(w, w)
    s = oracle.ssim_map(x, y)
    for c in range(C):
        for py in range(H):
            for px in range(W):
                xs = np.zeros((11, 11))
                ys = np.zeros((11, 11))
                for a in range(11):
                    for b in range(11):
                        qy, qx = py + a - 5, px + b - 5
                        if 0 <= qy < H and 0 <= qx < W:
                            xs[a, b] = x[qy, qx, c]
                            ys[a, b] = y[qy, qx, c]
                mx, my = (w2 * xs).sum(), (w2 * ys).sum()
                # centred second moments over the whole window (zeros outside)
                vx = (w2 * (xs - mx) ** 2).sum()
                vy = (w2 * (ys - my) ** 2).sum()
                cxy = (w2 * (xs - mx) * (ys - my)).sum()
                want = ((2 * mx * my + oracle.SSIM_C1) * (2 * cxy + oracle.SSIM_C2) /
                        ((mx * mx + my * my + oracle.SSIM_C1) * (vx + vy + oracle.SSIM_C2)))
                assert abs(s[py, px, c] - want) < 1e-12


def test_loss_value_parts():
    x, y = _imgs(14, 11, 6)
    loss, _, parts = oracle.l1_dssim_loss_grad(x, y, lam=0.2)
    l1 = np.abs(x - y).mean()
    assert abs(loss - (l1 + 0.2 * (1.0 - oracle.ssim_map(x, y).mean()))) < 1e-14
    loss0, _, _ = oracle.l1_dssim_loss_grad(x, y, lam=0.0)
    assert abs(loss0 - l1) < 1e-15


@pytest.mark.parametrize("lam", [0.2, 1.0])
def test_gradient_finite_differences(lam):
    x, y = _imgs(14, 11, 7)
    _, g, _ = oracle.l1_dssim_loss_grad(x, y, lam)
    rng = np.random.default_rng(8)
    H, W, C = x.shape
    picks = [(0, 0, 0), (H - 1, W - 1, 2), (0, W - 1, 1), (H - 1, 0, 0), (7, 5, 1)]
    picks += [tuple(int(v) for v in (rng.integers(H), rng.integers(W), rng.integers(C)))
              for _ in range(60)]
    h = 1e-6
    for (py, px, c) in picks:
        xp, xm = x.copy(), x.copy()
        xp[py, px, c] += h
        xm[py, px, c] -= h
        fd = (oracle.l1_dssim_loss_grad(xp, y, lam)[0] -
              oracle.l1_dssim_loss_grad(xm, y, lam)[0]) / (2 * h)
        assert abs(fd - g[py, px, c]) < 1e-8, (py, px, c, fd, g[py, px, c])


def test_error_scale_bounds_perturbed_statistics():
    """The fp32 error bound covers the gradient computed from statistics that
    carry relative errors up to delta (first order; planted on the CPU)."""
    x, y = _imgs(16, 19, 9)
    lam = 0.2
    delta = 32.0 * 2.0 ** -24
    _, g, parts = oracle.l1_dssim_loss_grad(x, y, lam)
    e = oracle.l1_dssim_errscale(x, y, lam, parts, delta)
    rng = np.random.default_rng(10)
    n = x.size
    for _ in range(4):
        st = [s * (1.0 + delta * rng.uniform(-1, 1, s.shape)) for s in parts["stats"]]
        _, d_mu, d_xx, d_xy = oracle.ssim_pointwise(*st)
        b = [oracle._channels(oracle.window_sum, d) for d in (d_mu, d_xx, d_xy)]
        gp = np.sign(x - y) / n - lam / n * (b[0] + 2 * x * b[1] + y * b[2])
        assert np.all(np.abs(gp - g) <= e)
    assert np.all(e >= 0) and e.max() < 1e-2 * np.abs(g).max()


# ------------------------------------------------------------------ Adam
def _params(N, K, seed):
    rng = np.random.default_rng(seed)
    raw = dict(means=rng.normal(size=(N, 3)), log_scales=rng.normal(-4, 0.5, (N, 3)),
               quats=rng.normal(size=(N, 4)), logits=rng.normal(size=N),
               sh=rng.normal(0, 0.2, (N, K, 3)))
    act = dict(scales=np.exp(raw["log_scales"]), opacities=1 / (1 + np.exp(-raw["logits"])))
    return raw, act


def test_adam_matches_torch_adam():
    rng = np.random.default_rng(11)
    for lr in (1.6e-4, 5e-2):
        p0 = rng.normal(size=(50, 3))
        tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
        opt = torch.optim.Adam([tp], lr=lr, betas=oracle.ADAM_BETAS, eps=oracle.ADAM_EPS)
        p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
        for step in range(1, 5):
            g = rng.normal(size=p0.shape) * 10.0 ** rng.integers(-6, 1)
            tp.grad = torch.tensor(g)
            opt.step()
            p, m, v = oracle.adam_update(p, g, m, v, step, lr)
            np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(m, opt.state[tp]["exp_avg"].numpy(), rtol=1e-13)
            np.testing.assert_allclose(v, opt.state[tp]["exp_avg_sq"].numpy(), rtol=1e-13)


def test_adam_first_step_moves_by_lr_times_sign():
    rng = np.random.default_rng(12)
    p0 = rng.normal(size=100)
    g = rng.normal(size=100)
    p, m, v = oracle.adam_update(p0, g, 0 * p0, 0 * p0, 1, 1e-3)
    # bias-corrected first moments are g and g^2
    np.testing.assert_allclose(p, p0 - 1e-3 * np.sign(g), rtol=0, atol=1e-15)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.01 * g * g, rtol=1e-14)


def test_packed_step_matches_torch_sparse_adam():
    """Packed rows: only the listed rows move (torch's SparseAdam). It places
    eps after the bias correction of v, a relative difference of order
    eps / sqrt(v_hat) = 1e-15 / 1e-4 here."""
    rng = np.random.default_rng(13)
    N = 40
    p0 = rng.normal(size=(N, 3))
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.SparseAdam([tp], lr=5e-3, betas=oracle.ADAM_BETAS, eps=oracle.ADAM_EPS)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for step in range(1, 5):
        rows = np.sort(rng.choice(N, size=15, replace=False))
        g = rng.normal(size=(15, 3)) * 1e-2
        tp.grad = torch.sparse_coo_tensor(torch.tensor(rows)[None, :], torch.tensor(g), (N, 3))
        opt.step()
        p[rows], m[rows], v[rows] = oracle.adam_update(p[rows], g, m[rows], v[rows], step, 5e-3)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-10, atol=1e-14)


def test_raw_gradients_by_finite_differences():
    raw, act = _params(20, 4, 14)
    rng = np.random.default_rng(15)
    cs, co = rng.normal(size=(20, 3)), rng.normal(size=20)
    # L = sum cs * s + sum co * o^2 with s = exp(log_s), o = sigmoid(logit)
    grads = dict(means=np.zeros((20, 3)), scales=cs, quats=np.zeros((20, 4)),
                 opacities=2 * co * act["opacities"], sh=np.zeros((20, 4, 3)))
    gr = oracle.raw_grads(grads, act, np.arange(20))
    h = 1e-6
    L = lambda ls, lg: (cs * np.exp(ls)).sum() + (co * (1 / (1 + np.exp(-lg))) ** 2).sum()
    for i in range(20):
        for k in range(3):
            a, b = raw["log_scales"].copy(), raw["log_scales"].copy()
            a[i, k] += h
            b[i, k] -= h
            fd = (L(a, raw["logits"]) - L(b, raw["logits"])) / (2 * h)
            assert abs(fd - gr["log_scales"][i, k]) < 1e-8
        a, b = raw["logits"].copy(), raw["logits"].copy()
        a[i] += h
        b[i] -= h
        fd = (L(raw["log_scales"], a) - L(raw["log_scales"], b)) / (2 * h)
        assert abs(fd - gr["logits"][i]) < 1e-8


def test_train_step_groups_and_packed_rows():
    N, K = 30, 4
    raw, act = _params(N, K, 16)
    rng = np.random.default_rng(17)
    zeros = {k: np.zeros_like(v) for k, v in raw.items()}
    rows = np.array([1, 4, 5, 17, 29])
    grads = dict(means=rng.normal(size=(5, 3)), scales=rng.normal(size=(5, 3)),
                 quats=rng.normal(size=(5, 4)), opacities=rng.normal(size=5),
                 sh=rng.normal(size=(5, K, 3)))
    r2, a2, m2, v2 = oracle.adam_train_step(raw, act, grads, zeros, zeros, 1, rows=rows)
    off = np.setdiff1d(np.arange(N), rows)
    for k in raw:
        np.testing.assert_array_equal(r2[k][off], raw[k][off])
        assert np.all(m2[k][off] == 0) and np.all(v2[k][off] == 0)
    # first step: each group moves by its learning rate
    gr = oracle.raw_grads(grads, act, rows)
    for k, grp in (("means", "means"), ("log_scales", "scales"), ("quats", "quats"),
                   ("logits", "opacities"), ("sh", "sh")):
        np.testing.assert_allclose(r2[k][rows], raw[k][rows] - oracle.ADAM_LR[grp] *
                                   np.sign(gr[k]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(a2["scales"][rows], np.exp(r2["log_scales"][rows]), rtol=1e-15)
    np.testing.assert_array_equal(a2["scales"][off], act["scales"][off])
