"""Edge cases of the HIP path through the C ABI, checked against the oracle
or against properties that hold exactly."""
import numpy as np
import pytest

import oracle
from differentiable_rasterization_amd import scenes

from parity_util import PIX_TOL, assert_bits_equal, gpu_frame, grad2d_rows

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def test_counting_variant_matches_and_counts_consistently():
    """The counting kernels produce the same outputs; the backward's gradient
    pairs are exactly the forward's blended pairs; evaluated pairs bound them."""
    torch = _torch()
    from differentiable_rasterization_amd import raster
    scene, cam = scenes.box_scene(n=20000, seed=12, width=500, height=270, fx=290.0)
    out = gpu_frame(scene, cam, loss_kind="l2", target=scenes.target_image(cam, 7))
    fr, g = out["frame"], raster.Gaussians.from_scene(scene)
    cnt = torch.zeros(8, dtype=torch.int64, device="cuda")
    img, fT, last = fr.image.clone(), fr.final_T.clone(), fr.last_idx.clone()
    rec = grad2d_rows(fr, g.N).clone()
    fr.rasterize(g, counters=cnt[0:4])
    fr.rasterize_backward(g, counters=cnt[4:8])
    torch.cuda.synchronize()
    assert torch.equal(img, fr.image) and torch.equal(fT, fr.final_T)
    assert torch.equal(last, fr.last_idx)
    # the backward sums in a fixed order: identical bits
    assert torch.equal(rec, grad2d_rows(fr, g.N))
    c = cnt.cpu().numpy()
    print("counters fwd", c[:4], "bwd", c[4:])
    assert c[5] == c[1] > 0            # gradient pairs == blended pairs
    assert c[1] <= c[0] and c[1] <= c[2]
    assert c[0] <= out["M"] * 256       # culling never adds work
    assert c[7] > 0
    # the plain tile loops: per-pixel work <= the tile loop's <= every entry
    assert c[2] <= c[3] <= out["M"] * 256
    assert c[4] <= c[6] <= c[3]


@pytest.mark.parametrize("packed", [False, True])
def test_zero_gaussians_and_all_culled(packed):
    torch = _torch()
    cam = scenes.identity_camera(40, 24, 30.0)
    bg = (0.25, 0.5, 0.75)
    empty = scenes.Scene(np.zeros((0, 3), np.float32), np.zeros((0, 3), np.float32),
                         np.zeros((0, 4), np.float32), np.zeros(0, np.float32),
                         np.zeros((0, 1, 3), np.float32), 0)
    behind, _ = scenes.tiny_scene(n=50)
    behind.means[:, 2] = -behind.means[:, 2]
    for sc in (empty, behind):
        out = gpu_frame(sc, cam, background=bg, loss_kind="l2",
                        target=scenes.target_image(cam, 1), packed=packed)
        assert out["M"] == 0
        if packed:
            assert out["V"] == 0
        np.testing.assert_array_equal(out["image"], np.broadcast_to(np.float32(bg), (24, 40, 3)))
        assert np.all(out["final_T"] == 1.0) and np.all(out["last"] == 0)
        assert np.all(out["ranges"] == 0)
        for k in ("g_means", "g_scales", "g_quats", "g_sh", "g_opacities"):
            assert np.all(out[k] == 0), k


def test_capacity_retry_and_leading_dimension():
    scene, cam = scenes.tiny_scene()
    ref = gpu_frame(scene, cam, loss_kind="l2", target=scenes.target_image(cam, 2))
    small = gpu_frame(scene, cam, loss_kind="l2", target=scenes.target_image(cam, 2), capacity=16)
    assert small["frame"].capacity >= small["M"] == ref["M"]
    for k in ("keys", "ids", "ranges", "image", "final_T", "last"):
        assert_bits_equal(small[k], ref[k], k)
    wide = gpu_frame(scene, cam, loss_kind="l2", target=scenes.target_image(cam, 2),
                     ld=scene.n + 37)
    for k in ("means2d", "conics", "depths", "radii", "tiles", "keys", "ids", "ranges", "image",
              "final_T", "last"):
        assert_bits_equal(wide[k], ref[k], k)
    # gradients are summed in a fixed order, independent of ld and capacity
    for k in ("g_means", "g_scales", "g_quats", "g_sh", "g_opacities"):
        assert_bits_equal(wide[k], ref[k], k)
        assert_bits_equal(small[k], ref[k], k)


@pytest.mark.parametrize("packed", [False, True])
def test_accumulate_adds_into_outputs(packed):
    """A second backward with accumulate on top of the first doubles the
    gradients with respect to the Gaussians (x + x == 2x in fp32); packed:
    the rows of the visible list."""
    torch = _torch()
    from differentiable_rasterization_amd import raster
    scene, cam = scenes.tiny_scene()
    out = gpu_frame(scene, cam, loss_kind="l2", target=scenes.target_image(cam, 3),
                    packed=packed)
    fr, g = out["frame"], raster.Gaussians.from_scene(scene)
    R = fr.V if packed else scene.n
    assert R > 0
    rows = lambda t: t[..., :R].cpu().numpy().copy()
    names = ("g_opacities", "g_means", "g_scales", "g_quats", "g_sh")
    first = {k: rows(getattr(fr, k)) for k in names}
    fr.backward(g, accumulate=1)  # second pass on top of the first
    torch.cuda.synchronize()
    for k in names:
        assert_bits_equal(rows(getattr(fr, k)), 2 * first[k], k)


def test_non_finite_and_degenerate_gaussians_are_culled():
    scene, cam = scenes.tiny_scene(n=200)
    scene.means[0, 0] = np.nan
    scene.scales[1, 1] = np.inf
    scene.quats[2] = 0.0
    scene.quats[3, 0] = np.nan
    scene.scales[4] = 0.0           # a point: dilation keeps it visible
    scene.opacities[5] = 0.0        # invisible but projected
    out = gpu_frame(scene, cam, loss_kind="l2", target=scenes.target_image(cam, 4))
    o = oracle.render(scene, cam)
    assert_bits_equal(out["radii"], o["proj"]["radii"], "radii")
    assert np.all(out["radii"][:4] == 0)
    for k in ("image", "final_T", "g_means", "g_scales", "g_quats", "g_sh", "g_opacities"):
        assert np.all(np.isfinite(out[k])), k
    assert np.abs(out["image"] - o["raster"]["image"]).max() <= PIX_TOL


def test_depth_and_alpha_outputs():
    scene, cam = scenes.box_scene(n=5000, seed=3, width=200, height=120, fx=110.0)
    out = gpu_frame(scene, cam, backward=False, depth_alpha=True)
    o = oracle.render(scene, cam, with_margin=True)
    r = o["raster"]
    ok = r["margin"] >= 2e-4
    np.testing.assert_allclose(out["alpha"], 1 - out["final_T"], rtol=0, atol=0)
    np.testing.assert_allclose(out["alpha"][ok], r["alpha"][ok], atol=PIX_TOL)
    # depth accumulates alpha T z with z of a few units
    np.testing.assert_allclose(out["depth"][ok], r["depth"][ok], atol=1e-4 * 12)


def test_whole_path_is_deterministic():
    scene, cam = scenes.box_scene(n=20000, seed=5, width=320, height=200, fx=180.0)
    a = gpu_frame(scene, cam, loss_kind="l2", target=scenes.target_image(cam, 6))
    b = gpu_frame(scene, cam, loss_kind="l2", target=scenes.target_image(cam, 6))
    for k in ("means2d", "conics", "colors", "keys", "ids", "ranges", "image", "final_T", "last",
              "g_means2d", "g_conics", "g_colors", "g_means", "g_scales", "g_quats", "g_sh",
              "g_opacities"):
        assert_bits_equal(a[k], b[k], k)


def test_exact_depth_ties_keep_index_order():
    """Clones share keys exactly; the stable sort keeps ascending index, as the
    oracle's stable sort does."""
    base, cam = scenes.tiny_scene(n=300, seed=9)
    idx = np.concatenate([np.arange(300), np.arange(0, 300, 3), np.arange(0, 300, 7)])
    scene = base.subset(idx)
    out = gpu_frame(scene, cam, loss_kind="l2", target=scenes.target_image(cam, 5))
    o = oracle.render(scene, cam)
    assert_bits_equal(out["keys"], o["bins"]["keys"], "keys")
    assert_bits_equal(out["ids"], o["bins"]["ids"], "ids")
    assert np.abs(out["image"] - o["raster"]["image"]).max() <= PIX_TOL


@pytest.mark.parametrize("n", [6000, 40000])
def test_long_tile_lists_keep_the_stable_order(n):
    """Thousands of instances per tile (the 64 x 64 image has 16 tiles): lists
    of about 900 and 6,000 entries, with exact depth ties from clones of
    every fifth Gaussian.  Keys, ids and ranges must equal the oracle's
    stable sort bit for bit."""
    base, cam = scenes.tiny_scene(n=n, seed=13)
    idx = np.concatenate([np.arange(n), np.arange(0, n, 5)])
    scene = base.subset(idx)
    out = gpu_frame(scene, cam, backward=False)
    o = oracle.render(scene, cam)
    lens = np.diff(o["bins"]["ranges"].reshape(-1, 2), axis=1)
    print("[edges] n=%d: M=%d, longest tile list %d" % (len(idx), out["M"], lens.max()),
          flush=True)
    assert lens.max() > (4096 if n > 10000 else 512)
    assert out["M"] == len(o["bins"]["keys"])
    assert_bits_equal(out["keys"], o["bins"]["keys"], "keys")
    assert_bits_equal(out["ids"], o["bins"]["ids"], "ids")
    assert_bits_equal(out["ranges"], o["bins"]["ranges"], "ranges")
    assert np.abs(out["image"] - o["raster"]["image"]).max() <= PIX_TOL


@pytest.mark.parametrize("kind", [0, 1])
def test_fused_loss_equals_separate_call(kind):
    """gs_rasterize_fwd_loss: the image and dL/dimage equal gs_rasterize_fwd
    followed by gs_image_loss_grad bit for bit; the loss value is the sum
    within fp32 rounding (its summation order is not fixed)."""
    torch = _torch()
    from differentiable_rasterization_amd import raster
    for scene, cam in ((scenes.cluster_scene(n=200_000, seed=13),
                        scenes.sphere_poses(1, 6.0, 31, 640, 416, scenes.focal_for(640))[0]),
                       scenes.box_scene(n=20000, seed=12, width=500, height=270, fx=290.0)):
        g = raster.Gaussians.from_scene(scene)
        tgt = torch.from_numpy(scenes.target_image(cam, 3)).cuda()
        a = raster.Frame(g.ld, scene.sh_degree, cam.width, cam.height)
        b = raster.Frame(g.ld, scene.sh_degree, cam.width, cam.height)
        for fr in (a, b):
            fr.project(g, cam)
            fr.bin_and_sort(g)
        a.rasterize(g)
        a.loss_grad(tgt, kind)
        b.dL_dimage.fill_(float("nan"))
        b.rasterize_loss(g, tgt, kind, with_loss=True)
        torch.cuda.synchronize()
        assert_bits_equal(b.image.cpu().numpy(), a.image.cpu().numpy(), "image")
        assert_bits_equal(b.dL_dimage.cpu().numpy(), a.dL_dimage.cpu().numpy(), "dL/dimage")
        r = a.image.cpu().numpy().astype(np.float64) - tgt.cpu().numpy()
        want = np.sum(r * r) if kind == 0 else np.sum(np.abs(r))
        assert abs(float(b.loss.item()) - want) <= 1e-5 * want


def test_loss_value_and_gradient():
    torch = _torch()
    from differentiable_rasterization_amd import raster
    rng = np.random.default_rng(0)
    n = 1_000_003
    img = rng.uniform(size=n).astype(np.float32)
    tgt = rng.uniform(size=n).astype(np.float32)
    tgt[:100] = img[:100]  # exact ties: sign(0) = 0
    ti, tt = torch.from_numpy(img).cuda(), torch.from_numpy(tgt).cuda()
    g = torch.empty_like(ti)
    loss = torch.zeros(1, device="cuda")
    for m in (1, 3, 5):  # shorter than one float4: element-wise tail only
        gs_ = torch.empty(m, device="cuda")
        raster.gs_image_loss_grad(0, m, ti, tt, gs_, loss)
        torch.cuda.synchronize()
        np.testing.assert_allclose(gs_.cpu().numpy(), 2 * (img[:m].astype(np.float64) - tgt[:m]),
                                   rtol=1e-6)
    for kind in (0, 1):
        raster.gs_image_loss_grad(kind, n, ti, tt, g, loss)
        torch.cuda.synchronize()
        r = img.astype(np.float64) - tgt
        ref_g = 2 * r if kind == 0 else np.sign(r)
        ref_l = np.sum(r * r) if kind == 0 else np.sum(np.abs(r))
        np.testing.assert_allclose(g.cpu().numpy(), ref_g, rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(float(loss.item()), ref_l, rtol=1e-5)


def test_absgrad_variant_keeps_the_gradients():
    """With the absolute-gradient planes the call only adds their sums
    (non-negative); every other plane is bit-identical to the call without
    them."""
    torch = _torch()
    from differentiable_rasterization_amd import raster
    scene, cam = scenes.box_scene(n=20000, seed=14, width=320, height=200, fx=180.0)
    out = gpu_frame(scene, cam, loss_kind="l1", target=scenes.target_image(cam, 8))
    fr, g = out["frame"], raster.Gaussians.from_scene(scene)
    plain = grad2d_rows(fr, g.N).clone()
    fr.g_abs.fill_(-3.0)
    fr.rasterize_backward(g, absgrad=True)
    torch.cuda.synchronize()
    a, b = plain.cpu().numpy(), grad2d_rows(fr, g.N, absgrad=True).cpu().numpy()
    assert_bits_equal(b[:, 0:9], a[:, 0:9], "fields 0-8")
    vis = (fr.radii[:g.N] > 0).cpu().numpy()
    assert np.all(b[~vis, 9:11] == 0)  # overwritten, zeros without tiles
    assert np.all(b[:, 9:11] >= 0) and np.count_nonzero(b[:, 9:11]) > 0
    # |sum| <= sum |.|
    assert np.all(np.abs(b[:, 0:2]) <= b[:, 9:11] * (1 + 1e-5) + 1e-30)


@pytest.mark.parametrize("absgrad", [False, True])
def test_backward_stages_its_own_records(absgrad):
    """gs_rasterize_bwd with staged = 0 stages the records from the planes
    itself, into a workspace and partial slots that hold NaN, and gives the
    same bits as reusing what the forward staged (staged = 1)."""
    torch = _torch()
    from differentiable_rasterization_amd import raster
    from test_parity_gpu import _case
    scene, cam, loss, bg = _case("cluster_200k_640x416")
    out = gpu_frame(scene, cam, background=bg, loss_kind=loss, target=scenes.target_image(cam, 7),
                    absgrad=absgrad)
    fr = out["frame"]
    g = raster.Gaussians.from_scene(scene)
    nan = lambda t: torch.full_like(t, float("nan"))
    ws, parts = nan(fr.records), nan(fr.partials)
    g2 = raster.Grad2D(nan(fr.g_means2d), nan(fr.g_conics), nan(fr.g_opacities),
                       nan(fr.g_colors), nan(fr.g_abs) if absgrad else None)
    raster.gs_rasterize_bwd(g.N, g.ld, fr.W, fr.H, fr.ranges, fr.ids, fr.planes(g), fr.offsets,
                            fr.tiles, fr.M, fr.background, fr.settings, fr.final_T, fr.last_idx,
                            fr.dL_dimage, ws, fr.rec_bytes, 0, parts, fr.capacity, g2, 0,
                            tile_order=fr.order)
    torch.cuda.synchronize()
    N = scene.n
    pairs = [(g2.means2d, fr.g_means2d), (g2.conics, fr.g_conics),
             (g2.opacities, fr.g_opacities), (g2.colors, fr.g_colors)]
    if absgrad:
        pairs.append((g2.abs, fr.g_abs))
    for a, b in pairs:
        assert_bits_equal(a[..., :N].cpu().numpy(), b[..., :N].cpu().numpy(), "staged=0")


@pytest.mark.parametrize("packed", [False, True])
def test_rasterize_bwd_accumulate_modes(packed):
    """gs_rasterize_bwd's accumulate modes on top of a first pass (x + x == 2x
    exactly in fp32): 1 adds to every 2D plane; 2 adds to the opacity and
    absolute-gradient planes and overwrites the per-camera mean, conic and
    colour planes.  Rows without tiles keep their (zero) values."""
    torch = _torch()
    from differentiable_rasterization_amd import raster
    from test_parity_gpu import _case
    scene, cam, loss, bg = _case("cluster_200k_640x416")
    out = gpu_frame(scene, cam, background=bg, loss_kind=loss, target=scenes.target_image(cam, 7),
                    absgrad=True, packed=packed)
    fr, g = out["frame"], raster.Gaussians.from_scene(scene)
    N = fr.V if packed else scene.n  # packed: the rows of the visible list
    get = lambda t: t[..., :N].cpu().numpy().copy()
    names = ("g_means2d", "g_conics", "g_colors", "g_opacities", "g_abs")
    first = {k: get(getattr(fr, k)) for k in names}
    assert np.count_nonzero(first["g_means2d"]) > 0
    fr.rasterize_backward(g, absgrad=True, accumulate=1)
    torch.cuda.synchronize()
    for k in names:
        assert_bits_equal(get(getattr(fr, k)), 2 * first[k], "accumulate=1 %s" % k)
    fr.rasterize_backward(g, absgrad=True, accumulate=2)
    torch.cuda.synchronize()
    for k in ("g_means2d", "g_conics", "g_colors"):
        assert_bits_equal(get(getattr(fr, k)), first[k], "accumulate=2 %s" % k)
    for k in ("g_opacities", "g_abs"):
        assert_bits_equal(get(getattr(fr, k)), 3 * first[k], "accumulate=2 %s" % k)
