"""GPU checks of the batched-camera forward (one launch per stage for a
batch of cameras, the 3M-Gaussian 4K workload's batch of four poses): for
every camera of a batch, the projection planes and records, the sorted keys
and ids, the tile ranges and the images must equal the single-camera calls'
bit for bit (those are checked against the oracle elsewhere), after removing
the batch's numbering (tile c * T + t, row c * ld + i, camera c's instances
after those of cameras 0 .. c-1).  One small batch is also checked against
the oracle directly."""
import numpy as np
import pytest

import oracle
from differentiable_rasterization_amd import scenes
from parity_util import (PIX_TOL, assert_bits_equal, check_e2e_2d, check_raster_fwd,
                         check_summed_grads, gpu_frame)

pytestmark = pytest.mark.gpu


def _batch(scene, cams, ld=None):
    import torch
    from differentiable_rasterization_amd import raster
    g = raster.Gaussians.from_scene(scene, ld=ld)
    bf = raster.BatchFrame(g.ld, scene.sh_degree, cams[0].width, cams[0].height, len(cams),
                           with_depth_alpha=True)
    bf.forward(g, cams)
    torch.cuda.synchronize()
    return g, bf


def _check_batch(name, scene, cams, ld=None):
    g, bf = _batch(scene, cams, ld)
    N, L, T = scene.n, g.ld, bf.T
    keys = bf.keys[:bf.M].cpu().numpy().view(np.uint64)
    ids = bf.ids[:bf.M].cpu().numpy().view(np.uint32)
    ranges = bf.ranges.cpu().numpy().view(np.uint32).reshape(len(cams), T, 2)
    base = 0
    for c, cam in enumerate(cams):
        one = gpu_frame(scene, cam, backward=False, depth_alpha=True, ld=ld)
        col = lambda t: t[c][:, :N].T if t.dim() == 3 else t[c][:N]
        for k in ("means2d", "conics", "chol", "depths", "radii", "colors"):
            assert_bits_equal(col(getattr(bf, k)).cpu().numpy(), one[k], "%s cam %d" % (k, c))
        assert_bits_equal(col(bf.tiles).cpu().numpy().view(np.uint32), one["tiles"], "tiles")
        # padding rows of the batch: no tiles
        assert np.all(bf.tiles[c][N:].cpu().numpy() == 0)
        M = one["M"]
        kc, ic = keys[base:base + M], ids[base:base + M]
        assert_bits_equal((kc >> np.uint64(32)) - np.uint64(c * T), one["keys"] >> np.uint64(32),
                          "key tiles cam %d" % c)
        assert_bits_equal(kc & np.uint64(0xFFFFFFFF), one["keys"] & np.uint64(0xFFFFFFFF),
                          "key depths cam %d" % c)
        assert_bits_equal(ic - np.uint32(c * L), one["ids"], "ids cam %d" % c)
        r = ranges[c].astype(np.int64)
        r1 = one["ranges"].reshape(T, 2).astype(np.int64)
        nz = r1[:, 1] > r1[:, 0]
        assert np.array_equal(r[nz] - base, r1[nz]), "ranges cam %d" % c
        assert np.all(r[~nz] == 0)
        for k, a in (("image", bf.image), ("final_T", bf.final_T), ("depth", bf.out_depth),
                     ("alpha", bf.out_alpha)):
            assert_bits_equal(a[c].cpu().numpy(), one[k], "%s cam %d" % (k, c))
        assert_bits_equal(bf.last_idx[c].cpu().numpy().view(np.uint32), one["last"], "last")
        base += M
    assert base == bf.M
    print("[batch] %s: %d cameras, M=%d" % (name, len(cams), bf.M), flush=True)
    return bf


def test_batch_against_oracle_small():
    scene = scenes.cluster_scene(n=20_000, seed=17)
    cams = scenes.sphere_poses(3, 6.0, 31, 200, 136, scenes.focal_for(200))
    g, bf = _batch(scene, cams)
    T = bf.T
    base = 0
    for c, cam in enumerate(cams):
        o = oracle.render(scene, cam)
        M = len(o["bins"]["keys"])
        kc = bf.keys[base:base + M].cpu().numpy().view(np.uint64)
        want = o["bins"]["keys"] + (np.uint64(c * T) << np.uint64(32))
        assert_bits_equal(kc, want, "keys cam %d" % c)
        assert_bits_equal(bf.ids[base:base + M].cpu().numpy().view(np.uint32) -
                          np.uint32(c * g.ld), o["bins"]["ids"], "ids cam %d" % c)
        d = np.abs(bf.image[c].cpu().numpy() - o["raster"]["image"]).max()
        assert d <= PIX_TOL, (c, d)
        base += M
    assert base == bf.M


def test_batch_cluster_1m_1080p_four_poses_against_oracle():
    """Four poses of the timed workload (1M Gaussians, 1920x1080, L1) as one
    batch, forward with the fused loss gradient and backward, against the
    oracle run per camera: each camera's image, T, last indices and 2D
    gradient planes to the parity bars, and the 3D and opacity gradients
    summed over the batch against the sum of the oracle's."""
    import torch
    from differentiable_rasterization_amd import raster
    scene, cams, _ = scenes.make_config("cluster_1m_1080p")
    cams = cams[:4]
    g = raster.Gaussians.from_scene(scene)
    bf = raster.BatchFrame(g.ld, scene.sh_degree, cams[0].width, cams[0].height, len(cams))
    tg = np.stack([scenes.target_image(c, 7) for c in cams])
    bf.forward(g, cams, target=torch.from_numpy(tg).cuda(), kind=1)
    bf.backward(g)
    torch.cuda.synchronize()
    n, K = scene.n, (scene.sh_degree + 1) ** 2
    P = lambda t, c: t[c][:, :n].T.contiguous().cpu().numpy()
    rs = []
    for c, cam in enumerate(cams):
        orc = oracle.render(scene, cam, None, (0.0, 0.0, 0.0), with_margin=True)
        dl = oracle.loss_grad_image(orc["raster"]["image"], tg[c], oracle.LOSS_L1)
        bw = oracle.backward(scene, cam, orc, dl, None, (0.0, 0.0, 0.0), with_abs=True)
        gpu = dict(image=bf.image[c].cpu().numpy(), final_T=bf.final_T[c].cpu().numpy(),
                   last=bf.last_idx[c].cpu().numpy().view(np.uint32),
                   dL_dimage=bf.dL_dimage[c].cpu().numpy(), g_means2d=P(bf.g_means2d, c),
                   g_conics=P(bf.g_conics, c), g_colors=P(bf.g_colors, c),
                   g_opac2d=bf.g_opacities_cams[c][:n].cpu().numpy())
        r = dict(name="cluster_1m_1080p batch camera %d" % c, scene=scene, cam=cam, orc=orc,
                 gpu=gpu, bw=bw, dl=dl.astype(np.float32))
        check_raster_fwd(r)
        check_e2e_2d(r)
        rs.append(r)
    T = lambda t: t[:, :n].T.contiguous().cpu().numpy()
    got = dict(means=T(bf.g_means), scales=T(bf.g_scales), quats=T(bf.g_quats),
               sh=T(bf.g_sh).reshape(n, K, 3), opacities=bf.g_opacities[:n].cpu().numpy())
    check_summed_grads(rs, got, "cluster_1m_1080p batch of 4")


def test_batch_cluster_200k_three_poses():
    scene = scenes.cluster_scene(n=200_000, seed=13)
    cams = scenes.sphere_poses(3, 6.0, 31, 640, 416, scenes.focal_for(640))
    _check_batch("cluster_200k_640x416", scene, cams)


def test_batch_ragged_box_padded_rows():
    s, cam = scenes.box_scene(n=20000, seed=12, width=500, height=270, fx=290.0)
    cam2 = scenes.look_at_camera(np.array([3.0, 2.0, -7.0]), 500, 270, 290.0)
    _check_batch("box_20k_ragged", s, [cam, cam2], ld=20011)


def test_batch_single_camera():
    scene = scenes.cluster_scene(n=50_000, seed=14)
    cams = scenes.sphere_poses(1, 6.0, 31, 320, 208, scenes.focal_for(320))
    _check_batch("one camera", scene, cams)


def test_batch_cluster_3m_4k_four_poses():
    """The 3M-Gaussian 3840 x 2160 workload's batch of four poses."""
    scene, cams, _ = scenes.make_config("cluster_3m_4k")
    _check_batch("cluster_3m_4k", scene, cams)


def _check_backward(name, scene, cams, ld=None, accumulate=0):
    """Batched backward against single-camera calls with accumulate (camera 0
    overwrites, the next ones add; with ``accumulate`` every camera adds to
    the same seeded starting values): the 2D planes of every camera and the
    summed 3D and opacity gradients, bit for bit."""
    import torch
    from differentiable_rasterization_amd import raster
    g, bf = _batch(scene, cams, ld)
    N, L, C = scene.n, g.ld, len(cams)
    tgt = torch.from_numpy(np.stack([scenes.target_image(c, k) for k, c in enumerate(cams)])).cuda()
    raster.gs_image_loss_grad(1, tgt.numel(), bf.image, tgt, bf.dL_dimage, None)
    fr = raster.Frame(g.ld, scene.sh_degree, cams[0].width, cams[0].height)
    if accumulate:
        rng = np.random.default_rng(17)
        for k in ("g_means", "g_scales", "g_quats", "g_opacities", "g_sh"):
            start = torch.from_numpy(
                rng.normal(0.0, 1.0, tuple(getattr(bf, k).shape)).astype(np.float32)).cuda()
            getattr(bf, k).copy_(start)
            getattr(fr, k).copy_(start)
    bf.backward(g, accumulate=accumulate)
    torch.cuda.synchronize()
    for c, cam in enumerate(cams):
        fr.forward(g, cam)
        fr.loss_grad(tgt[c], 1, with_loss=False)
        fr.backward(g, accumulate=int(c > 0 or bool(accumulate)))
        torch.cuda.synchronize()
        assert_bits_equal(bf.dL_dimage[c].cpu().numpy(), fr.dL_dimage.cpu().numpy(), "dL/dimage")
        # this camera's 2D planes (the single-camera frame overwrites them
        # per camera and adds only the opacity gradient)
        for k in ("g_means2d", "g_conics", "g_colors"):
            assert_bits_equal(getattr(bf, k)[c][:, :N].cpu().numpy(),
                              getattr(fr, k)[:, :N].cpu().numpy(), "%s cam %d" % (k, c))
    for k in ("g_means", "g_scales", "g_quats", "g_opacities", "g_sh"):
        a, b = getattr(bf, k), getattr(fr, k)
        a = a[..., :N].cpu().numpy()
        b = b[..., :N].cpu().numpy()
        assert_bits_equal(a, b, k)
    print("[batch] %s backward: %d cameras, M=%d" % (name, C, bf.M), flush=True)


def test_batch_fused_loss_matches_separate_loss():
    """gs_rasterize_fwd_loss_batched against gs_rasterize_fwd_batched followed
    by gs_image_loss_grad over the batch: images, T, last indices and the
    loss gradient bit for bit, for L1 and L2; the loss value to float
    summation tolerance."""
    import torch
    from differentiable_rasterization_amd import raster
    scene = scenes.cluster_scene(n=200_000, seed=13)
    cams = scenes.sphere_poses(3, 6.0, 31, 640, 416, scenes.focal_for(640))
    g, bf = _batch(scene, cams)
    tgt = torch.from_numpy(np.stack([scenes.target_image(c, k) for k, c in enumerate(cams)])).cuda()
    for kind in (0, 1):
        bf.forward(g, cams)
        ref_loss = torch.zeros(1, dtype=torch.float32, device="cuda")
        raster.gs_image_loss_grad(kind, tgt.numel(), bf.image, tgt, bf.dL_dimage, ref_loss)
        torch.cuda.synchronize()
        ref = {k: getattr(bf, k).clone() for k in ("image", "final_T", "last_idx", "dL_dimage")}
        bf.dL_dimage.zero_()
        loss = torch.zeros(1, dtype=torch.float32, device="cuda")
        bf.forward(g, cams, target=tgt, kind=kind, loss=loss)
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert_bits_equal(getattr(bf, k).cpu().numpy(), v.cpu().numpy(), "%s kind %d" % (k, kind))
        a, b = float(loss.item()), float(ref_loss.item())
        assert abs(a - b) <= 1e-5 * abs(b) + 1e-3, (kind, a, b)
    print("[batch] fused loss: 3 cameras, L1 and L2 bit-identical to the separate pass",
          flush=True)


def test_batch_backward_cluster_200k():
    scene = scenes.cluster_scene(n=200_000, seed=13)
    cams = scenes.sphere_poses(3, 6.0, 31, 640, 416, scenes.focal_for(640))
    _check_backward("cluster_200k_640x416", scene, cams)


def test_batch_backward_accumulate_cluster_200k():
    scene = scenes.cluster_scene(n=200_000, seed=13)
    cams = scenes.sphere_poses(3, 6.0, 31, 640, 416, scenes.focal_for(640))
    _check_backward("cluster_200k_640x416 accumulate", scene, cams, accumulate=1)


def test_batch_backward_ragged_padded():
    s, cam = scenes.box_scene(n=20000, seed=12, width=500, height=270, fx=290.0)
    cam2 = scenes.look_at_camera(np.array([3.0, 2.0, -7.0]), 500, 270, 290.0)
    _check_backward("box_20k_ragged", s, [cam, cam2, cam], ld=20011)


def test_batch_backward_cluster_1m_1080p_four_poses():
    scene, cams, _ = scenes.make_config("cluster_1m_1080p")
    _check_backward("cluster_1m_1080p", scene, cams[:4])


def test_batch_eight_cameras_forward_and_backward():
    """The largest batch the calls take (eight cameras): the forward and the
    backward against single-camera calls, bit for bit."""
    scene = scenes.cluster_scene(n=200_000, seed=13)
    cams = scenes.sphere_poses(8, 6.0, 33, 640, 416, scenes.focal_for(640))
    _check_batch("cluster_200k_640x416 x8", scene, cams)
    _check_backward("cluster_200k_640x416 x8", scene, cams)


def test_batch_all_culled():
    """A batch in which no camera sees any Gaussian (all behind every
    camera): no instances, every image the background with T = 1 and no
    last index, and zero gradients from the backward."""
    import torch
    from differentiable_rasterization_amd import raster
    scene, _ = scenes.tiny_scene(n=50)
    scene.means[:, 2] = -scene.means[:, 2]
    cams = [scenes.identity_camera(40, 24, 30.0), scenes.identity_camera(40, 24, 45.0)]
    bg = (0.25, 0.5, 0.75)
    g = raster.Gaussians.from_scene(scene)
    bf = raster.BatchFrame(g.ld, scene.sh_degree, 40, 24, len(cams), background=bg)
    bf.forward(g, cams)
    bf.dL_dimage.fill_(1.0)
    bf.backward(g)
    torch.cuda.synchronize()
    assert bf.M == 0
    assert np.all(bf.ranges.cpu().numpy() == 0)
    for c in range(len(cams)):
        np.testing.assert_array_equal(bf.image[c].cpu().numpy(),
                                      np.broadcast_to(np.float32(bg), (24, 40, 3)))
        assert np.all(bf.final_T[c].cpu().numpy() == 1.0)
        assert np.all(bf.last_idx[c].cpu().numpy() == 0)
    n = scene.n
    for k in ("g_means2d", "g_conics", "g_colors", "g_opacities_cams"):
        assert np.all(getattr(bf, k)[..., :n].cpu().numpy() == 0), k
    for k in ("g_means", "g_scales", "g_quats", "g_opacities", "g_sh"):
        assert np.all(getattr(bf, k)[..., :n].cpu().numpy() == 0), k


@pytest.mark.parametrize("deg", [0, 1, 2])
def test_batch_low_sh_degrees(deg):
    """The batched projection and projection backward at SH degrees 0, 1 and
    2 against single-camera calls, bit for bit."""
    s, cam = scenes.box_scene(n=20000, seed=15, sh_degree=deg, width=320, height=200,
                              fx=190.0)
    cam2 = scenes.look_at_camera(np.array([3.0, 2.0, -7.0]), 320, 200, 190.0)
    _check_batch("box_20k_sh%d" % deg, s, [cam, cam2])
    _check_backward("box_20k_sh%d" % deg, s, [cam, cam2])
