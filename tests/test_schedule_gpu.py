"""The compositing schedule (gs_tile_order).  It is a launch order, no step
of the method, so two things are checked:
- each camera's order is a permutation of its tiles with the length bucket
  (eight buckets per power of two, as the header states) never increasing;
- the compositing forward and backward, dense, packed and batched, give the
  same bits with the schedule as with the fixed order, because each tile's
  work is done by one workgroup whichever tile it takes first."""
import numpy as np
import pytest

from differentiable_rasterization_amd import scenes
from parity_util import assert_bits_equal, gpu_frame
from test_parity_gpu import _case

pytestmark = pytest.mark.gpu

# cluster_200k_5k: 57,600 tiles, past the 32,768 whose buckets the schedule
# keeps in LDS (its second pass recomputes them from the ranges)
CASES = ["tiny_1k_64", "box_20k_ragged", "cluster_200k_640x416", "cluster_200k_5k",
         "cluster_1m_1080p"]
OUTPUTS = ("image", "final_T", "last", "g_means2d", "g_conics", "g_opac2d", "g_colors",
           "g_means", "g_scales", "g_quats", "g_opacities", "g_sh")


def bucket(n):
    """Length bucket as specified: n below 8, else (e - 2) * 8 plus the three
    bits after the leading one, e = floor(log2 n)."""
    n = np.asarray(n, np.int64)
    e = np.floor(np.log2(np.maximum(n, 1))).astype(np.int64)
    e = np.where((np.int64(1) << e) > n, e - 1, e)           # exact floor(log2 n)
    e = np.where((np.int64(1) << (e + 1)) <= n, e + 1, e)
    big = (e - 2) * 8 + ((n >> np.maximum(e - 3, 0)) & 7)
    return np.where(n < 8, n, big)


def check_order(order, ranges, T):
    order = order.astype(np.int64)
    assert np.array_equal(np.sort(order), np.arange(T)), "not a permutation"
    lengths = ranges[:, 1].astype(np.int64) - ranges[:, 0].astype(np.int64)
    b = bucket(lengths[order])
    assert np.all(np.diff(b) <= 0), "length bucket increases along the order"


def test_bucket_spec():
    assert list(bucket([0, 1, 7, 8, 9, 15, 16, 17, 18, 31, 32])) == \
        [0, 1, 7, 8, 9, 15, 16, 16, 17, 23, 24]
    assert bucket(2 ** 32 - 1) == 29 * 8 + 7


@pytest.mark.parametrize("name", CASES)
def test_order_is_longest_first_permutation(name):
    scene, cam, loss, bg = _case(name)
    r = gpu_frame(scene, cam, background=bg, backward=False)
    fr = r["frame"]
    check_order(fr.order.cpu().numpy().view(np.uint32), r["ranges"].reshape(-1, 2), fr.T)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("name", CASES)
def test_schedule_leaves_outputs_unchanged(name, packed):
    scene, cam, loss, bg = _case(name)
    tgt = scenes.target_image(cam, 7)
    a = gpu_frame(scene, cam, background=bg, loss_kind=loss, target=tgt, packed=packed,
                  schedule=True)
    b = gpu_frame(scene, cam, background=bg, loss_kind=loss, target=tgt, packed=packed,
                  schedule=False)
    assert b["frame"].order is None
    for k in OUTPUTS:
        assert_bits_equal(a[k], b[k], k)


@pytest.mark.parametrize("W,H,ncam", [(640, 416, 3), (5120, 2880, 2)])
def test_batched_schedule(W, H, ncam):
    import torch
    from differentiable_rasterization_amd import raster
    scene = scenes.cluster_scene(n=200_000, seed=13)
    cams = scenes.sphere_poses(ncam, 6.0, 31, W, H, scenes.focal_for(W))
    g = raster.Gaussians.from_scene(scene)
    out = []
    for schedule in (True, False):
        bf = raster.BatchFrame(g.ld, scene.sh_degree, W, H, len(cams), schedule=schedule)
        bf.forward(g, cams)
        bf.dL_dimage.copy_(torch.sign(bf.image - 0.5))
        bf.backward(g)
        torch.cuda.synchronize()
        out.append(bf)
    a, b = out
    T = a.T
    order = a.order.cpu().numpy().view(np.uint32).reshape(len(cams), T)
    ranges = a.ranges.cpu().numpy().view(np.uint32).reshape(len(cams), T, 2)
    for c in range(len(cams)):
        check_order(order[c], ranges[c], T)
    for k in ("image", "final_T", "last_idx", "g_means2d", "g_conics", "g_opacities_cams",
              "g_colors", "g_means", "g_scales", "g_quats", "g_opacities", "g_sh"):
        assert_bits_equal(getattr(a, k).cpu().numpy(), getattr(b, k).cpu().numpy(), k)
