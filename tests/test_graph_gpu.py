"""Binning without the read-back (gs_bin_and_sort_device) and whole frames
captured into HIP graphs.

- The device-count frame equals the read-back frame bit for bit (keys, ids,
  ranges, images, every gradient), and the device count equals M.
- Too small a capacity: the overflow flag is set, M is still reported, the
  list is empty (background image), and nothing is read or written past the
  buffers; after growing them the frame is right.
- A fwd+bwd frame per pose captured into a graph and replayed several times,
  with eager frames of other poses and synchronisations in between: every
  replay equals the eager frame bit for bit."""
import numpy as np
import pytest

from differentiable_rasterization_amd import scenes
from parity_util import assert_bits_equal

pytestmark = pytest.mark.gpu

OUTS = ("image", "final_T", "last_idx", "g_means2d", "g_conics", "g_colors", "g_means",
        "g_scales", "g_quats", "g_opacities", "g_sh")


def _setup(n=200_000, poses=2):
    import torch
    from differentiable_rasterization_amd import raster
    scene = scenes.cluster_scene(n=n, seed=13)
    cams = scenes.sphere_poses(poses, 6.0, 31, 640, 416, scenes.focal_for(640))
    g = raster.Gaussians.from_scene(scene)
    tg = [torch.from_numpy(scenes.target_image(c, k)).cuda() for k, c in enumerate(cams)]
    return scene, cams, g, tg


def _frame(g, scene, cam, tgt, **kw):
    from differentiable_rasterization_amd import raster
    fr = raster.Frame(g.ld, scene.sh_degree, cam.width, cam.height, **kw)
    _step(fr, g, cam, tgt)
    return fr


def _step(fr, g, cam, tgt):
    fr.forward(g, cam)
    fr.loss_grad(tgt, 1, with_loss=False)
    fr.backward(g)


def _snap(fr, N):
    import torch
    torch.cuda.synchronize()
    out = {}
    for k in OUTS:
        t = getattr(fr, k)
        out[k] = (t[..., :N] if k.startswith("g_") else t).cpu().numpy().copy()
    return out


def _same(a, b, what):
    for k in OUTS:
        assert_bits_equal(a[k], b[k], "%s %s" % (what, k))


def test_device_count_equals_read_back():
    scene, cams, g, tg = _setup()
    N = scene.n
    for c, cam in enumerate(cams):
        host = _frame(g, scene, cam, tg[c])
        dev = _frame(g, scene, cam, tg[c], device_count=True, capacity=host.capacity)
        M, over = dev.check_counts()
        assert M == host.M and not over
        assert_bits_equal(dev.keys[:M].cpu().numpy(), host.keys[:M].cpu().numpy(), "keys")
        assert_bits_equal(dev.ids[:M].cpu().numpy(), host.ids[:M].cpu().numpy(), "ids")
        assert_bits_equal(dev.ranges.cpu().numpy(), host.ranges.cpu().numpy(), "ranges")
        _same(_snap(dev, N), _snap(host, N), "camera %d" % c)


def test_device_count_overflow_then_grow():
    import torch
    scene, cams, g, tg = _setup(poses=1)
    cam = cams[0]
    host = _frame(g, scene, cam, tg[0])
    dev = _frame(g, scene, cam, tg[0], device_count=True, capacity=host.M // 3)
    M, over = dev.check_counts()
    assert over and M == host.M
    assert np.all(dev.ranges.cpu().numpy() == 0)
    assert np.all(dev.image.cpu().numpy() == 0.0)  # black background
    # the backward of an overflowed frame stays in bounds; its gradients are
    # not meaningful until the frame runs again with larger buffers
    dev._alloc_sort(M + 1024)
    _step(dev, g, cam, tg[0])
    M2, over2 = dev.check_counts()
    assert M2 == host.M and not over2
    torch.cuda.synchronize()
    assert_bits_equal(dev.image.cpu().numpy(), host.image.cpu().numpy(), "image after growing")
    assert_bits_equal(dev.g_means[:, :scene.n].cpu().numpy(),
                      host.g_means[:, :scene.n].cpu().numpy(), "g_means after growing")


def test_graph_replays_equal_eager_frames():
    import torch
    from differentiable_rasterization_amd import raster
    scene, cams, g, tg = _setup(poses=3)
    N = scene.n
    eager = [_snap(_frame(g, scene, cam, tg[c]), N) for c, cam in enumerate(cams)]
    cap = 4 * g.ld
    frames, graphs = [], []
    for c in range(2):
        fr = raster.Frame(g.ld, scene.sh_degree, cams[c].width, cams[c].height,
                          device_count=True, capacity=cap)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            _step(fr, g, cams[c], tg[c])  # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            _step(fr, g, cams[c], tg[c])
        frames.append(fr)
        graphs.append(gr)
    other = raster.Frame(g.ld, scene.sh_degree, cams[2].width, cams[2].height)
    for rep in range(3):
        for c in range(2):
            for k in OUTS:  # poison the outputs: the replay must rewrite them
                getattr(frames[c], k).fill_(-7)
            graphs[c].replay()
            got = _snap(frames[c], N)
            _same(got, eager[c], "replay %d camera %d" % (rep, c))
            # eager work between replays
            _step(other, g, cams[2], tg[2])
            torch.cuda.synchronize()
            assert frames[c].check_counts()[1] is False
    _same(_snap(other, N), eager[2], "eager camera 2")


def test_full_size_device_count_and_graph_replays():
    """The benchmark's graph frames at full size (1M Gaussians, 1920x1080,
    buffers for 1.25 x the largest M of the poses + 8192, as the benchmark
    sizes them): device-count binning equals the read-back frame, and a
    captured frame replayed twice (outputs poisoned before each replay,
    eager work and synchronisations in between) equals the eager frame, bit
    for bit."""
    import torch
    from differentiable_rasterization_amd import raster
    scene, cams, _ = scenes.make_config("cluster_1m_1080p")
    cams = cams[:2]
    g = raster.Gaussians.from_scene(scene)
    tg = [torch.from_numpy(scenes.target_image(c, k)).cuda() for k, c in enumerate(cams)]
    N = scene.n
    hosts = [_frame(g, scene, c, tg[k]) for k, c in enumerate(cams)]
    Ms = [h.M for h in hosts]
    eager = [_snap(h, N) for h in hosts]
    del hosts
    cap = int(1.25 * max(Ms)) + 8192
    dev = _frame(g, scene, cams[0], tg[0], device_count=True, capacity=cap)
    M, over = dev.check_counts()
    assert M == Ms[0] and not over
    _same(_snap(dev, N), eager[0], "device count camera 0")
    fr = raster.Frame(g.ld, scene.sh_degree, cams[1].width, cams[1].height, device_count=True,
                      capacity=cap)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(fr, g, cams[1], tg[1])  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        _step(fr, g, cams[1], tg[1])
    for rep in range(2):
        for k in OUTS:
            getattr(fr, k).fill_(-7)
        gr.replay()
        _same(_snap(fr, N), eager[1], "full-size replay %d" % rep)
        assert fr.check_counts() == (Ms[1], False)
        _step(dev, g, cams[0], tg[0])
        torch.cuda.synchronize()
    _same(_snap(dev, N), eager[0], "device count camera 0 after the replays")
