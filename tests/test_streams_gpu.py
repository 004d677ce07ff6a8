"""Frames in flight on separate HIP streams (how bench.py times the
workload's poses): every call takes its stream from the caller and all its
memory from the caller's buffers, so frames issued concurrently, each with
its own buffers, must give the same bits as the same frames one at a time.
Six poses of a 200k-Gaussian clustered scene at 640x416, dense and packed,
on three streams, step i on stream i mod 3 with the frame buffers reused
(each frame's outputs copied out on its stream before the next use), in
the plain order and in the benchmark's order, where the next pose's
projection is issued before this pose's binning waits on its count.  Rows
a call leaves unwritten (the 2D records of culled Gaussians; packed rows past
the visible count) keep an earlier pose's values and are not compared."""
import numpy as np
import pytest

from differentiable_rasterization_amd import scenes
from parity_util import assert_bits_equal

pytestmark = pytest.mark.gpu

OUT = ("image", "final_T", "last_idx", "radii", "g_means2d", "g_conics", "g_colors", "g_means",
       "g_scales", "g_quats", "g_opacities", "g_sh")
ROWS = ("g_means2d", "g_conics", "g_colors", "g_means", "g_scales", "g_quats", "g_opacities",
        "g_sh")  # [..., rows]


def _run(packed, streams, ahead=False, full=False):
    import torch
    from differentiable_rasterization_amd import raster
    if full:
        # the benchmark's workload: 1M Gaussians, 1920x1080, its first poses
        s, cams, _ = scenes.make_config("cluster_1m_1080p")
        cams = cams[:4]
    else:
        s = scenes.cluster_scene(200_000)
        cams = scenes.sphere_poses(6, 6.0, 31, 640, 416, scenes.focal_for(640))
    W, H = cams[0].width, cams[0].height
    g = raster.Gaussians.from_scene(s)
    tg = [torch.from_numpy(scenes.target_image(c, i)).cuda() for i, c in enumerate(cams)]
    nf = max(1, len(streams))
    frs = [raster.Frame(g.ld, s.sh_degree, W, H, capacity=4 * s.n, packed=packed)
           for _ in range(nf)]
    outs = [None] * len(cams)

    def on(i):
        return torch.cuda.stream(streams[i % nf]) if streams else torch.cuda.stream(
            torch.cuda.current_stream())
    if ahead:
        with on(0):
            frs[0].project(g, cams[0])
    for i, c in enumerate(cams):
        k = i % nf
        if ahead and i + 1 < len(cams):
            with on(i + 1):
                frs[(i + 1) % nf].project(g, cams[i + 1])
        with on(i):
            fr = frs[k]
            if not ahead:
                fr.project(g, c)
            fr.bin_and_sort(g)
            fr.rasterize_loss(g, tg[i], 1)
            fr.rasterize_backward(g)
            fr.project_backward(g)
            outs[i] = {n: getattr(fr, n).clone() for n in OUT}
            outs[i]["V"] = fr.V if packed else None
    torch.cuda.synchronize()
    return [{n: (v.cpu().numpy() if hasattr(v, "cpu") else v) for n, v in o.items()}
            for o in outs], s.n


@pytest.mark.parametrize("ahead", [False, True])
@pytest.mark.parametrize("packed", [False, True])
def test_frames_in_flight_match_serial(packed, ahead):
    import torch
    ref, N = _run(packed, [])
    got, _ = _run(packed, [torch.cuda.Stream() for _ in range(3)], ahead)
    for i, (a, b) in enumerate(zip(ref, got)):
        for n in ("image", "final_T", "last_idx", "radii"):
            assert_bits_equal(b[n], a[n], "pose %d %s" % (i, n))
        if packed:
            assert a["V"] == b["V"]
            V = a["V"]
            for n in ROWS:
                assert_bits_equal(b[n][..., :V], a[n][..., :V], "pose %d %s" % (i, n))
        else:
            for n in ROWS:
                assert_bits_equal(b[n][..., :N], a[n][..., :N], "pose %d %s" % (i, n))
    print("[streams] packed=%s ahead=%s: 6 poses on 3 streams bit-identical to serial"
          % (packed, ahead), flush=True)


def test_full_size_frames_in_flight_match_serial():
    """The benchmark's launch configuration at full size: four poses of the
    1M-Gaussian 1080p workload, three frames in flight in its issue order,
    bit-identical to the same frames one at a time."""
    import torch
    ref, N = _run(False, [], full=True)
    got, _ = _run(False, [torch.cuda.Stream() for _ in range(3)], True, full=True)
    for i, (a, b) in enumerate(zip(ref, got)):
        for n in ("image", "final_T", "last_idx", "radii"):
            assert_bits_equal(b[n], a[n], "full pose %d %s" % (i, n))
        for n in ROWS:
            assert_bits_equal(b[n][..., :N], a[n][..., :N], "full pose %d %s" % (i, n))
