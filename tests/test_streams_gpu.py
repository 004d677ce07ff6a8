"""Frames in flight on separate HIP streams (how bench.py times the
workload's poses): every call takes its stream from the caller and all its
memory from the caller's buffers, so frames issued concurrently, each with
its own buffers, must give the same bits as the same frames one at a time.
Six poses of a 200k-Gaussian clustered scene at 640x416, dense and packed,
on three streams, step i on stream i mod 3 with the frame buffers reused
(each frame's outputs copied out on its stream before the next use).  Rows
a call leaves unwritten (the 2D records of culled Gaussians; packed rows past
the visible count) keep an earlier pose's values and are not compared."""
import numpy as np
import pytest

from differentiable_rasterization_amd import scenes
from parity_util import assert_bits_equal

pytestmark = pytest.mark.gpu

OUT = ("image", "final_T", "last_idx", "radii", "grads2d", "g_means", "g_scales",
       "g_quats", "g_opacities", "g_sh")
ROWS = ("g_means", "g_scales", "g_quats", "g_opacities", "g_sh")  # [..., rows]


def _run(packed, streams):
    import torch
    from differentiable_rasterization_amd import raster
    s = scenes.cluster_scene(200_000)
    cams = scenes.sphere_poses(6, 6.0, 31, 640, 416, scenes.focal_for(640))
    g = raster.Gaussians.from_scene(s)
    tg = [torch.from_numpy(scenes.target_image(c, i)).cuda() for i, c in enumerate(cams)]
    nf = max(1, len(streams))
    frs = [raster.Frame(g.ld, s.sh_degree, 640, 416, capacity=4 * s.n, packed=packed)
           for _ in range(nf)]
    outs = [None] * len(cams)
    for i, c in enumerate(cams):
        k = i % nf
        ctx = torch.cuda.stream(streams[k]) if streams else torch.cuda.stream(
            torch.cuda.current_stream())
        with ctx:
            fr = frs[k]
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


@pytest.mark.parametrize("packed", [False, True])
def test_frames_in_flight_match_serial(packed):
    import torch
    ref, N = _run(packed, [])
    got, _ = _run(packed, [torch.cuda.Stream() for _ in range(3)])
    for i, (a, b) in enumerate(zip(ref, got)):
        for n in ("image", "final_T", "last_idx", "radii"):
            assert_bits_equal(b[n], a[n], "pose %d %s" % (i, n))
        if packed:
            assert a["V"] == b["V"]
            V = a["V"]
            assert_bits_equal(b["grads2d"][:V], a["grads2d"][:V], "pose %d grads2d" % i)
            for n in ROWS:
                assert_bits_equal(b[n][..., :V], a[n][..., :V], "pose %d %s" % (i, n))
        else:
            vis = a["radii"][:N] > 0
            assert_bits_equal(b["grads2d"][:N][vis], a["grads2d"][:N][vis],
                              "pose %d grads2d" % i)
            for n in ROWS:
                assert_bits_equal(b[n][..., :N], a[n][..., :N], "pose %d %s" % (i, n))
    print("[streams] packed=%s: 6 poses on 3 streams bit-identical to serial" % packed,
          flush=True)
