"""GPU parity of the packed mode (the gsplat guide §4.1 trains with packed
and sparse gradients): only the visible Gaussians take part after the
projection and receive gradients, as (index, value) rows.

Checks, per case:
- the visible list equals the oracle's set of Gaussians with tiles
  (ascending index), bit for bit, and V its length;
- binning, sort and ranges as in the dense path, bit for bit;
- the compositing backward's packed records and the projection backward's
  packed rows, scattered back to one row per Gaussian, against the oracle
  with the same tolerances and exemption rules as the dense path;
- the packed rows equal the dense path's rows of the same Gaussians bit for
  bit (the same kernels sum in the same order)."""
import functools

import numpy as np
import pytest

from differentiable_rasterization_amd import scenes
from parity_util import (assert_bits_equal, check_bins, check_e2e_grads, check_project_bwd,
                         check_raster_bwd, gpu_frame, run_parity_case)
from test_parity_gpu import _case

pytestmark = pytest.mark.gpu

CASES = ["tiny_1k_64", "box_20k_ragged", "box_20k_sh1", "box_20k_sh2", "cluster_200k_640x416",
         "cluster_1m_1280x832"]


@functools.lru_cache(maxsize=None)
def run_case(name):
    scene, cam, loss, bg = _case(name)
    return run_parity_case(name, scene, cam, loss, bg, scenes.target_image(cam, 7), packed=True)


@pytest.mark.parametrize("name", CASES)
def test_visible_list_and_bins(name):
    r = run_case(name)
    g, o = r["gpu"], r["orc"]
    want = np.flatnonzero(o["proj"]["tiles"] > 0).astype(np.uint32)
    assert g["V"] == len(want)
    assert_bits_equal(g["vis_ids"], want, "vis_ids")
    check_bins(r)


@pytest.mark.parametrize("name", CASES)
def test_packed_rasterize_bwd(name):
    check_raster_bwd(run_case(name))


@pytest.mark.parametrize("name", CASES)
def test_packed_project_bwd(name):
    check_project_bwd(run_case(name))


@pytest.mark.parametrize("name", CASES)
def test_packed_end_to_end_gradients(name):
    check_e2e_grads(run_case(name))


@pytest.mark.parametrize("name", CASES)
def test_packed_rows_equal_dense_rows(name):
    r = run_case(name)
    scene, cam = r["scene"], r["cam"]
    dense = gpu_frame(scene, cam, background=r["bg"], loss_kind=r["loss"], target=r["target"])
    packed = r["gpu"]
    vis = packed["vis_ids"].astype(np.int64)
    for k in ("g_means2d", "g_conics", "g_opac2d", "g_colors", "g_means", "g_scales",
              "g_quats", "g_opacities", "g_sh"):
        assert_bits_equal(packed[k][vis], dense[k][vis], k)
        # nothing off the list: the dense path writes zeros there
        off = np.ones(scene.n, bool)
        off[vis] = False
        assert np.all(dense[k][off] == 0), k
    for k in ("image", "final_T", "last"):
        assert_bits_equal(packed[k], dense[k], k)
