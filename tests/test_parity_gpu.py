"""GPU parity of the five stages against the CPU oracle, on the same seeded
inputs, through the C ABI.

Cases span several tiles and ragged image edges, up to the full 100k-Gaussian
1920x1080 SH3 scene and one pose of the 1M-Gaussian clustered scene at
1920x1080 (the configuration the benchmark times).

Data flows from the oracle to the GPU only.  End to end, each side runs its
own whole path from the scene.  The backward stages are also compared in
isolation by feeding the GPU the oracle's own upstream gradient: the
oracle's dL/dimage (rounded to fp32) into the compositing backward, and the
oracle's 2D gradients into the projection backward.
"""
import functools

import pytest

from differentiable_rasterization_amd import scenes

from parity_util import (check_bins, check_e2e_grads, check_project_bwd, check_project_fwd,
                         check_raster_bwd, check_raster_fwd, run_parity_case)

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "tiny_1k_64":
        s, c = scenes.tiny_scene()
        return s, c, "l2", (0.0, 0.0, 0.0)
    if name == "box_20k_ragged":
        s, c = scenes.box_scene(n=20000, seed=12, width=500, height=270, fx=290.0)
        return s, c, "l2", (0.1, 0.2, 0.3)
    if name == "cluster_200k_640x416":
        s = scenes.cluster_scene(n=200_000, seed=13)
        c = scenes.sphere_poses(1, 6.0, 31, 640, 416, scenes.focal_for(640))[0]
        return s, c, "l1", (0.0, 0.0, 0.0)
    if name == "box_100k_1080p":
        s, c = scenes.box_scene()
        return s, c, "l2", (0.0, 0.0, 0.0)
    if name in ("cluster_1m_1080p", "cluster_1m_1280x832"):
        s, cams, loss = scenes.make_config(name)
        return s, cams[0], loss, (0.0, 0.0, 0.0)
    raise KeyError(name)


CASES = ["tiny_1k_64", "box_20k_ragged", "cluster_200k_640x416", "box_100k_1080p",
         "cluster_1m_1280x832", "cluster_1m_1080p"]


@functools.lru_cache(maxsize=None)
def run_case(name):
    scene, cam, loss, bg = _case(name)
    return run_parity_case(name, scene, cam, loss, bg, scenes.target_image(cam, 7))


@pytest.mark.parametrize("name", CASES)
def test_project_fwd_bit_exact(name):
    check_project_fwd(run_case(name))


@pytest.mark.parametrize("name", CASES)
def test_bin_and_sort_bit_exact(name):
    check_bins(run_case(name))


@pytest.mark.parametrize("name", CASES)
def test_rasterize_fwd(name):
    check_raster_fwd(run_case(name))


@pytest.mark.parametrize("name", CASES)
def test_rasterize_bwd(name):
    check_raster_bwd(run_case(name))


@pytest.mark.parametrize("name", CASES)
def test_project_bwd(name):
    check_project_bwd(run_case(name))


@pytest.mark.parametrize("name", CASES)
def test_end_to_end_gradients(name):
    check_e2e_grads(run_case(name))
