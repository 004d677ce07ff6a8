"""Seeded synthetic scenes and cameras.

This module only draws random inputs; it holds none of the rasterizer's
arithmetic and is the one piece both the HIP path's tests and the CPU oracle
are fed from.  The pages measure on datasets that are not available here
(Mip-NeRF 360 scenes and a bicycle capture in the gsplat guide
(lmnt.cn/news/262699) §3.3, DTU scan24 in the Moore Threads MUSA article
(qwbw.cn/news/278220) §4, an 8K architecture set in the A100 practice page
(codechina.net/…/390664) §3.1); these seeded scenes stand in for them with the
sizes the pages speak of (100k Gaussians at 1920x1080 in the gsplat guide
§2.1, scenes of about a million Gaussians in the A100 page §3.1).

Parameters are returned *activated*: scales = exp(log-scale),
opacities = sigmoid(logit), quaternions (w,x,y,z) of any norm (here unit),
SH coefficients [N, K, 3] with K = (degree+1)^2.  All arrays are float32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

Y00 = 0.28209479177387814  # 1 / (2 sqrt(pi)): the DC basis value, so that a
# uniform DC colour u maps to the coefficient (u - 0.5) / Y00 under the
# colour offset 0.5.


@dataclasses.dataclass
class Scene:
    means: np.ndarray      # [N,3] f32
    scales: np.ndarray     # [N,3] f32, > 0
    quats: np.ndarray      # [N,4] f32, (w,x,y,z)
    opacities: np.ndarray  # [N] f32, in (0,1)
    sh: np.ndarray         # [N,K,3] f32
    sh_degree: int

    @property
    def n(self) -> int:
        return int(self.means.shape[0])

    def subset(self, idx) -> "Scene":
        return Scene(self.means[idx], self.scales[idx], self.quats[idx], self.opacities[idx],
                     self.sh[idx], self.sh_degree)


@dataclasses.dataclass
class Camera:
    R: np.ndarray           # [3,3] world-to-camera rotation (OpenCV axes)
    t: np.ndarray           # [3]
    fx: float
    fy: float
    cx: float
    cy: float
    width: int
    height: int
    near: float = 0.01
    far: float = 1e10


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _sh(rng, n, degree, higher_std=0.2):
    K = (degree + 1) ** 2
    sh = np.zeros((n, K, 3), np.float64)
    u = rng.uniform(0.0, 1.0, size=(n, 3))
    sh[:, 0, :] = (u - 0.5) / Y00
    if K > 1:
        sh[:, 1:, :] = rng.normal(0.0, higher_std, size=(n, K - 1, 3))
    return sh


def _finish(rng, means, log_scales, degree):
    n = means.shape[0]
    quats = rng.normal(0.0, 1.0, size=(n, 4))
    quats /= np.linalg.norm(quats, axis=1, keepdims=True)
    opac = _sigmoid(rng.normal(0.0, 1.0, size=n))
    sh = _sh(rng, n, degree)
    return Scene(_f32(means), _f32(np.exp(log_scales)), _f32(quats), _f32(opac), _f32(sh),
                 degree)


def identity_camera(width, height, fx, fy=None) -> Camera:
    fy = fx if fy is None else fy
    f32 = lambda x: float(np.float32(x))
    return Camera(np.eye(3, dtype=np.float32), np.zeros(3, np.float32), f32(fx), f32(fy),
                  f32(width / 2.0), f32(height / 2.0), int(width), int(height))


def look_at_camera(eye, width, height, fx, fy=None, target=(0.0, 0.0, 0.0)) -> Camera:
    """World-to-camera pose at ``eye`` looking at ``target``: forward f, right
    r = normalize(f x (0,1,0)), down d = f x r, rows of R = [r; d; f]."""
    fy = fx if fy is None else fy
    eye = np.asarray(eye, np.float64)
    f = np.asarray(target, np.float64) - eye
    f /= np.linalg.norm(f)
    r = np.cross(f, np.array([0.0, 1.0, 0.0]))
    r /= np.linalg.norm(r)
    d = np.cross(f, r)
    R = np.stack([r, d, f], axis=0)
    t = -R @ eye
    # the library's camera is fp32: every value handed to either side is one
    return Camera(_f32(R), _f32(t), float(np.float32(fx)), float(np.float32(fy)),
                  float(np.float32(width / 2.0)), float(np.float32(height / 2.0)),
                  int(width), int(height))


def sphere_poses(n, radius, seed, width, height, fx, fy=None):
    """``n`` cameras on a sphere of ``radius`` looking at the origin; directions
    are normalised N(0,1)^3 draws with |d_y| > 0.9 rejected."""
    rng = np.random.default_rng(seed)
    cams = []
    while len(cams) < n:
        d = rng.normal(0.0, 1.0, size=3)
        d /= np.linalg.norm(d)
        if abs(d[1]) > 0.9:
            continue
        cams.append(look_at_camera(radius * d, width, height, fx, fy))
    return cams


def _random_rotation(rng):
    q, r = np.linalg.qr(rng.normal(size=(3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def clustered_means(rng, n, n_clusters, box):
    centers = rng.uniform(-box, box, size=(n_clusters, 3))
    rots = [_random_rotation(rng) for _ in range(n_clusters)]
    stds = np.stack([rng.uniform(0.5, 1.5, n_clusters), rng.uniform(0.5, 1.5, n_clusters),
                     np.full(n_clusters, 0.02)], axis=1)
    assign = rng.integers(0, n_clusters, size=n)
    local = rng.normal(0.0, 1.0, size=(n, 3)) * stds[assign]
    rot = np.stack(rots)[assign]
    return centers[assign] + np.einsum("nij,nj->ni", rot, local)


# ---------------------------------------------------------------------------
# The workload configurations
# ---------------------------------------------------------------------------
def tiny_scene(n=1024, seed=1, sh_degree=0):
    """1,024 Gaussians in camera space: x,y ~ U[-1,1], z ~ U[2,6]; log-scales
    N(-3, 0.5); random unit quaternions; opacity sigmoid(N(0,1)); SH degree 0
    with uniform RGB.  Camera: identity pose, fx = fy = 64, 64x64."""
    rng = np.random.default_rng(seed)
    means = np.concatenate([rng.uniform(-1, 1, size=(n, 2)), rng.uniform(2, 6, size=(n, 1))], 1)
    log_s = rng.normal(-3.0, 0.5, size=(n, 3))
    return _finish(rng, means, log_s, sh_degree), identity_camera(64, 64, 64.0)


def box_scene(n=100_000, seed=2, sh_degree=3, width=1920, height=1080, fx=1100.0):
    """100k Gaussians uniform in [-4,4]^3, SH degree 3; one camera at (0,0,-8)
    looking at the box centre, 1920x1080, fx = fy = 1100."""
    rng = np.random.default_rng(seed)
    means = rng.uniform(-4, 4, size=(n, 3))
    log_s = rng.normal(-3.0, 0.5, size=(n, 3))
    cam = Camera(np.eye(3, dtype=np.float32), np.array([0, 0, 8], np.float32), fx, fx,
                 width / 2.0, height / 2.0, width, height)
    return _finish(rng, means, log_s, sh_degree), cam


def cluster_scene(n=1_000_000, seed=3, sh_degree=3, n_clusters=64, box=5.0, log_s_mean=-5.5):
    """Surface-like clustered scene: ``n_clusters`` anisotropic clusters with
    centres U[-box,box]^3, random orientation and axis stds (U[.5,1.5],
    U[.5,1.5], 0.02); log-scales N(log_s_mean, 0.5); SH degree 3."""
    rng = np.random.default_rng(seed)
    means = clustered_means(rng, n, n_clusters, box)
    log_s = rng.normal(log_s_mean, 0.5, size=(n, 3))
    return _finish(rng, means, log_s, sh_degree)


def heavy_tail_scene(n=6_000_000, seed=5, sh_degree=3, n_clusters=512, box=24.0):
    """One device's shard of a large clustered scene with Student-t (nu=3)
    log-scales: -3.5 + 0.5 t_3, clipped at 1.0."""
    rng = np.random.default_rng(seed)
    means = clustered_means(rng, n, n_clusters, box)
    log_s = np.minimum(-3.5 + 0.5 * rng.standard_t(3, size=(n, 3)), 1.0)
    return _finish(rng, means, log_s, sh_degree)


def focal_for(width):
    return 1100.0 * width / 1920.0


def target_image(cam, seed):
    rng = np.random.default_rng(seed + 100)
    return _f32(rng.uniform(0.0, 1.0, size=(cam.height, cam.width, 3)))


CONFIGS = {
    "tiny_1k_64": "1,024 Gaussians, SH0, 64x64, L2",
    "box_100k_1080p": "100k Gaussians, SH3, 1920x1080, L2",
    "cluster_1m_1080p": "1M clustered Gaussians, SH3, 1920x1080, L1, 16 poses",
    "cluster_1m_1280x832": "1M clustered Gaussians, SH3, 1280x832, L1, 16 poses",
    "cluster_3m_4k": "3M clustered Gaussians, SH3, 3840x2160, forward only, 4 poses",
    "heavy_6m_1024": "6M heavy-tailed Gaussians, SH3, 1024x1024, 8 cameras",
}


def make_config(name, n=None):
    """Returns (scene, cameras, loss) for a named workload; ``n`` overrides the
    Gaussian count (same recipe, fewer draws) for reduced-size parity cases."""
    if name == "tiny_1k_64":
        s, c = tiny_scene(n or 1024)
        return s, [c], "l2"
    if name == "box_100k_1080p":
        s, c = box_scene(n or 100_000)
        return s, [c], "l2"
    if name in ("cluster_1m_1080p", "cluster_1m_1280x832"):
        w, h = (1920, 1080) if name.endswith("1080p") else (1280, 832)
        s = cluster_scene(n or 1_000_000)
        return s, sphere_poses(16, 6.0, 31, w, h, focal_for(w)), "l1"
    if name == "cluster_3m_4k":
        s = cluster_scene(n or 3_000_000, seed=4)
        return s, sphere_poses(4, 6.0, 41, 3840, 2160, 2200.0), None
    if name == "heavy_6m_1024":
        s = heavy_tail_scene(n or 6_000_000)
        return s, sphere_poses(8, 6.0, 51, 1024, 1024, focal_for(1024)), "l1"
    raise KeyError(name)
