"""CPU oracle of the tile-based 3D Gaussian Splatting rasterizer.

TEST INFRASTRUCTURE ONLY: a plain, slow, obviously-correct reference that the
HIP path is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the product package
never does.  It shares no code with the HIP path: ``liboracle.so`` is built
from ``oracle.cpp`` alone by ``g++`` (see :func:`build`).

Inputs use the natural per-Gaussian layout: means [N,3], scales [N,3]
(activated, > 0), quats [N,4] (w,x,y,z, any non-zero norm), opacities [N]
(activated, in [0,1]), sh [N,K,3] with K = (degree+1)^2.  ``cam`` is any
object with attributes R [3,3] (world-to-camera), t [3], fx, fy, cx, cy,
width, height, near, far.

Passages followed (the pages print no formulas; see oracle.cpp for the
step-by-step reading): gsplat guide (lmnt.cn/news/262699) §2.1 three-stage
pipeline, §2.2 separate backward, §3.3 quaternion order and activations;
Moore Threads MUSA article (qwbw.cn/news/278220) §3.3 covariance from scale
and rotation.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.cpp")

MODE_F32KEY = 0
MODE_F64 = 1
LOSS_L2 = 0
LOSS_L1 = 1

# fp32 constants of the method (the pages give none; textbook 3DGS values)
DEFAULT_SETTINGS = dict(eps2d=0.3, alpha_min=1.0 / 255.0, alpha_max=0.99,
                        T_min=1e-4, fov_clamp=1.3, sh_offset=0.5)


def build(force: bool = True) -> str:
    """Compile liboracle.so with g++ (IEEE fp32, no contraction, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Camera(C.Structure):
    _fields_ = [("R", C.c_double * 9), ("t", C.c_double * 3),
                ("fx", C.c_double), ("fy", C.c_double), ("cx", C.c_double), ("cy", C.c_double),
                ("width", C.c_int32), ("height", C.c_int32),
                ("near_plane", C.c_double), ("far_plane", C.c_double)]


class _Settings(C.Structure):
    _fields_ = [(k, C.c_float) for k in
                ("eps2d", "alpha_min", "alpha_max", "T_min", "fov_clamp", "sh_offset")]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        lib.orc_project.argtypes = [C.c_int, C.c_int64, C.c_int] + [P] * 16
        lib.orc_project.restype = C.c_int
        lib.orc_bin_f32.argtypes = [C.c_int64, P, P, P, C.c_int32, C.c_int32, C.c_int64, P, P, P, P]
        lib.orc_bin_f32.restype = C.c_int64
        lib.orc_bin_f64.argtypes = [C.c_int64, P, P, P, C.c_int32, C.c_int32, C.c_int64, P, P]
        lib.orc_bin_f64.restype = C.c_int64
        lib.orc_composite.argtypes = [C.c_int32, C.c_int32] + [P] * 15
        lib.orc_composite.restype = C.c_int
        lib.orc_composite_bwd.argtypes = [C.c_int32, C.c_int32, C.c_int64] + [P] * 15
        lib.orc_composite_bwd.restype = C.c_int
        lib.orc_project_bwd.argtypes = [C.c_int64, C.c_int] + [P] * 14
        lib.orc_project_bwd.restype = C.c_int
        lib.orc_project_bwd_bound.argtypes = [C.c_int64, C.c_int] + [P] * 14
        lib.orc_project_bwd_bound.restype = C.c_int
        lib.orc_loss_jvp.argtypes = [C.c_int64, C.c_int] + [P] * 13 + [C.c_int] + [P] * 5
        lib.orc_loss_jvp.restype = C.c_int64
        for name in ("orc_rotation",):
            getattr(lib, name).argtypes = [P, P]
        lib.orc_cov3d.argtypes = [P, P, P]
        lib.orc_set_threads.argtypes = [C.c_int]
        lib.orc_set_threads.restype = C.c_int
        lib.orc_sh_basis.argtypes = [C.c_int, P, P]
        lib.orc_sh_basis_grad.argtypes = [C.c_int, P, P]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f64(a, shape=None):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None:
        a = a.reshape(shape)
    return a


def camera_struct(cam) -> _Camera:
    c = _Camera()
    R = np.asarray(cam.R, dtype=np.float64).reshape(9)
    t = np.asarray(cam.t, dtype=np.float64).reshape(3)
    for i in range(9):
        c.R[i] = R[i]
    for i in range(3):
        c.t[i] = t[i]
    c.fx, c.fy, c.cx, c.cy = float(cam.fx), float(cam.fy), float(cam.cx), float(cam.cy)
    c.width, c.height = int(cam.width), int(cam.height)
    c.near_plane, c.far_plane = float(cam.near), float(cam.far)
    return c


def settings_struct(settings=None) -> _Settings:
    d = dict(DEFAULT_SETTINGS)
    if settings:
        d.update(settings)
    s = _Settings()
    for k, v in d.items():
        setattr(s, k, float(v))
    return s


def num_tiles(width: int, height: int) -> int:
    return ((width + 15) // 16) * ((height + 15) // 16)


def project(means, scales, quats, sh, sh_degree, cam, settings=None, mode=MODE_F32KEY):
    """Steps 1-8 for every Gaussian. Returns a dict of arrays (see oracle.h)."""
    lib = _load()
    means, scales, quats = _f64(means), _f64(scales), _f64(quats)
    N = means.shape[0]
    K = (sh_degree + 1) ** 2
    sh = _f64(sh, (N, K, 3))
    out = dict(means2d=np.zeros((N, 2)), conics=np.zeros((N, 3)), chol=np.zeros((N, 3)),
               cov2d=np.zeros((N, 3)),
               depths=np.zeros(N), radii=np.zeros(N, np.int32), tiles=np.zeros(N, np.uint32),
               rect=np.zeros((N, 4), np.int32), colors=np.zeros((N, 3)),
               clamped=np.zeros((N, 3), np.uint8))
    cs, ss = camera_struct(cam), settings_struct(settings)
    lib.orc_project(mode, N, sh_degree, _ptr(means), _ptr(scales), _ptr(quats), _ptr(sh),
                    C.addressof(cs), C.addressof(ss),
                    *[_ptr(out[k]) for k in ("means2d", "conics", "chol", "cov2d", "depths",
                                             "radii", "tiles", "rect", "colors", "clamped")])
    return out


def bin_f32(means2d, radii, depths, width, height):
    """Steps 9-11 on the fp32 key path. Returns dict(M, offsets, keys, ids, ranges)."""
    lib = _load()
    m2 = np.ascontiguousarray(np.asarray(means2d, dtype=np.float32).reshape(-1, 2))
    rad = np.ascontiguousarray(np.asarray(radii, dtype=np.int32))
    dep = np.ascontiguousarray(np.asarray(depths, dtype=np.float32))
    N = rad.shape[0]
    T = num_tiles(width, height)
    offsets = np.zeros(N, np.uint32)
    M = lib.orc_bin_f32(N, _ptr(m2), _ptr(rad), _ptr(dep), width, height, 0,
                        _ptr(offsets), None, None, None)
    keys = np.zeros(M, np.uint64)
    ids = np.zeros(M, np.uint32)
    ranges = np.zeros((T, 2), np.uint32)
    M2 = lib.orc_bin_f32(N, _ptr(m2), _ptr(rad), _ptr(dep), width, height, M,
                         _ptr(offsets), _ptr(keys), _ptr(ids), _ptr(ranges))
    assert M2 == M
    return dict(M=int(M), offsets=offsets, keys=keys, ids=ids, ranges=ranges)


def bin_f64(means2d, radii, depths, width, height):
    lib = _load()
    m2, dep = _f64(means2d, (-1, 2)), _f64(depths)
    rad = np.ascontiguousarray(np.asarray(radii, dtype=np.int32))
    N = rad.shape[0]
    T = num_tiles(width, height)
    M = lib.orc_bin_f64(N, _ptr(m2), _ptr(rad), _ptr(dep), width, height, 0, None, None)
    ids = np.zeros(M, np.uint32)
    ranges = np.zeros((T, 2), np.uint32)
    lib.orc_bin_f64(N, _ptr(m2), _ptr(rad), _ptr(dep), width, height, M, _ptr(ids), _ptr(ranges))
    return dict(M=int(M), ids=ids, ranges=ranges)


def composite(width, height, ranges, ids, means2d, chol, opacities, colors, depths,
              background=(0.0, 0.0, 0.0), settings=None, with_margin=False):
    """Step 12, with q from the conic's Cholesky factor ``chol`` [N,3] =
    (L11, L21, L22): q = (L11 dx + L21 dy)^2 + (L22 dy)^2.
    Returns dict(image [H,W,3], final_T, last, depth, alpha[, margin])."""
    lib = _load()
    ranges = np.ascontiguousarray(np.asarray(ranges, dtype=np.uint32))
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.uint32))
    m2, ch, op, col, dep = (_f64(means2d, (-1, 2)), _f64(chol, (-1, 3)), _f64(opacities),
                            _f64(colors, (-1, 3)), _f64(depths))
    bg = _f64(background, (3,))
    H, W = height, width
    out = dict(image=np.zeros((H, W, 3)), final_T=np.zeros((H, W)),
               last=np.zeros((H, W), np.uint32), depth=np.zeros((H, W)),
               alpha=np.zeros((H, W)))
    margin = np.zeros((H, W)) if with_margin else None
    ss = settings_struct(settings)
    lib.orc_composite(W, H, _ptr(ranges), _ptr(ids), _ptr(m2), _ptr(ch), _ptr(op), _ptr(col),
                      _ptr(dep), _ptr(bg), C.addressof(ss), _ptr(out["image"]),
                      _ptr(out["final_T"]), _ptr(out["last"]), _ptr(out["depth"]),
                      _ptr(out["alpha"]), _ptr(margin))
    if with_margin:
        out["margin"] = margin
    return out


def composite_bwd(width, height, ranges, ids, means2d, chol, conics, opacities, colors,
                  dL_dimage, background=(0.0, 0.0, 0.0), settings=None, with_abs=False):
    """Step 13a. Returns dict(means2d [N,2], conics [N,3], opacities [N], colors [N,3][, abs_sum])."""
    lib = _load()
    ranges = np.ascontiguousarray(np.asarray(ranges, dtype=np.uint32))
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.uint32))
    m2, ch, con, op, col = (_f64(means2d, (-1, 2)), _f64(chol, (-1, 3)), _f64(conics, (-1, 3)),
                            _f64(opacities), _f64(colors, (-1, 3)))
    N = op.shape[0]
    g = _f64(dL_dimage, (height, width, 3))
    bg = _f64(background, (3,))
    out = dict(means2d=np.zeros((N, 2)), conics=np.zeros((N, 3)), opacities=np.zeros(N),
               colors=np.zeros((N, 3)))
    abs_sum = np.zeros((N, 9)) if with_abs else None
    ss = settings_struct(settings)
    lib.orc_composite_bwd(width, height, N, _ptr(ranges), _ptr(ids), _ptr(m2), _ptr(ch), _ptr(con),
                          _ptr(op), _ptr(col), _ptr(bg), C.addressof(ss), _ptr(g),
                          _ptr(out["means2d"]), _ptr(out["conics"]), _ptr(out["opacities"]),
                          _ptr(out["colors"]), _ptr(abs_sum))
    if with_abs:
        out["abs_sum"] = abs_sum
    return out


def project_bwd(means, scales, quats, sh, sh_degree, cam, radii, g_means2d, g_conics,
                g_colors, settings=None):
    """Step 13b. Returns dict(means [N,3], scales [N,3], quats [N,4], sh [N,K,3])."""
    lib = _load()
    means, scales, quats = _f64(means), _f64(scales), _f64(quats)
    N = means.shape[0]
    K = (sh_degree + 1) ** 2
    sh = _f64(sh, (N, K, 3))
    rad = np.ascontiguousarray(np.asarray(radii, dtype=np.int32))
    gm2, gc, gcol = _f64(g_means2d, (N, 2)), _f64(g_conics, (N, 3)), _f64(g_colors, (N, 3))
    out = dict(means=np.zeros((N, 3)), scales=np.zeros((N, 3)), quats=np.zeros((N, 4)),
               sh=np.zeros((N, K, 3)))
    cs, ss = camera_struct(cam), settings_struct(settings)
    lib.orc_project_bwd(N, sh_degree, _ptr(means), _ptr(scales), _ptr(quats), _ptr(sh),
       C.addressof(cs), C.addressof(ss), _ptr(rad), _ptr(gm2), _ptr(gc),
       _ptr(gcol), _ptr(out["means"]), _ptr(out["scales"]), _ptr(out["quats"]),
       _ptr(out["sh"]))
    return out


def project_bwd_bound(means, scales, quats, sh, sh_degree, cam, radii, s_means2d, s_conics,
                      s_colors, settings=None):
    """Bound on how much :func:`project_bwd`'s outputs move when its 2D
    gradient inputs move by at most ``s_*`` each (elementwise, same shapes
    as the gradients): e = sum_k |d out / d g2_k| s_k, exact because the
    projection backward is linear in its 2D gradients (see oracle.h).
    Returns dict like project_bwd."""
    lib = _load()
    means, scales, quats = _f64(means), _f64(scales), _f64(quats)
    N = means.shape[0]
    K = (sh_degree + 1) ** 2
    sh = _f64(sh, (N, K, 3))
    rad = np.ascontiguousarray(np.asarray(radii, dtype=np.int32))
    sm2, sc, scol = _f64(s_means2d, (N, 2)), _f64(s_conics, (N, 3)), _f64(s_colors, (N, 3))
    out = dict(means=np.zeros((N, 3)), scales=np.zeros((N, 3)), quats=np.zeros((N, 4)),
               sh=np.zeros((N, K, 3)))
    cs, ss = camera_struct(cam), settings_struct(settings)
    lib.orc_project_bwd_bound(N, sh_degree, _ptr(means), _ptr(scales), _ptr(quats), _ptr(sh),
                              C.addressof(cs), C.addressof(ss), _ptr(rad), _ptr(sm2), _ptr(sc),
                              _ptr(scol), _ptr(out["means"]), _ptr(out["scales"]),
                              _ptr(out["quats"]), _ptr(out["sh"]))
    return out


def loss_jvp(means, scales, quats, opacities, sh, sh_degree, cam, target, loss_kind=LOSS_L2,
             background=(0.0, 0.0, 0.0), settings=None, direction=None, return_image=False):
    """Whole fp64 forward + loss; with ``direction`` (dict of tangents keyed like the
    parameters) also the exact directional derivative via dual numbers.
    Returns (loss, dloss, signature, M) and, if ``return_image``, the image."""
    lib = _load()
    means, scales, quats, op = _f64(means), _f64(scales), _f64(quats), _f64(opacities)
    N = means.shape[0]
    K = (sh_degree + 1) ** 2
    sh = _f64(sh, (N, K, 3))
    tgt = _f64(target, (cam.height, cam.width, 3))
    bg = _f64(background, (3,))
    d = direction or {}
    dm = _f64(d["means"], (N, 3)) if "means" in d else None
    ds = _f64(d["scales"], (N, 3)) if "scales" in d else None
    dq = _f64(d["quats"], (N, 4)) if "quats" in d else None
    do = _f64(d["opacities"], (N,)) if "opacities" in d else None
    dsh = _f64(d["sh"], (N, K, 3)) if "sh" in d else None
    loss = C.c_double()
    dloss = C.c_double()
    sig = C.c_uint64()
    cs, ss = camera_struct(cam), settings_struct(settings)
    img = np.zeros((cam.height, cam.width, 3)) if return_image else None
    M = lib.orc_loss_jvp(N, sh_degree, _ptr(means), _ptr(scales), _ptr(quats), _ptr(op), _ptr(sh),
                         _ptr(dm), _ptr(ds), _ptr(dq), _ptr(do), _ptr(dsh), C.addressof(cs),
                         C.addressof(ss), _ptr(bg), loss_kind, _ptr(tgt), C.byref(loss),
                         C.byref(dloss), C.byref(sig), _ptr(img))
    if return_image:
        return loss.value, dloss.value, sig.value, int(M), img
    return loss.value, dloss.value, sig.value, int(M)


def set_threads(n: int) -> int:
    """Threads of the oracle's parallel loops from now on (n > 0); returns
    the current setting."""
    return int(_load().orc_set_threads(int(n)))


def rotation(quat):
    lib = _load()
    q = _f64(quat, (4,))
    R = np.zeros(9)
    lib.orc_rotation(_ptr(q), _ptr(R))
    return R.reshape(3, 3)


def cov3d(quat, scale):
    lib = _load()
    q, s = _f64(quat, (4,)), _f64(scale, (3,))
    S = np.zeros(9)
    lib.orc_cov3d(_ptr(q), _ptr(s), _ptr(S))
    return S.reshape(3, 3)


def sh_basis(sh_degree, direction):
    lib = _load()
    d = _f64(direction, (3,))
    Y = np.zeros((sh_degree + 1) ** 2)
    lib.orc_sh_basis(sh_degree, _ptr(d), _ptr(Y))
    return Y


def sh_basis_grad(sh_degree, direction):
    lib = _load()
    d = _f64(direction, (3,))
    dY = np.zeros(((sh_degree + 1) ** 2, 3))
    lib.orc_sh_basis_grad(sh_degree, _ptr(d), _ptr(dY))
    return dY


# --------------------------------------------------------------------------
# Whole-frame helpers composed from the stages above (parity mode: fp32 key
# path, fp64 values).
# --------------------------------------------------------------------------
def render(scene, cam, settings=None, background=(0.0, 0.0, 0.0), with_margin=False):
    """Forward of one frame in parity mode. ``scene`` has means, scales, quats,
    opacities, sh, sh_degree. Returns dict with 'proj', 'bins', 'raster'."""
    proj = project(scene.means, scene.scales, scene.quats, scene.sh, scene.sh_degree, cam,
                   settings, MODE_F32KEY)
    bins = bin_f32(proj["means2d"].astype(np.float32), proj["radii"],
                   proj["depths"].astype(np.float32), cam.width, cam.height)
    raster = composite(cam.width, cam.height, bins["ranges"], bins["ids"], proj["means2d"],
                       proj["chol"], scene.opacities, proj["colors"], proj["depths"],
                       background, settings, with_margin)
    return dict(proj=proj, bins=bins, raster=raster)


def loss_grad_image(image, target, loss_kind):
    """dL/dimage of the sum-reduced loss: L2 -> 2 (C - T); L1 -> sign(C - T), sign(0) = 0."""
    r = np.asarray(image, np.float64) - np.asarray(target, np.float64)
    return 2.0 * r if loss_kind == LOSS_L2 else np.sign(r)


def backward(scene, cam, fwd, dL_dimage, settings=None, background=(0.0, 0.0, 0.0),
             with_abs=False):
    """Step 13 for a forward produced by :func:`render` (or the fp64 path)."""
    proj, bins = fwd["proj"], fwd["bins"]
    g2 = composite_bwd(cam.width, cam.height, bins["ranges"], bins["ids"], proj["means2d"],
                       proj["chol"], proj["conics"], scene.opacities, proj["colors"], dL_dimage,
                       background, settings, with_abs)
    g3 = project_bwd(scene.means, scene.scales, scene.quats, scene.sh, scene.sh_degree, cam,
                     proj["radii"], g2["means2d"], g2["conics"], g2["colors"], settings)
    return dict(g2=g2, g3=g3)


def render_f64(scene, cam, settings=None, background=(0.0, 0.0, 0.0)):
    """Forward of one frame with every step in fp64 (for the gradient pins)."""
    proj = project(scene.means, scene.scales, scene.quats, scene.sh, scene.sh_degree, cam,
                   settings, MODE_F64)
    bins = bin_f64(proj["means2d"], proj["radii"], proj["depths"], cam.width, cam.height)
    raster = composite(cam.width, cam.height, bins["ranges"], bins["ids"], proj["means2d"],
                       proj["chol"], scene.opacities, proj["colors"], proj["depths"],
                       background, settings)
    return dict(proj=proj, bins=bins, raster=raster)


# --------------------------------------------------------------------------
# Densify / prune between training steps (gsplat guide, lmnt.cn/news/262699,
# section 4.1: clone by the mean-gradient magnitude, prune below opacity
# 0.005).  The selection key is the fp32 value (gx*gx + gy*gy) + gz*gz of the
# given fp32 gradients, as the step is defined to take it.
# --------------------------------------------------------------------------
def densify_prune(means, scales, quats, opacities, sh, dL_dmeans, clone_fraction=0.02,
                  min_opacity=0.005):
    """Returns dict(means, scales, quats, opacities, sh, src) for the new
    Gaussians, src = the index each one was copied from."""
    N = len(means)
    g = np.asarray(dL_dmeans, np.float32).reshape(N, 3)
    key = (g[:, 0] * g[:, 0] + g[:, 1] * g[:, 1]) + g[:, 2] * g[:, 2]  # fp32, this order
    key = np.where(np.isnan(key), np.float32(np.inf), key).astype(np.float32)
    n_clone = int(np.floor(float(np.float32(clone_fraction)) * N + 0.5))
    # n_clone largest keys; equal keys by lower index
    order = np.lexsort((np.arange(N), -key.astype(np.float64)))
    chosen = np.sort(order[:n_clone].astype(np.int64))
    src = np.concatenate([np.arange(N, dtype=np.int64), chosen])
    src = src[np.asarray(opacities, np.float32)[src] >= np.float32(min_opacity)]
    pick = lambda a: np.asarray(a)[src]
    return dict(means=pick(means), scales=pick(scales), quats=pick(quats),
                opacities=pick(opacities), sh=pick(sh), src=src)


# --------------------------------------------------------------------------
# Image loss of a training step (gsplat guide, lmnt.cn/news/262699, section
# 4.1 training loop): the mean absolute error plus 0.2 times (1 - SSIM).  The
# page calls an ssim() it does not define; this is the structural similarity
# index of Wang et al. (2004) in its usual training form: per channel, an
# 11 x 11 Gaussian window of standard deviation 1.5 normalised to sum 1,
# zero padding outside the image (one value per pixel), C1 = 0.01^2 and
# C2 = 0.03^2 (dynamic range 1), averaged over every pixel and channel.
# --------------------------------------------------------------------------
SSIM_WINDOW = 11
SSIM_SIGMA = 1.5
SSIM_C1 = 0.01 ** 2
SSIM_C2 = 0.03 ** 2


def ssim_window_1d(size=SSIM_WINDOW, sigma=SSIM_SIGMA):
    """The 1D factor of the separable window: exp(-k^2 / (2 sigma^2)) for
    k = -(size-1)/2 .. (size-1)/2, normalised to sum 1."""
    k = np.arange(size, dtype=np.float64) - (size - 1) / 2.0
    g = np.exp(-k * k / (2.0 * sigma * sigma))
    return g / g.sum()


def window_sum(plane, w1=None):
    """Windowed sum of an [H, W] plane with the 2D window w1[a] w1[b]:
    out[y, x] = sum over a, b of w1[a] w1[b] plane[y + a - r, x + b - r],
    terms outside the plane taken as 0.  One array term per window offset."""
    w1 = ssim_window_1d() if w1 is None else w1
    plane = np.asarray(plane, np.float64)
    H, W = plane.shape
    r = len(w1) // 2
    out = np.zeros((H, W))
    for a in range(len(w1)):
        dy = a - r
        y0, y1 = max(0, -dy), min(H, H - dy)
        for b in range(len(w1)):
            dx = b - r
            x0, x1 = max(0, -dx), min(W, W - dx)
            if y0 < y1 and x0 < x1:
                out[y0:y1, x0:x1] += w1[a] * w1[b] * plane[y0 + dy:y1 + dy, x0 + dx:x1 + dx]
    return out


def _channels(f, img):
    return np.stack([f(img[..., c]) for c in range(img.shape[2])], axis=2)


def ssim_stats(x, y):
    """Windowed means and second moments of [H, W, C] images: mu_x, mu_y,
    E[x^2], E[y^2], E[xy] per pixel and channel."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return (_channels(window_sum, x), _channels(window_sum, y), _channels(window_sum, x * x),
            _channels(window_sum, y * y), _channels(window_sum, x * y))


def ssim_pointwise(mx, my, sxx, syy, sxy):
    """SSIM index from the windowed statistics, and its partial derivatives
    with respect to mu_x, E[x^2] and E[xy] (mu_y, E[y^2] held fixed):
    sigma_x^2 = E[x^2] - mu_x^2, sigma_xy = E[xy] - mu_x mu_y,
    s = (2 mu_x mu_y + C1)(2 sigma_xy + C2) / ((mu_x^2 + mu_y^2 + C1)(sigma_x^2 + sigma_y^2 + C2))."""
    vx = sxx - mx * mx
    vy = syy - my * my
    cxy = sxy - mx * my
    A1 = 2.0 * mx * my + SSIM_C1
    A2 = 2.0 * cxy + SSIM_C2
    B1 = mx * mx + my * my + SSIM_C1
    B2 = vx + vy + SSIM_C2
    s = A1 * A2 / (B1 * B2)
    # dA1/dmu_x = 2 mu_y, dA2/dmu_x = -2 mu_y, dB1/dmu_x = 2 mu_x, dB2/dmu_x = -2 mu_x
    d_mu = 2.0 * my * (A2 - A1) / (B1 * B2) + 2.0 * mx * s * (1.0 / B2 - 1.0 / B1)
    d_xx = -s / B2               # dB2/dE[x^2] = 1
    d_xy = 2.0 * A1 / (B1 * B2)  # dA2/dE[xy] = 2
    return s, d_mu, d_xx, d_xy


def ssim_map(x, y):
    return ssim_pointwise(*ssim_stats(x, y))[0]


def l1_dssim_loss_grad(image, target, lam=0.2):
    """Loss = mean|x - y| + lam (1 - mean ssim(x, y)) over the n = H W C
    elements of [H, W, C] images x = image, y = target, and dLoss/dx.

    L1 part: sign(x - y) / n (sign(0) = 0).  SSIM part: with s(p) a function
    of the windowed statistics at pixel p, d(sum_p s)/dx(q) = sum_p w(p - q)
    [ds/dmu_x(p) + 2 x(q) ds/dE[x^2](p) + y(q) ds/dE[xy](p)] over the pixels
    p of the image; the window is symmetric, so this is the same
    zero-padded windowed sum applied to the three derivative maps.
    Returns (loss, gradient, parts) with parts the per-pixel pieces that
    the error scale uses."""
    x = np.asarray(image, np.float64)
    y = np.asarray(target, np.float64)
    n = x.size
    stats = ssim_stats(x, y)
    s, d_mu, d_xx, d_xy = ssim_pointwise(*stats)
    b_mu, b_xx, b_xy = (_channels(window_sum, d) for d in (d_mu, d_xx, d_xy))
    g_ssim = b_mu + 2.0 * x * b_xx + y * b_xy
    g = np.sign(x - y) / n - lam / n * g_ssim
    loss = np.abs(x - y).sum() / n + lam * (1.0 - s.sum() / n)
    return loss, g, dict(stats=stats, s=s, d=(d_mu, d_xx, d_xy), b=(b_mu, b_xx, b_xy))


def l1_dssim_errscale(image, target, lam=0.2, parts=None, delta=None):
    """First-order bound on the gradient error of an fp32 evaluation that
    forms the five windowed statistics with relative error at most delta
    each (non-negative images: sums of non-negative terms), then the three
    derivative maps and their windowed sums in fp32.  The derivative maps'
    sensitivities to the statistics are taken by central differences of
    ssim_pointwise in fp64; the windowed sums of signed maps add delta times
    the sums of their magnitudes.  Returns a map of the gradient's shape."""
    x = np.asarray(image, np.float64)
    y = np.asarray(target, np.float64)
    n = x.size
    delta = 32.0 * 2.0 ** -24 if delta is None else delta
    if parts is None:
        parts = l1_dssim_loss_grad(x, y, lam)[2]
    stats = list(parts["stats"])
    err_d = [np.zeros_like(x) for _ in range(3)]
    for k in range(5):
        h = 1e-7 * np.maximum(np.abs(stats[k]), 1e-6)
        up, dn = list(stats), list(stats)
        up[k] = stats[k] + h
        dn[k] = stats[k] - h
        dp = ssim_pointwise(*up)[1:]
        dm = ssim_pointwise(*dn)[1:]
        for j in range(3):
            sens = np.abs(dp[j] - dm[j]) / (2.0 * h)
            err_d[j] += sens * np.abs(stats[k]) * delta
    d = parts["d"]
    # fp32 rounding of the maps themselves: a few ulp of each term, d_mu
    # counted by the magnitudes of its four terms (A2 - A1 and 1/B2 - 1/B1
    # can cancel)
    mx, my, sxx, syy, sxy = stats
    A1 = 2.0 * mx * my + SSIM_C1
    A2 = 2.0 * (sxy - mx * my) + SSIM_C2
    B1 = mx * mx + my * my + SSIM_C1
    B2 = (sxx - mx * mx) + (syy - my * my) + SSIM_C2
    s = A1 * A2 / (B1 * B2)
    mag_mu = (np.abs(2.0 * my * A2 / (B1 * B2)) + np.abs(2.0 * my * A1 / (B1 * B2)) +
              np.abs(2.0 * mx * s / B2) + np.abs(2.0 * mx * s / B1))
    err_d[0] += 8.0 * 2.0 ** -24 * mag_mu
    for j in (1, 2):
        err_d[j] += 8.0 * 2.0 ** -24 * np.abs(d[j])
    blur_err = [_channels(window_sum, e) for e in err_d]
    blur_mag = [_channels(window_sum, np.abs(dj)) for dj in d]
    b = parts["b"]
    e = (blur_err[0] + 2.0 * np.abs(x) * blur_err[1] + np.abs(y) * blur_err[2]
         + delta * (blur_mag[0] + 2.0 * np.abs(x) * blur_mag[1] + np.abs(y) * blur_mag[2])
         + 4.0 * 2.0 ** -24 * (np.abs(b[0]) + 2.0 * np.abs(x * b[1]) + np.abs(y * b[2])))
    return lam / n * e


# --------------------------------------------------------------------------
# Optimiser step (gsplat guide, lmnt.cn/news/262699, section 4.2: Adam with
# one learning rate per parameter group, eps 1e-15, betas (0.9, 0.99)).  The
# rasterizer takes activated scales (exp of the stored log-scales) and
# opacities (sigmoid of the stored logits), so the step first carries their
# gradients to the stored values: d/dlog_s = d/ds * s, d/dlogit = d/do *
# o (1 - o), with s and o the values the forward used.
# --------------------------------------------------------------------------
ADAM_LR = dict(means=1.6e-4, scales=5e-3, quats=1e-3, opacities=5e-2, sh=2.5e-3)
ADAM_BETAS = (0.9, 0.99)
ADAM_EPS = 1e-15


def adam_update(p, g, m, v, step, lr, betas=ADAM_BETAS, eps=ADAM_EPS):
    """One step of Adam (Kingma and Ba, 2015): m and v are exponential moving
    averages of g and g^2; with the bias corrections 1 - beta^step,
    p -= lr m_hat / (sqrt(v_hat) + eps).  fp64; returns (p, m, v)."""
    b1, b2 = betas
    g = np.asarray(g, np.float64)
    m = b1 * np.asarray(m, np.float64) + (1.0 - b1) * g
    v = b2 * np.asarray(v, np.float64) + (1.0 - b2) * g * g
    m_hat = m / (1.0 - b1 ** step)
    v_hat = v / (1.0 - b2 ** step)
    return np.asarray(p, np.float64) - lr * m_hat / (np.sqrt(v_hat) + eps), m, v


def raw_grads(grads, act, sel):
    """Gradients with respect to the stored parameters of the Gaussians sel,
    from those with respect to the activated ones: log-scales through
    s = exp(log_s) (ds/dlog_s = s), logits through o = 1 / (1 + exp(-x))
    (do/dx = o (1 - o)); means, quaternions and SH pass unchanged."""
    s_act = np.asarray(act["scales"], np.float64)[sel]
    o_act = np.asarray(act["opacities"], np.float64)[sel]
    return dict(means=np.asarray(grads["means"], np.float64),
                log_scales=np.asarray(grads["scales"], np.float64) * s_act,
                quats=np.asarray(grads["quats"], np.float64),
                logits=np.asarray(grads["opacities"], np.float64) * o_act * (1.0 - o_act),
                sh=np.asarray(grads["sh"], np.float64))


def adam_train_step(raw, act, grads, m, v, step, rows=None, lr=None, betas=ADAM_BETAS,
                    eps=ADAM_EPS):
    """One optimiser step over the Gaussians.

    raw: dict means [N,3], log_scales [N,3], quats [N,4], logits [N], sh [N,K,3]
    (the stored parameters); act: dict scales [N,3], opacities [N] (the
    activated values the forward used); grads: gradients with respect to
    means, scales, quats, opacities, sh as the backward returns them (dense
    [N,...], or with ``rows`` one gradient row per listed Gaussian: the
    packed form, where only the listed Gaussians are updated and the others
    keep parameters and moments); m, v: dicts of the moments, shaped as raw.
    Returns (raw, act, m, v), new dicts in fp64."""
    lr = dict(ADAM_LR, **(lr or {}))
    N = len(raw["means"])
    sel = np.arange(N) if rows is None else np.asarray(rows, np.int64)
    g_raw = raw_grads(grads, act, sel)
    group = dict(means="means", log_scales="scales", quats="quats", logits="opacities", sh="sh")
    out_raw, out_m, out_v = {}, {}, {}
    for k in ("means", "log_scales", "quats", "logits", "sh"):
        p = np.array(raw[k], np.float64)
        mk = np.array(m[k], np.float64)
        vk = np.array(v[k], np.float64)
        p[sel], mk[sel], vk[sel] = adam_update(p[sel], g_raw[k], mk[sel], vk[sel], step,
                                               lr[group[k]], betas, eps)
        out_raw[k], out_m[k], out_v[k] = p, mk, vk
    out_act = dict(scales=np.array(act["scales"], np.float64),
                   opacities=np.array(act["opacities"], np.float64))
    out_act["scales"][sel] = np.exp(out_raw["log_scales"][sel])
    out_act["opacities"][sel] = 1.0 / (1.0 + np.exp(-out_raw["logits"][sel]))
    return out_raw, out_act, out_m, out_v
