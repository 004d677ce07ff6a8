"""CPU checks of the C-ABI library: it loads, exports every entry point the
header declares, and rejects invalid arguments on the host before touching
the GPU (no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

from differentiable_rasterization_amd import raster

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsraster.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^GS_API [^;(]*?\b(gs_\w+)\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(raster.LIB_PATH):
        from differentiable_rasterization_amd import build
        build.build()
    return raster.load()


def test_header_declares_the_five_stages():
    names = declared_functions()
    for n in ("gs_project_fwd", "gs_bin_and_sort", "gs_rasterize_fwd", "gs_rasterize_bwd",
              "gs_project_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(raster.EXPORTED)


def test_only_the_api_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", raster.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == declared_functions()


def test_default_settings_and_tiles(lib):
    s = raster.default_settings()
    f = lambda x: float(C.c_float(x).value)
    assert (s.eps2d, s.alpha_min, s.alpha_max, s.T_min, s.fov_clamp, s.sh_offset) == \
        (f(0.3), f(1 / 255), f(0.99), f(1e-4), f(1.3), f(0.5))
    assert raster.num_tiles(1920, 1080) == 120 * 68
    assert raster.num_tiles(64, 64) == 16
    assert raster.num_tiles(17, 1) == 2
    assert raster.num_tiles(0, 10) == 0


def test_workspace_size_grows_with_capacity(lib):
    a = raster.gs_bin_and_sort_workspace_size(1000, 10_000, 64, 64)
    b = raster.gs_bin_and_sort_workspace_size(1000, 100_000, 64, 64)
    assert 0 < a < b
    assert raster.gs_bin_and_sort_workspace_size(-1, 10, 64, 64) == 0


def _cam(width=64, height=64):
    from differentiable_rasterization_amd import scenes
    return raster.make_camera(scenes.identity_camera(width, height, 64.0))


def _call_project(lib, N=4, ld=4, deg=0, cam=None, st=None, null_means=False):
    dummy = C.c_void_p(16)  # never dereferenced: validation fails first
    cam = cam if cam is not None else _cam()
    st = st if st is not None else raster.default_settings()
    return lib.gs_project_fwd(N, ld, deg, None if null_means else dummy, dummy, dummy, dummy,
                              C.byref(cam), C.byref(st), *([dummy] * 7), None)


@pytest.mark.parametrize("kw", [dict(N=-1), dict(N=5, ld=4), dict(deg=4), dict(deg=-1),
                                dict(null_means=True)])
def test_project_fwd_rejects_bad_arguments(lib, kw):
    assert _call_project(lib, **kw) == raster.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_last_error().decode()


def test_project_fwd_rejects_bad_camera_and_settings(lib):
    cam = _cam()
    cam.width = 0
    assert _call_project(lib, cam=cam) == raster.GS_ERR_INVALID_ARGUMENT
    cam = _cam()
    cam.near_plane = 0.0
    assert _call_project(lib, cam=cam) == raster.GS_ERR_INVALID_ARGUMENT
    st = raster.default_settings(alpha_max=1.5)
    assert _call_project(lib, st=st) == raster.GS_ERR_INVALID_ARGUMENT
    st = raster.default_settings(T_min=0.0)
    assert _call_project(lib, st=st) == raster.GS_ERR_INVALID_ARGUMENT


def test_bin_and_sort_rejects_bad_arguments(lib):
    dummy = C.c_void_p(256)
    M = C.c_uint64(0)
    base = dict(N=4, ld=4, W=64, H=64, cap=100, ws=dummy, wsb=1 << 30)

    def call(**kw):
        a = dict(base, **kw)
        return lib.gs_bin_and_sort(a["N"], a["ld"], dummy, dummy, dummy, dummy, a["W"], a["H"],
                                   dummy, a["cap"], C.byref(M), dummy, dummy, dummy, a["ws"],
                                   a["wsb"], None)
    assert call(ld=3) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(W=0) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(ws=C.c_void_p(260)) == raster.GS_ERR_INVALID_ARGUMENT  # misaligned
    assert call(wsb=16) == raster.GS_ERR_INVALID_ARGUMENT             # too small
    assert call(cap=1 << 30) == raster.GS_ERR_INVALID_ARGUMENT


def test_bin_and_sort_noalloc_rejects_bad_and_oversized_arguments(lib):
    dummy = C.c_void_p(256)
    M = C.c_uint64(0)
    base = dict(N=4, ld=4, W=64, H=64, cap=100)

    def call(**kw):
        a = dict(base, **kw)
        return lib.gs_bin_and_sort_noalloc(a["N"], a["ld"], dummy, dummy, dummy, dummy, a["W"],
                                           a["H"], dummy, a["cap"], C.byref(M), dummy, dummy,
                                           dummy, None)
    assert call(ld=3) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(W=0) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(cap=1 << 30) == raster.GS_ERR_INVALID_ARGUMENT
    # scratch beyond the library's 64 MiB: refused on the host, with the sizes
    big = 6_000_000
    assert raster.gs_bin_and_sort_workspace_size(4, big, 64, 64) > 64 << 20
    assert call(cap=big) == raster.GS_ERR_INVALID_ARGUMENT
    assert b"more than its 67108864" in lib.gs_last_error()


def _planes(dummy, **kw):
    """means2d, conics, chol, opacities, colors, radii (overridable by name)."""
    names = ("means2d", "conics", "chol", "opacities", "colors", "radii")
    return [kw.get(n, dummy) for n in names]


def _grads(dummy, **kw):
    names = ("g_means2d", "g_conics", "g_opacities", "g_colors")
    return [kw.get(n, dummy) for n in names] + [kw.get("g_abs", None)]


def test_raster_and_loss_reject_bad_arguments(lib):
    dummy = C.c_void_p(256)
    st = raster.default_settings()
    bg = (C.c_float * 3)(0, 0, 0)
    assert lib.gs_rasterize_workspace_size(10) >= 640
    assert lib.gs_rasterize_workspace_size(-1) == 0

    def fwd(ranges=dummy, ids=dummy, depths=None, out_depth=None, ws=dummy, wsb=1 << 20, **kw):
        return lib.gs_rasterize_fwd(4, 4, 64, 64, ranges, None, ids, *_planes(dummy, **kw),
                                    depths, bg, C.byref(st), dummy, dummy, dummy, out_depth,
                                    None, ws, wsb, None, None)
    assert fwd(ranges=None) == raster.GS_ERR_INVALID_ARGUMENT      # no tile ranges
    assert fwd(ids=None) == raster.GS_ERR_INVALID_ARGUMENT         # ids needed when N > 0
    assert fwd(chol=None) == raster.GS_ERR_INVALID_ARGUMENT        # every plane is read
    assert fwd(opacities=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert fwd(radii=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert fwd(out_depth=dummy) == raster.GS_ERR_INVALID_ARGUMENT  # depth output needs depths
    assert fwd(ws=None) == raster.GS_ERR_INVALID_ARGUMENT          # staging workspace
    assert fwd(ws=C.c_void_p(260)) == raster.GS_ERR_INVALID_ARGUMENT  # misaligned
    assert fwd(wsb=255) == raster.GS_ERR_INVALID_ARGUMENT          # 4 records need 256 bytes

    def bwd(offsets=dummy, M=10, cap=10, partials=dummy, staged=0, acc=0, wsb=1 << 20, **kw):
        pl = {k: v for k, v in kw.items() if not k.startswith("g_")}
        gr = {k: v for k, v in kw.items() if k.startswith("g_")}
        return lib.gs_rasterize_bwd(4, 4, 64, 64, dummy, None, dummy, *_planes(dummy, **pl),
                                    offsets, dummy, M, bg, C.byref(st), dummy, dummy, dummy,
                                    dummy, wsb, staged, partials, cap, *_grads(dummy, **gr), acc,
                                    None, None)
    assert bwd(offsets=None) == raster.GS_ERR_INVALID_ARGUMENT     # offsets needed
    assert bwd(cap=9) == raster.GS_ERR_INVALID_ARGUMENT            # slots < instances
    assert bwd(partials=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert bwd(partials=C.c_void_p(80)) == raster.GS_ERR_INVALID_ARGUMENT  # misaligned
    assert bwd(g_conics=None) == raster.GS_ERR_INVALID_ARGUMENT    # every 2D plane is written
    assert bwd(g_opacities=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert bwd(staged=2) == raster.GS_ERR_INVALID_ARGUMENT
    assert bwd(acc=3) == raster.GS_ERR_INVALID_ARGUMENT
    assert bwd(wsb=16) == raster.GS_ERR_INVALID_ARGUMENT
    r = lib.gs_project_bwd(4, 4, 0, dummy, dummy, dummy, dummy, C.byref(_cam()), C.byref(st),
                           dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 2, None)
    assert r == raster.GS_ERR_INVALID_ARGUMENT  # accumulate must be 0/1
    r = lib.gs_project_bwd(4, 4, 0, dummy, dummy, dummy, dummy, C.byref(_cam()), C.byref(st),
                           dummy, dummy, None, dummy, dummy, dummy, dummy, dummy, 0, None)
    assert r == raster.GS_ERR_INVALID_ARGUMENT  # the conic gradients are read
    assert lib.gs_image_loss_grad(2, 10, dummy, dummy, dummy, None, None) == \
        raster.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_image_loss_grad(0, -1, dummy, dummy, dummy, None, None) == \
        raster.GS_ERR_INVALID_ARGUMENT


def test_packed_calls_reject_bad_arguments(lib):
    dummy = C.c_void_p(256)
    st = raster.default_settings()
    bg = (C.c_float * 3)(0, 0, 0)
    counts = (C.c_uint64 * 2)()

    def bas(N=4, ld=4, vis=dummy, cnt=counts):
        return lib.gs_bin_and_sort_packed(N, ld, dummy, dummy, dummy, dummy, 64, 64, dummy, 100,
                                          cnt, dummy, dummy, dummy, vis, dummy, 1 << 30, None)
    assert bas(vis=None) == raster.GS_ERR_INVALID_ARGUMENT   # the visible list is required
    assert bas(cnt=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert bas(ld=3) == raster.GS_ERR_INVALID_ARGUMENT

    def rbwd(V=2, ldv=2, vis=dummy, **gr):
        return lib.gs_rasterize_bwd_packed(4, 4, 64, 64, dummy, None, dummy, *_planes(dummy),
                                           dummy, dummy, 10, vis, V, ldv, bg, C.byref(st), dummy,
                                           dummy, dummy, dummy, 1 << 20, 0, dummy, 10,
                                           *_grads(dummy, **gr), 0, None, None)
    assert rbwd(V=5, ldv=5) == raster.GS_ERR_INVALID_ARGUMENT  # more rows than Gaussians
    assert rbwd(V=-1) == raster.GS_ERR_INVALID_ARGUMENT
    assert rbwd(ldv=1) == raster.GS_ERR_INVALID_ARGUMENT       # ldv < num_visible
    assert rbwd(vis=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert rbwd(g_colors=None) == raster.GS_ERR_INVALID_ARGUMENT

    def pbwd(V=2, N=4, ldv=2, vis=dummy, acc=0, deg=3):
        return lib.gs_project_bwd_packed(V, vis, N, N, ldv, deg, dummy, dummy, dummy, dummy,
                                         C.byref(_cam()), C.byref(st), dummy, dummy, dummy,
                                         dummy, dummy, dummy, dummy, dummy, acc, None)
    assert pbwd(ldv=1) == raster.GS_ERR_INVALID_ARGUMENT      # ldv < num_visible
    assert pbwd(V=5) == raster.GS_ERR_INVALID_ARGUMENT
    assert pbwd(vis=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert pbwd(acc=2) == raster.GS_ERR_INVALID_ARGUMENT
    assert pbwd(deg=4) == raster.GS_ERR_INVALID_ARGUMENT
    assert pbwd(V=0, ldv=0, vis=None) == raster.GS_OK         # empty list: nothing to launch


def test_training_step_calls_reject_bad_arguments(lib):
    dummy = C.c_void_p(256)
    ws = lib.gs_l1_dssim_workspace_size(64, 48)
    assert ws >= 9 * 64 * 48 * 4
    assert lib.gs_l1_dssim_workspace_size(0, 48) == 0

    def loss(W=64, H=48, lam=0.2, img=dummy, g=C.c_void_p(512), wsp=dummy, wsb=ws):
        return lib.gs_l1_dssim_loss_grad(W, H, img, dummy, C.c_float(lam), g, None, wsp, wsb,
                                         None)
    assert loss(W=0) == raster.GS_ERR_INVALID_ARGUMENT
    assert loss(lam=-0.1) == raster.GS_ERR_INVALID_ARGUMENT
    assert loss(lam=float("nan")) == raster.GS_ERR_INVALID_ARGUMENT
    assert loss(img=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert loss(g=dummy) == raster.GS_ERR_INVALID_ARGUMENT        # aliases the image
    assert loss(wsp=C.c_void_p(260)) == raster.GS_ERR_INVALID_ARGUMENT
    assert loss(wsb=ws - 1) == raster.GS_ERR_INVALID_ARGUMENT

    cfg = lib.gs_default_adam_config()
    assert abs(cfg.lr_means - 1.6e-4) < 1e-10 and abs(cfg.lr_opacities - 5e-2) < 1e-9
    assert abs(cfg.beta2 - 0.99) < 1e-7 and abs(cfg.eps - 1e-15) < 1e-22

    def adam(N=10, step=1, deg=3, c=cfg, moment=dummy):
        return lib.gs_adam_step(N, N, deg, step, C.byref(c), *([dummy] * 12), moment, dummy,
                                None)
    assert adam(step=0) == raster.GS_ERR_INVALID_ARGUMENT
    assert adam(deg=4) == raster.GS_ERR_INVALID_ARGUMENT
    assert adam(moment=None) == raster.GS_ERR_INVALID_ARGUMENT
    bad = raster.gs_adam_config.from_buffer_copy(cfg)
    bad.beta1 = 1.0
    assert adam(c=bad) == raster.GS_ERR_INVALID_ARGUMENT
    bad = raster.gs_adam_config.from_buffer_copy(cfg)
    bad.lr_sh = -1.0
    assert adam(c=bad) == raster.GS_ERR_INVALID_ARGUMENT
    assert adam(N=0) == raster.GS_OK                               # nothing to launch

    def adam_p(V=3, ldv=3, vis=dummy):
        return lib.gs_adam_step_packed(V, vis, ldv, 10, 10, 3, 1, C.byref(cfg),
                                       *([dummy] * 14), None)
    assert adam_p(V=11, ldv=11) == raster.GS_ERR_INVALID_ARGUMENT
    assert adam_p(ldv=2) == raster.GS_ERR_INVALID_ARGUMENT
    assert adam_p(vis=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert adam_p(V=0, ldv=0, vis=None) == raster.GS_OK


def test_batched_calls_reject_bad_arguments(lib):
    dummy = C.c_void_p(256)
    st = raster.default_settings()
    cams = (raster.gs_camera * 9)(*([_cam()] * 9))

    def proj(n=2, ld=10):
        return lib.gs_project_fwd_batched(n, cams, 10, ld, 0, *([dummy] * 4), C.byref(st),
                                          *([dummy] * 7), None)
    assert proj(n=0) == raster.GS_ERR_INVALID_ARGUMENT
    assert proj(n=9) == raster.GS_ERR_INVALID_ARGUMENT
    assert proj(ld=9) == raster.GS_ERR_INVALID_ARGUMENT           # ld < N
    assert proj(ld=1 << 29, n=4) == raster.GS_ERR_INVALID_ARGUMENT  # 4 ld >= 2^31
    other = (raster.gs_camera * 2)(_cam(64, 64), _cam(32, 64))
    assert lib.gs_project_fwd_batched(2, other, 10, 10, 0, *([dummy] * 4), C.byref(st),
                                      *([dummy] * 7), None) == raster.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_bin_and_sort_batched_workspace_size(0, 10, 100, 64, 64) == 0
    assert lib.gs_bin_and_sort_batched_workspace_size(2, 10, 100, 64, 64) > 0
    M = C.c_uint64(0)
    r = lib.gs_bin_and_sort_batched(9, 10, *([dummy] * 4), 64, 64, dummy, 100, C.byref(M),
                                    dummy, dummy, dummy, dummy, 1 << 30, None)
    assert r == raster.GS_ERR_INVALID_ARGUMENT
    r = lib.gs_bin_and_sort_batched(2, 10, *([dummy] * 4), 64, 64, dummy, 100, C.byref(M),
                                    dummy, dummy, dummy, dummy, 16, None)
    assert r == raster.GS_ERR_INVALID_ARGUMENT                       # workspace too small
    bg = (C.c_float * 3)(0, 0, 0)

    def fwd(n=2, ranges=dummy, wsb=1 << 20):
        return lib.gs_rasterize_fwd_batched(n, 10, 64, 64, ranges, None, dummy, *_planes(dummy),
                                            None, bg, C.byref(st), dummy, dummy, dummy, None,
                                            None, dummy, wsb, None, None)
    assert fwd(ranges=None) == raster.GS_ERR_INVALID_ARGUMENT        # no tile ranges
    assert fwd(n=9) == raster.GS_ERR_INVALID_ARGUMENT
    assert fwd(wsb=2 * 10 * 64 - 1) == raster.GS_ERR_INVALID_ARGUMENT  # 20 records

    def bwd(n=2, M=10, cap=10):
        return lib.gs_rasterize_bwd_batched(n, 10, 64, 64, dummy, None, dummy, *_planes(dummy),
                                            dummy, dummy, M, bg, C.byref(st), dummy, dummy,
                                            dummy, dummy, 1 << 20, 1, dummy, cap,
                                            *_grads(dummy), 0, None, None)
    assert bwd(n=9) == raster.GS_ERR_INVALID_ARGUMENT                # too many cameras
    assert bwd(M=11) == raster.GS_ERR_INVALID_ARGUMENT               # partials too small

    def pbwd(n=2, acc=0, op_cams=dummy, op=dummy):
        return lib.gs_project_bwd_batched(n, cams, 10, 10, 0, *([dummy] * 4), C.byref(st),
                                          dummy, dummy, dummy, dummy, op_cams, dummy, dummy,
                                          dummy, op, dummy, acc, None)
    assert pbwd(acc=2) == raster.GS_ERR_INVALID_ARGUMENT             # accumulate 0/1
    assert pbwd(n=0) == raster.GS_ERR_INVALID_ARGUMENT
    assert pbwd(op=None) == raster.GS_ERR_INVALID_ARGUMENT           # the opacity pair together


def test_fused_loss_rejects_bad_arguments(lib):
    dummy, other = C.c_void_p(256), C.c_void_p(512)
    st = raster.default_settings()
    bg = (C.c_float * 3)(0, 0, 0)

    def call(kind=1, target=other, dl=C.c_void_p(768)):
        return lib.gs_rasterize_fwd_loss(4, 4, 64, 64, dummy, None, dummy, *_planes(dummy), None,
                                         bg, C.byref(st), kind, target, dummy, dummy, dummy, None,
                                         None, dl, None, dummy, 1 << 20, None, None)
    assert call(kind=2) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(target=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(dl=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(dl=dummy) == raster.GS_ERR_INVALID_ARGUMENT     # aliases the image
    assert call(dl=other) == raster.GS_ERR_INVALID_ARGUMENT     # aliases the target


def test_batched_fused_loss_rejects_bad_arguments(lib):
    dummy, other = C.c_void_p(256), C.c_void_p(512)
    st = raster.default_settings()
    bg = (C.c_float * 3)(0, 0, 0)

    def call(cams=2, kind=1, target=other, dl=C.c_void_p(768), ranges=dummy):
        return lib.gs_rasterize_fwd_loss_batched(cams, 10, 64, 64, ranges, None, dummy,
                                                 *_planes(dummy), None, bg, C.byref(st), kind,
                                                 target, dummy, dummy, dummy, None, None, dl,
                                                 None, dummy, 1 << 20, None, None)
    assert call(cams=0) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(cams=9) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(kind=2) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(ranges=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(target=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(dl=None) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(dl=dummy) == raster.GS_ERR_INVALID_ARGUMENT     # aliases the image
    assert call(dl=other) == raster.GS_ERR_INVALID_ARGUMENT     # aliases the target


def test_tile_order_rejects_bad_arguments(lib):
    dummy, other = C.c_void_p(64), C.c_void_p(128)
    assert lib.gs_tile_order(0, 64, 64, dummy, other, None) == raster.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_tile_order(9, 64, 64, dummy, other, None) == raster.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_tile_order(1, 0, 64, dummy, other, None) == raster.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_tile_order(1, 64, 64, None, other, None) == raster.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_tile_order(1, 64, 64, dummy, None, None) == raster.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_tile_order(1, 64, 64, dummy, dummy, None) == raster.GS_ERR_INVALID_ARGUMENT


def test_densify_rejects_bad_arguments(lib):
    dummy = C.c_void_p(256)
    n_out = C.c_int64(0)

    def call(N=10, ld=10, deg=0, frac=0.2, ld_out=12, ws=dummy, wsb=1 << 30):
        return lib.gs_densify_prune(N, ld, deg, dummy, dummy, dummy, dummy, dummy, dummy,
                                    C.c_float(frac), C.c_float(0.005), ld_out, dummy, dummy,
                                    dummy, dummy, dummy, C.byref(n_out), ws, wsb, None)
    assert call(frac=1.5) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(frac=-0.1) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(ld_out=11) == raster.GS_ERR_INVALID_ARGUMENT   # 10 + 2 clones
    assert call(deg=4) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(ws=C.c_void_p(260)) == raster.GS_ERR_INVALID_ARGUMENT
    assert call(wsb=8) == raster.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_densify_prune_workspace_size(10, C.c_float(2.0)) == 0
    assert lib.gs_densify_prune_workspace_size(1000, C.c_float(0.02)) > 0


def test_status_strings(lib):
    assert lib.gs_status_string(0) == b"GS_OK"
    assert lib.gs_status_string(2) == b"GS_ERR_CAPACITY"


def test_load_refuses_a_library_built_from_other_sources(lib, monkeypatch):
    """The library records the hash of the sources it was built from; a tree
    whose sources differ is refused rather than run with a stale build."""
    from differentiable_rasterization_amd import build
    monkeypatch.setattr(raster, "_lib", None)
    monkeypatch.setattr(build, "source_hash", lambda: "0" * 64)
    with pytest.raises(RuntimeError, match="current csrc"):
        raster.load()
