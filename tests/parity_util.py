"""Helpers shared by the GPU parity tests: run a frame through the HIP
library and through the CPU oracle on the same seeded inputs, and compare.

Tolerances (fp32 GPU against the oracle's fp32 key path + fp64 values):
  * integer outputs and the fp32 key path (means2d, conics, depths, radii,
    tiles touched, offsets, keys, ids, ranges): bit-exact;
  * pixels (image, final_T): max |diff| <= 1e-4;
  * gradients: |g_gpu - g_oracle| <= max(1e-3 |g_oracle|, 1e-5).
Mismatches are never hidden by widening these; they are classified, and
every class is counted and bounded by the checks below:
  * threshold flip: a pixel whose oracle decisions include one within
    FLIP_REL relative distance of its threshold (alpha vs alpha_min, o G vs
    alpha_max, T' vs T_min; the oracle's margin), where fp32 exp and rounding
    on the GPU may legitimately decide the other way.  Gradients of the
    Gaussians such a pixel evaluates (its tile's list up to one past the
    later of the two sides' last blended entries) inherit the exemption;
  * cancellation (compositing gradients): a sum of per-pixel terms of mixed
    sign whose error stays within COND_K * u * sum|terms| (u = 2^-24; each
    term carries the rounding of T recovered through its tile's layers plus
    the summation tree);
  * inherited (projection gradients): within the exact bound on what the
    projection backward, linear in its 2D gradients, inherits from 2D inputs
    known to within s (their fp32 rounding, or the 2D tolerance end to end),
    plus the rounding of the fp32 output.
"""
from __future__ import annotations

import numpy as np

import oracle

PIX_TOL = 1e-4
G_REL, G_ABS = 1e-3, 1e-5
FLIP_REL = 2e-4
EPS32 = 2.0 ** -24
COND_K = 256


def bounded(count, checked, rel=1e-3, floor=4):
    """Exemption counts are bounded: at most rel of the elements checked,
    plus a small floor for tiny cases."""
    return count <= rel * checked + floor


def torch_cuda():
    import torch
    return torch


def gpu_frame(scene, cam, *, ld=None, settings=None, background=(0.0, 0.0, 0.0),
              loss_kind=None, target=None, backward=True, depth_alpha=False, capacity=None,
              dL_dimage=None, absgrad=False, packed=False, schedule=True):
    """Run the five stages on the GPU; returns numpy arrays in the natural
    [N, ...] layout plus the raw Frame.  With ``packed`` the packed calls
    run, and their rows are scattered back to the [N, ...] layout (zeros off
    the visible list); ``vis_ids`` and ``V`` are returned too.  ``schedule``
    selects the longest-tile-first compositing order (Frame's default)."""
    import torch
    from differentiable_rasterization_amd import raster
    g = raster.Gaussians.from_scene(scene, ld=ld)
    st = raster.default_settings(**(settings or {}))
    fr = raster.Frame(g.ld, scene.sh_degree, cam.width, cam.height, capacity=capacity,
                      settings=st, background=background, with_depth_alpha=depth_alpha,
                      packed=packed, schedule=schedule)
    fr.forward(g, cam)
    out = {}
    if backward:
        if dL_dimage is not None:
            dl = torch.from_numpy(np.ascontiguousarray(dL_dimage, np.float32)).cuda()
            fr.backward(g, dl, absgrad=absgrad)
        else:
            tgt = torch.from_numpy(np.ascontiguousarray(target, np.float32)).cuda()
            fr.loss_grad(tgt, 0 if loss_kind == "l2" else 1)
            fr.backward(g, absgrad=absgrad)
    torch.cuda.synchronize()
    N = scene.n
    T = lambda t, P=None: t[:, :N].T.contiguous().cpu().numpy() if t.dim() == 2 else t[:N].cpu().numpy()
    M = fr.M
    out.update(
        means2d=T(fr.means2d), conics=T(fr.conics), chol=T(fr.chol), depths=T(fr.depths),
        radii=T(fr.radii), colors=T(fr.colors), tiles=T(fr.tiles).view(np.uint32),
        offsets=fr.offsets[:N].cpu().numpy().view(np.uint32), M=M,
        keys=fr.keys[:M].cpu().numpy().view(np.uint64), ids=fr.ids[:M].cpu().numpy().view(np.uint32),
        ranges=fr.ranges.cpu().numpy().view(np.uint32), image=fr.image.cpu().numpy(),
        final_T=fr.final_T.cpu().numpy(), last=fr.last_idx.cpu().numpy().view(np.uint32))
    if depth_alpha:
        out.update(depth=fr.out_depth.cpu().numpy(), alpha=fr.out_alpha.cpu().numpy())
    if packed:
        vis_ids = fr.vis_ids[:fr.V].cpu().numpy().view(np.uint32).copy()
        out.update(vis_ids=vis_ids, V=fr.V)
        rows = vis_ids.astype(np.int64)

        def unpack(t):
            a = (t[:, :fr.V].T.contiguous() if t.dim() == 2 else t[:fr.V]).cpu().numpy()
            d = np.zeros((N,) + a.shape[1:], a.dtype)
            d[rows] = a
            return d
        T = unpack
    if backward:
        K = (scene.sh_degree + 1) ** 2
        out.update(dL_dimage=fr.dL_dimage.cpu().numpy() if dL_dimage is None else dL_dimage,
                   loss=float(fr.loss.cpu().numpy()[0]),
                   g_means2d=T(fr.g_means2d), g_conics=T(fr.g_conics),
                   g_opac2d=T(fr.g_opacities), g_colors=T(fr.g_colors),
                   g_absgrad=T(fr.g_abs) if absgrad else np.zeros((N, 2), np.float32),
                   g_opacities=T(fr.g_opacities),
                   g_means=T(fr.g_means), g_scales=T(fr.g_scales), g_quats=T(fr.g_quats),
                   g_sh=T(fr.g_sh).reshape(N, K, 3))
    out["frame"] = fr
    return out


def grad2d_rows(fr, n, absgrad=False):
    """A Frame's 2D gradient planes as [n, 9] rows (u, v, A, B, C, opacity,
    r, g, b; [n, 11] with the absolute sums), for bitwise comparisons."""
    import torch
    planes = [fr.g_means2d, fr.g_conics, fr.g_opacities[None], fr.g_colors]
    if absgrad:
        planes.append(fr.g_abs)
    return torch.cat([p[:, :n] for p in planes], 0).T.contiguous()


def gpu_project_bwd(scene, cam, g2, ld=None, vis_ids=None, settings=None):
    """GPU projection backward fed the given 2D gradients (dict with means2d
    [N,2], conics [N,3], colors [N,3]), rounded to fp32 into its 2D gradient
    planes; returns the 3D gradients in [N, ...] layout.  With ``vis_ids``
    the packed call runs over that list (rows in list order) and its rows are
    scattered back (zeros off the list)."""
    import torch
    from differentiable_rasterization_amd import raster
    N = scene.n
    g = raster.Gaussians.from_scene(scene, ld=ld)
    fr = raster.Frame(g.ld, scene.sh_degree, cam.width, cam.height, capacity=1024,
                      packed=vis_ids is not None,
                      settings=raster.default_settings(**(settings or {})))
    fr.project(g, cam)
    rows = np.arange(N) if vis_ids is None else np.asarray(vis_ids, np.int64)
    V = len(rows)

    def put(plane, a):
        a = np.asarray(a, np.float32).reshape(N, -1)[rows]
        plane.zero_()
        if V:
            plane[:, :V].copy_(torch.from_numpy(np.ascontiguousarray(a.T)))
    put(fr.g_means2d, g2["means2d"])
    put(fr.g_conics, g2["conics"])
    put(fr.g_colors, g2["colors"])
    if vis_ids is not None:
        fr.V = V
        if V:
            fr.vis_ids[:V].copy_(torch.from_numpy(rows.astype(np.int32)))
    fr.project_backward(g)
    torch.cuda.synchronize()
    K = (scene.sh_degree + 1) ** 2

    def T(t):
        a = t[:, :V].T.contiguous().cpu().numpy()
        d = np.zeros((N,) + a.shape[1:], a.dtype)
        d[rows] = a
        return d
    return dict(radii=fr.radii[:N].cpu().numpy(), g_means=T(fr.g_means), g_scales=T(fr.g_scales),
                g_quats=T(fr.g_quats), g_sh=T(fr.g_sh).reshape(N, K, 3))


def assert_bits_equal(a, b, what):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype.kind == "f":
        a = a.astype(np.float32).view(np.uint32)
        b = b.astype(np.float32).view(np.uint32)
    bad = np.nonzero(a != b)
    assert bad[0].size == 0, "%s: %d mismatches, first at %s" % (what, bad[0].size,
                                                                 tuple(x[0] for x in bad))


def flip_rows(margin, width, height, ranges, ids, last_or, last_gpu, extra_pixels=None):
    """Gaussians a near-threshold decision can reach.  For every pixel whose
    oracle margin is below FLIP_REL (and every extra pixel), the entries of
    its tile's list up to one past the later of the two sides' last blended
    entries: a decision that flips at that pixel changes the terms of those
    entries only.  Returns (rows int64 array, number of such pixels)."""
    near = margin < FLIP_REL
    if extra_pixels is not None:
        near = near | extra_pixels
    gx = (width + 15) // 16
    ys, xs = np.nonzero(near)
    if ys.size == 0:
        return np.zeros(0, np.int64), 0
    tiles = (ys // 16) * gx + (xs // 16)
    reach = np.maximum(last_or[ys, xs], last_gpu[ys, xs]).astype(np.int64) + 1
    parts = []
    for t, n in zip(tiles.tolist(), reach.tolist()):
        a, b = int(ranges[t][0]), int(ranges[t][1])
        parts.append(ids[a:min(b, a + n)])
    return np.unique(np.concatenate(parts).astype(np.int64)), int(ys.size)


def compare_pixels(gpu_img, or_img, margin, name="image"):
    """Returns (n_fail_unexplained, n_flip_exempt, max_abs_diff_nonexempt)."""
    d = np.abs(np.asarray(gpu_img, np.float64) - or_img)
    if d.ndim == 3:
        d = d.max(axis=2)
    fail = d > PIX_TOL
    flip = fail & (margin < FLIP_REL)
    unexplained = fail & ~flip
    md = float(d[~flip].max()) if (~flip).any() else 0.0
    return int(unexplained.sum()), int(flip.sum()), md, np.argwhere(unexplained)[:5]


def compare_grad(g_gpu, g_or, abs_sum=None, exempt_rows=None, name="grad"):
    """Per-element |diff| <= max(G_REL |g|, G_ABS); classify the rest.
    Returns dict(fail, flip, cond, checked, worst)."""
    g_gpu = np.asarray(g_gpu, np.float64).reshape(g_or.shape[0], -1)
    g_or = np.asarray(g_or, np.float64).reshape(g_or.shape[0], -1)
    err = np.abs(g_gpu - g_or)
    tol = np.maximum(G_REL * np.abs(g_or), G_ABS)
    bad = err > tol
    flip = np.zeros_like(bad)
    if exempt_rows is not None and len(exempt_rows):
        rows = np.asarray(exempt_rows, dtype=np.int64)
        flip[rows] = bad[rows]
    cond = np.zeros_like(bad)
    if abs_sum is not None:
        a = np.asarray(abs_sum, np.float64).reshape(bad.shape)
        cond = bad & ~flip & (err <= COND_K * EPS32 * a)
    fail = bad & ~flip & ~cond
    worst = float((err / tol)[~flip & ~cond].max()) if (~flip & ~cond).any() else 0.0
    where = np.argwhere(fail)[:5]
    return dict(fail=int(fail.sum()), flip=int(flip.sum()), cond=int(cond.sum()),
                checked=int(bad.size), worst=worst, where=where.tolist(), name=name)


# ---------------------------------------------------------------------------
# One parity case: both sides run the same seeded scene and camera; the
# oracle's own loss gradient and 2D gradients also drive the GPU's backward
# stages in isolation (data flows from the oracle to the GPU only).
# ---------------------------------------------------------------------------
def run_parity_case(name, scene, cam, loss, bg, target, backward=True, depth_alpha=False,
                    ld=None, packed=False, settings=None):
    """Both whole paths on one case; ``settings`` (a dict of gs_settings
    fields, default values elsewhere) goes to both sides."""
    import time
    t0 = time.time()
    print("\n[parity] case %s" % name, flush=True)
    gpu = gpu_frame(scene, cam, background=bg, loss_kind=loss, target=target,
                    backward=backward, depth_alpha=depth_alpha, ld=ld, packed=packed,
                    settings=settings)
    t1 = time.time()
    orc = oracle.render(scene, cam, settings, bg, with_margin=True)
    r = dict(name=name, scene=scene, cam=cam, loss=loss, bg=bg, target=target, gpu=gpu, orc=orc,
             settings=settings)
    if backward:
        kind = oracle.LOSS_L2 if loss == "l2" else oracle.LOSS_L1
        dl = oracle.loss_grad_image(orc["raster"]["image"], target, kind).astype(np.float32)
        bw = oracle.backward(scene, cam, orc, dl.astype(np.float64), settings, bg, with_abs=True)
        r.update(dl=dl, bw=bw)
    t2 = time.time()
    if backward:
        # the isolated run also exercises the absolute-gradient variant
        r["gpu_iso"] = gpu_frame(scene, cam, background=bg, dL_dimage=r["dl"], ld=ld,
                                 absgrad=True, packed=packed, settings=settings)
        # packed: the projection backward runs over the oracle's visible list
        vis_ids = np.flatnonzero(orc["proj"]["tiles"] > 0) if packed else None
        r["gpu_pbwd"] = gpu_project_bwd(scene, cam, r["bw"]["g2"], ld=ld, vis_ids=vis_ids,
                                        settings=settings)
    print("[parity] %s: N=%d M=%d gpu %.1fs oracle %.1fs" % (
        name, scene.n, gpu["M"], t1 - t0 + time.time() - t2, t2 - t1), flush=True)
    return r


def check_project_fwd(r):
    g, p = r["gpu"], r["orc"]["proj"]
    for k in ("means2d", "conics", "chol", "depths"):
        assert_bits_equal(g[k], p[k].astype(np.float32), k)
    assert_bits_equal(g["radii"], p["radii"], "radii")
    assert_bits_equal(g["tiles"], p["tiles"], "tiles")
    vis = p["radii"] > 0
    assert vis.sum() > 0
    err = np.abs(g["colors"][vis] - p["colors"][vis])
    assert err.max() <= 2e-6 + 1e-5 * np.abs(p["colors"][vis]).max(), err.max()
    assert np.all(g["colors"][~vis] == 0)


def check_bins(r):
    g, b = r["gpu"], r["orc"]["bins"]
    assert g["M"] == b["M"]
    assert_bits_equal(g["offsets"], b["offsets"], "offsets")
    assert_bits_equal(g["keys"], b["keys"], "keys")
    assert_bits_equal(g["ids"], b["ids"], "ids")
    assert_bits_equal(g["ranges"], b["ranges"], "ranges")


def check_raster_fwd(r):
    g, cam, o = r["gpu"], r["cam"], r["orc"]["raster"]
    npx = cam.width * cam.height
    for k in ("image", "final_T"):
        nf, nflip, md, where = compare_pixels(g[k], o[k], o["margin"], k)
        print("[parity] %s %s: max|d| %.3g (non-exempt), flips %d, unexplained %d" %
              (r["name"], k, md, nflip, nf))
        assert nf == 0, (k, where)
        assert nflip <= max(2, 2e-5 * npx)
    last_bad = (g["last"] != o["last"]) & (o["margin"] >= FLIP_REL)
    assert last_bad.sum() == 0, np.argwhere(last_bad)[:5]
    if "depth" in g:
        ok = o["margin"] >= FLIP_REL
        assert np.array_equal(g["alpha"], (1.0 - g["final_T"]).astype(np.float32))
        assert np.abs(g["alpha"][ok] - o["alpha"][ok]).max() <= PIX_TOL
        # depth sums alpha T z with z up to the far side of the scene
        zmax = float(np.abs(r["orc"]["proj"]["depths"]).max())
        assert np.abs(g["depth"][ok] - o["depth"][ok]).max() <= PIX_TOL * max(1.0, zmax)


def _flip_rows(r, gpu, extra_pixels=None):
    o, cam = r["orc"], r["cam"]
    return flip_rows(o["raster"]["margin"], cam.width, cam.height, o["bins"]["ranges"],
                     o["bins"]["ids"], o["raster"]["last"], gpu["last"],
                     extra_pixels=extra_pixels)


def _assert_2d(r, reps, what):
    for rep in reps:
        print("[parity] %s %s %s" % (r["name"], what, rep))
    for rep in reps:
        assert rep["fail"] == 0, rep
        assert bounded(rep["cond"], rep["checked"]), rep
        # a flipped decision moves the terms of the pixel's own entries; few
        # Gaussians' sums move past the tolerance for it
        assert bounded(rep["flip"], rep["checked"], 1e-4, 16), rep


def check_raster_bwd(r):
    """Compositing backward given the oracle's dL/dimage on both sides."""
    g, ob, o = r["gpu_iso"], r["bw"]["g2"], r["orc"]
    ex, n_near = _flip_rows(r, g, extra_pixels=(g["last"] != o["raster"]["last"]))
    a = ob["abs_sum"]
    reps = [compare_grad(g["g_means2d"], ob["means2d"], a[:, 0:2], ex, "means2d"),
            compare_grad(g["g_conics"], ob["conics"], a[:, 2:5], ex, "conics"),
            compare_grad(g["g_opac2d"], ob["opacities"], a[:, 5], ex, "opacities"),
            compare_grad(g["g_colors"], ob["colors"], a[:, 6:9], ex, "colors"),
            # sums of positive terms: no cancellation allowance
            compare_grad(g["g_absgrad"], a[:, 0:2], None, ex, "absgrad")]
    print("[parity] %s raster_bwd: %d near-threshold pixels reach %d Gaussians" %
          (r["name"], n_near, len(ex)))
    _assert_2d(r, reps, "raster_bwd")


def _inherited(r, s_m2, s_con, s_col):
    scene, cam = r["scene"], r["cam"]
    return oracle.project_bwd_bound(scene.means, scene.scales, scene.quats, scene.sh,
                                    scene.sh_degree, cam, r["orc"]["proj"]["radii"], s_m2, s_con,
                                    s_col, r.get("settings"))


def _classify_3d(r, g, o, e, rows, what):
    """3D gradients outside max(1e-3 |g|, 1e-5): explained if within the
    inherited bound e plus the fp32 output rounding (counted, bounded), else
    exempt if the Gaussian is reached by a near-threshold pixel, whose 2D
    gradients may lie outside the allowance e assumes (counted, bounded);
    nothing else may fail."""
    n = r["scene"].n
    for k in ("means", "scales", "quats", "sh"):
        gg = np.asarray(g["g_" + k], np.float64).reshape(n, -1)
        oo = o[k].reshape(n, -1)
        ee = e[k].reshape(n, -1)
        err = np.abs(gg - oo)
        bad = err > np.maximum(G_REL * np.abs(oo), G_ABS)
        inh = bad & (err <= ee + 2 * EPS32 * np.abs(oo))
        flip = bad & ~inh & rows[:, None]
        unexplained = bad & ~inh & ~flip
        print("[parity] %s %s %s: outside tol %d (flip rows %d, inherited %d) of %d" %
              (r["name"], what, k, bad.sum(), flip.sum(), inh.sum(), bad.size))
        for i, j in np.argwhere(unexplained)[:5]:
            print("[parity]   unexplained %s[%d, %d]: gpu %.9g oracle %.9g |d| %.3g bound %.3g"
                  % (k, i, j, gg[i, j], oo[i, j], err[i, j], ee[i, j]))
        assert unexplained.sum() == 0, (k, np.argwhere(unexplained)[:5])
        assert bounded(inh.sum(), bad.size), (k, inh.sum())
        assert bounded(flip.sum(), bad.size, 1e-4, 16), (k, flip.sum())


def check_project_bwd(r):
    """Projection backward given the oracle's 2D gradients on both sides.
    The GPU receives them rounded to fp32 (|d| <= u |g2|); it computes the
    chain in fp64 and rounds once to fp32, so outside max(1e-3 |g|, 1e-5)
    an element must lie within the exact inherited bound of that rounding."""
    g, scene = r["gpu_pbwd"], r["scene"]
    g2, o = r["bw"]["g2"], r["bw"]["g3"]
    radii = r["orc"]["proj"]["radii"]
    assert_bits_equal(g["radii"], radii, "radii")
    vis = radii > 0
    for k in ("means", "scales", "quats", "sh"):
        assert np.all(g["g_" + k][~vis] == 0), k
    # fp32 rounding of each 2D input (2^-150: the absolute step below the
    # normal range)
    s = [EPS32 * np.abs(g2[k]) + 2.0 ** -150 for k in ("means2d", "conics", "colors")]
    e = _inherited(r, *s)
    _classify_3d(r, g, o, e, np.zeros(scene.n, bool), "project_bwd")


def _allow2d(g2, a, cols):
    """The 2D tolerance max(1e-3 |g|, 1e-5, COND_K u sum|terms|) per element."""
    return np.maximum(np.maximum(G_REL * np.abs(g2), G_ABS), COND_K * EPS32 * a[:, cols])


def _e2e_rows(r, g):
    """Rows reached by near-threshold pixels, L1 sign flips of dL/dimage and
    pixels whose last blended entry differs."""
    orc, dl = r["orc"], r["dl"]
    sign_flip = (np.sign(g["dL_dimage"]) != np.sign(dl)).any(axis=2)
    return _flip_rows(r, g, extra_pixels=(g["last"] != orc["raster"]["last"]) | sign_flip)


def check_e2e_2d(r, g=None):
    """The 2D gradients of a whole GPU path against the oracle's own."""
    g = r["gpu"] if g is None else g
    bw = r["bw"]
    ex, n_near = _e2e_rows(r, g)
    a = bw["g2"]["abs_sum"]
    reps = [compare_grad(g["g_means2d"], bw["g2"]["means2d"], a[:, 0:2], ex, "means2d"),
            compare_grad(g["g_conics"], bw["g2"]["conics"], a[:, 2:5], ex, "conics"),
            compare_grad(g["g_opac2d"], bw["g2"]["opacities"], a[:, 5], ex, "opacities"),
            compare_grad(g["g_colors"], bw["g2"]["colors"], a[:, 6:9], ex, "colors")]
    print("[parity] %s e2e: %d near-threshold or sign-flip pixels reach %d Gaussians" %
          (r["name"], n_near, len(ex)))
    _assert_2d(r, reps, "e2e")
    return ex


def _e2e_inherited(r):
    bw = r["bw"]
    a = bw["g2"]["abs_sum"]
    return _inherited(r, _allow2d(bw["g2"]["means2d"], a, slice(0, 2)),
                      _allow2d(bw["g2"]["conics"], a, slice(2, 5)),
                      _allow2d(bw["g2"]["colors"], a, slice(6, 9)))


def check_e2e_grads(r):
    """Whole path: GPU gradients against the oracle's own forward + backward.
    2D gradients: as in the stage check.  3D gradients: the GPU's 2D
    gradients feed its projection backward, and outside their near-threshold
    rows each is within a = max(1e-3 |g2|, 1e-5, COND_K u sum|terms|) of the
    oracle's; a 3D element outside max(1e-3 |g|, 1e-5) must lie within the
    exact bound inherited from 2D inputs known to within a."""
    ex = check_e2e_2d(r)
    rows = np.zeros(r["scene"].n, bool)
    rows[ex] = True
    _classify_3d(r, r["gpu"], r["bw"]["g3"], _e2e_inherited(r), rows, "e2e")


def check_summed_grads(rs, got, what):
    """Gradients summed over several cameras (accumulate, or a batch)
    against the sum of the oracle's per-camera gradients.  ``rs``: the
    per-camera parity records (their GPU forward outputs locate the
    near-threshold rows); ``got``: the GPU sums, dict with means, scales,
    quats, sh ([N, ...]) and opacities [N].  Per camera, an element may miss
    the oracle by its own allowance (the 2D tolerance for the opacity, the
    tolerance or the inherited bound for the 3D gradients); a sum outside
    max(1e-3 |sum|, 1e-5) must lie within the sum of those allowances plus
    one fp32 rounding per addition (counted, bounded), else in a
    near-threshold row of some camera (counted, bounded)."""
    n = rs[0]["scene"].n
    rows = np.zeros(n, bool)
    keys = ("means", "scales", "quats", "sh", "opacities")
    want = {k: 0.0 for k in keys}
    allow = {k: 0.0 for k in keys}
    mag = {k: 0.0 for k in keys}
    for r in rs:
        ex, _ = _e2e_rows(r, r["gpu"])
        rows[ex] = True
        bw = r["bw"]
        e = _e2e_inherited(r)
        for k in keys[:4]:
            oo = bw["g3"][k].reshape(n, -1)
            tol = np.maximum(G_REL * np.abs(oo), G_ABS)
            allow[k] = allow[k] + np.maximum(tol, e[k].reshape(n, -1) + 2 * EPS32 * np.abs(oo))
            want[k] = want[k] + oo
            mag[k] = mag[k] + np.abs(oo)
        o2 = bw["g2"]["opacities"].reshape(n, 1)
        allow["opacities"] = allow["opacities"] + _allow2d(
            o2, bw["g2"]["abs_sum"][:, 5:6], slice(0, 1))
        want["opacities"] = want["opacities"] + o2
        mag["opacities"] = mag["opacities"] + np.abs(o2)
    for k in keys:
        gg = np.asarray(got[k], np.float64).reshape(n, -1)
        err = np.abs(gg - want[k])
        bad = err > np.maximum(G_REL * np.abs(want[k]), G_ABS)
        inh = bad & (err <= allow[k] + len(rs) * EPS32 * mag[k])
        flip = bad & ~inh & rows[:, None]
        unexplained = bad & ~inh & ~flip
        print("[parity] %s sum of %d cameras %s: outside tol %d (flip rows %d, within the "
              "cameras' allowances %d) of %d" % (what, len(rs), k, bad.sum(), flip.sum(),
                                                inh.sum(), bad.size))
        assert unexplained.sum() == 0, (k, np.argwhere(unexplained)[:5])
        assert bounded(inh.sum(), bad.size), (k, inh.sum())
        assert bounded(flip.sum(), bad.size, 1e-4, 16), (k, flip.sum())
