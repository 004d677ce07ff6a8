"""Benchmark: forward+backward frames per second of the tile rasterizer on one
MI355X, with per-stage times, the dominant kernel's roofline fraction and the
CPU oracle timed on the host for context.

A step is one whole pass of the hot path for one camera: projection, binning
+ radix sort, compositing, loss gradient, compositing backward and
projection backward.  Inputs (Gaussians, targets, cameras) are resident in
HBM before the timed region; each step renders the next of the workload's
seeded poses.  The poses' frames are independent (the parameters do not
change between them), so --in-flight frames run concurrently, each on its
own HIP stream with its own buffers and gradients, step i on stream
i mod --in-flight; the per-stage times, the roofline and the "serial" figure
come from passes with one frame at a time.

The default line also carries short legs for the other workloads: the
100k-Gaussian box at 1080p, the 3M-Gaussian 4K inference batch of four poses
(forward with depth and alpha), and the 6M-Gaussian heavy-tailed shard's
step (eight cameras fwd+bwd, then densify/prune).

  python bench.py [--steps K] [--warmup W] [--config cluster_1m_1080p]
                  [--in-flight F] [--no-cpu-baseline] [--no-config-legs] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd frames/sec at 1M Gaussians 1920×1080 SH3; % of HBM roofline"
HBM_PEAK_GBS = 8000.0
# Plain fp32 VALU issue: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz = 39.3 T lane
# slots/s (one non-packed VALU instruction per lane per slot; transcendental
# exp2/rcp take four slots).
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
# VALU slots of the compositing inner loops, counted in the gfx950 assembly
# of raster.hip (a quarter-rate v_exp_f32 / v_rcp_f32 counts four slots):
#   forward: 49 VALU and two v_exp_f32 per two unrolled pairs -> 28.5 / pair;
#   backward: 20 VALU plus v_exp_f32 and v_rcp_f32 per evaluated pair (28
#   slots); a wavefront with a hit on the splat adds 13 VALU of gradient
#   terms and 32 of the nine-field reduction (lane swaps, an 8-lane merge
#   and DPP half-row totals, with the LDS addresses).
FWD_SLOTS_PER_PAIR = 28.5
BWD_EVAL_SLOTS = 28.0
BWD_GRAD_SLOTS = 13.0
BWD_REDUCE_SLOTS = 32.0
BWD_SLOTS_PER_PAIR = BWD_EVAL_SLOTS + BWD_GRAD_SLOTS


def algorithmic_bytes(N, V, M, M_fwd, M_bwd, Px, T, K, P, depth_alpha=False):
    """Algorithmic HBM bytes of each stage by its per-unit figures: N
    Gaussians, V visible, M tile instances (M_fwd / M_bwd of them staged by
    the compositing forward / backward before their tiles stop), Px pixels,
    T tiles, K SH coefficients per channel, P radix-sort passes.
      projection: mean in and radius, tile count out for every Gaussian
        (20 B); scales, quaternion, SH in and 2D mean, conic, depth, colour
        out for the visible (64 + 12 K B);
      binning and sort: the scan (8 N), the visible's rect inputs (20 V),
        keys and ids written and P passes of read + write (28 + 24 P per
        instance), the ranges (8 T);
      compositing: a 40-byte splat per staged instance, 20 B per pixel out
        (+8 with depth and alpha);
      compositing backward: the zero-filled 2D gradients (36 N), their
        visible rows (36 V), a 40-byte splat per staged instance, 20 B per
        pixel in;
      projection backward: radii (4 N), parameters, SH and 2D gradients in
        for the visible (72 + 12 K), gradients out for every Gaussian
        (40 + 12 K)."""
    return {
        "project_fwd": 20 * N + (64 + 12 * K) * V,
        "bin_and_sort": 8 * N + 20 * V + (28 + 24 * P) * M + 8 * T,
        "rasterize_fwd": 40 * M_fwd + 20 * Px + (8 * Px if depth_alpha else 0),
        "rasterize_bwd": 36 * N + 36 * V + 40 * M_bwd + 20 * Px,
        "project_bwd": 4 * N + (72 + 12 * K) * V + (40 + 12 * K) * N,
    }


def moved_bytes(N, V, M, M_bwd, Px, T, K, P, packed=False):
    """The bytes these kernels move, with the intermediates they keep: the
    staged 64-byte records, per-instance gradient slots, the fused loss
    gradient's target and dL/dimage."""
    if packed:
        b = moved_bytes(N, V, M, M_bwd, Px, T, K, P)
        # the visible list written by the scan; the reduction reads it and
        # writes rows for the visible only; so does the projection backward
        b["bin_and_sort"] += 4 * V
        b["rasterize_bwd"] += 4 * V + 36 * V - 36 * N
        b["project_bwd"] = 4 * V + (72 + 12 * K) * V + (40 + 12 * K) * V
        return b
    return {
        # means for all; scales, quats, SH for the visible; the seven output
        # planes (2D mean, conic, Cholesky factor, depth, radius, colour,
        # tile count: 56 B) for every Gaussian
        "project_fwd": 12 * N + (28 + 12 * K) * V + 56 * N,
        "bin_and_sort": 8 * N + 20 * V + (28 + 24 * P) * M + 8 * T,
        # staging: radii for all, 48 B of planes in and a 64-byte record out
        # per visible Gaussian; then id + 48 record bytes per instance; image,
        # final T, last index out; the fused loss gradient: target in,
        # dL/dimage out
        "rasterize_fwd": 4 * N + 112 * V + 52 * M + 20 * Px + 24 * Px,
        # per instance walked: id, offset, 64-byte record, 48-byte slot store;
        # per instance past the tile's last blend: id, offset, 32 record bytes,
        # zero store; final T, last index, dL/dimage in; then the reduction:
        # tiles + offsets, every slot read, nine 2D gradient planes written
        "rasterize_bwd": 120 * M_bwd + 88 * (M - M_bwd) + 20 * Px + 8 * N + 48 * M + 36 * N,
        "project_bwd": 4 * N + (72 + 12 * K) * V + (40 + 12 * K) * N,
    }


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_rasterize_bwd_cluster_1m_1080p.md")


def recorded_traffic():
    """HBM bytes per gs_rasterize_bwd call from the committed FETCH_SIZE /
    WRITE_SIZE counter runs, or None if the compositing source has changed
    since they were taken (or the record is missing)."""
    try:
        text = open(TRAFFIC_RECORD).read()
        src = b"".join(open(os.path.join(ROOT, "differentiable_rasterization_amd", "csrc", f),
                            "rb").read() for f in ("gs_common.h", "raster.hip"))
    except OSError:
        return None
    fields = dict(l.split(": ", 1) for l in text.splitlines()
                  if l.startswith(("source_sha256: ", "traffic_bytes_per_launch: ")))
    if fields.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(scene, cams, targets, loss_kind, frames, frames_one):
    """The oracle as it stands, fwd+bwd on poses of the same workload, on all
    the host's cores (OpenMP over Gaussians and tiles) and on one thread."""
    import oracle
    kind = oracle.LOSS_L2 if loss_kind == "l2" else oracle.LOSS_L1

    def run(n):
        t0 = time.perf_counter()
        for i in range(n):
            cam = cams[i % len(cams)]
            f = oracle.render(scene, cam)
            dl = oracle.loss_grad_image(f["raster"]["image"], targets[i % len(cams)], kind)
            oracle.backward(scene, cam, f, dl)
        return time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    dt = run(frames)
    oracle.set_threads(1)
    dt1 = run(frames_one)
    oracle.set_threads(threads)
    return {"value": frames / dt, "unit": "frames/s", "cores": threads, "kind": "oracle",
            "sample": "%d fwd+bwd frame(s) of the same workload (poses 0..%d), %.1f s" %
                      (frames, frames - 1, dt),
            "one_thread": {"value": frames_one / dt1, "unit": "frames/s", "cores": 1,
                           "sample": "%d fwd+bwd frame(s), pose 0.., %.1f s" % (frames_one,
                                                                              dt1)},
            "cpu_model": cpu_model()}


def stream_copy_gbs(torch, mib=1024, reps=20):
    """A plain device-to-device copy of `mib` MiB, read + write bytes per
    second (the HBM rate a streaming kernel reaches on this part)."""
    n = (mib << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * 4 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return gbs


def kernel_times(torch, fn, count):
    """Average device time (ms) and launch count of every kernel that `count`
    calls of fn() launch, from torch's profiler (None where it is missing)."""
    try:
        from torch.profiler import ProfilerActivity, profile
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for i in range(count):
                fn(i)
            torch.cuda.synchronize()
        out = {}
        for e in prof.key_averages():
            t = getattr(e, "device_time_total", None)
            if t is None:
                t = getattr(e, "cuda_time_total", 0.0)
            if e.count and t:
                out[e.key] = (t / 1e3 / e.count, e.count)
        return out
    except Exception:  # profiler unavailable on this build
        return None


def _sum_kernels(kt, prefixes, launches_per_call):
    """Per-call ms of the kernels whose names start with one of prefixes."""
    if not kt:
        return None
    tot = 0.0
    for name, (ms, n) in kt.items():
        short = name.split("(")[0].replace("void ", "")
        if any(short.startswith(p) for p in prefixes):
            tot += ms * n
    return tot / launches_per_call if tot else None


def densify_bench(args):
    """Times gs_densify_prune on the 6M-Gaussian heavy-tailed scene (2% clones,
    opacity threshold 0.005) with the mean gradients of one camera's
    fwd+bwd, and prints one JSON line."""
    import torch
    from differentiable_rasterization_amd import raster, scenes
    torch.cuda.set_device(0)
    scene, cams, _ = scenes.make_config("heavy_6m_1024")
    g = raster.Gaussians.from_scene(scene)
    fr = raster.Frame(g.ld, scene.sh_degree, cams[0].width, cams[0].height, capacity=4 * scene.n)
    tgt = torch.from_numpy(scenes.target_image(cams[0], 0)).cuda()
    fr.forward(g, cams[0])
    fr.loss_grad(tgt, 1)
    fr.backward(g)
    torch.cuda.synchronize()
    N = scene.n
    K = (scene.sh_degree + 1) ** 2
    P = 11 + 3 * K
    n_clone = int(np.floor(float(np.float32(0.02)) * N + 0.5))
    ld_out = N + n_clone
    e = lambda rows: torch.empty((rows, ld_out), dtype=torch.float32, device="cuda")
    outs = [e(3), e(3), e(4), e(1), e(3 * K)]
    ws_bytes = raster.gs_densify_prune_workspace_size(N, 0.02)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device="cuda")
    times = []
    n_out = 0
    for i in range(args.warmup + args.steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n_out = raster.gs_densify_prune(N, g.ld, scene.sh_degree, g.means, g.scales, g.quats,
                                        g.opacities, g.sh, fr.g_means, 0.02, 0.005, ld_out,
                                        *outs, ws, ws_bytes)
        dt = time.perf_counter() - t0   # the call ends with its count read-back
        if i >= args.warmup:
            times.append(dt)
    ms = 1e3 * float(np.median(times))
    # algorithmic bytes: the gradient planes, every parameter plane once in,
    # every output plane once out
    byts = 12 * N + 4 * P * (N + n_out)
    out = {"metric": "densify/prune ms per step at 6M Gaussians", "value": round(ms, 3),
           "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "heavy_6m_1024", "gaussians": N, "gaussians_out": n_out,
                      "clone_fraction": 0.02, "min_opacity": 0.005},
           "roofline": {"bound": "hbm", "achieved": round(byts / (ms * 1e-3) / 1e9, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "traffic": None},
           "note": "wall time of the gs_densify_prune call (its last step is the count read-back)"}
    print(json.dumps(out), flush=True)


def scenes_target(cam, k):
    from differentiable_rasterization_amd import scenes
    return scenes.target_image(cam, k)


def fwd_batch_bench(args, scene, cams, batch, depth_alpha):
    """Forward only, the poses in groups of ``batch``: each pose through the
    single-camera calls, then each group through the batched calls (one
    launch per stage).  Returns frames/s both ways."""
    import torch
    from differentiable_rasterization_amd import raster
    g = raster.Gaussians.from_scene(scene)
    W, H = cams[0].width, cams[0].height
    gc = [raster.make_camera(c) for c in cams]
    groups = [gc[i:i + batch] for i in range(0, len(gc) - batch + 1, batch)]
    fr = raster.Frame(g.ld, scene.sh_degree, W, H, with_depth_alpha=depth_alpha)
    bf = raster.BatchFrame(g.ld, scene.sh_degree, W, H, batch, with_depth_alpha=depth_alpha)
    reps = max(1, args.steps // (len(groups) * batch))

    def single():
        for grp in groups:
            for c in grp:
                fr.forward(g, c)

    def batched():
        for grp in groups:
            bf.forward(g, grp)

    # forward + backward of a group: the L1 loss gradient over the group's
    # images, the batched compositing backward, and the projection backward
    # summed over the group's cameras
    tg = [] if depth_alpha else [
        torch.from_numpy(np.stack([scenes_target(c, k) for k, c in
                                   enumerate(cams[i:i + batch])])).cuda()
        for i in range(0, len(cams) - batch + 1, batch)]

    def group_fb(b, grp, t):
        # the L1 loss gradient fused into the batch's compositing forward
        b.forward(g, grp, target=t, kind=1)
        b.backward(g)

    def batched_fb():
        for grp, t in zip(groups, tg):
            group_fb(bf, grp, t)

    # the groups are independent too: --in-flight of them at once, each on
    # its own stream with its own buffers, group k on stream k mod in-flight
    nf = max(1, args.in_flight)
    bfs = [bf] + ([] if depth_alpha else
                  [raster.BatchFrame(g.ld, scene.sh_degree, W, H, batch) for _ in range(nf - 1)])
    streams = [torch.cuda.Stream() for _ in range(nf)]

    issued = [0]

    def batched_fb_in_flight():
        for grp, t in zip(groups, tg):
            k = issued[0] % nf
            issued[0] += 1
            with torch.cuda.stream(streams[k]):
                group_fb(bfs[k], grp, t)

    out = {}
    fns = [("single", single), ("batched", batched)]
    if not depth_alpha:
        fns += [("batched_fb", batched_fb), ("batched_fb_in_flight", batched_fb_in_flight)]
    for name, fn in fns:
        fn()  # warm-up (also sizes the sort buffers)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        out[name] = reps * len(groups) * batch / (time.perf_counter() - t0)
    r = {"batch": batch, "frames": reps * len(groups) * batch,
         "fwd_fps_single_calls": round(out["single"], 2),
         "fwd_fps_batched_calls": round(out["batched"], 2),
         "speedup": round(out["batched"] / out["single"], 3),
         "depth_alpha": bool(depth_alpha)}
    if "batched_fb" in out:
        r["fwdbwd_fps_batched_calls"] = round(out["batched_fb"], 2)
        r["fwdbwd_fps_batched_in_flight"] = round(out["batched_fb_in_flight"], 2)
        r["groups_in_flight"] = nf
    return r


def graph_bench(args, scene, gcams, targets, kind, capacity):
    """The same fwd+bwd frames, each pose captured once into a HIP graph
    (binning without the read-back) and replayed."""
    import torch
    from differentiable_rasterization_amd import raster
    g = raster.Gaussians.from_scene(scene)
    W, H = gcams[0].width, gcams[0].height
    Px = W * H
    fr = raster.Frame(g.ld, scene.sh_degree, W, H, capacity=capacity, device_count=True)

    def frame(i):
        fr.project(g, gcams[i])
        fr.bin_and_sort(g)
        fr.rasterize_loss(g, targets[i], kind)
        fr.rasterize_backward(g)
        fr.project_backward(g)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(len(gcams)):
            frame(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(len(gcams)):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            frame(i)
        graphs.append(gr)
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    over = any(fr.check_counts()[1] for _ in [0])
    return {"value": round(args.steps / dt, 2), "ms_per_step": round(1e3 * dt / args.steps, 4),
            "form": "fwd+bwd frame per pose as a HIP graph, binning without the read-back",
            "capacity": int(capacity), "overflow": bool(over)}


def train_step_bench(args, scene, gcams, targets, capacity):
    """A whole training step as the gsplat guide 4.1 loop runs it: packed
    forward and backward, the mean-L1 + 0.2 D-SSIM loss gradient and the
    per-group Adam step on the visible rows, on a copy of the Gaussians
    (the parameters move every step)."""
    import torch
    from differentiable_rasterization_amd import raster
    g = raster.Gaussians.from_scene(scene)
    N, K, deg = scene.n, (scene.sh_degree + 1) ** 2, scene.sh_degree
    W, H = gcams[0].width, gcams[0].height
    log_s = torch.log(g.scales)
    logit = torch.log(g.opacities) - torch.log1p(-g.opacities)
    P = 11 + 3 * K
    m = torch.zeros((P, g.ld), device="cuda")
    v = torch.zeros((P, g.ld), device="cuda")
    fr = raster.Frame(g.ld, deg, W, H, capacity=capacity, packed=True)
    wsb = raster.gs_l1_dssim_workspace_size(W, H)
    buf = torch.empty(wsb + 256, dtype=torch.uint8, device="cuda")
    off = (-buf.data_ptr()) % 256
    ws = buf[off:off + wsb]
    cfg = raster.default_adam_config()
    names = ["project_fwd", "bin_and_sort", "rasterize_fwd", "l1_dssim", "rasterize_bwd",
             "project_bwd", "adam"]
    n_cam = len(gcams)

    def tstep(i, ev=None):
        rec = (lambda k: ev[k].record()) if ev is not None else (lambda k: None)
        rec(0)
        fr.project(g, gcams[i % n_cam])
        rec(1)
        fr.bin_and_sort(g)
        rec(2)
        fr.rasterize(g)
        rec(3)
        raster.gs_l1_dssim_loss_grad(W, H, fr.image, targets[i % n_cam], 0.2, fr.dL_dimage,
                                     None, ws, wsb)
        rec(4)
        fr.rasterize_backward(g)
        rec(5)
        fr.project_backward(g)
        rec(6)
        raster.gs_adam_step_packed(fr.V, fr.vis_ids, fr.ld, N, g.ld, deg, i + 1, cfg, g.means,
                                   log_s, g.quats, logit, g.sh, g.scales, g.opacities,
                                   fr.g_means, fr.g_scales, fr.g_quats, fr.g_opacities, fr.g_sh,
                                   m, v)
        rec(7)

    for i in range(args.warmup):
        tstep(i)
    torch.cuda.synchronize()
    # timed steps without instrumentation, then the stage times from a second
    # pass with an event between stages (as for the headline)
    t0 = time.perf_counter()
    for i in range(args.steps):
        tstep(args.warmup + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    for i in range(args.steps):
        tstep(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    ms = {n: sum(ev[k].elapsed_time(ev[k + 1]) for ev in evs) / args.steps
          for k, n in enumerate(names)}
    Px = W * H
    # algorithmic bytes: the loss reads both images and writes the gradient
    # (36 B/px); the two-pass kernels also write and read nine derivative
    # planes (132 B/px moved).  Adam, per visible Gaussian: parameter,
    # gradient, two moments in and three out per plane (28 B x P), the four
    # activated planes in and out, the list entry.
    V = fr.V
    loss_b, loss_moved = 36 * Px, 132 * Px
    adam_b = V * (28 * P + 8 * 4 + 4)
    gbs = lambda b, t: b / (t * 1e-3) / 1e9
    return {"value": round(args.steps / dt, 2), "unit": "steps/s",
            "ms_per_step": round(1e3 * dt / args.steps, 4),
            "form": "packed forward/backward, mean L1 + 0.2 D-SSIM, per-group Adam on the "
                    "visible rows",
            "stages_ms": {n: round(t, 4) for n, t in ms.items()},
            "l1_dssim": {"GB/s": round(gbs(loss_b, ms["l1_dssim"]), 1),
                         "hbm_frac": round(gbs(loss_b, ms["l1_dssim"]) / HBM_PEAK_GBS, 4),
                         "moved_GB/s": round(gbs(loss_moved, ms["l1_dssim"]), 1)},
            "adam": {"GB/s": round(gbs(adam_b, ms["adam"]), 1),
                     "hbm_frac": round(gbs(adam_b, ms["adam"]) / HBM_PEAK_GBS, 4),
                     "visible": V}}


def box_100k_bench(args):
    """The 100k-Gaussian box at 1920x1080 (SH3, L2), one frame at a time:
    forward frames/s (projection, binning, compositing) and fwd+bwd
    frames/s, with the per-stage times of an instrumented pass.  The gsplat
    guide (2.1) reports about 2.3 ms of forward rasterization for 100k
    Gaussians at 1920x1080 on an RTX 4090: quoted as context, another GPU
    and unstated scene, not a target."""
    import torch
    from differentiable_rasterization_amd import raster, scenes
    scene, cams, _ = scenes.make_config("box_100k_1080p")
    cam = raster.make_camera(cams[0])
    W, H = cams[0].width, cams[0].height
    g = raster.Gaussians.from_scene(scene)
    fr = raster.Frame(g.ld, scene.sh_degree, W, H)
    tgt = torch.from_numpy(scenes.target_image(cams[0], 7)).cuda()

    def fwd():
        fr.project(g, cam)
        fr.bin_and_sort(g)
        fr.rasterize(g)

    def fwdbwd():
        fr.project(g, cam)
        fr.bin_and_sort(g)
        fr.rasterize_loss(g, tgt, 0)
        fr.rasterize_backward(g)
        fr.project_backward(g)
    out = {}
    reps = max(8, args.steps // 2)
    for name, fn in (("fwd", fwd), ("fwdbwd", fwdbwd)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        out[name] = reps / (time.perf_counter() - t0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ms = [0.0, 0.0, 0.0]
    for _ in range(reps):
        ev[0].record()
        fr.project(g, cam)
        ev[1].record()
        fr.bin_and_sort(g)
        ev[2].record()
        fr.rasterize(g)
        ev[3].record()
        torch.cuda.synchronize()
        for k in range(3):
            ms[k] += ev[k].elapsed_time(ev[k + 1]) / reps
    return {"workload": "box_100k_1080p", "gaussians": scene.n, "width": W, "height": H,
            "sh_degree": scene.sh_degree, "instances": int(fr.M),
            "fwd_fps": round(out["fwd"], 2), "fwdbwd_fps": round(out["fwdbwd"], 2),
            "fwd_stages_ms": {"project_fwd": round(ms[0], 4), "bin_and_sort": round(ms[1], 4),
                              "rasterize_fwd": round(ms[2], 4)},
            "context": {"ms_fwd": 2.3, "hardware": "RTX 4090",
                        "source": "gsplat guide (lmnt.cn/news/262699) 2.1: forward "
                                  "rasterization of 100k Gaussians at 1920x1080",
                        "note": "another GPU and an unstated scene and SH degree; context, "
                                "not a target"}}


def cluster_3m_4k_bench(args):
    """The inference batch: 3M clustered Gaussians (SH3) rendered at
    3840x2160 for four seeded poses, forward only, with the depth and alpha
    buffers written beside the fp32 image.  Frames/s through the
    single-camera calls (one pose at a time) and through the batched calls
    (the four poses in one launch per stage)."""
    import torch
    from differentiable_rasterization_amd import scenes
    scene, cams, _ = scenes.make_config("cluster_3m_4k")
    r = fwd_batch_bench(args, scene, cams, len(cams), depth_alpha=True)
    out = {"workload": "cluster_3m_4k", "gaussians": scene.n, "width": cams[0].width,
           "height": cams[0].height, "sh_degree": scene.sh_degree, "poses": len(cams)}
    out.update(r)
    del scene
    torch.cuda.empty_cache()
    return out


def heavy_6m_step_bench(args, steps=3, warmup=1):
    """The 6M-Gaussian heavy-tailed shard (SH3, Student-t log-scales), one
    step at a time: each of its eight seeded 1024x1024 cameras goes forward
    and backward (L1) through the single-camera calls, the 3D gradients
    summed over the cameras in the buffers (accumulate), then
    gs_densify_prune clones the 2% of rows with the largest mean-gradient
    norm and drops those with opacity below 0.005 into the second parameter
    set, which the next step renders, so the count changes from step to
    step.  One frame buffer on one stream, since the cameras add into the
    same gradient sums; the densify call ends with its count read-back."""
    import torch
    from differentiable_rasterization_amd import raster, scenes
    scene, cams, _ = scenes.make_config("heavy_6m_1024")
    deg = scene.sh_degree
    K = (deg + 1) ** 2
    frac, min_op = 0.02, 0.005
    # room for every step's clones: N grows by at most round(frac N) a step
    ld = scene.n
    for _ in range(warmup + steps):
        ld += int(np.floor(float(np.float32(frac)) * ld + 0.5))
    z = lambda P: torch.zeros((P, ld), dtype=torch.float32, device="cuda")
    start = raster.Gaussians.from_scene(scene, ld=ld)
    sets = [raster.Gaussians(z(3), z(3), z(4), z(1), z(3 * K), deg, 0) for _ in range(2)]
    n0 = scene.n
    del scene
    W, H = cams[0].width, cams[0].height
    gc = [raster.make_camera(c) for c in cams]
    tg = [torch.from_numpy(scenes.target_image(c, k)).cuda() for k, c in enumerate(cams)]
    fr = raster.Frame(ld, deg, W, H, capacity=8 * ld)
    ws_bytes = raster.gs_densify_prune_workspace_size(ld, frac)
    ws_buf = torch.empty((ws_bytes + 256,), dtype=torch.uint8, device="cuda")
    off = (-ws_buf.data_ptr()) % 256
    ws = ws_buf[off:off + ws_bytes]

    def step(k):
        """Returns (N in, N out, instances over the cameras, fwd+bwd ms,
        densify ms)."""
        g, h = sets[k % 2], sets[(k + 1) % 2]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        m = 0
        for c, (cam, t) in enumerate(zip(gc, tg)):
            fr.project(g, cam)
            m += fr.bin_and_sort(g)
            fr.rasterize_loss(g, t, 1)
            fr.backward(g, accumulate=1 if c else 0)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        assert raster.gs_densify_prune_workspace_size(g.N, frac) <= ws_bytes
        h.N = raster.gs_densify_prune(g.N, g.ld, deg, g.means, g.scales, g.quats,
                                      g.opacities, g.sh, fr.g_means, frac, min_op, ld,
                                      h.means, h.scales, h.quats, h.opacities, h.sh, ws,
                                      ws_bytes)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        return g.N, h.N, m, 1e3 * (t1 - t0), 1e3 * (t2 - t1)

    def restart():
        for name in ("means", "scales", "quats", "opacities", "sh"):
            getattr(sets[0], name).copy_(getattr(start, name))
        sets[0].N = start.N

    # the instance count grows from step to step (the clones of large
    # splats add tiles): an untimed pass over the same steps sizes the sort
    # buffers for the largest, then the timed pass repeats the steps from
    # the starting parameters (the same counts, bit for bit)
    restart()
    for k in range(warmup + steps):
        step(k)
    cap0 = fr.capacity
    restart()
    rows = []
    for k in range(warmup + steps):
        r = step(k)
        if k >= warmup:
            rows.append(r)
    total = sum(r[3] + r[4] for r in rows) * 1e-3
    out = {"workload": "heavy_6m_1024", "gaussians": n0, "width": W, "height": H,
           "sh_degree": deg, "cameras_per_step": len(gc), "steps": steps, "warmup": warmup,
           "steps_per_s": round(steps / total, 3),
           "frames_per_s": round(steps * len(gc) / total, 2),
           "per_step": [{"gaussians_in": r[0], "gaussians_out": r[1], "instances": r[2],
                         "fwdbwd_ms": round(r[3], 3), "densify_ms": round(r[4], 3)}
                        for r in rows],
           "sort_buffers_regrown": fr.capacity != cap0,
           "clone_fraction": frac, "min_opacity": min_op,
           "form": "per step: fwd+bwd of the 8 cameras (gradients summed), then densify/prune "
                   "into the next step's parameters; the clones of the largest-gradient "
                   "rows add instances, so each step renders more than the last"}
    del sets, start, fr, ws_buf
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="cluster_1m_1080p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-frames", type=int, default=16)
    ap.add_argument("--cpu-frames-one-thread", type=int, default=1)
    ap.add_argument("--densify", action="store_true",
                    help="time gs_densify_prune on the 6M-Gaussian scene instead")
    ap.add_argument("--absgrad", action="store_true",
                    help="run the compositing backward with the absolute-gradient sums")
    ap.add_argument("--packed", action="store_true",
                    help="run the packed calls (visible list, sparse gradient rows)")
    ap.add_argument("--in-flight", type=int, default=3,
                    help="frames processed concurrently, each on its own stream and buffers")
    ap.add_argument("--no-packed-leg", action="store_true",
                    help="leave out the packed calls' leg (hardware counter runs use it, so "
                         "that every dispatch of a kernel belongs to the headline's frames)")
    ap.add_argument("--no-train-step", action="store_true",
                    help="skip the training-step measurement (packed calls, L1 + 0.2 D-SSIM, "
                         "per-group Adam)")
    ap.add_argument("--fwd-batch-only", action="store_true",
                    help="only the forward of the poses in batches of --batch (single-camera "
                         "calls against batched calls), e.g. with --config cluster_3m_4k")
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--no-config-legs", action="store_true",
                    help="leave out the 3M/4K inference batch and the 6M densify step legs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy (a reference "
                         "kernel of known traffic for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.densify:
        densify_bench(args)
        return

    import torch
    from differentiable_rasterization_amd import raster, scenes

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    scene, cams, loss_kind = scenes.make_config(args.config)
    if args.fwd_batch_only:
        r = fwd_batch_bench(args, scene, cams, args.batch, depth_alpha=(loss_kind is None))
        print(json.dumps({"metric": "forward frames/sec, batched-camera calls", "value":
                          r["fwd_fps_batched_calls"], "unit": "frames/s", "n_gpus": 1,
                          "higher_is_better": True, "dtype": "f32", "data": "synthetic",
                          "config": {"workload": args.config, "gaussians": scene.n,
                                     "width": cams[0].width, "height": cams[0].height,
                                     "sh_degree": scene.sh_degree, "poses": len(cams)},
                          "fwd_batch": r}), flush=True)
        return
    loss_kind = loss_kind or "l1"
    W, H = cams[0].width, cams[0].height
    N, K = scene.n, (scene.sh_degree + 1) ** 2
    targets_np = [scenes.target_image(c, i) for i, c in enumerate(cams)]
    targets = [torch.from_numpy(t).cuda() for t in targets_np]
    g = raster.Gaussians.from_scene(scene)
    nf = max(1, args.in_flight)
    frames = [raster.Frame(g.ld, scene.sh_degree, W, H, capacity=4 * N, packed=args.packed)
              for _ in range(nf)]
    streams = [torch.cuda.Stream() for _ in range(nf)]
    fr = frames[0]
    gcams = [raster.make_camera(c) for c in cams]
    kind = 0 if loss_kind == "l2" else 1
    P = len(cams)
    T = fr.T
    Px = W * H
    tile_bits = int(np.ceil(np.log2(max(T, 2))))

    names = ["project_fwd", "bin_and_sort", "rasterize_fwd", "rasterize_bwd", "project_bwd"]

    def step(i, ev=None, fr=fr, project=True):
        """The five stages of step i on frame fr (project=False: its
        projection was issued already)."""
        c = gcams[i % P]
        if ev is not None:
            ev[0].record()
        if project:
            fr.project(g, c)
        if ev is not None:
            ev[1].record()
        fr.bin_and_sort(g)
        if ev is not None:
            ev[2].record()
        # compositing with the loss gradient fused in
        fr.rasterize_loss(g, targets[i % P], kind)
        if ev is not None:
            ev[3].record()
        fr.rasterize_backward(g, absgrad=args.absgrad)
        if ev is not None:
            ev[4].record()
        fr.project_backward(g)
        if ev is not None:
            ev[5].record()
        return fr.M

    # workload statistics per pose: one untimed pass with the counting
    # variants, each pose on the frame and stream the timed steps give it.
    # What the statistics need is copied on the device and analysed on the
    # host after the timed passes, so the warm-up steps follow this pass
    # with no idle gap and every frame's buffers have been used before.
    raw = []
    for i in range(P):
        k = i % nf
        f = frames[k]
        # the timed steps' stream for this frame (one frame: the current one)
        with torch.cuda.stream(streams[k] if nf > 1 else torch.cuda.current_stream()):
            step(i, fr=f)
            c = torch.zeros(8, dtype=torch.int64, device="cuda")
            f.rasterize(g, counters=c[0:4])
            f.rasterize_backward(g, counters=c[4:8])
            d = f.depths[:N].view(torch.int32).to(torch.int64)
            has = f.tiles[:N] != 0
            raw.append(dict(M=f.M, cnt=c, V=(f.radii[:N] > 0).sum(),
                            ranges=f.ranges.clone(), last=f.last_idx.clone(),
                            dmax=torch.where(has, d, torch.full_like(d, -1)).max(),
                            dmin=torch.where(has, d, torch.full_like(d, 1 << 40)).min()))

    def analyse(r):
        """Per-pose counts from the statistics pass: V, M, the instances the
        backward stages, the pairs of each loop and the sort's passes (10-bit
        digits over the tile bits and the bits that the depths of the rows
        with tiles span)."""
        c = r["cnt"].cpu().numpy()
        rng = r["ranges"].cpu().numpy().view(np.uint32).astype(np.int64)
        lens = rng[:, 1] - rng[:, 0]
        last = r["last"].cpu().numpy().view(np.uint32).astype(np.int64)
        gx = (W + 15) // 16
        tile_of = (np.arange(H)[:, None] // 16) * gx + (np.arange(W)[None, :] // 16)
        maxlast = np.zeros(T, np.int64)
        np.maximum.at(maxlast, tile_of.ravel(), last.ravel())
        inside = np.bincount(tile_of.ravel(), minlength=T)
        dmax, dmin = int(r["dmax"].item()), int(r["dmin"].item())
        span = dmax - dmin if dmax >= 0 else 0
        return dict(V=int(r["V"].item()), M=r["M"], M_bwd=int(maxlast.sum()),
                    pairs_tile=int((inside * lens).sum()), fwd_eval=int(c[0]),
                    blended=int(c[1]), plain_pairs=int(c[2]), fwd_plain_tile=int(c[3]),
                    bwd_eval=int(c[4]), bwd_hit=int(c[5]), bwd_plain_tile=int(c[6]),
                    bwd_reductions=int(c[7]),
                    sort_passes=max(1, -(-(tile_bits + span.bit_length()) // 10)))

    def run_steps(frs, first, count):
        """Steps first .. first+count-1, step i on frame/stream i mod len(frs)
        (one frame: the current stream).  With several frames in flight, the
        next step's projection is issued before this step's binning waits
        for its instance count, so the host's wait overlaps it; each step
        still runs the five stages of its own frame, and no projection past
        the last step is issued."""
        n = len(frs)
        if n == 1:
            for i in range(first, first + count):
                step(i, fr=frs[0])
            return
        on = lambda i: torch.cuda.stream(streams[i % n])
        if count > 0:
            with on(first):
                frs[first % n].project(g, gcams[first % P])
        for i in range(first, first + count):
            if i + 1 < first + count:
                with on(i + 1):
                    frs[(i + 1) % n].project(g, gcams[(i + 1) % P])
            with on(i):
                step(i, fr=frs[i % n], project=False)

    def timed(frs):
        """Warm-up, then the timed steps with len(frs) frames in flight;
        returns (seconds, serial seconds, per-stage ms).  The timed steps run
        without instrumentation: an event recorded on the stream leaves the
        GPU idle for several microseconds, and six per step would be counted
        in the throughput.  Then the same steps one frame at a time (serial
        seconds), and a third pass, one frame at a time with an event between
        stages, for the per-stage times."""
        run_steps(frs, 0, args.warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(frs, 0, args.steps)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        t0 = time.perf_counter()
        run_steps(frs[:1], 0, args.steps)
        torch.cuda.synchronize()
        dt_serial = time.perf_counter() - t0
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
               for _ in range(args.steps)]
        for i in range(args.steps):
            step(i, evs[i], fr=frs[0])
        torch.cuda.synchronize()
        ms = {n: 0.0 for n in names}
        for ev in evs:
            for k, n in enumerate(names):
                ms[n] += ev[k].elapsed_time(ev[k + 1])
        return dt, dt_serial, {n: v / args.steps for n, v in ms.items()}

    dt, dt_serial, stage_ms = timed(frames)
    stats = [analyse(r) for r in raw]
    del raw
    packed_line = None
    train_line = None if args.no_train_step else train_step_bench(args, scene, gcams, targets,
                                                                   fr.capacity)
    batch_line = None if args.no_train_step else fwd_batch_bench(args, scene, cams, args.batch,
                                                                  depth_alpha=False)
    # the graph frames bin without reading M back, so their grids are sized
    # for the buffers' capacity: give them buffers 25% above the largest M
    # seen over the poses (the eager frame's 4N would launch 2.7x the sort
    # workgroups, most of them idle)
    graph_cap = int(1.25 * max(s_["M"] for s_ in stats)) + 8192
    graph_line = None if args.no_train_step else graph_bench(args, scene, gcams, targets, kind,
                                                              graph_cap)
    if not args.packed and not args.no_packed_leg:
        # the same steps through the packed calls (visible list, sparse
        # gradient rows), reported beside the dense headline
        frps = [raster.Frame(g.ld, scene.sh_degree, W, H, capacity=fr.capacity, packed=True)
                for _ in range(nf)]
        dtp, dtps, msp = timed(frps)
        packed_line = {"value": round(args.steps / dtp, 2),
                       "ms_per_step": round(1e3 * dtp / args.steps, 4),
                       "serial_value": round(args.steps / dtps, 2),
                       "stages_ms": {n: round(v, 4) for n, v in msp.items()}}
        del frps
    # average workload over the poses the timed steps visited
    visited = [stats[i % P] for i in range(args.steps)]
    avg = {k: float(np.mean([s[k] for s in visited])) for k in visited[0]}
    sort_passes = avg["sort_passes"]
    algo_b = algorithmic_bytes(N, avg["V"], avg["M"], avg["fwd_plain_tile"] / 256.0,
                               avg["M_bwd"], Px, T, K, sort_passes)
    moved_b = moved_bytes(N, avg["V"], avg["M"], avg["M_bwd"], Px, T, K, sort_passes,
                          packed=args.packed)
    stages = {}
    for n in names:
        ms = stage_ms[n]
        gbs = algo_b[n] / (ms * 1e-3) / 1e9
        stages[n] = {"ms": round(ms, 4), "GB/s": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "moved_GB/s": round(moved_b[n] / (ms * 1e-3) / 1e9, 1)}
    fps = args.steps / dt
    fwd_ms = stage_ms["project_fwd"] + stage_ms["bin_and_sort"] + stage_ms["rasterize_fwd"]
    frame_ms = sum(stage_ms.values())
    # kernel-level device times of one-frame-at-a-time steps (untimed pass)
    kt = kernel_times(torch, lambda i: step(i, fr=fr), P)
    sort_ms = _sum_kernels(kt, ("gs::sort_first_hist_kernel",
                                "gs::sort_pass_kernel"), P)
    bwd_kernel_ms = _sum_kernels(kt, ("gs::raster_bwd_kernel",), P)
    reduce_ms = _sum_kernels(kt, ("gs::reduce_partials_kernel",), P)
    # The compositing backward is bound by VALU issue.  Its work per call is
    # counted by its counting variant: the pairs the kernel evaluated (31
    # slots each) and the wavefront reductions it ran (64 lanes x 48 slots of
    # gradient terms and lane-swap reduction).  frac = those issued slots per
    # second of the whole gs_rasterize_bwd call (its segmented reduction
    # included) against the VALU peak; blended_frac counts only the pairs
    # whose result the method uses (a floor any loop must evaluate).
    issued = {"rasterize_bwd": avg["bwd_eval"] * BWD_EVAL_SLOTS +
              avg["bwd_reductions"] * 64 * (BWD_GRAD_SLOTS + BWD_REDUCE_SLOTS),
              "rasterize_fwd": avg["fwd_eval"] * FWD_SLOTS_PER_PAIR}
    useful = {"rasterize_bwd": avg["bwd_hit"] * BWD_SLOTS_PER_PAIR,
              "rasterize_fwd": avg["blended"] * FWD_SLOTS_PER_PAIR}
    plain = {"rasterize_bwd": avg["bwd_plain_tile"] * BWD_SLOTS_PER_PAIR,
             "rasterize_fwd": avg["fwd_plain_tile"] * FWD_SLOTS_PER_PAIR}
    work = {"pairs_blended": int(avg["blended"]), "pairs_evaluated_fwd": int(avg["fwd_eval"]),
            "pairs_evaluated_bwd": int(avg["bwd_eval"]),
            "pairs_plain_method": int(avg["plain_pairs"]),
            "pairs_plain_tile_loop_fwd": int(avg["fwd_plain_tile"]),
            "pairs_plain_tile_loop_bwd": int(avg["bwd_plain_tile"]),
            "pairs_all_tile_pixels": int(avg["pairs_tile"]),
            "wave_reductions_bwd": int(avg["bwd_reductions"]),
            "slots_per_evaluated_pair_bwd": BWD_EVAL_SLOTS,
            "slots_per_reduction_lane_bwd": BWD_GRAD_SLOTS + BWD_REDUCE_SLOTS}
    dominant = max(names, key=lambda n: stage_ms[n])
    if dominant in issued:
        t = stage_ms[dominant] * 1e-3
        ach = issued[dominant] / t / 1e12
        traffic = (recorded_traffic() if (dominant == "rasterize_bwd" and not args.absgrad and
                                          not args.packed and
                                          args.config == "cluster_1m_1080p") else None)
        roof = {"bound": "alu", "kernel": "gs_rasterize_bwd" if dominant == "rasterize_bwd"
                else "gs_rasterize_fwd_loss",
                "achieved": round(ach, 3), "peak": round(VALU_PEAK_TOPS, 2), "unit": "TOP/s",
                "frac": round(ach / VALU_PEAK_TOPS, 4), "traffic": traffic,
                "blended_frac": round(useful[dominant] / t / 1e12 / VALU_PEAK_TOPS, 4),
                "speedup_over_plain_tile_loop_at_peak":
                    round(plain[dominant] / t / 1e12 / VALU_PEAK_TOPS, 4),
                "hbm_frac": stages[dominant]["hbm_frac"], "call_ms": round(stage_ms[dominant], 4),
                "work_per_launch": work}
        if dominant == "rasterize_bwd" and bwd_kernel_ms:
            roof["kernels_ms"] = {"raster_bwd_kernel": round(bwd_kernel_ms, 4),
                                  "reduce_partials_kernel": round(reduce_ms or 0.0, 4)}
            roof["frac_compositing_kernel_alone"] = round(
                issued[dominant] / (bwd_kernel_ms * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4)
    else:
        ach = algo_b[dominant] / (stage_ms[dominant] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dominant, "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": None}
    c = cams[0]
    out = {
        "metric": METRIC, "value": round(fps, 2), "unit": "frames/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(1e3 * dt / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.config, "gaussians": N, "width": W, "height": H,
                   "sh_degree": scene.sh_degree, "poses": P, "loss": loss_kind,
                   "visible": int(avg["V"]), "instances": int(avg["M"]),
                   "sort_passes": sort_passes,
                   "absgrad": bool(args.absgrad), "packed": bool(args.packed),
                   "frames_in_flight": nf},
        "serial": {"value": round(args.steps / dt_serial, 2),
                   "ms_per_step": round(1e3 * dt_serial / args.steps, 4),
                   "form": "the same steps one frame at a time on one stream"},
        "one_frame": {"value": round(1e3 / frame_ms, 2), "ms": round(frame_ms, 4),
                      "form": "1 / (sum of the five stage times of one frame, measured one "
                              "frame at a time with events between the stages)"},
        "fwd_fps": round(1e3 / fwd_ms, 2),
        "sort_keys_per_s": round(avg["M"] / (stage_ms["bin_and_sort"] * 1e-3), 1),
        "sort_keys_per_s_sort_kernels": (round(avg["M"] / (sort_ms * 1e-3), 1)
                                         if sort_ms else None),
        "sort_kernels_ms": round(sort_ms, 4) if sort_ms else None,
        "stages": stages,
        "roofline": roof,
        "stream_copy_GB/s": round(stream_copy_gbs(torch), 1),
    }
    if packed_line is not None:
        out["packed"] = packed_line
    if train_line is not None:
        out["train_step"] = train_line
    if batch_line is not None:
        out["fwd_batch"] = batch_line
    if graph_line is not None:
        out["graph"] = graph_line
    if not args.no_train_step and args.config == "cluster_1m_1080p":
        out["box_100k_1080p"] = box_100k_bench(args)
        if not args.no_config_legs:
            out["cluster_3m_4k"] = cluster_3m_4k_bench(args)
            out["heavy_6m_1024"] = heavy_6m_step_bench(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(scene, cams, targets_np, loss_kind, args.cpu_frames,
                                           args.cpu_frames_one_thread)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
