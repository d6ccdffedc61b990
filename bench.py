"""Benchmark: 768x512 synthetic target, 50,000 2D Gaussians, accumulated-sum rendering.

One "step" is the whole hot path on the GPU, one gi_fit_step_sum call: tile binning, the fused
per-tile forward raster + L2 loss gradient + backward raster, and Adam with the gather of the
per-pair gradients (which also reduces the loss and sets up the updated parameters for the next
step's binning).  `value` is fwd+bwd training steps per second on one MI355X with every input
resident in HBM.  Also reported: render FPS (preprocess + bin/sort + raster) and cached-raster FPS
(raster only, binning reused); kernel times from HIP events on the launch stream over passes of the
fused raster kernel (and of the separate forward / backward kernels) on the trained parameters'
binning; the roofline of the dominant kernel; and the CPU oracle timed on a bounded pixel sample of
the same workload.  With an alpha-compositing workload (--workload alpha_2048x2048_500k) a step is
binning + alpha forward + L2 loss + alpha backward + Adam, and the roofline is that of the slower
of the alpha forward / backward kernels.

usage: python bench.py [--gpus 1] [--steps 2800] [--warmup 50] [--workload NAME] [--no-cpu-baseline]
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
sys.path.insert(0, ROOT)

METRIC = "render FPS + fwd+bwd steps/s, 768×512 × 50K 2D Gaussians; % FP32 VALU peak"
PEAK_FP32 = 157.3          # TFLOP/s, MI355X FP32 vector (AMD published)
PEAK_HBM = 8000.0          # GB/s
FLOP_FWD = 17              # per binned pair: dx, dy 2; cutoff exponent 7; scale + exp2 2; 3 colour FMA 6
FLOP_BWD = 32              # per binned pair (recompute 11, colour/h 9, mean/conic partials 11, reduce 1)
FLOP_FWD_ALPHA = 21        # per binned pair: the sum forward's 17 + alpha, alpha T, T update and the stop test
FLOP_BWD_ALPHA = 55        # per binned pair: recompute, T_j and the suffix colour, mean/conic/opacity partials


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def provenance():
    """Where a result comes from: a hash of the sources the library is built from (and the git
    revision when the tree has one), the library's version string, the GPU, the host CPU, and the
    GPU's shader-clock level at the end of the run when the driver exposes it."""
    import glob
    import subprocess
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "rasterizer_gaussian_raster_amd", "csrc", "*"))) + [
            os.path.join(ROOT, "include", "gi.h")]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    git = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"], capture_output=True, text=True,
                           timeout=10)
        git = r.stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        pass
    cpu = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    sclk = None
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(f) as fh:
                for line in fh:
                    if line.strip().endswith("*"):
                        sclk = line.split(":", 1)[1].replace("*", "").strip()
                        break
        except OSError:
            continue
        if sclk:
            break
    out = {"sources_sha256_16": h.hexdigest()[:16], "git_rev": git, "host_cpu": cpu, "sclk_level_at_end": sclk}
    try:
        import torch
        from rasterizer_gaussian_raster_amd import gi
        out["lib"] = gi.version()
        out["gpu"] = torch.cuda.get_device_name(0) if torch.cuda.is_available() else None
        out["torch"], out["hip"] = torch.__version__, torch.version.hip
    except Exception as e:           # provenance never fails a run
        out["error"] = repr(e)
    return out


def emit(out):
    """The result line: one JSON object on stdout, with the run's provenance."""
    out = dict(out)
    out["provenance"] = provenance()
    print(json.dumps(out), flush=True)


def stats_us(x_us):
    x = np.asarray(x_us, np.float64)
    return {"median": round(float(np.median(x)), 2), "p10": round(float(np.percentile(x, 10)), 2),
            "p90": round(float(np.percentile(x, 90)), 2), "mean": round(float(np.mean(x)), 2), "n": int(x.size)}


def batch_time_us(fn, per_batch=20, batches=15, warm=5):
    """Per-call time of fn from batches of back-to-back calls on the current stream, bracketed by HIP
    events (the events' own overhead is spread over a batch): one value per batch, in microseconds."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [(E(), E()) for _ in range(batches)]
    for a, b in ev:
        a.record()
        for _ in range(per_batch):
            fn()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev]) * 1e3 / per_batch


def binned_pairs(W, H, ranges):
    """sum over tiles of (list length) x (in-image pixels of the tile)."""
    tx = -(-W // 16)
    T = ranges.shape[0]
    t = np.arange(T)
    x0, y0 = (t % tx) * 16, (t // tx) * 16
    npx = np.minimum(16, W - x0) * np.minimum(16, H - y0)
    ln = ranges[:, 1].astype(np.int64) - ranges[:, 0].astype(np.int64)
    return int((ln * npx).sum())


def evaluated_pairs(W, H, keys, vals, pixbox):
    """Pairs the forward kernel evaluates: 64 per (list entry, 8x8 quadrant its box overlaps)."""
    tx = -(-W // 16)
    k = keys.astype(np.int64)
    b = pixbox[vals.astype(np.int64)].astype(np.int64)
    x0, y0 = (k % tx) * 16, (k // tx) * 16
    tot = 0
    for q in range(4):
        qx, qy = x0 + (q & 1) * 8, y0 + (q >> 1) * 8
        ov = (b[:, 0] <= qx + 7) & (b[:, 2] >= qx) & (b[:, 1] <= qy + 7) & (b[:, 3] >= qy)
        tot += int(ov.sum())
    return tot * 64


def kernel_source_hash(name):
    src = os.path.join(ROOT, "rasterizer_gaussian_raster_amd", "csrc", name)
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def load_traffic(kernel_file, kernel_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        e = d.get(kernel_name)
        if e and e.get("source_sha256_16") == kernel_source_hash(kernel_file):
            return float(e["hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None
    return None


def cpu_baseline(wl, params, target_seconds=15.0):
    """The oracle (brute force over all N Gaussians per pixel, fp64) on a bounded pixel sample:
    sum render + analytic gradient of the same pixels, extrapolated to one full-frame step."""
    import oracle
    W, H = wl.width, wl.height
    p64 = params.astype(np.float64)
    rng = np.random.default_rng(12345)

    def run(npix):
        idx = rng.choice(W * H, size=npix, replace=False)
        pix = np.stack([idx // W, idx % W], 1).astype(np.int32)
        G = np.zeros((3, H, W))
        G[:, pix[:, 0], pix[:, 1]] = rng.normal(size=(3, npix))
        t0 = time.perf_counter()
        oracle.render_sum(W, H, p64, pixels=pix)
        oracle.grad_sum(W, H, p64, G)
        return time.perf_counter() - t0

    run(64)                                    # load + warm
    npix = 256
    t = run(npix)
    # grow the sample until it holds most of the time budget (small samples are overhead-bound)
    while t < 0.6 * target_seconds and npix < W * H:
        npix = int(min(W * H, npix * min(16.0, max(2.0, target_seconds / max(t, 1e-3)))))
        t = run(npix)
    per_frame = t * (W * H) / npix
    what = (f"every pixel of the {W}x{H} frame ({npix}), all {params.shape[0]} Gaussians per pixel "
            f"(render + gradient), {t:.1f} s: one full step, not extrapolated" if npix == W * H else
            f"{npix} random pixels of the {W}x{H} frame, all {params.shape[0]} Gaussians per pixel "
            f"(render + gradient), {t:.1f} s, extrapolated linearly to the full frame")
    return {"value": 1.0 / per_frame, "unit": "fwd+bwd steps/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": what, "seconds": round(t, 3)}


def cpu_baseline_alpha(wl, params, logit, bg, target_seconds=15.0):
    """The oracle's alpha compositing (brute force over all N Gaussians per pixel, fp64) on a bounded
    pixel sample: render + analytic gradient of the same pixels, extrapolated to one full-frame step."""
    import oracle
    W, H = wl.width, wl.height
    p64, l64, b64 = params.astype(np.float64), logit.astype(np.float64), bg.astype(np.float64)
    rng = np.random.default_rng(12345)
    G = np.zeros((3, H, W))

    def run(npix):
        idx = rng.choice(W * H, size=npix, replace=False)
        pix = np.stack([idx // W, idx % W], 1).astype(np.int32)
        G[:] = 0.0
        G[:, pix[:, 0], pix[:, 1]] = rng.normal(size=(3, npix))
        t0 = time.perf_counter()
        oracle.render_alpha(W, H, p64, l64, b64, pixels=pix)
        oracle.grad_alpha(W, H, p64, l64, b64, G)
        return time.perf_counter() - t0

    run(16)
    npix = 64
    t = run(npix)
    while t < 0.6 * target_seconds and npix < W * H:
        npix = int(min(W * H, npix * min(16.0, max(2.0, target_seconds / max(t, 1e-3)))))
        t = run(npix)
    per_frame = t * (W * H) / npix
    return {"value": 1.0 / per_frame, "unit": "fwd+bwd steps/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{npix} random pixels of the {W}x{H} frame, all {params.shape[0]} Gaussians per pixel "
                      f"(alpha render + gradient), {t:.1f} s, extrapolated linearly to the full frame",
            "seconds": round(t, 3)}


def bench_alpha(args, w, target, params, dev):
    """The alpha-compositing workload: one step = bin (with preprocess) + alpha forward + L2 loss +
    alpha backward + Adam on the parameters, logits and background (separate launches)."""
    import torch
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Fitter, Raster

    wl = w["workload"]
    W, H = wl.width, wl.height
    logit = torch.from_numpy(w["logit"]).to(dev)
    bg = torch.from_numpy(w["background"]).to(dev)
    fit = Fitter(target, params, logit=logit, background=bg, capacity_slack=2.0)
    for _ in range(args.warmup):
        fit.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fit.step()
    torch.cuda.synchronize()
    t_train = time.perf_counter() - t0
    r = fit.raster
    M_now = int(r.d_num[0].item()) & 0xFFFFFFFF
    assert M_now <= r.capacity, "tile-pair capacity exceeded during the timed run"
    ms_step = 1e3 * t_train / args.steps
    final_loss = float(fit.loss.item())
    log(f"[bench] train: {ms_step:.4f} ms/step, loss {final_loss:.4e}")

    # kernel timing on one binning of the trained parameters
    rend = Raster(W, H, wl.n, gi.MODE_ALPHA)
    rend.preprocess(fit.params, fit.logit)
    M = rend.bin(sync=True)
    rend.set_capacity(int(M * 1.5) + 4096)
    rend.bin(sync=True, order=True, params=fit.params, logit=fit.logit)
    bg4 = fit.bg4
    dL = torch.empty_like(target)
    loss = torch.zeros(1, dtype=torch.float32, device=dev)
    loss_ws = torch.empty(gi.gi_loss_workspace_bytes(target.numel()), dtype=torch.uint8, device=dev)
    rend.forward(bg4)
    gi.gi_loss_l2(target.numel(), rend.image, target, dL, loss, loss_ws)
    # batches of back-to-back calls between HIP events on the launch stream: the forward, and the
    # backward to the pair slots as the fit step calls it (the entry-record packing + the raster)
    fwd_us = batch_time_us(lambda: rend.forward(bg4), per_batch=5, batches=9, warm=2)
    bwd_us = batch_time_us(lambda: rend.backward(dL, None, logit=fit.logit, background=bg4), per_batch=5,
                           batches=9, warm=2)
    log(f"[bench] alpha fwd {np.median(fwd_us):.1f} us, bwd (packing + raster, to the slots) "
        f"{np.median(bwd_us):.1f} us")
    reps = max(20, args.steps // 4)

    def loop_time(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps

    t_render = loop_time(lambda: rend.render(fit.params, logit=fit.logit, background=bg4, sync=False))
    t_cached = loop_time(lambda: rend.forward(bg4))
    log(f"[bench] render {t_render*1e6:.1f} us ({1/t_render:.0f} FPS), cached raster {t_cached*1e6:.1f} us")

    rend.preprocess(fit.params, fit.logit)
    M = rend.bin(sync=True)
    torch.cuda.synchronize()
    ranges = rend.ranges.cpu().numpy().view(np.uint32)
    pairs = binned_pairs(W, H, ranges)
    t_fin = rend.t_final.cpu().numpy()
    fwd_s = float(np.median(fwd_us)) * 1e-6
    bwd_s = float(np.median(bwd_us)) * 1e-6

    def roof(kname, flop, secs):
        tf = flop * pairs / secs / 1e12
        return {"bound": "alu", "kernel": kname, "achieved": round(tf, 3), "peak": PEAK_FP32, "unit": "TFLOP/s",
                "frac": round(tf / PEAK_FP32, 4), "traffic": load_traffic("k_raster_alpha.hip", kname),
                "avg_launch_us": round(secs * 1e6, 2)}

    roof_fwd = roof("k_render_alpha_fwd<false>", FLOP_FWD_ALPHA, fwd_s)
    roof_bwd = roof("k_alpha_pack + k_render_alpha_bwd", FLOP_BWD_ALPHA, bwd_s)   # one gi_render_bwd call
    dominant, other = (roof_bwd, roof_fwd) if bwd_s >= fwd_s else (roof_fwd, roof_bwd)
    out = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 2),
        "unit": "fwd+bwd steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "width": W, "height": H, "gaussians": wl.n, "mode": "alpha",
                   "tiles": int(rend.T), "tile_pairs": int(M), "binned_pixel_pairs": pairs,
                   "pixels_stopped_early": int((t_fin < 1e-4).sum())},
        "render_fps": round(1.0 / t_render, 1),
        "mpix_per_s": round(W * H / t_render / 1e6, 1),
        "cached_raster_fps": round(1.0 / t_cached, 1),
        "timing": "value: K steps after W warm-up steps, host clock with device syncs on both sides; "
                  "roofline: medians of batches of back-to-back calls between HIP events on the launch stream, "
                  "on the trained parameters' binning: the alpha forward, and the backward to the pair slots "
                  "(entry-record packing + raster, one gi_render_bwd call)",
        "final_loss": final_loss,
        "kernels_us": {"render_alpha_fwd": stats_us(fwd_us), "render_alpha_bwd": stats_us(bwd_us)},
        "roofline": dominant,
        "roofline_other": other,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a pixel sample ...")
        out["cpu_baseline"] = cpu_baseline_alpha(wl, w["params"], w["logit"], w["background"])
    else:
        out["cpu_baseline"] = None
    emit(out)


def bench_ssim(args, w, target, params, dev):
    """Sum mode with the SSIM pixel loss: one step = preprocess and binning + forward + gi_loss_ssim
    (one fused stencil kernel) + backward with the gather + Adam."""
    import torch
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Fitter

    wl = w["workload"]
    W, H = wl.width, wl.height
    lw = tuple(float(v) for v in args.loss.split(","))
    if len(lw) != 3:
        raise SystemExit("--loss takes l2 or three weights w1,w2,ws")
    fit = Fitter(target, params, capacity_slack=2.0, loss=lw)
    for _ in range(args.warmup):
        fit.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fit.step()
    torch.cuda.synchronize()
    t_train = time.perf_counter() - t0
    r = fit.raster
    M_now = int(r.d_num[0].item()) & 0xFFFFFFFF
    assert M_now <= r.capacity, "tile-pair capacity exceeded during the timed run"
    ms_step = 1e3 * t_train / args.steps
    final_loss = float(fit.loss.item())
    log(f"[bench] ssim-loss train: {ms_step:.4f} ms/step, loss {final_loss:.4e}")
    flags = gi.SSIM_TARGET_PREPARED     # the fit's call: the target's statistics formed once
    st = stats_us(batch_time_us(lambda: gi.gi_loss_ssim(W, H, r.image, fit.target, *lw, fit.dL, fit.loss,
                                                         fit.ssim_ws, flags=flags)))
    st_full = stats_us(batch_time_us(lambda: gi.gi_loss_ssim(W, H, r.image, fit.target, *lw, fit.dL, fit.loss,
                                                              fit.ssim_ws)))
    ssim_s = st["median"] * 1e-6
    nbytes = 20 * 3 * W * H           # per entry: image, target, the target's (mean, E[T^2]) read; dL written
    gbs = nbytes / ssim_s / 1e9
    # per entry: two separable 11-tap filterings of three maps (x, x^2, x y, then D0..D2): 264 flop;
    # the products, the map's derivatives and the output: 51 flop
    nflop = 315 * 3 * W * H
    tfs = nflop / ssim_s / 1e12
    log(f"[bench] gi_loss_ssim {st['median']:.1f} us ({tfs:.1f} TFLOP/s, {gbs:.0f} GB/s algorithmic); "
        f"without the prepared target {st_full['median']:.1f} us")
    out = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 2),
        "unit": "fwd+bwd steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "width": W, "height": H, "gaussians": wl.n, "mode": "sum",
                   "loss": {"w1": lw[0], "w2": lw[1], "ws": lw[2]}},
        "timing": "value: K steps after W warm-up steps, host clock with device syncs on both sides; "
                  "roofline: medians over batches of back-to-back gi_loss_ssim calls (one kernel) between HIP "
                  "events on the launch stream",
        "final_loss": final_loss,
        "kernels_us": {"loss_ssim": st, "loss_ssim_target_unprepared": st_full},
        "roofline": {"bound": "alu", "kernel": "k_ssim_loss", "achieved": round(tfs, 2), "peak": PEAK_FP32,
                     "unit": "TFLOP/s", "frac": round(tfs / PEAK_FP32, 4),
                     "traffic": load_traffic("k_ssim.hip", "k_ssim_loss"),
                     "avg_launch_us": round(ssim_s * 1e6, 2), "flop_per_entry": 315,
                     "hbm": {"achieved": round(gbs, 1), "peak": PEAK_HBM, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM, 4), "bytes_per_entry": 20}},
        "cpu_baseline": None,
    }
    emit(out)


def bench_absgrad(args, wlname, target, params, dev):
    """The sum backward with the per-Gaussian gather, with and without the absgrad output, on the
    workload's parameters (HIP events on the launch stream)."""
    import torch
    from rasterizer_gaussian_raster_amd.pipeline import Raster

    W, H = target.shape[2], target.shape[1]
    n = params.shape[0]
    r = Raster(W, H, n)
    r.render(params)
    dL = torch.empty_like(target)
    r.forward_l2(target, dL)
    dp = torch.zeros((n, 8), dtype=torch.float32, device=dev)
    da = torch.zeros((n, 2), dtype=torch.float32, device=dev)
    nk = max(20, min(args.steps, 500))
    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[E() for _ in range(3)] for _ in range(nk)]
    for _ in range(args.warmup):
        r.backward(dL, dp)
        r.backward_absgrad(dL, dp, da)
    for k in range(nk):
        ev[k][0].record()
        r.backward(dL, dp)
        ev[k][1].record()
        r.backward_absgrad(dL, dp, da)
        ev[k][2].record()
    torch.cuda.synchronize()
    ms = np.array([[ev[k][i].elapsed_time(ev[k][i + 1]) for i in range(2)] for k in range(nk)]).mean(0)
    plain_s, abs_s = float(ms[0]) * 1e-3, float(ms[1]) * 1e-3
    pairs = binned_pairs(W, H, r.ranges.cpu().numpy().view(np.uint32))
    tf = FLOP_BWD * pairs / abs_s / 1e12
    log(f"[bench] backward + gather {plain_s*1e6:.1f} us, with absgrad {abs_s*1e6:.1f} us")
    emit({
        "metric": METRIC, "value": round(1.0 / abs_s, 1), "unit": "backward passes/s (with absgrad)",
        "n_gpus": 1, "steps": nk, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wlname, "width": W, "height": H, "gaussians": n, "op": "absgrad"},
        "timing": "HIP events on the launch stream around gi_render_bwd and gi_render_bwd_absgrad (each with "
                  "its gather)",
        "kernels_us": {"bwd_gather": round(plain_s * 1e6, 2), "bwd_gather_absgrad": round(abs_s * 1e6, 2)},
        "roofline": {"bound": "alu", "kernel": "k_render_sum_bwd<true> (+ gather)", "achieved": round(tf, 3),
                     "peak": PEAK_FP32, "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32, 4), "traffic": None,
                     "avg_launch_us": round(abs_s * 1e6, 2)},
        "cpu_baseline": None})


def bench_merge(args, target, dev):
    """The merge phase of an overcomplete fit at 768x512: 80,000 Gaussians fitted for a few hundred
    steps, merged down to 50,000 (gi_merge_to), then fitted further; the merge pass is timed (host
    clock around the call, which waits for each round's pair count), and gi_merge_pairs alone on
    30K disjoint pairs with HIP events."""
    import torch
    from rasterizer_gaussian_raster_amd import gi, synth
    from rasterizer_gaussian_raster_amd.pipeline import Fitter, merge_to

    W, H, n, tgt_n = 768, 512, 80_000, 50_000
    w = synth.make_workload("kodak_768x512_50k", n=n)
    fit = Fitter(target, torch.from_numpy(w["params"]).to(dev), capacity_slack=2.0)
    pre = max(args.warmup, 200)
    for _ in range(pre):
        fit.step()
    torch.cuda.synchronize()
    loss_pre = float(fit.loss.item())
    merge_to(fit.params, W, H, tgt_n)                   # warm-up of the merge kernels
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    merged, rounds = merge_to(fit.params, W, H, tgt_n)
    torch.cuda.synchronize()
    t_merge = time.perf_counter() - t0
    fit2 = Fitter(target, merged, capacity_slack=2.0)
    fit2.step()
    torch.cuda.synchronize()
    loss_after = float(fit2.loss.item())
    for _ in range(pre):
        fit2.step()
    torch.cuda.synchronize()
    loss_post = float(fit2.loss.item())
    log(f"[bench] 80K fit {pre} steps: loss {loss_pre:.4e}; merge to {merged.shape[0]} in {rounds} rounds, "
        f"{t_merge*1e3:.2f} ms; loss right after {loss_after:.4e}, after {pre} more steps {loss_post:.4e}")
    # the per-pair op alone: 30K disjoint pairs
    npairs = 30000
    perm = np.random.default_rng(302).permutation(n)
    pairs = torch.from_numpy(np.stack([perm[:npairs], perm[npairs:2 * npairs]], 1).astype(np.int32)).to(dev)
    out = torch.empty((npairs, 8), dtype=torch.float32, device=dev)
    p = fit.params
    for _ in range(10):
        gi.gi_merge_pairs(npairs, pairs, n, p, out)
    nk = max(20, min(args.steps, 1000))
    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[E(), E()] for _ in range(nk)]
    for k in range(nk):
        ev[k][0].record()
        gi.gi_merge_pairs(npairs, pairs, n, p, out)
        ev[k][1].record()
    torch.cuda.synchronize()
    secs = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    nbytes = 104 * npairs             # two 32 B records + 8 B of indices read, 32 B written per pair
    gbs = nbytes / secs / 1e9
    log(f"[bench] gi_merge_pairs: {secs*1e6:.2f} us for {npairs} pairs ({gbs:.0f} GB/s algorithmic)")
    emit({
        "metric": "merge 80K -> 50K Gaussians (768x512), merges/s", "value": round((n - merged.shape[0]) / t_merge, 1),
        "unit": "merges/s", "n_gpus": 1, "steps": 1, "warmup": 1, "ms_per_step": round(t_merge * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": "merge_768x512_80k_to_50k", "gaussians": n, "target": tgt_n,
                   "result": int(merged.shape[0]), "rounds": rounds, "fit_steps_each_phase": pre},
        "loss": {"before_merge": loss_pre, "right_after": loss_after, "after_finetune": loss_post},
        "timing": "value: host clock around gi_merge_to (it waits for each round's count); "
                  "merge_pairs_us: median of HIP events around gi_merge_pairs on 30K pairs",
        "merge_pairs_us": round(secs * 1e6, 2),
        "roofline": {"bound": "hbm", "kernel": "k_merge_pairs", "achieved": round(gbs, 1), "peak": PEAK_HBM,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM, 4), "traffic": None,
                     "avg_launch_us": round(secs * 1e6, 2)},
        "cpu_baseline": None})


def bench_adc(args, target, params, dev):
    """One adaptive-density-control pass at 768x512 / 50K after some fitting (gi_adc: flags, pixel
    errors, the top-K pixel select, relocation), timed with HIP events."""
    import torch
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Fitter

    fit = Fitter(target, params, capacity_slack=2.0)
    for _ in range(max(args.warmup, 150)):
        fit.step()
    torch.cuda.synchronize()
    r = fit.raster
    d, n = r.desc, fit.n
    ws = torch.empty(gi.gi_adc_workspace_bytes(d, n), dtype=torch.uint8, device=dev)
    moved = torch.zeros(1, dtype=torch.int32, device=dev)
    P0 = fit.params.clone()
    nk = max(20, min(args.steps, 200))
    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[E(), E()] for _ in range(nk)]
    P = P0.clone()
    for k in range(nk):
        P.copy_(P0)
        ev[k][0].record()
        gi.gi_adc(d, n, P, None, None, r.image, target, 1.5, None, moved, ws)
        ev[k][1].record()
    torch.cuda.synchronize()
    us = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    mv = int(moved.item())
    log(f"[bench] gi_adc at 768x512 / {n}: median {np.median(us):.1f} us, {mv} Gaussians moved")
    emit({
        "metric": "adaptive density control pass (768x512, 50K)", "value": round(1e6 / float(np.median(us)), 1),
        "unit": "passes/s", "n_gpus": 1, "steps": nk, "warmup": 0, "ms_per_step": round(float(np.median(us)) / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "adc_768x512_50k", "gaussians": n, "moved": mv},
        "timing_us": {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
                      "p90": round(float(np.percentile(us, 90)), 2)},
        "timing": "HIP events on the launch stream around each gi_adc call (params restored between calls)",
        "cpu_baseline": None})


def bench_rs(args, wlname, target, dev):
    """Rotation-scale Gaussians on a sum workload: one step = gi_fit_step_sum without its update
    (preprocess and binning of the Cholesky form, the fused forward / L2 / backward raster, which
    finishes the sort per tile) + gi_adam_step_pairs_rs (gather of the pair sums, their map to the
    rotation-scale gradient, Adam, the loss, and the updated Gaussians' Cholesky form for the next
    step).  The breakdown times the stand-alone conversion, the fused raster on the step's binning,
    and the update pass, between HIP events."""
    import torch
    from rasterizer_gaussian_raster_amd import gi, synth
    from rasterizer_gaussian_raster_amd.pipeline import FitterRS

    w = synth.make_workload_rs(wlname)
    wl = w["workload"]
    W, H = wl.width, wl.height
    fit = FitterRS(target, torch.from_numpy(w["params_rs"]).to(dev), capacity_slack=2.0)
    for _ in range(args.warmup):
        fit.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fit.step()
    torch.cuda.synchronize()
    t_train = time.perf_counter() - t0
    r = fit.raster
    M_now = int(r.d_num[0].item()) & 0xFFFFFFFF
    assert M_now <= r.capacity, "tile-pair capacity exceeded during the timed run"
    ms_step = 1e3 * t_train / args.steps
    final_loss = float(fit.loss.item())
    log(f"[bench] rotation-scale train: {ms_step:.4f} ms/step, loss {final_loss:.4e}")

    # HIP events on the launch stream: the conversion, the fused raster, and gather + chain rule + Adam
    # (on copies of the optimiser state, so the trained parameters stay as they are)
    n = fit.n
    nk = max(20, min(args.steps, 500))
    p2, m2, v2, c2 = fit.params.clone(), fit.m.clone(), fit.v.clone(), torch.empty_like(fit.chol)
    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[E() for _ in range(4)] for _ in range(nk)]
    for k in range(nk):
        ev[k][0].record()
        gi.gi_params_to_cholesky(gi.PARAMS_RS, n, fit.params, 1.0, 1.0, fit.chol)
        ev[k][1].record()
        r.forward_backward_l2(fit.target)
        ev[k][2].record()
        gi.gi_adam_step_pairs_rs(r.desc, n, r.offsets, r.capacity, r.bwd_ws, p2, m2, v2, fit.lr, 0.9, 0.999, 1e-8,
                                 fit.step_count + 1, chol_out=c2)
        ev[k][3].record()
    torch.cuda.synchronize()
    ms = np.array([[ev[k][i].elapsed_time(ev[k][i + 1]) for i in range(3)] for k in range(nk)])
    conv_s, fused_s, chain_s = (float(x) * 1e-3 for x in ms.mean(0))
    log(f"[bench] convert {conv_s*1e6:.1f} us, fused raster {fused_s*1e6:.1f} us, gather+map+adam "
        f"{chain_s*1e6:.1f} us")
    ranges = r.ranges.cpu().numpy().view(np.uint32)
    pairs = binned_pairs(W, H, ranges)

    def roof_alu(kname, flop, secs):
        tf = flop * pairs / secs / 1e12
        return {"bound": "alu", "kernel": kname, "achieved": round(tf, 3), "peak": PEAK_FP32, "unit": "TFLOP/s",
                "frac": round(tf / PEAK_FP32, 4), "traffic": None, "avg_launch_us": round(secs * 1e6, 2)}

    def roof_hbm(kname, nbytes, secs):
        gbs = nbytes / secs / 1e9
        return {"bound": "hbm", "kernel": kname, "achieved": round(gbs, 1), "peak": PEAK_HBM, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM, 4), "traffic": None, "avg_launch_us": round(secs * 1e6, 2)}

    out = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 2),
        "unit": "fwd+bwd steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wlname, "width": W, "height": H, "gaussians": wl.n, "mode": "sum",
                   "params": "rotation-scale", "binned_pixel_pairs": pairs},
        "timing": "value: K steps after W warm-up steps, host clock with device syncs on both sides; "
                  "kernels_us: HIP events on the launch stream around each launch, on the trained parameters",
        "final_loss": final_loss,
        "kernels_us": {"params_to_cholesky": round(conv_s * 1e6, 2), "render_fwd_bwd_fused": round(fused_s * 1e6, 2),
                       "adam_pairs_rs": round(chain_s * 1e6, 2)},
        "roofline": roof_alu("k_render_sum_fused", FLOP_FWD + FLOP_BWD, fused_s),
        "roofline_convert": roof_hbm("k_params_to_cholesky", 64 * n, conv_s),
        "cpu_baseline": None,
    }
    emit(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2800)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="kodak_768x512_50k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm", action="store_true", help="skip the 3840x2160 HBM-rate measurements")
    ap.add_argument("--params", choices=["cholesky", "rs"], default="cholesky",
                    help="parameter form of the Gaussians (rs: rotation-scale, converted on the GPU each step)")
    ap.add_argument("--loss", default="l2", help="l2, or weights w1,w2,ws of w1 L1 + w2 L2 + ws (1 - SSIM)")
    ap.add_argument("--op", choices=["fit", "merge", "absgrad", "adc"], default="fit",
                    help="merge: fit 80K Gaussians, merge them down to 50K (gi_merge_to, timed), fit on; "
                         "absgrad: the sum backward with and without the absgrad output; "
                         "adc: one adaptive-density-control pass after some fitting")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (calibrates rocprofv3 FETCH/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(the multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from rasterizer_gaussian_raster_amd import gi, synth
    from rasterizer_gaussian_raster_amd.pipeline import Fitter, Raster

    gi.load()
    wlname = args.workload
    w = synth.make_workload(wlname)
    wl = w["workload"]
    W, H = wl.width, wl.height
    dev = torch.device("cuda:0")
    target = torch.from_numpy(w["target"]).to(dev)
    params = torch.from_numpy(w["params"]).to(dev)
    log(f"[bench] {wlname}: {W}x{H}, N={wl.n}, steps={args.steps}, warmup={args.warmup}")

    if args.copy_calibration:
        a = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 256 MiB device-to-device copies")
    if wl.mode != "sum":
        return bench_alpha(args, w, target, params, dev)
    if args.op == "merge":
        return bench_merge(args, target, dev)
    if args.op == "adc":
        return bench_adc(args, target, params, dev)
    if args.op == "absgrad":
        return bench_absgrad(args, wlname, target, params, dev)
    if args.params == "rs":
        return bench_rs(args, wlname, target, dev)
    if args.loss != "l2":
        return bench_ssim(args, w, target, params, dev)

    # ---------------- training step (the whole hot path) ----------------
    fit = Fitter(target, params, capacity_slack=2.0)
    r = fit.raster
    fit.track_max = True                # every step raises d_num[1] to its pair count (on the device)
    for _ in range(args.warmup):
        fit._step()
    torch.cuda.synchronize()
    r.d_num[1] = 0
    M_start = int(r.d_num[0].item()) & 0xFFFFFFFF
    # the timed region: K eager steps, no host wait in between
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fit._step()
    torch.cuda.synchronize()
    t_train = time.perf_counter() - t0
    M_max = int(r.d_num[1].item()) & 0xFFFFFFFF
    M_end = int(r.d_num[0].item()) & 0xFFFFFFFF
    assert 0 < M_max <= r.capacity, "tile-pair capacity exceeded in a timed step"
    ms_step = 1e3 * t_train / args.steps
    final_loss = float(fit.loss.item())
    log(f"[bench] train: {ms_step:.4f} ms/step, loss {final_loss:.4e}, pairs {M_start} -> {M_end} (max {M_max})")
    # per-step distribution (after the timed run): steps one by one between HIP events
    E = lambda: torch.cuda.Event(enable_timing=True)
    sev = [(E(), E()) for _ in range(40)]
    for a, b in sev:
        a.record()
        fit._step()
        b.record()
    torch.cuda.synchronize()
    step_us = np.array([a.elapsed_time(b) for a, b in sev]) * 1e3

    # ---------------- render-only: preprocess + bin/sort + raster, and raster alone ----------------
    rend = Raster(W, H, wl.n)
    rend.preprocess(fit.params)
    M = rend.bin(sync=True)
    rend.set_capacity(int(M * 1.5) + 4096)
    rend.bin(sync=True, order=True)
    # kernel timing: batches of back-to-back launches between HIP events on the launch stream, on
    # this binning: the fused raster of the training step, the forward with the L2 terms, the
    # plain forward, the backward to the pair slots
    dL = torch.empty_like(target)
    rend.forward_l2(target, dL)
    fused_us = batch_time_us(lambda: rend.forward_backward_l2(target))
    fwd_us = batch_time_us(lambda: rend.forward_l2(target, dL))
    fwd0_us = batch_time_us(lambda: rend.forward())
    rend.forward_l2(target, dL)
    bwd_us = batch_time_us(lambda: rend.backward(dL, None))
    log(f"[bench] fused fwd+bwd {np.median(fused_us):.1f} us (separate: fwd {np.median(fwd_us):.1f} us, "
        f"bwd {np.median(bwd_us):.1f} us; plain forward {np.median(fwd0_us):.1f} us)")
    render_us = batch_time_us(lambda: rend.render(fit.params, sync=False))
    t_render = float(np.median(render_us)) * 1e-6
    t_cached = float(np.median(fwd0_us)) * 1e-6
    log(f"[bench] render {t_render*1e6:.1f} us ({1/t_render:.0f} FPS), cached raster {t_cached*1e6:.1f} us")

    # ---------------- work counts of the timed problem ----------------
    rend.preprocess(fit.params)
    M = rend.bin(sync=True)
    torch.cuda.synchronize()
    ranges = rend.ranges.cpu().numpy().view(np.uint32)
    keys = rend.keys.cpu().numpy().view(np.uint32)[:M]
    vals = rend.vals.cpu().numpy().view(np.uint32)[:M]
    pixbox = rend.pixbox.cpu().numpy().view(np.uint16)
    pairs = binned_pairs(W, H, ranges)
    evald = evaluated_pairs(W, H, keys, vals, pixbox)
    fwd_s = float(np.median(fwd_us)) * 1e-6
    bwd_s = float(np.median(bwd_us)) * 1e-6
    fused_s = float(np.median(fused_us)) * 1e-6

    def roof(kname, flop, secs, us):
        tf = flop * pairs / secs / 1e12
        return {"bound": "alu", "kernel": kname, "achieved": round(tf, 3), "peak": PEAK_FP32,
                "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32, 4),
                "traffic": load_traffic("k_raster_sum.hip", kname), "avg_launch_us": round(secs * 1e6, 2),
                "launch_us": stats_us(us)}

    roof_fwd = roof("k_render_sum_fwd<true>", FLOP_FWD, fwd_s, fwd_us)
    # the same launch priced on the pairs the kernel evaluates (its quadrant lists)
    tf_e = FLOP_FWD * evald / fwd_s / 1e12
    roof_fwd["achieved_on_evaluated_pairs"] = round(tf_e, 3)
    roof_fwd["frac_on_evaluated_pairs"] = round(tf_e / PEAK_FP32, 4)
    roof_bwd = roof("k_render_sum_bwd<false>", FLOP_BWD, bwd_s, bwd_us)
    roof_fused = roof("k_render_sum_fused", FLOP_FWD + FLOP_BWD, fused_s, fused_us)

    out = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 2),
        "unit": "fwd+bwd steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wlname, "width": W, "height": H, "gaussians": wl.n, "mode": "sum",
                   "tiles": int(rend.T), "tile_pairs": int(M), "binned_pixel_pairs": pairs,
                   "evaluated_pixel_pairs_fwd": evald,
                   "tile_pairs_timed_steps": {"first": M_start, "last": M_end, "max": M_max}},
        "step_us": stats_us(step_us),
        "render_fps": round(1.0 / t_render, 1),
        "mpix_per_s": round(W * H / t_render / 1e6, 1),
        "cached_raster_fps": round(1.0 / t_cached, 1),
        "render_us": stats_us(render_us),
        "projected_fit_seconds_2800_steps": round(2800 * ms_step / 1e3, 3),
        "timing": "value: K steps after W warm-up steps, host clock with device syncs on both sides; step_us: "
                  "40 later steps one by one between HIP events; kernels and render: medians over batches of 20 "
                  "back-to-back launches between HIP events on the launch stream, on the trained parameters' "
                  "binning (work counts of that binning)",
        "final_loss": final_loss,
        "kernels_us": {"render_fwd_bwd_fused": round(fused_s * 1e6, 2), "render_fwd_l2": round(fwd_s * 1e6, 2),
                       "render_fwd": round(t_cached * 1e6, 2), "render_bwd": round(bwd_s * 1e6, 2)},
        "roofline": roof_fused,
        "roofline_fwd": roof_fwd,
        "roofline_bwd": roof_bwd,
    }
    if not args.no_hbm:
        log("[bench] HBM rates of the memory-bound kernels at 3840x2160 / 2M ...")
        out["hbm_3840x2160_2m"] = hbm_rates_4k(dev)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a pixel sample ...")
        out["cpu_baseline"] = cpu_baseline(wl, w["params"])
    else:
        out["cpu_baseline"] = None
    emit(out)


def hbm_rates_4k(dev):
    """Achieved HBM rate (algorithmic bytes / time) of the preprocess, the binning (all its kernels)
    and the Adam pass with the per-pair gather on the 3840x2160 / 2M workload, whose buffers (64 MB of
    params, 70+ MB of pairs) exceed the caches: medians of batches of back-to-back calls."""
    import torch
    from rasterizer_gaussian_raster_amd import gi, synth
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    w = synth.make_workload("render_3840x2160_2m")
    W, H, n = 3840, 2160, w["workload"].n
    P = torch.from_numpy(w["params"]).to(dev)
    r = Raster(W, H, n)
    r.preprocess(P)
    M = r.bin(sync=True)
    r.set_capacity(int(M * 1.25) + 4096)
    r.bin(sync=True)
    T = r.T
    pre = batch_time_us(lambda: r.preprocess(P), per_batch=10, batches=7)
    bins = batch_time_us(lambda: r.bin(sync=False, order=False), per_batch=5, batches=7)
    G = torch.zeros((3, H, W), dtype=torch.float32, device=dev)
    G[:, ::7, ::5] = 1e-3
    r.backward(G, None)
    Mo, V = torch.zeros_like(P), torch.zeros_like(P)
    Pc = P.clone()
    lr = [0.0] * 8                                  # the update pass itself, params left unchanged
    adam = batch_time_us(lambda: gi.gi_adam_step_pairs(r.desc, n, r.offsets, r.capacity, r.bwd_ws, Pc, Mo, V, lr,
                                                       0.9, 0.999, 1e-8, 1), per_batch=10, batches=7)
    rows = {
        "k_preprocess": (32 + 44) * n,
        "binning (gi_bin_sort)": 12 * n + 4 * n + (8 + 8 + 8) * M + 8 * T,
        "k_adam_pairs": (3 * 32 * 2 + 4) * n + 32 * M,
    }
    out = {"gaussians": n, "tile_pairs": M, "tiles": T,
           "bytes_per_unit": {"k_preprocess": "32 B read + 44 B written per Gaussian",
                              "binning (gi_bin_sort)": "12 B read + 4 B written per Gaussian; 8 B written (first "
                                                       "pass), 8 B read + 8 B written (bucket pass) per pair; "
                                                       "8 B per tile",
                              "k_adam_pairs": "p, m, v read and written (192 B) + offsets (4 B) per Gaussian, "
                                              "32 B per pair slot"}}
    for name, us in (("k_preprocess", pre), ("binning (gi_bin_sort)", bins), ("k_adam_pairs", adam)):
        t = float(np.median(us)) * 1e-6
        gbs = rows[name] / t / 1e9
        out[name] = {"us": stats_us(us), "algorithmic_bytes": int(rows[name]), "achieved_gbs": round(gbs, 1),
                     "frac_of_8tbs": round(gbs / PEAK_HBM, 4)}
        log(f"[bench]   {name}: {t*1e6:.1f} us, {gbs:.0f} GB/s ({gbs / PEAK_HBM:.2f} of 8 TB/s)")
    return out

if __name__ == "__main__":
    main()
