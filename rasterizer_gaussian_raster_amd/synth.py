"""Seeded synthetic inputs: targets and Gaussian sets of the benchmark workloads.

This module holds only input generation (random numbers, target images and
initial Gaussian parameters); it contains none of the rasterizer's arithmetic
and imports neither the HIP binding nor the oracle, so both sides may use it.

The pages fit Kodak (768x512) and DIV2K-valid-LR-X2 (about 1020x678) images
("GaussianImage", quick start datasets; "FlashImgs", bench).  Those datasets
are not available here; the targets below are synthetic stand-ins of the same
shapes: band-limited sinusoids with step edges, and 1/f ("natural image")
spectral noise with filled polygons.  Nothing from the datasets is reproduced.

Parameter layout (one Gaussian = 8 fp32): mux, muy, l11, l21, l22, cr, cg, cb.
Means are in pixels; (l11, l21, l22) is the lower-triangular Cholesky factor
of the covariance; colours are the weighted colour channels.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_target", "make_gaussians", "make_workload", "random_case"]


@dataclass(frozen=True)
class Workload:
    name: str
    width: int
    height: int
    n: int
    sigma: tuple            # (min, max) of the log-uniform Cholesky diagonal, px
    offdiag_std: float      # std of the N(0, s) Cholesky off-diagonal
    means: str              # "uniform" | "gradient"
    target: str             # "sines" | "noise_poly" | "noise" | "none"
    mode: str = "sum"       # "sum" | "alpha"
    seed: int = 0
    steps: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny_fit_64x64": Workload("tiny_fit_64x64", 64, 64, 256, (0.5, 6.0), 0.3, "uniform", "sines",
                               seed=1, steps=300),
    "kodak_768x512_50k": Workload("kodak_768x512_50k", 768, 512, 50_000, (0.5, 8.0), 0.3, "gradient",
                                  "noise_poly", seed=2, steps=2800),
    "div2k_1020x678_70k": Workload("div2k_1020x678_70k", 1020, 678, 70_000, (0.5, 10.0), 0.3,
                                   "gradient", "noise", seed=3, steps=200),
    "alpha_2048x2048_500k": Workload("alpha_2048x2048_500k", 2048, 2048, 500_000, (0.5, 16.0), 0.5,
                                     "uniform", "noise", mode="alpha", seed=4, steps=200),
    "render_3840x2160_2m": Workload("render_3840x2160_2m", 3840, 2160, 2_000_000, (0.3, 12.0), 0.5,
                                    "uniform", "none", seed=5),
}


def _sines(rng, H, W):
    yy, xx = np.mgrid[0:H, 0:W].astype(np.float64)
    img = np.full((3, H, W), 0.5)
    for k in range(3):
        for _ in range(8):
            amp = rng.uniform(0.0, 0.15)
            f = rng.uniform(0.5, 8.0)
            th = rng.uniform(0, 2 * np.pi)
            ph = rng.uniform(0, 2 * np.pi)
            img[k] += amp * np.sin(2 * np.pi * f * (np.cos(th) * xx / W + np.sin(th) * yy / H) + ph)
    for _ in range(4):
        px, py = rng.uniform(0, W), rng.uniform(0, H)
        th = rng.uniform(0, 2 * np.pi)
        side = (np.cos(th) * (xx - px) + np.sin(th) * (yy - py)) > 0
        step = rng.uniform(-0.3, 0.3, 3)
        for k in range(3):
            img[k] += step[k] * side
    return np.clip(img, 0.0, 1.0)


def _pink(rng, H, W):
    fy = np.fft.fftfreq(H)[:, None]
    fx = np.fft.rfftfreq(W)[None, :]
    f = np.sqrt(fx * fx + fy * fy)
    f[0, 0] = np.inf
    out = np.empty((3, H, W))
    for k in range(3):
        spec = (rng.normal(size=f.shape) + 1j * rng.normal(size=f.shape)) / f
        x = np.fft.irfft2(spec, s=(H, W))
        out[k] = (x - x.min()) / (x.max() - x.min())
    return out


def _polygons(rng, img, count=12):
    _, H, W = img.shape
    for _ in range(count):
        nv = int(rng.integers(3, 9))
        cx, cy = rng.uniform(0, W), rng.uniform(0, H)
        rad = rng.uniform(0.05, 0.3) * min(W, H)
        ang = np.sort(rng.uniform(0, 2 * np.pi, nv))
        r = rad * rng.uniform(0.4, 1.0, nv)
        vx, vy = cx + r * np.cos(ang), cy + r * np.sin(ang)
        col = rng.uniform(0, 1, 3)
        x0, x1 = int(max(0, np.floor(vx.min()))), int(min(W, np.ceil(vx.max()) + 1))
        y0, y1 = int(max(0, np.floor(vy.min()))), int(min(H, np.ceil(vy.max()) + 1))
        if x0 >= x1 or y0 >= y1:
            continue
        yy, xx = np.mgrid[y0:y1, x0:x1].astype(np.float64) + 0.5
        inside = np.zeros(xx.shape, bool)
        for a in range(nv):                      # even-odd ray casting
            b = (a + 1) % nv
            cond = (vy[a] > yy) != (vy[b] > yy)
            xint = vx[a] + (yy - vy[a]) * (vx[b] - vx[a]) / (vy[b] - vy[a] + 1e-300)
            inside ^= cond & (xx < xint)
        for k in range(3):
            img[k, y0:y1, x0:x1][inside] = col[k]
    return img


def make_target(kind: str, W: int, H: int, seed: int) -> np.ndarray:
    """[3,H,W] float32 target in [0,1] (zeros for kind "none")."""
    rng = np.random.default_rng([seed, 7])
    if kind == "sines":
        img = _sines(rng, H, W)
    elif kind == "noise_poly":
        img = _polygons(rng, _pink(rng, H, W))
    elif kind == "noise":
        img = _pink(rng, H, W)
    elif kind == "none":
        img = np.zeros((3, H, W))
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(img, dtype=np.float32)


def make_gaussians(n, W, H, sigma, offdiag_std, seed, means="uniform", target=None, alpha=False):
    """[n,8] float32 params (and [n] float32 logit opacities when alpha)."""
    rng = np.random.default_rng([seed, 11])
    p = np.zeros((n, 8), np.float64)
    if means == "gradient" and target is not None:
        gy, gx = np.gradient(target.astype(np.float64), axis=(1, 2))
        wgt = np.sqrt(gx * gx + gy * gy).sum(axis=0).reshape(-1) + 1e-6
        idx = rng.choice(wgt.size, size=n, p=wgt / wgt.sum())
        p[:, 0] = (idx % W) + rng.uniform(0, 1, n)
        p[:, 1] = (idx // W) + rng.uniform(0, 1, n)
    else:
        p[:, 0] = rng.uniform(0, W, n)
        p[:, 1] = rng.uniform(0, H, n)
    lo, hi = np.log(sigma[0]), np.log(sigma[1])
    p[:, 2] = np.exp(rng.uniform(lo, hi, n))
    p[:, 3] = rng.normal(0.0, offdiag_std, n)
    p[:, 4] = np.exp(rng.uniform(lo, hi, n))
    p[:, 5:8] = rng.uniform(0.0, 1.0, (n, 3))
    params = np.ascontiguousarray(p, dtype=np.float32)
    if alpha:
        logit = np.ascontiguousarray(rng.normal(-2.0, 1.0, n), dtype=np.float32)
        return params, logit
    return params


def make_workload(name: str, n: int | None = None):
    """dict(workload, target [3,H,W], params [N,8], logit [N] or None, background [3] or None)."""
    wl = WORKLOADS[name]
    N = wl.n if n is None else n
    tgt = make_target(wl.target, wl.width, wl.height, wl.seed)
    alpha = wl.mode == "alpha"
    g = make_gaussians(N, wl.width, wl.height, wl.sigma, wl.offdiag_std, wl.seed, wl.means, tgt,
                       alpha=alpha)
    params, logit = (g if alpha else (g, None))
    bg = np.full(3, 0.5, np.float32) if alpha else None
    return {"workload": wl, "target": tgt, "params": params, "logit": logit, "background": bg}


def make_gaussians_rs(n, W, H, sigma, seed, means="uniform", target=None):
    """[n,8] float32 rotation-scale params (mux, muy, sx, sy, theta, cr, cg, cb): means as
    make_gaussians, scales log-uniform over sigma, theta uniform over (-pi, pi]."""
    rng = np.random.default_rng([seed, 17])
    p = np.zeros((n, 8), np.float64)
    if means == "gradient" and target is not None:
        gy, gx = np.gradient(target.astype(np.float64), axis=(1, 2))
        wgt = np.sqrt(gx * gx + gy * gy).sum(axis=0).reshape(-1) + 1e-6
        idx = rng.choice(wgt.size, size=n, p=wgt / wgt.sum())
        p[:, 0] = (idx % W) + rng.uniform(0, 1, n)
        p[:, 1] = (idx // W) + rng.uniform(0, 1, n)
    else:
        p[:, 0] = rng.uniform(0, W, n)
        p[:, 1] = rng.uniform(0, H, n)
    lo, hi = np.log(sigma[0]), np.log(sigma[1])
    p[:, 2] = np.exp(rng.uniform(lo, hi, n))
    p[:, 3] = np.exp(rng.uniform(lo, hi, n))
    p[:, 4] = rng.uniform(-np.pi, np.pi, n)
    p[:, 5:8] = rng.uniform(0.0, 1.0, (n, 3))
    return np.ascontiguousarray(p, dtype=np.float32)


def make_workload_rs(name: str, n: int | None = None):
    """A sum-mode workload with rotation-scale Gaussians of the same sizes and distributions:
    dict(workload, target [3,H,W], params_rs [N,8])."""
    wl = WORKLOADS[name]
    if wl.mode != "sum":
        raise ValueError("rotation-scale workloads are sum-mode")
    N = wl.n if n is None else n
    tgt = make_target(wl.target, wl.width, wl.height, wl.seed)
    prs = make_gaussians_rs(N, wl.width, wl.height, wl.sigma, wl.seed, wl.means, tgt)
    return {"workload": wl, "target": tgt, "params_rs": prs}


def random_case_rs(seed, W, H, n, sigma=(0.5, 6.0), margin=0.0):
    """Small seeded rotation-scale parity case (signed scales, any angle)."""
    rng = np.random.default_rng([seed, 19])
    p = np.zeros((n, 8), np.float64)
    p[:, 0] = rng.uniform(-margin, W + margin, n)
    p[:, 1] = rng.uniform(-margin, H + margin, n)
    lo, hi = np.log(sigma[0]), np.log(sigma[1])
    p[:, 2] = np.exp(rng.uniform(lo, hi, n)) * rng.choice([-1.0, 1.0], n)
    p[:, 3] = np.exp(rng.uniform(lo, hi, n)) * rng.choice([-1.0, 1.0], n)
    p[:, 4] = rng.uniform(-4.0, 4.0, n)
    p[:, 5:8] = rng.uniform(-0.2, 1.0, (n, 3))
    return np.ascontiguousarray(p, dtype=np.float32)


def random_case(seed, W, H, n, sigma=(0.5, 6.0), offdiag_std=0.3, alpha=False, margin=0.0):
    """Small seeded parity case; margin extends the mean range beyond the image (px)."""
    rng = np.random.default_rng([seed, 13])
    p = np.zeros((n, 8), np.float64)
    p[:, 0] = rng.uniform(-margin, W + margin, n)
    p[:, 1] = rng.uniform(-margin, H + margin, n)
    lo, hi = np.log(sigma[0]), np.log(sigma[1])
    p[:, 2] = np.exp(rng.uniform(lo, hi, n)) * rng.choice([-1.0, 1.0], n)
    p[:, 3] = rng.normal(0.0, offdiag_std, n)
    p[:, 4] = np.exp(rng.uniform(lo, hi, n)) * rng.choice([-1.0, 1.0], n)
    p[:, 5:8] = rng.uniform(-0.2, 1.0, (n, 3))
    params = np.ascontiguousarray(p, dtype=np.float32)
    if alpha:
        logit = np.ascontiguousarray(rng.normal(-2.0, 1.0, n), dtype=np.float32)
        bg = np.ascontiguousarray(rng.uniform(0, 1, 3), dtype=np.float32)
        return params, logit, bg
    return params
