"""Helpers for the GPU parity tests: device transfers, the HIP path, and the error metrics.

Image metric: max over (channel, pixel) of |I_gpu - I_ref| / S, S = the oracle's sum of
|colour| x weight at that pixel (0/0 counts as 0; S = 0 requires I_gpu == 0 exactly).
Gradient metric: |g_gpu - g_ref| / C per entry, C = the oracle's running-error scale (sum over
pairs of each contribution with its inner sums taken over absolute values).
"""
import numpy as np
import pytest
import torch

IMAGE_TOL = 1e-5
GRAD_TOL = 1e-4


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rasterizer_gaussian_raster_amd import gi
    gi.load()           # raises if libgi.so is missing: never a silent fallback
    return gi


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def u32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def u16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def gpu_bin(W, H, params, logit=None, capacity=None, fused=False):
    """Preprocess and bin on the GPU: two calls, or gi_preprocess_bin_sort when fused."""
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    n = params.shape[0]
    mode = gi.MODE_ALPHA if logit is not None else gi.MODE_SUM
    r = Raster(W, H, n, mode, capacity=capacity)
    P, L = dev(params), None if logit is None else dev(logit)
    if fused:
        M = r.bin(sync=True, params=P, logit=L)
    else:
        r.preprocess(P, L)
        M = r.bin(sync=True)
    torch.cuda.synchronize()
    return r, {
        "M": M,
        "counts": u32(r.counts)[:n],
        "pixbox": u16(r.pixbox)[:n].astype(np.int64),
        "offsets": u32(r.offsets),
        "keys": u32(r.keys)[:M],
        "vals": u32(r.vals)[:M],
        "ranges": u32(r.ranges)[: r.T],
    }


def image_error(gpu, ref, sabs):
    gpu = np.asarray(gpu, np.float64)
    diff = np.abs(gpu - ref)
    zero = sabs == 0
    if np.any(gpu[zero] != 0):
        return np.inf
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(zero, 0.0, diff / np.where(zero, 1.0, sabs))
    return float(rel.max()) if rel.size else 0.0


def grad_error(gpu, ref, aabs):
    gpu = np.asarray(gpu, np.float64)
    diff = np.abs(gpu - ref)
    zero = aabs == 0
    if np.any(gpu[zero] != 0):
        return np.inf
    rel = np.where(zero, 0.0, diff / np.where(zero, 1.0, aabs))
    return float(rel.max()) if rel.size else 0.0


def grad_error_plain(gpu, ref, aabs, cond, factor=10.0):
    """The plain metric |g_gpu - g_ref| / A (A = sum of |contribution|) over the entries where the
    running-error scale C is at most factor * A (no contribution there is much of a cancellation),
    and the number of such entries."""
    gpu = np.asarray(gpu, np.float64)
    m = (aabs > 0) & (cond <= factor * aabs)
    if not np.any(m):
        return 0.0, 0
    return float((np.abs(gpu[m] - ref[m]) / aabs[m]).max()), int(m.sum())


def sample_pixels(W, H, n_random, n_tiles, seed):
    """n_random random pixels plus every pixel of n_tiles random tiles, as [P,2] (row, col)."""
    rng = np.random.default_rng(seed)
    pix = [np.stack([rng.integers(0, H, n_random), rng.integers(0, W, n_random)], 1)]
    tx, ty = -(-W // 16), -(-H // 16)
    for t in rng.choice(tx * ty, size=min(n_tiles, tx * ty), replace=False):
        x0, y0 = (t % tx) * 16, (t // tx) * 16
        yy, xx = np.mgrid[y0:min(y0 + 16, H), x0:min(x0 + 16, W)]
        pix.append(np.stack([yy.ravel(), xx.ravel()], 1))
    return np.concatenate(pix).astype(np.int32)


def pixel_tile_start(W, ranges, pix):
    tx = -(-W // 16)
    t = (pix[:, 0] // 16) * tx + pix[:, 1] // 16
    return ranges[t, 0]


def gpu_last_to_index(last, vals, starts):
    """GPU `last` (one past the list position of the last composited Gaussian, or the tile's range
    start) -> Gaussian index, -1 when none."""
    last = np.asarray(last, np.int64)
    out = np.full(last.shape, -1, np.int64)
    has = last > starts
    out[has] = vals[last[has] - 1]
    return out
