"""GPU forward images vs the oracle (max relative error <= 1e-5 under the S-weighted metric),
bitwise determinism, and alpha-mode stopping points."""
import numpy as np
import pytest
import torch

from gpu_util import (IMAGE_TOL, dev, gpu_last_to_index, image_error, pixel_tile_start, require_gpu,
                      sample_pixels, u32)
from rasterizer_gaussian_raster_amd import synth

pytestmark = pytest.mark.gpu


def _render_sum(W, H, params):
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    r = Raster(W, H, params.shape[0])
    img = r.render(dev(params)).clone()
    torch.cuda.synchronize()
    return r, img.cpu().numpy()


@pytest.mark.parametrize("seed,W,H,n,sig,margin", [
    (111, 64, 64, 256, (0.5, 6.0), 0),
    (112, 100, 37, 600, (0.3, 12.0), 20),
    (113, 17, 33, 80, (0.3, 8.0), 10),
    (114, 300, 200, 3000, (0.3, 20.0), 30),
    (115, 257, 129, 1500, (0.3, 40.0), 50),
])
def test_sum_image_full(seed, W, H, n, sig, margin):
    require_gpu()
    import oracle
    p = synth.random_case(seed, W, H, n, sigma=sig, margin=margin)
    _, img = _render_sum(W, H, p)
    ref, S = oracle.render_sum(W, H, p.astype(np.float64))
    err = image_error(img, ref, S)
    print(f"sum image {W}x{H} n={n}: max rel err {err:.3e}")
    assert err <= IMAGE_TOL


@pytest.mark.parametrize("name,nrand,ntiles", [("tiny_fit_64x64", 0, 0), ("kodak_768x512_50k", 0, 0),
                                               ("div2k_1020x678_70k", 0, 0),
                                               ("render_3840x2160_2m", 512, 2)])
def test_sum_image_workloads(name, nrand, ntiles):
    """Full frames (nrand = 0: every pixel against the oracle's sum over all N Gaussians), or
    sampled pixels plus whole tiles at 3840x2160 / 2M."""
    require_gpu()
    import oracle
    w = synth.make_workload(name)
    wl = w["workload"]
    W, H = wl.width, wl.height
    _, img = _render_sum(W, H, w["params"])
    p64 = w["params"].astype(np.float64)
    if nrand == 0:
        ref, S = oracle.render_sum(W, H, p64)
        err = image_error(img, ref, S)
    else:
        pix = sample_pixels(W, H, nrand, ntiles, seed=wl.seed)
        ref, S = oracle.render_sum(W, H, p64, pixels=pix)
        err = image_error(img[:, pix[:, 0], pix[:, 1]], ref, S)
    print(f"{name}: max rel err {err:.3e}")
    assert err <= IMAGE_TOL


def test_sum_forward_is_bitwise_reproducible():
    require_gpu()
    w = synth.make_workload("kodak_768x512_50k")
    _, a = _render_sum(768, 512, w["params"])
    _, b = _render_sum(768, 512, w["params"])
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_sum_edge_cases():
    require_gpu()
    import oracle
    W, H = 70, 45
    # no Gaussians: zero image
    _, img = _render_sum(W, H, np.zeros((0, 8), np.float32))
    assert np.all(img == 0)
    # culled and degenerate parameters leave the others' image unchanged
    p = synth.random_case(3, W, H, 40)
    base = p[20:].copy()
    p[0, 0] = np.nan
    p[1, 2] = 0.0
    p[2, 7] = np.inf
    p[3, 4] = 1e-39
    p[4:10, 2] = 0.01          # hits no pixel centre
    p[4:10, 4] = 0.01
    p[4:10, 0] = np.floor(p[4:10, 0])
    p[4:10, 1] = np.floor(p[4:10, 1])
    p[10:12, 2] = 400.0        # one Gaussian in every tile
    p[10:12, 4] = 300.0
    _, img = _render_sum(W, H, p)
    assert np.all(np.isfinite(img))
    ref, S = oracle.render_sum(W, H, p.astype(np.float64))
    assert image_error(img, ref, S) <= IMAGE_TOL
    _, img2 = _render_sum(W, H, np.concatenate([p[4:20], base]))
    ref2, S2 = oracle.render_sum(W, H, np.concatenate([p[4:20], base]).astype(np.float64))
    assert image_error(img2, ref2, S2) <= IMAGE_TOL


def test_sum_long_list():
    require_gpu()
    import oracle
    n = 70_000
    rng = np.random.default_rng(3)
    p = np.zeros((n, 8), np.float32)
    p[:, 0] = rng.uniform(2, 14, n)
    p[:, 1] = rng.uniform(2, 14, n)
    p[:, 2] = rng.uniform(0.3, 0.6, n)
    p[:, 4] = rng.uniform(0.3, 0.6, n)
    p[:, 5:] = rng.uniform(0, 1, (n, 3))
    _, img = _render_sum(32, 32, p)
    ref, S = oracle.render_sum(32, 32, p.astype(np.float64))
    assert image_error(img, ref, S) <= IMAGE_TOL


# ------------------------------------------------------------------------------------------------
# alpha mode
# ------------------------------------------------------------------------------------------------

def _render_alpha(W, H, params, logit, bg):
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    r = Raster(W, H, params.shape[0], gi.MODE_ALPHA)
    img = r.render(dev(params), dev(logit), dev(bg)).clone()
    torch.cuda.synchronize()
    return r, img.cpu().numpy(), r.t_final.cpu().numpy(), u32(r.last).astype(np.int64)


def _check_alpha(W, H, p, lg, bg, pix=None):
    import oracle
    r, img, tf, last = _render_alpha(W, H, p, lg, bg)
    vals = u32(r.vals)[: r.M].astype(np.int64)
    ranges = u32(r.ranges).astype(np.int64)
    if pix is None:
        yy, xx = np.mgrid[0:H, 0:W]
        pix = np.stack([yy.ravel(), xx.ravel()], 1).astype(np.int32)
    gl = gpu_last_to_index(last[pix[:, 0], pix[:, 1]], vals, pixel_tile_start(W, ranges, pix))
    p64, l64, b64 = p.astype(np.float64), lg.astype(np.float64), bg.astype(np.float64)
    own = oracle.render_alpha(W, H, p64, l64, b64, pixels=pix)
    # the stop is unique wherever no transmittance met by the stop test is within 1e-3 of 1e-4
    amb = own["ambiguous"].astype(bool)
    np.testing.assert_array_equal(gl[~amb], own["last"][~amb])
    forced = oracle.render_alpha(W, H, p64, l64, b64, pixels=pix, force_last=gl)
    g_img = img[:, pix[:, 0], pix[:, 1]]
    err = image_error(g_img, forced["image"], forced["sabs"])
    t_err = np.max(np.abs(tf[pix[:, 0], pix[:, 1]] - forced["t_final"]) / np.maximum(forced["t_final"], 1e-30))
    stopped = (forced["t_final"] < 1e-4).mean()
    print(f"alpha {W}x{H}: max rel err {err:.3e}, T rel err {t_err:.3e}, stopped {stopped:.3f}, "
          f"ambiguous {amb.sum()}")
    assert err <= IMAGE_TOL
    assert t_err <= 1e-4
    return stopped


@pytest.mark.parametrize("seed,W,H,n", [(121, 64, 64, 256), (122, 100, 37, 500), (123, 17, 33, 60)])
def test_alpha_image_random(seed, W, H, n):
    require_gpu()
    p, lg, bg = synth.random_case(seed, W, H, n, sigma=(0.5, 8.0), alpha=True, margin=10)
    _check_alpha(W, H, p, lg, bg)


def test_alpha_termination_stress():
    """64x64, 2000 opaque Gaussians (o in [0.5, 0.95], sigma 4-12 px): most pixels stop early."""
    require_gpu()
    rng = np.random.default_rng(131)
    n = 2000
    p = np.zeros((n, 8), np.float32)
    p[:, 0] = rng.uniform(0, 64, n)
    p[:, 1] = rng.uniform(0, 64, n)
    p[:, 2] = rng.uniform(4, 12, n)
    p[:, 3] = rng.normal(0, 0.5, n)
    p[:, 4] = rng.uniform(4, 12, n)
    p[:, 5:] = rng.uniform(0, 1, (n, 3))
    o = rng.uniform(0.5, 0.95, n)
    lg = np.log(o / (1 - o)).astype(np.float32)
    bg = np.array([0.2, 0.4, 0.6], np.float32)
    stopped = _check_alpha(64, 64, p, lg, bg)
    assert stopped > 0.9


def test_alpha_workload_sampled():
    require_gpu()
    w = synth.make_workload("alpha_2048x2048_500k")
    wl = w["workload"]
    pix = sample_pixels(wl.width, wl.height, 768, 2, seed=wl.seed)
    _check_alpha(wl.width, wl.height, w["params"], w["logit"], w["background"], pix)


def test_alpha_forward_is_bitwise_reproducible():
    require_gpu()
    p, lg, bg = synth.random_case(141, 300, 200, 4000, sigma=(0.5, 16.0), alpha=True)
    _, a, ta, la = _render_alpha(300, 200, p, lg, bg)
    _, b, tb, lb = _render_alpha(300, 200, p, lg, bg)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    np.testing.assert_array_equal(la, lb)
