"""The SSIM pixel loss on the GPU (gi_loss_ssim) vs the oracle's fp64 definition.

Bounds: loss |L_gpu - L_ref| <= 1e-5 * (|w1| L1 + |w2| L2 + |ws| (1 + mean|SSIM map|));
dL/dI per entry <= 1e-4 * the oracle's running-error scale of the gradient (every sum and inner sum
of the formula over absolute values)."""
import numpy as np
import pytest
import torch

from gpu_util import dev, require_gpu
from rasterizer_gaussian_raster_amd import synth

pytestmark = pytest.mark.gpu


def _gpu_ssim(x, y, w):
    from rasterizer_gaussian_raster_amd import gi
    _, H, W = x.shape
    X, Y = dev(x.astype(np.float32)), dev(y.astype(np.float32))
    dL = torch.empty_like(X)
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(gi.gi_loss_ssim_workspace_bytes(W, H), dtype=torch.uint8, device="cuda")
    gi.gi_loss_ssim(W, H, X, Y, *w, dL, loss, ws)
    torch.cuda.synchronize()
    return float(loss.item()), dL.cpu().numpy()


def _check(x, y, w):
    import oracle
    L, g = _gpu_ssim(x, y, w)
    r = oracle.loss_ssim(x.astype(np.float32).astype(np.float64), y.astype(np.float32).astype(np.float64), *w)
    e = x.astype(np.float64) - y
    scale = abs(w[0]) * np.abs(e).mean() + abs(w[1]) * (e * e).mean() + abs(w[2]) * (1 + np.abs(r["map"]).mean())
    lerr = abs(L - r["loss"]) / scale
    gerr = float((np.abs(g - r["grad"]) / np.where(r["scale"] > 0, r["scale"], 1.0)).max())
    print(f"ssim {x.shape} w={w}: loss {L:.6f} (ref {r['loss']:.6f}) rel err {lerr:.2e}; grad rel err {gerr:.2e}")
    assert lerr <= 1e-5
    assert gerr <= 1e-4
    return L, g


@pytest.mark.parametrize("W,H,w", [(64, 64, (0.8, 0.0, 0.2)), (100, 37, (0.0, 1.0, 0.2)), (17, 33, (0.7, 0.1, 0.3)),
                                   (5, 3, (0.8, 0.0, 0.2)), (1, 1, (0.5, 0.5, 0.5)), (300, 200, (0.8, 0.0, 0.2))])
def test_ssim_random(W, H, w):
    require_gpu()
    rng = np.random.default_rng(W * 1000 + H)
    y = rng.uniform(0, 1, (3, H, W))
    x = np.clip(y + rng.normal(0, 0.1, y.shape), -0.2, 1.2)
    _check(x, y, w)


def test_ssim_workload():
    """The 768x512 target against a perturbed copy (a fitted render stands in)."""
    require_gpu()
    w = synth.make_workload("kodak_768x512_50k")
    y = w["target"].astype(np.float64)
    x = y + np.random.default_rng(901).normal(0, 0.05, y.shape)
    _check(x, y, (0.8, 0.0, 0.2))


def test_ssim_identical_and_deterministic():
    require_gpu()
    rng = np.random.default_rng(902)
    y = rng.uniform(0, 1, (3, 40, 50))
    L, g = _gpu_ssim(y, y, (0.8, 0.0, 0.2))
    assert abs(L) < 1e-6
    x = y + rng.normal(0, 0.1, y.shape)
    L1, g1 = _gpu_ssim(x, y, (0.8, 0.0, 0.2))
    L2, g2 = _gpu_ssim(x, y, (0.8, 0.0, 0.2))
    assert L1 == L2
    np.testing.assert_array_equal(g1.view(np.uint32), g2.view(np.uint32))


def test_fit_with_ssim_loss():
    require_gpu()
    from rasterizer_gaussian_raster_amd.pipeline import Fitter
    w = synth.make_workload("tiny_fit_64x64")
    fit = Fitter(dev(w["target"]), dev(w["params"]), loss=(0.8, 0.0, 0.2))
    fit.step()
    torch.cuda.synchronize()
    first = float(fit.loss.item())
    for _ in range(60):
        fit.step()
    torch.cuda.synchronize()
    last = float(fit.loss.item())
    print(f"ssim fit: loss {first:.4e} -> {last:.4e}")
    assert np.isfinite(last) and last < 0.8 * first
