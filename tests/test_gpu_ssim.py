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


def _gpu_ssim(x, y, w, prepared=False):
    """gi_loss_ssim; prepared: the target's statistics from gi_loss_ssim_target first."""
    from rasterizer_gaussian_raster_amd import gi
    _, H, W = x.shape
    X, Y = dev(x.astype(np.float32)), dev(y.astype(np.float32))
    dL = torch.empty_like(X)
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(gi.gi_loss_ssim_workspace_bytes(W, H), dtype=torch.uint8, device="cuda")
    if prepared:
        gi.gi_loss_ssim_target(W, H, Y, ws)
    gi.gi_loss_ssim(W, H, X, Y, *w, dL, loss, ws, flags=gi.SSIM_TARGET_PREPARED if prepared else 0)
    torch.cuda.synchronize()
    return float(loss.item()), dL.cpu().numpy()


def _check(x, y, w, prepared=False):
    import oracle
    L, g = _gpu_ssim(x, y, w, prepared)
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
                                   (5, 3, (0.8, 0.0, 0.2)), (1, 1, (0.5, 0.5, 0.5)), (300, 200, (0.8, 0.0, 0.2)),
                                   (131, 97, (0.8, 0.1, 0.2))])
def test_ssim_random(W, H, w):
    require_gpu()
    rng = np.random.default_rng(W * 1000 + H)
    y = rng.uniform(0, 1, (3, H, W))
    x = np.clip(y + rng.normal(0, 0.1, y.shape), -0.2, 1.2)
    _check(x, y, w)


@pytest.mark.parametrize("W,H", [(64, 64), (100, 37), (1, 1), (300, 200)])
def test_ssim_prepared_target_is_the_same_bits(W, H):
    """With the target's statistics formed once (gi_loss_ssim_target), the loss and gradient are the
    unprepared call's bits, and both meet the oracle."""
    require_gpu()
    rng = np.random.default_rng(W * 7 + H)
    y = rng.uniform(0, 1, (3, H, W))
    x = np.clip(y + rng.normal(0, 0.1, y.shape), -0.2, 1.2)
    w = (0.8, 0.1, 0.2)
    L0, g0 = _gpu_ssim(x, y, w)
    L1, g1 = _check(x, y, w, prepared=True)
    assert np.float32(L0).view(np.uint32) == np.float32(L1).view(np.uint32)
    np.testing.assert_array_equal(g0.view(np.uint32), g1.view(np.uint32))


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


def test_ssim_loss_pointer_optional_and_unaligned_planes():
    """Calls without d_loss leave the workspace ready for calls with it (the loss is the same bits each
    time), and planes that are not 16-byte aligned (element-wise staging) give the bits of aligned ones."""
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    W, H = 96, 70
    rng = np.random.default_rng(903)
    y = rng.uniform(0, 1, (3, H, W)).astype(np.float32)
    x = np.clip(y + rng.normal(0, 0.1, y.shape), -0.2, 1.2).astype(np.float32)
    X, Y = dev(x), dev(y)
    ws = torch.empty(gi.gi_loss_ssim_workspace_bytes(W, H), dtype=torch.uint8, device="cuda")
    gi.gi_loss_ssim_target(W, H, Y, ws)
    w = (0.8, 0.1, 0.2)
    losses, grads = [], []
    for with_loss in (True, False, False, True, True):
        dL = torch.empty_like(X)
        loss = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        gi.gi_loss_ssim(W, H, X, Y, *w, dL, loss if with_loss else None, ws, flags=gi.SSIM_TARGET_PREPARED)
        torch.cuda.synchronize()
        if with_loss:
            losses.append(float(loss.item()))
        else:
            assert float(loss.item()) == -1.0
        grads.append(dL.cpu().numpy())
    assert losses[0] == losses[1] == losses[2]
    for g in grads[1:]:
        np.testing.assert_array_equal(g.view(np.uint32), grads[0].view(np.uint32))
    # planes one element past a 16-byte boundary
    xb = torch.zeros(X.numel() + 1, dtype=torch.float32, device="cuda")
    xb[1:] = X.reshape(-1)
    Xu = xb[1:].view(3, H, W)
    assert Xu.data_ptr() % 16 != 0
    dLu = torch.empty_like(X)
    lu = torch.zeros(1, dtype=torch.float32, device="cuda")
    gi.gi_loss_ssim(W, H, Xu, Y, *w, dLu, lu, ws, flags=gi.SSIM_TARGET_PREPARED)
    torch.cuda.synchronize()
    assert float(lu.item()) == losses[0]
    np.testing.assert_array_equal(dLu.cpu().numpy().view(np.uint32), grads[0].view(np.uint32))


@pytest.mark.parametrize("case", ["small", "kodak_768x512_50k"])
def test_ssim_fit_step_matches_separate_calls(case):
    """gi_fit_step_sum_ssim (Fitter.step with the SSIM loss: binning, forward, loss, backward into the
    pair slots, Adam with the set-up of the next binning) against the separate calls (binning,
    forward, gi_loss_ssim, backward with the gather, gi_adam_step): the same bits every step.  At
    768x512 (more than 256 tiles) the forward finishes the sort per tile, and the 20 steps cross a
    tile-order refresh."""
    require_gpu()
    from rasterizer_gaussian_raster_amd.pipeline import Fitter
    if case == "small":
        p = synth.random_case(321, 96, 80, 600, sigma=(0.5, 8.0))
        tgt = np.random.default_rng(322).uniform(0, 1, (3, 80, 96)).astype(np.float32)
    else:
        wl = synth.make_workload(case)
        p, tgt = wl["params"], wl["target"]
    w = (0.8, 0.1, 0.2)
    a = Fitter(dev(tgt), dev(p), loss=w)
    b = Fitter(dev(tgt), dev(p), loss=w)
    for k in range(20):
        a.step()
        b.step_separate()
        if k in (0, 19):
            torch.cuda.synchronize()
            for x, y in [(a.params, b.params), (a.m, b.m), (a.v, b.v), (a.loss, b.loss), (a.dL, b.dL)]:
                np.testing.assert_array_equal(x.cpu().numpy().view(np.uint32), y.cpu().numpy().view(np.uint32))
    print(f"ssim fit step: loss {a.loss.item():.6e} after 20 steps")
