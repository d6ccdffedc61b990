"""Divergence recovery in the fit loop (Fitter.guarded_steps): a loss spike injected from the host
(the colours of the set blown up between two checks) is rolled back to the last good check, bit for
bit, and the fit goes on."""
import numpy as np
import pytest
import torch

from gpu_util import dev, require_gpu
from rasterizer_gaussian_raster_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("alpha", [False, True])
def test_loss_spike_is_rolled_back(alpha):
    require_gpu()
    from rasterizer_gaussian_raster_amd.pipeline import Fitter
    w = synth.make_workload("tiny_fit_64x64", n=300)
    kw = {}
    if alpha:
        rng = np.random.default_rng(5)
        kw = dict(logit=dev(rng.normal(-1.0, 0.5, 300).astype(np.float32)),
                  background=dev(np.full(3, 0.5, np.float32)))
    fit = Fitter(dev(w["target"]), dev(w["params"]), **kw)
    assert fit.guarded_steps(20)
    assert fit.guarded_steps(20)
    good = [t.detach().clone() for t in fit._state()]
    good_step, good_loss = fit.step_count, float(fit.loss.item())
    fit.params[:, 5:] *= 1e4                     # the injected spike
    assert not fit.guarded_steps(5)
    assert fit.step_count == good_step
    for t, g in zip(fit._state(), good):
        np.testing.assert_array_equal(t.cpu().numpy().view(np.uint32), g.cpu().numpy().view(np.uint32))
    assert fit.guarded_steps(20)
    last = float(fit.loss.item())
    print(f"{'alpha' if alpha else 'sum'}: loss at the good check {good_loss:.4e}, after recovery {last:.4e}")
    assert np.isfinite(last) and last < good_loss


def test_non_finite_loss_is_rolled_back():
    require_gpu()
    from rasterizer_gaussian_raster_amd.pipeline import Fitter
    w = synth.make_workload("tiny_fit_64x64", n=200)
    fit = Fitter(dev(w["target"]), dev(w["params"]))
    assert fit.guarded_steps(10)
    good = fit.params.detach().clone()
    fit.params[3, 5:] = 3e38                     # finite, but its pixels' squared residuals overflow: L = inf
    assert not fit.guarded_steps(2)
    np.testing.assert_array_equal(fit.params.cpu().numpy().view(np.uint32), good.cpu().numpy().view(np.uint32))
