"""The sum-mode training step captured as HIP graphs: every replay must leave exactly the state the
eager step leaves (parameters, Adam moments, loss), with eager work and synchronisations between the
replays, across the steps that refresh the tile order."""
import numpy as np
import pytest
import torch

from gpu_util import dev, require_gpu
from rasterizer_gaussian_raster_amd import synth

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("name,steps", [("tiny_fit_64x64", 40), ("kodak_768x512_50k", 36)])
def test_graph_replays_match_eager_steps(name, steps):
    require_gpu()
    from rasterizer_gaussian_raster_amd.pipeline import Fitter
    w = synth.make_workload(name)
    T, P = dev(w["target"]), dev(w["params"])
    eager = Fitter(T, P, capacity_slack=2.0)
    graph = Fitter(T, P, capacity_slack=2.0)
    graph.capture(warmup=2)                      # two real steps, then the graphs
    for _ in range(2):
        eager.step()
    torch.cuda.synchronize()
    for name_, a, b in [("params", eager.params, graph.params), ("m", eager.m, graph.m), ("v", eager.v, graph.v)]:
        np.testing.assert_array_equal(_bits(a), _bits(b), err_msg=f"after warm-up: {name_}")
    for k in range(steps):
        eager.step()
        graph.step()
        torch.cuda.synchronize()
        assert graph.step_count == eager.step_count
        for name_, a, b in [("params", eager.params, graph.params), ("m", eager.m, graph.m),
                            ("v", eager.v, graph.v), ("loss", eager.loss, graph.loss)]:
            np.testing.assert_array_equal(_bits(a), _bits(b), err_msg=f"replay {k}: {name_}")
        assert int(graph.d_step.item()) == graph.step_count
