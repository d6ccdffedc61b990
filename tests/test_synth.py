"""Seeded input generators: shapes, ranges, determinism."""
import numpy as np

from rasterizer_gaussian_raster_amd import synth


def test_workload_shapes_and_ranges():
    for name in ["tiny_fit_64x64", "kodak_768x512_50k"]:
        w = synth.make_workload(name)
        wl = w["workload"]
        assert w["target"].shape == (3, wl.height, wl.width)
        assert w["target"].dtype == np.float32
        assert 0.0 <= w["target"].min() and w["target"].max() <= 1.0
        p = w["params"]
        assert p.shape == (wl.n, 8) and p.dtype == np.float32
        assert np.all((p[:, 0] >= 0) & (p[:, 0] <= wl.width) & (p[:, 1] >= 0) & (p[:, 1] <= wl.height))
        assert np.all((p[:, 2] >= wl.sigma[0] * 0.999) & (p[:, 2] <= wl.sigma[1] * 1.001))
        assert np.all((p[:, 5:] >= 0) & (p[:, 5:] <= 1))


def test_alpha_workload_small():
    g = synth.make_gaussians(1000, 2048, 2048, (0.5, 16), 0.5, 4, alpha=True)
    p, lg = g
    assert lg.shape == (1000,) and abs(lg.mean() + 2) < 0.2


def test_deterministic():
    a = synth.make_workload("tiny_fit_64x64")
    b = synth.make_workload("tiny_fit_64x64")
    np.testing.assert_array_equal(a["params"], b["params"])
    np.testing.assert_array_equal(a["target"], b["target"])
