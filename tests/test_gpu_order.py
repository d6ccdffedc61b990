"""The tile order of gi_bin_sort only schedules work: it must be a permutation of the tiles ranked by
list length and dealt in serpentine layers of the CU count, and every raster output must be
bit-identical with and without it."""
import numpy as np
import pytest
import torch

from gpu_util import dev, require_gpu, u32
from rasterizer_gaussian_raster_amd import synth

pytestmark = pytest.mark.gpu


def _serpentine(p, period, n):
    layer, c = divmod(p, period)
    base = layer * period
    width = min(period, n - base)
    return base + (width - 1 - c if layer % 2 else c)


def _check_order(r):
    """A permutation of the tiles; read in rank order (launch position serp(rank)), the list
    lengths are non-increasing."""
    order = u32(r.order)[: r.T].astype(np.int64)
    rg = u32(r.ranges)[: r.T].astype(np.int64)
    np.testing.assert_array_equal(np.sort(order), np.arange(r.T))
    period = torch.cuda.get_device_properties(0).multi_processor_count
    pos = np.array([_serpentine(p, period, r.T) for p in range(r.T)])
    np.testing.assert_array_equal(np.sort(pos), np.arange(r.T))
    ln = np.minimum(rg[:, 1] - rg[:, 0], 1023)[order[pos]]
    assert np.all(np.diff(ln) <= 0)


@pytest.mark.parametrize("case", ["kodak_768x512_50k", "div2k_1020x678_70k", "random_300x200", "single_tile"])
def test_tile_order_is_serpentine_by_length(case):
    require_gpu()
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    if case == "random_300x200":
        W, H, p = 300, 200, synth.random_case(31, 300, 200, 3000, sigma=(0.3, 20.0))
    elif case == "single_tile":
        W, H, p = 13, 9, synth.random_case(32, 13, 9, 50)
    else:           # 1536 tiles (6 full layers of 256) and 2752 (a partial last layer)
        w = synth.make_workload(case)
        W, H, p = w["workload"].width, w["workload"].height, w["params"]
    r = Raster(W, H, p.shape[0])
    r.preprocess(dev(p))
    r.bin(sync=True)
    torch.cuda.synchronize()
    _check_order(r)


def test_sum_outputs_do_not_depend_on_tile_order():
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    w = synth.make_workload("kodak_768x512_50k")
    W, H, n = 768, 512, 50_000
    r = Raster(W, H, n)
    P, T = dev(w["params"]), dev(w["target"])
    r.render(P)
    G = dev(np.random.default_rng(8).normal(size=(3, H, W)).astype(np.float32) * 1e-4)
    ws = torch.empty(gi.gi_render_bwd_workspace_bytes(r.desc, n, r.capacity), dtype=torch.uint8, device="cuda")
    outs = []
    for order in (r.order, None):
        img = torch.empty_like(T)
        dL = torch.empty_like(T)
        lp = torch.empty_like(r.loss_partials)
        gi.gi_render_fwd_l2(r.desc, n, r.records, r.pixbox, r.ranges, r.vals, T, img, dL, lp, tile_order=order)
        d = torch.zeros_like(P)
        gi.gi_render_bwd(r.desc, n, r.records, None, None, r.pixbox, r.offsets, r.ranges, r.vals, r.capacity,
                         None, None, None, G, d, None, None, ws, tile_order=order)
        torch.cuda.synchronize()
        outs.append([img.cpu().numpy(), dL.cpu().numpy(), lp.cpu().numpy(), d.cpu().numpy()])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_alpha_outputs_do_not_depend_on_tile_order():
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    W, H = 300, 200
    p, lg, bg = synth.random_case(192, W, H, 4000, sigma=(0.5, 16.0), alpha=True)
    n = p.shape[0]
    r = Raster(W, H, n, gi.MODE_ALPHA)
    P, L, B = dev(p), dev(lg), dev(bg)
    r.render(P, L, B)
    G = dev(np.random.default_rng(9).normal(size=(3, H, W)).astype(np.float32))
    ws = torch.empty(gi.gi_render_bwd_workspace_bytes(r.desc, n, r.capacity), dtype=torch.uint8, device="cuda")
    outs = []
    for order in (r.order, None):
        img = torch.empty((3, H, W), dtype=torch.float32, device="cuda")
        tf = torch.empty((H, W), dtype=torch.float32, device="cuda")
        last = torch.empty((H, W), dtype=torch.int32, device="cuda")
        gi.gi_render_fwd(r.desc, n, r.records, r.opacity, r.pixbox, r.ranges, r.vals, B, img, tf, last,
                         tile_order=order)
        dp = torch.zeros_like(P)
        dl = torch.zeros_like(L)
        db = torch.zeros(3, dtype=torch.float32, device="cuda")
        gi.gi_render_bwd(r.desc, n, r.records, r.opacity, L, r.pixbox, r.offsets, r.ranges, r.vals, r.capacity,
                         B, tf, last, G, dp, dl, db, ws, tile_order=order)
        torch.cuda.synchronize()
        outs.append([img.cpu().numpy(), tf.cpu().numpy(), last.cpu().numpy(), dp.cpu().numpy(),
                     dl.cpu().numpy(), db.cpu().numpy()])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
