"""GPU binning vs the oracle: pixel boxes, tile counts, offsets, M, sorted keys/vals and tile ranges
must be bit-identical."""
import numpy as np
import pytest
import torch

from gpu_util import dev, gpu_bin, require_gpu, u32
from rasterizer_gaussian_raster_amd import synth

pytestmark = pytest.mark.gpu


def _check_bin(W, H, params, logit=None, fused=False):
    import oracle
    ref = oracle.bin(W, H, params.astype(np.float64), None if logit is None else logit.astype(np.float64))
    box, _ = oracle.footprint(W, H, params.astype(np.float64),
                              None if logit is None else logit.astype(np.float64))
    _, got = gpu_bin(W, H, params, logit, fused=fused)
    assert got["M"] == ref["M"]
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    nz = ref["counts"] > 0
    np.testing.assert_array_equal(got["pixbox"][nz], box[nz])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["keys"], ref["keys"])
    np.testing.assert_array_equal(got["vals"], ref["vals"])
    np.testing.assert_array_equal(got["ranges"], ref["ranges"])
    return got


@pytest.mark.parametrize("seed,W,H,n,sig,margin", [
    (101, 64, 64, 256, (0.5, 6.0), 0),
    (102, 100, 37, 500, (0.3, 12.0), 20),
    (103, 17, 33, 60, (0.3, 8.0), 10),
    (104, 300, 200, 3000, (0.3, 20.0), 30),
    (105, 1, 1, 10, (0.3, 2.0), 2),
    (106, 257, 129, 2000, (0.3, 40.0), 50),
])
@pytest.mark.parametrize("fused", [False, True])
def test_bin_random_cases(seed, W, H, n, sig, margin, fused):
    require_gpu()
    p = synth.random_case(seed, W, H, n, sigma=sig, margin=margin)
    _check_bin(W, H, p, fused=fused)


@pytest.mark.parametrize("name", ["tiny_fit_64x64", "kodak_768x512_50k", "div2k_1020x678_70k"])
def test_bin_workloads_full(name):
    require_gpu()
    w = synth.make_workload(name)
    wl = w["workload"]
    _check_bin(wl.width, wl.height, w["params"])


def _check_bin_properties(W, H, p, lg, got):
    """A binning checked by its defining properties against the oracle's footprint: counts, M, offsets
    (the exclusive scan of the counts), keys/vals (every (tile, index) pair of the boxes exactly once,
    sorted by tile and stably by index) and the tile ranges."""
    import oracle
    box, cnt = oracle.footprint(W, H, p.astype(np.float64), None if lg is None else lg.astype(np.float64))
    np.testing.assert_array_equal(got["counts"], cnt)
    assert got["M"] == int(cnt.astype(np.int64).sum())
    np.testing.assert_array_equal(got["offsets"], np.concatenate([[0], np.cumsum(cnt.astype(np.int64))]))
    keys, vals = got["keys"].astype(np.int64), got["vals"].astype(np.int64)
    assert np.all(np.diff(keys) >= 0)
    same = np.diff(keys) == 0
    assert np.all(np.diff(vals)[same] > 0)          # stable: ascending index within a tile
    # every (tile, index) pair of the boxes appears exactly once
    tx = -(-W // 16)
    nz = cnt > 0
    j0, i0, j1, i1 = (box[nz, k] // 16 for k in range(4))
    idx = np.nonzero(nz)[0]
    w_t = (j1 - j0 + 1)
    exp_cnt = w_t * (i1 - i0 + 1)
    rep = np.repeat(np.arange(len(idx)), exp_cnt)
    r_ = np.arange(len(rep)) - np.repeat(np.cumsum(exp_cnt) - exp_cnt, exp_cnt)
    ek = (i0[rep] + r_ // w_t[rep]) * tx + j0[rep] + r_ % w_t[rep]
    ev = idx[rep]
    order = np.lexsort((ev, ek))
    np.testing.assert_array_equal(keys, ek[order])
    np.testing.assert_array_equal(vals, ev[order])
    rg = got["ranges"].astype(np.int64)
    T = rg.shape[0]
    lo = np.searchsorted(keys, np.arange(T), "left")
    hi = np.searchsorted(keys, np.arange(T), "right")
    np.testing.assert_array_equal(rg[:, 0], np.where(hi > lo, lo, 0))
    np.testing.assert_array_equal(rg[:, 1], np.where(hi > lo, hi, 0))


@pytest.mark.parametrize("name", ["alpha_2048x2048_500k", "render_3840x2160_2m"])
def test_bin_large_workloads(name):
    """Full-size binning checked by its defining properties; a 5% subset checked bit-exactly."""
    require_gpu()
    w = synth.make_workload(name)
    wl = w["workload"]
    W, H = wl.width, wl.height
    p = w["params"]
    lg = w["logit"]
    r, got = gpu_bin(W, H, p, lg)
    _check_bin_properties(W, H, p, lg, got)
    # bit-exact against the oracle's definition on a 5% subset
    sub = np.random.default_rng(7).choice(wl.n, size=wl.n // 20, replace=False)
    sub.sort()
    _check_bin(W, H, p[sub], None if lg is None else lg[sub])


def test_bin_more_than_8192_groups():
    """2,200,000 small Gaussians: more than 8192 groups of 256, so the single-workgroup scan of the
    group sums takes more than one round of its register-held loads."""
    require_gpu()
    W, H, n = 512, 512, 2_200_000
    p = synth.random_case(211, W, H, n, sigma=(0.3, 1.5), margin=4)
    _, got = gpu_bin(W, H, p, None)
    _check_bin_properties(W, H, p, None, got)


@pytest.mark.parametrize("fused", [False, True])
def test_bin_edge_cases(fused):
    require_gpu()
    W, H = 70, 45
    # empty set
    _check_bin(W, H, np.zeros((0, 8), np.float32), fused=fused)
    # all off-image
    p = synth.random_case(1, W, H, 50)
    p[:, 0] += 1000
    got = _check_bin(W, H, p, fused=fused)
    assert got["M"] == 0 and np.all(got["ranges"] == 0)
    # tiny Gaussians between pixel centres, huge Gaussians covering every tile, culled parameters
    p = synth.random_case(2, W, H, 40)
    p[:10, 2] = 0.01
    p[:10, 4] = 0.01
    p[:10, 3] = 0.0
    p[10:15, 2] = 500.0
    p[10:15, 4] = 300.0
    p[15, 0] = np.nan
    p[16, 2] = 0.0
    p[17, 4] = 0.0
    p[18, 6] = np.inf
    p[19, 4] = 1e-39
    got = _check_bin(W, H, p, fused=fused)
    assert np.all(got["counts"][15:20] == 0)
    assert np.all(got["counts"][10:15] == (-(-W // 16)) * (-(-H // 16)))


def test_bin_long_tile_list():
    """One tile holding more than 65,536 Gaussians (long lists, many sort blocks per digit)."""
    require_gpu()
    n = 70_000
    rng = np.random.default_rng(3)
    p = np.zeros((n, 8), np.float32)
    p[:, 0] = rng.uniform(2, 14, n)
    p[:, 1] = rng.uniform(2, 14, n)
    p[:, 2] = rng.uniform(0.3, 0.6, n)
    p[:, 4] = rng.uniform(0.3, 0.6, n)
    p[:, 5:] = rng.uniform(0, 1, (n, 3))
    got = _check_bin(64, 48, p)
    assert got["ranges"][0, 1] - got["ranges"][0, 0] == n


def test_bin_large_boxes():
    """Groups of 256 Gaussians with far more pairs than one 4096-key sort chunk."""
    require_gpu()
    p = synth.random_case(11, 640, 600, 700, sigma=(20.0, 150.0), margin=100)
    got = _check_bin(640, 600, p)
    assert got["M"] > 40 * 4096


def test_bin_capacity_overflow():
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    W, H = 128, 96
    p = synth.random_case(5, W, H, 400, sigma=(1, 10))
    r = Raster(W, H, 400)
    r.preprocess(dev(p))
    M = r.bin(sync=True)
    r2 = Raster(W, H, 400, capacity=M - 1)
    r2.preprocess(dev(p))
    with pytest.raises(gi.GiError) as ei:
        gi.gi_bin_sort(r2.desc, r2.n, r2.pixbox, r2.counts, r2.offsets, r2.keys, r2.vals, r2.ranges,
                       r2.capacity, r2.d_num, r2.ws, sync_count=True)
    assert ei.value.status == gi.GI_ERR_CAPACITY
    torch.cuda.synchronize()
    assert int(u32(r2.d_num)[0]) == M
    assert np.all(u32(r2.ranges) == 0)
    # asynchronous form: no error, overflow visible in d_num, ranges empty
    r2.bin(sync=False)
    torch.cuda.synchronize()
    assert int(u32(r2.d_num)[0]) == M and np.all(u32(r2.ranges) == 0)


def test_bin_repeatable():
    require_gpu()
    p = synth.random_case(9, 300, 200, 3000, sigma=(0.3, 20.0))
    _, a = gpu_bin(300, 200, p)
    _, b = gpu_bin(300, 200, p)
    for k in ["keys", "vals", "ranges", "offsets"]:
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("capacity", [None, 1 << 20])
def test_bin_lsd_more_than_16_key_bits(fused, capacity):
    """A grid of more than 65,536 tiles (17 key bits): the LSD passes (k_count / k_scatter, then
    k_ranges), with small and larger sort blocks; bit-exact against the oracle, and the image of
    that binning against the oracle on sampled pixels."""
    require_gpu()
    import oracle
    from gpu_util import image_error, sample_pixels
    W, H, n = 4400, 4000, 3000                       # 275 x 250 = 68,750 tiles
    p = synth.random_case(107, W, H, n, sigma=(0.3, 40.0), margin=50)
    ref = oracle.bin(W, H, p.astype(np.float64))
    r, got = gpu_bin(W, H, p, capacity=capacity if capacity else None, fused=fused)
    print(f"[lsd] {W}x{H}: M = {got['M']}, capacity {r.capacity}", flush=True)
    for k in ["counts", "offsets", "keys", "vals", "ranges"]:
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    assert got["M"] == ref["M"]
    img = r.forward().cpu().numpy()
    pix = sample_pixels(W, H, 2048, 4, seed=108)
    want, S = oracle.render_sum(W, H, p.astype(np.float64), pixels=pix)
    assert image_error(img[:, pix[:, 0], pix[:, 1]], want, S) <= 1e-5


@pytest.mark.parametrize("fused", [False, True])
def test_bin_lsd_capacity_above_bucket_limit(fused):
    """A pair buffer of 2^26 + 1 entries takes the LSD passes even at 11 key bits (the bucket pass
    is limited to 2^26); bit-exact against the oracle."""
    require_gpu()
    import oracle
    W, H, n = 768, 512, 3000
    p = synth.random_case(109, W, H, n, sigma=(0.3, 30.0), margin=20)
    ref = oracle.bin(W, H, p.astype(np.float64))
    r, got = gpu_bin(W, H, p, capacity=(1 << 26) + 1, fused=fused)
    print(f"[lsd] {W}x{H}: M = {got['M']}, capacity {r.capacity}", flush=True)
    for k in ["counts", "offsets", "keys", "vals", "ranges"]:
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    del r
    torch.cuda.empty_cache()
