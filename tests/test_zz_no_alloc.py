"""gi_render_image_noalloc (the library's fixed bin workspace, no allocation) against gi_render_image
(caller's workspace): every output bit for bit, on two calls in a row -- the second a smaller
problem -- so that the second call runs over what the first left in the fixed array; the alpha mode
too; and the size limit (GI_ERR_UNSUPPORTED before anything is enqueued)."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import dev, require_gpu, u32
from rasterizer_gaussian_raster_amd import synth

pytestmark = pytest.mark.gpu


def _outputs(r, M):
    o = [u32(r.image), u32(r.offsets), u32(r.keys)[:M], u32(r.vals)[:M], u32(r.ranges)[: r.T],
         u32(r.records)[: r.n], u32(r.pixbox.view(torch.int32))[: r.n], u32(r.counts)[: r.n], u32(r.d_num)[:1]]
    if r.t_final is not None:
        o += [u32(r.t_final), u32(r.last)]
    return o


def _render_both(W, H, p, logit=None, bg=None, order_flags=0):
    """(M, outputs) of gi_render_image and of gi_render_image_noalloc on fresh buffers of the same size."""
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    n = p.shape[0]
    mode = gi.MODE_ALPHA if logit is not None else gi.MODE_SUM
    P, L = dev(p), None if logit is None else dev(logit)
    B = None if bg is None else dev(bg)
    res = []
    for noalloc in (False, True):
        r = Raster(W, H, n, mode)
        M0 = r.bin(sync=True, params=P, logit=L)
        r.set_capacity(int(M0 * 1.5) + 1024)
        r.image.fill_(-1.0)
        r.ranges.fill_(-1)
        flags = order_flags if r.order is not None else 0
        if noalloc:
            M = gi.gi_render_image_noalloc(r.desc, n, P, L, B, r.records, r.opacity, r.pixbox, r.counts, r.offsets,
                                           r.keys, r.vals, r.ranges, r.order, flags, r.capacity, r.d_num, r.image,
                                           r.t_final, r.last, sync_count=True)
        else:
            M = gi.gi_render_image(r.desc, n, P, L, B, r.records, r.opacity, r.pixbox, r.counts, r.offsets, r.keys,
                                   r.vals, r.ranges, r.order, flags, r.capacity, r.d_num, r.ws, r.image, r.t_final,
                                   r.last, sync_count=True)
        torch.cuda.synchronize()
        res.append((M, _outputs(r, M)))
    return res


def _check_same(res, what):
    (Ma, a), (Mb, b) = res
    assert Ma == Mb, what
    for k, (x, y) in enumerate(zip(a, b)):
        np.testing.assert_array_equal(x, y, err_msg=f"{what}: output {k}")


def test_noalloc_render_equals_render_image_two_calls():
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    w = synth.make_workload("kodak_768x512_50k")
    print("[noalloc] 768x512, 50000 Gaussians", flush=True)
    big = _render_both(768, 512, w["params"], order_flags=gi.FIT_ORDER)
    _check_same(big, "768x512 / 50K")
    # the second call: a smaller image and fewer Gaussians, over the first call's leftovers
    print("[noalloc] 300x200, 4000 Gaussians", flush=True)
    small = _render_both(300, 200, synth.random_case(81, 300, 200, 4000, sigma=(0.3, 20.0), margin=20))
    _check_same(small, "300x200 / 4000")
    print(f"[noalloc] M = {big[0][0]}, then {small[0][0]}", flush=True)


def test_noalloc_alpha_and_empty():
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    rng = np.random.default_rng(82)
    W, H, n = 200, 150, 3000
    p = synth.random_case(83, W, H, n, sigma=(0.5, 10.0), margin=10)
    lg = rng.normal(-1.0, 1.0, n).astype(np.float32)
    bg = np.array([0.2, 0.5, 0.7, 0.0], np.float32)
    print("[noalloc] alpha 200x150, 3000 Gaussians", flush=True)
    _check_same(_render_both(W, H, p, lg, bg), "alpha 200x150")
    print("[noalloc] empty set", flush=True)
    _check_same(_render_both(70, 45, np.zeros((0, 8), np.float32)), "empty")


def test_noalloc_rejects_problems_beyond_the_fixed_workspace():
    """A bin workspace above gi_render_image_noalloc_max_bytes() is refused with GI_ERR_UNSUPPORTED
    and nothing is written."""
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    lib = gi.load()
    cap_max = lib.gi_render_image_noalloc_max_bytes()
    assert cap_max == 64 << 20
    W, H, n = 256, 256, 1000
    r = Raster(W, H, n)
    d = r.desc
    big = 1
    while gi.gi_bin_sort_workspace_bytes(d, n, big) <= cap_max:
        big *= 2
    P = dev(synth.random_case(84, W, H, n))
    r.set_capacity(1024)
    r.image.fill_(-1.0)
    torch.cuda.synchronize()
    with pytest.raises(gi.GiError) as e:
        gi.gi_render_image_noalloc(d, n, P, None, None, r.records, None, r.pixbox, r.counts, r.offsets, r.keys,
                                   r.vals, r.ranges, None, 0, big, r.d_num, r.image)
    assert e.value.status == gi.GI_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert float(r.image.max()) == -1.0 and float(r.image.min()) == -1.0
