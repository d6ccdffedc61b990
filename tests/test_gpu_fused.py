"""The fused entry points must give exactly what the separate calls give:
gi_preprocess_bin_sort == gi_preprocess then gi_bin_sort (every output, bit for bit), and the loss
reduced in the backward launch (d_loss) == gi_loss_reduce, with unchanged gradients."""
import numpy as np
import pytest
import torch

from gpu_util import dev, require_gpu, u32
from rasterizer_gaussian_raster_amd import synth

pytestmark = pytest.mark.gpu


def _outputs(r, M):
    out = {"records": u32(r.records)[: r.n], "pixbox": r.pixbox.cpu().numpy()[: r.n],
           "counts": u32(r.counts)[: r.n], "offsets": u32(r.offsets), "keys": u32(r.keys)[:M],
           "vals": u32(r.vals)[:M], "ranges": u32(r.ranges)[: r.T], "d_num": u32(r.d_num)}
    if r.opacity is not None:
        out["opacity"] = u32(r.opacity)[: r.n]
    if r.order is not None:
        out["order_len"] = np.minimum(np.diff(out["ranges"].astype(np.int64), axis=1)[:, 0], 1023)[
            u32(r.order)[: r.T].astype(np.int64)]
    return out


def _case(name):
    if name == "kodak_768x512_50k" or name == "render_3840x2160_2m":
        w = synth.make_workload(name)
        return w["workload"].width, w["workload"].height, w["params"], w["logit"]
    if name == "alpha_300x200":
        p, lg, _ = synth.random_case(51, 300, 200, 4000, sigma=(0.5, 16.0), alpha=True)
        return 300, 200, p, lg
    if name == "empty":
        return 70, 45, np.zeros((0, 8), np.float32), None
    if name == "off_image":
        p = synth.random_case(52, 70, 45, 50)
        p[:, 0] += 1000
        return 70, 45, p, None
    if name == "large_boxes":
        return 640, 600, synth.random_case(11, 640, 600, 700, sigma=(20.0, 150.0), margin=100), None
    raise KeyError(name)


@pytest.mark.parametrize("name", ["kodak_768x512_50k", "alpha_300x200", "empty", "off_image", "large_boxes",
                                  "render_3840x2160_2m"])
def test_preprocess_bin_sort_equals_two_calls(name):
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    W, H, p, lg = _case(name)
    n = p.shape[0]
    mode = gi.MODE_ALPHA if lg is not None else gi.MODE_SUM
    P, L = dev(p), None if lg is None else dev(lg)
    outs = []
    for fused in (False, True):
        r = Raster(W, H, n, mode)
        if fused:
            M = r.bin(sync=True, params=P, logit=L)
        else:
            r.preprocess(P, L)
            M = r.bin(sync=True)
        # a second, asynchronous pass over the same buffers (stale contents in ranges and workspace)
        if fused:
            r.bin(sync=False, order=True, params=P, logit=L)
        else:
            r.preprocess(P, L)
            r.bin(sync=False, order=True)
        torch.cuda.synchronize()
        outs.append(_outputs(r, M))
    a, b = outs
    assert a.keys() == b.keys()
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_fused_capacity_overflow_reports_like_bin_sort():
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    W, H = 128, 96
    p = dev(synth.random_case(5, W, H, 400, sigma=(1, 10)))
    r = Raster(W, H, 400)
    M = r.bin(sync=True, params=p)
    r2 = Raster(W, H, 400, capacity=M - 1)
    with pytest.raises(gi.GiError) as ei:
        gi.gi_preprocess_bin_sort(r2.desc, r2.n, p, None, r2.records, None, r2.pixbox, r2.counts, r2.offsets,
                                  r2.keys, r2.vals, r2.ranges, r2.capacity, r2.d_num, r2.ws, sync_count=True)
    assert ei.value.status == gi.GI_ERR_CAPACITY
    torch.cuda.synchronize()
    assert int(u32(r2.d_num)[0]) == M and np.all(u32(r2.ranges) == 0)


@pytest.mark.parametrize("name", ["tiny_fit_64x64", "kodak_768x512_50k", "div2k_1020x678_70k"])
def test_backward_loss_equals_loss_reduce(name):
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    w = synth.make_workload(name)
    wl = w["workload"]
    W, H, n = wl.width, wl.height, wl.n
    r = Raster(W, H, n)
    P, T = dev(w["params"]), dev(w["target"])
    r.render(P)
    dL = torch.empty_like(T)
    r.forward_l2(T, dL)
    ref = torch.full((1,), -1.0, device="cuda")
    gi.gi_loss_reduce(r.T, r.loss_partials, T.numel(), ref)
    d0 = torch.zeros_like(P)
    r.backward(dL, d0)
    g0 = r.bwd_ws.clone()
    d1 = torch.zeros_like(P)
    got = torch.full((1,), -2.0, device="cuda")
    r.backward(dL, d1, d_loss=got)
    g1 = r.bwd_ws.clone()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u32(got), u32(ref))
    np.testing.assert_array_equal(u32(d1), u32(d0))
    np.testing.assert_array_equal(g1.cpu().numpy(), g0.cpu().numpy())
    # pair-gradient form (dparams NULL), as the fit step calls it
    got2 = torch.full((1,), -3.0, device="cuda")
    r.backward(dL, None, d_loss=got2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u32(got2), u32(ref))


def test_backward_loss_argument_checks():
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    W, H = 64, 48
    p = dev(synth.random_case(7, W, H, 100))
    r = Raster(W, H, 100)
    r.render(p)
    G = torch.zeros((3, H, W), device="cuda")
    loss = torch.zeros(1, device="cuda")
    r.backward(G, None)                 # sizes the workspace
    with pytest.raises(gi.GiError):     # d_loss without the partials
        gi.gi_render_bwd(r.desc, r.n, r.records, None, None, r.pixbox, r.offsets, r.ranges, r.vals, r.capacity,
                         None, None, None, G, None, None, None, r.bwd_ws, d_loss=loss)
    with pytest.raises(gi.GiError):     # count < 1
        gi.gi_render_bwd(r.desc, r.n, r.records, None, None, r.pixbox, r.offsets, r.ranges, r.vals, r.capacity,
                         None, None, None, G, None, None, None, r.bwd_ws, loss_partials=r.loss_partials,
                         loss_count=0, d_loss=loss)


def _fused_case(name):
    if name in ("tiny_fit_64x64", "kodak_768x512_50k", "div2k_1020x678_70k"):
        w = synth.make_workload(name)
        return w["workload"].width, w["workload"].height, w["params"], w["target"]
    rng = np.random.default_rng(61)
    if name == "ragged_300x200":
        W, H, p = 300, 200, synth.random_case(62, 300, 200, 4000, sigma=(0.3, 20.0), margin=20)
    elif name == "long_lists":                      # every tile list longer than one staging batch
        W, H = 64, 48
        n = 3000
        p = np.zeros((n, 8), np.float32)
        p[:, 0] = rng.uniform(0, W, n)
        p[:, 1] = rng.uniform(0, H, n)
        p[:, 2] = rng.uniform(2.0, 12.0, n)
        p[:, 3] = rng.uniform(-3.0, 3.0, n)
        p[:, 4] = rng.uniform(2.0, 12.0, n)
        p[:, 5:] = rng.uniform(-0.1, 0.1, (n, 3))
    elif name == "empty":
        W, H, p = 70, 45, np.zeros((0, 8), np.float32)
    elif name == "dense_400x300":                   # 475 tiles: buckets of 8 tiles, > 2048 pairs, lists > 128
        W, H = 400, 300
        n = 20000
        p = np.zeros((n, 8), np.float32)
        p[:, 0] = rng.uniform(0, W, n)
        p[:, 1] = rng.uniform(0, H, n)
        p[:, 2] = rng.uniform(3.0, 14.0, n)
        p[:, 3] = rng.uniform(-2.0, 2.0, n)
        p[:, 4] = rng.uniform(3.0, 14.0, n)
        p[:, 5:] = rng.uniform(-0.05, 0.1, (n, 3))
    else:
        raise KeyError(name)
    return W, H, p, rng.uniform(0, 1, (3, H, W)).astype(np.float32)


@pytest.mark.parametrize("name", ["tiny_fit_64x64", "kodak_768x512_50k", "div2k_1020x678_70k", "ragged_300x200",
                                  "long_lists", "empty"])
@pytest.mark.parametrize("use_order", [False, True])
def test_fwd_bwd_fused_equals_separate_calls(name, use_order):
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    W, H, p, tgt = _fused_case(name)
    n = p.shape[0]
    r = Raster(W, H, n)
    P, T = dev(p), dev(tgt)
    M = r.bin(sync=True, params=P, order=True)
    if not use_order:
        r.has_order = False
    ws_bytes = gi.gi_render_bwd_workspace_bytes(r.desc, n, r.capacity)
    # separate: forward with L2, then backward (pair gradients left in the workspace)
    img1, dl1, lp1 = torch.empty_like(T), torch.empty_like(T), torch.empty_like(r.loss_partials)
    ws1 = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    gi.gi_render_fwd_l2(r.desc, n, r.records, r.pixbox, r.ranges, r.vals, T, img1, dl1, lp1, tile_order=r._order())
    gi.gi_render_bwd(r.desc, n, r.records, None, None, r.pixbox, r.offsets, r.ranges, r.vals, r.capacity, None, None,
                     None, dl1, None, None, None, ws1, tile_order=r._order())
    # fused
    img2, dl2, lp2 = torch.full_like(T, 7.0), torch.full_like(T, 7.0), torch.full_like(r.loss_partials, 7.0)
    ws2 = torch.full((ws_bytes,), 0x5a, dtype=torch.uint8, device="cuda")
    gi.gi_render_fwd_bwd_l2(r.desc, n, r.records, r.pixbox, r.offsets, r.ranges, r.vals, r.capacity, T, img2, dl2,
                            lp2, ws2, tile_order=r._order())
    # and without the optional dL/dI output
    img3 = torch.empty_like(T)
    ws3 = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    lp3 = torch.empty_like(r.loss_partials)
    gi.gi_render_fwd_bwd_l2(r.desc, n, r.records, r.pixbox, r.offsets, r.ranges, r.vals, r.capacity, T, img3, None,
                            lp3, ws3, tile_order=r._order())
    torch.cuda.synchronize()
    for a, b in [(img1, img2), (dl1, dl2), (lp1[: r.T], lp2[: r.T]), (img1, img3), (lp1[: r.T], lp3[: r.T])]:
        np.testing.assert_array_equal(u32(a), u32(b))
    g1 = ws1[: 32 * M].cpu().numpy()
    np.testing.assert_array_equal(g1, ws2[: 32 * M].cpu().numpy())
    np.testing.assert_array_equal(g1, ws3[: 32 * M].cpu().numpy())


def test_adam_pairs_loss_equals_loss_reduce():
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    w = synth.make_workload("kodak_768x512_50k")
    W, H, n = 768, 512, 50_000
    r = Raster(W, H, n)
    P, T = dev(w["params"]), dev(w["target"])
    r.bin(sync=True, params=P)
    r.forward_backward_l2(T)
    ref = torch.full((1,), -1.0, device="cuda")
    gi.gi_loss_reduce(r.T, r.loss_partials, T.numel(), ref)
    lr = [0.05, 0.05, 0.01, 0.01, 0.01, 0.005, 0.005, 0.005]
    outs = []
    for with_loss in (False, True):
        p2, m2, v2 = P.clone(), torch.full_like(P, 0.01), torch.full_like(P, 0.02)
        got = torch.full((1,), -2.0, device="cuda")
        kw = dict(loss_partials=r.loss_partials, loss_count=T.numel(), d_loss=got) if with_loss else {}
        gi.gi_adam_step_pairs(r.desc, n, r.offsets, r.capacity, r.bwd_ws, p2, m2, v2, lr, 0.9, 0.999, 1e-8, 3, **kw)
        torch.cuda.synchronize()
        outs.append([u32(p2), u32(m2), u32(v2)])
        if with_loss:
            np.testing.assert_array_equal(u32(got), u32(ref))
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
    # n = 0: only the loss workgroup runs
    got0 = torch.full((1,), -3.0, device="cuda")
    gi.gi_adam_step_pairs(r.desc, 0, r.offsets, r.capacity, r.bwd_ws, None, None, None, lr, 0.9, 0.999, 1e-8, 1,
                          loss_partials=r.loss_partials, loss_count=T.numel(), d_loss=got0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u32(got0), u32(ref))


@pytest.mark.parametrize("name", ["tiny_fit_64x64", "kodak_768x512_50k", "ragged_300x200", "long_lists",
                                  "dense_400x300"])
def test_fit_step_equals_the_three_calls(name):
    """gi_fit_step_sum (binning, fused raster, Adam + set-up of the next binning in one call, the
    next call skipping its preprocess) gives, step after step, the same bits as
    gi_preprocess_bin_sort -> gi_render_fwd_bwd_l2 -> gi_adam_step_pairs."""
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    W, H, p, tgt = _fused_case(name)
    n = p.shape[0]
    T = dev(tgt)
    lr = [0.05, 0.05, 0.01, 0.01, 0.01, 0.005, 0.005, 0.005]
    b1, b2, eps = 0.9, 0.999, 1e-8
    states = []
    for one_call in (False, True):
        P = dev(p)
        Mo, V = torch.zeros_like(P), torch.zeros_like(P)
        r = Raster(W, H, n)
        M = r.bin(sync=True, params=P)
        r.set_capacity(int(M * 2) + 4096)
        r.bwd_ws = torch.empty(gi.gi_render_bwd_workspace_bytes(r.desc, n, r.capacity), dtype=torch.uint8,
                               device="cuda")
        loss = torch.zeros(1, device="cuda")
        fb = gi.fit_buffers(P, Mo, V, T, r.image, r.loss_partials, loss, r.records, r.pixbox, r.counts, r.offsets,
                            r.keys, r.vals, r.ranges, r.order, r.d_num, r.capacity, r.ws, r.bwd_ws)
        hp = gi.adam_hparams(lr, b1, b2, eps)
        hist = []
        for step in range(1, 8):
            order = step in (1, 5)
            if one_call:
                flags = ((gi.FIT_PREPARED if step not in (1, 4) else 0) | (gi.FIT_ORDER if order else 0) |
                         (gi.FIT_USE_ORDER if step > 1 else 0))
                gi.gi_fit_step_sum(r.desc, n, fb, hp, step, flags=flags)
            else:
                r.bin(sync=False, params=P, order=order)
                r.forward_backward_l2(T)
                gi.gi_adam_step_pairs(r.desc, n, r.offsets, r.capacity, r.bwd_ws, P, Mo, V, lr, b1, b2, eps, step,
                                      loss_partials=r.loss_partials, loss_count=3 * W * H, d_loss=loss)
            torch.cuda.synchronize()
            Mb = int(u32(r.d_num)[0])
            hist.append([u32(P).copy(), u32(Mo).copy(), u32(V).copy(), u32(loss).copy(), u32(r.image).copy(),
                         u32(r.offsets).copy(), u32(r.keys)[:Mb].copy(), u32(r.vals)[:Mb].copy()])
        states.append(hist)
    for step, (a, b) in enumerate(zip(*states)):
        for k, (x, y) in enumerate(zip(a, b)):
            np.testing.assert_array_equal(x, y, err_msg=f"step {step + 1} output {k}")


@pytest.mark.parametrize("name", ["kodak_768x512_50k", "ragged_300x200", "dense_400x300", "empty", "alpha_300x200"])
def test_render_image_equals_the_two_calls(name):
    """gi_render_image (the raster finishing the sort in sum mode where it can) gives the same image,
    offsets, sorted keys / vals and ranges as gi_preprocess_bin_sort -> gi_render_fwd."""
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    if name == "alpha_300x200":
        W, H, p, lg = _case(name)
        bg = dev(np.array([0.2, 0.5, 0.7, 0.0], np.float32))
    else:
        W, H, p, _ = _fused_case(name)
        lg, bg = None, None
    n = p.shape[0]
    mode = gi.MODE_ALPHA if lg is not None else gi.MODE_SUM
    P, L = dev(p), None if lg is None else dev(lg)
    outs = []
    for one_call in (False, True):
        r = Raster(W, H, n, mode)
        M = r.bin(sync=True, params=P, logit=L)
        r.set_capacity(int(M * 2) + 1024)
        if one_call:
            M2 = gi.gi_render_image(r.desc, n, P, L, bg, r.records, r.opacity, r.pixbox, r.counts, r.offsets, r.keys,
                                    r.vals, r.ranges, r.order, 0, r.capacity, r.d_num, r.ws, r.image, r.t_final,
                                    r.last, sync_count=True)
        else:
            M2 = r.bin(sync=True, params=P, logit=L, order=False)
            r.forward(bg)
        torch.cuda.synchronize()
        o = [u32(r.image), u32(r.offsets), u32(r.keys)[:M2], u32(r.vals)[:M2], u32(r.ranges)[: r.T],
             u32(r.records)[:n], u32(r.counts)[:n]]
        if r.t_final is not None:
            o += [u32(r.t_final), u32(r.last)]
        outs.append((M2, o))
    assert outs[0][0] == outs[1][0]
    for k, (a, b) in enumerate(zip(outs[0][1], outs[1][1])):
        np.testing.assert_array_equal(a, b, err_msg=f"output {k}")


def test_fit_step_tracks_the_largest_pair_count():
    """GI_FIT_TRACK_MAX: d_num[1] ends as the largest M of the steps since it was cleared, so one read
    after asynchronous steps shows an overflow (a capacity below M) that d_num[0] alone would hide
    once a later binning fits again."""
    require_gpu()
    from rasterizer_gaussian_raster_amd import gi
    from rasterizer_gaussian_raster_amd.pipeline import Raster
    W, H, p, tgt = _fused_case("kodak_768x512_50k")
    n = p.shape[0]
    T = dev(tgt)
    lr = [0.5, 0.5, 0.3, 0.3, 0.3, 0.005, 0.005, 0.005]      # large steps: M moves from step to step
    P = dev(p)
    Mo, V = torch.zeros_like(P), torch.zeros_like(P)
    r = Raster(W, H, n)
    M0 = r.bin(sync=True, params=P)
    r.set_capacity(int(M0 * 2) + 4096)
    r.bwd_ws = torch.empty(gi.gi_render_bwd_workspace_bytes(r.desc, n, r.capacity), dtype=torch.uint8,
                           device="cuda")
    loss = torch.zeros(1, device="cuda")
    fb = gi.fit_buffers(P, Mo, V, T, r.image, r.loss_partials, loss, r.records, r.pixbox, r.counts, r.offsets,
                        r.keys, r.vals, r.ranges, r.order, r.d_num, r.capacity, r.ws, r.bwd_ws)
    hp = gi.adam_hparams(lr, 0.9, 0.999, 1e-8)
    r.d_num.zero_()
    seen = []
    for step in range(1, 7):
        gi.gi_fit_step_sum(r.desc, n, fb, hp, step, flags=gi.FIT_TRACK_MAX | (gi.FIT_PREPARED if step > 1 else 0))
        torch.cuda.synchronize()
        d = u32(r.d_num)
        seen.append(int(d[0]))
        assert int(d[1]) == max(seen), (seen, d)
    print(f"pair counts per step: {seen}")
    assert len(set(seen)) > 1
    # without the flag d_num[1] is left alone
    before = int(u32(r.d_num)[1])
    gi.gi_fit_step_sum(r.desc, n, fb, hp, 7, flags=gi.FIT_PREPARED)
    torch.cuda.synchronize()
    assert int(u32(r.d_num)[1]) == before
