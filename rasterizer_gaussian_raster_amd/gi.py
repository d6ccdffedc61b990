"""ctypes binding of libgi.so (include/gi.h): one Python function per C entry point.

Argument marshalling only: tensors are passed as device pointers, the current
torch stream as the hipStream_t, and a non-OK status raises GiError.  Every
computation happens in the HIP kernels behind the C ABI.  There is no fallback:
if libgi.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgi.so")

GI_OK, GI_ERR_INVALID_ARG, GI_ERR_HIP, GI_ERR_CAPACITY, GI_ERR_UNSUPPORTED = 0, 1, 2, 3, 4
MODE_SUM, MODE_ALPHA = 0, 1
PARAMS_CHOLESKY, PARAMS_RS = 0, 1
TILE = 16

_lib = None


class GiError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status) if _lib else status}")


class gi_desc(ctypes.Structure):
    _fields_ = [("width", ctypes.c_int32), ("height", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


def desc(width: int, height: int, mode: int = MODE_SUM) -> gi_desc:
    return gi_desc(int(width), int(height), int(mode), 0)


FIT_PREPARED, FIT_ORDER, FIT_USE_ORDER, FIT_NO_UPDATE, FIT_TRACK_MAX = 1, 2, 4, 8, 16
SSIM_TARGET_PREPARED = 1


class gi_fit_buffers(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("params", "m", "v", "target", "image", "loss_partials", "d_loss", "records", "pixbox", "counts",
                 "offsets", "keys", "vals", "ranges", "tile_order", "d_num")] + [
        ("capacity", ctypes.c_int64), ("bin_workspace", ctypes.c_void_p), ("bin_workspace_bytes", ctypes.c_size_t),
        ("bwd_workspace", ctypes.c_void_p), ("bwd_workspace_bytes", ctypes.c_size_t)]


class gi_adam_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float * 8), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double)]


def load():
    """Open libgi.so (built by rasterizer_gaussian_raster_amd.build); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m rasterizer_gaussian_raster_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P, D = ctypes.c_void_p, ctypes.POINTER(gi_desc)
    i64, i32, f64, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_size_t
    sigs = {
        "gi_status_string": ([i32], ctypes.c_char_p),
        "gi_version": ([], ctypes.c_char_p),
        "gi_num_tiles": ([D], i64),
        "gi_preprocess": ([D, i64, P, P, P, P, P, P, P], i32),
        "gi_bin_sort_workspace_bytes": ([D, i64, i64], sz),
        "gi_bin_sort": ([D, i64, P, P, P, P, P, P, P, i64, P, P, P, sz, P], i32),
        "gi_preprocess_bin_sort": ([D, i64, P, P, P, P, P, P, P, P, P, P, P, i64, P, P, P, sz, P], i32),
        "gi_render_fwd": ([D, i64, P, P, P, P, P, P, P, P, P, P, P], i32),
        "gi_render_bwd_workspace_bytes": ([D, i64, i64], sz),
        "gi_render_bwd": ([D, i64, P, P, P, P, P, P, P, P, i64, P, P, P, P, P, P, P, P, i64, P, P, sz, P], i32),
        "gi_loss_workspace_bytes": ([i64], sz),
        "gi_loss_l2": ([i64, P, P, P, P, P, sz, P], i32),
        "gi_adam_step": ([i64, i32, P, P, P, P, P, f64, f64, f64, i32, i32, P], i32),
        "gi_params_to_cholesky": ([i32, i64, P, ctypes.c_float, ctypes.c_float, P, P], i32),
        "gi_loss_ssim_workspace_bytes": ([i32, i32], sz),
        "gi_merge_pairs": ([i64, P, i64, P, P, P], i32),
        "gi_render_fwd_alpha_l2": ([D, i64, P, P, P, P, P, P, P, P, P, P, P, P, P, P], i32),
        "gi_adam_step_pairs_alpha": ([D, i64, P, i64, P, sz, P, P, P, P, P, P, P, ctypes.c_float, P, P, P,
                                      ctypes.c_float, f64, f64, f64, i32, P, i64, P, P], i32),
        "gi_render_bwd_absgrad": ([D, i64, P, P, P, P, P, P, i64, P, P, P, P, sz, P], i32),
        "gi_loss_ssim": ([i32, i32, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_float, P, P, P, sz, ctypes.c_uint32,
                          P], i32),
        "gi_loss_ssim_target": ([i32, i32, P, P, sz, P], i32),
        "gi_params_to_cholesky_grad": ([i32, i64, P, ctypes.c_float, ctypes.c_float, P, P, i32, P], i32),
        "gi_grad_gather": ([D, i32, i64, P, ctypes.c_float, ctypes.c_float, P, P, i64, P, sz, P, P], i32),
        "gi_render_fwd_l2": ([D, i64, P, P, P, P, P, P, P, P, P, P], i32),
        "gi_loss_reduce": ([i64, P, i64, P, P], i32),
        "gi_adam_step_pairs": ([D, i64, P, i64, P, sz, P, P, P, P, f64, f64, f64, i32, P, P, i64, P, P], i32),
        "gi_adam_step_pairs_rs": ([D, i64, P, i64, P, sz, P, P, P, P, f64, f64, f64, i32, P, i64, P, P, P], i32),
        "gi_render_fwd_bwd_l2": ([D, i64, P, P, P, P, P, P, i64, P, P, P, P, P, sz, P], i32),
        "gi_render_image": ([D, i64, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_uint32, i64, P, P, P, sz, P, P, P,
                             P], i32),
        "gi_merge_workspace_bytes": ([D, i64], sz),
        "gi_merge_round": ([D, i64, P, i64, P, P, P, sz, P], i32),
        "gi_merge_apply": ([D, i64, P, i64, P, P, P, sz, P], i32),
        "gi_merge_to": ([D, i64, P, i64, P, P, P, P, sz, P], i32),
        "gi_adc_workspace_bytes": ([D, i64], sz),
        "gi_adc": ([D, i64, P, P, P, P, P, ctypes.c_float, P, P, P, sz, P], i32),
        "gi_render_image_noalloc_max_bytes": ([], sz),
        "gi_render_image_noalloc": ([D, i64, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_uint32, i64, P, P, P, P, P,
                                     P], i32),
        "gi_fit_step_sum": ([D, i64, ctypes.POINTER(gi_fit_buffers), ctypes.POINTER(gi_adam_hparams), i32, P,
                             ctypes.c_uint32, P], i32),
        "gi_fit_step_sum_ssim": ([D, i64, ctypes.POINTER(gi_fit_buffers), ctypes.POINTER(gi_adam_hparams),
                                  ctypes.c_float, ctypes.c_float, ctypes.c_float, P, P, sz, i32, P, ctypes.c_uint32,
                                  P], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        if not t.is_cuda:
            raise ValueError("device tensor expected")
        if not t.is_contiguous():
            raise ValueError("contiguous tensor expected")
        return ctypes.c_void_p(t.data_ptr())
    return ctypes.c_void_p(int(t))


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    """hipStream_t of `stream` (a torch stream or a raw handle); None: torch's current stream."""
    if stream is None:
        if _raw_stream is not None:      # the raw handle without building a Stream object
            return ctypes.c_void_p(_raw_stream(torch.cuda.current_device()))
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(st: int, what: str):
    if st != GI_OK:
        raise GiError(st, what)


def status_string(st: int) -> str:
    return load().gi_status_string(int(st)).decode()


def version() -> str:
    return load().gi_version().decode()


def num_tiles(d: gi_desc) -> int:
    return int(load().gi_num_tiles(ctypes.byref(d)))


def gi_preprocess(d, n, params, logit, records, opacity, pixbox, counts, stream=None):
    _check(load().gi_preprocess(ctypes.byref(d), int(n), _ptr(params), _ptr(logit), _ptr(records),
                                _ptr(opacity), _ptr(pixbox), _ptr(counts), _stream(stream)), "gi_preprocess")


def gi_bin_sort_workspace_bytes(d, n, capacity) -> int:
    return int(load().gi_bin_sort_workspace_bytes(ctypes.byref(d), int(n), int(capacity)))


def gi_bin_sort(d, n, pixbox, counts, offsets, keys, vals, ranges, capacity, d_num, workspace,
                sync_count=False, stream=None, tile_order=None):
    """Returns M (host int) when sync_count, else None.  Raises GiError(GI_ERR_CAPACITY) on overflow
    when sync_count."""
    h = ctypes.c_int64(-1)
    st = load().gi_bin_sort(ctypes.byref(d), int(n), _ptr(pixbox), _ptr(counts), _ptr(offsets), _ptr(keys),
                            _ptr(vals), _ptr(ranges), _ptr(tile_order), int(capacity), _ptr(d_num),
                            ctypes.byref(h) if sync_count else None, _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gi_bin_sort")
    return int(h.value) if sync_count else None


def gi_preprocess_bin_sort(d, n, params, logit, records, opacity, pixbox, counts, offsets, keys, vals, ranges,
                           capacity, d_num, workspace, sync_count=False, stream=None, tile_order=None):
    """gi_preprocess then gi_bin_sort in one call; returns as gi_bin_sort."""
    h = ctypes.c_int64(-1)
    st = load().gi_preprocess_bin_sort(ctypes.byref(d), int(n), _ptr(params), _ptr(logit), _ptr(records),
                                       _ptr(opacity), _ptr(pixbox), _ptr(counts), _ptr(offsets), _ptr(keys),
                                       _ptr(vals), _ptr(ranges), _ptr(tile_order), int(capacity), _ptr(d_num),
                                       ctypes.byref(h) if sync_count else None, _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gi_preprocess_bin_sort")
    return int(h.value) if sync_count else None


def gi_render_image(d, n, params, logit, background, records, opacity, pixbox, counts, offsets, keys, vals, ranges,
                    tile_order, flags, capacity, d_num, workspace, image, t_final=None, last=None, sync_count=False,
                    stream=None):
    """Preprocess, bin and render in one call.  Returns M when sync_count (raising GiError(GI_ERR_CAPACITY)
    on overflow), else None."""
    h = ctypes.c_int64(-1)
    st = load().gi_render_image(ctypes.byref(d), int(n), _ptr(params), _ptr(logit), _ptr(background), _ptr(records),
                                _ptr(opacity), _ptr(pixbox), _ptr(counts), _ptr(offsets), _ptr(keys), _ptr(vals),
                                _ptr(ranges), _ptr(tile_order), int(flags), int(capacity), _ptr(d_num),
                                ctypes.byref(h) if sync_count else None, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _ptr(image), _ptr(t_final), _ptr(last),
                                _stream(stream))
    _check(st, "gi_render_image")
    return int(h.value) if sync_count else None


def gi_render_image_noalloc(d, n, params, logit, background, records, opacity, pixbox, counts, offsets, keys, vals,
                            ranges, tile_order, flags, capacity, d_num, image, t_final=None, last=None,
                            sync_count=False, stream=None):
    """gi_render_image with the library's fixed bin workspace (no workspace argument).  Returns M when
    sync_count, else None."""
    h = ctypes.c_int64(-1)
    st = load().gi_render_image_noalloc(ctypes.byref(d), int(n), _ptr(params), _ptr(logit), _ptr(background),
                                        _ptr(records), _ptr(opacity), _ptr(pixbox), _ptr(counts), _ptr(offsets),
                                        _ptr(keys), _ptr(vals), _ptr(ranges), _ptr(tile_order), int(flags),
                                        int(capacity), _ptr(d_num), ctypes.byref(h) if sync_count else None,
                                        _ptr(image), _ptr(t_final), _ptr(last), _stream(stream))
    _check(st, "gi_render_image_noalloc")
    return int(h.value) if sync_count else None


def gi_render_fwd(d, n, records, opacity, pixbox, ranges, vals, background, image, t_final, last, stream=None,
                  tile_order=None):
    _check(load().gi_render_fwd(ctypes.byref(d), int(n), _ptr(records), _ptr(opacity), _ptr(pixbox),
                                _ptr(ranges), _ptr(tile_order), _ptr(vals), _ptr(background), _ptr(image),
                                _ptr(t_final), _ptr(last), _stream(stream)), "gi_render_fwd")


def gi_render_bwd_workspace_bytes(d, n, capacity) -> int:
    return int(load().gi_render_bwd_workspace_bytes(ctypes.byref(d), int(n), int(capacity)))


def gi_render_bwd(d, n, records, opacity, logit, pixbox, offsets, ranges, vals, capacity, background, t_final,
                  last, dL_dimage, dparams, dlogit, dbackground, workspace, stream=None, tile_order=None,
                  loss_partials=None, loss_count=0, d_loss=None):
    """Sum mode: with d_loss, also reduces the forward's loss partials into d_loss (as gi_loss_reduce)."""
    _check(load().gi_render_bwd(ctypes.byref(d), int(n), _ptr(records), _ptr(opacity), _ptr(logit),
                                _ptr(pixbox), _ptr(offsets), _ptr(ranges), _ptr(tile_order), _ptr(vals),
                                int(capacity),
                                _ptr(background), _ptr(t_final), _ptr(last), _ptr(dL_dimage), _ptr(dparams),
                                _ptr(dlogit), _ptr(dbackground), _ptr(loss_partials), int(loss_count),
                                _ptr(d_loss), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream)), "gi_render_bwd")


def gi_loss_workspace_bytes(count) -> int:
    return int(load().gi_loss_workspace_bytes(int(count)))


def gi_loss_l2(count, image, target, dL_dimage, d_loss, workspace, stream=None):
    _check(load().gi_loss_l2(int(count), _ptr(image), _ptr(target), _ptr(dL_dimage), _ptr(d_loss),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "gi_loss_l2")


def gi_adam_step(rows, row_len, p, g, m, v, lr, beta1, beta2, eps, step, zero_grad, stream=None):
    lr_arr = (ctypes.c_float * int(row_len))(*[float(x) for x in lr])
    _check(load().gi_adam_step(int(rows), int(row_len), _ptr(p), _ptr(g), _ptr(m), _ptr(v), lr_arr,
                               float(beta1), float(beta2), float(eps), int(step), int(zero_grad),
                               _stream(stream)), "gi_adam_step")


def gi_adam_step_pairs_rs(d, n, offsets, capacity, workspace, p, m, v, lr, beta1, beta2, eps, step, stream=None,
                          loss_partials=None, loss_count=0, d_loss=None, chol_out=None):
    lr_arr = (ctypes.c_float * 8)(*[float(x) for x in lr])
    _check(load().gi_adam_step_pairs_rs(ctypes.byref(d), int(n), _ptr(offsets), int(capacity), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(p), _ptr(m), _ptr(v),
                                        lr_arr, float(beta1), float(beta2), float(eps), int(step),
                                        _ptr(loss_partials), int(loss_count), _ptr(d_loss), _ptr(chol_out),
                                        _stream(stream)),
           "gi_adam_step_pairs_rs")


def gi_params_to_cholesky(kind, n, params, fx, fy, out, stream=None):
    _check(load().gi_params_to_cholesky(int(kind), int(n), _ptr(params), float(fx), float(fy), _ptr(out),
                                        _stream(stream)), "gi_params_to_cholesky")


def gi_params_to_cholesky_grad(kind, n, params, fx, fy, dout, dparams, accumulate=False, stream=None):
    _check(load().gi_params_to_cholesky_grad(int(kind), int(n), _ptr(params), float(fx), float(fy), _ptr(dout),
                                             _ptr(dparams), 1 if accumulate else 0, _stream(stream)),
           "gi_params_to_cholesky_grad")


def gi_grad_gather(d, kind, n, params, fx, fy, records, offsets, capacity, workspace, dparams, stream=None):
    _check(load().gi_grad_gather(ctypes.byref(d), int(kind), int(n), _ptr(params), float(fx), float(fy),
                                 _ptr(records), _ptr(offsets), int(capacity), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _ptr(dparams), _stream(stream)),
           "gi_grad_gather")


def gi_merge_workspace_bytes(d, n):
    return int(load().gi_merge_workspace_bytes(ctypes.byref(d), int(n)))


def gi_merge_round(d, n, params, max_pairs, pairs, workspace, stream=None):
    """One merge round; returns the number of pairs written to pairs [n/2][2] (int32)."""
    h = ctypes.c_int64(-1)
    _check(load().gi_merge_round(ctypes.byref(d), int(n), _ptr(params), int(max_pairs), _ptr(pairs), ctypes.byref(h),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "gi_merge_round")
    return int(h.value)


def gi_merge_apply(d, n, params, n_pairs, pairs, out, workspace, stream=None):
    _check(load().gi_merge_apply(ctypes.byref(d), int(n), _ptr(params), int(n_pairs), _ptr(pairs), _ptr(out),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "gi_merge_apply")


def gi_merge_to(d, n, params, target, out, workspace, stream=None):
    """Merge rounds down to target; returns (rows of out used, rounds)."""
    h, r = ctypes.c_int64(-1), ctypes.c_int32(-1)
    _check(load().gi_merge_to(ctypes.byref(d), int(n), _ptr(params), int(target), _ptr(out), ctypes.byref(h),
                              ctypes.byref(r), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)), "gi_merge_to")
    return int(h.value), int(r.value)


def gi_adc_workspace_bytes(d, n):
    return int(load().gi_adc_workspace_bytes(ctypes.byref(d), int(n)))


def gi_adc(d, n, params, m, v, image, target, s0, flags, d_moved, workspace, stream=None):
    _check(load().gi_adc(ctypes.byref(d), int(n), _ptr(params), _ptr(m), _ptr(v), _ptr(image), _ptr(target),
                         float(s0), _ptr(flags), _ptr(d_moved), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(stream)), "gi_adc")


def gi_render_bwd_absgrad(d, n, records, pixbox, offsets, ranges, vals, capacity, dL_dimage, dparams, dabs,
                          workspace, stream=None, tile_order=None):
    _check(load().gi_render_bwd_absgrad(ctypes.byref(d), int(n), _ptr(records), _ptr(pixbox), _ptr(offsets),
                                        _ptr(ranges), _ptr(tile_order), _ptr(vals), int(capacity), _ptr(dL_dimage),
                                        _ptr(dparams), _ptr(dabs), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)),
           "gi_render_bwd_absgrad")


def gi_render_fwd_alpha_l2(d, n, records, opacity, pixbox, ranges, vals, background, target, image, t_final, last,
                           dL_dimage, loss_partials, stream=None, tile_order=None):
    _check(load().gi_render_fwd_alpha_l2(ctypes.byref(d), int(n), _ptr(records), _ptr(opacity), _ptr(pixbox),
                                         _ptr(ranges), _ptr(tile_order), _ptr(vals), _ptr(background), _ptr(target),
                                         _ptr(image), _ptr(t_final), _ptr(last), _ptr(dL_dimage),
                                         _ptr(loss_partials), _stream(stream)), "gi_render_fwd_alpha_l2")


def gi_adam_step_pairs_alpha(d, n, offsets, capacity, workspace, p, m, v, lr, logit, m_logit, v_logit, lr_logit,
                             bg, m_bg, v_bg, lr_bg, beta1, beta2, eps, step, loss_partials=None, loss_count=0,
                             d_loss=None, stream=None):
    lr_arr = (ctypes.c_float * 8)(*[float(x) for x in lr])
    _check(load().gi_adam_step_pairs_alpha(ctypes.byref(d), int(n), _ptr(offsets), int(capacity), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _ptr(p), _ptr(m), _ptr(v),
                                           lr_arr, _ptr(logit), _ptr(m_logit), _ptr(v_logit), float(lr_logit),
                                           _ptr(bg), _ptr(m_bg), _ptr(v_bg), float(lr_bg), float(beta1),
                                           float(beta2), float(eps), int(step), _ptr(loss_partials),
                                           int(loss_count), _ptr(d_loss), _stream(stream)),
           "gi_adam_step_pairs_alpha")


def gi_merge_pairs(n_pairs, pairs, n, params, out, stream=None):
    _check(load().gi_merge_pairs(int(n_pairs), _ptr(pairs), int(n), _ptr(params), _ptr(out), _stream(stream)),
           "gi_merge_pairs")


def gi_loss_ssim_workspace_bytes(W, H):
    return int(load().gi_loss_ssim_workspace_bytes(int(W), int(H)))


def gi_loss_ssim_target(W, H, target, workspace, stream=None):
    _check(load().gi_loss_ssim_target(int(W), int(H), _ptr(target), _ptr(workspace), int(workspace.numel()),
                                      _stream(stream)), "gi_loss_ssim_target")


def gi_loss_ssim(W, H, image, target, w1, w2, ws, dL_dimage, d_loss, workspace, stream=None, flags=0):
    _check(load().gi_loss_ssim(int(W), int(H), _ptr(image), _ptr(target), float(w1), float(w2), float(ws),
                               _ptr(dL_dimage), _ptr(d_loss), _ptr(workspace), int(workspace.numel()), int(flags),
                               _stream(stream)), "gi_loss_ssim")


def gi_render_fwd_l2(d, n, records, pixbox, ranges, vals, target, image, dL_dimage, loss_partials, stream=None,
                     tile_order=None):
    _check(load().gi_render_fwd_l2(ctypes.byref(d), int(n), _ptr(records), _ptr(pixbox), _ptr(ranges),
                                   _ptr(tile_order), _ptr(vals),
                                   _ptr(target), _ptr(image), _ptr(dL_dimage), _ptr(loss_partials),
                                   _stream(stream)), "gi_render_fwd_l2")


def gi_loss_reduce(nparts, loss_partials, count, d_loss, stream=None):
    _check(load().gi_loss_reduce(int(nparts), _ptr(loss_partials), int(count), _ptr(d_loss), _stream(stream)),
           "gi_loss_reduce")


def gi_adam_step_pairs(d, n, offsets, capacity, workspace, p, m, v, lr, beta1, beta2, eps, step, stream=None,
                       d_step=None, loss_partials=None, loss_count=0, d_loss=None):
    """d_step: optional device int32 [1] holding the step (read on the device; `step` is then ignored).
    d_loss: also reduce loss_partials into it (as gi_loss_reduce) in the same launch."""
    lr_arr = (ctypes.c_float * 8)(*[float(x) for x in lr])
    _check(load().gi_adam_step_pairs(ctypes.byref(d), int(n), _ptr(offsets), int(capacity), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _ptr(p), _ptr(m), _ptr(v),
                                     lr_arr, float(beta1), float(beta2), float(eps), int(step), _ptr(d_step),
                                     _ptr(loss_partials), int(loss_count), _ptr(d_loss), _stream(stream)),
           "gi_adam_step_pairs")


def gi_render_fwd_bwd_l2(d, n, records, pixbox, offsets, ranges, vals, capacity, target, image, dL_dimage,
                         loss_partials, workspace, stream=None, tile_order=None):
    """Forward with the L2 loss and backward (pair gradients into workspace) in one launch."""
    _check(load().gi_render_fwd_bwd_l2(ctypes.byref(d), int(n), _ptr(records), _ptr(pixbox), _ptr(offsets),
                                       _ptr(ranges), _ptr(tile_order), _ptr(vals), int(capacity), _ptr(target),
                                       _ptr(image), _ptr(dL_dimage), _ptr(loss_partials), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)),
           "gi_render_fwd_bwd_l2")


def _addr(t):
    p = _ptr(t)
    return None if p is None else p.value


def fit_buffers(params, m, v, target, image, loss_partials, d_loss, records, pixbox, counts, offsets, keys, vals,
                ranges, tile_order, d_num, capacity, bin_workspace, bwd_workspace) -> gi_fit_buffers:
    """The gi_fit_buffers struct of gi_fit_step_sum from device tensors (tile_order / d_loss may be None)."""
    b = gi_fit_buffers()
    for name, t in (("params", params), ("m", m), ("v", v), ("target", target), ("image", image),
                    ("loss_partials", loss_partials), ("d_loss", d_loss), ("records", records), ("pixbox", pixbox),
                    ("counts", counts), ("offsets", offsets), ("keys", keys), ("vals", vals), ("ranges", ranges),
                    ("tile_order", tile_order), ("d_num", d_num)):
        setattr(b, name, _addr(t))
    b.capacity = int(capacity)
    b.bin_workspace = _addr(bin_workspace)
    b.bin_workspace_bytes = bin_workspace.numel() * bin_workspace.element_size()
    b.bwd_workspace = _addr(bwd_workspace)
    b.bwd_workspace_bytes = bwd_workspace.numel() * bwd_workspace.element_size()
    return b


def adam_hparams(lr, beta1, beta2, eps) -> gi_adam_hparams:
    h = gi_adam_hparams()
    for i, x in enumerate(lr):
        h.lr[i] = float(x)
    h.beta1, h.beta2, h.eps = float(beta1), float(beta2), float(eps)
    return h


def gi_fit_step_sum(d, n, buffers: gi_fit_buffers, hparams: gi_adam_hparams, step, d_step=None, flags=0,
                    stream=None):
    """One sum-mode training step (binning, fused raster, Adam + set-up of the next binning)."""
    _check(load().gi_fit_step_sum(ctypes.byref(d), int(n), ctypes.byref(buffers), ctypes.byref(hparams), int(step),
                                  _ptr(d_step), int(flags), _stream(stream)), "gi_fit_step_sum")


def gi_fit_step_sum_ssim(d, n, buffers: gi_fit_buffers, hparams: gi_adam_hparams, w1, w2, ws, dL_dimage,
                         ssim_workspace, step, d_step=None, flags=0, stream=None):
    """gi_fit_step_sum with the SSIM pixel loss (forward, gi_loss_ssim, backward in the raster pass)."""
    _check(load().gi_fit_step_sum_ssim(ctypes.byref(d), int(n), ctypes.byref(buffers), ctypes.byref(hparams),
                                       float(w1), float(w2), float(ws), _ptr(dL_dimage), _ptr(ssim_workspace),
                                       int(ssim_workspace.numel()), int(step), _ptr(d_step), int(flags),
                                       _stream(stream)), "gi_fit_step_sum_ssim")
