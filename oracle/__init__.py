"""CPU oracle for the 2D-Gaussian tile rasterizer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never imports, links or calls it, and it never
imports the product path.

``liboracle.so`` is built from ``oracle.c`` (plain C, fp64 values, fp32 cutoff
decision, OpenMP over pixels) by :func:`build`.  The wrappers below only
marshal numpy arrays; every piece of arithmetic is in ``oracle.c``, whose
header states the definitions and the pages they come from.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, a library normal density, exact rational arithmetic for the
fp32 cutoff, numpy's stable sort for the bin order, central finite
differences, torch's Adam; for the rotation-scale form and rendering at another
scale: numpy's Cholesky factor fed to the Cholesky-form oracle, rotation
symmetries, numpy's matrix inverse for the cutoff set; for the SSIM loss:
scipy's Gaussian window and zero-padded correlation, closed forms for shifted
and scaled images, central finite differences; for the merge: moments and
channel integrals by numerical quadrature of the two summed Gaussians, and
identical pairs; for the merge cost: a closed form for equal isotropic pairs,
quadrature moments with numpy's slogdet, non-negativity; for a merge round:
the rule re-implemented with numpy over all pairs; for merging down: channel
integrals kept and isolated Gaussians left alone; for density control: a
hand-worked case and numpy's eigenvalues for the bloated flag).  No function
is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

TILE = 16


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wno-unused-function", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.oracle_cutoff_exponent.argtypes = [P, i32, i32, P]
    lib.oracle_cutoff_exponent.restype = ctypes.c_float
    lib.oracle_const.argtypes = [i32]
    lib.oracle_const.restype = ctypes.c_float
    lib.oracle_footprint.argtypes = [i32, i32, i64, P, P, P, P]
    lib.oracle_footprint.restype = i64
    lib.oracle_bin.argtypes = [i32, i32, i64, P, P, P, P, P, P, i64]
    lib.oracle_bin.restype = i64
    lib.oracle_box_leaks.argtypes = [i32, i32, i64, P]
    lib.oracle_box_leaks.restype = i64
    lib.oracle_cutoff_margin.argtypes = [i32, i32, i64, P]
    lib.oracle_cutoff_margin.restype = ctypes.c_double
    lib.oracle_render_sum.argtypes = [i32, i32, i64, P, P, i64, i32, P, P]
    lib.oracle_render_sum.restype = None
    lib.oracle_grad_sum.argtypes = [i32, i32, i64, P, P, i32, P, P, P]
    lib.oracle_grad_sum.restype = None
    lib.oracle_render_alpha.argtypes = [i32, i32, i64, P, P, P, P, i64, P, P, P, P, P, P]
    lib.oracle_render_alpha.restype = None
    lib.oracle_grad_alpha.argtypes = [i32, i32, i64, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_grad_alpha.restype = None
    lib.oracle_loss_l2.argtypes = [i64, P, P, P]
    lib.oracle_loss_l2.restype = ctypes.c_double
    lib.oracle_adam.argtypes = [i64, i32, P, P, P, P, P, ctypes.c_double, ctypes.c_double,
                                ctypes.c_double, i32]
    lib.oracle_adam.restype = None
    f64 = ctypes.c_double
    lib.oracle_render_sum_rs.argtypes = [i32, i32, i64, P, f64, f64, P, i64, i32, P, P, P]
    lib.oracle_render_sum_rs.restype = None
    lib.oracle_grad_sum_rs.argtypes = [i32, i32, i64, P, f64, f64, P, i32, P, P, P]
    lib.oracle_grad_sum_rs.restype = None
    lib.oracle_rs_cholesky_grad.argtypes = [i64, P, f64, f64, P, P, P]
    lib.oracle_rs_cholesky_grad.restype = None
    lib.oracle_merge_cost.argtypes = [P, P]
    lib.oracle_merge_cost.restype = f64
    lib.oracle_merge_round.argtypes = [i32, i32, i64, P, i64, P, P]
    lib.oracle_merge_round.restype = i64
    lib.oracle_merge_apply.argtypes = [i64, P, i64, P, P]
    lib.oracle_merge_apply.restype = i64
    lib.oracle_merge_to.argtypes = [i32, i32, i64, P, i64, P, P]
    lib.oracle_merge_to.restype = i64
    lib.oracle_adc.argtypes = [i32, i32, i64, P, P, P, ctypes.c_float, P]
    lib.oracle_adc.restype = i64
    lib.oracle_loss_ssim.argtypes = [i32, i32, P, P, f64, f64, f64, P, P, P, P]
    lib.oracle_loss_ssim.restype = f64
    lib.oracle_merge_pairs.argtypes = [i64, P, P, P]
    lib.oracle_merge_pairs.restype = None
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = i32
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def threads() -> int:
    return int(_load().oracle_threads())


def constants() -> dict:
    """The fp32 constants of the cutoff decision, as the oracle defines them."""
    lib = _load()
    return {"scale": lib.oracle_const(0), "e9": lib.oracle_const(1), "logit_max": lib.oracle_const(2)}


def cutoff_exponent(param, i: int, j: int):
    """fp32 exponent e = (a dx)^2 + (b dx + c dy)^2 at pixel (i, j), and (mx, my, a, b, c)."""
    par = _f64(param).reshape(8)
    abc = np.zeros(5, np.float32)
    e = _load().oracle_cutoff_exponent(_p(par), int(i), int(j), _p(abc))
    return np.float32(e), abc


def footprint(W, H, params, logit=None):
    """Per-Gaussian pixel box [N,4] = (j0, i0, j1, i1) (-1s: none) and tile count [N]."""
    par = _f64(params).reshape(-1, 8)
    n = par.shape[0]
    box = np.zeros((n, 4), np.int32)
    cnt = np.zeros(n, np.uint32)
    _load().oracle_footprint(W, H, n, _p(par), _p(_f64(logit)), _p(box), _p(cnt))
    return box, cnt


def bin(W, H, params, logit=None):
    """Binning by definition: dict(offsets, keys, vals, ranges, M)."""
    par = _f64(params).reshape(-1, 8)
    n = par.shape[0]
    _, cnt = footprint(W, H, par, logit)
    M = int(cnt.astype(np.int64).sum())
    tx, ty = -(-W // TILE), -(-H // TILE)
    offsets = np.zeros(n + 1, np.uint32)
    keys = np.zeros(max(M, 1), np.uint32)
    vals = np.zeros(max(M, 1), np.uint32)
    ranges = np.zeros((tx * ty, 2), np.uint32)
    got = _load().oracle_bin(W, H, n, _p(par), _p(_f64(logit)), _p(offsets), _p(keys), _p(vals),
                             _p(ranges), M)
    assert got == M
    return {"offsets": offsets, "keys": keys[:M], "vals": vals[:M], "ranges": ranges, "M": M,
            "counts": cnt}


def box_leaks(W, H, params) -> int:
    par = _f64(params).reshape(-1, 8)
    return int(_load().oracle_box_leaks(W, H, par.shape[0], _p(par)))


def cutoff_margin(W, H, params) -> float:
    par = _f64(params).reshape(-1, 8)
    return float(_load().oracle_cutoff_margin(W, H, par.shape[0], _p(par)))


def _pix(pixels):
    if pixels is None:
        return None
    return np.ascontiguousarray(pixels, dtype=np.int32).reshape(-1, 2)


def render_sum(W, H, params, pixels=None, cutoff=True):
    """Sum image.  pixels: None (all, returns [3,H,W]) or int [P,2] of (row, col) (returns [3,P]).
    Returns (image, sabs) with sabs = sum_n |c| w (the error-metric scale)."""
    par = _f64(params).reshape(-1, 8)
    pix = _pix(pixels)
    npix = W * H if pix is None else pix.shape[0]
    out = np.zeros((3, npix))
    sabs = np.zeros((3, npix))
    _load().oracle_render_sum(W, H, par.shape[0], _p(par), _p(pix), npix, int(bool(cutoff)), _p(out),
                              _p(sabs))
    if pix is None:
        return out.reshape(3, H, W), sabs.reshape(3, H, W)
    return out, sabs


def grad_sum(W, H, params, dL_dI, cutoff=True, with_cond=False):
    """(dparams [N,8], abs-sum [N,8]) for L = <dL_dI, I>; with_cond also returns the running-error
    scale [N,8] (inner sums of each contribution taken over absolute values)."""
    par = _f64(params).reshape(-1, 8)
    G = _f64(dL_dI).reshape(3, H, W)
    n = par.shape[0]
    d = np.zeros((n, 8))
    a = np.zeros((n, 8))
    c = np.zeros((n, 8))
    _load().oracle_grad_sum(W, H, n, _p(par), _p(G), int(bool(cutoff)), _p(d), _p(a), _p(c))
    return (d, a, c) if with_cond else (d, a)


def render_alpha(W, H, params, logit, bg, pixels=None, force_last=None):
    """Alpha image.  Returns dict(image, sabs, t_final, last, ambiguous); shapes [3,H,W]/[H,W] for
    all pixels or [3,P]/[P] for a pixel list.  last = index of the last Gaussian composited (-1:
    none); sabs = sum |c| alpha T + T |bg| (error-metric scale)."""
    par = _f64(params).reshape(-1, 8)
    lg = _f64(logit).reshape(-1)
    b = _f64(bg).reshape(3)
    pix = _pix(pixels)
    npix = W * H if pix is None else pix.shape[0]
    fl = None if force_last is None else np.ascontiguousarray(force_last, dtype=np.int64).reshape(npix)
    out = np.zeros((3, npix))
    tf = np.zeros(npix)
    last = np.zeros(npix, np.int64)
    amb = np.zeros(npix, np.int32)
    sabs = np.zeros((3, npix))
    _load().oracle_render_alpha(W, H, par.shape[0], _p(par), _p(lg), _p(b), _p(pix), npix, _p(fl),
                                _p(out), _p(tf), _p(last), _p(amb), _p(sabs))
    if pix is None:
        return {"image": out.reshape(3, H, W), "sabs": sabs.reshape(3, H, W), "t_final": tf.reshape(H, W),
                "last": last.reshape(H, W), "ambiguous": amb.reshape(H, W)}
    return {"image": out, "sabs": sabs, "t_final": tf, "last": last, "ambiguous": amb}


def grad_alpha(W, H, params, logit, bg, dL_dI, force_last=None, with_cond=False):
    """(dparams [N,8], dlogit [N], dbg [3], abs-sum [N,9]) for L = <dL_dI, C>; with_cond also
    returns the running-error scale [N,9]."""
    par = _f64(params).reshape(-1, 8)
    lg = _f64(logit).reshape(-1)
    b = _f64(bg).reshape(3)
    G = _f64(dL_dI).reshape(3, H, W)
    n = par.shape[0]
    fl = None if force_last is None else np.ascontiguousarray(force_last, dtype=np.int64).reshape(H * W)
    d = np.zeros((n, 8))
    dl = np.zeros(n)
    dbg = np.zeros(3)
    a = np.zeros((n, 9))
    c = np.zeros((n, 9))
    _load().oracle_grad_alpha(W, H, n, _p(par), _p(lg), _p(b), _p(G), _p(fl), _p(d), _p(dl), _p(dbg),
                              _p(a), _p(c))
    return (d, dl, dbg, a, c) if with_cond else (d, dl, dbg, a)


def render_sum_rs(W, H, params_rs, fx=1.0, fy=1.0, pixels=None, cutoff=True):
    """Sum image of rotation-scale Gaussians (mux, muy, sx, sy, theta, cr, cg, cb) rendered at scale
    (fx, fy) into a W x H image.  Returns (image, sabs, amb): [3,H,W] for all pixels or [3,P] for a
    pixel list; amb = sum |c| w over the pairs whose cutoff decision is ambiguous in fp32."""
    par = _f64(params_rs).reshape(-1, 8)
    pix = _pix(pixels)
    npix = W * H if pix is None else pix.shape[0]
    out, sabs, amb = np.zeros((3, npix)), np.zeros((3, npix)), np.zeros((3, npix))
    _load().oracle_render_sum_rs(W, H, par.shape[0], _p(par), float(fx), float(fy), _p(pix), npix,
                                 1 if cutoff else 0, _p(out), _p(sabs), _p(amb))
    if pix is None:
        return out.reshape(3, H, W), sabs.reshape(3, H, W), amb.reshape(3, H, W)
    return out, sabs, amb


def grad_sum_rs(W, H, params_rs, dL_dI, fx=1.0, fy=1.0, cutoff=True):
    """(dparams [N,8], running-error scale [N,8], ambiguous-pair magnitude [N,8]) of
    L = <dL_dI, I> for the rotation-scale sum image rendered at scale (fx, fy)."""
    par = _f64(params_rs).reshape(-1, 8)
    G = _f64(dL_dI).reshape(3, H, W)
    n = par.shape[0]
    d, c, a = np.zeros((n, 8)), np.zeros((n, 8)), np.zeros((n, 8))
    _load().oracle_grad_sum_rs(W, H, n, _p(par), float(fx), float(fy), _p(G), 1 if cutoff else 0, _p(d), _p(c),
                               _p(a))
    return d, c, a


def rs_cholesky_grad(params_rs, dout, fx=1.0, fy=1.0):
    """(J^T dout, |J|^T |dout|) [N,8]: the chain rule of the conversion of rotation-scale params to
    the Cholesky form at scale (fx, fy), applied to a gradient dout w.r.t. that form."""
    par = _f64(params_rs).reshape(-1, 8)
    d = _f64(dout).reshape(-1, 8)
    n = par.shape[0]
    out, sc = np.zeros((n, 8)), np.zeros((n, 8))
    _load().oracle_rs_cholesky_grad(n, _p(par), float(fx), float(fy), _p(d), _p(out), _p(sc))
    return out, sc


def loss_ssim(image, target, w1=0.8, w2=0.0, ws=0.2, with_grad=True):
    """L = w1 mean|x - y| + w2 mean (x - y)^2 + ws (1 - SSIM) of [3,H,W] images.  Returns dict(loss,
    ssim (mean), map [3,H,W], grad [3,H,W], scale [3,H,W]: running-error scale of the gradient)."""
    x = _f64(image)
    y = _f64(target)
    _, H, W = x.shape
    smap = np.zeros_like(x)
    g = np.zeros_like(x) if with_grad else None
    sc = np.zeros_like(x) if with_grad else None
    ss = ctypes.c_double(0.0)
    L = _load().oracle_loss_ssim(W, H, _p(x), _p(y), float(w1), float(w2), float(ws), _p(g), _p(smap), _p(sc),
                                 ctypes.byref(ss))
    return {"loss": float(L), "ssim": float(ss.value), "map": smap, "grad": g, "scale": sc}


def merge_pairs(params, pairs):
    """Moment-matching merge of the Gaussian pairs [P,2] (indices into params [N,8]) -> [P,8]."""
    par = _f64(params).reshape(-1, 8)
    pr = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    out = np.zeros((pr.shape[0], 8))
    _load().oracle_merge_pairs(pr.shape[0], _p(par), _p(pr), _p(out))
    return out


def loss_l2(image, target):
    """(L, dL/dI) with L = mean (I - T)^2."""
    img = _f64(image)
    tgt = _f64(target)
    g = np.zeros_like(img)
    L = _load().oracle_loss_l2(img.size, _p(img), _p(tgt), _p(g))
    return float(L), g


def adam(p, g, m, v, lr, step, beta1=0.9, beta2=0.999, eps=1e-8):
    """One Adam step in fp64 on [rows, row_len] arrays (updated copies returned)."""
    p = _f64(p).copy()
    m = _f64(m).copy()
    v = _f64(v).copy()
    g = _f64(g)
    rows, row_len = p.shape
    lr = _f64(lr).reshape(row_len)
    _load().oracle_adam(rows, row_len, _p(p), _p(g), _p(m), _p(v), _p(lr), beta1, beta2, eps, int(step))
    return p, m, v


def merge_cost(a, b):
    """Merge cost of two Gaussians (Cholesky-form rows; a is taken as the one of smaller index)."""
    a, b = _f64(a).reshape(8), _f64(b).reshape(8)
    return float(_load().oracle_merge_cost(_p(a), _p(b)))


def merge_round(W, H, params, max_pairs):
    """One merge round: (pairs [m,2] int64, ascending smaller index; each Gaussian's pick [n], -1 none)."""
    par = _f64(params).reshape(-1, 8)
    n = par.shape[0]
    pairs = np.zeros((max(n // 2, 1), 2), np.int64)
    best = np.zeros(max(n, 1), np.int64)
    m = _load().oracle_merge_round(W, H, n, _p(par), int(max_pairs), _p(pairs), _p(best))
    return pairs[:m].copy(), best[:n].copy()


def merge_apply(params, pairs):
    """The set after merging the given disjoint pairs (ascending smaller index): [n - m, 8]."""
    par = _f64(params).reshape(-1, 8)
    pr = np.ascontiguousarray(np.asarray(pairs, np.int64).reshape(-1, 2))
    out = np.zeros((max(par.shape[0], 1), 8))
    m = _load().oracle_merge_apply(par.shape[0], _p(par), pr.shape[0], _p(pr), _p(out))
    return out[:m].copy()


def merge_to(W, H, params, target):
    """Merge rounds down to `target` Gaussians (or until no pair is found): (params [n_out, 8], rounds)."""
    par = _f64(params).reshape(-1, 8)
    out = np.zeros((max(par.shape[0], 1), 8))
    rounds = np.zeros(1, np.int64)
    m = _load().oracle_merge_to(W, H, par.shape[0], _p(par), int(target), _p(out), _p(rounds))
    return out[:m].copy(), int(rounds[0])


def adc(W, H, params, image, target, s0):
    """Adaptive density control on fp32 params [n,8] with fp32 image / target [3,H,W]:
    (new params fp32 [n,8], flags int32 [n] (1 dead, 2 out of bounds, 4 bloated), moved)."""
    par = np.ascontiguousarray(np.asarray(params, np.float32).reshape(-1, 8)).copy()
    img = np.ascontiguousarray(np.asarray(image, np.float32))
    tgt = np.ascontiguousarray(np.asarray(target, np.float32))
    n = par.shape[0]
    flags = np.zeros(max(n, 1), np.int32)
    moved = _load().oracle_adc(W, H, n, _p(par), _p(img), _p(tgt), float(s0), _p(flags))
    return par, flags[:n].copy(), int(moved)
