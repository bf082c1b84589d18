"""CPU oracle for the fused conv2d layer and its pools.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow reference that the
GPU library is checked against. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library itself never does, and
the two share no code. The arithmetic lives in ``conv_oracle.c`` (fp64 direct
loops, built by :func:`oracle.build.build`); this module only marshals numpy
arrays into it and holds the round-to-nearest-even storage quantizer.

Layouts: "nhwc" means x [N,H,W,Cin], w [Cout,kh,kw,Cin] (OHWI), residual and
y [N,OH,OW,Cout]; "nchw" means x [N,Cin,H,W], w [Cout,Cin,kh,kw] (OIHW),
residual and y [N,Cout,OH,OW]. The C code works in the NCHW/OIHW order; the
permutation here is a plain numpy transpose.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

ACT_NONE = 0
ACT_RELU = 1
ACT_SILU = 2
ACT_PRELU = 3
RES_BEFORE_ACT = 0x100

_ACT_NAMES = {"none": ACT_NONE, "relu": ACT_RELU, "silu": ACT_SILU, "prelu": ACT_PRELU}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build

        _build.build()
    _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    dp = ctypes.POINTER(ctypes.c_double)
    fp = ctypes.POINTER(ctypes.c_float)
    i = ctypes.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = i
    lib.oracle_out_dim.argtypes = [i, i, i, i]
    lib.oracle_out_dim.restype = i
    lib.oracle_conv2d_nchw.argtypes = [dp, dp, dp, dp, dp, dp] + [i] * 11
    lib.oracle_conv2d_nchw.restype = i
    lib.oracle_conv2d_points_nchw.argtypes = [dp, dp, dp, dp, dp,
                                              ctypes.POINTER(ctypes.c_int64),
                                              ctypes.c_int64, dp] + [i] * 11
    lib.oracle_conv2d_points_nchw.restype = i
    lib.oracle_maxpool3x3s2_nchw.argtypes = [dp, dp, i, i, i, i, i]
    lib.oracle_maxpool3x3s2_nchw.restype = i
    lib.oracle_avgpool2x2_nchw.argtypes = [fp, fp, i, i, i, i, i]
    lib.oracle_avgpool2x2_nchw.restype = i
    lib.oracle_conv_transpose4x4s2_nchw.argtypes = [dp, dp, dp, dp, dp] + [i] * 7
    lib.oracle_conv_transpose4x4s2_nchw.restype = i
    return lib


def _dptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _act_flags(act, res_before_act):
    code = _ACT_NAMES[act] if isinstance(act, str) else int(act)
    return code | (RES_BEFORE_ACT if res_before_act else 0)


def threads() -> int:
    """Threads the oracle uses by default (OpenMP's maximum)."""
    return int(_load().oracle_threads())


def out_dim(n_in: int, k: int, stride: int, pad: int) -> int:
    """floor((n_in + 2*pad - k)/stride) + 1, or -1 when no output fits."""
    return int(_load().oracle_out_dim(n_in, k, stride, pad))


def _to_nchw(x, w, residual, layout):
    if layout == "nhwc":
        x = x.transpose(0, 3, 1, 2)
        w = w.transpose(0, 3, 1, 2)
        if residual is not None:
            residual = residual.transpose(0, 3, 1, 2)
    elif layout != "nchw":
        raise ValueError(f"unknown layout {layout!r}")
    return _f64(x), _f64(w), _f64(residual)


def conv2d(x, w, bias=None, alpha=None, residual=None, *, stride=1, pad=0, act="none",
           res_before_act=False, layout="nhwc", threads=0):
    """The layer, in fp64: tap sum, bias, residual and activation.

    Inputs are widened to fp64 exactly (bf16/f16/f32 storage values embed in
    fp64). Returns an fp64 array in ``layout``.
    """
    x = np.asarray(x)
    w = np.asarray(w)
    xc, wc, rc = _to_nchw(x, w, None if residual is None else np.asarray(residual), layout)
    N, Cin, H, W = xc.shape
    Cout, wcin, kh, kw = wc.shape
    if wcin != Cin:
        raise ValueError("weight Cin does not match input")
    OH, OW = out_dim(H, kh, stride, pad), out_dim(W, kw, stride, pad)
    if OH < 1 or OW < 1:
        raise ValueError("no output fits")
    b = _f64(bias)
    a = _f64(alpha)
    y = np.empty((N, Cout, OH, OW), dtype=np.float64)
    rc_ = _load().oracle_conv2d_nchw(_dptr(xc), _dptr(wc), _dptr(b), _dptr(a), _dptr(rc),
                                     _dptr(y), N, H, W, Cin, Cout, kh, kw, stride, pad,
                                     _act_flags(act, res_before_act), threads)
    if rc_ != 0:
        raise ValueError("oracle rejected the arguments")
    if layout == "nhwc":
        y = np.ascontiguousarray(y.transpose(0, 2, 3, 1))
    return y


def conv2d_points(x, w, bias, alpha, residual, idx, *, stride=1, pad=0, act="none",
                  res_before_act=False, layout="nhwc", threads=0):
    """The layer at selected outputs only.

    ``idx`` is an integer array [P, 4] of (n, oh, ow, co) for "nhwc" or
    (n, co, oh, ow) for "nchw": the index of each output in ``layout``.
    Returns fp64 values [P].
    """
    x = np.asarray(x)
    w = np.asarray(w)
    xc, wc, rc = _to_nchw(x, w, None if residual is None else np.asarray(residual), layout)
    N, Cin, H, W = xc.shape
    Cout, _, kh, kw = wc.shape
    idx = np.asarray(idx, dtype=np.int64).reshape(-1, 4)
    if layout == "nhwc":
        idx = idx[:, [0, 3, 1, 2]]
    idx = np.ascontiguousarray(idx)
    out = np.empty(idx.shape[0], dtype=np.float64)
    rc_ = _load().oracle_conv2d_points_nchw(
        _dptr(xc), _dptr(wc), _dptr(_f64(bias)), _dptr(_f64(alpha)), _dptr(rc),
        idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), idx.shape[0], _dptr(out),
        N, H, W, Cin, Cout, kh, kw, stride, pad, _act_flags(act, res_before_act), threads)
    if rc_ != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def maxpool3x3s2(x, *, layout="nhwc", threads=0):
    """3x3 stride-2 pad-1 max pool in fp64 (exact: the result is one of the inputs)."""
    x = np.asarray(x)
    xc = _f64(x.transpose(0, 3, 1, 2) if layout == "nhwc" else x)
    N, C, H, W = xc.shape
    OH, OW = out_dim(H, 3, 2, 1), out_dim(W, 3, 2, 1)
    y = np.empty((N, C, OH, OW), dtype=np.float64)
    if _load().oracle_maxpool3x3s2_nchw(_dptr(xc), _dptr(y), N, C, H, W, threads) != 0:
        raise ValueError("oracle rejected the arguments")
    return np.ascontiguousarray(y.transpose(0, 2, 3, 1)) if layout == "nhwc" else y


def avgpool2x2(x, *, layout="nhwc", threads=0):
    """2x2 stride-2 average pool in single precision, in the pinned order.

    ``x`` holds storage values (any float dtype whose values fit fp32 exactly).
    Returns the fp32 result before the final rounding to the storage type.
    """
    x = np.asarray(x)
    xt = x.transpose(0, 3, 1, 2) if layout == "nhwc" else x
    xc = np.ascontiguousarray(xt.astype(np.float32))
    if not np.array_equal(xc.astype(np.float64), np.asarray(xt, dtype=np.float64)):
        raise ValueError("avgpool input is not exactly representable in fp32")
    N, C, H, W = xc.shape
    y = np.empty((N, C, H // 2, W // 2), dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    if _load().oracle_avgpool2x2_nchw(xc.ctypes.data_as(fp), y.ctypes.data_as(fp), N, C, H,
                                      W, threads) != 0:
        raise ValueError("oracle rejected the arguments")
    return np.ascontiguousarray(y.transpose(0, 2, 3, 1)) if layout == "nhwc" else y


# Binary formats: (significant bits including the hidden one, min normal exponent,
# max exponent). IEEE binary32, bfloat16 (binary32's exponent range, 8-bit
# significand) and IEEE binary16.
_FORMATS = {"f32": (24, -126, 127), "bf16": (8, -126, 127), "f16": (11, -14, 15)}


def quantize(v, dtype: str):
    """Round fp64 values to the storage format, nearest-even, in one rounding.

    Subnormals are kept; values at or past the overflow threshold become
    +-inf; NaN stays NaN. Returns fp64 values that the format represents
    exactly.
    """
    p, emin, emax = _FORMATS[dtype]
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(a)
        e = np.maximum(e.astype(np.int64) - 1, emin)  # floor(log2 a), clamped at emin
        quantum = np.ldexp(1.0, (e - (p - 1)).astype(np.int32))
        r = np.rint(a / quantum) * quantum  # np.rint rounds half to even
        max_finite = np.ldexp(2.0 - 2.0 ** (1 - p), emax)
        r = np.where(r > max_finite, np.inf, r)
        r = np.where(np.isfinite(a), r, a)
    return np.copysign(r, v)


def conv_transpose4x4s2(x, w, bias=None, alpha=None, *, act="none", layout="nhwc", threads=0):
    """ConvTranspose2d 4x4, stride 2, pad 1 in fp64 (framecast `wgslDeconv`): each
    input pixel (iy, ix) adds x * w[ci, co, ky, kx] to output (2*iy - 1 + ky,
    2*ix - 1 + kx); then bias and the activation. ``w`` is [Cin, Cout, 4, 4] in both
    layouts; x and the result are [N,H,W,C] ("nhwc") or [N,C,H,W] ("nchw"); the
    output is 2H x 2W."""
    x = np.asarray(x)
    xc = _f64(x.transpose(0, 3, 1, 2) if layout == "nhwc" else x)
    wc = _f64(w)
    N, Cin, H, W = xc.shape
    if wc.shape[0] != Cin or wc.shape[2:] != (4, 4):
        raise ValueError("weight must be [Cin, Cout, 4, 4]")
    Cout = wc.shape[1]
    y = np.empty((N, Cout, 2 * H, 2 * W), dtype=np.float64)
    code = _ACT_NAMES[act] if isinstance(act, str) else int(act)
    if _load().oracle_conv_transpose4x4s2_nchw(_dptr(xc), _dptr(wc), _dptr(_f64(bias)), _dptr(_f64(alpha)),
                                                _dptr(y), N, H, W, Cin, Cout, code, threads) != 0:
        raise ValueError("oracle rejected the arguments")
    return np.ascontiguousarray(y.transpose(0, 2, 3, 1)) if layout == "nhwc" else y


def upsample_nearest2x(x, *, layout="nhwc"):
    """Nearest-neighbour 2x upsample (inferencelayer `UPSAMPLE_SRC`): output pixel
    (oy, ox) is input pixel (oy // 2, ox // 2). Exact."""
    x = np.asarray(x)
    if layout == "nhwc":
        N, H, W, C = x.shape
        oy = np.arange(2 * H) // 2
        ox = np.arange(2 * W) // 2
        return x[:, oy][:, :, ox]
    N, C, H, W = x.shape
    oy = np.arange(2 * H) // 2
    ox = np.arange(2 * W) // 2
    return x[:, :, oy][:, :, :, ox]


def concat_channels(a, b, *, layout="nhwc"):
    """Per-pixel channel concat (inferencelayer `CONCAT_SRC`): a's channels, then b's."""
    return np.concatenate([np.asarray(a), np.asarray(b)], axis=3 if layout == "nhwc" else 1)
