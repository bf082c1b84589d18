"""Fused conv2d (+bias, activation, residual) and pools for MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libconv2d_fused.so``
(include/conv2d_fused.h). PyTorch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels. The
binding only checks tensor shapes, dtypes and devices, derives the sizes the C
ABI takes, allocates outputs and workspaces when none are given and raises on an
error code. There is no fallback: if the library is not built, importing the ops
raises.

Workspace: the library allocates no device memory; kernel variants that need
scratch use a caller-owned workspace registered per thread and device. Every call
here takes ``workspace=``: ``None`` (default) uses a buffer this module keeps per
(device, stream), allocated with torch.empty and grown to what the call's preferred
variant needs (so calls on different streams never share one); ``False`` runs the
call without a workspace (variants that need none); a uint8 CUDA tensor is used as
given.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["conv2d_fused", "conv2d_fused_maxpool3x3s2", "maxpool3x3s2", "avgpool2x2", "out_dim",
           "check_args", "plan", "plan_maxpool", "Op", "conv_op", "pool_op", "copy_op", "stack_check",
           "stack_plan", "stack_run", "StackGraph", "conv_transpose4x4s2", "plan_deconv",
           "upsample_nearest2x", "concat_channels", "upsample2x_concat", "deconv_op", "upsample_op",
           "concat_op", "tune", "tune_save", "tune_load", "tune_clear", "deconv_pack", "conv_transpose4x4s2_prepacked", "weights_to_ohwi", "WEIGHTS_OHWI", "Y_TRANSIENT",
           "last_error", "library_path", "Conv2dError", "ACT_NONE", "ACT_RELU", "ACT_SILU",
           "workspace_size", "stack_workspace_size", "set_workspace", "DEFAULT_WORKSPACE_BYTES",
           "ACT_PRELU", "RES_BEFORE_ACT", "LAYOUT_NHWC", "LAYOUT_NCHW", "DTYPE_F32",
           "DTYPE_BF16", "DTYPE_F16"]

# Codes of include/conv2d_fused.h
LAYOUT_NHWC, LAYOUT_NCHW = 0, 1
DTYPE_F32, DTYPE_BF16, DTYPE_F16 = 0, 1, 2
ACT_NONE, ACT_RELU, ACT_SILU, ACT_PRELU = 0, 1, 2, 3
RES_BEFORE_ACT = 0x100
WEIGHTS_OHWI = 0x200
Y_TRANSIENT = 0x400
OK, EINVAL, EUNSUPPORTED, EHIP = 0, -1, -2, -3

_ACTS = {"none": ACT_NONE, "relu": ACT_RELU, "silu": ACT_SILU, "prelu": ACT_PRELU}
_LAYOUTS = {"nhwc": LAYOUT_NHWC, "nchw": LAYOUT_NCHW}
_DTYPES = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libconv2d_fused.so")

# Every exported symbol of the C ABI, with (restype, argtypes).
_vp, _fp, _i, _cp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p
OP_CONV, OP_CONV_MAXPOOL, OP_MAXPOOL, OP_AVGPOOL, OP_COPY = 0, 1, 2, 3, 4
OP_DECONV, OP_UPSAMPLE, OP_CONCAT, OP_UPSAMPLE_CONCAT = 5, 6, 7, 8


class Op(ctypes.Structure):
    """One op of a stack (struct conv2d_op of include/conv2d_fused.h)."""
    _fields_ = [("kind", ctypes.c_int), ("x", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("alpha", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("y", ctypes.c_void_p)] + [(f, ctypes.c_int) for f in
                                           ("N", "H", "W", "Cin", "Cout", "kh", "kw", "stride", "pad", "act")]


_op_p = ctypes.POINTER(Op)

SIGNATURES = {
    "conv2d_fused": (_i, [_vp, _vp, _fp, _fp, _vp, _vp] + [_i] * 12 + [_vp]),
    "maxpool3x3s2": (_i, [_vp, _vp] + [_i] * 6 + [_vp]),
    "avgpool2x2": (_i, [_vp, _vp] + [_i] * 6 + [_vp]),
    "conv2d_out_dim": (_i, [_i] * 4),
    "conv2d_check_args": (_i, [_vp, _vp, _fp, _fp, _vp, _vp] + [_i] * 12),
    "conv2d_plan": (_i, [_i] * 12 + [_cp, _i]),
    "conv2d_fused_maxpool3x3s2": (_i, [_vp, _vp, _fp, _fp, _vp] + [_i] * 12 + [_vp]),
    "conv2d_fused_maxpool_plan": (_i, [_i] * 12 + [_cp, _i]),
    "conv2d_stack_check": (_i, [_op_p, _i, _i, _i, ctypes.POINTER(ctypes.c_int)]),
    "conv2d_stack_plan": (_i, [_op_p, _i, _i, _i, _i, _cp, _i]),
    "conv2d_stack_run": (_i, [_op_p, _i, _i, _i, _vp]),
    "conv2d_stack_graph_create": (_i, [_op_p, _i, _i, _i, ctypes.POINTER(ctypes.c_void_p)]),
    "conv2d_stack_graph_launch": (_i, [_vp, _vp]),
    "conv2d_stack_graph_destroy": (_i, [_vp]),
    "conv_transpose4x4s2": (_i, [_vp, _vp, _fp, _fp, _vp] + [_i] * 9 + [_vp]),
    "conv_transpose4x4s2_plan": (_i, [_i] * 9 + [_cp, _i]),
    "upsample_nearest2x": (_i, [_vp, _vp] + [_i] * 6 + [_vp]),
    "concat_channels": (_i, [_vp, _vp, _vp] + [_i] * 7 + [_vp]),
    "upsample2x_concat": (_i, [_vp, _vp, _vp] + [_i] * 7 + [_vp]),
    "conv2d_tune": (_i, [_i] * 14 + [ctypes.POINTER(ctypes.c_float), _cp, _i]),
    "conv2d_tune_save": (_i, [_cp]),
    "conv2d_tune_load": (_i, [_cp]),
    "conv2d_tune_clear": (_i, []),
    "conv_transpose4x4s2_packed_bytes": (_i, [_i, _i, _i, ctypes.POINTER(ctypes.c_size_t)]),
    "conv_transpose4x4s2_pack": (_i, [_vp, _vp, _i, _i, _i, _vp]),
    "conv_transpose4x4s2_prepacked": (_i, [_vp, _vp, _fp, _fp, _vp] + [_i] * 9 + [_vp]),
    "conv2d_weights_to_ohwi": (_i, [_vp, _vp] + [_i] * 5 + [_vp]),
    "conv2d_fused_noalloc": (_i, [_vp, _vp, _fp, _fp, _vp, _vp] + [_i] * 12 + [_vp]),
    "conv2d_set_workspace": (_i, [_vp, ctypes.c_size_t]),
    "conv2d_workspace_size": (_i, [_i] * 12 + [ctypes.POINTER(ctypes.c_size_t)]),
    "conv2d_stack_workspace_size": (_i, [_op_p, _i, _i, _i, ctypes.POINTER(ctypes.c_size_t)]),
    "conv2d_last_error": (_cp, []),
    "conv2d_abi_version": (_i, []),
}

_lib = None


class Conv2dError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"conv2d library error {code}: {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def last_error() -> str:
    return _load().conv2d_last_error().decode()


def _check(rc):
    if rc != OK:
        raise Conv2dError(rc, last_error())


def out_dim(n_in: int, k: int, stride: int, pad: int) -> int:
    return _load().conv2d_out_dim(n_in, k, stride, pad)


def _act_code(act, res_before_act):
    code = _ACTS[act] if isinstance(act, str) else int(act)
    return code | (RES_BEFORE_ACT if res_before_act else 0)


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


DEFAULT_WORKSPACE_BYTES = 64 << 20
_ws_cache = {}  # (device index, stream handle) -> uint8 tensor


def set_workspace(ws, device=None):
    """Register ``ws`` (a uint8 CUDA tensor, or None for none) as the workspace of this
    thread's later calls on its device (conv2d_set_workspace). Returns nothing."""
    lib = _load()
    if ws is None:
        _check(lib.conv2d_set_workspace(None, 0))
        return
    if ws.dtype != torch.uint8 or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("a workspace is a contiguous uint8 CUDA tensor")
    if ws.data_ptr() % 256:
        raise ValueError("a workspace must be 256-byte aligned")
    with torch.cuda.device(ws.device):
        _check(lib.conv2d_set_workspace(ctypes.c_void_p(ws.data_ptr()), ws.numel()))


def _stream_of(device, stream):
    return torch.cuda.current_stream(device) if stream is None else stream


def _default_workspace(device, stream, need):
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream.cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        # torch's allocator is stream-ordered: the old buffer is reused only by work
        # queued after the calls that still use it on this stream
        ws = torch.empty(max(need, DEFAULT_WORKSPACE_BYTES), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _use_workspace(device, stream, workspace, need=0):
    """Registers the workspace for a call on `stream` (see the module doc); returns it."""
    lib = _load()
    with torch.cuda.device(device):
        if workspace is False:
            _check(lib.conv2d_set_workspace(None, 0))
            return None
        ws = _default_workspace(device, stream, need) if workspace is None else workspace
        if ws.dtype != torch.uint8 or ws.device != device or not ws.is_contiguous() or ws.data_ptr() % 256:
            raise ValueError("a workspace is a contiguous, 256-byte aligned uint8 tensor on the call's device")
        _check(lib.conv2d_set_workspace(ctypes.c_void_p(ws.data_ptr()), ws.numel()))
        return ws


def workspace_size(N, H, W, Cin, Cout, kh, kw, stride, pad, act, layout, dtype) -> int:
    """Bytes of workspace conv2d_fused's preferred variant for a shape writes (host only)."""
    n = ctypes.c_size_t(0)
    _check(_load().conv2d_workspace_size(N, H, W, Cin, Cout, kh, kw, stride, pad, act, layout, dtype,
                                         ctypes.byref(n)))
    return n.value


def _dims(x, w, layout, weights_ohwi=False):
    if x.dim() != 4 or w.dim() != 4:
        raise ValueError("x and w must be 4-D")
    if weights_ohwi:
        N, Cin, H, W = x.shape
        Cout, kh, kw, wc = w.shape
    elif layout == "nhwc":
        N, H, W, Cin = x.shape
        Cout, kh, kw, wc = w.shape
    else:
        N, Cin, H, W = x.shape
        Cout, wc, kh, kw = w.shape
    if wc != Cin:
        raise ValueError(f"weight has {wc} input channels, x has {Cin}")
    return N, H, W, Cin, Cout, kh, kw


def _require(t, name, dtype, device):
    if t is None:
        return
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _conv_args(x, w, bias, alpha, stride, pad, layout, weights_ohwi=False):
    lay = _LAYOUTS[layout]
    dt = _DTYPES.get(x.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {x.dtype}")
    dims = _dims(x, w, layout, weights_ohwi)
    N, H, W, Cin, Cout, kh, kw = dims
    OH, OW = out_dim(H, kh, stride, pad), out_dim(W, kw, stride, pad)
    if OH < 1 or OW < 1:
        raise ValueError("the kernel does not fit the padded input")
    dev = x.device
    _require(x, "x", x.dtype, dev)
    _require(w, "w", x.dtype, dev)
    _require(bias, "bias", torch.float32, dev)
    _require(alpha, "alpha", torch.float32, dev)
    for t, name in ((bias, "bias"), (alpha, "alpha")):
        if t is not None and tuple(t.shape) != (Cout,):
            raise ValueError(f"{name} must have shape ({Cout},)")
    return lay, dt, dims, (OH, OW)


def _out(out, shape, x):
    if out is None:
        return torch.empty(shape, dtype=x.dtype, device=x.device)
    _require(out, "out", x.dtype, x.device)
    if tuple(out.shape) != shape:
        raise ValueError(f"out must have shape {shape}")
    return out


def conv2d_fused(x, w, bias=None, alpha=None, residual=None, *, stride=1, pad=0, act="none",
                 res_before_act=False, layout="nhwc", weights_ohwi=False, out=None, stream=None,
                 workspace=None):
    """y = epilogue(conv(x, w)) on the GPU; see include/conv2d_fused.h.

    x, w, residual, out: CUDA tensors of one storage dtype (float32, bfloat16 or
    float16), contiguous, in ``layout`` ("nhwc" with OHWI weights or "nchw" with
    OIHW weights; with ``weights_ohwi`` a channel-first layer takes OHWI weights, see
    weights_to_ohwi). bias, alpha: float32 [Cout] or None. Returns y.
    """
    lib = _load()
    lay, dt, (N, H, W, Cin, Cout, kh, kw), (OH, OW) = _conv_args(x, w, bias, alpha, stride, pad, layout,
                                                                  weights_ohwi)
    yshape = (N, OH, OW, Cout) if layout == "nhwc" else (N, Cout, OH, OW)
    _require(residual, "residual", x.dtype, x.device)
    if residual is not None and tuple(residual.shape) != yshape:
        raise ValueError(f"residual must have shape {yshape}")
    out = _out(out, yshape, x)
    code = _act_code(act, res_before_act) | (WEIGHTS_OHWI if weights_ohwi else 0)
    st = _stream_of(x.device, stream)
    need = 0 if workspace is not None else workspace_size(N, H, W, Cin, Cout, kh, kw, stride, pad, code, lay, dt)
    with torch.cuda.device(x.device):
        _use_workspace(x.device, st, workspace, need)
        rc = lib.conv2d_fused(_ptr(x), _ptr(w), _ptr(bias), _ptr(alpha), _ptr(residual), _ptr(out),
                              N, H, W, Cin, Cout, kh, kw, stride, pad, code, lay, dt, _stream_handle(st))
    _check(rc)
    return out


def conv2d_fused_maxpool3x3s2(x, w, bias=None, alpha=None, *, stride=1, pad=0, act="none",
                              layout="nhwc", out=None, stream=None, workspace=None):
    """maxpool3x3s2(conv2d_fused(x, w, bias, alpha)) with only the pooled map written;
    see include/conv2d_fused.h. Returns the pooled y."""
    lib = _load()
    lay, dt, (N, H, W, Cin, Cout, kh, kw), (OH, OW) = _conv_args(x, w, bias, alpha, stride, pad, layout)
    PH, PW = (OH - 1) // 2 + 1, (OW - 1) // 2 + 1
    out = _out(out, (N, PH, PW, Cout) if layout == "nhwc" else (N, Cout, PH, PW), x)
    st = _stream_of(x.device, stream)
    # the two-kernel form holds the unpooled conv output in the workspace
    need = -(-N * OH * OW * Cout * x.element_size() // 256) * 256
    with torch.cuda.device(x.device):
        _use_workspace(x.device, st, workspace, need)
        rc = lib.conv2d_fused_maxpool3x3s2(_ptr(x), _ptr(w), _ptr(bias), _ptr(alpha), _ptr(out),
                                           N, H, W, Cin, Cout, kh, kw, stride, pad,
                                           _act_code(act, False), lay, dt, _stream_handle(st))
    _check(rc)
    return out


def _pool(fn_name, x, layout, out, stream, oh_of):
    lib = _load()
    lay = _LAYOUTS[layout]
    dt = _DTYPES.get(x.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {x.dtype}")
    if x.dim() != 4:
        raise ValueError("x must be 4-D")
    _require(x, "x", x.dtype, x.device)
    if layout == "nhwc":
        N, H, W, C = x.shape
    else:
        N, C, H, W = x.shape
    OH, OW = oh_of(H), oh_of(W)
    yshape = (N, OH, OW, C) if layout == "nhwc" else (N, C, OH, OW)
    if out is None:
        if OH < 1 or OW < 1:
            raise ValueError("input too small")
        out = torch.empty(yshape, dtype=x.dtype, device=x.device)
    else:
        _require(out, "out", x.dtype, x.device)
        if tuple(out.shape) != yshape:
            raise ValueError(f"out must have shape {yshape}")
    rc = getattr(lib, fn_name)(_ptr(x), _ptr(out), N, H, W, C, lay, dt, _stream_handle(stream))
    _check(rc)
    return out


def maxpool3x3s2(x, *, layout="nhwc", out=None, stream=None):
    """3x3 stride-2 pad-1 max pool on the GPU (bit-exact)."""
    return _pool("maxpool3x3s2", x, layout, out, stream, lambda n: (n - 1) // 2 + 1)


def avgpool2x2(x, *, layout="nhwc", out=None, stream=None):
    """2x2 stride-2 average pool on the GPU (bit-exact, fixed summation order)."""
    return _pool("avgpool2x2", x, layout, out, stream, lambda n: n // 2)


def check_args(x_ptr, w_ptr, bias_ptr, alpha_ptr, res_ptr, y_ptr, N, H, W, Cin, Cout, kh, kw,
               stride, pad, act, layout, dtype):
    """Host-only validation (no GPU needed); returns the C status code."""
    return _load().conv2d_check_args(x_ptr, w_ptr, bias_ptr, alpha_ptr, res_ptr, y_ptr, N, H, W,
                                     Cin, Cout, kh, kw, stride, pad, act, layout, dtype)


_WS_STANDIN = 0x4000000000  # 256-byte aligned; host-only planning never dereferences it


class _planning_workspace:
    """Registers a stand-in workspace of `nbytes` (0: none) for host-only planning calls,
    and no workspace again afterwards."""

    def __init__(self, nbytes):
        self.nbytes = int(nbytes)

    def __enter__(self):
        lib = _load()
        _check(lib.conv2d_set_workspace(ctypes.c_void_p(_WS_STANDIN) if self.nbytes else None, self.nbytes))
        return self

    def __exit__(self, *exc):
        _load().conv2d_set_workspace(None, 0)
        return False


def plan(N, H, W, Cin, Cout, kh, kw, stride, pad, act, layout, dtype, workspace_bytes=DEFAULT_WORKSPACE_BYTES) -> str:
    """Name of the kernel variant conv2d_fused picks for a shape with a workspace of
    ``workspace_bytes`` (0: none; host only)."""
    buf = ctypes.create_string_buffer(256)
    with _planning_workspace(workspace_bytes):
        n = _load().conv2d_plan(N, H, W, Cin, Cout, kh, kw, stride, pad, act, layout, dtype, buf, 256)
    _check(n if n < 0 else OK)
    return buf.value.decode()


def plan_maxpool(N, H, W, Cin, Cout, kh, kw, stride, pad, act, layout, dtype,
                 workspace_bytes=DEFAULT_WORKSPACE_BYTES) -> str:
    """Kernel variants conv2d_fused_maxpool3x3s2 picks for a shape (host only)."""
    buf = ctypes.create_string_buffer(256)
    with _planning_workspace(workspace_bytes):
        n = _load().conv2d_fused_maxpool_plan(N, H, W, Cin, Cout, kh, kw, stride, pad, act, layout, dtype,
                                              buf, 256)
    _check(n if n < 0 else OK)
    return buf.value.decode()


def _tensor_ptr(t):
    return None if t is None else t.data_ptr()


def conv_op(x, w, y, bias=None, alpha=None, residual=None, *, stride=1, pad=0, act="none",
            res_before_act=False, layout="nhwc", pool=False, weights_ohwi=False, transient=False):
    """An Op for conv2d_fused (or, with pool=True, conv2d_fused_maxpool3x3s2) on these
    tensors. transient=True marks y as an intermediate only the next op reads
    (CONV2D_Y_TRANSIENT): the stack may then leave it unwritten. The tensors must stay
    alive while the stack (or its graph) is in use."""
    N, H, W, Cin, Cout, kh, kw = _dims(x, w, layout, weights_ohwi)
    return Op(OP_CONV_MAXPOOL if pool else OP_CONV, _tensor_ptr(x), _tensor_ptr(w), _tensor_ptr(bias),
              _tensor_ptr(alpha), _tensor_ptr(residual), _tensor_ptr(y), N, H, W, Cin, Cout, kh, kw, stride, pad,
              _act_code(act, res_before_act) | (WEIGHTS_OHWI if weights_ohwi else 0) |
              (Y_TRANSIENT if transient else 0))


def _nhwc_dims(x, layout):
    if layout == "nhwc":
        return tuple(x.shape)
    N, C, H, W = x.shape
    return N, H, W, C


def pool_op(kind, x, y, *, layout="nhwc"):
    """An Op for maxpool3x3s2 (kind "max") or avgpool2x2 (kind "avg")."""
    N, H, W, C = _nhwc_dims(x, layout)
    return Op(OP_MAXPOOL if kind == "max" else OP_AVGPOOL, x.data_ptr(), None, None, None, None, y.data_ptr(),
              N, H, W, C, C, 0, 0, 0, 0, 0)


def copy_op(x, y):
    """An Op that copies x into y (same element count; a snapshot inside a stack)."""
    if x.numel() != y.numel() or x.dtype != y.dtype:
        raise ValueError("copy needs tensors of one dtype and size")
    return Op(OP_COPY, x.data_ptr(), None, None, None, None, y.data_ptr(), 1, 1, 1, x.numel(), 0, 0, 0, 0, 0, 0)


def _op_array(ops):
    arr = (Op * len(ops))(*ops)
    return arr, len(ops)


def stack_check(ops, layout="nhwc", dtype=DTYPE_BF16):
    """Host-only validation of a stack: (status, index of the first bad op or -1)."""
    arr, n = _op_array(ops)
    bad = ctypes.c_int(-1)
    rc = _load().conv2d_stack_check(arr, n, _LAYOUTS[layout], dtype, ctypes.byref(bad))
    return rc, bad.value


def stack_workspace_size(ops, layout="nhwc", dtype=DTYPE_BF16) -> int:
    """Bytes of workspace the stack's preferred variants write (host only)."""
    arr, n = _op_array(ops)
    nb = ctypes.c_size_t(0)
    _check(_load().conv2d_stack_workspace_size(arr, n, _LAYOUTS[layout], dtype, ctypes.byref(nb)))
    return nb.value


def stack_plan(ops, index, layout="nhwc", dtype=DTYPE_BF16, workspace_bytes=None) -> str:
    """Kernel variants of op `index` with a workspace of ``workspace_bytes`` (None: what the
    stack wants, as stack_run and StackGraph give it; 0: none). Host only."""
    arr, n = _op_array(ops)
    if workspace_bytes is None:
        workspace_bytes = stack_workspace_size(ops, layout, dtype)
    buf = ctypes.create_string_buffer(256)
    with _planning_workspace(workspace_bytes):
        rc = _load().conv2d_stack_plan(arr, n, _LAYOUTS[layout], dtype, index, buf, 256)
    _check(rc if rc < 0 else OK)
    return buf.value.decode()


def _stack_device(ops):
    # every op's tensors live on the current device (the stack calls take raw pointers)
    return torch.device("cuda", torch.cuda.current_device())


def stack_run(ops, layout="nhwc", dtype=DTYPE_BF16, stream=None, workspace=None):
    """Validate the whole stack, then enqueue its ops in order on the stream."""
    arr, n = _op_array(ops)
    dev = _stack_device(ops)
    st = _stream_of(dev, stream)
    need = 0 if workspace is not None else stack_workspace_size(ops, layout, dtype)
    _use_workspace(dev, st, workspace, need)
    _check(_load().conv2d_stack_run(arr, n, _LAYOUTS[layout], dtype, _stream_handle(st)))


class StackGraph:
    """A stack recorded once into a HIP graph; launch() replays it on a stream.

    The graph keeps the workspace it was made with: by default one of its own (sized by
    stack_workspace_size, held by this object), so replays never share it with other
    calls; ``workspace=False`` records the variants that need none."""

    def __init__(self, ops, layout="nhwc", dtype=DTYPE_BF16, workspace=None):
        arr, n = _op_array(ops)
        dev = _stack_device(ops)
        lib = _load()
        if workspace is None:
            need = stack_workspace_size(ops, layout, dtype)
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev) if need else False
        self.workspace = workspace if workspace is not False else None
        if self.workspace is None:
            _check(lib.conv2d_set_workspace(None, 0))
        else:
            set_workspace(self.workspace)
        h = ctypes.c_void_p()
        _check(lib.conv2d_stack_graph_create(arr, n, _LAYOUTS[layout], dtype, ctypes.byref(h)))
        self._h = h

    def launch(self, stream=None):
        _check(_load().conv2d_stack_graph_launch(self._h, _stream_handle(stream)))

    def close(self):
        if self._h:
            _check(_load().conv2d_stack_graph_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _dtype_code(dtype):
    dt = _DTYPES.get(dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {dtype}")
    return dt


def _deconv_ws_need(Cin, Cout, x):
    # the packed weights, then (channel-first, width not a multiple of 8) a copy of x
    e = x.element_size()
    return (16 * (-(-Cout // 32) * 32) * (-(-Cin // 64) * 64) * e + 255) // 256 * 256 + \
        (x.numel() * e + 255) // 256 * 256


def conv_transpose4x4s2(x, w, bias=None, alpha=None, *, act="none", layout="nhwc", out_dtype=None,
                        out=None, stream=None, workspace=None):
    """ConvTranspose2d 4x4, stride 2, pad 1 (+bias, activation) on the GPU; see
    include/conv2d_fused.h. w is [Cin, Cout, 4, 4] in x's dtype for both layouts; the
    output is [N, 2H, 2W, Cout] ("nhwc") or [N, Cout, 2H, 2W] ("nchw") in ``out_dtype``
    (x's dtype, or torch.float32)."""
    lib = _load()
    lay = _LAYOUTS[layout]
    dt = _dtype_code(x.dtype)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    odt = _dtype_code(out_dtype)
    if x.dim() != 4 or w.dim() != 4 or tuple(w.shape[2:]) != (4, 4):
        raise ValueError("x must be 4-D and w [Cin, Cout, 4, 4]")
    if layout == "nhwc":
        N, H, W, Cin = x.shape
    else:
        N, Cin, H, W = x.shape
    if w.shape[0] != Cin:
        raise ValueError(f"weight has {w.shape[0]} input channels, x has {Cin}")
    Cout = w.shape[1]
    dev = x.device
    _require(x, "x", x.dtype, dev)
    _require(w, "w", x.dtype, dev)
    _require(bias, "bias", torch.float32, dev)
    _require(alpha, "alpha", torch.float32, dev)
    for t, name in ((bias, "bias"), (alpha, "alpha")):
        if t is not None and tuple(t.shape) != (Cout,):
            raise ValueError(f"{name} must have shape ({Cout},)")
    yshape = (N, 2 * H, 2 * W, Cout) if layout == "nhwc" else (N, Cout, 2 * H, 2 * W)
    if out is None:
        out = torch.empty(yshape, dtype=out_dtype, device=dev)
    else:
        _require(out, "out", out_dtype, dev)
        if tuple(out.shape) != yshape:
            raise ValueError(f"out must have shape {yshape}")
    st = _stream_of(dev, stream)
    with torch.cuda.device(dev):
        _use_workspace(dev, st, workspace, _deconv_ws_need(Cin, Cout, x))
        rc = lib.conv_transpose4x4s2(_ptr(x), _ptr(w), _ptr(bias), _ptr(alpha), _ptr(out), N, H, W, Cin, Cout,
                                     _act_code(act, False), lay, dt, odt, _stream_handle(st))
    _check(rc)
    return out


def plan_deconv(N, H, W, Cin, Cout, act, layout, dtype, out_dtype=None, workspace_bytes=DEFAULT_WORKSPACE_BYTES) -> str:
    """Kernel variants conv_transpose4x4s2 picks for a shape (host only)."""
    buf = ctypes.create_string_buffer(256)
    with _planning_workspace(workspace_bytes):
        n = _load().conv_transpose4x4s2_plan(N, H, W, Cin, Cout, act, layout, dtype,
                                             dtype if out_dtype is None else out_dtype, buf, 256)
    _check(n if n < 0 else OK)
    return buf.value.decode()


def _resample(fn_name, a, b, up, layout, out, stream):
    lib = _load()
    lay = _LAYOUTS[layout]
    dt = _dtype_code(a.dtype)
    if a.dim() != 4 or (b is not None and b.dim() != 4):
        raise ValueError("inputs must be 4-D")
    N, H, W, Ca = _nhwc_dims(a, layout)
    s = 2 if up else 1
    _require(a, "a", a.dtype, a.device)
    Cb = 0
    if b is not None:
        _require(b, "b", a.dtype, a.device)
        Nb, Hb, Wb, Cb = _nhwc_dims(b, layout)
        if (Nb, Hb, Wb) != (N, s * H, s * W):
            raise ValueError(f"b must be {s * H}x{s * W} with batch {N}")
    C = Ca + Cb
    yshape = (N, s * H, s * W, C) if layout == "nhwc" else (N, C, s * H, s * W)
    if out is None:
        out = torch.empty(yshape, dtype=a.dtype, device=a.device)
    else:
        _require(out, "out", a.dtype, a.device)
        if tuple(out.shape) != yshape:
            raise ValueError(f"out must have shape {yshape}")
    if b is None:
        rc = getattr(lib, fn_name)(_ptr(a), _ptr(out), N, H, W, Ca, lay, dt, _stream_handle(stream))
    else:
        rc = getattr(lib, fn_name)(_ptr(a), _ptr(b), _ptr(out), N, H, W, Ca, Cb, lay, dt, _stream_handle(stream))
    _check(rc)
    return out


def upsample_nearest2x(x, *, layout="nhwc", out=None, stream=None):
    """Nearest-neighbour 2x upsample on the GPU (bit-exact copy)."""
    return _resample("upsample_nearest2x", x, None, True, layout, out, stream)


def concat_channels(a, b, *, layout="nhwc", out=None, stream=None):
    """Channel concat [a, b] of two same-size maps on the GPU (bit-exact copy)."""
    return _resample("concat_channels", a, b, False, layout, out, stream)


def upsample2x_concat(a, b, *, layout="nhwc", out=None, stream=None):
    """concat_channels(upsample_nearest2x(a), b) in one pass (b is twice a's size)."""
    return _resample("upsample2x_concat", a, b, True, layout, out, stream)


def deconv_op(x, w, y, bias=None, alpha=None, *, act="none", layout="nhwc"):
    """An Op for conv_transpose4x4s2 (output in the stack's dtype)."""
    N, H, W, Cin = _nhwc_dims(x, layout)
    return Op(OP_DECONV, x.data_ptr(), w.data_ptr(), _tensor_ptr(bias), _tensor_ptr(alpha), None, y.data_ptr(),
              N, H, W, Cin, w.shape[1], 4, 4, 2, 1, _act_code(act, False))


def upsample_op(x, y, *, layout="nhwc"):
    """An Op for upsample_nearest2x."""
    N, H, W, C = _nhwc_dims(x, layout)
    return Op(OP_UPSAMPLE, x.data_ptr(), None, None, None, None, y.data_ptr(), N, H, W, C, 0, 0, 0, 0, 0, 0)


def concat_op(a, b, y, *, up=False, layout="nhwc"):
    """An Op for concat_channels, or with up=True upsample2x_concat (a is the small map)."""
    N, H, W, Ca = _nhwc_dims(a, layout)
    Cb = _nhwc_dims(b, layout)[3]
    return Op(OP_UPSAMPLE_CONCAT if up else OP_CONCAT, a.data_ptr(), None, None, None, b.data_ptr(),
              y.data_ptr(), N, H, W, Ca, Cb, 0, 0, 0, 0, 0)


def tune(N, H, W, Cin, Cout, kh, kw, stride, pad, act="none", *, residual=False, res_before_act=False,
         layout="nhwc", dtype=DTYPE_BF16, reps=20, workspace=None):
    """Time the kernel variants of one conv shape on the current device and keep the
    fastest for later calls of that shape (include/conv2d_fused.h, conv2d_tune).
    The candidates are those the workspace allows (default: the current stream's, grown
    to hold split-K in four); later calls use an entry only where their workspace allows
    it. Returns (variant name, average launch time in microseconds)."""
    buf = ctypes.create_string_buffer(256)
    us = ctypes.c_float(0.0)
    if torch.cuda.is_available():  # (without a device the call itself reports CONV2D_EHIP)
        dev = torch.device("cuda", torch.cuda.current_device())
        OH, OW = out_dim(H, kh, stride, pad), out_dim(W, kw, stride, pad)
        need = 4 * N * max(OH, 0) * max(OW, 0) * Cout * 4
        _use_workspace(dev, _stream_of(dev, None), workspace, need)
    n = _load().conv2d_tune(N, H, W, Cin, Cout, kh, kw, stride, pad, _act_code(act, res_before_act),
                            1 if residual else 0, _LAYOUTS[layout], dtype, reps, ctypes.byref(us), buf, 256)
    _check(n if n < 0 else OK)
    return buf.value.decode(), us.value


def tune_save(path) -> int:
    """Write the tuned-plan table to a text file; returns the number of records."""
    n = _load().conv2d_tune_save(os.fsencode(path))
    _check(n if n < 0 else OK)
    return n


def tune_load(path) -> int:
    """Add the records of a file written by tune_save; returns the number read."""
    n = _load().conv2d_tune_load(os.fsencode(path))
    _check(n if n < 0 else OK)
    return n


def tune_clear():
    """Forget every tuned plan."""
    _check(_load().conv2d_tune_clear())


def deconv_pack(w, stream=None):
    """Pack transposed-conv weights w [Cin, Cout, 4, 4] (bf16/f16, Cin % 8 == 0) once;
    returns (packed tensor, Cout) for conv_transpose4x4s2_prepacked."""
    lib = _load()
    dt = _dtype_code(w.dtype)
    if w.dim() != 4 or tuple(w.shape[2:]) != (4, 4):
        raise ValueError("w must be [Cin, Cout, 4, 4]")
    _require(w, "w", w.dtype, w.device)
    Cin, Cout = int(w.shape[0]), int(w.shape[1])
    nbytes = ctypes.c_size_t(0)
    _check(lib.conv_transpose4x4s2_packed_bytes(Cin, Cout, dt, ctypes.byref(nbytes)))
    wp = torch.empty(nbytes.value // w.element_size(), dtype=w.dtype, device=w.device)
    _check(lib.conv_transpose4x4s2_pack(_ptr(w), _ptr(wp), Cin, Cout, dt, _stream_handle(stream)))
    return wp, Cout


def conv_transpose4x4s2_prepacked(x, packed, bias=None, alpha=None, *, act="none", layout="nhwc", out_dtype=None,
                                  out=None, stream=None, workspace=None):
    """conv_transpose4x4s2 with weights packed by deconv_pack (``packed`` = its result)."""
    lib = _load()
    wp, Cout = packed
    lay = _LAYOUTS[layout]
    dt = _dtype_code(x.dtype)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    odt = _dtype_code(out_dtype)
    if layout == "nhwc":
        N, H, W, Cin = x.shape
    else:
        N, Cin, H, W = x.shape
    dev = x.device
    _require(x, "x", x.dtype, dev)
    _require(wp, "wp", x.dtype, dev)
    _require(bias, "bias", torch.float32, dev)
    _require(alpha, "alpha", torch.float32, dev)
    yshape = (N, 2 * H, 2 * W, Cout) if layout == "nhwc" else (N, Cout, 2 * H, 2 * W)
    if out is None:
        out = torch.empty(yshape, dtype=out_dtype, device=dev)
    else:
        _require(out, "out", out_dtype, dev)
        if tuple(out.shape) != yshape:
            raise ValueError(f"out must have shape {yshape}")
    st = _stream_of(dev, stream)
    with torch.cuda.device(dev):
        _use_workspace(dev, st, workspace, (x.numel() * x.element_size() + 255) // 256 * 256)
        rc = lib.conv_transpose4x4s2_prepacked(_ptr(x), _ptr(wp), _ptr(bias), _ptr(alpha), _ptr(out), N, H, W, Cin,
                                               Cout, _act_code(act, False), lay, dt, odt, _stream_handle(st))
    _check(rc)
    return out


def weights_to_ohwi(w, stream=None):
    """OIHW conv weights [Cout, Cin, kh, kw] (bf16/f16) -> a new OHWI tensor [Cout, kh, kw, Cin],
    for channel-first convs called with weights_ohwi=True (convert once, reuse)."""
    lib = _load()
    dt = _dtype_code(w.dtype)
    if w.dim() != 4:
        raise ValueError("w must be 4-D")
    _require(w, "w", w.dtype, w.device)
    Cout, Cin, kh, kw = (int(v) for v in w.shape)
    w2 = torch.empty((Cout, kh, kw, Cin), dtype=w.dtype, device=w.device)
    _check(lib.conv2d_weights_to_ohwi(_ptr(w), _ptr(w2), Cout, Cin, kh, kw, dt, _stream_handle(stream)))
    return w2
