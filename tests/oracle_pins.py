"""Pins that tie the CPU oracle to facts fixed outside it.

Each ``pin_*`` function raises AssertionError when the oracle ``orc`` (the
``oracle`` package, or a copy loaded from a deliberately broken build) gives
a wrong answer. The pins use hand-worked values, closed forms, invariants,
brute force and independent library routines (numpy matmul, torch's CPU
conv2d/max_pool2d/avg_pool2d in fp64, numpy/torch dtype casts); none of them
retypes the oracle's own loop.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch
import torch.nn.functional as F

from conftest import read_golden


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rel=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rel * scale, f"{what}: max err {err} > {rel} * {scale}"


# --- convolution -------------------------------------------------------------------------


def pin_worked_example(orc):
    """Hand-worked 3x3 example (tests/golden/conv3x3_worked_example.txt)."""
    g = read_golden("conv3x3_worked_example.txt")
    x = g["x"].reshape(1, 1, 3, 3)
    w = g["w"].reshape(1, 1, 3, 3)
    assert np.array_equal(orc.conv2d(x, w, stride=1, pad=1, layout="nchw")[0, 0], g["y_s1_p1"])
    assert np.array_equal(orc.conv2d(x, w, stride=2, pad=1, layout="nchw")[0, 0], g["y_s2_p1"])
    assert np.array_equal(orc.conv2d(x, w, stride=1, pad=0, layout="nchw")[0, 0], g["y_s1_p0"])
    y = orc.conv2d(x, w, np.array([-150.0]), stride=1, pad=1, act="relu", layout="nchw")
    assert np.array_equal(y[0, 0], g["y_s1_p1_bias_m150_relu"])


def pin_geometry(orc):
    """Output sizes: floor((H + 2p - k)/s) + 1 (inferencelayer `conv()`), pools."""
    cases = [((32, 3, 1, 1), 32), ((640, 3, 2, 1), 320), ((320, 3, 2, 1), 160),
             ((160, 3, 2, 1), 80), ((80, 3, 2, 1), 40), ((40, 3, 2, 1), 20),
             ((80, 1, 1, 0), 80), ((68, 3, 1, 1), 68), ((120, 3, 1, 1), 120),
             ((7, 3, 2, 0), 3), ((2, 3, 1, 0), -1), ((1, 1, 2, 0), 1), ((5, 5, 1, 2), 5)]
    for (n, k, s, p), want in cases:
        assert orc.out_dim(n, k, s, p) == want, (n, k, s, p)
    # conv output shapes follow the same formula
    x = np.zeros((1, 7, 9, 2))
    w = np.zeros((3, 3, 3, 2))
    assert orc.conv2d(x, w, stride=2, pad=1).shape == (1, 4, 5, 3)
    # maxpool 3x3 s2 p1 and avgpool 2x2 s2
    assert orc.maxpool3x3s2(np.zeros((1, 320, 320, 1))).shape == (1, 160, 160, 1)
    assert orc.maxpool3x3s2(np.zeros((1, 7, 6, 1))).shape == (1, 4, 3, 1)
    assert orc.avgpool2x2(np.zeros((1, 160, 160, 1))).shape == (1, 80, 80, 1)
    assert orc.avgpool2x2(np.zeros((1, 7, 5, 1))).shape == (1, 3, 2, 1)


def pin_pointwise_is_matmul(orc):
    """A 1x1 stride-1 conv is a GEMM over pixels (inferencelayer `conv()`: the NHWC
    map is the [m,k] GEMM input)."""
    r = _rng(11)
    x = r.standard_normal((2, 5, 7, 6))
    w = r.standard_normal((4, 1, 1, 6))
    b = r.uniform(-1, 1, 4)
    ref = np.maximum(x.reshape(-1, 6) @ w.reshape(4, 6).T + b, 0.0).reshape(2, 5, 7, 4)
    _close(orc.conv2d(x, w, b, act="relu"), ref, what="1x1 nhwc")
    ref2 = (x.reshape(-1, 6) @ w.reshape(4, 6).T).reshape(2, 5, 7, 4).transpose(0, 3, 1, 2)
    _close(orc.conv2d(x.transpose(0, 3, 1, 2), w.transpose(0, 3, 1, 2), layout="nchw"), ref2,
           what="1x1 nchw")


def pin_delta_kernel(orc):
    """A one-hot kernel copies (or shifts) the input; stride 2 subsamples."""
    r = _rng(12)
    C = 3
    x = r.standard_normal((2, C, 6, 5))
    w = np.zeros((C, C, 3, 3))
    for c in range(C):
        w[c, c, 1, 1] = 1.0
    assert np.array_equal(orc.conv2d(x, w, stride=1, pad=1, layout="nchw"), x)
    assert np.array_equal(orc.conv2d(x, w, stride=2, pad=1, layout="nchw"), x[:, :, ::2, ::2])
    # off-centre tap (ky=0, kx=2) reads x[oh-1, ow+1] (no kernel flip), zero outside
    w2 = np.zeros((C, C, 3, 3))
    for c in range(C):
        w2[c, c, 0, 2] = 1.0
    want = np.zeros_like(x)
    want[:, :, 1:, :-1] = x[:, :, :-1, 1:]
    assert np.array_equal(orc.conv2d(x, w2, stride=1, pad=1, layout="nchw"), want)
    # channel routing: output co reads input channel (co + 1) % C
    w3 = np.zeros((C, C, 1, 1))
    for c in range(C):
        w3[c, (c + 1) % C, 0, 0] = 1.0
    assert np.array_equal(orc.conv2d(x, w3, layout="nchw"), x[:, [1, 2, 0]])


def _im2col_nhwc(x, kh, kw, s, p):
    """Explicit patch matrix [N*OH*OW, kh*kw*C] in (dy, dx, c) order, zero outside the image
    (inferencelayer `IM2COL_SRC`)."""
    N, H, W, C = x.shape
    OH, OW = (H + 2 * p - kh) // s + 1, (W + 2 * p - kw) // s + 1
    cols = np.zeros((N, OH, OW, kh * kw * C))
    for n, oy, ox, dy, dx in itertools.product(range(N), range(OH), range(OW), range(kh),
                                               range(kw)):
        iy, ix = oy * s + dy - p, ox * s + dx - p
        if 0 <= iy < H and 0 <= ix < W:
            tap = dy * kw + dx
            cols[n, oy, ox, tap * C:(tap + 1) * C] = x[n, iy, ix, :]
    return cols.reshape(N * OH * OW, kh * kw * C), (N, OH, OW)


def pin_im2col_bruteforce(orc, exhaustive=False):
    """Brute-force im2col then matmul with the [k, n]-transposed weight equals the oracle."""
    r = _rng(13)
    ns = (1, 2)
    hs = (1, 2, 3, 5, 7) if exhaustive else (1, 3, 5)
    cs = (1, 2, 5) if exhaustive else (1, 3)
    count = 0
    for N, H, W, Cin, Cout, k, s, p in itertools.product(ns, hs, hs, cs, cs, (1, 3), (1, 2),
                                                         (0, 1)):
        if H + 2 * p < k or W + 2 * p < k:
            continue
        if not exhaustive and (H == W) and count % 2:
            count += 1
            continue
        count += 1
        x = r.standard_normal((N, H, W, Cin))
        w = r.standard_normal((Cout, k, k, Cin))
        cols, (n_, OH, OW) = _im2col_nhwc(x, k, k, s, p)
        wt = w.reshape(Cout, k * k * Cin).T  # [k, n]
        ref = (cols @ wt).reshape(n_, OH, OW, Cout)
        _close(orc.conv2d(x, w, stride=s, pad=p), ref, what=f"im2col {N,H,W,Cin,Cout,k,s,p}")


def pin_constant_borders(orc):
    """x == 1, w == 1, no bias: each output counts Cin times its in-range taps."""
    for (H, W, k, s, p, Cin) in [(5, 6, 3, 1, 1, 3), (7, 7, 3, 2, 1, 2), (4, 9, 5, 1, 2, 1),
                                 (6, 5, 3, 2, 0, 4)]:
        x = np.ones((1, Cin, H, W))
        w = np.ones((2, Cin, k, k))
        y = orc.conv2d(x, w, stride=s, pad=p, layout="nchw")
        OH, OW = y.shape[2:]
        for oh in range(OH):
            rows = sum(0 <= oh * s + ky - p < H for ky in range(k))
            for ow in range(OW):
                cols = sum(0 <= ow * s + kx - p < W for kx in range(k))
                assert y[0, 0, oh, ow] == Cin * rows * cols == y[0, 1, oh, ow]


def pin_linearity(orc):
    r = _rng(14)
    x1, x2 = r.standard_normal((2, 2, 6, 6, 3))
    w = r.standard_normal((4, 3, 3, 3))
    a, b = 0.75, -1.5
    lhs = orc.conv2d(a * x1 + b * x2, w, stride=1, pad=1)
    rhs = a * orc.conv2d(x1, w, stride=1, pad=1) + b * orc.conv2d(x2, w, stride=1, pad=1)
    _close(lhs, rhs, what="linearity")


def pin_layout_equivalence(orc):
    r = _rng(15)
    x = r.standard_normal((2, 7, 6, 3))
    w = r.standard_normal((5, 3, 3, 3))
    b = r.uniform(-1, 1, 5)
    al = r.uniform(0, 0.25, 5)
    res = r.standard_normal((2, 4, 3, 5))
    y1 = orc.conv2d(x, w, b, al, res, stride=2, pad=1, act="prelu")
    y2 = orc.conv2d(x.transpose(0, 3, 1, 2), w.transpose(0, 3, 1, 2), b, al,
                    res.transpose(0, 3, 1, 2), stride=2, pad=1, act="prelu", layout="nchw")
    assert np.array_equal(y1, y2.transpose(0, 2, 3, 1))


def pin_batch_independence(orc):
    r = _rng(16)
    x = r.standard_normal((3, 5, 5, 4))
    w = r.standard_normal((2, 3, 3, 4))
    yb = orc.conv2d(x, w, stride=1, pad=1, act="silu")
    for n in range(3):
        assert np.array_equal(yb[n:n + 1], orc.conv2d(x[n:n + 1], w, stride=1, pad=1, act="silu"))


def _torch_layer(x, w, b, al, res, s, p, act, pre):
    """torch CPU fp64 conv2d (channel-first) plus the epilogue built from torch ops."""
    xt, wt = torch.from_numpy(x), torch.from_numpy(w)
    v = F.conv2d(xt, wt, torch.from_numpy(b) if b is not None else None, stride=s, padding=p)

    def act_fn(u):
        if act == "relu":
            return torch.relu(u)
        if act == "silu":
            return F.silu(u)
        if act == "prelu":
            return F.prelu(u, torch.from_numpy(al))
        return u
    if res is not None:
        rt = torch.from_numpy(res)
        v = act_fn(v + rt) if pre else act_fn(v) + rt
    else:
        v = act_fn(v)
    return v.numpy()


def pin_torch_conv2d(orc):
    """Cross-check with torch's CPU conv2d in fp64 over random shapes and epilogues."""
    r = _rng(17)
    shapes = [(1, 3, 9, 11, 4, 3, 1, 1), (2, 5, 8, 8, 6, 3, 2, 1), (1, 2, 7, 5, 3, 5, 1, 2),
              (2, 4, 6, 7, 5, 1, 1, 0), (1, 3, 10, 9, 2, 3, 2, 0), (1, 1, 4, 4, 1, 3, 1, 1)]
    acts = ["none", "relu", "silu", "prelu"]
    for i, (N, Cin, H, W, Cout, k, s, p) in enumerate(shapes):
        for act in acts:
            for resmode in (None, "pre", "post"):
                x = r.standard_normal((N, Cin, H, W))
                w = r.standard_normal((Cout, Cin, k, k))
                b = r.uniform(-0.5, 0.5, Cout)
                al = r.uniform(0, 0.25, Cout)
                OH, OW = (H + 2 * p - k) // s + 1, (W + 2 * p - k) // s + 1
                res = r.standard_normal((N, Cout, OH, OW)) if resmode else None
                got = orc.conv2d(x, w, b, al if act == "prelu" else None, res, stride=s,
                                 pad=p, act=act, res_before_act=resmode == "pre", layout="nchw")
                want = _torch_layer(x, w, b, al, res, s, p, act, resmode == "pre")
                _close(got, want, what=f"torch case {i} {act} {resmode}")


def _scalar_layer(orc, v, act, alpha=None, r=None, pre=False):
    """Push scalar v through a 1x1 conv with weight 1, so the output is act(v) etc."""
    x = np.array([[[[v]]]])
    w = np.ones((1, 1, 1, 1))
    al = None if alpha is None else np.array([alpha])
    res = None if r is None else np.array([[[[r]]]])
    return float(orc.conv2d(x, w, None, al, res, act=act, res_before_act=pre)[0, 0, 0, 0])


def pin_activations(orc):
    """ReLU max(v,0), SiLU v/(1+e^-v) (rlx-wgpu `apply_activation_host`), PReLU per channel
    (framecast `wgslConv`), checked at closed-form points."""
    assert _scalar_layer(orc, -1.0, "relu") == 0.0
    assert _scalar_layer(orc, 2.0, "relu") == 2.0
    assert _scalar_layer(orc, 0.0, "silu") == 0.0
    assert abs(_scalar_layer(orc, 1.0, "silu") - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(_scalar_layer(orc, -2.0, "silu") - (-2.0 / (1.0 + math.exp(2.0)))) < 1e-15
    assert _scalar_layer(orc, -2.0, "prelu", alpha=0.25) == -0.5
    assert _scalar_layer(orc, 3.0, "prelu", alpha=0.25) == 3.0
    assert _scalar_layer(orc, 0.0, "prelu", alpha=0.25) == 0.0
    assert _scalar_layer(orc, -3.0, "none") == -3.0
    # silu saturates to ~v for large v and to ~0 for very negative v
    assert _scalar_layer(orc, 50.0, "silu") == 50.0
    assert abs(_scalar_layer(orc, -800.0, "silu")) < 1e-300
    # per-channel slopes: two channels, two alphas
    x = np.full((1, 1, 1, 2), -4.0)
    w = np.zeros((2, 1, 1, 2))
    w[0, 0, 0, 0] = 1.0
    w[1, 0, 0, 1] = 1.0
    y = orc.conv2d(x, w, None, np.array([0.25, 0.125]), act="prelu")
    assert y[0, 0, 0, 0] == -1.0 and y[0, 0, 0, 1] == -0.5


def pin_residual_order(orc):
    """Residual before the activation (inferencelayer block sum + `addact` relu) vs after it
    (framecast `wgslConv`): v=-1, r=2, ReLU gives 1 and 2 respectively."""
    assert _scalar_layer(orc, -1.0, "relu", r=2.0, pre=True) == 1.0
    assert _scalar_layer(orc, -1.0, "relu", r=2.0, pre=False) == 2.0
    assert _scalar_layer(orc, -3.0, "relu", r=2.0, pre=True) == 0.0
    assert _scalar_layer(orc, -4.0, "prelu", alpha=0.25, r=0.5, pre=False) == -0.5
    # bias joins before the residual and the activation
    x = np.array([[[[1.0]]]])
    y = orc.conv2d(x, np.ones((1, 1, 1, 1)), np.array([-3.0]), None, np.array([[[[1.5]]]]),
                   act="relu", res_before_act=True)
    assert y[0, 0, 0, 0] == 0.0


def pin_points_match_full(orc):
    r = _rng(18)
    x = r.standard_normal((2, 9, 8, 5))
    w = r.standard_normal((6, 3, 3, 5))
    b = r.uniform(-1, 1, 6)
    res = r.standard_normal((2, 5, 4, 6))
    full = orc.conv2d(x, w, b, None, res, stride=2, pad=1, act="silu", res_before_act=True)
    idx = np.array([[n, oh, ow, co] for n in range(2) for oh in (0, 4) for ow in (0, 3)
                    for co in (0, 5)])
    pts = orc.conv2d_points(x, w, b, None, res, idx, stride=2, pad=1, act="silu",
                            res_before_act=True)
    assert np.array_equal(pts, full[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]])


# --- pools -------------------------------------------------------------------------------


def pin_maxpool(orc):
    g = read_golden("pools_worked_example.txt")
    x4 = g["maxpool_ramp4_x"].reshape(1, 1, 4, 4)
    assert np.array_equal(orc.maxpool3x3s2(x4, layout="nchw")[0, 0], g["maxpool_ramp4_y"])
    x5 = np.arange(25, dtype=np.float64).reshape(1, 1, 5, 5)
    assert np.array_equal(orc.maxpool3x3s2(x5, layout="nchw")[0, 0], g["maxpool_ramp5_y"])
    r = _rng(19)
    for shape in [(2, 3, 7, 8), (1, 4, 6, 5), (1, 1, 1, 1), (1, 2, 2, 3)]:
        x = r.standard_normal(shape)
        want = F.max_pool2d(torch.from_numpy(x), 3, 2, 1).numpy()
        assert np.array_equal(orc.maxpool3x3s2(x, layout="nchw"), want), shape
    # all-negative input: the -inf padding never wins
    x = -np.abs(r.standard_normal((1, 2, 5, 5))) - 1.0
    assert np.all(orc.maxpool3x3s2(x, layout="nchw") <= -1.0)
    # NaN taps are skipped, an all-NaN window gives -inf, and of equal zeros the first in
    # row-major tap order is kept (hand-worked, tests/golden/pools_worked_example.txt)
    for xk, yk, shape in [("maxpool_nan_x", "maxpool_nan_y", (4, 4)), ("maxpool_zeros_x", "maxpool_zeros_y", (3, 3))]:
        y = orc.maxpool3x3s2(g[xk].reshape(1, 1, *shape), layout="nchw")[0, 0]
        assert np.array_equal(y, g[yk]) and np.array_equal(np.signbit(y), np.signbit(g[yk])), (xk, y)
    y = orc.maxpool3x3s2(np.full((1, 1, 3, 3), np.nan), layout="nchw")[0, 0]
    assert np.array_equal(y, g["maxpool_allnan_y"]), y


def pin_avgpool(orc):
    g = read_golden("pools_worked_example.txt")
    x = g["avgpool_order_x"].reshape(1, 1, 2, 2)
    assert np.array_equal(orc.avgpool2x2(x, layout="nchw")[0, 0], g["avgpool_order_y"])
    # constant maps stay constant
    for c in (0.3, -7.25, 1e-3):
        x = np.full((1, 2, 4, 6), np.float32(c), dtype=np.float64)
        assert np.all(orc.avgpool2x2(x, layout="nchw") == np.float32(c))
    # small integers: every order is exact, so torch's avg_pool2d must agree; odd sizes drop
    # the last row/column
    r = _rng(20)
    for shape in [(2, 3, 6, 8), (1, 2, 7, 5), (1, 1, 2, 2)]:
        x = r.integers(-50, 50, size=shape).astype(np.float64)
        want = F.avg_pool2d(torch.from_numpy(x), 2, 2).numpy()
        assert np.array_equal(orc.avgpool2x2(x, layout="nchw").astype(np.float64), want), shape
    # channel-last equals channel-first
    x = r.standard_normal((2, 6, 4, 3)).astype(np.float32)
    a = orc.avgpool2x2(x, layout="nhwc")
    b = orc.avgpool2x2(x.transpose(0, 3, 1, 2), layout="nchw")
    assert np.array_equal(a, b.transpose(0, 2, 3, 1))


# --- storage rounding --------------------------------------------------------------------


def _quantize_probe_values(seed):
    r = _rng(seed)
    vals = [r.standard_normal(20000) * 10.0 ** r.integers(-9, 6, 20000),
            np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 7e4,
                      6.1e-5, 5.96e-8, 2.98e-8, 2.99e-8, 1e-9, 3.4e38, 3.5e38, 1e-40, 1e-46])]
    # exact ties between neighbours of each format
    base = r.uniform(1, 2, 2000)
    for bits in (8, 11, 24):
        q = np.ldexp(np.floor(np.ldexp(base, bits - 1)), 1 - bits)
        vals.append(q + np.ldexp(1.0, -bits))
    return np.concatenate(vals)


def pin_quantize(orc):
    v = _quantize_probe_values(21)
    got16 = orc.quantize(v, "f16")
    want16 = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(got16, want16)
    got32 = orc.quantize(v, "f32")
    with np.errstate(over="ignore"):
        want32 = v.astype(np.float32).astype(np.float64)
    assert np.array_equal(got32, want32)
    # bf16: torch's CPU cast from fp32 is one round-to-nearest-even; start from fp32 values
    v32 = want32[np.isfinite(want32)]
    gotb = orc.quantize(v32, "bf16")
    wantb = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(gotb, wantb)
    nan = orc.quantize(np.array([np.nan]), "bf16")
    assert np.isnan(nan[0])


# --- transposed convolution, upsample, concat -------------------------------------------


def _deconv_scatter(x, w):
    """ConvTranspose2d 4x4 s2 p1 written as the scatter the layer is defined by:
    every input pixel adds x * w[ci, co, ky, kx] to output (2*iy - 1 + ky, 2*ix - 1 + kx)
    when that output exists. Pure Python loops, NCHW, tiny sizes only."""
    N, Cin, H, W = x.shape
    Cout = w.shape[1]
    y = np.zeros((N, Cout, 2 * H, 2 * W))
    for n in range(N):
        for ci in range(Cin):
            for iy in range(H):
                for ix in range(W):
                    for ky in range(4):
                        for kx in range(4):
                            oy, ox = 2 * iy - 1 + ky, 2 * ix - 1 + kx
                            if 0 <= oy < 2 * H and 0 <= ox < 2 * W:
                                for co in range(Cout):
                                    y[n, co, oy, ox] += x[n, ci, iy, ix] * w[ci, co, ky, kx]
    return y


def pin_deconv_scatter_bruteforce(orc):
    """The gather the oracle evaluates equals the scatter definition on small shapes,
    including 1x1 and odd sizes."""
    r = _rng(40)
    for (N, Cin, Cout, H, W) in [(1, 1, 1, 1, 1), (2, 3, 2, 3, 4), (1, 2, 3, 5, 2), (1, 4, 1, 2, 7)]:
        x = r.standard_normal((N, Cin, H, W))
        w = r.standard_normal((Cin, Cout, 4, 4))
        _close(orc.conv_transpose4x4s2(x, w, layout="nchw"), _deconv_scatter(x, w), what=f"scatter {N, Cin, H, W}")


def pin_deconv_is_adjoint_of_conv(orc):
    """A transposed conv is the adjoint of the stride-2 pad-1 4x4 conv with the same
    weights read as [out = Cin][in = Cout]: <T(x), y> = <x, C(y)> (the conv side is the
    oracle's own, separately pinned conv)."""
    r = _rng(41)
    N, Cin, Cout, H, W = 2, 5, 3, 6, 7
    x = r.standard_normal((N, Cin, H, W))
    w = r.standard_normal((Cin, Cout, 4, 4))
    y = r.standard_normal((N, Cout, 2 * H, 2 * W))
    lhs = float(np.sum(orc.conv_transpose4x4s2(x, w, layout="nchw") * y))
    cy = orc.conv2d(y, w, stride=2, pad=1, layout="nchw")
    assert cy.shape == x.shape
    rhs = float(np.sum(x * cy))
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), (lhs, rhs)


def pin_deconv_single_pixel(orc):
    """One input pixel of one channel set to 1: the output is that channel's 4x4 kernel
    placed with its top-left tap at (2*iy - 1, 2*ix - 1), cut at the border; bias is
    added everywhere and the activation applied (closed form)."""
    Cin, Cout, H, W = 2, 3, 4, 5
    w = np.arange(Cin * Cout * 16, dtype=np.float64).reshape(Cin, Cout, 4, 4) / 7.0
    b = np.array([0.5, -1.0, 2.0])
    for (ci, iy, ix) in [(0, 0, 0), (1, 2, 3), (1, 3, 4)]:
        x = np.zeros((1, Cin, H, W))
        x[0, ci, iy, ix] = 1.0
        want = np.zeros((1, Cout, 2 * H, 2 * W)) + b[None, :, None, None]
        for ky in range(4):
            for kx in range(4):
                oy, ox = 2 * iy - 1 + ky, 2 * ix - 1 + kx
                if 0 <= oy < 2 * H and 0 <= ox < 2 * W:
                    want[0, :, oy, ox] += w[ci, :, ky, kx]
        _close(orc.conv_transpose4x4s2(x, w, b, layout="nchw"), want, what="single pixel")
        got = orc.conv_transpose4x4s2(x.transpose(0, 2, 3, 1), w, b, act="relu", layout="nhwc")
        _close(got, np.maximum(want, 0.0).transpose(0, 2, 3, 1), what="single pixel nhwc relu")


def pin_deconv_torch(orc):
    """torch.nn.functional.conv_transpose2d (fp64, CPU; weight [Cin, Cout, 4, 4],
    stride 2, padding 1) with bias and PReLU."""
    r = _rng(42)
    x = r.standard_normal((2, 6, 5, 4))
    w = r.standard_normal((6, 4, 4, 4))
    b = r.uniform(-1, 1, 4)
    al = r.uniform(0, 0.25, 4)
    t = torch.nn.functional.conv_transpose2d(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b),
                                             stride=2, padding=1)
    t = torch.where(t >= 0, t, torch.from_numpy(al)[None, :, None, None] * t).numpy()
    _close(orc.conv_transpose4x4s2(x, w, b, al, act="prelu", layout="nchw"), t, what="torch deconv")


def pin_upsample_concat(orc):
    """Nearest 2x upsample of a ramp is the ramp at (oy // 2, ox // 2); concat puts a's
    channels first (closed forms, both layouts)."""
    N, H, W, C = 2, 3, 5, 4
    x = np.arange(N * H * W * C, dtype=np.float64).reshape(N, H, W, C)
    up = orc.upsample_nearest2x(x)
    assert up.shape == (N, 2 * H, 2 * W, C)
    for oy in range(2 * H):
        for ox in range(2 * W):
            assert np.array_equal(up[:, oy, ox], x[:, oy // 2, ox // 2])
    assert np.array_equal(orc.upsample_nearest2x(x.transpose(0, 3, 1, 2), layout="nchw"), up.transpose(0, 3, 1, 2))
    b = -np.arange(N * H * W * 3, dtype=np.float64).reshape(N, H, W, 3)
    cat = orc.concat_channels(x, b)
    assert cat.shape == (N, H, W, C + 3)
    assert np.array_equal(cat[..., :C], x) and np.array_equal(cat[..., C:], b)
    catc = orc.concat_channels(x.transpose(0, 3, 1, 2), b.transpose(0, 3, 1, 2), layout="nchw")
    assert np.array_equal(catc, cat.transpose(0, 3, 1, 2))


ALL_PINS = [pin_worked_example, pin_geometry, pin_pointwise_is_matmul, pin_delta_kernel,
            pin_im2col_bruteforce, pin_constant_borders, pin_linearity, pin_layout_equivalence,
            pin_batch_independence, pin_torch_conv2d, pin_activations, pin_residual_order,
            pin_points_match_full, pin_maxpool, pin_avgpool, pin_deconv_scatter_bruteforce,
            pin_deconv_is_adjoint_of_conv, pin_deconv_single_pixel, pin_deconv_torch, pin_upsample_concat]
