"""GPU parity of conv2d_fused_maxpool3x3s2 (conv + 3x3/s2/p1 max pool in one call)
against the CPU oracle, and bit for bit against the two-call path (needs an MI355X)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import bits_equal, gate, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")
DT = {"f32": 0, "bf16": 1, "f16": 2}


def _dev(t):
    return None if t is None else t.to(DEV)


def _fused(x, spec, layout):
    return c2d.conv2d_fused_maxpool3x3s2(_dev(x), _dev(spec.w), _dev(spec.bias), _dev(spec.alpha),
                                         stride=spec.stride, pad=spec.pad, act=spec.act, layout=layout)


def _two_calls(x, spec, layout):
    y = c2d.conv2d_fused(_dev(x), _dev(spec.w), _dev(spec.bias), _dev(spec.alpha), stride=spec.stride,
                         pad=spec.pad, act=spec.act, layout=layout)
    return c2d.maxpool3x3s2(y, layout=layout)


def _oracle(x, spec, layout):
    conv = oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias) if spec.bias is not None else None,
                         to64(spec.alpha) if spec.alpha is not None else None, None, stride=spec.stride,
                         pad=spec.pad, act=spec.act, layout=layout)
    return oracle.maxpool3x3s2(conv, layout=layout)


def _check(x, spec, layout, dtype, what, want_fused, bitexact_vs_two_calls=True):
    n, h, w = (x.shape[0], x.shape[1], x.shape[2]) if layout == "nhwc" else (x.shape[0], x.shape[2], x.shape[3])
    args = (n, h, w, spec.cin, spec.cout, spec.k, spec.k, spec.stride, spec.pad, 0,
            0 if layout == "nhwc" else 1, DT[dtype])
    plan = c2d.plan_maxpool(*args)
    print(f"case {what} plan {plan}", flush=True)
    assert ("fused" in plan) == want_fused, plan
    y = _fused(x, spec, layout)
    torch.cuda.synchronize()
    gate(to64(y), _oracle(x, spec, layout), dtype, what=what)
    if bitexact_vs_two_calls:
        # same conv kernel family (the per-pixel sums do not depend on the tiling);
        # rounding is monotone, so pooling before or after the rounding gives the same bits
        assert c2d.plan(*args).split()[0] == plan.split()[0], (c2d.plan(*args), plan)
        y2 = _two_calls(x, spec, layout)
        torch.cuda.synchronize()
        assert bits_equal(y, y2), what


# The 3-channel stem in one kernel: (n, h, w, cout, stride, act, dtype). Ragged pooled
# widths (not a multiple of the 15 columns a wave pools, nor of the 4 waves), odd and
# even conv sizes (the last pool window clipped or not), one-row images and the
# narrowest width.
FUSED = [
    (1, 17, 24, 32, 2, "silu", "bf16"),
    (2, 32, 40, 64, 2, "relu", "f16"),
    (1, 21, 16, 32, 1, "prelu", "bf16"),
    (3, 9, 8, 16, 1, "none", "bf16"),
    (1, 64, 248, 48, 2, "relu", "bf16"),
    (1, 1, 8, 32, 2, "relu", "bf16"),
    (1, 2, 8, 32, 1, "silu", "f16"),
    (2, 130, 136, 64, 2, "relu", "bf16"),
    (1, 40, 488, 24, 1, "silu", "f16"),
    (1, 61, 960, 32, 2, "prelu", "bf16"),
    (2, 33, 1208, 8, 1, "relu", "bf16"),
    # fp32 storage: the 32x32x2 fp32 kernel
    (1, 17, 24, 32, 2, "silu", "f32"),
    (2, 21, 20, 64, 1, "relu", "f32"),
    (1, 9, 36, 12, 2, "prelu", "f32"),
    (1, 1, 4, 32, 2, "relu", "f32"),
    (1, 61, 964, 32, 2, "none", "f32"),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "-".join(map(str, c)))
def test_fused_stem_maxpool(case):
    n, h, w, cout, s, act, dtype = case
    x, spec, _ = wl.random_conv_case(zlib.crc32(repr(case).encode()), n=n, h=h, w=w, cin=3, cout=cout, k=3,
                                     stride=s, pad=1, act=act, layout="nhwc", dtype=dtype, x_dist="uniform")
    _check(x, spec, "nhwc", dtype, str(case), want_fused=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_fused_stem_maxpool_full_image(dtype):
    """The 640x640 stem conv (3 -> 32, stride 2, SiLU) and its max pool: 1x160x160x32."""
    wk = wl.conv2_stem(dtype)
    spec = wk.layers[0]
    _check(wk.x, spec, "nhwc", dtype, f"stem 640x640 {dtype}", want_fused=True)


# Narrow 3x3 stride-1 layers (Cin 16 or 32) on the halo-tile kernel with the pool in its
# epilogue: (n, h, w, cin, cout, act, dtype). Runs of tiles down the image with a carry
# row between tiles, ragged pooled widths and heights, partial channel blocks, images
# of one pixel, and the ResNet-D stem's third conv at full size.
HALO_FUSED = [
    (1, 9, 11, 16, 16, "relu", "bf16"),
    (2, 37, 45, 32, 64, "prelu", "f16"),
    (1, 1, 1, 32, 32, "relu", "bf16"),
    (2, 33, 65, 16, 40, "silu", "bf16"),
    (3, 8, 32, 32, 24, "none", "bf16"),
    (1, 130, 66, 32, 64, "relu", "bf16"),
    (2, 64, 100, 16, 64, "silu", "f16"),
    (1, 320, 64, 32, 64, "relu", "bf16"),
    (2, 4, 4, 32, 8, "prelu", "bf16"),
    (4, 160, 160, 32, 64, "relu", "bf16"),
    (4, 320, 320, 32, 64, "relu", "bf16"),
    # ReLU in f16 (the packed-maximum pool path converts pairs with the f16 instruction)
    (2, 37, 45, 32, 64, "relu", "f16"),
    (1, 64, 100, 16, 32, "relu", "f16"),
]


@pytest.mark.parametrize("case", HALO_FUSED, ids=lambda c: "-".join(map(str, c)))
def test_fused_halo_maxpool(case):
    n, h, w, cin, cout, act, dtype = case
    x, spec, _ = wl.random_conv_case(zlib.crc32(repr(case).encode()), n=n, h=h, w=w, cin=cin, cout=cout, k=3,
                                     stride=1, pad=1, act=act, layout="nhwc", dtype=dtype)
    _check(x, spec, "nhwc", dtype, str(case), want_fused=True)


# Shapes outside the fused kernel: the conv into the library scratch, then the pool.
# (n, h, w, cin, cout, k, stride, pad, act, layout, dtype, same kernels as two calls)
UNFUSED = [
    (1, 23, 19, 3, 32, 3, 2, 1, "silu", "nhwc", "f32", True),     # fp32 stem, W % 4 != 0: direct kernel
    (1, 20, 22, 3, 32, 3, 2, 1, "relu", "nhwc", "bf16", True),    # W % 8 != 0
    (2, 18, 16, 3, 72, 3, 2, 1, "relu", "nhwc", "bf16", True),    # Cout > 64
    (1, 30, 26, 64, 64, 3, 1, 1, "prelu", "nhwc", "f16", True),   # halo kernel, Cin 64
    (2, 17, 23, 40, 72, 3, 2, 1, "relu", "nchw", "f16", False),   # channel-first: general kernel
    (1, 16, 18, 3, 16, 3, 2, 1, "silu", "nchw", "f32", True),
    (1, 10, 10, 512, 512, 3, 1, 1, "relu", "nhwc", "bf16", False),  # wide layer: halo-tile GEMM
    (1, 12, 14, 16, 24, 5, 2, 2, "none", "nhwc", "bf16", True),
]


@pytest.mark.parametrize("case", UNFUSED, ids=lambda c: "-".join(map(str, c)))
def test_two_kernel_path(case):
    n, h, w, cin, cout, k, s, p, act, layout, dtype, same = case
    x, spec, _ = wl.random_conv_case(zlib.crc32(repr(case).encode()), n=n, h=h, w=w, cin=cin, cout=cout, k=k,
                                     stride=s, pad=p, act=act, layout=layout, dtype=dtype)
    _check(x, spec, layout, dtype, str(case), want_fused=False, bitexact_vs_two_calls=same)


def test_fused_writes_only_the_pooled_map():
    """Guard bytes around y keep their value, and repeated calls give the same bits."""
    x, spec, _ = wl.random_conv_case(11, n=2, h=50, w=64, cin=3, cout=32, k=3, stride=2, pad=1, act="relu",
                                     layout="nhwc", dtype="bf16", x_dist="uniform")
    ph, pw = (25 - 1) // 2 + 1, (32 - 1) // 2 + 1  # conv 25 x 32
    numel = 2 * ph * pw * 32
    buf = torch.full((numel + 2 * 4096,), 7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[4096:4096 + numel].view(2, ph, pw, 32)
    c2d.conv2d_fused_maxpool3x3s2(_dev(x), _dev(spec.w), _dev(spec.bias), None, stride=2, pad=1, act="relu",
                                  out=out)
    first = out.clone()
    c2d.conv2d_fused_maxpool3x3s2(_dev(x), _dev(spec.w), _dev(spec.bias), None, stride=2, pad=1, act="relu",
                                  out=out)
    torch.cuda.synchronize()
    assert bits_equal(first, out)
    assert torch.all(buf[:4096] == 7.0) and torch.all(buf[4096 + numel:] == 7.0)
    gate(to64(out), _oracle(x, spec, "nhwc"), "bf16", what="guarded")


# NaN in the input (a NaN pixel makes every conv output whose window holds it NaN): the
# fused kernels skip NaN and give -inf for an all-NaN window, bit for bit as the two-call
# path, and agree with the oracle chain (finite outputs within the gate, -inf exactly
# where the oracle has it). (kind, n, h, w, cin, cout, stride, act, NaN block rows, cols)
NAN_CASES = [
    ("stem", 1, 40, 48, 3, 32, 2, "silu", (4, 13), (12, 21)),
    ("halo", 1, 30, 40, 32, 64, 1, "none", (8, 14), (10, 16)),
    ("halo", 2, 17, 33, 16, 24, 1, "silu", (0, 6), (26, 33)),
]


@pytest.mark.parametrize("case", NAN_CASES, ids=lambda c: "-".join(map(str, c[:8])))
def test_fused_maxpool_with_nan_inputs(case):
    kind, n, h, w, cin, cout, s, act, (r0, r1), (c0, c1) = case
    x, spec, _ = wl.random_conv_case(zlib.crc32(repr(case).encode()), n=n, h=h, w=w, cin=cin, cout=cout, k=3,
                                     stride=s, pad=1, act=act, layout="nhwc", dtype="bf16",
                                     x_dist="uniform" if kind == "stem" else "normal")
    x = x.clone()
    rng = np.random.default_rng(5)
    pts = rng.integers(0, [n, h, w], size=(6, 3))
    for b, i, j in pts:
        x[b, i, j, rng.integers(0, cin)] = float("nan")
    x[0, r0:r1, c0:c1, :] = float("nan")
    args = (n, h, w, cin, cout, 3, 3, s, 1, c2d._ACTS[act], 0, c2d.DTYPE_BF16)
    assert c2d.plan_maxpool(*args).startswith("stem3x3_mfma" if kind == "stem" else "halo3x3_nhwc")
    y = _fused(x, spec, "nhwc")
    y2 = _two_calls(x, spec, "nhwc")
    torch.cuda.synchronize()
    assert bits_equal(y, y2), "fused and two-call results differ"
    got, ref = to64(y), _oracle(x, spec, "nhwc")
    assert not np.isnan(got).any()
    assert np.isneginf(ref).any(), "the case should hold an all-NaN window"
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    gate(got[fin], ref[fin], "bf16", what=str(case))


# ReLU on the halo kernel pools in 16-bit integer order: NaN inputs (ReLU maps NaN to 0,
# as the oracle does) and exact zeros (all-negative windows) must give the bits of the
# two-call path. (n, h, w, cin, cout, dtype)
RELU_SPECIAL = [
    (1, 30, 40, 32, 64, "bf16"),
    (2, 17, 33, 16, 24, "f16"),
]


@pytest.mark.parametrize("case", RELU_SPECIAL, ids=lambda c: "-".join(map(str, c)))
def test_fused_relu_maxpool_nan_and_zero_windows(case):
    n, h, w, cin, cout, dtype = case
    x, spec, _ = wl.random_conv_case(zlib.crc32(repr(case).encode()), n=n, h=h, w=w, cin=cin, cout=cout, k=3,
                                     stride=1, pad=1, act="relu", layout="nhwc", dtype=dtype)
    x = x.clone()
    x[0, 2:9, 3:12, :] = float("nan")
    x[-1, h - 8:, : w // 2, :] = 0.0  # zero input: conv = bias there; bias < 0 -> a window of zeros
    spec.bias[: cout // 2] = -torch.abs(spec.bias[: cout // 2]) - 0.25
    args = (n, h, w, cin, cout, 3, 3, 1, 1, c2d.ACT_RELU, 0, DT[dtype])
    assert c2d.plan_maxpool(*args).startswith("halo3x3_nhwc")
    y = _fused(x, spec, "nhwc")
    y2 = _two_calls(x, spec, "nhwc")
    torch.cuda.synchronize()
    assert bits_equal(y, y2), "fused and two-call results differ"
    got, ref = to64(y), _oracle(x, spec, "nhwc")
    assert not np.isnan(got).any() and not np.isnan(ref).any()
    assert (ref == 0).any(), "the case should hold windows of zeros"
    gate(got, ref, dtype, what=str(case))
