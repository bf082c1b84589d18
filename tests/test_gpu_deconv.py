"""GPU parity of conv_transpose4x4s2 against the CPU oracle (needs an MI355X).

The oracle evaluates the transposed conv of framecast's `wgslDeconv` in fp64 from the
same stored inputs; the gate is the conv gate of parity.py (an fp32 output from 16-bit
inputs takes the fp32 gate: only the accumulation order differs)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import bits_equal, gate, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
CODES = {"f32": c2d.DTYPE_F32, "bf16": c2d.DTYPE_BF16, "f16": c2d.DTYPE_F16}


def _run(x, w, bias, alpha, act, layout, out_dtype):
    return c2d.conv_transpose4x4s2(x.to(DEV), w.to(DEV), bias.to(DEV) if bias is not None else None,
                                   alpha.to(DEV) if alpha is not None else None, act=act, layout=layout,
                                   out_dtype=TD[out_dtype])


def _ref(x, w, bias, alpha, act, layout):
    return oracle.conv_transpose4x4s2(to64(x), to64(w), to64(bias) if bias is not None else None,
                                      to64(alpha) if alpha is not None else None, act=act, layout=layout)


# (n, h, w, cin, cout, act, layout, dtype, out_dtype, kernel)
CASES = [
    (1, 5, 7, 16, 8, "none", "nhwc", "bf16", "bf16", "mfma"),
    (2, 9, 37, 40, 33, "relu", "nhwc", "bf16", "bf16", "mfma"),      # ragged tile, 2 co blocks, K tail
    (1, 13, 70, 64, 64, "prelu", "nhwc", "f16", "f32", "mfma"),
    (1, 17, 30, 240, 5, "none", "nchw", "f16", "f32", "mfma"),       # IFNet deconv, reduced frame
    (2, 8, 8, 128, 96, "silu", "nchw", "bf16", "bf16", "mfma"),
    (3, 3, 33, 24, 40, "relu", "nchw", "f16", "f16", "mfma"),
    (1, 1, 1, 8, 4, "relu", "nhwc", "bf16", "bf16", "mfma"),         # 1x1 input
    (1, 2, 65, 8, 1, "silu", "nhwc", "f16", "f16", "mfma"),          # one output channel
    (1, 7, 40, 264, 40, "prelu", "nhwc", "bf16", "bf16", "mfma"),    # Cin > 256: chunked ring, K tail
    (1, 9, 35, 320, 33, "relu", "nchw", "f16", "f32", "mfma"),       # chunked, channel-first staging
    (3, 5, 21, 256, 8, "silu", "nchw", "bf16", "bf16", "mfma"),      # whole strip, channel-first copy
    # whole strip read from the planes (W % 8 == 0): ragged last tile column, partial
    # 64-channel chunk, two Cout blocks, several images, odd heights
    (2, 5, 40, 40, 33, "relu", "nchw", "bf16", "bf16", "mfma"),
    (1, 7, 16, 200, 5, "prelu", "nchw", "f16", "f32", "mfma"),
    (3, 4, 64, 8, 16, "silu", "nchw", "f16", "f16", "mfma"),
    (1, 3, 8, 256, 40, "none", "nchw", "bf16", "f32", "mfma"),
    # enough tiles for the two-row whole-strip tiles (the small cases above run one-row tiles)
    (2, 41, 256, 64, 24, "relu", "nchw", "f16", "f16", "mfma"),
    (1, 33, 200, 40, 40, "prelu", "nchw", "bf16", "f32", "mfma"),
    (1, 6, 9, 12, 7, "relu", "nhwc", "bf16", "bf16", "direct"),      # Cin % 8 != 0
    (1, 6, 9, 16, 7, "prelu", "nhwc", "f32", "f32", "direct"),
    (2, 5, 6, 10, 3, "silu", "nchw", "f32", "f32", "direct"),
    (1, 7, 5, 3, 9, "none", "nchw", "f16", "f32", "direct"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_deconv_parity(case):
    n, h, w, cin, cout, act, layout, dt, odt, kern = case
    x, wt, b, al = wl.random_deconv_case(11 + n * h + w + cin, n=n, h=h, w=w, cin=cin, cout=cout, act=act,
                                         layout=layout, dtype=dt)
    plan = c2d.plan_deconv(n, h, w, cin, cout, c2d._ACTS[act], c2d._LAYOUTS[layout], CODES[dt], CODES[odt])
    assert ("mfma" in plan) == (kern == "mfma"), plan
    y = _run(x, wt, b, al, act, layout, odt)
    torch.cuda.synchronize()
    want = (n, 2 * h, 2 * w, cout) if layout == "nhwc" else (n, cout, 2 * h, 2 * w)
    assert tuple(y.shape) == want and y.dtype == TD[odt]
    gate(to64(y), _ref(x, wt, b, al, act, layout), odt, what=f"{case} {plan}")


def test_deconv_ifnet_full_size():
    """The IFNet block-0 deconv at a 1920x1088 frame: [1,240,68,120] f16 -> [1,5,136,240] fp32."""
    x, wt, b, al = wl.ifnet_deconv()
    y = _run(x, wt, b, al, "none", "nchw", "f32")
    torch.cuda.synchronize()
    gate(to64(y), _ref(x, wt, b, al, "none", "nchw"), "f32", what="ifnet deconv")


def test_deconv_decoder_full_size():
    """A decoder-sized layer: [1,64,64,256] -> [1,128,128,128] bf16 NHWC, ReLU."""
    x, wt, b, al = wl.random_deconv_case(21, n=1, h=64, w=64, cin=256, cout=128, act="relu", layout="nhwc",
                                         dtype="bf16")
    y = _run(x, wt, b, al, "relu", "nhwc", "bf16")
    torch.cuda.synchronize()
    gate(to64(y), _ref(x, wt, b, al, "relu", "nhwc"), "bf16", what="decoder deconv")


def test_deconv_layouts_agree():
    """Channel-first and channel-last calls on the same data give the same values."""
    x, wt, b, al = wl.random_deconv_case(5, n=2, h=11, w=19, cin=32, cout=24, act="prelu", layout="nhwc",
                                         dtype="bf16")
    y1 = _run(x, wt, b, al, "prelu", "nhwc", "f32")
    y2 = _run(x.permute(0, 3, 1, 2).contiguous(), wt, b, al, "prelu", "nchw", "f32")
    torch.cuda.synchronize()
    assert torch.allclose(y1.permute(0, 3, 1, 2), y2, rtol=0, atol=1e-5)


def test_deconv_in_stack_matches_single_call():
    x, wt, b, al = wl.random_deconv_case(9, n=1, h=12, w=40, cin=64, cout=32, act="relu", layout="nhwc",
                                         dtype="f16")
    xd, wd, bd = x.to(DEV), wt.to(DEV), b.to(DEV)
    y1 = c2d.conv_transpose4x4s2(xd, wd, bd, act="relu", layout="nhwc")
    y2 = torch.empty_like(y1)
    c2d.stack_run([c2d.deconv_op(xd, wd, y2, bd, act="relu")], layout="nhwc", dtype=c2d.DTYPE_F16)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_deconv_rejects_bad_arguments():
    x = torch.zeros(1, 4, 4, 8, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(8, 8, 4, 4, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(c2d.Conv2dError):
        c2d.conv_transpose4x4s2(x, w, act="prelu")  # PReLU without slopes
    with pytest.raises(c2d.Conv2dError):
        c2d.conv_transpose4x4s2(x, w, out_dtype=torch.float16)  # neither x's dtype nor fp32


@pytest.mark.parametrize("layout,dt,odt,n,h,w,cin,cout", [
    ("nhwc", "bf16", "bf16", 1, 16, 40, 256, 128),
    ("nhwc", "f16", "f32", 2, 9, 37, 40, 33),
    ("nchw", "f16", "f32", 1, 17, 30, 240, 5),
    ("nchw", "bf16", "bf16", 1, 7, 40, 264, 40),
])
def test_prepacked_weights_give_identical_results(layout, dt, odt, n, h, w, cin, cout):
    """Packing once and calling the pre-packed entry point gives the bit-identical output
    of the per-call-pack entry point (same kernels, same packed operands)."""
    x, wt, b, _ = wl.random_deconv_case(91 + cin, n=n, h=h, w=w, cin=cin, cout=cout, act="relu", layout=layout,
                                        dtype=dt)
    xd, wd, bd = x.to(DEV), wt.to(DEV), b.to(DEV)
    packed = c2d.deconv_pack(wd)
    y1 = c2d.conv_transpose4x4s2(xd, wd, bd, act="relu", layout=layout, out_dtype=TD[odt])
    y2 = c2d.conv_transpose4x4s2_prepacked(xd, packed, bd, act="relu", layout=layout, out_dtype=TD[odt])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_channel_first_input_not_16_byte_aligned():
    """A channel-first input whose width allows reading the planes directly but whose
    pointer is not 16-byte aligned takes the channel-last copy instead; both give the
    oracle's result."""
    n, h, w, cin, cout = 1, 6, 16, 40, 24
    x, wt, b, al = wl.random_deconv_case(77, n=n, h=h, w=w, cin=cin, cout=cout, act="relu", layout="nchw",
                                         dtype="f16")
    big = torch.empty(x.numel() + 1, dtype=x.dtype, device=DEV)
    xs = big[1:].view(x.shape)  # 2 bytes past a 16-byte boundary
    xs.copy_(x.to(DEV))
    assert xs.data_ptr() % 16 != 0
    y = c2d.conv_transpose4x4s2(xs, wt.to(DEV), b.to(DEV), act="relu", layout="nchw")
    ya = _run(x, wt, b, al, "relu", "nchw", "f16")
    torch.cuda.synchronize()
    assert bits_equal(y, ya)
    gate(to64(y), _ref(x, wt, b, al, "relu", "nchw"), "f16", what="unaligned channel-first input")
