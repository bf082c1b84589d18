"""GPU parity of conv2d_avgpool2x2_conv1x1 (the ResNet-D shortcut in one call) against the
oracle: the 1x1 conv of the exact 2x2 average (fp64, no intermediate rounding, which the
fused call does not perform either)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import gate, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")


def _avg64(x, layout):
    """fp64 2x2 stride-2 mean (an odd last row or column dropped)."""
    x = to64(x)
    if layout == "nchw":
        x = x.transpose(0, 2, 3, 1)
    n, h, w, c = x.shape
    h2, w2 = h // 2, w // 2
    a = x[:, :2 * h2, :2 * w2].reshape(n, h2, 2, w2, 2, c).mean(axis=(2, 4))
    return np.ascontiguousarray(a.transpose(0, 3, 1, 2) if layout == "nchw" else a)


# (n, h, w, cin, cout, act, layout, dtype)
CASES = [
    (4, 20, 20, 64, 128, "none", "nhwc", "bf16"),
    (2, 21, 19, 128, 96, "relu", "nhwc", "bf16"),    # odd sizes: last row and column dropped
    (1, 14, 30, 40, 24, "prelu", "nhwc", "f16"),     # Cin % 64 != 0
    (2, 18, 12, 64, 40, "silu", "nchw", "f16"),      # channel-first via channel-last copies
    (1, 10, 13, 12, 20, "relu", "nhwc", "f32"),      # general kernel
    (2, 9, 9, 3, 16, "none", "nchw", "bf16"),        # few input channels: direct kernel
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_avgpool_conv1x1_parity(case):
    n, h, w, cin, cout, act, layout, dt = case
    x, spec, _ = wl.random_conv_case(51 + h + cin, n=n, h=h, w=w, cin=cin, cout=cout, k=1, stride=1, pad=0, act=act,
                                     layout=layout, dtype=dt)
    y = c2d.avgpool2x2_conv1x1(x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV),
                               spec.alpha.to(DEV) if spec.alpha is not None else None, act=act, layout=layout)
    torch.cuda.synchronize()
    ref = oracle.conv2d(_avg64(x, layout), to64(spec.w), to64(spec.bias),
                        to64(spec.alpha) if spec.alpha is not None else None, None, stride=1, pad=0, act=act,
                        layout=layout)
    assert tuple(y.shape) == ref.shape
    gate(to64(y), ref, dt, what=str(case))


@pytest.mark.parametrize("hw,cin,cout", [(160, 64, 128), (80, 128, 256), (40, 256, 512)])
def test_resnet_d_shortcuts_full_size(hw, cin, cout):
    """The backbone's three downsampling shortcuts at N=4, 640x640 input (bf16, NHWC)."""
    x, spec, _ = wl.random_conv_case(61 + cin, n=4, h=hw, w=hw, cin=cin, cout=cout, k=1, stride=1, pad=0,
                                     act="none", layout="nhwc", dtype="bf16")
    y = c2d.avgpool2x2_conv1x1(x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.conv2d(_avg64(x, "nhwc"), to64(spec.w), to64(spec.bias), None, None, stride=1, pad=0, act="none")
    gate(to64(y), ref, "bf16", what=f"shortcut {hw} {cin}->{cout}")


def test_fused_equals_two_calls_within_one_rounding():
    """Against avgpool2x2 then conv2d_fused: the same up to the pooled map's rounding."""
    x, spec, _ = wl.random_conv_case(71, n=2, h=32, w=32, cin=64, cout=64, k=1, stride=1, pad=0, act="none",
                                     layout="nhwc", dtype="bf16")
    xd, wd, bd = x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV)
    fused = c2d.avgpool2x2_conv1x1(xd, wd, bd)
    two = c2d.conv2d_fused(c2d.avgpool2x2(xd), wd, bd)
    torch.cuda.synchronize()
    gate(to64(fused), to64(two), "bf16", what="fused vs two calls")


def test_in_stack_and_graph():
    x, spec, _ = wl.random_conv_case(81, n=1, h=24, w=40, cin=64, cout=128, k=1, stride=1, pad=0, act="relu",
                                     layout="nhwc", dtype="bf16")
    xd, wd, bd = x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV)
    y1 = c2d.avgpool2x2_conv1x1(xd, wd, bd, act="relu")
    y2 = torch.empty_like(y1)
    ops = [c2d.pool_conv_op(xd, wd, y2, bd, act="relu")]
    c2d.stack_run(ops)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    g = c2d.StackGraph(ops)
    for _ in range(3):
        y2.zero_()
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
    g.close()
