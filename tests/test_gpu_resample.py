"""GPU upsample and concat against the oracle: bit-exact (pure copies; needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import bits_equal, quantized_tensor

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")


def _shape(n, h, w, c, layout):
    return (n, h, w, c) if layout == "nhwc" else (n, c, h, w)


def _as(ref64, dtype):
    return quantized_tensor(ref64, dtype)


# (n, h, w, ca, cb, layout, dtype): h, w are the small map's size for the upsampling calls
CASES = [
    (1, 5, 7, 16, 8, "nhwc", "bf16"),
    (2, 9, 13, 24, 40, "nhwc", "f16"),
    (1, 4, 6, 12, 4, "nhwc", "f32"),
    (2, 3, 5, 3, 5, "nhwc", "bf16"),     # channels not a 16-byte multiple: element kernel
    (1, 1, 1, 8, 8, "nhwc", "bf16"),
    (2, 6, 4, 5, 3, "nchw", "f16"),      # H*W = 24: 16-byte planes for the plain concat
    (1, 7, 9, 4, 6, "nchw", "bf16"),     # H*W = 63: element kernel
    (1, 8, 8, 2, 3, "nchw", "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_upsample(case):
    n, h, w, ca, _, layout, dt = case
    x = wl.random_map(1, _shape(n, h, w, ca, layout), dt)
    y = c2d.upsample_nearest2x(x.to(DEV), layout=layout)
    torch.cuda.synchronize()
    assert bits_equal(y, _as(oracle.upsample_nearest2x(x.double().numpy(), layout=layout), dt))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_concat(case):
    n, h, w, ca, cb, layout, dt = case
    a = wl.random_map(2, _shape(n, h, w, ca, layout), dt)
    b = wl.random_map(3, _shape(n, h, w, cb, layout), dt)
    y = c2d.concat_channels(a.to(DEV), b.to(DEV), layout=layout)
    torch.cuda.synchronize()
    want = oracle.concat_channels(a.double().numpy(), b.double().numpy(), layout=layout)
    assert bits_equal(y, _as(want, dt))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_upsample_concat(case):
    n, h, w, ca, cb, layout, dt = case
    a = wl.random_map(4, _shape(n, h, w, ca, layout), dt)
    b = wl.random_map(5, _shape(n, 2 * h, 2 * w, cb, layout), dt)
    y = c2d.upsample2x_concat(a.to(DEV), b.to(DEV), layout=layout)
    torch.cuda.synchronize()
    up = oracle.upsample_nearest2x(a.double().numpy(), layout=layout)
    want = oracle.concat_channels(up, b.double().numpy(), layout=layout)
    assert bits_equal(y, _as(want, dt))


@pytest.mark.parametrize("hw", [20, 40])
def test_ccfm_top_down_full_size(hw):
    """The neck's top-down steps at a 640x640 image, batch 4: the 256-channel lateral
    map at stride 32 (20x20) or 16 (40x40), upsampled and joined with the 256-channel
    backbone map of the next level: [4, 2hw, 2hw, 512] bf16."""
    a = wl.random_map(6, (4, hw, hw, 256), "bf16")
    b = wl.random_map(7, (4, 2 * hw, 2 * hw, 256), "bf16")
    ad, bd = a.to(DEV), b.to(DEV)
    fused = c2d.upsample2x_concat(ad, bd)
    two = c2d.concat_channels(c2d.upsample_nearest2x(ad), bd)
    torch.cuda.synchronize()
    up = oracle.upsample_nearest2x(a.double().numpy())
    want = _as(oracle.concat_channels(up, b.double().numpy()), "bf16")
    assert bits_equal(fused, want)
    assert bits_equal(two, want)


def test_resample_stack_and_graph():
    a = wl.random_map(8, (2, 10, 12, 32), "f16").to(DEV)
    b = wl.random_map(9, (2, 20, 24, 16), "f16").to(DEV)
    up = torch.empty(2, 20, 24, 32, dtype=torch.float16, device=DEV)
    cat = torch.empty(2, 20, 24, 48, dtype=torch.float16, device=DEV)
    fused = torch.empty_like(cat)
    ops = [c2d.upsample_op(a, up), c2d.concat_op(up, b, cat), c2d.concat_op(a, b, fused, up=True)]
    assert c2d.stack_check(ops, dtype=c2d.DTYPE_F16) == (0, -1)
    c2d.stack_run(ops, dtype=c2d.DTYPE_F16)
    torch.cuda.synchronize()
    assert torch.equal(cat, fused)
    assert torch.equal(cat, torch.cat([a.repeat_interleave(2, 1).repeat_interleave(2, 2), b], dim=3))
    g = c2d.StackGraph(ops, dtype=c2d.DTYPE_F16)
    for _ in range(3):
        cat.zero_()
        fused.zero_()
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(cat, fused) and torch.equal(fused[..., 32:], b)
    g.close()


def test_resample_rejects_bad_arguments():
    a = torch.zeros(1, 4, 4, 8, dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(1, 4, 4, 8, dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        c2d.concat_channels(a, b)  # dtype mismatch, caught by the binding
    buf = torch.zeros(64 + 256, dtype=torch.bfloat16, device=DEV)
    a2 = buf[:128].view(1, 4, 4, 8)
    with pytest.raises(c2d.Conv2dError):
        c2d.concat_channels(a2, a, out=buf[64:].view(1, 4, 4, 16))  # y overlaps a
