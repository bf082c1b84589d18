"""GPU pools against the oracle, bit for bit (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import bits_equal, quantized_tensor, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")

SHAPES = [(1, 7, 9, 8), (2, 20, 17, 64), (1, 1, 1, 16), (3, 2, 3, 5), (1, 33, 31, 3),
          (2, 16, 16, 24), (1, 320, 320, 32)]


def _x(shape, layout, dtype, seed):
    n, h, w, c = shape
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, h, w, c) if layout == "nhwc" else (n, c, h, w))
    return wl.to_storage(a, dtype)


@pytest.mark.parametrize("layout", ["nhwc", "nchw"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_maxpool_bitexact(shape, layout, dtype):
    x = _x(shape, layout, dtype, 1)
    y = c2d.maxpool3x3s2(x.to(DEV), layout=layout)
    torch.cuda.synchronize()
    assert np.array_equal(to64(y), oracle.maxpool3x3s2(to64(x), layout=layout))


@pytest.mark.parametrize("layout", ["nhwc", "nchw"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [s for s in SHAPES if s[1] >= 2 and s[2] >= 2], ids=str)
def test_avgpool_bitexact(shape, layout, dtype):
    x = _x(shape, layout, dtype, 2)
    y = c2d.avgpool2x2(x.to(DEV), layout=layout)
    torch.cuda.synchronize()
    ref = oracle.quantize(oracle.avgpool2x2(to64(x), layout=layout).astype(np.float64), dtype)
    assert np.array_equal(to64(y), ref)


def test_avgpool_summation_order():
    """2^24, 1, 1, -2^24 in the pinned order gives 0 (another order gives 0.5)."""
    x = torch.tensor([16777216.0, 1.0, 1.0, -16777216.0], dtype=torch.float32).reshape(1, 1, 2, 2)
    y = c2d.avgpool2x2(x.to(DEV), layout="nchw")
    assert float(y.cpu()[0, 0, 0, 0]) == 0.0


def test_maxpool_all_negative_and_ramp():
    x = -torch.arange(1, 1 + 2 * 9 * 11, dtype=torch.float32).reshape(1, 9, 11, 2).to(torch.bfloat16)
    y = c2d.maxpool3x3s2(x.to(DEV), layout="nhwc")
    assert np.array_equal(to64(y), oracle.maxpool3x3s2(to64(x)))
    assert float(y.float().max()) < 0


@pytest.mark.parametrize("layout", ["nhwc", "nchw"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("c", [16, 5])
def test_maxpool_nan_zeros_and_inf_bitexact(layout, dtype, c):
    """NaN taps are skipped, an all-NaN window gives -inf, -inf taps never win over the
    rest, and of equal zeros (-0, +0) the first in row-major tap order is kept: the
    oracle's bits exactly (c = 16: the 16-byte kernel in channel-last layout; c = 5: the
    scalar one)."""
    n, h, w = 2, 13, 17
    rng = np.random.default_rng(31 + c)
    shape = (n, h, w, c) if layout == "nhwc" else (n, c, h, w)
    a = rng.standard_normal(shape)
    u = rng.random(shape)
    a[u < 0.25] = np.nan
    a[(u >= 0.25) & (u < 0.35)] = -0.0
    a[(u >= 0.35) & (u < 0.42)] = 0.0
    a[(u >= 0.42) & (u < 0.46)] = -np.inf
    a[(u >= 0.46) & (u < 0.60)] = -np.abs(a[(u >= 0.46) & (u < 0.60)])
    # a NaN block that covers whole pool windows (rows 4..8, columns 6..10 of image 0)
    if layout == "nhwc":
        a[0, 4:9, 6:11, :] = np.nan
    else:
        a[0, :, 4:9, 6:11] = np.nan
    x = wl.to_storage(a, dtype)
    y = c2d.maxpool3x3s2(x.to(DEV), layout=layout)
    torch.cuda.synchronize()
    ref = oracle.maxpool3x3s2(to64(x), layout=layout)
    assert not np.isnan(ref).any() and np.isneginf(ref).any()
    assert bits_equal(y, quantized_tensor(ref, dtype))
