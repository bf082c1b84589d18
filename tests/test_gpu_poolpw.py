"""The ResNet-D shortcut (2x2 average pool, then a 1x1 conv of the pooled map) in a
stack runs as one kernel: both outputs equal a pool call followed by a conv call bit for
bit, and the conv output meets the oracle's gate (needs an MI355X)."""
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
DT = {"bf16": c2d.DTYPE_BF16, "f16": c2d.DTYPE_F16}

# (n, h, w, cin, cout, act, dtype): the three ResNet-18-D shortcut shapes at batch 4, odd
# input sizes (the pool drops the last row and column), a partial 128-channel tile, a
# pixel count that leaves the last pixel tile ragged, and every epilogue
CASES = [
    (4, 160, 160, 64, 128, "none", "bf16"),
    (4, 80, 80, 128, 256, "none", "bf16"),
    (4, 40, 40, 256, 512, "none", "bf16"),
    (1, 9, 13, 256, 72, "relu", "bf16"),
    (2, 22, 30, 128, 136, "silu", "f16"),
    (1, 7, 5, 64, 8, "prelu", "bf16"),
    (3, 10, 14, 64, 256, "none", "f16"),
]


def _case(case):
    n, h, w, cin, cout, act, dtype = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    x = wl.to_storage(rng.standard_normal((n, h, w, cin)).astype(np.float32), dtype)
    _, spec, _ = wl.random_conv_case(zlib.crc32(repr(case).encode()) + 1, n=1, h=1, w=1, cin=cin, cout=cout, k=1,
                                     stride=1, pad=0, act=act, layout="nhwc", dtype=dtype)
    return x, spec


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_pool_then_pointwise_in_one_kernel(case):
    n, h, w, cin, cout, act, dtype = case
    x, spec = _case(case)
    xd, wd, bd = x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV)
    ad = spec.alpha.to(DEV) if spec.alpha is not None else None
    ph, pw = h // 2, w // 2
    p = torch.full((n, ph, pw, cin), float("nan"), dtype=x.dtype, device=DEV)
    y = torch.full((n, ph, pw, cout), float("nan"), dtype=x.dtype, device=DEV)
    ops = [c2d.pool_op("avg", xd, p), c2d.conv_op(p, wd, y, bd, ad, stride=1, pad=0, act=act)]
    names = [c2d.stack_plan(ops, i, dtype=DT[dtype]) for i in range(2)]
    print(case, names, flush=True)
    assert names[0].startswith("avgpool2x2 (in the next op"), names
    assert names[1].startswith("avgpool2x2+conv1x1_nhwc"), names
    c2d.stack_run(ops, dtype=DT[dtype])
    p2 = c2d.avgpool2x2(xd)
    y2 = c2d.conv2d_fused(p2, wd, bd, ad, stride=1, pad=0, act=act)
    torch.cuda.synchronize()
    assert bits_equal(p, p2), "pooled map"
    assert bits_equal(y, y2), "conv output"
    pool_ref = oracle.avgpool2x2(to64(x))
    ref = oracle.conv2d(oracle.quantize(pool_ref, dtype), to64(spec.w), to64(spec.bias),
                        to64(spec.alpha) if spec.alpha is not None else None, None, stride=1, pad=0, act=act)
    gate(to64(y), ref, dtype, what=str(case))


def test_no_fusion_with_a_residual_or_a_second_reader():
    """A residual on the conv keeps the two launches; so does a pool whose output is not
    the next op's input."""
    x, spec = _case((1, 8, 8, 64, 64, "none", "bf16"))
    xd, wd = x.to(DEV), spec.w.to(DEV)
    p = torch.empty(1, 4, 4, 64, dtype=x.dtype, device=DEV)
    y = torch.empty(1, 4, 4, 64, dtype=x.dtype, device=DEV)
    r = torch.zeros_like(y)
    ops = [c2d.pool_op("avg", xd, p), c2d.conv_op(p, wd, y, None, None, r, stride=1, pad=0)]
    assert c2d.stack_plan(ops, 0) == "avgpool2x2" and not c2d.stack_plan(ops, 1).startswith("avgpool")
    other = torch.empty_like(p)
    ops = [c2d.pool_op("avg", xd, p), c2d.conv_op(other, wd, y, None, None, stride=1, pad=0)]
    assert c2d.stack_plan(ops, 0) == "avgpool2x2"
