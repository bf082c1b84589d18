"""Layers at the size limits (needs an MI355X): an input just under 2 GiB, at the top of
the channel-last kernel's 32-bit byte offsets, and one just over, which the planner sends
to the general kernel. Checked against the oracle on sampled outputs and every axis's
last element."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import gate, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")


def _weights(seed, cout, cin, k):
    rng = np.random.default_rng(seed)
    w = wl.to_storage(rng.standard_normal((cout, k, k, cin)) * np.sqrt(2.0 / (cin * k * k)), "bf16")
    b = torch.from_numpy(rng.uniform(-0.1, 0.1, cout).astype(np.float32))
    return w, b


def _sampled(x, w, b, y, stride, pad, act, count=3000):
    rng = np.random.default_rng(7)
    shape = tuple(y.shape)
    idx = np.stack([rng.integers(0, d, count) for d in shape], axis=1)
    tails = np.array([[d - 1 for d in shape]] + [[shape[j] - 1 if j == i else rng.integers(0, shape[j])
                                                  for j in range(4)] for i in range(4) for _ in range(32)])
    idx = np.concatenate([idx, tails])
    ref = oracle.conv2d_points(to64(x), to64(w), to64(b), None, None, idx, stride=stride, pad=pad, act=act)
    got = to64(y)[tuple(idx.T)]
    gate(got, ref, "bf16", what="limit layer")


@pytest.mark.parametrize("h,w,cin,cout,family", [
    (4094, 4096, 64, 32, "igemm_nhwc_pipe"),   # x = 2,146,435,072 bytes: just under 2 GiB
    (4096, 4096, 72, 16, "igemm_nhwc_vec"),    # x = 2,415,919,104 bytes: the general kernel
])
def test_conv_at_the_2gib_offset_limit(h, w, cin, cout, family):
    print(f"limit case {h}x{w}x{cin}->{cout}", flush=True)
    x = wl.large_map(13, 1, h, w, cin)
    wt, b = _weights(17, cout, cin, 3)
    plan = c2d.plan(1, h, w, cin, cout, 3, 3, 2, 1, c2d.ACT_RELU, c2d.LAYOUT_NHWC, c2d.DTYPE_BF16)
    assert plan.startswith(family), plan
    xd = x.to(DEV)
    y = c2d.conv2d_fused(xd, wt.to(DEV), b.to(DEV), stride=2, pad=1, act="relu")
    torch.cuda.synchronize()
    del xd
    _sampled(x, wt, b, y, 2, 1, "relu")
