"""The stem conv pair of a stack (CONV2D_Y_TRANSIENT on the first conv): a 3-channel
stride-2 stem conv and the stride-1 3x3 conv of its output in one kernel that never
stores the first output. The second output must equal the two launches bit for bit (the
same roundings, the same order of products), meet the gate against the oracle chain, and
leave the first conv's marked output untouched."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import bits_equal, gate, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")


def _layer(seed, cin, cout, act, dtype):
    _, spec, _ = wl.random_conv_case(seed, n=1, h=3, w=3, cin=cin, cout=cout, k=3, stride=1, pad=1, act=act,
                                     layout="nhwc", dtype=dtype)
    return spec.w.to(DEV), spec.bias.to(DEV), spec.alpha.to(DEV) if spec.alpha is not None else None


def _pair(n, h, w, cout2, act1, act2, dtype, seed):
    rng = np.random.default_rng(seed)
    x = wl.to_storage(rng.uniform(0, 1, (n, h, w, 3)).astype(np.float32), dtype).to(DEV)
    w1, b1, a1 = _layer(seed + 1, 3, 32, act1, dtype)
    w2, b2, a2 = _layer(seed + 2, 32, cout2, act2, dtype)
    oh, ow = (h - 1) // 2 + 1, (w - 1) // 2 + 1
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    s1 = torch.full((n, oh, ow, 32), 3.0, dtype=tdt, device=DEV)
    y = torch.full((n, oh, ow, cout2), 7.0, dtype=tdt, device=DEV)

    def ops(transient):
        return [c2d.conv_op(x, w1, s1, b1, a1, stride=2, pad=1, act=act1, transient=transient),
                c2d.conv_op(s1, w2, y, b2, a2, stride=1, pad=1, act=act2)]
    return x, (w1, b1, a1), (w2, b2, a2), s1, y, ops


# (n, h, w, cout2, act1, act2, dtype): the backbone's stem pair, ragged tiles on both edges
# (a 36 x 44 map in 8 x 32 tiles), a map narrower than one tile, fewer output channels
CASES = [
    (1, 64, 64, 32, "relu", "relu", "bf16"),
    (2, 72, 88, 32, "silu", "prelu", "f16"),
    (1, 40, 16, 16, "prelu", "none", "bf16"),
    (3, 50, 96, 24, "relu", "silu", "f16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_pair_equals_two_launches_and_meets_the_gate(case):
    n, h, w, cout2, act1, act2, dtype = case
    dt = c2d.DTYPE_BF16 if dtype == "bf16" else c2d.DTYPE_F16
    x, L1, L2, s1, y, ops = _pair(n, h, w, cout2, act1, act2, dtype, 500 + h)
    fused = ops(True)
    plans = [c2d.stack_plan(fused, i, dtype=dt) for i in range(2)]
    print("plans", plans, flush=True)
    assert "pair" in plans[1] and "not stored" in plans[0], plans
    c2d.stack_run(fused, dtype=dt)
    torch.cuda.synchronize()
    got = y.clone()
    assert bool((s1 == 3.0).all()), "the transient output was written"
    c2d.stack_run(ops(False), dtype=dt)  # the two launches
    torch.cuda.synchronize()
    assert bits_equal(got, y), "pair differs from the two launches"
    v1 = oracle.quantize(oracle.conv2d(to64(x), to64(L1[0]), to64(L1[1]), to64(L1[2]) if L1[2] is not None else None,
                                       None, stride=2, pad=1, act=act1), dtype)
    ref = oracle.conv2d(v1, to64(L2[0]), to64(L2[1]), to64(L2[2]) if L2[2] is not None else None, None, stride=1,
                        pad=1, act=act2)
    gate(to64(got), ref, dtype, what=f"stem pair {case}")


def test_pair_at_the_backbone_size_in_a_graph():
    """4 x 640 x 640 (the ResNet-D stem's first two convs), replayed from a captured graph:
    every replay equals the two launches."""
    x, L1, L2, s1, y, ops = _pair(4, 640, 640, 32, "relu", "relu", "bf16", 900)
    c2d.stack_run(ops(False))
    torch.cuda.synchronize()
    want = y.clone()
    y.fill_(0.0)
    g = c2d.StackGraph(ops(True))
    try:
        for rep in range(3):
            g.launch()
            torch.cuda.synchronize()
            assert bits_equal(y, want), f"replay {rep}"
            y.fill_(0.0)
            torch.cuda.synchronize()
    finally:
        g.close()


def test_marked_output_of_a_conv_without_a_partner_is_stored():
    """A transient mark on a conv that no pair takes (here the second conv has a
    residual) changes nothing: both convs run and store as usual."""
    x, L1, L2, s1, y, ops = _pair(1, 32, 32, 32, "relu", "relu", "bf16", 950)
    r = torch.ones_like(y)
    marked = [c2d.conv_op(x, L1[0], s1, L1[1], stride=2, pad=1, act="relu", transient=True),
              c2d.conv_op(s1, L2[0], y, L2[1], residual=r, stride=1, pad=1, act="relu")]
    assert "pair" not in c2d.stack_plan(marked, 1)
    c2d.stack_run(marked)
    torch.cuda.synchronize()
    want1 = c2d.conv2d_fused(x, L1[0], L1[1], stride=2, pad=1, act="relu")
    want2 = c2d.conv2d_fused(want1, L2[0], L2[1], residual=r, stride=1, pad=1, act="relu")
    torch.cuda.synchronize()
    assert bits_equal(s1, want1) and bits_equal(y, want2)
