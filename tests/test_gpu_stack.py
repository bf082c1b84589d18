"""Stacks of layers through conv2d_stack_run and a captured graph (needs an MI355X):
the same bits as one call per op, and the oracle's chain within the end-to-end gate."""
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


def _layer(seed, cin, cout, k, stride, pad, act, layout, dtype):
    _, spec, _ = wl.random_conv_case(seed, n=1, h=k, w=k, cin=cin, cout=cout, k=k, stride=stride, pad=pad,
                                     act=act, layout=layout, dtype=dtype)
    return spec.w.to(DEV), spec.bias.to(DEV), spec.alpha.to(DEV) if spec.alpha is not None else None


def _ifnet_chain(layout="nchw", dtype="f16", c=240, h=17, w=30, ohwi=False):
    """The IFNet block: eight 3x3 convs with PReLU, the block input added to the last
    one's output; the input buffer is reused as a ping-pong buffer, so the block first
    copies it aside. ohwi: the ops take the weights converted to channel-last once."""
    rng = np.random.default_rng(7)
    x = wl.to_storage(rng.standard_normal((1, c, h, w) if layout == "nchw" else (1, h, w, c)).astype(np.float32),
                      dtype).to(DEV)
    x0 = x.clone()
    layers = [_layer(100 + i, c, c, 3, 1, 1, "prelu", layout, dtype) for i in range(8)]
    a, b, snap, out = (torch.empty_like(x) for _ in range(4))
    bufs = [x, a, b]
    ops = [c2d.copy_op(x, snap)]
    keep = []
    src = x
    for i, (wt, bs, al) in enumerate(layers):
        last = i == 7
        dst = out if last else bufs[(i + 1) % 3]
        wo = c2d.weights_to_ohwi(wt) if ohwi else wt
        keep.append(wo)
        ops.append(c2d.conv_op(src, wo, dst, bs, al, residual=snap if last else None, stride=1, pad=1,
                               act="prelu", layout=layout, weights_ohwi=ohwi))
        src = dst
    # the ops hold raw pointers: the buffers must outlive them
    return x, x0, layers, ops, out, (a, b, snap, keep)


def _ifnet_oracle(x0, layers, layout, dtype):
    v = to64(x0)
    for i, (wt, bs, al) in enumerate(layers):
        r = to64(x0) if i == 7 else None
        y = oracle.conv2d(v, to64(wt), to64(bs), to64(al), r, stride=1, pad=1, act="prelu", layout=layout)
        v = y if i == 7 else oracle.quantize(y, dtype)
    return v


def _ifnet_calls(x0, layers, layout):
    v = x0
    for i, (wt, bs, al) in enumerate(layers):
        v = c2d.conv2d_fused(v, wt, bs, al, residual=x0 if i == 7 else None, stride=1, pad=1, act="prelu",
                             layout=layout)
    return v


def test_ifnet_block_stack_matches_calls_and_oracle():
    x, x0, layers, ops, out, _keep = _ifnet_chain()
    c2d.stack_run(ops, layout="nchw", dtype=c2d.DTYPE_F16)
    torch.cuda.synchronize()
    assert not bits_equal(x, x0)  # the input buffer was a ping-pong buffer
    want = _ifnet_calls(x0, layers, "nchw")
    torch.cuda.synchronize()
    assert bits_equal(out, want)
    gate(to64(out), _ifnet_oracle(x0, layers, "nchw", "f16"), "f16", what="ifnet stack", elementwise=False)


def test_ifnet_block_graph_replays():
    x, x0, layers, ops, out, _keep = _ifnet_chain()
    g = c2d.StackGraph(ops, layout="nchw", dtype=c2d.DTYPE_F16)
    want = _ifnet_calls(x0, layers, "nchw")
    try:
        for rep in range(3):
            # eager work between replays: restore the block input, poison the output
            x.copy_(x0)
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.launch()
            torch.cuda.synchronize()
            assert bits_equal(out, want), f"replay {rep}"
    finally:
        g.close()


def test_ifnet_chain_with_channel_last_weights():
    """With channel-last weights the chained channel-first convs hand each other their
    input's channel-last copy (written by the producing conv's epilogue into alternating
    scratch halves) instead of copying it again: the same bits as one call per op, in a
    stack run and in every replay of its graph."""
    x, x0, layers, ops, out, _keep = _ifnet_chain(ohwi=True)
    names = [c2d.stack_plan(ops, i, layout="nchw", dtype=c2d.DTYPE_F16) for i in range(1, 9)]
    assert names[0].startswith("x_to_nhwc+") and names[0].endswith(" +y_nhwc"), names[0]
    assert all(n.startswith("chained+") and n.endswith(" +y_nhwc") for n in names[1:7]), names
    assert names[7].startswith("chained+") and not names[7].endswith(" +y_nhwc"), names[7]
    want = _ifnet_calls(x0, layers, "nchw")
    torch.cuda.synchronize()
    c2d.stack_run(ops, layout="nchw", dtype=c2d.DTYPE_F16)
    torch.cuda.synchronize()
    assert bits_equal(out, want)
    gate(to64(out), _ifnet_oracle(x0, layers, "nchw", "f16"), "f16", what="ifnet chain", elementwise=False)
    g = c2d.StackGraph(ops, layout="nchw", dtype=c2d.DTYPE_F16)
    try:
        for rep in range(3):
            x.copy_(x0)
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.launch()
            torch.cuda.synchronize()
            assert bits_equal(out, want), f"replay {rep}"
    finally:
        g.close()


def test_resnet_blocks_and_stem_stack():
    """The ResNet-D stem (three convs, the third with the max pool), a stage-1 block and
    the first conv of a stride-2 block with its average-pool shortcut."""
    rng = np.random.default_rng(11)
    x = wl.to_storage(rng.uniform(0, 1, (2, 96, 128, 3)).astype(np.float32), "bf16").to(DEV)
    L = [_layer(200, 3, 32, 3, 2, 1, "relu", "nhwc", "bf16"), _layer(201, 32, 32, 3, 1, 1, "relu", "nhwc", "bf16"),
         _layer(202, 32, 64, 3, 1, 1, "relu", "nhwc", "bf16"), _layer(203, 64, 64, 3, 1, 1, "relu", "nhwc", "bf16"),
         _layer(204, 64, 64, 3, 1, 1, "none", "nhwc", "bf16"), _layer(205, 64, 128, 3, 2, 1, "relu", "nhwc", "bf16"),
         _layer(206, 64, 128, 1, 1, 0, "none", "nhwc", "bf16")]
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=DEV)
    s1, s2, p = e(2, 48, 64, 32), e(2, 48, 64, 32), e(2, 24, 32, 64)
    t, blk, c1, ap, sc = e(2, 24, 32, 64), e(2, 24, 32, 64), e(2, 12, 16, 128), e(2, 12, 16, 64), e(2, 12, 16, 128)
    ops = [c2d.conv_op(x, L[0][0], s1, L[0][1], stride=2, pad=1, act="relu"),
           c2d.conv_op(s1, L[1][0], s2, L[1][1], stride=1, pad=1, act="relu"),
           c2d.conv_op(s2, L[2][0], p, L[2][1], stride=1, pad=1, act="relu", pool=True),
           c2d.conv_op(p, L[3][0], t, L[3][1], stride=1, pad=1, act="relu"),
           c2d.conv_op(t, L[4][0], blk, L[4][1], residual=p, stride=1, pad=1, act="relu", res_before_act=True),
           c2d.conv_op(blk, L[5][0], c1, L[5][1], stride=2, pad=1, act="relu"),
           c2d.pool_op("avg", blk, ap),
           c2d.conv_op(ap, L[6][0], sc, L[6][1], stride=1, pad=0, act="none")]
    plans = [c2d.stack_plan(ops, i) for i in range(len(ops))]
    print("plans", plans, flush=True)
    assert "fused with maxpool3x3s2" in plans[2]
    c2d.stack_run(ops)
    torch.cuda.synchronize()
    # one call per op on the same inputs
    y1 = c2d.conv2d_fused(x, L[0][0], L[0][1], stride=2, pad=1, act="relu")
    y2 = c2d.conv2d_fused(y1, L[1][0], L[1][1], stride=1, pad=1, act="relu")
    y3 = c2d.conv2d_fused_maxpool3x3s2(y2, L[2][0], L[2][1], stride=1, pad=1, act="relu")
    y4 = c2d.conv2d_fused(y3, L[3][0], L[3][1], stride=1, pad=1, act="relu")
    y5 = c2d.conv2d_fused(y4, L[4][0], L[4][1], residual=y3, stride=1, pad=1, act="relu", res_before_act=True)
    y6 = c2d.conv2d_fused(y5, L[5][0], L[5][1], stride=2, pad=1, act="relu")
    y7 = c2d.avgpool2x2(y5)
    y8 = c2d.conv2d_fused(y7, L[6][0], L[6][1], stride=1, pad=0, act="none")
    torch.cuda.synchronize()
    for got, want, name in ((p, y3, "stem"), (blk, y5, "block"), (c1, y6, "s2 conv"), (sc, y8, "shortcut")):
        assert bits_equal(got, want), name
    # each layer against the oracle on the GPU's own input to it
    ref = oracle.maxpool3x3s2(oracle.conv2d(to64(s2), to64(L[2][0]), to64(L[2][1]), None, None, stride=1, pad=1,
                                            act="relu"))
    gate(to64(p), ref, "bf16", what="stem3 + pool")
    ref = oracle.conv2d(to64(t), to64(L[4][0]), to64(L[4][1]), None, to64(p), stride=1, pad=1, act="relu",
                        res_before_act=True)
    gate(to64(blk), ref, "bf16", what="block conv2")


def test_invalid_op_launches_nothing():
    rng = np.random.default_rng(3)
    x = wl.to_storage(rng.standard_normal((1, 16, 16, 32)).astype(np.float32), "bf16").to(DEV)
    w0, b0, _ = _layer(300, 32, 32, 3, 1, 1, "relu", "nhwc", "bf16")
    y0 = torch.full((1, 16, 16, 32), 5.0, dtype=torch.bfloat16, device=DEV)
    y1 = torch.full((1, 16, 16, 32), 5.0, dtype=torch.bfloat16, device=DEV)
    good = c2d.conv_op(x, w0, y0, b0, stride=1, pad=1, act="relu")
    bad = c2d.conv_op(y0, w0, y1, b0, stride=3, pad=1, act="relu")  # stride 3
    bad.stride = 3
    with pytest.raises(c2d.Conv2dError) as e:
        c2d.stack_run([good, good, bad])
    assert e.value.code == c2d.EINVAL and "op 2" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(y0 == 5.0)
