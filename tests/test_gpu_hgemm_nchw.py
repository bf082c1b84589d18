"""The halo-tile GEMM on channel-first layers (the IFNet block's convs): the input copied
channel-last (or handed over by the previous conv of a stack), the output and the
residual written channel-first by the GEMM's own epilogue. Every variant that takes
channel-first outputs is forced through a tuned-plan record (family 3, tile 100 + the
variant) and gated against the oracle, in both tile orders, with channel-last weights
(CONV2D_WEIGHTS_OHWI) and with channel-first ones (copied per call). The shapes have
ragged tiles, images smaller than one tile, input-channel counts that leave the last K
chunk partial (240 = 7.5 chunks of 32, 40 = 1.25), output-channel counts that leave a
32-channel block half empty, every activation and both residual orders.
"""
import os
import tempfile

import pytest
import torch

import oracle
import workloads as wl
from parity import bits_equal, gate, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")

FAM_NCHW = 3
HG_TILE = 100                                  # tuned-plan tile of halo-tile GEMM variant v: HG_TILE + v
STRIDE = [1, 1, 1, 1, 1, 1, 2, 2, 2, 1, 1, 1, 2]  # the stride each variant computes
WAVE_SPECIALISED = (1, 2)                      # variants without channel-first outputs


@pytest.fixture(autouse=True)
def _clean_table():
    c2d.tune_clear()
    yield
    c2d.tune_clear()


def _device_key(n, h, w, cin, cout, dt, res, stride):
    """Table key of a 3x3 pad-1 channel-first shape on this device."""
    c2d.tune(1, 8, 8, 64, 64, 3, 3, 1, 1, "relu", dtype=c2d.DTYPE_BF16, reps=1)
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "t.txt")
        c2d.tune_save(p)
        line = [ln for ln in open(p) if not ln.startswith("#")][0]
    c2d.tune_clear()
    dev = line.split("|")[0]
    return f"{dev}|{n}|{h}|{w}|{cin}|{cout}|3|3|{stride}|1|{c2d.LAYOUT_NCHW}|{dt}|{res}"


# (n, h, w, cin, cout, stride, act, residual, res_before_act, dtype, weights_ohwi)
CASES = [
    (1, 19, 33, 240, 48, 1, "prelu", True, False, "f16", True),    # Cin 240: a half K chunk at the end
    (2, 9, 20, 40, 72, 1, "silu", False, False, "bf16", False),     # Cin 40; Cout 72: 8 channels in the third block
    (1, 17, 15, 128, 240, 1, "relu", True, True, "f16", True),      # one 17 x 15 tile; Cout 240: 7.5 blocks
    (1, 6, 7, 96, 32, 1, "none", False, False, "bf16", False),      # image smaller than a tile
    (1, 23, 19, 64, 40, 2, "relu", True, False, "f16", True),       # stride 2, odd sizes
    (2, 16, 26, 56, 64, 2, "prelu", False, False, "bf16", False),   # stride 2, even sizes, Cin 56
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_every_channel_first_variant_meets_the_gate(case, tmp_path):
    n, h, w, cin, cout, stride, act, residual, pre, dtype, ohwi = case
    dt = {"bf16": c2d.DTYPE_BF16, "f16": c2d.DTYPE_F16}[dtype]
    actc = c2d._ACTS[act] | (c2d.RES_BEFORE_ACT if pre else 0) | (c2d.WEIGHTS_OHWI if ohwi else 0)
    key0 = _device_key(n, h, w, cin, cout, dt, 0, stride)  # conv2d_plan looks up the record without residual
    key1 = key0[:-1] + "1"
    x, spec, r = wl.random_conv_case(311 + cin + h, n=n, h=h, w=w, cin=cin, cout=cout, k=3, stride=stride, pad=1,
                                     act=act, layout="nchw", dtype=dtype, residual=residual, res_before_act=pre)
    ref = oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias), to64(spec.alpha) if spec.alpha is not None else None,
                        to64(r) if r is not None else None, stride=stride, pad=1, act=act, layout="nchw",
                        res_before_act=pre)
    wd = (c2d.weights_to_ohwi(spec.w.to(DEV)) if ohwi else spec.w.to(DEV)).contiguous()
    xd, bd = x.to(DEV), spec.bias.to(DEV)
    ad = spec.alpha.to(DEV) if spec.alpha is not None else None
    rd = r.to(DEV) if r is not None else None
    ran = 0
    for v in range(len(STRIDE)):
        if STRIDE[v] != stride or v in WAVE_SPECIALISED:
            continue
        for order in (0, 1):
            table = tmp_path / f"v{v}_{order}.txt"
            table.write_text(f"{key0} {FAM_NCHW} {HG_TILE + v} 1 {order}\n{key1} {FAM_NCHW} {HG_TILE + v} 1 {order}\n")
            c2d.tune_clear()
            assert c2d.tune_load(str(table)) == 2
            name = c2d.plan(n, h, w, cin, cout, 3, 3, stride, 1, actc, c2d.LAYOUT_NCHW, dt)
            prefix = "x_to_nhwc+" if ohwi else "to_nhwc+"
            assert name.startswith(f"{prefix}hgemm3x3_nchw_out {dtype} v{v} ") and name.endswith(" tuned"), name
            assert ("cfast" if order else "pfast") in name, name
            print(f"variant {v} order {order}: {name}", flush=True)
            y = c2d.conv2d_fused(xd, wd, bd, ad, rd, stride=stride, pad=1, act=act, layout="nchw",
                                 res_before_act=pre, weights_ohwi=ohwi)
            torch.cuda.synchronize()
            gate(to64(y), ref, dtype, what=f"variant {v} order {order} ({name})")
            ran += 1
    assert ran >= 6


def test_default_plan_of_the_ifnet_conv():
    """68 x 120 x 240 -> 240 (the IFNet block's conv): the 17 x 15-pixel tiles, 256 of them."""
    f16 = c2d.DTYPE_F16
    name = c2d.plan(1, 68, 120, 240, 240, 3, 3, 1, 1, c2d.ACT_PRELU | c2d.WEIGHTS_OHWI, c2d.LAYOUT_NCHW, f16)
    assert name.startswith("x_to_nhwc+hgemm3x3_nchw_out f16 v9 17x15x32 "), name
    # narrow layers stay on the pipelined kernel
    name = c2d.plan(1, 68, 120, 64, 64, 3, 3, 1, 1, c2d.ACT_PRELU | c2d.WEIGHTS_OHWI, c2d.LAYOUT_NCHW, f16)
    assert name.startswith("x_to_nhwc+igemm_nhwc_pipe"), name


@pytest.mark.parametrize("forced", [None, 11], ids=["default", "pipelined-64x128d5"])
def test_ifnet_chain_on_either_kernel(forced, tmp_path):
    """Chained channel-first convs (channel-last weights): each producer writes the next
    conv's channel-last input copy from its epilogue. On the halo-tile GEMM (the default)
    and on the pipelined kernel (forced by a record), the stack gives the bits of one call
    per op, and both meet the gate against the oracle chain."""
    import numpy as np
    rng = np.random.default_rng(77)
    c, h, w, dtype = 240, 21, 34, "f16"
    dt = c2d.DTYPE_F16
    x = wl.to_storage(rng.standard_normal((1, c, h, w)).astype(np.float32), dtype).to(DEV)
    layers, ops, keep = [], [], []
    src = x
    for i in range(4):
        wt = wl.to_storage((rng.standard_normal((c, c, 3, 3)) / np.sqrt(9 * c)).astype(np.float32), dtype)
        b = torch.from_numpy(rng.uniform(-0.1, 0.1, c).astype(np.float32))
        al = torch.from_numpy(rng.uniform(0.05, 0.3, c).astype(np.float32))
        res = x if i == 3 else None
        y = torch.empty_like(x)
        wo = c2d.weights_to_ohwi(wt.to(DEV)).contiguous()
        keep += [wo, b.to(DEV), al.to(DEV), y]
        ops.append(c2d.conv_op(src, wo, y, keep[-3], keep[-2], residual=res, stride=1, pad=1, act="prelu",
                               layout="nchw", weights_ohwi=True))
        layers.append((wt, b, al, res is not None))
        src = y
    if forced is not None:
        key0 = _device_key(1, h, w, c, c, dt, 0, 1)
        key1 = key0[:-1] + "1"
        table = tmp_path / "t.txt"
        table.write_text(f"{key0} {FAM_NCHW} {forced} 1 0\n{key1} {FAM_NCHW} {forced} 1 0\n")
        assert c2d.tune_load(str(table)) == 2
    names = [c2d.stack_plan(ops, i, layout="nchw", dtype=dt) for i in range(4)]
    kernel = "hgemm3x3_nchw_out" if forced is None else "igemm_nhwc_pipe"
    assert all(kernel in nm for nm in names), names
    assert names[0].startswith("x_to_nhwc+") and " +y_nhwc" in names[0], names
    assert all(nm.startswith("chained+") for nm in names[1:]), names
    # one call per op (no chaining), then the stack
    want = []
    s = x
    for k, (wt, b, al, has_res) in enumerate(layers):
        yk = c2d.conv2d_fused(s, keep[4 * k], keep[4 * k + 1], keep[4 * k + 2], x if has_res else None, stride=1,
                              pad=1, act="prelu", layout="nchw", weights_ohwi=True)
        want.append(yk)
        s = yk
    torch.cuda.synchronize()
    c2d.stack_run(ops, layout="nchw", dtype=dt)
    torch.cuda.synchronize()
    for k in range(4):
        assert bits_equal(keep[4 * k + 3], want[k]), f"layer {k}"
    # the oracle chain, each intermediate map rounded to f16 as the GPU stores it
    x64 = to64(x)
    ref = x64
    for wt, b, al, has_res in layers:
        ref = oracle.conv2d(ref, to64(wt), to64(b), to64(al), x64 if has_res else None, stride=1, pad=1,
                            act="prelu", layout="nchw")
        if not has_res:
            ref = oracle.quantize(ref, dtype)
    gate(to64(keep[-1]), ref, dtype, what=f"chain ({names[0]})", elementwise=False)
