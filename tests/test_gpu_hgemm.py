"""Every variant of the halo-tile GEMM kernel (wide 3x3 stride-1 and stride-2 channel-last
layers) against the oracle, in both tile orders.

Each variant is forced through a tuned-plan table record (the text format that
conv2d_tune_save writes). The shapes have ragged tiles on both image edges, images
smaller than one tile, output-channel counts that leave a channel tile or a 32-channel
block partly or wholly empty, odd and even numbers of K chunks, all three activations
and both residual orders, in bf16 and f16 (input-channel counts that leave the last K
chunk partial are taken by the channel-first form only: test_gpu_hgemm_nchw.py).
"""
import os
import tempfile

import pytest
import torch

import oracle
import workloads as wl
from parity import gate, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")

FAM_HGEMM = 7
CK = [32, 64, 64, 32, 32, 32, 32, 32, 32, 32, 32, 32, 32]  # input channels per K chunk of each variant
STRIDE = [1, 1, 1, 1, 1, 1, 2, 2, 2, 1, 1, 1, 2]  # the stride each variant computes
NVARIANTS = len(CK)


def _takes(v, cin, stride):
    return STRIDE[v] == stride and cin % CK[v] == 0


@pytest.fixture(autouse=True)
def _clean_table():
    c2d.tune_clear()
    yield
    c2d.tune_clear()


def _device_key(n, h, w, cin, cout, dt, res, stride=1):
    """Table key of a 3x3 pad-1 channel-last shape on this device: the tuner writes one
    for a small shape, whose device part is reused."""
    c2d.tune(1, 8, 8, 64, 64, 3, 3, 1, 1, "relu", dtype=c2d.DTYPE_BF16, reps=1)
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "t.txt")
        c2d.tune_save(p)
        line = [ln for ln in open(p) if not ln.startswith("#")][0]
    c2d.tune_clear()
    dev = line.split("|")[0]
    return f"{dev}|{n}|{h}|{w}|{cin}|{cout}|3|3|{stride}|1|0|{dt}|{res}"


# (n, h, w, cin, cout, act, residual, res_before_act, dtype)
CASES = [
    (1, 13, 11, 64, 96, "relu", True, False, "bf16"),    # ragged tiles; Cout 96: a half-empty 64-channel tile
    (2, 9, 20, 96, 40, "silu", False, False, "f16"),     # 3 K chunks of 32; Cout 40: 8 channels in the second block
    (1, 17, 18, 128, 64, "prelu", True, True, "bf16"),   # residual before the activation
    (1, 6, 7, 256, 32, "relu", False, False, "bf16"),    # image smaller than a tile, 8 K chunks
    (1, 21, 12, 64, 136, "none", False, False, "f16"),   # Cout 136: five 32-channel blocks, the last one with 8
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_every_variant_meets_the_gate(case, tmp_path):
    n, h, w, cin, cout, act, residual, pre, dtype = case
    dt = {"bf16": c2d.DTYPE_BF16, "f16": c2d.DTYPE_F16}[dtype]
    actc = c2d._ACTS[act] | (c2d.RES_BEFORE_ACT if pre else 0)
    key0 = _device_key(n, h, w, cin, cout, dt, 0)  # conv2d_plan looks up the record without residual
    key1 = key0[:-1] + "1"
    x, spec, r = wl.random_conv_case(71 + cin + h, n=n, h=h, w=w, cin=cin, cout=cout, k=3, stride=1, pad=1,
                                     act=act, layout="nhwc", dtype=dtype, residual=residual, res_before_act=pre)
    ref = oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias), to64(spec.alpha) if spec.alpha is not None else None,
                        to64(r) if r is not None else None, stride=1, pad=1, act=act, layout="nhwc",
                        res_before_act=pre)
    xd, wd, bd = x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV)
    ad = spec.alpha.to(DEV) if spec.alpha is not None else None
    rd = r.to(DEV) if r is not None else None
    ran = 0
    for v in range(NVARIANTS):
        if not _takes(v, cin, 1):
            continue
        for order in (0, 1):
            table = tmp_path / f"v{v}_{order}.txt"
            table.write_text(f"{key0} {FAM_HGEMM} {v} 1 {order}\n{key1} {FAM_HGEMM} {v} 1 {order}\n")
            c2d.tune_clear()
            assert c2d.tune_load(str(table)) == 2
            name = c2d.plan(n, h, w, cin, cout, 3, 3, 1, 1, actc, c2d.LAYOUT_NHWC, dt)
            kernel = "hgemmws3x3_nhwc" if v in (1, 2) else "hgemm3x3_nhwc"
            assert name.startswith(f"{kernel} {dtype} v{v} ") and name.endswith(" tuned"), name
            assert ("cfast" if order else "pfast") in name and f" ck{CK[v]} " in name, name
            print(f"variant {v} order {order}: {name}", flush=True)
            y = c2d.conv2d_fused(xd, wd, bd, ad, rd, stride=1, pad=1, act=act, layout="nhwc", res_before_act=pre)
            torch.cuda.synchronize()
            gate(to64(y), ref, dtype, what=f"variant {v} order {order} ({name})")
            ran += 1
    assert ran >= 2


def test_default_plan_of_wide_layers():
    bf = c2d.DTYPE_BF16
    plan = lambda n, h, w, c: c2d.plan(n, h, w, c, c, 3, 3, 1, 1, c2d.ACT_RELU, c2d.LAYOUT_NHWC, bf)
    assert plan(4, 40, 40, 256).startswith("hgemm3x3_nhwc bf16 v0 ")
    assert plan(4, 20, 20, 512).startswith("hgemmws3x3_nhwc bf16 v1 ")
    assert plan(4, 80, 80, 128).startswith("hgemm3x3_nhwc bf16 v4 ")
    assert plan(4, 40, 40, 128).startswith("igemm_nhwc_pipe")


def test_delta_kernel_is_identity_bit_exact():
    """w[co, ky, kx, ci] = [co == ci][ky == kx == 1], no bias: y == x bit for bit (one
    product of 1.0 per output, every other term an exact zero)."""
    n, h, w, c = 2, 23, 17, 128
    g = torch.Generator().manual_seed(5)
    x = torch.randn(n, h, w, c, generator=g).to(torch.bfloat16)
    wt = torch.zeros(c, 3, 3, c, dtype=torch.bfloat16)
    wt[torch.arange(c), 1, 1, torch.arange(c)] = 1.0
    for v in range(NVARIANTS):
        if STRIDE[v] != 1:
            continue
        key = _device_key(n, h, w, c, c, c2d.DTYPE_BF16, 0)
        with tempfile.TemporaryDirectory() as d:
            p = os.path.join(d, "t.txt")
            open(p, "w").write(f"{key} {FAM_HGEMM} {v} 1 {v % 2}\n")
            c2d.tune_clear()
            assert c2d.tune_load(p) == 1
        y = c2d.conv2d_fused(x.to(DEV), wt.to(DEV), None, None, None, stride=1, pad=1, act="none", layout="nhwc")
        torch.cuda.synchronize()
        assert torch.equal(y.cpu().view(torch.int16), x.view(torch.int16)), f"variant {v}"


# Stride 2 (the downsampling convs): odd and even input sizes (the last output row and
# column read one padding pixel or not), ragged tiles, images smaller than one tile,
# partial channel blocks, every epilogue.
# (n, h, w, cin, cout, act, residual, res_before_act, dtype)
CASES_S2 = [
    (1, 23, 19, 64, 128, "relu", True, True, "bf16"),
    (2, 16, 26, 32, 72, "silu", False, False, "f16"),
    (1, 9, 7, 128, 64, "prelu", True, False, "bf16"),
    (1, 41, 40, 96, 40, "none", False, False, "bf16"),
]


@pytest.mark.parametrize("case", CASES_S2, ids=lambda c: "-".join(map(str, c)))
def test_stride2_variants_meet_the_gate(case, tmp_path):
    n, h, w, cin, cout, act, residual, pre, dtype = case
    dt = {"bf16": c2d.DTYPE_BF16, "f16": c2d.DTYPE_F16}[dtype]
    actc = c2d._ACTS[act] | (c2d.RES_BEFORE_ACT if pre else 0)
    key0 = _device_key(n, h, w, cin, cout, dt, 0, stride=2)
    key1 = key0[:-1] + "1"
    x, spec, r = wl.random_conv_case(171 + cin + h, n=n, h=h, w=w, cin=cin, cout=cout, k=3, stride=2, pad=1,
                                     act=act, layout="nhwc", dtype=dtype, residual=residual, res_before_act=pre)
    ref = oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias), to64(spec.alpha) if spec.alpha is not None else None,
                        to64(r) if r is not None else None, stride=2, pad=1, act=act, layout="nhwc",
                        res_before_act=pre)
    xd, wd, bd = x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV)
    ad = spec.alpha.to(DEV) if spec.alpha is not None else None
    rd = r.to(DEV) if r is not None else None
    ran = 0
    for v in range(NVARIANTS):
        if not _takes(v, cin, 2):
            continue
        for order in (0, 1):
            table = tmp_path / f"v{v}_{order}.txt"
            table.write_text(f"{key0} {FAM_HGEMM} {v} 1 {order}\n{key1} {FAM_HGEMM} {v} 1 {order}\n")
            c2d.tune_clear()
            assert c2d.tune_load(str(table)) == 2
            name = c2d.plan(n, h, w, cin, cout, 3, 3, 2, 1, actc, c2d.LAYOUT_NHWC, dt)
            assert name.startswith(f"hgemm3x3_nhwc {dtype} v{v} ") and name.endswith(" tuned"), name
            print(f"variant {v} order {order}: {name}", flush=True)
            y = c2d.conv2d_fused(xd, wd, bd, ad, rd, stride=2, pad=1, act=act, layout="nhwc", res_before_act=pre)
            torch.cuda.synchronize()
            gate(to64(y), ref, dtype, what=f"variant {v} order {order} ({name})")
            ran += 1
    assert ran >= 4
