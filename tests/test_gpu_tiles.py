"""Every tile of the channel-last matrix-core conv kernel against the oracle.

The built-in planner and the tuner only ever pick some tiles for a given shape, so
this test forces each one in turn through a tuned-plan table record (the same text
format conv2d_tune_save writes) and checks the conv gate on shapes with a ragged
pixel count, a partial output-channel block, both K orders (taps innermost when Cin
is a multiple of 64, channel runs across taps otherwise), an odd number of K steps
(the second K group of the two-group tiles then idles on the last one), split-K
and the channel-first output path.
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

FAM_NHWC, FAM_NCHW_VIA_NHWC = 2, 3
LAYOUT_NCHW = 1


@pytest.fixture(autouse=True)
def _clean_table():
    c2d.tune_clear()
    yield
    c2d.tune_clear()


def _tile_count(tmp_path, key):
    """Number of tiles: the table loader accepts tile indices below it and no others."""
    t = 0
    while True:
        p = tmp_path / f"probe{t}.txt"
        p.write_text(f"{key} {FAM_NHWC} {t} 1 0\n")
        try:
            c2d.tune_load(str(p))
        except c2d.Conv2dError:
            c2d.tune_clear()
            return t
        t += 1
        assert t < 64


def _device_key(n, h, w, cin, cout, k, stride, pad, layout, dt, res):
    """Table key of a shape on this device: the tuner writes it for one small shape, the
    device part (architecture and CU count) is reused."""
    c2d.tune(1, 8, 8, 64, 64, 3, 3, 1, 1, "relu", dtype=c2d.DTYPE_BF16, reps=1)
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "t.txt")
        c2d.tune_save(p)
        line = [ln for ln in open(p) if not ln.startswith("#")][0]
    c2d.tune_clear()
    dev = line.split("|")[0]
    return f"{dev}|{n}|{h}|{w}|{cin}|{cout}|{k}|{k}|{stride}|{pad}|{layout}|{dt}|{res}"


# (n, h, w, cin, cout, k, stride, pad, act, residual, layout, dtype, splits)
CASES = [
    (1, 13, 11, 128, 96, 3, 1, 1, "relu", True, "nhwc", "bf16", 1),   # taps innermost, 18 K steps, ragged M and N
    (2, 9, 7, 72, 40, 3, 2, 1, "silu", False, "nhwc", "f16", 1),      # channel runs across taps, 11 K steps
    (1, 10, 10, 256, 64, 3, 1, 1, "relu", False, "nhwc", "bf16", 3),  # split-K: 3 slices of 12 K steps
    (1, 9, 14, 64, 48, 3, 1, 1, "prelu", True, "nchw", "f16", 1),     # channel-first output, 9 K steps
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_every_tile_meets_the_gate(case, tmp_path):
    n, h, w, cin, cout, k, stride, pad, act, residual, layout, dtype, splits = case
    dt = {"bf16": c2d.DTYPE_BF16, "f16": c2d.DTYPE_F16}[dtype]
    lay = LAYOUT_NCHW if layout == "nchw" else 0
    fam = FAM_NCHW_VIA_NHWC if layout == "nchw" else FAM_NHWC
    key0 = _device_key(n, h, w, cin, cout, k, stride, pad, lay, dt, 0)
    key1 = key0[:-1] + "1"
    ntiles = _tile_count(tmp_path, key0)
    assert ntiles >= 17
    x, spec, r = wl.random_conv_case(53 + cin + h, n=n, h=h, w=w, cin=cin, cout=cout, k=k, stride=stride, pad=pad,
                                     act=act, layout=layout, dtype=dtype, residual=residual,
                                     res_before_act=False)
    ref = oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias), to64(spec.alpha) if spec.alpha is not None else None,
                        to64(r) if r is not None else None, stride=stride, pad=pad, act=act, layout=layout)
    xd, wd, bd = x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV)
    ad = spec.alpha.to(DEV) if spec.alpha is not None else None
    rd = r.to(DEV) if r is not None else None
    actc = c2d._ACTS[act]
    seen = set()
    for t in range(ntiles):
        table = tmp_path / f"tile{t}.txt"
        table.write_text(f"{key0} {fam} {t} {splits} 0\n{key1} {fam} {t} {splits} 0\n")
        c2d.tune_clear()
        assert c2d.tune_load(str(table)) == 2
        name = c2d.plan(n, h, w, cin, cout, k, k, stride, pad, actc, lay, dt)
        assert "igemm_nhwc" in name and name.endswith(" tuned") and f"splitk={splits}" in name, name
        seen.add(name)
        print(f"tile {t}: {name}", flush=True)
        y = c2d.conv2d_fused(xd, wd, bd, ad, rd, stride=stride, pad=pad, act=act, layout=layout)
        torch.cuda.synchronize()
        gate(to64(y), ref, dtype, what=f"tile {t} ({name})")
    assert len(seen) == ntiles
