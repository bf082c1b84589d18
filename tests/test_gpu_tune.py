"""The shape-keyed tuner on the GPU: the tuned variant is used by later calls, still
meets the conv gate against the oracle, and survives a save / clear / load round trip."""
import pytest
import torch

import oracle
import workloads as wl
from parity import gate, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")


@pytest.fixture(autouse=True)
def _clean_table():
    c2d.tune_clear()
    yield
    c2d.tune_clear()


def _parity(n, h, w, cin, cout, k, stride, pad, act, residual, dtype):
    x, spec, r = wl.random_conv_case(31 + h + cin, n=n, h=h, w=w, cin=cin, cout=cout, k=k, stride=stride, pad=pad,
                                     act=act, layout="nhwc", dtype=dtype, residual=residual,
                                     res_before_act=residual)
    y = c2d.conv2d_fused(x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV), None, r.to(DEV) if r is not None else None,
                         stride=stride, pad=pad, act=act, res_before_act=residual, layout="nhwc")
    torch.cuda.synchronize()
    ref = oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias), None, to64(r) if r is not None else None,
                        stride=stride, pad=pad, act=act, res_before_act=residual, layout="nhwc")
    gate(to64(y), ref, dtype, what=f"tuned {n}x{h}x{w}x{cin}->{cout}")


# (n, h, w, cin, cout, k, stride, pad, act, residual, dtype)
SHAPES = [
    (1, 20, 20, 256, 256, 3, 1, 1, "relu", True, "bf16"),    # ResNet stage-3-like, deep K
    (2, 17, 23, 128, 96, 3, 2, 1, "relu", False, "f16"),
    (1, 48, 40, 32, 64, 3, 1, 1, "relu", False, "bf16"),     # halo-kernel shape
    (4, 10, 10, 512, 256, 1, 1, 0, "relu", False, "bf16"),   # pointwise
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_tuned_plan_is_used_and_meets_the_gate(shape, tmp_path):
    n, h, w, cin, cout, k, stride, pad, act, residual, dtype = shape
    dt = {"bf16": c2d.DTYPE_BF16, "f16": c2d.DTYPE_F16}[dtype]
    actc = c2d._ACTS[act] | (c2d.RES_BEFORE_ACT if residual else 0)
    name, us = c2d.tune(n, h, w, cin, cout, k, k, stride, pad, act, residual=residual, res_before_act=residual,
                        dtype=dt, reps=5)
    assert name.endswith(" tuned") and us > 0, name
    if residual:
        # the table is keyed on the residual: the plan of the call without one is untouched
        assert not c2d.plan(n, h, w, cin, cout, k, k, stride, pad, c2d._ACTS[act], 0, dt).endswith("tuned")
    else:
        assert c2d.plan(n, h, w, cin, cout, k, k, stride, pad, actc, 0, dt) == name
    _parity(n, h, w, cin, cout, k, stride, pad, act, residual, dtype)
    path = tmp_path / "plans.txt"
    assert c2d.tune_save(str(path)) == 1
    c2d.tune_clear()
    assert c2d.tune_load(str(path)) == 1
    if not residual:
        assert c2d.plan(n, h, w, cin, cout, k, k, stride, pad, actc, 0, dt) == name


def test_untunable_shape_keeps_the_builtin_choice():
    name, us = c2d.tune(1, 32, 32, 16, 32, 3, 3, 1, 1, "relu", dtype=c2d.DTYPE_F32, reps=3)
    assert not name.endswith("tuned") and us > 0
    assert c2d.tune_save("/dev/null") == 0


def test_tune_rejects_bad_arguments():
    with pytest.raises(c2d.Conv2dError):
        c2d.tune(1, 8, 8, 16, 16, 3, 3, 5, 1, "relu")  # stride 5
    with pytest.raises(c2d.Conv2dError):
        c2d.tune(1, 8, 8, 16, 16, 3, 3, 1, 1, "relu", reps=0)


def test_tuned_channel_first_layer():
    """A channel-first f16 layer (the IFNet conv at a reduced frame): the tuner picks the
    kernel that runs after the layout copy (a tile of the pipelined kernel or a variant of
    the halo-tile GEMM); parity holds."""
    name, us = c2d.tune(1, 17, 30, 240, 240, 3, 3, 1, 1, "prelu", residual=True, layout="nchw",
                        dtype=c2d.DTYPE_F16, reps=5)
    assert name.startswith(("to_nhwc+igemm_nhwc_pipe", "to_nhwc+hgemm3x3_nchw_out")) and name.endswith(" tuned"), name
    x, spec, r = wl.random_conv_case(41, n=1, h=17, w=30, cin=240, cout=240, k=3, stride=1, pad=1, act="prelu",
                                     layout="nchw", dtype="f16", residual=True)
    y = c2d.conv2d_fused(x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV), spec.alpha.to(DEV), r.to(DEV), stride=1,
                         pad=1, act="prelu", layout="nchw")
    torch.cuda.synchronize()
    ref = oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias), to64(spec.alpha), to64(r), stride=1, pad=1,
                        act="prelu", layout="nchw")
    gate(to64(y), ref, "f16", what="tuned nchw")
