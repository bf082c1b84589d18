"""The caller-owned workspace on the GPU: calls with and without one agree with the oracle
(different kernel variants, the same layer); two streams with two workspaces give the same
bits as one stream; shapes with no workspace-free variant fail before launching."""
import pytest
import torch

import oracle
import workloads as wl
from parity import bits_equal, gate, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")

# layers whose preferred variant writes the workspace: a channel-first 16-bit conv
# (channel-last copies) and a deep-K strided channel-last conv with few tiles whose Cin
# (520) the halo-tile GEMM does not take (split-K)
CASES = [
    dict(n=1, h=34, w=40, cin=64, cout=96, k=3, stride=1, pad=1, act="prelu", layout="nchw", dtype="f16"),
    dict(n=2, h=10, w=10, cin=520, cout=512, k=3, stride=2, pad=1, act="relu", layout="nhwc", dtype="bf16"),
]


def _case(i):
    c = CASES[i]
    x, spec, _ = wl.random_conv_case(40 + i, residual=False, **c)
    return c, x, spec


def _run(c, x, spec, **kw):
    return c2d.conv2d_fused(x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV),
                            spec.alpha.to(DEV) if spec.alpha is not None else None, None,
                            stride=c["stride"], pad=c["pad"], act=c["act"], layout=c["layout"], **kw)


def _ref(c, x, spec):
    return oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias),
                         to64(spec.alpha) if spec.alpha is not None else None, None,
                         stride=c["stride"], pad=c["pad"], act=c["act"], layout=c["layout"])


def _plan(c, spec, nbytes):
    lay = c2d.LAYOUT_NCHW if c["layout"] == "nchw" else c2d.LAYOUT_NHWC
    dt = c2d.DTYPE_F16 if c["dtype"] == "f16" else c2d.DTYPE_BF16
    return c2d.plan(c["n"], c["h"], c["w"], c["cin"], c["cout"], c["k"], c["k"], c["stride"], c["pad"],
                    c2d._ACTS[c["act"]], lay, dt, workspace_bytes=nbytes)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_with_and_without_workspace_match_the_oracle(i):
    c, x, spec = _case(i)
    with_ws, without = _plan(c, spec, c2d.DEFAULT_WORKSPACE_BYTES), _plan(c, spec, 0)
    assert with_ws != without, (with_ws, without)
    ref = _ref(c, x, spec)
    y1 = _run(c, x, spec)
    y0 = _run(c, x, spec, workspace=False)
    torch.cuda.synchronize()
    gate(to64(y1), ref, c["dtype"], what=f"case {i} with workspace ({with_ws})")
    gate(to64(y0), ref, c["dtype"], what=f"case {i} without workspace ({without})")


def test_two_streams_two_workspaces_match_one_stream():
    """Both workspace-using layers, each repeated on two streams at the same time with a
    workspace per stream, give the bits of the same calls run one after another on one
    stream."""
    runs = [_case(i) for i in range(len(CASES))]
    dev_in = [(c, x.to(DEV), spec) for c, x, spec in runs]
    serial = []
    for c, x, spec in dev_in:
        serial.append(_run(c, x, spec))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1 = torch.empty(c2d.DEFAULT_WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)
    ws2 = torch.empty(c2d.DEFAULT_WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)
    outs = {1: [], 2: []}
    for rep in range(4):
        for c, x, spec in dev_in:
            outs[1].append(_run(c, x, spec, stream=s1, workspace=ws1))
            outs[2].append(_run(c, x, spec, stream=s2, workspace=ws2))
    torch.cuda.synchronize()
    for k in (1, 2):
        for j, y in enumerate(outs[k]):
            assert bits_equal(y, serial[j % len(serial)]), f"stream {k} call {j}"


def test_default_workspaces_are_per_stream():
    """The binding's default workspace: one buffer per (device, stream)."""
    c, x, spec = _case(0)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    y1 = _run(c, x, spec, stream=s1)
    y2 = _run(c, x, spec, stream=s2)
    torch.cuda.synchronize()
    k1 = (torch.cuda.current_device(), s1.cuda_stream)
    k2 = (torch.cuda.current_device(), s2.cuda_stream)
    assert c2d._ws_cache[k1].data_ptr() != c2d._ws_cache[k2].data_ptr()
    assert bits_equal(y1, y2)


def test_shapes_without_a_workspace_free_variant_fail_before_launch():
    x, spec, _ = wl.random_conv_case(7, n=1, h=64, w=64, cin=64, cout=64, k=3, stride=1, pad=1, act="relu",
                                     layout="nhwc", dtype="bf16")
    xd = x.to(DEV)
    out = torch.full((1, 32, 32, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(c2d.Conv2dError) as e:
        c2d.conv2d_fused_maxpool3x3s2(xd, spec.w.to(DEV), spec.bias.to(DEV), act="relu", stride=1, pad=1,
                                      out=out, workspace=False)
    assert e.value.code == c2d.EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 7.0), "a failed call wrote its output"
    # with a workspace the same call runs (conv into the workspace, then the pool kernel):
    # within the gate of the oracle, and bit for bit the pool of the library's own conv
    # output (the conv's fp32 sums may round differently from the fp64 oracle's)
    y = c2d.conv2d_fused_maxpool3x3s2(xd, spec.w.to(DEV), spec.bias.to(DEV), act="relu", stride=1, pad=1)
    conv = oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias), stride=1, pad=1, act="relu")
    gate(to64(y), oracle.maxpool3x3s2(conv), "bf16", what="conv then pool through the workspace")
    y2 = c2d.maxpool3x3s2(c2d.conv2d_fused(xd, spec.w.to(DEV), spec.bias.to(DEV), act="relu", stride=1, pad=1))
    torch.cuda.synchronize()
    assert bits_equal(y, y2)


def test_deconv_without_workspace_runs_on_the_vector_alus():
    x, w, b, _ = wl.random_deconv_case(9, n=1, h=12, w=16, cin=64, cout=32, act="relu", layout="nhwc",
                                       dtype="bf16")
    assert c2d.plan_deconv(1, 12, 16, 64, 32, 1, 0, c2d.DTYPE_BF16, workspace_bytes=0).startswith("deconv4x4s2_direct")
    y0 = c2d.conv_transpose4x4s2(x.to(DEV), w.to(DEV), b.to(DEV), act="relu", workspace=False)
    y1 = c2d.conv_transpose4x4s2(x.to(DEV), w.to(DEV), b.to(DEV), act="relu")
    torch.cuda.synchronize()
    ref = oracle.conv_transpose4x4s2(to64(x), to64(w), to64(b), act="relu")
    gate(to64(y0), ref, "bf16", what="deconv without workspace")
    gate(to64(y1), ref, "bf16", what="deconv with workspace")
