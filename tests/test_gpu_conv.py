"""GPU parity of conv2d_fused against the CPU oracle (needs an MI355X)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import bits_equal, gate, quantized_tensor, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")


def _gpu_conv(x, spec, r, layout, out=None):
    return c2d.conv2d_fused(x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV) if spec.bias is not None else None,
                            spec.alpha.to(DEV) if spec.alpha is not None else None,
                            r.to(DEV) if r is not None else None, stride=spec.stride, pad=spec.pad,
                            act=spec.act, res_before_act=spec.res_before_act, layout=layout, out=out)


def _oracle_conv(x, spec, r, layout):
    return oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias) if spec.bias is not None else None,
                         to64(spec.alpha) if spec.alpha is not None else None,
                         to64(r) if r is not None else None, stride=spec.stride, pad=spec.pad,
                         act=spec.act, res_before_act=spec.res_before_act, layout=layout)


# (n, h, w, cin, cout, k, stride, pad, act, residual, layout, dtype)
SWEEP = [
    (1, 9, 11, 8, 16, 3, 1, 1, "relu", None, "nhwc", "bf16"),
    (2, 33, 29, 64, 130, 3, 1, 1, "silu", None, "nhwc", "bf16"),
    (2, 33, 29, 64, 130, 3, 2, 1, "relu", "pre", "nhwc", "bf16"),
    (3, 17, 20, 40, 33, 3, 1, 0, "prelu", "post", "nhwc", "f16"),
    (1, 40, 37, 24, 64, 5, 1, 2, "none", "post", "nhwc", "bf16"),
    (2, 21, 22, 16, 100, 1, 1, 0, "relu", None, "nhwc", "bf16"),
    (2, 21, 22, 128, 256, 1, 2, 0, "relu", None, "nhwc", "f16"),
    (1, 30, 30, 5, 48, 3, 1, 1, "relu", None, "nhwc", "bf16"),
    (1, 30, 30, 100, 7, 3, 2, 1, "silu", "pre", "nhwc", "f16"),
    (2, 23, 19, 3, 32, 3, 2, 1, "silu", None, "nhwc", "bf16"),
    (2, 23, 19, 3, 32, 3, 2, 1, "silu", None, "nhwc", "f32"),
    (1, 25, 27, 4, 20, 3, 1, 1, "prelu", "post", "nhwc", "f16"),
    (1, 32, 32, 16, 32, 3, 1, 1, "relu", None, "nhwc", "f32"),
    (2, 19, 26, 12, 70, 3, 2, 1, "prelu", "pre", "nhwc", "f32"),
    (1, 14, 15, 9, 9, 3, 1, 1, "relu", "post", "nhwc", "f32"),
    (1, 34, 30, 48, 48, 3, 1, 1, "prelu", "post", "nchw", "f16"),
    (2, 17, 23, 40, 72, 3, 2, 1, "relu", "pre", "nchw", "f16"),
    (1, 20, 24, 32, 130, 1, 1, 0, "silu", None, "nchw", "bf16"),
    (1, 31, 33, 7, 24, 3, 1, 1, "prelu", None, "nchw", "f16"),
    (2, 16, 18, 3, 16, 3, 2, 1, "relu", None, "nchw", "f32"),
    (1, 22, 21, 20, 40, 5, 2, 2, "none", "post", "nchw", "f32"),
    (3, 12, 13, 64, 64, 3, 1, 1, "relu", "pre", "nhwc", "bf16"),
    (1, 5, 5, 32, 16, 5, 1, 0, "relu", None, "nhwc", "bf16"),   # one output pixel
    (1, 1, 1, 64, 64, 1, 1, 0, "none", None, "nhwc", "bf16"),   # 1x1 image
    (1, 2, 3, 16, 8, 3, 2, 2, "relu", None, "nhwc", "f16"),     # padding wider than input
    (4, 7, 9, 8, 1, 3, 1, 1, "silu", None, "nhwc", "bf16"),     # one output channel
    (1, 11, 13, 1, 5, 3, 1, 1, "relu", None, "nchw", "bf16"),   # one input channel
    # channel-first through channel-last copies + the matrix-core kernel
    (2, 9, 7, 64, 40, 3, 1, 1, "prelu", "post", "nchw", "f16"),  # 63 pixels: per-element stores
    (1, 16, 16, 128, 96, 3, 2, 1, "relu", "pre", "nchw", "bf16"),
    (3, 12, 12, 72, 200, 1, 1, 0, "silu", None, "nchw", "f16"),
    (1, 17, 30, 240, 240, 3, 1, 1, "prelu", "post", "nchw", "f16"),  # IFNet conv, reduced frame
    # few output tiles, deep K (split-K: fp32 slices, then a second pass for the epilogue)
    (1, 10, 10, 512, 512, 3, 1, 1, "relu", "pre", "nhwc", "bf16"),
    (2, 7, 9, 384, 64, 3, 1, 1, "prelu", "post", "nhwc", "f16"),
    (1, 9, 11, 512, 200, 3, 1, 1, "silu", None, "nhwc", "bf16"),
    (1, 10, 10, 256, 256, 3, 1, 1, "relu", "pre", "nhwc", "bf16"),
    (2, 9, 7, 72, 200, 3, 2, 1, "silu", "post", "nhwc", "f16"),  # Cin % 64 != 0, K tail
    (1, 6, 6, 512, 64, 3, 1, 1, "none", None, "nhwc", "bf16"),
    (1, 7, 9, 320, 40, 3, 2, 1, "prelu", "post", "nhwc", "bf16"),
    (3, 5, 5, 128, 96, 1, 1, 0, "relu", None, "nhwc", "f16"),
    (2, 12, 12, 256, 512, 3, 2, 1, "relu", None, "nhwc", "bf16"),
    (1, 64, 64, 64, 64, 3, 1, 1, "relu", "pre", "nhwc", "bf16"),  # many tiles, taps innermost
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: "-".join(map(str, c)))
def test_sweep(case):
    n, h, w, cin, cout, k, s, p, act, res, layout, dtype = case
    seed = zlib.crc32(repr(case).encode())
    x, spec, r = wl.random_conv_case(seed, n=n, h=h, w=w, cin=cin, cout=cout, k=k, stride=s, pad=p,
                                     act=act, layout=layout, dtype=dtype, residual=res is not None,
                                     res_before_act=res == "pre")
    plan = c2d.plan(n, h, w, cin, cout, k, k, s, p, 0, 0 if layout == "nhwc" else 1,
                    {"f32": 0, "bf16": 1, "f16": 2}[dtype])
    print(f"case {case} plan {plan}", flush=True)
    y = _gpu_conv(x, spec, r, layout)
    torch.cuda.synchronize()
    gate(to64(y), _oracle_conv(x, spec, r, layout), dtype, what=str(case))


# Narrow 3x3 stride-1 layers on the halo-tile kernel: ragged tile rows and columns,
# partial channel blocks, every epilogue, and enough tiles that each persistent
# workgroup walks several (both halo buffers, the prefetch of tiles past the end).
# (n, h, w, cin, cout, act, residual, dtype)
HALO = [
    (1, 9, 11, 16, 16, "relu", None, "bf16"),
    (2, 37, 45, 32, 32, "silu", None, "bf16"),
    (2, 37, 45, 32, 64, "prelu", "post", "f16"),
    (1, 70, 100, 64, 64, "relu", "pre", "bf16"),
    (2, 33, 65, 64, 24, "none", "post", "bf16"),
    (3, 8, 32, 16, 40, "relu", "pre", "f16"),
    (1, 1, 1, 32, 32, "relu", None, "bf16"),
    (1, 130, 66, 32, 8, "silu", None, "bf16"),
    (4, 256, 256, 16, 32, "relu", None, "bf16"),
    (2, 150, 200, 64, 64, "prelu", "pre", "f16"),
    (2, 160, 160, 32, 48, "silu", "post", "bf16"),
    (4, 256, 256, 64, 32, "relu", "pre", "bf16"),
    (2, 64, 100, 16, 64, "silu", None, "f16"),
    # 64 input channels (the kernel with specialised waves): one pixel, two tiles (fewer
    # workgroups than CUs), a wide short map, channel groups past Cout, every epilogue
    (1, 1, 1, 64, 64, "relu", "post", "bf16"),
    (1, 8, 40, 64, 64, "silu", "pre", "bf16"),
    (1, 5, 300, 64, 56, "silu", "post", "f16"),
    (3, 17, 31, 64, 8, "none", None, "bf16"),
    (2, 41, 77, 64, 40, "prelu", None, "bf16"),
]


@pytest.mark.parametrize("case", HALO, ids=lambda c: "-".join(map(str, c)))
def test_halo(case):
    n, h, w, cin, cout, act, res, dtype = case
    seed = zlib.crc32(repr(case).encode())
    x, spec, r = wl.random_conv_case(seed, n=n, h=h, w=w, cin=cin, cout=cout, k=3, stride=1, pad=1,
                                     act=act, layout="nhwc", dtype=dtype, residual=res is not None,
                                     res_before_act=res == "pre")
    plan = c2d.plan(n, h, w, cin, cout, 3, 3, 1, 1, 0, 0, {"bf16": 1, "f16": 2}[dtype])
    print(f"case {case} plan {plan}", flush=True)
    assert plan.startswith("halo3x3"), plan
    y = _gpu_conv(x, spec, r, "nhwc")
    torch.cuda.synchronize()
    gate(to64(y), _oracle_conv(x, spec, r, "nhwc"), dtype, what=str(case))


# 3-channel images on the matrix-core stem kernel: stride 1 and 2, partial last
# 32-pixel group of a row, partial channel blocks, single-row images, every epilogue.
# (n, h, w, cout, stride, act, residual, dtype)
STEM = [
    (1, 17, 24, 32, 2, "relu", None, "bf16"),
    (2, 32, 40, 64, 2, "silu", "post", "f16"),
    (1, 21, 16, 32, 1, "prelu", "pre", "bf16"),
    (3, 9, 8, 16, 1, "none", None, "bf16"),
    (1, 64, 88, 48, 2, "relu", None, "bf16"),
    (1, 1, 8, 32, 2, "relu", None, "bf16"),
    (2, 130, 136, 64, 2, "relu", "pre", "bf16"),
    (1, 40, 72, 24, 1, "silu", None, "f16"),
    # fp32 storage: the 32x32x2 fp32 kernel (Cout % 4 == 0, W % 4 == 0)
    (1, 17, 24, 32, 2, "silu", None, "f32"),
    (2, 21, 20, 64, 1, "relu", "pre", "f32"),
    (1, 9, 36, 12, 2, "prelu", "post", "f32"),
    (1, 1, 4, 32, 2, "relu", None, "f32"),
    (3, 33, 132, 40, 1, "none", None, "f32"),
]


@pytest.mark.parametrize("case", STEM, ids=lambda c: "-".join(map(str, c)))
def test_stem(case):
    n, h, w, cout, s, act, res, dtype = case
    seed = zlib.crc32(repr(case).encode())
    x, spec, r = wl.random_conv_case(seed, n=n, h=h, w=w, cin=3, cout=cout, k=3, stride=s, pad=1,
                                     act=act, layout="nhwc", dtype=dtype, residual=res is not None,
                                     res_before_act=res == "pre", x_dist="uniform")
    plan = c2d.plan(n, h, w, 3, cout, 3, 3, s, 1, 0, 0, {"f32": 0, "bf16": 1, "f16": 2}[dtype])
    print(f"case {case} plan {plan}", flush=True)
    assert plan.startswith("stem3x3"), plan
    y = _gpu_conv(x, spec, r, "nhwc")
    torch.cuda.synchronize()
    gate(to64(y), _oracle_conv(x, spec, r, "nhwc"), dtype, what=str(case))


@pytest.mark.parametrize("layout", ["nhwc", "nchw"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_delta_kernel_is_identity(layout, dtype):
    """A centred one-hot 3x3 kernel with no bias copies the input bit for bit."""
    x, spec, _ = wl.random_conv_case(5, n=2, h=21, w=18, cin=24, cout=24, k=3, stride=1, pad=1,
                                     act="none", layout=layout, dtype=dtype)
    wd = torch.zeros(spec.w.shape, dtype=torch.float32)
    for c in range(24):
        if layout == "nhwc":
            wd[c, 1, 1, c] = 1.0
        else:
            wd[c, c, 1, 1] = 1.0
    spec.w = wd.to(spec.w.dtype)
    spec.bias = None
    y = _gpu_conv(x, spec, None, layout)
    assert bits_equal(y, x)


def test_conv1_single_full():
    work = wl.conv1_single()
    spec = work.layers[0]
    y = _gpu_conv(work.x, spec, None, "nhwc")
    torch.cuda.synchronize()
    gate(to64(y), _oracle_conv(work.x, spec, None, "nhwc"), "f32", what="conv1")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv2_stem_and_maxpool_full(dtype):
    work = wl.conv2_stem(dtype)
    conv, _ = work.layers
    y = _gpu_conv(work.x, conv, None, "nhwc")
    p = c2d.maxpool3x3s2(y, layout="nhwc")
    torch.cuda.synchronize()
    gate(to64(y), _oracle_conv(work.x, conv, None, "nhwc"), dtype, what=f"stem {dtype}")
    assert np.array_equal(to64(p), oracle.maxpool3x3s2(to64(y)))


def _sample_idx(rng, shape, count):
    """Random output indices plus the last element of every axis (the ragged tails)."""
    idx = np.stack([rng.integers(0, d, count) for d in shape], axis=1)
    tails = np.array([[d - 1 for d in shape], [0] * len(shape)] +
                     [[rng.integers(0, d) if j != i else shape[i] - 1 for j, d in enumerate(shape)]
                      for i in range(len(shape)) for _ in range(16)])
    return np.concatenate([idx, tails])


def _check_sampled(x, spec, r, y, layout, dtype, rng, count=6000, what=""):
    idx = _sample_idx(rng, tuple(y.shape), count)
    ref = oracle.conv2d_points(to64(x), to64(spec.w), to64(spec.bias),
                               to64(spec.alpha) if spec.alpha is not None else None,
                               to64(r) if r is not None else None, idx, stride=spec.stride,
                               pad=spec.pad, act=spec.act, res_before_act=spec.res_before_act,
                               layout=layout)
    yc = to64(y)
    got = yc[tuple(idx.T)]
    return gate(got, ref, dtype, what=what)


def test_conv3_pointwise_full():
    work = wl.conv3_pointwise()
    spec = work.layers[0]
    y = _gpu_conv(work.x, spec, None, "nhwc")
    torch.cuda.synchronize()
    gate(to64(y), _oracle_conv(work.x, spec, None, "nhwc"), "bf16", what="conv3")


def test_conv3_pointwise_sampled_points():
    """The oracle's point-wise entry on random outputs and the tails of every axis."""
    work = wl.conv3_pointwise()
    spec = work.layers[0]
    y = _gpu_conv(work.x, spec, None, "nhwc")
    torch.cuda.synchronize()
    _check_sampled(work.x, spec, None, y, "nhwc", "bf16", np.random.default_rng(1), what="conv3")


_CHAINS = {}


def oracle_chain(key, work):
    """The workload run by the oracle alone, from the seeded input: per map name the fp64
    output of the producing layer ("ref") and its storage rounding ("q", the next layer's
    input). Cached per workload."""
    if key in _CHAINS:
        return _CHAINS[key]
    q = {"x": to64(work.x)}
    ref = {}
    for spec in work.layers:
        src = q[spec.src]
        if isinstance(spec, wl.ConvSpec):
            r = q[spec.res] if spec.res is not None else None
            y = oracle.conv2d(src, to64(spec.w), to64(spec.bias),
                              to64(spec.alpha) if spec.alpha is not None else None, r,
                              stride=spec.stride, pad=spec.pad, act=spec.act,
                              res_before_act=spec.res_before_act, layout=work.layout)
        elif spec.kind == "max":
            y = oracle.maxpool3x3s2(src, layout=work.layout)
        else:
            y = oracle.avgpool2x2(src, layout=work.layout).astype(np.float64)
        ref[spec.out] = y
        q[spec.out] = oracle.quantize(y, work.dtype)
    _CHAINS[key] = (q, ref)
    return q, ref


def _gpu_layer(spec, work, inputs):
    src = inputs[spec.src]
    if isinstance(spec, wl.ConvSpec):
        r = inputs[spec.res] if spec.res is not None else None
        return _gpu_conv(src, spec, r, work.layout)
    if spec.kind == "max":
        return c2d.maxpool3x3s2(src, layout=work.layout)
    return c2d.avgpool2x2(src, layout=work.layout)


def _per_layer(key, work):
    """Every layer on the GPU, fed the oracle chain's own (rounded) maps, against the oracle's
    output of that layer: convs by the gate, pools bit for bit."""
    q, ref = oracle_chain(key, work)
    stats = {}
    for spec in work.layers:
        names = [spec.src] + ([spec.res] if getattr(spec, "res", None) else [])
        inputs = {n: quantized_tensor(q[n], work.dtype).to(DEV) for n in names}
        print(f"layer {spec.name}", flush=True)
        y = _gpu_layer(spec, work, inputs)
        torch.cuda.synchronize()
        if isinstance(spec, wl.ConvSpec):
            stats[spec.name] = gate(to64(y), ref[spec.out], work.dtype, what=spec.name)
        else:
            assert np.array_equal(to64(y), q[spec.out]), spec.name
    return stats


def _end_to_end(key, work):
    """The GPU chain fed only its own outputs against the oracle chain (aggregate gates)."""
    q, ref = oracle_chain(key, work)
    t = {"x": work.x.to(DEV)}
    for spec in work.layers:
        t[spec.out] = _gpu_layer(spec, work, t)
    torch.cuda.synchronize()
    last = work.layers[-1].out
    return gate(to64(t[last]), ref[last], work.dtype, what=f"{key} end to end", elementwise=False)


def test_conv4_ifnet_block_per_layer_full():
    """Full frame (240 x 68 x 120, NCHW f16): each of the 8 convs, full output."""
    stats = _per_layer("ifnet", wl.conv4_ifnet_block())
    assert len(stats) == 8


def test_conv4_ifnet_block_end_to_end_full():
    _end_to_end("ifnet", wl.conv4_ifnet_block())


def test_conv5_resnet18d_per_layer_full():
    """Full backbone (4 x 640 x 640, NHWC bf16): all 22 convs on full maps, pools bit-exact."""
    stats = _per_layer("resnet", wl.conv5_resnet18d())
    assert len(stats) == 22


def test_conv5_resnet18d_end_to_end_full():
    _end_to_end("resnet", wl.conv5_resnet18d())


def test_repeatable():
    """Every output is one fixed-order fp32 sum (split-K slices are added in slice
    order): repeated calls agree bit for bit."""
    x, spec, r = wl.random_conv_case(11, n=1, h=20, w=20, cin=512, cout=512, k=3, stride=1, pad=1,
                                     act="relu", layout="nhwc", dtype="bf16", residual=True,
                                     res_before_act=True)
    assert "splitk=1" not in c2d.plan(1, 20, 20, 512, 512, 3, 3, 1, 1, 0x101, 0, 1)
    ys = [_gpu_conv(x, spec, r, "nhwc") for _ in range(4)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert bits_equal(y, ys[0])
    gate(to64(ys[0]), _oracle_conv(x, spec, r, "nhwc"), "bf16")


def test_batch_equals_separate_runs():
    x, spec, r = wl.random_conv_case(9, n=3, h=20, w=20, cin=64, cout=64, k=3, stride=1, pad=1,
                                     act="relu", layout="nhwc", dtype="bf16", residual=True,
                                     res_before_act=True)
    yb = _gpu_conv(x, spec, r, "nhwc")
    for i in range(3):
        yi = _gpu_conv(x[i:i + 1].contiguous(), spec, r[i:i + 1].contiguous(), "nhwc")
        gate(to64(yi), to64(yb[i:i + 1]), "bf16", what=f"image {i}")


def test_output_buffer_and_stream():
    """Writes into a caller buffer on a caller stream; nothing outside y changes."""
    x, spec, _ = wl.random_conv_case(10, n=1, h=16, w=16, cin=32, cout=32, k=3, stride=1, pad=1,
                                     act="relu", layout="nhwc", dtype="bf16")
    big = torch.full((3, 16, 16, 32), 7.0, dtype=torch.bfloat16, device=DEV)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        c2d.conv2d_fused(x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV), stride=1, pad=1, act="relu",
                         out=big[1:2], stream=st)
    st.synchronize()
    assert torch.all(big[0] == 7.0) and torch.all(big[2] == 7.0)
    gate(to64(big[1:2]), _oracle_conv(x, spec, None, "nhwc"), "bf16")


def test_invalid_arguments_raise_without_writing():
    x = torch.zeros((1, 8, 8, 16), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((16, 3, 3, 16), dtype=torch.bfloat16, device=DEV)
    y = torch.full((1, 8, 8, 16), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(c2d.Conv2dError) as e:
        c2d.conv2d_fused(x, w, None, None, None, stride=1, pad=1, act="prelu", out=y)
    assert e.value.code == c2d.EINVAL
    y3 = torch.full((1, 3, 3, 16), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(c2d.Conv2dError) as e:
        c2d.conv2d_fused(x, w, stride=3, pad=1, out=y3)  # the library accepts strides 1 and 2
    assert e.value.code == c2d.EINVAL
    with pytest.raises(c2d.Conv2dError) as e:
        c2d.conv2d_fused(x, w, stride=1, pad=1, out=x.view(1, 8, 8, 16))  # y aliases x
    assert e.value.code == c2d.EINVAL
    torch.cuda.synchronize()
    assert torch.all(y == 3.0) and torch.all(y3 == 3.0)


@pytest.mark.parametrize("n,h,w,cin,cout,k,stride,act,dt", [
    (1, 17, 30, 240, 240, 3, 1, "prelu", "f16"),
    (2, 9, 7, 64, 40, 3, 2, "relu", "bf16"),
    (3, 12, 12, 72, 200, 1, 1, "silu", "f16"),
])
def test_channel_first_with_ohwi_weights(n, h, w, cin, cout, k, stride, act, dt):
    """Weights converted once to OHWI (weights_to_ohwi) and passed with weights_ohwi give the
    bit-identical output of the OIHW call, which is checked against the oracle."""
    x, spec, r = wl.random_conv_case(101 + cin, n=n, h=h, w=w, cin=cin, cout=cout, k=k, stride=stride, pad=k // 2,
                                     act=act, layout="nchw", dtype=dt, residual=True)
    xd, wd, bd, rd = x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV), r.to(DEV)
    ad = spec.alpha.to(DEV) if spec.alpha is not None else None
    y1 = c2d.conv2d_fused(xd, wd, bd, ad, rd, stride=stride, pad=k // 2, act=act, layout="nchw")
    w2 = c2d.weights_to_ohwi(wd)
    y2 = c2d.conv2d_fused(xd, w2, bd, ad, rd, stride=stride, pad=k // 2, act=act, layout="nchw", weights_ohwi=True)
    torch.cuda.synchronize()
    assert torch.equal(w2.cpu(), spec.w.permute(0, 2, 3, 1).contiguous())
    assert torch.equal(y1, y2)
    gate(to64(y2), _oracle_conv(x, spec, r, "nchw"), dt, what="ohwi weights")
