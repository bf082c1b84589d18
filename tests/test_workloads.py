"""Host-side checks of the synthetic workloads (CPU only)."""
import numpy as np
import torch

import workloads as wl
from workloads.inputs import ConvSpec, PoolSpec, conv_out


def _walk(work):
    """Propagate shapes through a workload's layers; returns total conv FLOPs."""
    shapes = {"x": tuple(work.x.shape)}
    flops = 0
    for spec in work.layers:
        s = shapes[spec.src]
        n, h, w, c = s if work.layout == "nhwc" else (s[0], s[2], s[3], s[1])
        if isinstance(spec, ConvSpec):
            assert c == spec.cin, spec.name
            oh, ow = conv_out(h, spec.k, spec.stride, spec.pad), conv_out(w, spec.k, spec.stride, spec.pad)
            flops += wl.conv_flops(spec, n, h, w)
            out = (n, oh, ow, spec.cout) if work.layout == "nhwc" else (n, spec.cout, oh, ow)
            if spec.res is not None:
                assert shapes[spec.res] == out, spec.name
            assert spec.w.dtype == wl.inputs.TORCH_DTYPES[work.dtype]
            assert spec.bias.dtype == torch.float32 and spec.bias.shape == (spec.cout,)
        else:
            oh, ow = ((h - 1) // 2 + 1, (w - 1) // 2 + 1) if spec.kind == "max" else (h // 2, w // 2)
            out = (n, oh, ow, c) if work.layout == "nhwc" else (n, c, oh, ow)
        shapes[spec.out] = out
    return flops, shapes


def test_resnet18d_structure_and_flops():
    work = wl.conv5_resnet18d()
    convs = [s for s in work.layers if isinstance(s, ConvSpec)]
    pools = [s for s in work.layers if isinstance(s, PoolSpec)]
    assert len(convs) == 22
    assert sorted(p.kind for p in pools) == ["avg", "avg", "avg", "max"]
    flops, shapes = _walk(work)
    assert round(flops / 1e9, 2) == 134.09
    assert shapes["l4b1.y"] == (4, 20, 20, 512)
    assert shapes["p0"] == (4, 160, 160, 64)


def test_other_workloads():
    f1, s1 = _walk(wl.conv1_single())
    assert f1 == 2 * 32 * 32 * 32 * 16 * 9 and s1["y"] == (1, 32, 32, 32)
    for dt in ("f32", "bf16"):
        f2, s2 = _walk(wl.conv2_stem(dt))
        assert s2["y"] == (1, 160, 160, 32) and s2["stem"] == (1, 320, 320, 32)
    f3, s3 = _walk(wl.conv3_pointwise())
    assert f3 == 2 * 25600 * 256 * 512
    f4, s4 = _walk(wl.conv4_ifnet_block())
    assert f4 == 8 * 2 * 8160 * 240 * 2160 and s4["y"] == (1, 240, 68, 120)


def test_inputs_are_seeded_and_in_range():
    a = wl.conv2_stem("bf16")
    b = wl.conv2_stem("bf16")
    assert torch.equal(a.x, b.x) and torch.equal(a.layers[0].w, b.layers[0].w)
    x = a.x.float()
    assert float(x.min()) >= 0.0 and float(x.max()) <= 1.0
    w4 = wl.conv4_ifnet_block().layers[0]
    assert float(w4.alpha.min()) >= 0 and float(w4.alpha.max()) <= 0.25
    # He-normal variance 2/fan_in, checked loosely on a big weight
    w = wl.conv5_resnet18d().layers[-1].w.float().numpy()
    assert abs(w.var() * 4608 / 2 - 1) < 0.05
    assert np.abs(a.layers[0].bias.numpy()).max() <= 0.1
