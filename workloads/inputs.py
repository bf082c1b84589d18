"""Seeded synthetic workloads shaped like the pages' layers.

No weights, images or video frames come with the pages, so every tensor here
is drawn from numpy's PCG64 generator (``numpy.random.default_rng(seed)``) and
stands in for the real data by shape and value range:

* images are U[0,1] (the inferencelayer page divides 8-bit pixels by 255);
* activations inside the IFNet block and the 1x1 projection are N(0,1);
* weights are He-normal, variance 2/fan_in with fan_in = Cin*kh*kw, unless a
  workload states another variance; biases are U[-0.1,0.1]; PReLU slopes are
  U[0,0.25].

Draw order: the input first, then for each conv in network order its weight,
bias and (for PReLU) slope. Values are drawn in fp64, cast to fp32, then
rounded to nearest-even into the storage type by torch's CPU cast. Tensors are
returned on the CPU in their storage dtype and in the workload's layout:
channel-last x [N,H,W,C] with OHWI weights, or channel-first x [N,C,H,W] with
OIHW weights.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to_storage(a, dtype: str) -> torch.Tensor:
    """fp32 values -> CPU tensor of the storage dtype (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(TORCH_DTYPES[dtype]).contiguous()


def _uniform(rng, shape, lo, hi):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def _normal(rng, shape, var):
    return (rng.standard_normal(size=shape) * np.sqrt(var)).astype(np.float32)


@dataclass
class ConvSpec:
    """One fused conv layer of a workload.

    ``src``/``res``/``out`` name tensors in the workload's dataflow; "x" is the
    workload input.
    """
    name: str
    cin: int
    cout: int
    k: int
    stride: int
    pad: int
    act: str
    src: str
    out: str
    res: Optional[str] = None
    res_before_act: bool = False
    w: Optional[torch.Tensor] = None
    bias: Optional[torch.Tensor] = None
    alpha: Optional[torch.Tensor] = None


@dataclass
class PoolSpec:
    name: str
    kind: str  # "max" (3x3 s2 p1) or "avg" (2x2 s2)
    src: str
    out: str


@dataclass
class Workload:
    name: str
    layout: str  # "nhwc" or "nchw"
    dtype: str  # "f32", "bf16", "f16"
    x: torch.Tensor
    layers: List[object] = field(default_factory=list)

    @property
    def n(self):
        return self.x.shape[0]


def _draw_conv(rng, spec: ConvSpec, layout: str, dtype: str, w_var: Optional[float] = None):
    fan_in = spec.cin * spec.k * spec.k
    var = 2.0 / fan_in if w_var is None else w_var
    shape = ((spec.cout, spec.k, spec.k, spec.cin) if layout == "nhwc"
             else (spec.cout, spec.cin, spec.k, spec.k))
    spec.w = to_storage(_normal(rng, shape, var), dtype)
    spec.bias = torch.from_numpy(_uniform(rng, (spec.cout,), -0.1, 0.1))
    if spec.act == "prelu":
        spec.alpha = torch.from_numpy(_uniform(rng, (spec.cout,), 0.0, 0.25))
    return spec


def conv1_single(seed: int = 0) -> Workload:
    """Single conv3x3 s1 p1, NHWC fp32, 1x32x32x16 -> 32 channels, bias+ReLU.

    x ~ U[-1,1], w ~ N(0, 1/(9*Cin)), bias ~ U[-0.1,0.1].
    """
    rng = np.random.default_rng(seed)
    x = to_storage(_uniform(rng, (1, 32, 32, 16), -1.0, 1.0), "f32")
    spec = ConvSpec("conv", 16, 32, 3, 1, 1, "relu", "x", "y")
    _draw_conv(rng, spec, "nhwc", "f32", w_var=1.0 / (9 * 16))
    return Workload("conv3x3_s1_16to32_32x32_nhwc_f32", "nhwc", "f32", x, [spec])


def conv2_stem(dtype: str = "f32", seed: int = 1, n: int = 1, hw: int = 640) -> Workload:
    """Stem conv3x3 s2 p1 3->32 + SiLU, then maxpool 3x3 s2 p1 (NHWC).

    x ~ U[0,1] image-like, He-normal weights.
    """
    rng = np.random.default_rng(seed)
    x = to_storage(_uniform(rng, (n, hw, hw, 3), 0.0, 1.0), dtype)
    conv = _draw_conv(rng, ConvSpec("stem", 3, 32, 3, 2, 1, "silu", "x", "stem"), "nhwc", dtype)
    pool = PoolSpec("maxpool", "max", "stem", "y")
    return Workload(f"stem_conv3x3s2_3to32_silu_maxpool_{n}x{hw}x{hw}_nhwc_{dtype}", "nhwc",
                    dtype, x, [conv, pool])


def conv2_stem_bf16(seed: int = 1) -> Workload:
    """The stem workload with bf16 storage."""
    return conv2_stem("bf16", seed)


def conv3_pointwise(seed: int = 2, n: int = 4, hw: int = 80) -> Workload:
    """1x1 conv 512->256 + bias + ReLU, NHWC bf16, x ~ N(0,1), w ~ N(0, 1/512)."""
    rng = np.random.default_rng(seed)
    x = to_storage(_normal(rng, (n, hw, hw, 512), 1.0), "bf16")
    spec = ConvSpec("proj", 512, 256, 1, 1, 0, "relu", "x", "y")
    _draw_conv(rng, spec, "nhwc", "bf16", w_var=1.0 / 512)
    return Workload(f"conv1x1_512to256_relu_{n}x{hw}x{hw}_nhwc_bf16", "nhwc", "bf16", x, [spec])


def conv4_ifnet_block(seed: int = 3, c: int = 240, h: int = 68, w: int = 120,
                      depth: int = 8) -> Workload:
    """IFNet-style conv block: ``depth`` conv3x3 s1 p1 C->C + bias + PReLU, NCHW f16.

    The last conv adds the block input after its activation. x ~ N(0,1).
    """
    rng = np.random.default_rng(seed)
    x = to_storage(_normal(rng, (1, c, h, w), 1.0), "f16")
    layers = []
    src = "x"
    for i in range(depth):
        last = i == depth - 1
        out = "y" if last else f"b{i}"
        spec = ConvSpec(f"conv{i}", c, c, 3, 1, 1, "prelu", src, out,
                        res="x" if last else None, res_before_act=False)
        layers.append(_draw_conv(rng, spec, "nchw", "f16"))
        src = out
    return Workload(f"ifnet_convblock_{depth}x_conv3x3_{c}ch_{h}x{w}_nchw_f16", "nchw", "f16",
                    x, layers)


def conv5_resnet18d(seed: int = 4, n: int = 4, hw: int = 640, dtype: str = "bf16",
                    widths=(64, 128, 256, 512), stem=(32, 32, 64)) -> Workload:
    """ResNet-18-D-style backbone, NHWC.

    Stem: conv3x3 s2 3->32, conv3x3 32->32, conv3x3 32->64 (ReLU each), then
    maxpool 3x3 s2 p1. Four stages of two BasicBlocks; a block is conv3x3 +
    ReLU, then conv3x3 whose output joins the shortcut before the ReLU. The
    first block of stages 2-4 has a stride-2 conv1 and the ResNet-D shortcut
    avgpool 2x2 + conv1x1 (no activation); other shortcuts are the identity.
    Batch-norm is taken as folded into the bias. Convs are listed (and drawn)
    in network order: stem1-3, then per block conv1, conv2, shortcut conv.
    """
    rng = np.random.default_rng(seed)
    x = to_storage(_uniform(rng, (n, hw, hw, 3), 0.0, 1.0), dtype)
    layers: list = []

    def conv(name, cin, cout, k, s, src, out, act="relu", res=None):
        spec = ConvSpec(name, cin, cout, k, s, k // 2, act, src, out, res=res,
                        res_before_act=res is not None)
        layers.append(spec)
        return spec

    conv("stem1", 3, stem[0], 3, 2, "x", "s1")
    conv("stem2", stem[0], stem[1], 3, 1, "s1", "s2")
    conv("stem3", stem[1], stem[2], 3, 1, "s2", "s3")
    layers.append(PoolSpec("maxpool", "max", "s3", "p0"))
    cur, cin = "p0", stem[2]
    for si, cw in enumerate(widths):
        for bi in range(2):
            tag = f"l{si + 1}b{bi}"
            down = si > 0 and bi == 0
            c1 = conv(f"{tag}.conv1", cin, cw, 3, 2 if down else 1, cur, f"{tag}.a")
            if down:
                c2 = ConvSpec(f"{tag}.conv2", cw, cw, 3, 1, 1, "relu", f"{tag}.a", f"{tag}.y",
                              res=f"{tag}.sc", res_before_act=True)
                layers.append(c2)
                layers.append(PoolSpec(f"{tag}.avgpool", "avg", cur, f"{tag}.ap"))
                sc = ConvSpec(f"{tag}.short", cin, cw, 1, 1, 0, "none", f"{tag}.ap",
                              f"{tag}.sc")
                layers.append(sc)
            else:
                conv(f"{tag}.conv2", cw, cw, 3, 1, f"{tag}.a", f"{tag}.y", res=cur)
            cur, cin = f"{tag}.y", cw
    # Draw weights in network order (stem, then per block conv1, conv2, shortcut),
    # then reorder execution so each shortcut runs before the conv2 that adds it.
    for spec in layers:
        if isinstance(spec, ConvSpec):
            _draw_conv(rng, spec, "nhwc", dtype)
    ordered = []
    pending = []
    for spec in layers:
        if isinstance(spec, ConvSpec) and spec.res is not None and spec.res.endswith(".sc"):
            pending.append(spec)
            continue
        ordered.append(spec)
        if isinstance(spec, ConvSpec) and spec.out.endswith(".sc"):
            ordered.extend(pending)
            pending = []
    assert not pending
    return Workload(f"resnet18d_backbone_{n}x{hw}x{hw}_nhwc_{dtype}", "nhwc", dtype, x, ordered)


def conv_out(h, k, s, p):
    return (h + 2 * p - k) // s + 1


def conv_flops(spec: ConvSpec, n: int, h: int, w: int) -> int:
    """2*N*OH*OW*Cout*Cin*kh*kw for a conv whose input is n x h x w."""
    oh, ow = conv_out(h, spec.k, spec.stride, spec.pad), conv_out(w, spec.k, spec.stride, spec.pad)
    return 2 * n * oh * ow * spec.cout * spec.cin * spec.k * spec.k


def random_conv_case(seed: int, *, n, h, w, cin, cout, k, stride, pad, act, layout, dtype,
                     residual=False, res_before_act=False, x_dist="normal"):
    """One random layer for shape sweeps: returns (x, spec, residual-or-None)."""
    rng = np.random.default_rng(seed)
    xshape = (n, h, w, cin) if layout == "nhwc" else (n, cin, h, w)
    xa = _normal(rng, xshape, 1.0) if x_dist == "normal" else _uniform(rng, xshape, 0.0, 1.0)
    x = to_storage(xa, dtype)
    spec = ConvSpec("case", cin, cout, k, stride, pad, act, "x", "y",
                    res="r" if residual else None, res_before_act=res_before_act)
    _draw_conv(rng, spec, layout, dtype)
    r = None
    if residual:
        oh, ow = conv_out(h, k, stride, pad), conv_out(w, k, stride, pad)
        rshape = (n, oh, ow, cout) if layout == "nhwc" else (n, cout, oh, ow)
        r = to_storage(_normal(rng, rshape, 1.0), dtype)
    return x, spec, r


def random_deconv_case(seed: int, *, n, h, w, cin, cout, act, layout, dtype, x_dist="normal"):
    """One random 4x4 stride-2 transposed-conv layer: returns (x, w, bias, alpha-or-None).

    x ~ N(0,1) (or U[0,1]) in ``layout``; w [Cin, Cout, 4, 4] He-normal with fan_in =
    4*Cin (each output pixel takes 2x2 taps of every input channel); bias U[-0.1,0.1];
    PReLU slope U[0,0.25]. Draw order: x, w, bias, slope.
    """
    rng = np.random.default_rng(seed)
    xshape = (n, h, w, cin) if layout == "nhwc" else (n, cin, h, w)
    xa = _normal(rng, xshape, 1.0) if x_dist == "normal" else _uniform(rng, xshape, 0.0, 1.0)
    x = to_storage(xa, dtype)
    wt = to_storage(_normal(rng, (cin, cout, 4, 4), 2.0 / (4 * cin)), dtype)
    bias = torch.from_numpy(_uniform(rng, (cout,), -0.1, 0.1))
    alpha = torch.from_numpy(_uniform(rng, (cout,), 0.0, 0.25)) if act == "prelu" else None
    return x, wt, bias, alpha


def ifnet_deconv(seed: int = 5, c: int = 240, h: int = 68, w: int = 120, cout: int = 5):
    """The transposed conv that ends IFNet block 0 at a 1920x1088 frame: the stride-16
    map [1, 240, 68, 120] (NCHW f16, N(0,1)) to the 5-channel stride-8 map (4 flow
    channels and a mask), no activation; the output is kept in fp32 as framecast does."""
    return random_deconv_case(seed, n=1, h=h, w=w, cin=c, cout=cout, act="none", layout="nchw", dtype="f16")


def random_map(seed: int, shape, dtype: str) -> torch.Tensor:
    """A map of N(0,1) values in the storage dtype (upsample and concat inputs)."""
    rng = np.random.default_rng(seed)
    return to_storage(_normal(rng, shape, 1.0), dtype)


def large_map(seed: int, n: int, h: int, w: int, c: int, dtype: str = "bf16") -> torch.Tensor:
    """A channel-last map of n*h*w*c elements for tests at the size limits, built row by
    row so that no full-size fp32 or fp64 temporary is needed: a seeded N(0,1) block of
    61 x 67 pixels repeated over the map, plus a second seeded [29, c] table indexed by
    (row + 2*column) % 29, so that a read displaced by a whole block period still sees
    different values. Rounded to the storage dtype per row."""
    rng = np.random.default_rng(seed)
    base = _normal(rng, (61, 67, c), 1.0)
    tab = _normal(rng, (29, c), 0.25)
    cols = np.arange(w)
    base_w = base[:, cols % 67, :]                     # [61, w, c]
    out = torch.empty((n, h, w, c), dtype=TORCH_DTYPES[dtype])
    for b in range(n):
        for r in range(h):
            row = base_w[r % 61] + tab[(r + 2 * cols) % 29]
            out[b, r] = torch.from_numpy(row).to(TORCH_DTYPES[dtype])
    return out
