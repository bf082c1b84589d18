"""conv2d_fused_noalloc through the C ABI: the entry point for callers that cannot allocate,
whose scratch is the library's static device array. Its output must equal conv2d_fused's
(given a workspace) bit for bit and meet the oracle gate, on two calls in a row on one GPU,
the second with a smaller input (the array keeps the first call's data)."""
import ctypes

import pytest
import torch

import oracle
import workloads as wl
from parity import bits_equal, gate, to64

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
DEV = torch.device("cuda")

# (layout, dtype, act, cin, cout, k, stride, pad, [(n, h, w) first call, (n, h, w) second])
VARIANTS = {
    # channel-first 16-bit: channel-last copies of x and w in the scratch
    "channel_first_copies": ("nchw", "f16", "prelu", 64, 96, 3, 1, 1, [(1, 34, 40), (1, 20, 24)]),
    # deep K, few tiles: split-K partial sums in the scratch
    "split_k": ("nhwc", "bf16", "relu", 512, 512, 3, 1, 1, [(2, 10, 10), (1, 6, 6)]),
    # a layer whose kernels use no scratch at all
    "no_scratch": ("nhwc", "bf16", "silu", 64, 64, 3, 1, 1, [(1, 40, 40), (1, 17, 19)]),
}


def _noalloc(x, wd, bd, ad, spec, y, layout):
    """One conv2d_fused_noalloc call on device tensors; asserts CONV2D_OK."""
    lib = c2d._load()
    if layout == "nhwc":
        n, h, w, cin = x.shape
    else:
        n, cin, h, w = x.shape
    P = ctypes.c_void_p
    print(f"conv2d_fused_noalloc {layout} {x.dtype} n={n} h={h} w={w} cin={cin} cout={spec.cout}", flush=True)
    rc = lib.conv2d_fused_noalloc(P(x.data_ptr()), P(wd.data_ptr()), P(bd.data_ptr()),
                                  P(ad.data_ptr()) if ad is not None else None, None, P(y.data_ptr()),
                                  n, h, w, cin, spec.cout, spec.k, spec.k, spec.stride, spec.pad,
                                  c2d._ACTS[spec.act], c2d._LAYOUTS[layout], c2d._DTYPES[x.dtype],
                                  P(torch.cuda.current_stream().cuda_stream))
    assert rc == c2d.OK, c2d.last_error()


@pytest.mark.parametrize("name", list(VARIANTS))
def test_noalloc_matches_conv2d_fused_on_two_calls(name):
    layout, dtype, act, cin, cout, k, s, p, sizes = VARIANTS[name]
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
    for i, (n, h, w) in enumerate(sizes):
        x, spec, _ = wl.random_conv_case(100 + i, n=n, h=h, w=w, cin=cin, cout=cout, k=k, stride=s, pad=p, act=act,
                                         layout=layout, dtype=dtype)
        xd, wd, bd = x.to(DEV), spec.w.to(DEV), spec.bias.to(DEV)
        ad = spec.alpha.to(DEV) if spec.alpha is not None else None
        oh, ow = c2d.out_dim(h, k, s, p), c2d.out_dim(w, k, s, p)
        shape = (n, oh, ow, cout) if layout == "nhwc" else (n, cout, oh, ow)
        y_na = torch.full(shape, float("nan"), dtype=xd.dtype, device=DEV)
        _noalloc(xd, wd, bd, ad, spec, y_na, layout)
        y_ref = c2d.conv2d_fused(xd, wd, bd, ad, None, stride=s, pad=p, act=act, layout=layout, workspace=ws)
        torch.cuda.synchronize()
        assert bits_equal(y_na, y_ref), f"{name} call {i}: differs from conv2d_fused"
        ref = oracle.conv2d(to64(x), to64(spec.w), to64(spec.bias),
                            to64(spec.alpha) if spec.alpha is not None else None, None, stride=s, pad=p, act=act,
                            layout=layout)
        gate(to64(y_na), ref, dtype, what=f"{name} call {i}")
