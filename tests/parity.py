"""Parity gates between the GPU library and the CPU oracle (shared by the GPU tests).

Floating-point gates (the layer's stated acceptance bar):
* fp32 storage: max|y - ref| <= 1e-4 * max|ref|;
* bf16/f16 storage (fp32 accumulation): cosine(y, ref) >= 0.9999 and
  max|y - ref| / max|ref| <= 2e-2.
On top of that, an element-wise bound catches a few wrong outputs that the
aggregate gates could average away: |y - ref| <= 2^-p |ref| + atol, with
p = 8 (bf16, 8 significant bits: one rounding costs at most 2^-9), 10 (f16) or
16 (f32), and atol = 2e-3 * max|ref| for 16-bit storage (1e-4 for fp32), which
covers fp32 accumulation-order differences over K <= 4608 terms.
"""
import numpy as np
import torch

TOL_BITS = {"f32": 16, "bf16": 8, "f16": 10}
DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def gate(got, ref, dtype, what="", elementwise=True):
    """Assert the conv gate; returns a dict of the measured figures.

    ``elementwise=False`` keeps only the aggregate gates: for a chain of layers
    compared end to end, where one-ulp rounding differences of intermediate maps
    propagate and the per-output bound of a single layer does not apply.
    """
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    scale = float(np.max(np.abs(ref)))
    err = np.abs(got - ref)
    maxerr = float(np.max(err))
    rel = maxerr / scale if scale > 0 else maxerr
    den = float(np.linalg.norm(got) * np.linalg.norm(ref))
    cos = float(np.dot(got, ref) / den) if den > 0 else (1.0 if maxerr == 0 else 0.0)
    atol = (1e-4 if dtype == "f32" else 2e-3) * scale
    bound = np.ldexp(np.abs(ref), -TOL_BITS[dtype]) + atol
    bad = int(np.count_nonzero(err > bound))
    info = dict(max_err=maxerr, max_rel=rel, cos=cos, bad=bad, n=got.size)
    if dtype == "f32":
        assert maxerr <= 1e-4 * scale, f"{what}: fp32 max err {maxerr} > 1e-4*{scale}"
    else:
        assert cos >= 0.9999, f"{what}: cosine {cos}"
        assert rel <= 2e-2, f"{what}: max rel err {rel}"
    if elementwise:
        assert bad == 0, f"{what}: {bad} of {got.size} outputs outside the element-wise bound"
    return info


def bits_equal(a, b):
    """Bit-exact comparison of two same-dtype tensors (CPU)."""
    a = a.detach().cpu().contiguous()
    b = b.detach().cpu().contiguous()
    assert a.dtype == b.dtype and a.shape == b.shape
    iv = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.float16: torch.int16}
    return torch.equal(a.view(iv[a.dtype]), b.view(iv[b.dtype]))


def quantized_tensor(values64, dtype):
    """fp64 values already representable in ``dtype`` -> CPU tensor of that dtype."""
    t = torch.from_numpy(np.ascontiguousarray(values64, dtype=np.float64))
    out = t.to(DTYPES[dtype])
    assert np.array_equal(out.double().numpy(), values64), "value not representable"
    return out
