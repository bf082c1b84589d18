"""Plant plausible mistakes in copies of the oracle (CPU only) and check the pins catch them.

Each mutant is the oracle's C source with one textual change, compiled into a
temporary library. The pins in ``oracle_pins`` run against it; at least one
must fail. The real oracle source is never modified.
"""
import contextlib
import ctypes
import os
import subprocess

import pytest

import oracle
import oracle_pins as pins
from oracle import build as obuild

MUTANTS = {
    "flipped_kernel": ("acc += xc[(size_t)iy * W + ix] * wc[ky * kw + kx];",
                       "acc += xc[(size_t)iy * W + ix] * wc[(kh - 1 - ky) * kw + (kw - 1 - kx)];"),
    "transposed_taps": ("wc[ky * kw + kx]", "wc[kx * kh + ky]"),
    "pad_sign_rows": ("int iy = oh * stride + ky - pad;", "int iy = oh * stride + ky + pad;"),
    "stride_dropped_cols": ("int ix = ow * stride + kx - pad;", "int ix = ow + kx - pad;"),
    "last_channel_dropped": ("for (int ci = 0; ci < Cin; ++ci) {",
                             "for (int ci = 0; ci < Cin - 1; ++ci) {"),
    "batch_index_dropped": ("const double *xc = x + ((size_t)n * Cin + ci)",
                            "const double *xc = x + ((size_t)0 * Cin + ci)"),
    "bias_dropped": ("double v = acc + (bias ? bias[co] : 0.0);", "double v = acc;"),
    "residual_order_swapped": ("if (act_flags & ORACLE_RES_BEFORE_ACT) {",
                               "if (!(act_flags & ORACLE_RES_BEFORE_ACT)) {"),
    "prelu_alpha_not_per_channel": ("double a = alpha ? alpha[co] : 0.0;",
                                    "double a = alpha ? alpha[0] : 0.0;"),
    "silu_sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "relu_leaky": ("return v > 0.0 ? v : 0.0;", "return v > 0.0 ? v : 0.01 * v;"),
    "out_dim_short": ("return span / stride + 1;", "return span / stride;"),
    "maxpool_no_pad": ("int iy = 2 * oh + dy - 1;", "int iy = 2 * oh + dy;"),
    "maxpool_zero_init": ("double best = -INFINITY;", "double best = 0.0;"),
    "maxpool_skips_last_col": ("for (int dx = 0; dx < 3; ++dx) {", "for (int dx = 0; dx < 2; ++dx) {"),
    "maxpool_nan_wins": ("if (v > best) best = v;", "if (!(v <= best)) best = v;"),
    "maxpool_last_of_equal": ("if (v > best) best = v;", "if (v >= best) best = v;"),
    "avgpool_order": ("float s = t[0] + t[1];\n                s = s + t[W];\n"
                      "                s = s + t[W + 1];",
                      "float s = t[0] + t[W + 1];\n                s = s + t[1];\n"
                      "                s = s + t[W];"),
    "avgpool_scale": ("s * 0.25f", "s * 0.5f"),
    "avgpool_row_offset": ("s = s + t[W];", "s = s + t[1];"),
    "deconv_pad_sign": ("const int ty = oy + 1 - ky;", "const int ty = oy - 1 - ky;"),
    "deconv_flipped_taps": ("acc += xc[(size_t)(ty / 2) * W + tx / 2] * wc[ky * 4 + kx];",
                            "acc += xc[(size_t)(ty / 2) * W + tx / 2] * wc[(3 - ky) * 4 + (3 - kx)];"),
    "deconv_weight_transposed": ("const double *wc = w + ((size_t)ci * Cout + co) * 16;",
                                 "const double *wc = w + ((size_t)co * Cin + ci) * 16;"),
    "deconv_odd_taps_kept": ("if (tx < 0 || (tx % 2) != 0 || tx / 2 >= W) continue;",
                             "if (tx < 0 || tx / 2 >= W) continue;"),
    "deconv_bias_dropped": ("const double v = acc + (bias ? bias[co] : 0.0);", "const double v = acc;"),
}


@contextlib.contextmanager
def _mutant_oracle(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    cpath = os.path.join(tmp_path, f"{name}.c")
    lpath = os.path.join(tmp_path, f"lib{name}.so")
    with open(cpath, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", *obuild.CFLAGS, cpath, "-o", lpath, "-lm"], check=True)
    saved = oracle._load()
    oracle._lib = oracle._bind(ctypes.CDLL(lpath))
    try:
        yield
    finally:
        oracle._lib = saved


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    caught = []
    with _mutant_oracle(str(tmp_path), name, old, new):
        for pin in pins.ALL_PINS:
            try:
                pin(oracle)
            except (AssertionError, ValueError) as e:
                caught.append((pin.__name__, str(e)[:80]))
                break
    assert caught, f"no pin caught the planted mistake {name!r}"
