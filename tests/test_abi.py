"""The C ABI without a GPU: the library loads, exports what the header declares, and the
host-only entry points validate arguments (CPU only; no kernel is launched)."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

import conv2d_bias_activation_amd as c2d

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv2d_fused.h")

# stand-in device addresses: never dereferenced by the host-only calls
X, Wp, Y, R, A = (ctypes.c_void_p(v << 32) for v in (1, 9, 17, 25, 33))


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(c2d.library_path())
    names = _declared()
    assert {"conv2d_fused", "maxpool3x3s2", "avgpool2x2"} <= names
    for name in names:
        assert hasattr(lib, name), name
    assert names == set(c2d.SIGNATURES)
    assert c2d._load().conv2d_abi_version() == 10


def test_out_dim():
    assert c2d.out_dim(640, 3, 2, 1) == 320
    assert c2d.out_dim(32, 3, 1, 1) == 32
    assert c2d.out_dim(80, 1, 1, 0) == 80
    assert c2d.out_dim(2, 3, 1, 0) == -1
    assert c2d.out_dim(5, 3, 0, 1) == -1


def _check(**kw):
    a = dict(x=X, w=Wp, bias=None, alpha=None, res=None, y=Y, N=1, H=8, W=8, Cin=16, Cout=16,
             kh=3, kw=3, stride=1, pad=1, act=c2d.ACT_RELU, layout=c2d.LAYOUT_NHWC,
             dtype=c2d.DTYPE_BF16)
    a.update(kw)
    return c2d.check_args(a["x"], a["w"], a["bias"], a["alpha"], a["res"], a["y"], a["N"], a["H"],
                          a["W"], a["Cin"], a["Cout"], a["kh"], a["kw"], a["stride"], a["pad"],
                          a["act"], a["layout"], a["dtype"])


def test_check_args_accepts_valid():
    assert _check() == c2d.OK
    assert _check(act=c2d.ACT_PRELU, alpha=A) == c2d.OK
    assert _check(res=R, act=c2d.ACT_RELU | c2d.RES_BEFORE_ACT) == c2d.OK
    assert _check(layout=c2d.LAYOUT_NCHW, dtype=c2d.DTYPE_F16, stride=2) == c2d.OK


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), c2d.EINVAL), (dict(w=None), c2d.EINVAL), (dict(y=None), c2d.EINVAL),
    (dict(N=0), c2d.EINVAL), (dict(Cin=-1), c2d.EINVAL), (dict(stride=3), c2d.EINVAL),
    (dict(stride=0), c2d.EINVAL), (dict(pad=-1), c2d.EINVAL), (dict(kh=11, pad=0), c2d.EINVAL),
    (dict(act=7), c2d.EINVAL), (dict(act=0x200), c2d.EINVAL), (dict(act=c2d.ACT_PRELU), c2d.EINVAL),
    (dict(layout=2), c2d.EINVAL), (dict(dtype=5), c2d.EINVAL), (dict(y=X), c2d.EINVAL),
    (dict(res=Y), c2d.EINVAL), (dict(N=4, H=2048, W=2048, Cin=256), c2d.EUNSUPPORTED),
])
def test_check_args_rejects(kw, code):
    assert _check(**kw) == code
    assert c2d.last_error() != ""


def test_plan_names_a_kernel_for_every_workload_shape():
    bf16, f16, f32 = c2d.DTYPE_BF16, c2d.DTYPE_F16, c2d.DTYPE_F32
    # (shape, expected kernel family): the workload layers and the narrow/stem special cases
    cases = [((1, 32, 32, 16, 32, 3, 3, 1, 1, 1, 0, f32), "igemm_nhwc_vec"),
             ((1, 640, 640, 3, 32, 3, 3, 2, 1, 2, 0, f32), "stem3x3_mfma f32"),
             ((1, 640, 642, 3, 32, 3, 3, 2, 1, 2, 0, f32), "direct_nhwc"),  # W % 4 != 0
             ((1, 640, 640, 3, 32, 3, 3, 2, 1, 2, 0, bf16), "stem3x3_mfma"),
             ((2, 23, 19, 3, 32, 3, 3, 2, 1, 2, 0, bf16), "direct_nhwc"),  # W % 8 != 0
             ((4, 80, 80, 512, 256, 1, 1, 1, 0, 1, 0, bf16), "igemm_nhwc_pipe"),
             ((1, 68, 120, 240, 240, 3, 3, 1, 1, 3, 1, f16), "to_nhwc+hgemm3x3_nchw_out"),
             ((4, 40, 40, 256, 256, 3, 3, 1, 1, 1, 0, bf16), "hgemm3x3_nhwc"),
             ((4, 320, 320, 32, 64, 3, 3, 1, 1, 1, 0, bf16), "halo3x3_nhwc"),
             ((4, 160, 160, 64, 64, 3, 3, 1, 1, 1, 0, bf16), "halo3x3ws_nhwc"),
             ((4, 160, 160, 64, 128, 3, 3, 2, 1, 1, 0, bf16), "igemm_nhwc_pipe"),
             ((4, 80, 80, 128, 256, 3, 3, 2, 1, 1, 0, bf16), "hgemm3x3_nhwc bf16 v6"),
             ((4, 40, 40, 256, 512, 3, 3, 2, 1, 1, 0, bf16), "hgemm3x3_nhwc bf16 v12")]
    for s, family in cases:
        name = c2d.plan(*s)
        assert name.startswith(family), (s, name)
    with pytest.raises(c2d.Conv2dError):
        c2d.plan(1, 8, 8, 4, 4, 3, 3, 5, 1, 0, 0, bf16)


def test_conv_pool_plan_and_argument_checks():
    """Host-only: which kernels conv2d_fused_maxpool3x3s2 picks, and what it rejects
    before launching anything."""
    bf16, f32 = c2d.DTYPE_BF16, c2d.DTYPE_F32
    assert c2d.plan_maxpool(1, 640, 640, 3, 32, 3, 3, 2, 1, 2, 0, bf16) == "stem3x3_mfma bf16 fused with maxpool3x3s2"
    assert c2d.plan_maxpool(4, 320, 320, 32, 64, 3, 3, 1, 1, 1, 0, bf16).endswith("fused with maxpool3x3s2")
    assert c2d.plan_maxpool(4, 160, 160, 64, 64, 3, 3, 1, 1, 1, 0, bf16).endswith("then maxpool3x3s2")
    assert c2d.plan_maxpool(1, 640, 640, 3, 32, 3, 3, 2, 1, 2, 0, f32) == "stem3x3_mfma f32 fused with maxpool3x3s2"
    assert c2d.plan_maxpool(1, 640, 642, 3, 32, 3, 3, 2, 1, 2, 0, f32).startswith("direct_nhwc")
    assert c2d.plan_maxpool(1, 640, 642, 3, 32, 3, 3, 2, 1, 2, 0, f32).endswith("then maxpool3x3s2")
    # channel-first 16-bit layers leave the workspace to the conv output: the general kernel
    assert c2d.plan_maxpool(1, 17, 23, 40, 72, 3, 3, 2, 1, 1, 1, bf16).startswith("igemm_nchw")
    # split-K is turned off for the same reason
    assert "splitk=1" in c2d.plan_maxpool(1, 10, 10, 520, 512, 3, 3, 2, 1, 1, 0, bf16)
    # an unpooled conv output over the 64 MiB workspace
    with pytest.raises(c2d.Conv2dError) as e:
        c2d.plan_maxpool(4, 640, 640, 64, 64, 3, 3, 1, 1, 1, 0, bf16)
    assert e.value.code == c2d.EUNSUPPORTED
    lib = c2d._load()
    P = ctypes.c_void_p
    x, w, y = P(0x100000000), P(0x900000000), P(0x1100000000)
    # a residual-order flag: there is no residual in this entry point
    rc = lib.conv2d_fused_maxpool3x3s2(x, w, None, None, y, 1, 16, 16, 3, 32, 3, 3, 2, 1,
                                       1 | c2d.RES_BEFORE_ACT, 0, bf16, None)
    assert rc == c2d.EINVAL
    # pooled y overlapping x (1x16x16x3 bf16 = 1536 bytes)
    rc = lib.conv2d_fused_maxpool3x3s2(x, w, None, None, P(0x100000000 + 1024), 1, 16, 16, 3, 32, 3, 3, 2, 1,
                                       1, 0, bf16, None)
    assert rc == c2d.EINVAL and "overlaps" in c2d.last_error()
    # y just past x is fine for the check (the conv-size extent is not used)
    assert lib.conv2d_check_args(x, w, None, None, None, P(0x100000000 + 1536), 1, 16, 16, 3, 32, 3, 3, 2, 1,
                                 1, 0, bf16) == c2d.OK
    rc = lib.conv2d_fused_maxpool3x3s2(x, w, None, None, y, 1, 16, 16, 3, 32, 3, 3, 3, 1, 1, 0, bf16, None)
    assert rc == c2d.EINVAL  # stride 3


def test_op_struct_layout_matches_the_header(tmp_path):
    """ctypes' Op has the size and field offsets the C compiler gives struct conv2d_op."""
    src = tmp_path / "layout.c"
    fields = [f for f, _ in c2d.Op._fields_]
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "conv2d_fused.h"\nint main(void) {\n'
                   '  printf("%zu", sizeof(conv2d_op));\n' +
                   "".join(f'  printf(" %zu", offsetof(conv2d_op, {f}));\n' for f in fields) + "  return 0;\n}\n")
    import subprocess
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [ctypes.sizeof(c2d.Op)] + [getattr(c2d.Op, f).offset for f in fields]
    assert got == want


def test_stack_check_names_the_bad_op():
    P = ctypes.c_void_p
    ok = c2d.Op(c2d.OP_CONV, 1 << 32, 9 << 32, None, None, None, 17 << 32, 1, 16, 16, 32, 32, 3, 3, 1, 1, 1)
    pool = c2d.Op(c2d.OP_MAXPOOL, 17 << 32, None, None, None, None, 25 << 32, 1, 16, 16, 32, 32, 0, 0, 0, 0, 0)
    copy = c2d.Op(c2d.OP_COPY, 1 << 32, None, None, None, None, 33 << 32, 1, 16, 16, 32, 0, 0, 0, 0, 0, 0)
    assert c2d.stack_check([ok, pool, copy]) == (c2d.OK, -1)
    bad = c2d.Op(c2d.OP_CONV, 1 << 32, 9 << 32, None, None, None, 17 << 32, 1, 16, 16, 32, 32, 3, 3, 5, 1, 1)
    assert c2d.stack_check([ok, pool, bad, copy]) == (c2d.EINVAL, 2)
    overlap = c2d.Op(c2d.OP_COPY, 1 << 32, None, None, None, None, (1 << 32) + 64, 1, 16, 16, 32, 0, 0, 0, 0, 0, 0)
    assert c2d.stack_check([ok, overlap]) == (c2d.EINVAL, 1)
    unknown = c2d.Op(9, 1 << 32, None, None, None, None, 17 << 32, 1, 1, 1, 1, 0, 0, 0, 0, 0, 0)
    assert c2d.stack_check([unknown])[0] == c2d.EINVAL
    assert c2d.stack_check([]) == (c2d.OK, -1)
    assert c2d.stack_plan([ok, pool, copy], 1) == "maxpool3x3s2"
    assert c2d.stack_plan([ok, pool, copy], 2) == "copy"
    assert c2d.stack_plan([ok, pool, copy], 0) == c2d.plan(1, 16, 16, 32, 32, 3, 3, 1, 1, 1, 0, c2d.DTYPE_BF16)


def test_deconv_plan_and_argument_checks():
    """Host-only: which kernels conv_transpose4x4s2 picks, and what it rejects."""
    bf16, f16, f32 = c2d.DTYPE_BF16, c2d.DTYPE_F16, c2d.DTYPE_F32
    nhwc, nchw = c2d.LAYOUT_NHWC, c2d.LAYOUT_NCHW
    # channel-first, W % 8 == 0: the whole-strip kernel reads the planes itself
    assert c2d.plan_deconv(1, 68, 120, 240, 5, 0, nchw, f16, f32) == \
        "deconv4x4s2_pack+deconv4x4s2_mfma_all_nchw f16 out f32"
    # W % 8 != 0: a channel-last copy first
    assert c2d.plan_deconv(1, 17, 30, 240, 5, 0, nchw, f16, f32) == \
        "deconv4x4s2_pack+to_nhwc+deconv4x4s2_mfma_all_nchw f16 out f32"
    assert c2d.plan_deconv(1, 64, 64, 256, 128, 1, nhwc, bf16) == "deconv4x4s2_pack+deconv4x4s2_mfma_nhwc bf16"
    # past 256 input channels: 64-channel chunks through a double-buffered LDS ring
    assert c2d.plan_deconv(1, 16, 16, 264, 64, 1, nhwc, bf16) == "deconv4x4s2_pack+deconv4x4s2_mfma_nhwc bf16"
    assert c2d.plan_deconv(1, 16, 16, 512, 64, 1, nchw, bf16) == "deconv4x4s2_pack+deconv4x4s2_mfma_nchw bf16"
    # a channel-first input whose channel-last copy does not fit the workspace beside the weights
    assert c2d.plan_deconv(4, 512, 516, 64, 8, 0, nchw, bf16) == "deconv4x4s2_pack+deconv4x4s2_mfma_nchw bf16"
    # the same map with W % 8 == 0 needs no copy
    assert c2d.plan_deconv(4, 512, 512, 64, 8, 0, nchw, bf16) == "deconv4x4s2_pack+deconv4x4s2_mfma_all_nchw bf16"
    assert c2d.plan_deconv(1, 8, 8, 12, 8, 1, nhwc, bf16) == "deconv4x4s2_direct bf16"  # Cin % 8 != 0
    assert c2d.plan_deconv(1, 8, 8, 16, 8, 1, nhwc, f32) == "deconv4x4s2_direct f32"
    # packed weights over a 64 MiB workspace: 16 * 2048 * 1024 bf16 = 64 MiB fits, one more
    # output block or input chunk does not
    assert c2d.plan_deconv(1, 8, 8, 1024, 2048, 0, nhwc, bf16).startswith("deconv4x4s2_pack")
    assert c2d.plan_deconv(1, 8, 8, 1024, 2049, 0, nhwc, bf16).startswith("deconv4x4s2_direct")
    assert c2d.plan_deconv(1, 8, 8, 1032, 2048, 0, nhwc, bf16).startswith("deconv4x4s2_direct")
    for args in [(1, 8, 8, 16, 8, 3, nhwc, bf16, bf16),             # PReLU: alpha is given by the plan stand-in
                 ]:
        assert c2d.plan_deconv(*args)
    bad = [(0, 8, 8, 16, 8, 0, nhwc, bf16, bf16),                     # N = 0
           (1, 8, 8, 16, 8, 0, 2, bf16, bf16),                        # layout
           (1, 8, 8, 16, 8, 0, nhwc, bf16, f16),                      # out dtype neither x's nor fp32
           (1, 8, 8, 16, 8, 1 | c2d.RES_BEFORE_ACT, nhwc, bf16, bf16),  # no residual here
           (1, 8, 8, 16, 8, 9, nhwc, bf16, bf16)]                     # activation code
    for args in bad:
        with pytest.raises(c2d.Conv2dError) as e:
            c2d.plan_deconv(*args)
        assert e.value.code == c2d.EINVAL, args
    with pytest.raises(c2d.Conv2dError) as e:
        c2d.plan_deconv(1, 32768, 32768, 8, 8, 0, nhwc, bf16)
    assert e.value.code == c2d.EUNSUPPORTED
    lib = c2d._load()
    P = ctypes.c_void_p
    x, w, y = P(0x100000000), P(0x900000000), P(0x1100000000)
    # PReLU without slopes, and y overlapping x (1x4x4x16 bf16 = 512 bytes)
    assert lib.conv_transpose4x4s2(x, w, None, None, y, 1, 4, 4, 16, 8, 3, nhwc, bf16, bf16, None) == c2d.EINVAL
    assert lib.conv_transpose4x4s2(x, w, None, None, P(0x100000000 + 256), 1, 4, 4, 16, 8, 0, nhwc, bf16, bf16,
                                   None) == c2d.EINVAL
    assert "overlaps" in c2d.last_error()


def test_resample_ops_in_stack_check():
    """Upsample and concat ops: valid shapes pass the host-only stack check; overlaps,
    a missing second input and bad sizes are named by index."""
    up = c2d.Op(c2d.OP_UPSAMPLE, 1 << 32, None, None, None, None, 9 << 32, 2, 10, 12, 32, 0, 0, 0, 0, 0, 0)
    cat = c2d.Op(c2d.OP_CONCAT, 9 << 32, None, None, None, 17 << 32, 25 << 32, 2, 20, 24, 32, 16, 0, 0, 0, 0, 0)
    upcat = c2d.Op(c2d.OP_UPSAMPLE_CONCAT, 1 << 32, None, None, None, 17 << 32, 33 << 32, 2, 10, 12, 32, 16,
                   0, 0, 0, 0, 0)
    dec = c2d.Op(c2d.OP_DECONV, 1 << 32, 41 << 32, None, None, None, 49 << 32, 2, 10, 12, 32, 16, 4, 4, 2, 1, 1)
    assert c2d.stack_check([up, cat, upcat, dec]) == (c2d.OK, -1)
    assert c2d.stack_plan([up, cat, upcat, dec], 0) == "upsample2x_vec16"
    assert c2d.stack_plan([up, cat, upcat, dec], 1) == "concat_vec16"
    assert c2d.stack_plan([up, cat, upcat, dec], 2) == "upsample2x_concat_vec16"
    assert c2d.stack_plan([up, cat, upcat, dec], 3) == "deconv4x4s2_pack+deconv4x4s2_mfma_nhwc bf16"
    no_b = c2d.Op(c2d.OP_CONCAT, 9 << 32, None, None, None, None, 25 << 32, 2, 20, 24, 32, 16, 0, 0, 0, 0, 0)
    assert c2d.stack_check([up, no_b]) == (c2d.EINVAL, 1)
    zero_cb = c2d.Op(c2d.OP_CONCAT, 9 << 32, None, None, None, 17 << 32, 25 << 32, 2, 20, 24, 32, 0, 0, 0, 0, 0, 0)
    assert c2d.stack_check([zero_cb]) == (c2d.EINVAL, 0)
    # the upsampled output (2x20x24x32 bf16 = 61440 bytes) runs into the next buffer
    clash = c2d.Op(c2d.OP_UPSAMPLE, 1 << 32, None, None, None, None, (1 << 32) + 4096, 2, 10, 12, 32, 0, 0, 0, 0,
                   0, 0)
    assert c2d.stack_check([clash]) == (c2d.EINVAL, 0)
    odd = c2d.Op(c2d.OP_UPSAMPLE, 1 << 32, None, None, None, None, 9 << 32, 2, 10, 12, 5, 0, 0, 0, 0, 0, 0)
    assert c2d.stack_plan([odd], 0) == "upsample2x_scalar"


def test_tune_table_file_round_trip(tmp_path):
    """Host only: tuned-plan records load, save and clear without a device; malformed
    files are rejected whole; a loaded record for another device changes no plan."""
    c2d.tune_clear()
    good = tmp_path / "plans.txt"
    good.write_text("# comment\n"
                    "gfx000:1|4|40|40|256|256|3|3|1|1|0|1|0 2 5 1 0\n"
                    "gfx000:1|4|160|160|64|64|3|3|1|1|0|1|1 4 0 1 4\n")
    before = c2d.plan(4, 40, 40, 256, 256, 3, 3, 1, 1, 1, 0, c2d.DTYPE_BF16)
    assert c2d.tune_load(str(good)) == 2
    assert c2d.plan(4, 40, 40, 256, 256, 3, 3, 1, 1, 1, 0, c2d.DTYPE_BF16) == before
    out = tmp_path / "saved.txt"
    assert c2d.tune_save(str(out)) == 2
    lines = [l for l in out.read_text().splitlines() if not l.startswith("#")]
    assert sorted(lines) == sorted(l for l in good.read_text().splitlines() if not l.startswith("#"))
    for bad in ["gfx000:1|4|40|40 2 5 1 0\n",                             # short key
                "gfx000:1|4|40|40|256|256|3|3|1|1|0|1|0 2 99 1 0\n",      # tile out of range
                "gfx000:1|4|40|40|256|256|3|3|1|1|0|1|0 4 0 1 5\n",       # halo height
                "gfx000:1|4|40|40|256|256|3|3|1|1|0|1|0 2 5\n"]:          # missing fields
        f = tmp_path / "bad.txt"
        f.write_text(bad)
        with pytest.raises(c2d.Conv2dError):
            c2d.tune_load(str(f))
    with pytest.raises(c2d.Conv2dError):
        c2d.tune_load(str(tmp_path / "missing.txt"))
    assert c2d.tune_save(str(out)) == 2  # failed loads added nothing
    c2d.tune_clear()
    assert c2d.tune_save(str(out)) == 0


def test_deconv_pack_sizes_and_checks():
    """Host only: packed sizes, and what the pack and pre-packed calls reject before launching."""
    lib = c2d._load()
    nb = ctypes.c_size_t(0)
    assert lib.conv_transpose4x4s2_packed_bytes(240, 5, c2d.DTYPE_F16, ctypes.byref(nb)) == c2d.OK
    assert nb.value == 16 * 32 * 256 * 2
    assert lib.conv_transpose4x4s2_packed_bytes(256, 128, c2d.DTYPE_BF16, ctypes.byref(nb)) == c2d.OK
    assert nb.value == 16 * 128 * 256 * 2
    assert lib.conv_transpose4x4s2_packed_bytes(16, 16, c2d.DTYPE_F32, ctypes.byref(nb)) == c2d.EUNSUPPORTED
    P = ctypes.c_void_p
    w, wp, x, y = P(1 << 32), P(9 << 32), P(17 << 32), P(25 << 32)
    assert lib.conv_transpose4x4s2_pack(w, wp, 12, 8, c2d.DTYPE_BF16, None) == c2d.EUNSUPPORTED   # Cin % 8
    assert lib.conv_transpose4x4s2_pack(w, P((9 << 32) + 2), 16, 8, c2d.DTYPE_BF16, None) == c2d.EINVAL  # alignment
    assert lib.conv_transpose4x4s2_pack(w, P((1 << 32) + 64), 16, 8, c2d.DTYPE_BF16, None) == c2d.EINVAL  # overlap
    assert lib.conv_transpose4x4s2_prepacked(x, wp, None, None, y, 1, 8, 8, 12, 8, 0, 0, c2d.DTYPE_BF16,
                                             c2d.DTYPE_BF16, None) == c2d.EUNSUPPORTED            # Cin % 8
    assert lib.conv_transpose4x4s2_prepacked(x, wp, None, None, y, 1, 8, 8, 16, 8, 0, 0, c2d.DTYPE_F32,
                                             c2d.DTYPE_F32, None) == c2d.EUNSUPPORTED             # fp32
    assert lib.conv_transpose4x4s2_prepacked(x, P((9 << 32) + 8), None, None, y, 1, 8, 8, 16, 8, 0, 0,
                                             c2d.DTYPE_BF16, c2d.DTYPE_BF16, None) == c2d.EINVAL  # wp alignment


def test_weights_ohwi_flag_checks():
    """Host only: channel-first convs may take OHWI weights (16-bit, Cin % 8 == 0); elsewhere
    the flag is rejected before anything is launched."""
    f16, f32 = c2d.DTYPE_F16, c2d.DTYPE_F32
    nchw, nhwc = c2d.LAYOUT_NCHW, c2d.LAYOUT_NHWC
    act = c2d.ACT_PRELU | c2d.WEIGHTS_OHWI
    assert c2d.plan(1, 68, 120, 240, 240, 3, 3, 1, 1, act, nchw, f16).startswith("x_to_nhwc+hgemm3x3_nchw_out")
    assert c2d.plan(1, 68, 120, 64, 64, 3, 3, 1, 1, act, nchw, f16).startswith("x_to_nhwc+igemm_nhwc_pipe")
    # the input's channel-last copy goes to the workspace: needed for this flag
    assert _check(layout=nchw, dtype=f16, Cin=16, act=c2d.ACT_RELU | c2d.WEIGHTS_OHWI) == c2d.EUNSUPPORTED
    with c2d._planning_workspace(1 << 20):
        assert _check(layout=nchw, dtype=f16, Cin=16, act=c2d.ACT_RELU | c2d.WEIGHTS_OHWI) == c2d.OK
    assert _check(layout=nhwc, act=c2d.ACT_RELU | c2d.WEIGHTS_OHWI) == c2d.EINVAL            # channel-last layer
    assert _check(layout=nchw, dtype=f32, act=c2d.ACT_RELU | c2d.WEIGHTS_OHWI) == c2d.EUNSUPPORTED
    assert _check(layout=nchw, dtype=f16, Cin=12, act=c2d.ACT_RELU | c2d.WEIGHTS_OHWI) == c2d.EUNSUPPORTED
    with pytest.raises(c2d.Conv2dError):
        c2d.plan_maxpool(1, 64, 64, 16, 16, 3, 3, 1, 1, c2d.ACT_RELU | c2d.WEIGHTS_OHWI, nchw, f16)
    lib = c2d._load()
    P = ctypes.c_void_p
    assert lib.conv2d_weights_to_ohwi(P(1 << 32), P((1 << 32) + 64), 8, 8, 3, 3, f16, None) == c2d.EINVAL
    assert lib.conv2d_weights_to_ohwi(P(1 << 32), P(9 << 32), 8, 8, 3, 3, f32, None) == c2d.EUNSUPPORTED


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="needs a machine without a GPU: the stand-in pointers would be launched on a real device")
def test_no_device_returns_ehip_not_a_crash():
    """Without a GPU, every launching entry point validates, then reports CONV2D_EHIP with a
    message (the library loads and fails cleanly)."""
    lib = c2d._load()
    P = ctypes.c_void_p
    G = 1 << 32
    bf16 = c2d.DTYPE_BF16
    calls = {
        "conv2d_fused": lambda: lib.conv2d_fused(P(G), P(9 * G), None, None, None, P(17 * G), 1, 8, 8, 16, 16, 3, 3,
                                                 1, 1, 1, 0, bf16, None),
        "maxpool3x3s2": lambda: lib.maxpool3x3s2(P(G), P(17 * G), 1, 8, 8, 16, 0, bf16, None),
        "avgpool2x2": lambda: lib.avgpool2x2(P(G), P(17 * G), 1, 8, 8, 16, 0, bf16, None),
        "conv_transpose4x4s2": lambda: lib.conv_transpose4x4s2(P(G), P(9 * G), None, None, P(17 * G), 1, 8, 8, 16, 8,
                                                               0, 0, bf16, bf16, None),
        "upsample2x_concat": lambda: lib.upsample2x_concat(P(G), P(9 * G), P(17 * G), 1, 4, 4, 8, 8, 0, bf16, None),
    }
    for name, call in calls.items():
        assert call() == c2d.EHIP, name
        assert "device" in c2d.last_error(), name
    op = c2d.Op(c2d.OP_CONV, G, 9 * G, None, None, None, 17 * G, 1, 8, 8, 16, 16, 3, 3, 1, 1, 1)
    arr = (c2d.Op * 1)(op)
    h = ctypes.c_void_p()
    assert lib.conv2d_stack_graph_create(arr, 1, 0, bf16, ctypes.byref(h)) == c2d.EHIP and not h.value
    assert lib.conv2d_stack_run(arr, 1, 0, bf16, None) == c2d.EHIP
    with pytest.raises(c2d.Conv2dError) as e:
        c2d.tune(1, 8, 8, 16, 16, 3, 3, 1, 1, "relu", reps=3)
    assert e.value.code == c2d.EHIP


def test_channel_first_chain_links():
    """Host only: consecutive channel-first convs with channel-last weights, each reading
    the previous one's output, are linked (the producer also writes a channel-last copy
    that the consumer reads); a producer with a residual, channel-first weights or a
    consumer reading another buffer breaks the link."""
    G = 1 << 32
    f16 = c2d.DTYPE_F16
    act = c2d._ACTS["prelu"] | c2d.WEIGHTS_OHWI
    x, y0, y1, y2, w, al, b = G, 3 * G, 5 * G, 7 * G, 9 * G, 10 * G, 11 * G

    def conv(src, dst, res=None, a=act):
        return c2d.Op(c2d.OP_CONV, src, w, b, al, res, dst, 1, 68, 120, 240, 240, 3, 3, 1, 1, a)

    def names(ops):
        return [c2d.stack_plan(ops, i, layout="nchw", dtype=f16) for i in range(len(ops))]

    n = names([conv(x, y0), conv(y0, y1), conv(y1, y2, res=x)])
    assert n[0].startswith("x_to_nhwc+") and n[0].endswith(" +y_nhwc"), n
    assert n[1].startswith("chained+") and n[1].endswith(" +y_nhwc"), n
    assert n[2].startswith("chained+") and not n[2].endswith(" +y_nhwc"), n
    # the producer adds a residual: its channel-last copy would differ from y
    n = names([conv(x, y0, res=y2), conv(y0, y1)])
    assert n[0].startswith("x_to_nhwc+") and not n[0].endswith(" +y_nhwc") and n[1].startswith("x_to_nhwc+"), n
    # channel-first weights: no link
    plain = c2d._ACTS["prelu"]
    n = names([conv(x, y0, a=plain), conv(y0, y1, a=plain)])
    assert all(k.startswith("to_nhwc+") and not k.endswith(" +y_nhwc") for k in n), n
    # the next conv reads another buffer
    n = names([conv(x, y0), conv(y1, y2)])
    assert not n[0].endswith(" +y_nhwc") and n[1].startswith("x_to_nhwc+"), n


def test_workspace_registration_and_sizes():
    """Host only: the caller-owned workspace. Registration checks its arguments; the size
    queries report what the preferred variants write; planning without a workspace (or
    with one too small) picks variants that need none, and rejects only what has none."""
    lib = c2d._load()
    P = ctypes.c_void_p
    bf16, f16 = c2d.DTYPE_BF16, c2d.DTYPE_F16
    nhwc, nchw = c2d.LAYOUT_NHWC, c2d.LAYOUT_NCHW
    assert lib.conv2d_set_workspace(P(0x4000000010), 1 << 20) == c2d.EINVAL   # not 256-byte aligned
    assert lib.conv2d_set_workspace(None, 4096) == c2d.EINVAL                 # null with a size
    assert lib.conv2d_set_workspace(None, 0) == c2d.OK
    c2d.tune_clear()
    # a deep-K strided layer with few tiles whose Cin (520) the halo-tile GEMM does not
    # take: split-K in three, 3 * M * Cout fp32 partial sums
    deep = (4, 20, 20, 520, 512, 3, 3, 2, 1, 1, nhwc, bf16)
    assert "splitk=3" in c2d.plan(*deep)
    assert c2d.workspace_size(*deep) == 3 * 400 * 512 * 4
    assert "splitk=1" in c2d.plan(*deep, workspace_bytes=0)
    assert "splitk=1" in c2d.plan(*deep, workspace_bytes=3 * 400 * 512 * 4 - 1)
    # the same layer at stride 1: the halo-tile GEMM kernel, which needs no workspace
    assert c2d.plan(4, 20, 20, 512, 512, 3, 3, 1, 1, 1, nhwc, bf16).startswith("hgemmws3x3_nhwc")
    assert c2d.workspace_size(4, 20, 20, 512, 512, 3, 3, 1, 1, 1, nhwc, bf16) == 0
    # a channel-first 16-bit layer: channel-last copies of x and w (each rounded to 256 bytes)
    ifn = (1, 68, 120, 240, 240, 3, 3, 1, 1, 3, nchw, f16)
    xb, wb = 68 * 120 * 240 * 2, 240 * 9 * 240 * 2
    assert c2d.workspace_size(*ifn) == (xb + 255) // 256 * 256 + (wb + 255) // 256 * 256
    assert c2d.plan(*ifn).startswith("to_nhwc+")
    assert c2d.plan(*ifn, workspace_bytes=0).startswith("igemm_nchw")
    ohwi = ifn[:9] + (3 | c2d.WEIGHTS_OHWI,) + ifn[10:]
    assert c2d.workspace_size(*ohwi) == (xb + 255) // 256 * 256
    with pytest.raises(c2d.Conv2dError) as e:
        c2d.plan(*ohwi, workspace_bytes=0)
    assert e.value.code == c2d.EUNSUPPORTED and "workspace" in str(e.value)
    # layers on kernels without scratch
    assert c2d.workspace_size(4, 160, 160, 64, 64, 3, 3, 1, 1, 1, nhwc, bf16) == 0
    assert c2d.workspace_size(1, 640, 640, 3, 32, 3, 3, 2, 1, 2, nhwc, bf16) == 0
    # conv + max pool: the fused kernels need none, the two-kernel form needs the
    # unpooled output and has no other variant
    assert c2d.plan_maxpool(4, 320, 320, 32, 64, 3, 3, 1, 1, 1, 0, bf16, workspace_bytes=0).endswith(
        "fused with maxpool3x3s2")
    with pytest.raises(c2d.Conv2dError) as e:
        c2d.plan_maxpool(1, 64, 64, 64, 64, 3, 3, 1, 1, 1, 0, bf16, workspace_bytes=64 * 64 * 64 * 2 - 256)
    assert e.value.code == c2d.EUNSUPPORTED
    assert c2d.plan_maxpool(1, 64, 64, 64, 64, 3, 3, 1, 1, 1, 0, bf16,
                            workspace_bytes=64 * 64 * 64 * 2).endswith("then maxpool3x3s2")
    # transposed conv: the matrix cores need the packed weights in the workspace
    assert c2d.plan_deconv(1, 64, 64, 256, 128, 1, nhwc, bf16, workspace_bytes=0) == "deconv4x4s2_direct bf16"
    assert c2d.plan_deconv(1, 64, 64, 256, 128, 1, nhwc, bf16,
                           workspace_bytes=16 * 128 * 256 * 2).startswith("deconv4x4s2_pack+")
    # a stack: the largest op's need, or both halves of a chain of channel-first convs
    G = 1 << 32
    act = c2d._ACTS["prelu"] | c2d.WEIGHTS_OHWI
    chain = [c2d.Op(c2d.OP_CONV, s, 9 * G, 11 * G, 10 * G, None, d, 1, 68, 120, 240, 240, 3, 3, 1, 1, act)
             for s, d in ((G, 3 * G), (3 * G, 5 * G))]
    need = c2d.stack_workspace_size(chain, layout="nchw", dtype=f16)
    assert need == 2 * ((xb + 255) // 256 * 256)
    assert c2d.stack_plan(chain, 1, layout="nchw", dtype=f16).startswith("chained+")
    assert c2d.stack_plan(chain, 1, layout="nchw", dtype=f16, workspace_bytes=need - 512).startswith("x_to_nhwc+")
    with pytest.raises(c2d.Conv2dError):
        c2d.stack_plan(chain, 1, layout="nchw", dtype=f16, workspace_bytes=0)
    assert lib.conv2d_set_workspace(None, 0) == c2d.OK


@pytest.mark.parametrize("what", ["w", "bias", "alpha"])
def test_output_may_not_overlap_weights_bias_or_slopes(what):
    """y overlapping w, bias or alpha is rejected before launch (other workgroups still read
    them while one stores y)."""
    inside = ctypes.c_void_p((17 << 32) + 64)
    kw = dict(act=c2d.ACT_PRELU, alpha=A, bias=ctypes.c_void_p(41 << 32))
    kw[what] = inside
    assert _check(**kw) == c2d.EINVAL
    assert "overlaps " + what in c2d.last_error()
    assert _check(act=c2d.ACT_PRELU, alpha=A, bias=ctypes.c_void_p(41 << 32)) == c2d.OK


def test_noalloc_rejects_layers_over_its_static_scratch():
    """Host only: conv2d_fused_noalloc refuses, before touching any device, a layer whose
    kernels need more scratch than its 16 MiB static array (here the channel-last copies
    of a channel-first 128-channel 256x256 f16 input and its weights)."""
    lib = c2d._load()
    P = ctypes.c_void_p
    G = 1 << 32
    assert c2d.workspace_size(1, 256, 256, 128, 64, 3, 3, 1, 1, 1, c2d.LAYOUT_NCHW, c2d.DTYPE_F16) > 16 << 20
    rc = lib.conv2d_fused_noalloc(P(G), P(9 * G), None, None, None, P(17 * G), 1, 256, 256, 128, 64, 3, 3, 1, 1, 1,
                                  c2d.LAYOUT_NCHW, c2d.DTYPE_F16, None)
    assert rc == c2d.EUNSUPPORTED and "static scratch" in c2d.last_error()
    # argument errors come first, as for conv2d_fused
    rc = lib.conv2d_fused_noalloc(P(G), P(9 * G), None, None, None, P(17 * G), 1, 8, 8, 16, 16, 3, 3, 3, 1, 1,
                                  c2d.LAYOUT_NHWC, c2d.DTYPE_BF16, None)
    assert rc == c2d.EINVAL
