/*
 * conv2d_fused.h - C ABI of the fused 2-D convolution library for MI355X (gfx950).
 *
 * The layer is the one the inferencelayer page (docs.rs, src/rtdetr_gpu.rs:
 * `conv()`, `IM2COL_SRC`, `ADDACT_SRC`, `MAXPOOL_SRC`, `AVGPOOL_SRC`) and the
 * framecast page (package/rt.js: `wgslConv`) state: a k x k zero-padded
 * cross-correlation lowered to a GEMM over im2col patches, with bias, an
 * activation and an optional residual add applied in the GEMM epilogue, plus
 * the 3x3/s2/p1 max pool and the 2x2/s2 average pool that sit beside it.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller (for example
 *    torch tensors' data_ptr()). The library never frees them, never keeps them
 *    after the call returns, and writes only the output tensor.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues kernels on that stream and returns; it never synchronises. A
 *    device fault therefore surfaces at the caller's next synchronisation.
 *  - Arguments are validated on the host before anything is launched: a call
 *    that returns an error has written nothing.
 *  - Return value: CONV2D_OK (0) or a negative CONV2D_E* code; the message of
 *    the last error on the calling thread is returned by conv2d_last_error().
 *  - Tensors are dense and contiguous. Every tensor must hold fewer than 2^31
 *    elements (CONV2D_EUNSUPPORTED otherwise).
 *  - The output may not overlap any input: x, w, bias, alpha or the residual
 *    (CONV2D_EINVAL).
 *  - The library allocates no device memory (conv2d_tune aside, which allocates and
 *    frees its own timing buffers). Some kernel variants need device scratch memory
 *    (split-K fp32 partial sums, channel-last copies of a channel-first layer's input
 *    and weights, the unpooled output of a conv + max pool that runs as two kernels,
 *    the repacked weights of a transposed conv). It comes from a caller-owned
 *    WORKSPACE registered with conv2d_set_workspace for the calling thread and the
 *    current device; it replaces the library-reserved scratch arena that the
 *    rlx-wgpu page sizes with `compute_scratch_bytes`. Calls plan their kernels for
 *    the workspace registered when they are made: without one, or with one too small,
 *    they take a variant that needs none (no split-K; channel-first layers on the
 *    general kernel; the transposed conv on the vector ALUs) and return
 *    CONV2D_EUNSUPPORTED only where no such variant exists (said per call below).
 *    conv2d_workspace_size and conv2d_stack_workspace_size report how much the
 *    preferred variants use. Two calls that may run at the same time (on two streams)
 *    must not share a workspace; a call reads and writes its workspace only on its own
 *    stream, in its own launches, so calls queued on one stream may share one.
 *  - Other state kept between calls: the last-error message (per thread), the
 *    compute-unit count and arch name of each device (queried once), the registered
 *    workspaces (per thread and device) and the tuned-plan table (conv2d_tune).
 */
#ifndef CONV2D_FUSED_H
#define CONV2D_FUSED_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Memory layouts. NHWC: x [N][H][W][Cin], w [Cout][kh][kw][Cin] (OHWI), residual and
 * y [N][OH][OW][Cout]. NCHW: x [N][Cin][H][W], w [Cout][Cin][kh][kw] (OIHW), residual
 * and y [N][Cout][OH][OW]. */
#define CONV2D_LAYOUT_NHWC 0
#define CONV2D_LAYOUT_NCHW 1

/* Storage types of x, w, residual and y. Arithmetic is always fp32 accumulate;
 * results are rounded to the storage type to nearest-even. bias and alpha are
 * always fp32 (framecast `wgslConv` keeps them fp32 under f16 storage). */
#define CONV2D_DTYPE_F32 0
#define CONV2D_DTYPE_BF16 1
#define CONV2D_DTYPE_F16 2

/* Activation, in the low byte of `act`:
 *   NONE  v
 *   RELU  max(v, 0)                      (inferencelayer `ADDACT_SRC`)
 *   SILU  v / (1 + exp(-v))              (inferencelayer `ADDACT_SRC`,
 *                                         rlx-wgpu `apply_activation_host`)
 *   PRELU v >= 0 ? v : alpha[co] * v     (framecast `wgslConv`, one slope per
 *                                         output channel)
 * OR-ed with CONV2D_RES_BEFORE_ACT, a residual is added before the activation
 * (y = act(conv + bias + r), the ResNet block sum that inferencelayer's
 * `encoder_maps` sends through `addact(.., relu)`); without it a residual is
 * added after the activation (y = act(conv + bias) + r, framecast `wgslConv`). */
#define CONV2D_ACT_NONE 0
#define CONV2D_ACT_RELU 1
#define CONV2D_ACT_SILU 2
#define CONV2D_ACT_PRELU 3
#define CONV2D_RES_BEFORE_ACT 0x100

/* OR-ed into `act` of a channel-first (CONV2D_LAYOUT_NCHW) conv: the weights are given
 * in OHWI order [Cout][kh][kw][Cin] instead of OIHW, e.g. converted once at model load by
 * conv2d_weights_to_ohwi (weight residency: such a layer then copies only its input to
 * channel-last form per call). Only for 16-bit layers with Cin % 8 == 0 whose input copy
 * fits the workspace (CONV2D_EUNSUPPORTED otherwise); not accepted by
 * conv2d_fused_maxpool3x3s2 (CONV2D_EINVAL). */
#define CONV2D_WEIGHTS_OHWI 0x200

/* OR-ed into `act` of a stack's CONV2D_OP_CONV op (not accepted by the single calls): the
 * op's output is only an intermediate read by the next op, so the stack need not store
 * it. A 16-bit channel-last stem conv (Cin 3 -> Cout 32, 3x3, stride 2, pad 1, W % 8 == 0)
 * so marked, followed by the 3x3 stride-1 pad-1 conv of its output (Cout <= 32, Cout % 8
 * == 0, no residual; the second conv of inferencelayer's `encoder_maps` stem) then runs as
 * one kernel that writes only the second output, bit-identical to the two launches; y of
 * the marked op is left as it was. Any other marked op runs and stores its output as
 * usual. */
#define CONV2D_Y_TRANSIENT 0x400

/* Status codes. */
#define CONV2D_OK 0
#define CONV2D_EINVAL (-1)      /* bad argument: null required pointer, size <= 0, stride
                                   not 1 or 2, pad < 0, no output fits, unknown code,
                                   PRELU without alpha, output overlapping an input */
#define CONV2D_EUNSUPPORTED (-2) /* valid but not handled (a tensor of 2^31 or more
                                   elements) */
#define CONV2D_EHIP (-3)        /* the HIP runtime failed (no device, launch failure) */

/*
 * y = epilogue(conv(x, w)) for one layer.
 *
 * Source: inferencelayer page, `conv()` (output size (h + 2*pad - kh)/stride + 1,
 * im2col in (dy, dx, c) order with zero fill, GEMM with bias + activation in the
 * epilogue); framecast page, `wgslConv` (bias, per-channel PReLU, residual added
 * after the activation).
 *
 * x        [N,H,W,Cin] or [N,Cin,H,W] in `dtype` (required)
 * w        [Cout,kh,kw,Cin] or [Cout,Cin,kh,kw] in `dtype` (required)
 * bias     fp32 [Cout], or NULL for no bias
 * alpha    fp32 [Cout]; required when the activation is PRELU, ignored otherwise
 * residual y's shape, layout and dtype, or NULL for none
 * y        [N,OH,OW,Cout] or [N,Cout,OH,OW] in `dtype`, OH = (H + 2*pad - kh)/stride
 *          + 1 (floor), OW likewise (required)
 * stride   1 or 2; pad >= 0 (zero padding on all four sides); kh, kw >= 1
 * act      CONV2D_ACT_* optionally OR-ed with CONV2D_RES_BEFORE_ACT
 * layout   CONV2D_LAYOUT_*; dtype CONV2D_DTYPE_*
 * stream   hipStream_t or NULL
 *
 * Accumulation is fp32 in any order; the result is rounded once to `dtype`.
 * With a workspace (conv2d_set_workspace) of the size conv2d_workspace_size reports,
 * layers with a deep K and few output tiles may run as split-K (fp32 partial sums of
 * K slices in the workspace, added in slice order by a second kernel that applies the
 * epilogue), and 16-bit channel-first layers with Cin % 8 == 0 are first copied to
 * channel-last form there. Without it they run as one kernel on the caller's tensors;
 * the result differs only by fp32 accumulation order.
 */
int conv2d_fused(const void *x, const void *w, const float *bias, const float *alpha,
                 const void *residual, void *y, int N, int H, int W, int Cin, int Cout, int kh,
                 int kw, int stride, int pad, int act, int layout, int dtype, void *stream);

/*
 * conv2d_fused for callers that cannot allocate device memory or register a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, layouts and results, with the scratch of the
 * kernel variant conv2d_fused takes when given all the workspace it wants (split-K
 * partial sums, channel-last copies of a channel-first layer) taken from a static
 * device array inside the library: 16 MiB, one copy per GPU the library runs on, held
 * until the process ends. Its device address is looked up once per device on the first
 * call there; nothing is allocated, by this call or later ones.
 *
 * The output is the same as conv2d_fused's with a workspace of at least
 * conv2d_workspace_size bytes (the same kernels). A layer whose variant needs more than
 * 16 MiB of scratch returns CONV2D_EUNSUPPORTED with a message and launches nothing.
 * Every call on one GPU shares that GPU's array and leaves it holding its own data
 * (each call writes all the scratch it reads; none needs it zeroed), so calls that may
 * run at the same time on one GPU (two streams, two threads) race: serialise them, or
 * use conv2d_fused with a workspace per stream. Errors as conv2d_fused.
 */
int conv2d_fused_noalloc(const void *x, const void *w, const float *bias, const float *alpha,
                         const void *residual, void *y, int N, int H, int W, int Cin, int Cout, int kh,
                         int kw, int stride, int pad, int act, int layout, int dtype, void *stream);

/*
 * 3x3 max pool, stride 2, padding 1 with -infinity (out-of-range taps never win).
 * Source: inferencelayer page, `MAXPOOL_SRC` and the max-pool step of
 * `encoder_maps` (output (h + 2 - 3)/2 + 1).
 *
 * x [N,H,W,C] or [N,C,H,W] in `dtype`; y [N,OH,OW,C] or [N,C,OH,OW] with
 * OH = (H - 1)/2 + 1 (floor), OW likewise. The result is bit-exactly one of the
 * input values: the page's `v > best` from -infinity over the taps in row-major order,
 * so the first largest is kept (of -0 and +0, the first), NaN inputs are skipped, and a
 * window of NaN alone gives -infinity.
 */
int maxpool3x3s2(const void *x, void *y, int N, int H, int W, int C, int layout, int dtype,
                 void *stream);

/*
 * y = maxpool3x3s2(conv2d_fused(x, w, bias, alpha, no residual)): the image stem
 * conv and the max pool after it, with only the pooled map written.
 * Source: inferencelayer page, `encoder_maps` (the stem conv followed by the 3x3
 * stride-2 max pool) with `conv()` and `MAXPOOL_SRC` as above.
 *
 * Arguments as conv2d_fused (no residual; act may not carry CONV2D_RES_BEFORE_ACT),
 * except y: [N,PH,PW,Cout] or [N,Cout,PH,PW] in `dtype` with PH = (OH - 1)/2 + 1,
 * PW = (OW - 1)/2 + 1 and OH, OW the conv's output size. y may not overlap x.
 *
 * The max is taken on rounded values (rounding is monotone, so rounding first and
 * pooling after gives the same bits), skipping NaN as maxpool3x3s2 does, so the result
 * equals maxpool3x3s2(conv2d_fused(...)) bit for bit. Channel-last 16-bit 3-channel
 * 3x3 pad-1 convs (Cout <= 64, Cout % 8 == 0, W % 8 == 0, W <= 3000, x and y 16-byte
 * aligned) and channel-last 16-bit 3x3 stride-1 pad-1 convs with Cin 16 or 32 and
 * Cout <= 64 run as one kernel that keeps the conv output on chip. Any other shape
 * runs the conv into the workspace and then the pool kernel; that needs a workspace
 * of N*OH*OW*Cout elements of `dtype` (rounded up to 256 bytes;
 * CONV2D_EUNSUPPORTED otherwise).
 */
int conv2d_fused_maxpool3x3s2(const void *x, const void *w, const float *bias, const float *alpha,
                              void *y, int N, int H, int W, int Cin, int Cout, int kh, int kw,
                              int stride, int pad, int act, int layout, int dtype, void *stream);

/* Host-only: the kernel variants conv2d_fused_maxpool3x3s2 would launch for this
 * shape (as conv2d_plan), e.g. "stem3x3_mfma bf16 fused with maxpool3x3s2". */
int conv2d_fused_maxpool_plan(int N, int H, int W, int Cin, int Cout, int kh, int kw, int stride,
                              int pad, int act, int layout, int dtype, char *buf, int cap);

/*
 * 2x2 average pool, stride 2, no padding.
 * Source: inferencelayer page, `AVGPOOL_SRC` (the sum of the four taps taken
 * left to right, then times 0.25) and the ResNet-D shortcut of `encoder_maps`.
 *
 * x [N,H,W,C] or [N,C,H,W] in `dtype` (H, W >= 2); y [N,H/2,W/2,C] or
 * [N,C,H/2,W/2] (floor: an odd last row or column is dropped). Computed in fp32
 * as ((x00 + x01) + x10) + x11, times 0.25, then rounded once to `dtype`, so the
 * result is bit-exact and reproducible.
 */
int avgpool2x2(const void *x, void *y, int N, int H, int W, int C, int layout, int dtype,
               void *stream);

/*
 * Transposed convolution (ConvTranspose2d), 4x4 kernel, stride 2, padding 1: the layer
 * that ends an IFNet block (framecast page, `wgslDeconv`, the 4x4 stride-2 deconv from
 * the stride-16 map to the stride-8 map). Input pixel (iy, ix) with tap (ky, kx) adds
 * x[ci] * w[ci][co][ky][kx] to output (2*iy - 1 + ky, 2*ix - 1 + kx) when that lies in
 * the 2H x 2W output; then bias[co] and the activation are applied (no residual).
 *
 * x      [N,H,W,Cin] or [N,Cin,H,W] in `dtype` (required)
 * w      [Cin][Cout][4][4] in `dtype`, the transposed conv's own layout in both
 *        layouts (required)
 * bias   fp32 [Cout] or NULL; alpha fp32 [Cout], required when act is PRELU
 * y      [N,2H,2W,Cout] or [N,Cout,2H,2W] in `out_dtype` (required; may not overlap x
 *        or w)
 * act    CONV2D_ACT_* (CONV2D_RES_BEFORE_ACT is rejected)
 * out_dtype  `dtype`, or CONV2D_DTYPE_F32 for an fp32 output from 16-bit inputs
 *        (framecast keeps the deconv output in fp32 under f16 storage)
 *
 * Accumulation is fp32 in any order, rounded once to out_dtype. 16-bit inputs with
 * Cin % 8 == 0 (channel-last x 16-byte aligned) run on the matrix cores when the
 * workspace holds the repacked weights (16 * ceil(Cout/32)*32 * ceil(Cin/64)*64
 * elements; conv_transpose4x4s2_pack does this once instead); otherwise (and for fp32)
 * a direct kernel on the vector ALUs runs. Errors as conv2d_fused.
 */
int conv_transpose4x4s2(const void *x, const void *w, const float *bias, const float *alpha, void *y, int N, int H,
                        int W, int Cin, int Cout, int act, int layout, int dtype, int out_dtype, void *stream);

/*
 * Weight residency for the transposed conv: pack a layer's weights once (for example at
 * model load) into a caller-owned buffer, then run calls without the per-call repack.
 *
 * conv_transpose4x4s2_packed_bytes: *bytes = the packed size for (Cin, Cout) in a 16-bit
 *   dtype (16 * ceil(Cout/32)*32 * ceil(Cin/64)*64 elements); CONV2D_EUNSUPPORTED for
 *   fp32. Host only.
 * conv_transpose4x4s2_pack: w [Cin][Cout][4][4] (bf16/f16, Cin % 8 == 0) -> wp, a device
 *   buffer of that size, 16-byte aligned, not overlapping w (enqueued on `stream`).
 * conv_transpose4x4s2_prepacked: conv_transpose4x4s2 with the packed weights wp in place
 *   of w; needs 16-bit x with Cin % 8 == 0 (16-byte aligned when channel-last), x and wp
 *   under 2 GiB (CONV2D_EUNSUPPORTED otherwise). Results are bit-identical to
 *   conv_transpose4x4s2 on the unpacked weights. A channel-first input whose width is
 *   not a multiple of 8 (or that is not 16-byte aligned) uses the workspace, when it
 *   has room, for a channel-last copy of x; other calls write nothing but y.
 */
int conv_transpose4x4s2_packed_bytes(int Cin, int Cout, int dtype, size_t *bytes);
int conv_transpose4x4s2_pack(const void *w, void *wp, int Cin, int Cout, int dtype, void *stream);
int conv_transpose4x4s2_prepacked(const void *x, const void *wp, const float *bias, const float *alpha, void *y, int N,
                                  int H, int W, int Cin, int Cout, int act, int layout, int dtype, int out_dtype,
                                  void *stream);

/* Host-only: the kernel variants conv_transpose4x4s2 would launch (as conv2d_plan). */
int conv_transpose4x4s2_plan(int N, int H, int W, int Cin, int Cout, int act, int layout, int dtype, int out_dtype,
                             char *buf, int cap);

/*
 * Nearest-neighbour 2x upsample: y[n, oy, ox, c] = x[n, oy/2, ox/2, c] (floor).
 * Source: inferencelayer page, `UPSAMPLE_SRC` and the top-down path of the CCFM neck.
 * x [N,H,W,C] or [N,C,H,W] in `dtype`; y [N,2H,2W,C] or [N,C,2H,2W]. Bit-exact copy.
 */
int upsample_nearest2x(const void *x, void *y, int N, int H, int W, int C, int layout, int dtype, void *stream);

/*
 * Per-pixel channel concat: y holds a's Ca channels, then b's Cb channels.
 * Source: inferencelayer page, `CONCAT_SRC` and the CCFM neck ([upsampled, backbone]
 * on the top-down path, [downsampled, top-down] on the bottom-up path).
 * a [N,H,W,Ca] / [N,Ca,H,W], b [N,H,W,Cb] / [N,Cb,H,W], y [N,H,W,Ca+Cb] /
 * [N,Ca+Cb,H,W], all in `dtype`; y may not overlap a or b. Bit-exact copy.
 */
int concat_channels(const void *a, const void *b, void *y, int N, int H, int W, int Ca, int Cb, int layout, int dtype,
                    void *stream);

/*
 * y = concat_channels(upsample_nearest2x(a), b) in one pass, without writing the
 * upsampled map: the upsample and concat of the CCFM top-down path (inferencelayer
 * page, `UPSAMPLE_SRC` then `CONCAT_SRC`). a [N,H,W,Ca] / [N,Ca,H,W] (the small map);
 * b [N,2H,2W,Cb] / [N,Cb,2H,2W]; y [N,2H,2W,Ca+Cb] / [N,Ca+Cb,2H,2W]. Bit-exact copy.
 */
int upsample2x_concat(const void *a, const void *b, void *y, int N, int H, int W, int Ca, int Cb, int layout,
                      int dtype, void *stream);

/* w [Cout][Cin][kh][kw] (OIHW) -> w2 [Cout][kh][kw][Cin] (OHWI), 16-bit types, for
 * channel-first convs called with CONV2D_WEIGHTS_OHWI. w2 is a caller-owned device
 * buffer of the same size that may not overlap w; enqueued on `stream`. */
int conv2d_weights_to_ohwi(const void *w, void *w2, int Cout, int Cin, int kh, int kw, int dtype, void *stream);

/* floor((in + 2*pad - k)/stride) + 1, or -1 if in, k, stride <= 0, pad < 0 or the
 * kernel does not fit the padded input (inferencelayer `conv()`). Host only. */
int conv2d_out_dim(int in, int k, int stride, int pad);

/* Host-only validation of conv2d_fused's arguments, without launching anything
 * and without touching the GPU: returns what conv2d_fused would return before
 * its launch (CONV2D_OK, CONV2D_EINVAL or CONV2D_EUNSUPPORTED). Pointers are only
 * compared, never dereferenced. */
int conv2d_check_args(const void *x, const void *w, const float *bias, const float *alpha,
                      const void *residual, const void *y, int N, int H, int W, int Cin,
                      int Cout, int kh, int kw, int stride, int pad, int act, int layout,
                      int dtype);

/* Host-only: writes into buf (capacity cap bytes, NUL-terminated) the name of the
 * kernel variant conv2d_fused would launch for this shape, e.g.
 * "igemm_nhwc_pipe_tapinner bf16 128x128w8 splitk=1". Returns the name's length, or a
 * negative CONV2D_E* code for invalid arguments. */
int conv2d_plan(int N, int H, int W, int Cin, int Cout, int kh, int kw, int stride, int pad,
                int act, int layout, int dtype, char *buf, int cap);

/*
 * Registers the caller-owned workspace of the calling thread on the current device
 * (hipSetDevice's device; device 0's entry on a host where no device can be queried,
 * for the host-only planning calls): p, a device buffer of `bytes` bytes, 256-byte
 * aligned, or
 * NULL with bytes 0 to have none (the initial state). Replaces the library-reserved
 * scratch of the rlx-wgpu page (`compute_scratch_bytes` sizes one arena for a whole
 * network) with memory the caller allocates, e.g. torch.empty on the device.
 *
 * The library keeps only the pointer: it never frees the buffer, and the buffer must
 * stay allocated until every call (and every stack graph) planned with it has finished
 * on the GPU. Each later call from this thread on this device plans its kernels for
 * this workspace (a call's variant may change with it; see conv2d_plan) and enqueues
 * kernels that read and write it on the call's own stream. Calls that may run at the
 * same time need distinct workspaces: register the one for a stream before each call
 * on that stream (registering is a host-side store, cheap enough for every call).
 * Host only. CONV2D_EINVAL for a misaligned p or a NULL p with bytes > 0; success
 * leaves conv2d_last_error() as it was.
 */
int conv2d_set_workspace(void *p, size_t bytes);

/* Host-only: *bytes = the workspace that conv2d_fused's preferred variant for this shape
 * writes (0 when it needs none), with the tuned-plan table applied as for a call.
 * Argument errors as conv2d_plan. */
int conv2d_workspace_size(int N, int H, int W, int Cin, int Cout, int kh, int kw, int stride, int pad, int act,
                          int layout, int dtype, size_t *bytes);

/*
 * Stacks of layers: a list of ops run in order on one stream, like one call per op,
 * but validated as a whole first (a stack that returns an error has launched
 * nothing) and, optionally, captured once into a HIP graph and replayed. This is how
 * the pages run a network section: inferencelayer's `Recorder` records a whole
 * encoder into one submission, and framecast runs the eight convs of an IFNet block
 * back to back, having first copied the block input aside because the ping-pong
 * buffers reuse it, so that the last conv can add it as its residual. An op reads its
 * inputs when its turn comes, so a later op sees what earlier ops wrote; a snapshot
 * that a later op needs is an explicit CONV2D_OP_COPY.
 *
 * One op (fields that a kind does not use are ignored):
 *   CONV2D_OP_CONV          conv2d_fused(x, w, bias, alpha, residual, y, N, H, W, Cin,
 *                           Cout, kh, kw, stride, pad, act)
 *   CONV2D_OP_CONV_MAXPOOL  conv2d_fused_maxpool3x3s2(x, w, bias, alpha, y, ...); residual
 *                           must be NULL
 *   CONV2D_OP_MAXPOOL       maxpool3x3s2(x, y, N, H, W, C = Cin)
 *   CONV2D_OP_AVGPOOL       avgpool2x2(x, y, N, H, W, C = Cin)
 *   CONV2D_OP_COPY          y = x, N*H*W*Cin elements of dtype (y may not overlap x)
 *   CONV2D_OP_DECONV        conv_transpose4x4s2(x, w, bias, alpha, y, N, H, W, Cin, Cout,
 *                           act) with out_dtype = dtype
 *   CONV2D_OP_UPSAMPLE      upsample_nearest2x(x, y, N, H, W, C = Cin)
 *   CONV2D_OP_CONCAT        concat_channels(a = x, b = residual, y, N, H, W, Ca = Cin,
 *                           Cb = Cout)
 *   CONV2D_OP_UPSAMPLE_CONCAT upsample2x_concat(a = x, b = residual, y, N, H, W,
 *                           Ca = Cin, Cb = Cout)
 * Layout and dtype are shared by the whole stack.
 */
#define CONV2D_OP_CONV 0
#define CONV2D_OP_CONV_MAXPOOL 1
#define CONV2D_OP_MAXPOOL 2
#define CONV2D_OP_AVGPOOL 3
#define CONV2D_OP_COPY 4
#define CONV2D_OP_DECONV 5
#define CONV2D_OP_UPSAMPLE 6
#define CONV2D_OP_CONCAT 7
#define CONV2D_OP_UPSAMPLE_CONCAT 8

typedef struct conv2d_op {
    int kind;
    const void *x;
    const void *w;
    const float *bias;
    const float *alpha;
    const void *residual;
    void *y;
    int N, H, W, Cin, Cout, kh, kw, stride, pad, act;
} conv2d_op;

/* Host-only validation of every op of a stack (ops[0..n-1]), without touching the GPU.
 * Returns CONV2D_OK or the code of the first invalid op, whose index goes to
 * *bad_index (-1 when the stack is valid or the list itself is invalid; bad_index may
 * be NULL). */
int conv2d_stack_check(const conv2d_op *ops, int n, int layout, int dtype, int *bad_index);

/* Host-only: the kernel variants of op `index` of a stack, as conv2d_plan. */
int conv2d_stack_plan(const conv2d_op *ops, int n, int layout, int dtype, int index, char *buf, int cap);

/* Host-only: *bytes = the workspace the stack's preferred variants write (the largest op,
 * or twice the largest copy of a chain of channel-first convs), as
 * conv2d_workspace_size. Argument errors as conv2d_stack_check. */
int conv2d_stack_workspace_size(const conv2d_op *ops, int n, int layout, int dtype, size_t *bytes);

/* Validates the whole stack, then enqueues its ops in order on `stream`. Same memory
 * and workspace rules as the single calls (the workspace registered now is used by
 * every op). Consecutive channel-first 16-bit convs given channel-last weights
 * (CONV2D_WEIGHTS_OHWI), where one conv's y is the next one's x with matching sizes
 * and the first has no residual, are chained when each half of the workspace holds
 * their input and output copies: the first also writes its output channel-last into
 * one half of the workspace and the next reads its input from there instead of copying
 * it (conv2d_stack_plan names show "+y_nhwc" and "chained+"). The results are
 * bit-identical to running the ops one call at a time. */
int conv2d_stack_run(const conv2d_op *ops, int n, int layout, int dtype, void *stream);

/* Validates the stack and records it once into a HIP graph (stream capture on a
 * private stream; nothing is allocated). The graph holds the ops' pointers and sizes as
 * given and the workspace registered at creation: every replay runs the same ops on the
 * same buffers and workspace, which must stay allocated until the graph is destroyed;
 * replays that may overlap (on two streams) need two graphs made with two workspaces.
 * *out receives an opaque handle (NULL on error). */
typedef struct conv2d_graph conv2d_graph;
int conv2d_stack_graph_create(const conv2d_op *ops, int n, int layout, int dtype, conv2d_graph **out);

/* Enqueues one replay of the graph on `stream` (asynchronous, like the other calls). */
int conv2d_stack_graph_launch(conv2d_graph *g, void *stream);

/* Frees the graph (NULL is allowed). The caller makes sure no replay is still running. */
int conv2d_stack_graph_destroy(conv2d_graph *g);

/*
 * Tuning: time the candidate kernel variants of one conv shape on the current device
 * and keep the fastest for later calls of that shape, like framecast's `tuneConvRB`,
 * which benchmarks its conv variants once per device and resolution and persists the
 * winner because the best variant flips with the shape; inferencelayer's per-shape
 * GEMM tile table is the static form of the same choice.
 *
 * conv2d_tune allocates its own inputs and output for the shape (zero-filled device
 * buffers; act, has_residual, layout and dtype as conv2d_fused's arguments would be;
 * this is the library's only device allocation), uses the calling thread's registered
 * workspace for the variants that need one (only those it has room for are timed, so
 * nothing else may use that workspace meanwhile), times the built-in choice and, for
 * shapes on the channel-last matrix-core kernels,
 * every tile shape and split-K depth (1-4) of the implicit-GEMM kernel and the tile
 * heights of the halo kernel (for channel-first 16-bit layers, which run on that
 * kernel after a layout copy, every tile shape): each variant runs twice, then `reps` times between two
 * events on a private stream, queued behind a short idle kernel so that the host's launch cost does
 * not enter the timing. It synchronises that stream, frees its buffers and
 * records the fastest variant in a process-wide table keyed by (device arch and
 * compute units, N, H, W, Cin, Cout, kh, kw, stride, pad, layout, dtype, residual or
 * not). From then on conv2d_fused, the fused conv + max pool and the stacks (and
 * conv2d_plan, whose name then ends in " tuned") use it for that shape whenever the
 * variant is valid for the call (alignment, workspace size); otherwise they fall back
 * to the built-in choice. Not for use under HIP graph capture (it allocates and
 * synchronises). Writes the winner's name to buf (as conv2d_plan) and its average
 * launch time in microseconds to *best_us (if not NULL); returns the name's length or
 * a negative CONV2D_E* code. Argument errors as conv2d_fused, plus reps outside
 * 1..10000.
 */
int conv2d_tune(int N, int H, int W, int Cin, int Cout, int kh, int kw, int stride, int pad, int act, int has_residual,
                int layout, int dtype, int reps, float *best_us, char *buf, int cap);

/* Writes the whole table to a text file (a comment line, then one record per line:
 * the key with '|' separators, then four integers). Returns the number of records or
 * CONV2D_EINVAL if the file cannot be written. Host only. */
int conv2d_tune_save(const char *path);

/* Adds the records of a file written by conv2d_tune_save to the table (a record for a
 * key already present replaces it). Records of other devices are kept but never match
 * this device's calls. Returns the number of records read, or CONV2D_EINVAL (nothing
 * added) if the file cannot be read or a line is not a record. Host only. */
int conv2d_tune_load(const char *path);

/* Empties the table: every shape goes back to the built-in choice. Host only. */
int conv2d_tune_clear(void);

/* Message of the last error on the calling thread ("" if none). The pointer stays
 * valid until the thread's next call into the library. */
const char *conv2d_last_error(void);

/* ABI version of this header: 10 (CONV2D_Y_TRANSIENT for stack ops; 9: conv2d_fused_noalloc; 8: caller-owned workspace: conv2d_set_workspace and the
 * size queries replace the library's own scratch; conv2d_avgpool2x2_conv1x1 and its op
 * kind are gone; 7 added CONV2D_WEIGHTS_OHWI and conv2d_weights_to_ohwi; 6
 * added the transposed conv's weight packing calls; 5
 * added conv2d_avgpool2x2_conv1x1; 4 added the tuning calls; 3 added the transposed conv,
 * upsample and concat calls and their stack ops; 2 the stack calls and the fused conv +
 * max pool). */
int conv2d_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONV2D_FUSED_H */
