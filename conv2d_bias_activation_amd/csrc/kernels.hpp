// Host-side launchers of the library's kernels (one per kernel family).
#pragma once

#include "common.hpp"

namespace c2d {

enum IgemmTile {
    IGEMM_TILE_128x128 = 0,
    IGEMM_TILE_128x64 = 1,
    IGEMM_TILE_64x64 = 2,
    IGEMM_TILE_256x32 = 3,
};

struct IgemmPlan {
    int tile;   // IgemmTile
    bool nchw;  // channel-first layout
    bool avec;  // channel-last, Cin a multiple of the 16-byte vector, x and w aligned
    bool bvec;  // K a multiple of the 16-byte vector, w aligned
};

// MFMA implicit GEMM, any k/stride/pad, both layouts, f32/bf16/f16 storage.
hipError_t launch_igemm(const ConvArgs &a, int dtype, const IgemmPlan &p, hipStream_t st);

enum NhwcTile {
    NHWC_TILE_256x128_W8 = 0,
    NHWC_TILE_128x128 = 1,
    NHWC_TILE_128x64 = 2,
    NHWC_TILE_256x64_W8 = 3,
    NHWC_TILE_256x32 = 4,
    NHWC_TILE_64x64 = 5,
    NHWC_TILE_128x128_W8 = 6,
    NHWC_TILE_128x256_W8 = 7,
    NHWC_TILE_64x64_D6 = 8,
    NHWC_TILE_128x64_D5 = 9,
    NHWC_TILE_128x128_W8_D4 = 10,
    NHWC_TILE_64x128_D5 = 11,
    NHWC_TILE_64x64_D4 = 12,
    NHWC_TILE_256x128_W8_D3 = 13,
    NHWC_TILE_64x64_K2 = 14,
    NHWC_TILE_64x64_K2_D4 = 15,
    NHWC_TILE_64x64_K2_D2 = 16,
    NHWC_TILE_COUNT = 17,
};

struct NhwcPlan {
    int tile;        // NhwcTile
    int splits;      // K slices; > 1 needs splits * M * Cout floats of scratch
    bool tap_inner;  // Cin % 64 == 0: taps innermost in the K loop
    bool nchw_out;   // y and the residual are channel-first (x and w still channel-last)
};

// Channel-first input and OIHW weight to channel-last copies (16-bit types).
hipError_t launch_to_channel_last(const void *x, void *x_nhwc, int N, int C, int HW, const void *w,
                                  void *w_ohwi, int Cout, int taps, int dtype, hipStream_t st);

int nhwc_tile_bm(int tile);
int nhwc_tile_bn(int tile);
int nhwc_tile_waves(int tile);

// Pipelined channel-last MFMA implicit GEMM (bf16/f16, Cin % 8 == 0, x, w and y
// under 2 GiB, x and w 16-byte aligned). With p.splits > 1 (needs Cout % 8 == 0 and
// 16-byte aligned y and residual), the GEMM writes fp32 partial sums of each K
// slice to `partials` and a second kernel adds them and applies the epilogue.
hipError_t launch_igemm_nhwc(const ConvArgs &a, int dtype, const NhwcPlan &p, float *partials,
                             hipStream_t st);

struct HaloPlan {
    int th;        // output rows per 32-pixel-wide tile
    int fn;        // 32-channel output blocks per wave: 1 (Cout <= 32) or 2 (Cout <= 64)
    int waves;     // per workgroup: 8, or 4 (two workgroups per CU)
    int grid_cap;  // persistent workgroups
};

// 3x3 stride-1 pad-1 channel-last 16-bit convolution with halo tiles and weights held
// in registers: Cin 16, 32 or 64, Cout <= 32 * p.fn with Cout % 8 == 0, x and w
// 16-byte aligned, y and the residual 16-byte aligned (a.vec_out), tensors under
// 2 GiB. With WM = p.waves (Cin <= 32) or p.waves / 2 (Cin 64): p.th in {WM, 2*WM}
// for p.fn = 1, p.th = WM for p.fn = 2.
hipError_t launch_halo3x3(const ConvArgs &a, int dtype, const HaloPlan &p, hipStream_t st);

// The same convolution for Cin 64 (Cout <= 64) with specialised waves: four compute
// waves with their weights in registers run only the matrix-core products, four
// loader/epilogue waves prefetch the halos and run the previous tile's epilogue; one
// persistent workgroup of 8 waves per CU (grid_cap workgroups). Limits as launch_halo3x3.
hipError_t launch_halo3x3_ws(const ConvArgs &a, int dtype, int grid_cap, hipStream_t st);

// Geometry of one hgemm launch (host-computed).
struct HgemmGeo {
    int tiles_x, tiles_y, tiles_c;  // output tiles along W, H and the output channels
    int ntiles_p;                   // pixel tiles (N * tiles_y * tiles_x)
    int cfast;                      // consecutive tile ids vary the channel tile fastest
};

struct HgemmPlan {
    int cfg;     // kernel variant (tile shape, wave grid, ring depth, K chunk)
    bool cfast;  // tile order: channel tiles fastest (true) or pixel tiles fastest
};

struct HgemmInfo {
    int ck;           // input channels per K chunk
    int th, tw, cb;   // tile: output rows, columns, channels
    int waves, lds;   // waves and LDS bytes per workgroup
    bool ws;          // the specialised-wave kernel (loader and compute waves)
    int stride;       // the convolution stride the variant computes (1 or 2)
    long long tiles;  // workgroups of the launch
};

// The 2x2 average pool of x followed by a 1x1 convolution of the pooled map, one kernel
// (channel-last, 16-bit, Cin 64/128/256, Cout % 8 == 0, OH = H/2, OW = W/2): y is the
// conv output, p (if not null) receives the pooled map as well.
struct PoolPwArgs {
    const void *x;      // [N, H, W, Cin]
    const void *w;      // [Cout, Cin] (1x1 weights)
    const float *bias;  // may be null
    const float *alpha; // may be null unless PReLU
    void *y;            // [N, OH, OW, Cout]
    void *p;            // [N, OH, OW, Cin] or null
    int N, H, W, OH, OW, Cin, Cout, act;
    int tiles_n;        // set by the launcher
};
bool poolpw_fits(int Cin, int Cout, int dtype);
hipError_t launch_poolpw(const PoolPwArgs &a, int dtype, hipStream_t st);

// 3x3 stride-1 or stride-2 pad-1 channel-last 16-bit convolution of wide layers with halo tiles
// and weights staged per K chunk: Cin a multiple of the variant's K chunk (32 or 64),
// Cout % 8 == 0, y and the residual 16-byte aligned (a.vec_out), x, w and y under 2 GiB.
// With nchw_out, y and the residual are channel-first (no alignment needed), Cin need
// only be a multiple of 8, and a.y2, if set and 16-byte aligned, receives the same output
// channel-last; the specialised-wave variants do not take it.
hipError_t launch_hgemm3x3(const ConvArgs &a, int dtype, const HgemmPlan &p, bool nchw_out, hipStream_t st);
int hgemm_cfg_count();
bool hgemm_cfg_info(int cfg, const ConvArgs &a, HgemmInfo *out);

// The same convolution for Cin 16 or 32 followed by the 3x3 stride-2 pad-1 max pool in
// one kernel: only the pooled map is written, to y ([N, PH, PW, Cout], PH = (H-1)/2 + 1,
// 16-byte aligned); no residual. About grid_cap workgroups of 4 waves (two per CU).
hipError_t launch_halo3x3_maxpool(const ConvArgs &a, void *y, int dtype, int grid_cap, hipStream_t st);

// 3x3 convolution of a 3-channel channel-last 16-bit image on the matrix cores:
// stride 1 or 2, pad 1, Cout <= 64 with Cout % 8 == 0, W % 8 == 0 and W <= 3000, x
// 16-byte aligned, y and the residual 16-byte aligned (a.vec_out), tensors under 2 GiB.
// fp32 storage (dtype CONV2D_DTYPE_F32) goes to launch_stem3_f32.
hipError_t launch_stem3(const ConvArgs &a, int dtype, hipStream_t st);

// Two 3x3 convs, only the second one's output written: a1 = the stem conv (3 -> 32
// channels, stride 2, pad 1, no residual, W % 8 == 0), a2 = a stride-1 pad-1 conv of a1's
// output (a2.x == a1.y, Cin 32, Cout <= 32 with Cout % 8 == 0, no residual, y 16-byte
// aligned); 16-bit storage, channel-last. Bit-identical to the stem kernel followed by
// the halo kernel. grid_cap: persistent workgroups (three per CU).
bool stem_pair_fits(const ConvArgs &a1, const ConvArgs &a2, int dtype);
hipError_t launch_stem_pair(const ConvArgs &a1, const ConvArgs &a2, int dtype, int grid_cap, hipStream_t st);

// The same for fp32 storage (32x32x2 fp32 products): Cout <= 64 with Cout % 4 == 0,
// W % 4 == 0 and W <= 1700, same alignment and size limits.
hipError_t launch_stem3_f32(const ConvArgs &a, hipStream_t st);
// ... followed by the 3x3 stride-2 pad-1 max pool, only the pooled map written to y.
hipError_t launch_stem3_f32_maxpool(const ConvArgs &a, void *y, hipStream_t st);

// The same convolution followed by the 3x3 stride-2 pad-1 max pool in one kernel: only
// the pooled map is written, to y ([N, PH, PW, Cout] with PH = (OH - 1) / 2 + 1, 16-byte
// aligned); a.y and a.res are ignored. Same limits as launch_stem3 except the width.
hipError_t launch_stem3_maxpool(const ConvArgs &a, void *y, int dtype, hipStream_t st);

// Direct convolution on the vector ALUs for few input channels (the image stem):
// one thread per output pixel and a block of output channels.
hipError_t launch_direct(const ConvArgs &a, int dtype, bool nchw, hipStream_t st);

// y = x, `bytes` bytes (a snapshot inside a stream of layers).
hipError_t launch_copy(const void *x, void *y, size_t bytes, hipStream_t st);

// One wave that idles for rounds x s_sleep 127 (about 3.4 us each at 2.4 GHz), 0..4096.
hipError_t launch_idle(int rounds, hipStream_t st);

// Pools (layout: CONV2D_LAYOUT_*). vec: C a multiple of the 16-byte vector and
// both pointers aligned (channel-last only).
hipError_t launch_maxpool(const void *x, void *y, int N, int H, int W, int C, bool nchw,
                          int dtype, bool vec, hipStream_t st);
hipError_t launch_avgpool(const void *x, void *y, int N, int H, int W, int C, bool nchw,
                          int dtype, bool vec, hipStream_t st);

// Transposed convolution 4x4, stride 2, pad 1 (output 2H x 2W).
struct DeconvArgs {
    const void *x;       // [N,H,W,Cin] (channel-last kernel) or the caller's layout (direct kernel)
    const void *w;       // caller's [Cin][Cout][4][4] (direct kernel)
    const void *wp;      // packed in MFMA operand order, 16 * CoP * ceil(Cin/64)*64 elements
    const float *bias;   // may be null
    const float *alpha;  // null unless PReLU
    void *y;
    int N, H, W, Cin, Cout;
    int CoP;  // Cout rounded up to 32
    int act;  // CONV2D_ACT_*
    uint32_t x_bytes, wp_bytes;  // buffer extents (matrix-core kernel; both under 2^31)
};

// w [Cin][Cout][4][4] -> wp (16-bit types, 16 * CoP * ceil(Cin/64)*64 elements): per
// output parity class, 32-channel output block, 64-channel input chunk, tap and 16-deep
// step, the 64 lanes' MFMA B operands in lane order; padding is zero.
hipError_t launch_deconv_pack(const void *w, void *wp, int Cin, int Cout, int CoP, int dtype, hipStream_t st);

// Matrix-core kernel: 16-bit x with Cin % 8 == 0 (channel-last: 16-byte aligned), wp
// 16-byte aligned, x and wp under 2^31 bytes, y under 2^31 elements; x and y both channel-last or (nchw) both
// channel-first; y in the input's type or (out_f32) fp32.
hipError_t launch_deconv_mfma(const DeconvArgs &a, int dtype, bool out_f32, bool nchw, hipStream_t st);

// The same products with the whole input strip staged at once, Cin % 8 == 0 and
// Cin <= 256: channel-last x (the channel-last copy of a channel-first layer's input)
// or, with nchw_in, the channel-first x itself (W % 8 == 0, 16-byte aligned);
// y channel-first (nchw_out must be true).
hipError_t launch_deconv_mfma_all(const DeconvArgs &a, int dtype, bool out_f32, bool nchw_out, bool nchw_in,
                                  hipStream_t st);

// OIHW -> OHWI weights alone (16-bit types).
hipError_t launch_oihw_to_ohwi(const void *w, void *w2, int Cout, int Cin, int taps, int dtype, hipStream_t st);

// Channel-first 16-bit map to channel-last (N planes of C x HW; 16-byte accesses when C
// and HW are multiples of 8 and both pointers are 16-byte aligned).
hipError_t launch_nchw_to_nhwc(const void *x, void *y, int N, int C, int HW, int dtype, hipStream_t st);

// Any layout and type, one thread per output (weights in the caller's layout).
hipError_t launch_deconv_direct(const DeconvArgs &a, int dtype, bool out_f32, bool nchw, hipStream_t st);

// y = concat(up ? upsample2x(a) : a, b) along channels; a alone (Cb = 0, b unused) is
// the plain upsample. H, W: y's size (even when up). vec: channel-last with Ca and Cb
// multiples of the 16-byte vector, or channel-first without up and H*W a multiple of it;
// all pointers 16-byte aligned.
hipError_t launch_concat(const void *a, const void *b, void *y, int N, int H, int W, int Ca, int Cb, bool up,
                         bool nchw, int dtype, bool vec, hipStream_t st);

}  // namespace c2d
