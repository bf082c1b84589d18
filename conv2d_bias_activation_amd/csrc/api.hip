// C ABI of the library: argument validation, kernel-variant choice and launch.
// Declarations and the contract of every entry point: include/conv2d_fused.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"

namespace {

using namespace c2d;

thread_local std::string g_err;

int set_error(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int set_ok() {
    g_err.clear();
    return CONV2D_OK;
}

int dtype_bytes(int dtype) {
    switch (dtype) {
    case CONV2D_DTYPE_F32:
        return 4;
    case CONV2D_DTYPE_BF16:
    case CONV2D_DTYPE_F16:
        return 2;
    default:
        return 0;
    }
}

const char *dtype_name(int dtype) {
    switch (dtype) {
    case CONV2D_DTYPE_F32:
        return "f32";
    case CONV2D_DTYPE_BF16:
        return "bf16";
    case CONV2D_DTYPE_F16:
        return "f16";
    default:
        return "?";
    }
}

int out_dim(int in, int k, int s, int p) {
    if (in <= 0 || k <= 0 || s <= 0 || p < 0) return -1;
    long long span = (long long)in + 2ll * p - k;
    if (span < 0) return -1;
    long long o = span / s + 1;
    return o > 0x7fffffff ? -1 : (int)o;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void *a, long long abytes, const void *b, long long bbytes) {
    if (!a || !b) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

constexpr long long kMaxElems = 0x7fffffffll;

// Validates conv2d_fused's arguments; fills the derived geometry into `a`. With
// pooled_y, y holds the 3x3 stride-2 max pool of the conv output instead.
int check_conv(const void *x, const void *w, const float *bias, const float *alpha, const void *residual,
               const void *y, int N, int H, int W, int Cin, int Cout, int kh, int kw,
               int stride, int pad, int act, int layout, int dtype, ConvArgs *a, bool pooled_y = false) {
    if (!x || !w || !y) return set_error(CONV2D_EINVAL, "x, w and y must not be null");
    if (N <= 0 || H <= 0 || W <= 0 || Cin <= 0 || Cout <= 0 || kh <= 0 || kw <= 0)
        return set_error(CONV2D_EINVAL, "sizes must be positive (N=%d H=%d W=%d Cin=%d Cout=%d kh=%d kw=%d)",
                         N, H, W, Cin, Cout, kh, kw);
    if (stride != 1 && stride != 2) return set_error(CONV2D_EINVAL, "stride must be 1 or 2 (got %d)", stride);
    if (pad < 0) return set_error(CONV2D_EINVAL, "pad must be >= 0 (got %d)", pad);
    if (layout != CONV2D_LAYOUT_NHWC && layout != CONV2D_LAYOUT_NCHW)
        return set_error(CONV2D_EINVAL, "unknown layout %d", layout);
    if (!dtype_bytes(dtype)) return set_error(CONV2D_EINVAL, "unknown dtype %d", dtype);
    int code = act & 0xff;
    if (code > CONV2D_ACT_PRELU || (act & ~(0xff | CONV2D_RES_BEFORE_ACT | CONV2D_WEIGHTS_OHWI)))
        return set_error(CONV2D_EINVAL, "unknown activation flags 0x%x", act);
    if ((act & CONV2D_WEIGHTS_OHWI) && layout != CONV2D_LAYOUT_NCHW)
        return set_error(CONV2D_EINVAL, "CONV2D_WEIGHTS_OHWI is for channel-first layers");
    if (code == CONV2D_ACT_PRELU && !alpha) return set_error(CONV2D_EINVAL, "PRELU needs alpha");
    int OH = out_dim(H, kh, stride, pad), OW = out_dim(W, kw, stride, pad);
    if (OH < 1 || OW < 1)
        return set_error(CONV2D_EINVAL, "kernel %dx%d does not fit the padded %dx%d input", kh, kw, H, W);
    long long xe = (long long)N * H * W * Cin;
    long long we = (long long)Cout * kh * kw * Cin;
    long long ye = (long long)N * OH * OW * Cout;
    long long m = (long long)N * OH * OW;
    if (xe > kMaxElems || we > kMaxElems || ye > kMaxElems || m > kMaxElems)
        return set_error(CONV2D_EUNSUPPORTED, "tensors of 2^31 or more elements are not supported");
    int eb = dtype_bytes(dtype);
    const long long yb = pooled_y ? (long long)N * out_dim(OH, 3, 2, 1) * out_dim(OW, 3, 2, 1) * Cout * eb : ye * eb;
    if (overlap(y, yb, x, xe * eb)) return set_error(CONV2D_EINVAL, "y overlaps x");
    if (overlap(y, yb, residual, ye * eb)) return set_error(CONV2D_EINVAL, "y overlaps the residual");
    // other workgroups still read the weights, bias and slopes while one stores y
    if (overlap(y, yb, w, we * eb)) return set_error(CONV2D_EINVAL, "y overlaps w");
    if (overlap(y, yb, bias, (long long)Cout * 4)) return set_error(CONV2D_EINVAL, "y overlaps bias");
    if (code == CONV2D_ACT_PRELU && overlap(y, yb, alpha, (long long)Cout * 4))
        return set_error(CONV2D_EINVAL, "y overlaps alpha");
    a->x = x;
    a->w = w;
    a->alpha = alpha;
    a->res = residual;
    a->y = const_cast<void *>(y);
    a->N = N;
    a->H = H;
    a->W = W;
    a->Cin = Cin;
    a->Cout = Cout;
    a->kh = kh;
    a->kw = kw;
    a->stride = stride;
    a->pad = pad;
    a->OH = OH;
    a->OW = OW;
    a->M = (int)m;
    a->K = (int)we / Cout;
    a->act = code;
    a->res_before_act = (act & CONV2D_RES_BEFORE_ACT) ? 1 : 0;
    a->w_ohwi = (act & CONV2D_WEIGHTS_OHWI) ? 1 : 0;
    a->vec_out = aligned16(y) && (!residual || aligned16(residual));
    a->y2 = nullptr;  // set per launch for chained channel-first layers
    return CONV2D_OK;
}

enum Family {
    FAM_DIRECT = 0,
    FAM_IGEMM = 1,
    FAM_NHWC = 2,
    FAM_NCHW_VIA_NHWC = 3,
    FAM_HALO = 4,
    FAM_STEM = 5,
    FAM_HALO_WS = 6,
    FAM_HGEMM = 7
};

struct Plan {
    int family;
    IgemmPlan ig;
    NhwcPlan nh;
    HaloPlan halo;
    HgemmPlan hg;
    bool nchw_hg;  // FAM_NCHW_VIA_NHWC: the halo-tile GEMM (hg) instead of the pipelined kernel (nh)
    bool tuned;  // chosen by a conv2d_tune measurement rather than the built-in heuristics
    bool w_ohwi; // channel-first layer with channel-last weights: only the input is copied
    // chained channel-first layers of a stack (FAM_NCHW_VIA_NHWC, set by link_chains)
    bool chain_in;   // the input's channel-last copy is already in the workspace at x_at
    size_t x_at;
    bool chain_out;  // also write the output channel-last into the workspace at y2_at
    size_t y2_at;
};

// Caller-owned workspace (device scratch) of the calls made from this thread on one
// device, registered by conv2d_set_workspace. It holds split-K fp32 partial sums, the
// channel-last copies of a channel-first layer's input and weight, the unpooled output
// of a conv + max pool that runs as two kernels, and a transposed conv's packed
// weights. Without one (or when it is too small) every call takes a variant that
// needs no scratch, or returns CONV2D_EUNSUPPORTED where none exists.
struct Workspace {
    char *p;
    size_t bytes;
};
constexpr int kMaxDevices = 64;
thread_local Workspace g_ws[kMaxDevices];
// a planning-only stand-in for "as much workspace as the preferred variants want"
constexpr size_t kUnlimitedWs = (size_t)1 << 50;

// The registry slot of the current device: device 0's when no device can be queried, so
// that host-only planning calls see a registered size on a machine without a GPU.
int ws_slot() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    return dev;
}

Workspace current_ws() {
    const int dev = ws_slot();
    return dev >= 0 && dev < kMaxDevices ? g_ws[dev] : Workspace{nullptr, 0};
}

// Compute units of the current device (queried once per device).
std::atomic<int> g_cus[kMaxDevices];

int device_cus(int *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(CONV2D_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return set_error(CONV2D_EHIP, "device index %d out of range", dev);
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || n <= 0) return set_error(CONV2D_EHIP, "compute unit count: %s", hipGetErrorString(e));
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    *out = n;
    return CONV2D_OK;
}

const char *tile_name(int t) {
    switch (t) {
    case IGEMM_TILE_128x128:
        return "128x128";
    case IGEMM_TILE_128x64:
        return "128x64";
    case IGEMM_TILE_64x64:
        return "64x64";
    case IGEMM_TILE_256x32:
        return "256x32";
    default:
        return "?";
    }
}

// Tile choice: the fewest "rounds" of 256 workgroups (one per CU), weighted by how
// efficiently each tile shape feeds the matrix cores.
int choose_tile(const ConvArgs &a) {
    struct Cand {
        int tile, bm, bn;
        double eff;
    } cands[] = {{IGEMM_TILE_128x128, 128, 128, 1.0},
                 {IGEMM_TILE_128x64, 128, 64, 0.8},
                 {IGEMM_TILE_256x32, 256, 32, 0.7},
                 {IGEMM_TILE_64x64, 64, 64, 0.6}};
    int best = IGEMM_TILE_128x128;
    double best_cost = 1e300;
    for (const Cand &c : cands) {
        long long tm = (a.M + c.bm - 1) / c.bm, tn = (a.Cout + c.bn - 1) / c.bn;
        long long tiles = tm * tn;
        long long rounds = (tiles + 255) / 256;
        double cost = (double)rounds * c.bm * c.bn / c.eff;
        if (cost < best_cost) {
            best_cost = cost;
            best = c.tile;
        }
    }
    return best;
}

const char *nhwc_tile_name(int t) {
    static const char *names[NHWC_TILE_COUNT] = {
        "256x128w8", "128x128",  "128x64",   "256x64w8",    "256x32",   "64x64",   "128x128w8",
        "128x256w8", "64x64d6",  "128x64d5", "128x128w8d4", "64x128d5", "64x64d4", "256x128w8d3",
        "64x64k2",   "64x64k2d4", "64x64k2d2"};
    return (t >= 0 && t < NHWC_TILE_COUNT) ? names[t] : "?";
}

// Channel-last 16-bit layers. Tile shapes from measurements on MI355X (ResNet-style
// layer shapes): 8-wave 128x128 tiles while there are enough of them to occupy the
// GPU, 64x64 tiles for the small-M deep layers (more workgroups in flight beat
// bigger tiles there), 128x256 for wide pointwise layers, 128x64 for narrow outputs.
size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

NhwcPlan plan_nhwc(const ConvArgs &a, size_t ws) {
    NhwcPlan p{};
    auto tiles = [&](int bm, int bn) {
        return (long long)((a.M + bm - 1) / bm) * ((a.Cout + bn - 1) / bn);
    };
    if (a.Cout <= 64)
        p.tile = NHWC_TILE_128x64;
    else if (a.Cout >= 256 && a.K >= 256 && a.kh * a.kw == 1 && tiles(128, 256) >= 100)
        p.tile = NHWC_TILE_128x256_W8;
    else if (tiles(128, 128) >= 160)
        p.tile = NHWC_TILE_128x128_W8;
    else
        p.tile = NHWC_TILE_64x64;
    // Deep-K layers whose tiles leave most SIMDs idle (ResNet stage 4: 800 waves for
    // 1024 SIMDs, K = 4608) split K in three: measured 39 -> 25 us. Elsewhere the
    // second pass and the fp32 partial traffic cost more than the extra waves gain.
    const long long waves = tiles(nhwc_tile_bm(p.tile), nhwc_tile_bn(p.tile)) * nhwc_tile_waves(p.tile);
    const int nsteps = (a.K + 63) / 64;
    p.splits = 1;
    if (waves < 1200 && nsteps >= 48 && (a.Cout % 8) == 0 && a.vec_out &&
        3ull * a.M * a.Cout * 4 <= ws)
        p.splits = 3;
    p.tap_inner = (a.Cin % 64) == 0 && a.kh * a.kw <= 32;  // tap masks are 32-bit
    return p;
}

// Halo-tile kernel for narrow 3x3 stride-1 layers: one wave covers all the output
// channels (32 or 64). Cin <= 32: 4-wave workgroups, two per CU (their epilogues
// overlap each other's products); Cin 64: 8-wave workgroups with k split over wave
// pairs (a 4-wave one would have 2-row tiles, whose halo costs as much as the tile).
// Tile height WM rows (one per wave along the rows) or, for 32 channels, possibly
// 2*WM, taking the height with the least work per workgroup slot over one GPU's 256
// CUs, counting a tile of TH rows as TH + 4 (its two halo rows and a fixed cost;
// from MI355X timings of the ResNet stem and stage-1 layers); ties go to the taller.
HaloPlan plan_halo(const ConvArgs &a) {
    HaloPlan p{};
    p.fn = a.Cout <= 32 ? 1 : 2;
    p.waves = a.Cin == 64 ? 8 : 4;
    const int wm = a.Cin == 64 ? p.waves / 2 : p.waves;
    const int slots = 256 * (8 / p.waves);
    p.th = wm;
    if (p.fn == 1) {
        long long best = 0;
        for (int th : {2 * wm, wm}) {
            const long long nt = (long long)a.N * ((a.W + 31) / 32) * ((a.H + th - 1) / th);
            const long long cost = (nt + slots - 1) / slots * (th + 4);
            if (best == 0 || cost < best) {
                best = cost;
                p.th = th;
            }
        }
    }
    p.grid_cap = slots;
    return p;
}

bool halo_fits(const ConvArgs &a, int layout, int dtype) {
    return layout == CONV2D_LAYOUT_NHWC && dtype != CONV2D_DTYPE_F32 && a.kh == 3 && a.kw == 3 &&
           a.stride == 1 && a.pad == 1 && (a.Cin == 16 || a.Cin == 32 || a.Cin == 64) && a.Cout <= 64 &&
           (a.Cout % 8) == 0 && a.vec_out && aligned16(a.x) && aligned16(a.w);
}

// Matrix-core stem kernels: 3-channel channel-last image, 3x3, pad 1; 16-bit storage
// (32x32x16 products) or fp32 (32x32x2 fp32 products).
bool stem_fits(const ConvArgs &a, int layout, int dtype) {
    const bool f32 = dtype == CONV2D_DTYPE_F32;
    const int eb = dtype_bytes(dtype);
    return layout == CONV2D_LAYOUT_NHWC && a.Cin == 3 && a.kh == 3 && a.kw == 3 && a.pad == 1 &&
           (a.stride == 1 || a.stride == 2) && a.Cout <= 64 && (a.Cout % (f32 ? 4 : 8)) == 0 && a.vec_out &&
           aligned16(a.x) && (a.W % (f32 ? 4 : 8)) == 0 && a.W <= (f32 ? 1700 : 3000) &&
           (long long)a.N * a.H * a.W * 3 * eb < (1ll << 31) && (long long)a.M * a.Cout * eb < (1ll << 31);
}

// Halo-tile GEMM kernel for wide 3x3 stride-1 layers (channel-last, 16-bit, Cin a
// multiple of 32; variants with 64-channel K chunks need Cin % 64 == 0).
bool hgemm_shape_ok(const ConvArgs &a, int dtype) {
    const int eb = dtype_bytes(dtype);
    return dtype != CONV2D_DTYPE_F32 && a.kh == 3 && a.kw == 3 && (a.stride == 1 || a.stride == 2) && a.pad == 1 &&
           a.Cin >= 32 && (a.Cin % 8) == 0 && (a.Cout % 8) == 0 && (long long)a.N * a.H * a.W * a.Cin * eb < (1ll << 31) &&
           (long long)a.Cout * a.K * eb < (1ll << 31) && (long long)a.M * a.Cout * eb < (1ll << 31);
}

bool hgemm_fits(const ConvArgs &a, int layout, int dtype) {
    return layout == CONV2D_LAYOUT_NHWC && hgemm_shape_ok(a, dtype) && (a.Cin % 32) == 0 && a.vec_out &&
           aligned16(a.x) && aligned16(a.w);
}

// A channel-first layer on the halo-tile GEMM: its input copied channel-last into the
// workspace (or handed over by the previous conv of a stack), weights channel-last,
// output (and residual) written channel-first by the GEMM's epilogue.
bool hgemm_nchw_fits(const ConvArgs &a, int layout, int dtype) {
    return layout == CONV2D_LAYOUT_NCHW && hgemm_shape_ok(a, dtype) && (!a.w_ohwi || aligned16(a.w));
}

// Channel-last outputs need Cin a multiple of the variant's K chunk; channel-first ones
// (not on the specialised-wave variants) take a partial last chunk.
bool hgemm_cfg_ok(const ConvArgs &a, int cfg, bool nchw = false) {
    HgemmInfo in{};
    return hgemm_cfg_info(cfg, a, &in) && in.stride == a.stride && (nchw ? !in.ws : (a.Cin % in.ck) == 0) &&
           in.tiles > 0 && in.tiles < (1ll << 31);
}

// Tile order: each XCD (one L2) gets a contiguous run of tile ids; with the channel
// tile fastest an XCD reads about 1/8 of the input and all the weights, with the pixel
// tile fastest all the input and 1/8 of the weights. The smaller total wins.
bool hgemm_cfast(const ConvArgs &a) {
    const double xb = (double)a.N * a.H * a.W * a.Cin, wb = (double)a.Cout * a.K;
    return xb / 8 + wb <= xb + wb / 8;
}

// Variant: the specialised-wave kernel (1) where its tiles fit one round of workgroups
// over `cus` CUs (a deep K on few pixels, e.g. ResNet stage 4); the 10 x 20-pixel tiles
// (4) where they give at least two workgroups per CU (e.g. ResNet stage 2, 80 x 80 x 128
// at batch 4); else the 10 x 10-pixel tiles (0). Stride 2: the three-stage ring (12)
// where its tiles fit one round, else the 10 x 10 x 64 tiles (6). From MI355X timings
// (256 CUs) of the ResNet stage 2, 3 and 4 layers.
HgemmPlan plan_hgemm(const ConvArgs &a, int cus) {
    HgemmPlan p{};
    p.cfast = hgemm_cfast(a);
    HgemmInfo in{};
    if (a.stride == 2) {
        if (hgemm_cfg_ok(a, 12) && hgemm_cfg_info(12, a, &in) && in.tiles <= cus)
            p.cfg = 12;
        else
            p.cfg = hgemm_cfg_ok(a, 6) ? 6 : -1;
        return p;
    }
    if (hgemm_cfg_ok(a, 1) && hgemm_cfg_info(1, a, &in) && in.tiles <= cus)
        p.cfg = 1;
    else if (hgemm_cfg_ok(a, 4) && hgemm_cfg_info(4, a, &in) && in.tiles >= 2ll * cus)
        p.cfg = 4;
    else
        p.cfg = hgemm_cfg_ok(a, 0) ? 0 : -1;
    return p;
}

// The general MFMA implicit GEMM: any shape, layout and dtype, no workspace.
Plan igemm_plan(const ConvArgs &a, int layout, int dtype) {
    Plan p{};
    const int ve = 16 / dtype_bytes(dtype);
    p.family = FAM_IGEMM;
    p.ig.nchw = layout == CONV2D_LAYOUT_NCHW;
    p.ig.avec = !p.ig.nchw && (a.Cin % ve) == 0 && aligned16(a.x) && aligned16(a.w);
    p.ig.bvec = (a.K % ve) == 0 && aligned16(a.w);
    p.ig.tile = choose_tile(a);
    return p;
}

Plan make_plan_default(const ConvArgs &a, int layout, int dtype, size_t ws) {
    Plan p{};
    if (stem_fits(a, layout, dtype)) {
        p.family = FAM_STEM;
        return p;
    }
    if (a.Cin <= 4) {
        p.family = FAM_DIRECT;
        return p;
    }
    const long long xbytes = (long long)a.N * a.H * a.W * a.Cin * dtype_bytes(dtype);
    const long long wbytes = (long long)a.Cout * a.K * dtype_bytes(dtype);
    const long long ybytes = (long long)a.M * a.Cout * dtype_bytes(dtype);
    if (halo_fits(a, layout, dtype) && xbytes < (1ll << 31) && ybytes < (1ll << 31)) {
        // 64 input channels: the kernel with specialised compute and loader waves
        // (measured on MI355X, ResNet-D stage 1: 21 -> see the design notes)
        p.family = a.Cin == 64 ? FAM_HALO_WS : FAM_HALO;
        p.halo = plan_halo(a);
        return p;
    }
    // wide 3x3 layers with at least 256 input channels, or 128 where the 10 x 20-pixel
    // tiles fill two workgroups per CU or the stride is 2 (narrower or smaller ones are
    // faster on the tiled GEMM below)
    if (hgemm_fits(a, layout, dtype) && a.Cin >= 128) {
        p.hg = plan_hgemm(a, 256);
        if (p.hg.cfg >= 0 && (a.Cin >= 256 || p.hg.cfg == 4 || a.stride == 2)) {
            p.family = FAM_HGEMM;
            return p;
        }
    }
    if (layout == CONV2D_LAYOUT_NHWC && dtype != CONV2D_DTYPE_F32 && (a.Cin % 8) == 0 &&
        aligned16(a.x) && aligned16(a.w) && xbytes < (1ll << 31) && wbytes < (1ll << 31) &&
        ybytes < (1ll << 31)) {
        p.family = FAM_NHWC;
        p.nh = plan_nhwc(a, ws);
        return p;
    }
    // Channel-first 16-bit layers: channel-last copies of x (and of w, unless given
    // channel-last) in the workspace, the channel-last kernel, and an epilogue that
    // writes the channel-first output.
    if (layout == CONV2D_LAYOUT_NCHW && dtype != CONV2D_DTYPE_F32 && (a.Cin % 8) == 0 && a.N <= 65535 &&
        round256((size_t)xbytes) + (a.w_ohwi ? 0 : round256((size_t)wbytes)) <= ws && ybytes < (1ll << 31)) {
        p.family = FAM_NCHW_VIA_NHWC;
        p.nh = plan_nhwc(a, ws);
        p.nh.splits = 1;
        p.nh.nchw_out = true;
        // wide layers on the halo-tile GEMM: the 17 x 15-pixel tiles where one round of
        // workgroups covers the layer (the IFNet block: 256 tiles), else the 10 x 10 ones
        if (hgemm_nchw_fits(a, layout, dtype) && a.Cin >= 128) {
            HgemmInfo in{};
            p.nchw_hg = true;
            p.hg.cfg = hgemm_cfg_ok(a, 9, true) && hgemm_cfg_info(9, a, &in) && in.tiles <= 256 ? 9 : 0;
            p.hg.cfast = false;
            if (!hgemm_cfg_ok(a, p.hg.cfg, true)) p.nchw_hg = false;
        }
        return p;
    }
    return igemm_plan(a, layout, dtype);
}

// ---- tuned plans (framecast's `tuneConvRB`: time the candidate variants of a shape on
// this device once, keep the fastest, persist the answer) ----
//
// The table maps a shape key (device, sizes, layout, dtype, residual or not) to a kernel
// variant of the channel-last matrix-core families. make_plan consults it for shapes
// whose built-in choice is one of those families, and uses an entry only if the variant
// is valid for the call at hand (alignment, workspace size).
constexpr int kNchwHgTile = 100;  // FAM_NCHW_VIA_NHWC entries at or above: halo-tile GEMM variants

struct TunedEntry {
    int family;  // FAM_NHWC, FAM_NCHW_VIA_NHWC, FAM_HALO, FAM_HALO_WS or FAM_HGEMM
    int tile;    // NhwcTile (FAM_NHWC, FAM_NCHW_VIA_NHWC), kernel variant (FAM_HGEMM), or
                 // kNchwHgTile + kernel variant (FAM_NCHW_VIA_NHWC on the halo-tile GEMM)
    int splits;  // K slices (FAM_NHWC; 1 for FAM_NCHW_VIA_NHWC and FAM_HGEMM)
    int th;      // tile height (FAM_HALO); tile order, channel tiles fastest or not (FAM_HGEMM)
};
std::mutex g_tune_mu;
std::map<std::string, TunedEntry> g_tuned;
std::atomic<int> g_tuned_n{0};  // entries in g_tuned (the planner skips the lookup at 0)
std::string g_dev_tag[kMaxDevices];
std::once_flag g_dev_tag_once[kMaxDevices];

// "<gfx arch>:<compute units>" of the current device, or "" without one.
std::string device_tag() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return "";
    std::call_once(g_dev_tag_once[dev], [dev] {
        hipDeviceProp_t pr;
        if (hipGetDeviceProperties(&pr, dev) == hipSuccess) {
            std::string arch = pr.gcnArchName;
            arch = arch.substr(0, arch.find(':'));
            g_dev_tag[dev] = arch + ":" + std::to_string(pr.multiProcessorCount);
        }
    });
    return g_dev_tag[dev];
}

std::string tune_key(const std::string &dev, const ConvArgs &a, int layout, int dtype) {
    char k[192];
    snprintf(k, sizeof k, "%s|%d|%d|%d|%d|%d|%d|%d|%d|%d|%d|%d|%d", dev.c_str(), a.N, a.H, a.W, a.Cin, a.Cout,
             a.kh, a.kw, a.stride, a.pad, layout, dtype, a.res ? 1 : 0);
    return k;
}

bool splits_ok(const ConvArgs &a, int splits, size_t ws) {
    if (splits <= 1) return true;
    return (a.Cout % 8) == 0 && a.vec_out && (unsigned long long)splits * a.M * a.Cout * 4 <= ws &&
           (a.K + 63) / 64 >= splits;
}

bool halo_th_ok(const ConvArgs &a, int th) {
    const int wm = 4;  // waves along the rows: 4-wave workgroups, or 8 with k split over wave pairs
    const int fn = a.Cout <= 32 ? 1 : 2;
    return fn == 1 ? (th == wm || th == 2 * wm) : th == wm;
}

// Applies the table's entry for this call, if any and valid; p is the built-in choice.
void apply_tuned(const ConvArgs &a, int layout, int dtype, size_t ws, Plan *p) {
    if (g_tuned_n.load(std::memory_order_acquire) == 0) return;
    if (p->family != FAM_NHWC && p->family != FAM_HALO && p->family != FAM_HALO_WS && p->family != FAM_NCHW_VIA_NHWC &&
        p->family != FAM_HGEMM)
        return;
    const std::string dev = device_tag();
    if (dev.empty()) return;
    TunedEntry e;
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        auto it = g_tuned.find(tune_key(dev, a, layout, dtype));
        if (it == g_tuned.end()) return;
        e = it->second;
    }
    if (p->family == FAM_NCHW_VIA_NHWC || e.family == FAM_NCHW_VIA_NHWC) {
        // channel-first layers: the tile of the channel-last kernel (tile < NHWC_TILE_COUNT),
        // or halo-tile GEMM variant tile - kNchwHgTile with th the tile order
        if (p->family != FAM_NCHW_VIA_NHWC || e.family != FAM_NCHW_VIA_NHWC || e.tile < 0) return;
        if (e.tile < NHWC_TILE_COUNT) {
            p->nh.tile = e.tile;
            p->nchw_hg = false;
        } else {
            const int cfg = e.tile - kNchwHgTile;
            if (!hgemm_nchw_fits(a, layout, dtype) || !hgemm_cfg_ok(a, cfg, true) || (e.th != 0 && e.th != 1)) return;
            p->nchw_hg = true;
            p->hg.cfg = cfg;
            p->hg.cfast = e.th == 1;
        }
        p->tuned = true;
    } else if (e.family == FAM_HALO) {
        if (!halo_fits(a, layout, dtype) || !halo_th_ok(a, e.th)) return;
        p->family = FAM_HALO;
        p->halo = plan_halo(a);
        p->halo.th = e.th;
        p->tuned = true;
    } else if (e.family == FAM_HALO_WS) {
        if (!halo_fits(a, layout, dtype) || a.Cin != 64) return;
        p->family = FAM_HALO_WS;
        p->halo = plan_halo(a);
        p->tuned = true;
    } else if (e.family == FAM_HGEMM) {
        if (!hgemm_fits(a, layout, dtype) || !hgemm_cfg_ok(a, e.tile) || (e.th != 0 && e.th != 1)) return;
        p->family = FAM_HGEMM;
        p->hg.cfg = e.tile;
        p->hg.cfast = e.th == 1;
        p->tuned = true;
    } else if (e.family == FAM_NHWC) {
        if (e.tile < 0 || e.tile >= NHWC_TILE_COUNT || !splits_ok(a, e.splits, ws)) return;
        p->family = FAM_NHWC;
        p->nh = plan_nhwc(a, ws);
        p->nh.tile = e.tile;
        p->nh.splits = e.splits > 1 ? e.splits : 1;
        p->tuned = true;
    }
}

Plan make_plan(const ConvArgs &a, int layout, int dtype, size_t ws) {
    Plan p = make_plan_default(a, layout, dtype, ws);
    apply_tuned(a, layout, dtype, ws, &p);
    p.w_ohwi = a.w_ohwi != 0;
    return p;
}

// Channel-first layers with channel-last weights run only on the channel-last kernel
// (after the input's layout copy): 16-bit, Cin % 8 == 0, the copy within the workspace.
int check_w_ohwi(const ConvArgs &a, const Plan &p) {
    if (a.w_ohwi && p.family != FAM_NCHW_VIA_NHWC)
        return set_error(CONV2D_EUNSUPPORTED,
                         "CONV2D_WEIGHTS_OHWI needs a 16-bit layer with Cin %% 8 == 0 whose channel-last input copy "
                         "(%lld bytes) fits the workspace set by conv2d_set_workspace",
                         (long long)round256((size_t)a.N * a.H * a.W * a.Cin * 2));
    return CONV2D_OK;
}

int describe(const Plan &p, int layout, int dtype, char *buf, int cap) {
    char tmp[160];
    if (p.family == FAM_DIRECT) {
        snprintf(tmp, sizeof tmp, "direct_%s %s cob32", layout == CONV2D_LAYOUT_NCHW ? "nchw" : "nhwc",
                 dtype_name(dtype));
    } else if (p.family == FAM_STEM) {
        snprintf(tmp, sizeof tmp, "stem3x3_mfma %s", dtype_name(dtype));
    } else if (p.family == FAM_HALO) {
        snprintf(tmp, sizeof tmp, "halo3x3_nhwc %s th%d co%d w%d", dtype_name(dtype), p.halo.th, 32 * p.halo.fn,
                 p.halo.waves);
    } else if (p.family == FAM_HALO_WS) {
        snprintf(tmp, sizeof tmp, "halo3x3ws_nhwc %s th4 w4+4", dtype_name(dtype));
    } else if (p.family == FAM_HGEMM) {
        ConvArgs z{};
        HgemmInfo in{};
        (void)hgemm_cfg_info(p.hg.cfg, z, &in);
        snprintf(tmp, sizeof tmp, "%s %s v%d %dx%dx%d ck%d w%d %s", in.ws ? "hgemmws3x3_nhwc" : "hgemm3x3_nhwc",
                 dtype_name(dtype), p.hg.cfg, in.th, in.tw, in.cb, in.ck, in.waves, p.hg.cfast ? "cfast" : "pfast");
    } else if (p.family == FAM_NCHW_VIA_NHWC && p.nchw_hg) {
        ConvArgs z{};
        HgemmInfo in{};
        (void)hgemm_cfg_info(p.hg.cfg, z, &in);
        snprintf(tmp, sizeof tmp, "%shgemm3x3_nchw_out %s v%d %dx%dx%d ck%d w%d %s%s",
                 p.chain_in ? "chained+" : p.w_ohwi ? "x_to_nhwc+" : "to_nhwc+", dtype_name(dtype), p.hg.cfg, in.th,
                 in.tw, in.cb, in.ck, in.waves, p.hg.cfast ? "cfast" : "pfast", p.chain_out ? " +y_nhwc" : "");
    } else if (p.family == FAM_NHWC || p.family == FAM_NCHW_VIA_NHWC) {
        snprintf(tmp, sizeof tmp, "%sigemm_nhwc_pipe%s %s %s splitk=%d%s",
                 p.family == FAM_NCHW_VIA_NHWC ? (p.chain_in ? "chained+" : p.w_ohwi ? "x_to_nhwc+" : "to_nhwc+") : "",
                 p.nh.tap_inner ? "_tapinner" : "",
                 dtype_name(dtype), nhwc_tile_name(p.nh.tile), p.nh.splits, p.chain_out ? " +y_nhwc" : "");
    } else {
        snprintf(tmp, sizeof tmp, "igemm_%s%s %s %s", p.ig.nchw ? "nchw" : "nhwc",
                 p.ig.avec ? "_vec" : "_gather", dtype_name(dtype), tile_name(p.ig.tile));
    }
    if (p.tuned) strncat(tmp, " tuned", sizeof tmp - strlen(tmp) - 1);
    int n = (int)strlen(tmp);
    if (buf && cap > 0) {
        strncpy(buf, tmp, (size_t)cap - 1);
        buf[cap - 1] = 0;
    }
    return n;
}

int hip_fail(hipError_t e, const char *what) {
    return set_error(CONV2D_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int check_pool(const void *x, const void *y, int N, int H, int W, int C, int layout, int dtype,
               int OH, int OW, const char *name) {
    if (!x || !y) return set_error(CONV2D_EINVAL, "%s: x and y must not be null", name);
    if (N <= 0 || H <= 0 || W <= 0 || C <= 0)
        return set_error(CONV2D_EINVAL, "%s: sizes must be positive", name);
    if (layout != CONV2D_LAYOUT_NHWC && layout != CONV2D_LAYOUT_NCHW)
        return set_error(CONV2D_EINVAL, "%s: unknown layout %d", name, layout);
    if (!dtype_bytes(dtype)) return set_error(CONV2D_EINVAL, "%s: unknown dtype %d", name, dtype);
    if (OH < 1 || OW < 1) return set_error(CONV2D_EINVAL, "%s: input too small", name);
    long long xe = (long long)N * H * W * C, ye = (long long)N * OH * OW * C;
    if (xe > kMaxElems) return set_error(CONV2D_EUNSUPPORTED, "%s: tensor too large", name);
    int eb = dtype_bytes(dtype);
    if (overlap(y, ye * eb, x, xe * eb)) return set_error(CONV2D_EINVAL, "%s: y overlaps x", name);
    return CONV2D_OK;
}

// Launches the kernels of plan p for a validated conv (y = a.y); ws is the workspace the
// plan was made for. Returns a status code.
int launch_conv(const ConvArgs &a, const Plan &p, int layout, int dtype, const Workspace &ws, hipStream_t st) {
    hipError_t e;
    int rc;
    if (p.family == FAM_DIRECT) {
        e = launch_direct(a, dtype, layout == CONV2D_LAYOUT_NCHW, st);
    } else if (p.family == FAM_STEM) {
        e = launch_stem3(a, dtype, st);
    } else if (p.family == FAM_HALO) {
        int cus = 0;
        rc = device_cus(&cus);
        if (rc) return rc;
        HaloPlan h = p.halo;
        h.grid_cap = cus * (8 / h.waves);
        e = launch_halo3x3(a, dtype, h, st);
    } else if (p.family == FAM_HALO_WS) {
        int cus = 0;
        rc = device_cus(&cus);
        if (rc) return rc;
        e = launch_halo3x3_ws(a, dtype, cus, st);
    } else if (p.family == FAM_HGEMM) {
        e = launch_hgemm3x3(a, dtype, p.hg, false, st);
    } else if (p.family == FAM_NHWC) {
        e = launch_igemm_nhwc(a, dtype, p.nh, p.nh.splits > 1 ? reinterpret_cast<float *>(ws.p) : nullptr, st);
    } else if (p.family == FAM_NCHW_VIA_NHWC) {
        const int eb = dtype_bytes(dtype);
        char *base = ws.p;
        char *xs = base + (p.chain_in ? p.x_at : 0);
        char *ws = xs + round256((size_t)a.N * a.H * a.W * a.Cin * eb);
        // weights given channel-last (converted once by the caller) need no copy; a
        // chained layer's input copy was written by the layer before it
        if (p.chain_in)
            e = hipSuccess;
        else
            e = a.w_ohwi ? launch_nchw_to_nhwc(a.x, xs, a.N, a.Cin, a.H * a.W, dtype, st)
                         : launch_to_channel_last(a.x, xs, a.N, a.Cin, a.H * a.W, a.w, ws, a.Cout, a.kh * a.kw, dtype,
                                                  st);
        if (e == hipSuccess) {
            ConvArgs b = a;
            b.x = xs;
            b.w = a.w_ohwi ? a.w : ws;
            b.y2 = p.chain_out ? base + p.y2_at : nullptr;
            e = p.nchw_hg ? launch_hgemm3x3(b, dtype, p.hg, true, st) : launch_igemm_nhwc(b, dtype, p.nh, nullptr, st);
        }
    } else {
        e = launch_igemm(a, dtype, p.ig, st);
    }
    if (e != hipSuccess) return hip_fail(e, "conv2d_fused launch");
    return CONV2D_OK;
}

enum PoolKernel { POOL_TWO_KERNELS = 0, POOL_FUSED_STEM = 1, POOL_FUSED_HALO = 2 };

struct PoolFusion {
    int kind;        // PoolKernel
    Plan conv_plan;  // POOL_TWO_KERNELS: this conv into the workspace, then the pool kernel
};

// Validates conv2d_fused_maxpool3x3s2's arguments (y is the pooled map) and picks the
// fused kernel or the two-kernel path.
int check_conv_pool(const void *x, const void *w, const float *bias, const float *alpha, const void *y, int N, int H,
                    int W,
                    int Cin, int Cout, int kh, int kw, int stride, int pad, int act, int layout, int dtype,
                    size_t ws, ConvArgs *a, PoolFusion *f) {
    if (act & CONV2D_RES_BEFORE_ACT)
        return set_error(CONV2D_EINVAL, "conv2d_fused_maxpool3x3s2 takes no residual");
    if (act & CONV2D_WEIGHTS_OHWI)
        return set_error(CONV2D_EINVAL, "conv2d_fused_maxpool3x3s2 takes the weights in the layout's own order");
    int rc = check_conv(x, w, bias, alpha, nullptr, y, N, H, W, Cin, Cout, kh, kw, stride, pad, act, layout, dtype, a,
                        true);
    if (rc) return rc;
    const long long xbytes = (long long)N * H * W * Cin * dtype_bytes(dtype);
    f->kind = stem_fits(*a, layout, dtype) ? POOL_FUSED_STEM
              : (halo_fits(*a, layout, dtype) && Cin <= 32 && xbytes < (1ll << 31)) ? POOL_FUSED_HALO
                                                                                     : POOL_TWO_KERNELS;
    if (f->kind == POOL_TWO_KERNELS) {
        // the conv output goes to the workspace, which the conv kernels then must not
        // use themselves (planned without a workspace: no split-K, channel-first layers
        // on the general kernel)
        if ((unsigned long long)a->M * Cout * dtype_bytes(dtype) > ws)
            return set_error(CONV2D_EUNSUPPORTED,
                             "conv2d_fused_maxpool3x3s2: this shape runs as a conv and a pool kernel, whose unpooled "
                             "conv output (%lld bytes) needs a workspace of that size (conv2d_set_workspace; set: "
                             "%zu bytes); or call conv2d_fused and maxpool3x3s2",
                             (long long)a->M * Cout * dtype_bytes(dtype), ws);
        ConvArgs b = *a;
        b.vec_out = true;  // the workspace is 256-byte aligned
        f->conv_plan = make_plan(b, layout, dtype, 0);
    }
    return CONV2D_OK;
}

// Transposed conv 4x4/s2/p1: the matrix-core kernel for 16-bit types with Cin % 8 == 0
// (weights repacked into the workspace first; a channel-first input is transposed while
// it is staged), the direct kernel otherwise.
struct DeconvPlan {
    bool mfma;
    bool prepacked;  // the weights come packed by conv_transpose4x4s2_pack (da.wp)
    bool all;      // Cin <= 256: the kernel that stages the whole input strip at once
    bool x_copy;   // channel-first input copied to channel-last in the workspace first (all);
                   // else the kernel reads the planes (W % 8 == 0, x 16-byte aligned)
    size_t x_off;  // byte offset of that copy in the workspace (after the packed weights)
    bool out_f32;  // y in fp32 (16-bit input)
};

size_t deconv_packed_bytes(int Cin, int Cout, int eb) {
    return (size_t)16 * ((Cout + 31) / 32 * 32) * ((Cin + 63) / 64 * 64) * eb;
}

// packed: w is the caller's copy of the packed weights (conv_transpose4x4s2_pack).
int check_deconv(const void *x, const void *w, const float *bias, const float *alpha, const void *y, int N, int H,
                 int W, int Cin, int Cout, int act, int layout, int dtype, int out_dtype, size_t ws,
                 DeconvArgs *a, DeconvPlan *p, bool packed = false) {
    if (!x || !w || !y) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2: x, w and y must not be null");
    if (N <= 0 || H <= 0 || W <= 0 || Cin <= 0 || Cout <= 0)
        return set_error(CONV2D_EINVAL, "conv_transpose4x4s2: sizes must be positive (N=%d H=%d W=%d Cin=%d Cout=%d)",
                         N, H, W, Cin, Cout);
    if (layout != CONV2D_LAYOUT_NHWC && layout != CONV2D_LAYOUT_NCHW)
        return set_error(CONV2D_EINVAL, "conv_transpose4x4s2: unknown layout %d", layout);
    if (!dtype_bytes(dtype)) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2: unknown dtype %d", dtype);
    if (out_dtype != dtype && out_dtype != CONV2D_DTYPE_F32)
        return set_error(CONV2D_EINVAL, "conv_transpose4x4s2: out_dtype must be dtype or CONV2D_DTYPE_F32 (got %d)",
                         out_dtype);
    const int code = act & 0xff;
    if (code > CONV2D_ACT_PRELU || (act & ~0xff))
        return set_error(CONV2D_EINVAL, "conv_transpose4x4s2: unknown activation flags 0x%x", act);
    if (code == CONV2D_ACT_PRELU && !alpha) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2: PRELU needs alpha");
    const long long xe = (long long)N * H * W * Cin, we = 16ll * Cin * Cout, ye = 4ll * N * H * W * Cout;
    if (xe > kMaxElems || we > kMaxElems || ye > kMaxElems)
        return set_error(CONV2D_EUNSUPPORTED, "conv_transpose4x4s2: tensors of 2^31 or more elements are not supported");
    const int eb = dtype_bytes(dtype), ob = dtype_bytes(out_dtype);
    if (overlap(y, ye * ob, x, xe * eb)) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2: y overlaps x");
    const long long wbytes = packed ? (long long)deconv_packed_bytes(Cin, Cout, eb) : we * eb;
    if (overlap(y, ye * ob, w, wbytes)) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2: y overlaps w");
    *a = DeconvArgs{};
    a->x = x;
    a->w = w;
    a->bias = bias;
    a->alpha = code == CONV2D_ACT_PRELU ? alpha : nullptr;
    a->y = const_cast<void *>(y);
    a->N = N;
    a->H = H;
    a->W = W;
    a->Cin = Cin;
    a->Cout = Cout;
    a->CoP = (Cout + 31) / 32 * 32;
    a->act = code;
    *p = DeconvPlan{};
    p->out_f32 = out_dtype == CONV2D_DTYPE_F32 && dtype != CONV2D_DTYPE_F32;
    const bool nchw = layout == CONV2D_LAYOUT_NCHW;
    const size_t wp_bytes = (size_t)16 * a->CoP * ((Cin + 63) / 64 * 64) * eb;
    // the matrix cores need the weights packed into the workspace first (or packed once
    // by the caller); without room for them the direct kernel runs
    p->mfma = dtype != CONV2D_DTYPE_F32 && (Cin % 8) == 0 && wp_bytes <= ws && (nchw || aligned16(x)) &&
              xe * eb < (1ll << 31);
    // channel-first inputs with up to 256 channels: the kernel that stages the whole input
    // strip at once, reading the planes with 16-byte loads of 8-pixel segments when W % 8
    // == 0 and x is 16-byte aligned, else from a channel-last copy in the workspace (when
    // that fits beside the weights) made by a 16-byte transpose (element-by-element
    // staging from the planes measured slower than that copy; for channel-last inputs the
    // chunked kernel measured faster)
    if (packed) {
        // caller-owned packed weights: the matrix-core path only, the workspace only for the
        // channel-last copy of a channel-first input
        if (!(dtype != CONV2D_DTYPE_F32 && (Cin % 8) == 0 && wp_bytes < (1ull << 31) && (nchw || aligned16(x)) &&
              xe * eb < (1ll << 31)))
            return set_error(CONV2D_EUNSUPPORTED,
                             "conv_transpose4x4s2_prepacked: needs 16-bit x with Cin %% 8 == 0 (16-byte aligned "
                             "when channel-last) under 2 GiB");
        if (!aligned16(w)) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2_prepacked: wp must be 16-byte aligned");
        p->mfma = true;
        p->prepacked = true;
        a->wp = w;
    }
    p->x_off = packed ? 0 : round256(wp_bytes);
    p->x_copy = nchw && !((W % 8) == 0 && aligned16(x));
    p->all = p->mfma && nchw && Cin <= 256 && N <= 65535 &&
             p->x_off + (p->x_copy ? round256((size_t)(xe * eb)) : 0) <= ws;
    a->x_bytes = (uint32_t)(xe * eb < (1ll << 31) ? xe * eb : 0);
    a->wp_bytes = (uint32_t)wp_bytes;
    return CONV2D_OK;
}

// Upsample and concat: y = concat(up ? upsample2x(a) : a, b). H, W: a's size when up,
// else the common size.
int check_concat(const void *a, const void *b, const void *y, int N, int H, int W, int Ca, int Cb, bool up,
                 int layout, int dtype, const char *name) {
    if (!a || !y || (Cb > 0 && !b)) return set_error(CONV2D_EINVAL, "%s: inputs and y must not be null", name);
    if (N <= 0 || H <= 0 || W <= 0 || Ca <= 0 || Cb < 0)
        return set_error(CONV2D_EINVAL, "%s: sizes must be positive", name);
    if (layout != CONV2D_LAYOUT_NHWC && layout != CONV2D_LAYOUT_NCHW)
        return set_error(CONV2D_EINVAL, "%s: unknown layout %d", name, layout);
    if (!dtype_bytes(dtype)) return set_error(CONV2D_EINVAL, "%s: unknown dtype %d", name, dtype);
    const long long s = up ? 4 : 1;
    const long long ae = (long long)N * H * W * Ca, be = s * N * H * W * Cb, ye = s * N * H * W * (Ca + (long long)Cb);
    if (ye > kMaxElems) return set_error(CONV2D_EUNSUPPORTED, "%s: tensors of 2^31 or more elements are not supported",
                                         name);
    const int eb = dtype_bytes(dtype);
    if (overlap(y, ye * eb, a, ae * eb)) return set_error(CONV2D_EINVAL, "%s: y overlaps an input", name);
    if (Cb > 0 && overlap(y, ye * eb, b, be * eb)) return set_error(CONV2D_EINVAL, "%s: y overlaps an input", name);
    return CONV2D_OK;
}

bool concat_vec(const void *a, const void *b, const void *y, int H, int W, int Ca, int Cb, bool up, int layout,
                int dtype) {
    const int ve = 16 / dtype_bytes(dtype);
    const bool al = aligned16(a) && aligned16(y) && (Cb == 0 || aligned16(b));
    if (layout == CONV2D_LAYOUT_NHWC) return al && (Ca % ve) == 0 && (Cb % ve) == 0;
    return al && !up && ((long long)H * W) % ve == 0;
}

// One validated op of a call or a stack: everything its launch needs, decided on
// the host before anything is launched.
struct OpPlan {
    int kind;  // CONV2D_OP_*
    int layout, dtype;
    ConvArgs a;     // convs (a.y is the conv output, or the pooled map for the fused kernels)
    Plan plan;      // CONV2D_OP_CONV
    PoolFusion pf;  // CONV2D_OP_CONV_MAXPOOL
    const void *x;  // pools, copy
    void *y;
    int N, H, W, C;
    bool vec;      // pools, upsample/concat: the 16-byte kernels
    size_t bytes;  // copy
    DeconvArgs da;  // CONV2D_OP_DECONV
    DeconvPlan dp;
    const void *b;  // concat: second input
    int Ca, Cb;     // concat channels (Cb = 0: upsample)
    bool up;        // upsample the first input
    // stack fusion of a 2x2 average pool with the 1x1 conv that reads its output:
    // the pool op launches nothing (pool_by_next), the conv op runs both (pool_pw)
    bool pool_by_next;
    bool pool_pw;
    PoolPwArgs pp;
    // a conv whose output is marked transient (CONV2D_Y_TRANSIENT), and the stack fusion of
    // a stem conv with the stride-1 conv that reads its output: the first launches nothing
    // (pair_by_next), the second runs both (stem_pair, pa = the first conv's arguments)
    bool y_transient;
    bool pair_by_next;
    bool stem_pair;
    ConvArgs pa;
};

// Bytes of workspace the launch of a planned op writes (0 for none).
size_t ws_need(const OpPlan &o) {
    const int eb = dtype_bytes(o.dtype);
    if (o.kind == CONV2D_OP_CONV) {
        const ConvArgs &a = o.a;
        if (o.plan.family == FAM_NHWC && o.plan.nh.splits > 1) return (size_t)o.plan.nh.splits * a.M * a.Cout * 4;
        if (o.plan.family == FAM_NCHW_VIA_NHWC) {
            const size_t xb = round256((size_t)a.N * a.H * a.W * a.Cin * eb);
            const size_t wb = a.w_ohwi ? 0 : round256((size_t)a.Cout * a.K * eb);
            size_t need = (o.plan.chain_in ? o.plan.x_at : 0) + xb + wb;
            if (o.plan.chain_out) need = std::max(need, o.plan.y2_at + round256((size_t)a.M * a.Cout * eb));
            return need;
        }
        return 0;
    }
    if (o.kind == CONV2D_OP_CONV_MAXPOOL)
        return o.pf.kind == POOL_TWO_KERNELS ? round256((size_t)o.a.M * o.a.Cout * eb) : 0;
    if (o.kind == CONV2D_OP_DECONV && o.dp.mfma) {
        const size_t wp = o.dp.prepacked ? 0 : round256(o.da.wp_bytes);
        return wp + (o.dp.all && o.dp.x_copy ? round256((size_t)o.da.N * o.da.H * o.da.W * o.da.Cin * eb) : 0);
    }
    return 0;
}

int check_op(const conv2d_op &op, int layout, int dtype, size_t ws, OpPlan *o) {
    *o = OpPlan{};
    o->kind = op.kind;
    o->layout = layout;
    o->dtype = dtype;
    switch (op.kind) {
    case CONV2D_OP_CONV: {
        o->y_transient = (op.act & CONV2D_Y_TRANSIENT) != 0;
        int rc = check_conv(op.x, op.w, op.bias, op.alpha, op.residual, op.y, op.N, op.H, op.W, op.Cin, op.Cout, op.kh,
                            op.kw, op.stride, op.pad, op.act & ~CONV2D_Y_TRANSIENT, layout, dtype, &o->a);
        if (rc) return rc;
        o->a.bias = op.bias;
        if ((op.act & 0xff) != CONV2D_ACT_PRELU) o->a.alpha = nullptr;
        o->plan = make_plan(o->a, layout, dtype, ws);
        return check_w_ohwi(o->a, o->plan);
    }
    case CONV2D_OP_CONV_MAXPOOL: {
        if (op.residual) return set_error(CONV2D_EINVAL, "conv2d_fused_maxpool3x3s2 takes no residual");
        int rc = check_conv_pool(op.x, op.w, op.bias, op.alpha, op.y, op.N, op.H, op.W, op.Cin, op.Cout, op.kh, op.kw,
                                 op.stride, op.pad, op.act, layout, dtype, ws, &o->a, &o->pf);
        if (rc) return rc;
        o->a.bias = op.bias;
        if ((op.act & 0xff) != CONV2D_ACT_PRELU) o->a.alpha = nullptr;
        return CONV2D_OK;
    }
    case CONV2D_OP_MAXPOOL:
    case CONV2D_OP_AVGPOOL: {
        const bool mx = op.kind == CONV2D_OP_MAXPOOL;
        const int OH = mx ? out_dim(op.H, 3, 2, 1) : op.H / 2, OW = mx ? out_dim(op.W, 3, 2, 1) : op.W / 2;
        int rc = check_pool(op.x, op.y, op.N, op.H, op.W, op.Cin, layout, dtype, OH, OW,
                            mx ? "maxpool3x3s2" : "avgpool2x2");
        if (rc) return rc;
        const int ve = 16 / dtype_bytes(dtype);
        o->x = op.x;
        o->y = op.y;
        o->N = op.N;
        o->H = op.H;
        o->W = op.W;
        o->C = op.Cin;
        o->vec = layout == CONV2D_LAYOUT_NHWC && (op.Cin % ve) == 0 && aligned16(op.x) && aligned16(op.y);
        return CONV2D_OK;
    }
    case CONV2D_OP_COPY: {
        if (!op.x || !op.y) return set_error(CONV2D_EINVAL, "copy: x and y must not be null");
        if (op.N <= 0 || op.H <= 0 || op.W <= 0 || op.Cin <= 0)
            return set_error(CONV2D_EINVAL, "copy: sizes must be positive");
        if (!dtype_bytes(dtype)) return set_error(CONV2D_EINVAL, "copy: unknown dtype %d", dtype);
        const long long e = (long long)op.N * op.H * op.W * op.Cin;
        if (e > kMaxElems) return set_error(CONV2D_EUNSUPPORTED, "copy: tensor too large");
        o->bytes = (size_t)e * dtype_bytes(dtype);
        if (overlap(op.y, (long long)o->bytes, op.x, (long long)o->bytes))
            return set_error(CONV2D_EINVAL, "copy: y overlaps x");
        o->x = op.x;
        o->y = op.y;
        return CONV2D_OK;
    }
    case CONV2D_OP_DECONV:
        return check_deconv(op.x, op.w, op.bias, op.alpha, op.y, op.N, op.H, op.W, op.Cin, op.Cout, op.act, layout,
                            dtype, dtype, ws, &o->da, &o->dp);
    case CONV2D_OP_UPSAMPLE:
    case CONV2D_OP_CONCAT:
    case CONV2D_OP_UPSAMPLE_CONCAT: {
        const bool up = op.kind != CONV2D_OP_CONCAT;
        const int Cb = op.kind == CONV2D_OP_UPSAMPLE ? 0 : op.Cout;
        const char *name = op.kind == CONV2D_OP_UPSAMPLE ? "upsample_nearest2x"
                           : op.kind == CONV2D_OP_CONCAT ? "concat_channels"
                                                         : "upsample2x_concat";
        if (op.kind != CONV2D_OP_UPSAMPLE && Cb <= 0) return set_error(CONV2D_EINVAL, "%s: Cb must be positive", name);
        const void *b = Cb > 0 ? op.residual : nullptr;
        int rc = check_concat(op.x, b, op.y, op.N, op.H, op.W, op.Cin, Cb, up, layout, dtype, name);
        if (rc) return rc;
        o->x = op.x;
        o->b = b;
        o->y = op.y;
        o->N = op.N;
        o->H = up ? 2 * op.H : op.H;  // y's size
        o->W = up ? 2 * op.W : op.W;
        o->Ca = op.Cin;
        o->Cb = Cb;
        o->up = up;
        o->vec = concat_vec(op.x, b, op.y, o->H, o->W, op.Cin, Cb, up, layout, dtype);
        return CONV2D_OK;
    }
    default:
        return set_error(CONV2D_EINVAL, "unknown op kind %d", op.kind);
    }
}

// Chained channel-first convs of a stack: when a conv's output is the next op's input
// and both run on the channel-last kernel with channel-last weights (the IFNet block's
// chain), the producer (without a residual) also writes its output channel-last into
// one half of the workspace and the consumer reads that instead of copying its input;
// the halves alternate along the chain, so a layer never writes the half it reads.
void link_chains(std::vector<OpPlan> &plans, size_t ws) {
    const size_t half = ws / 2 & ~(size_t)255;
    for (size_t i = 0; i + 1 < plans.size(); ++i) {
        OpPlan &p = plans[i], &q = plans[i + 1];
        if (p.kind != CONV2D_OP_CONV || q.kind != CONV2D_OP_CONV) continue;
        if (p.plan.family != FAM_NCHW_VIA_NHWC || q.plan.family != FAM_NCHW_VIA_NHWC) continue;
        if (!p.plan.w_ohwi || !q.plan.w_ohwi || p.a.res || p.dtype != q.dtype) continue;
        if (q.a.x != p.a.y || q.a.N != p.a.N || q.a.H != p.a.OH || q.a.W != p.a.OW || q.a.Cin != p.a.Cout) continue;
        const int eb = dtype_bytes(p.dtype);
        const size_t in_bytes = round256((size_t)p.a.N * p.a.H * p.a.W * p.a.Cin * eb);
        const size_t out_bytes = round256((size_t)p.a.M * p.a.Cout * eb);
        const size_t at_in = p.plan.chain_in ? p.plan.x_at : 0;
        if (in_bytes > half || out_bytes > half) continue;
        p.plan.chain_out = true;
        p.plan.y2_at = at_in == 0 ? half : 0;
        q.plan.chain_in = true;
        q.plan.x_at = p.plan.y2_at;
    }
}

// A 2x2 average pool followed by a 1x1 stride-1 conv of its output (the ResNet-D
// shortcut) runs as one kernel: the conv op computes the pool while it stages its input
// and still writes the pooled map. Only where that kernel reproduces the two launches
// bit for bit: channel-last 16-bit, the conv on the general channel-last GEMM without a
// K split (products over k in increasing order from zero, bias in the epilogue), no
// residual, and no overlap between the conv output and the pool's tensors.
void link_pool_pw(std::vector<OpPlan> &plans) {
    for (size_t i = 0; i + 1 < plans.size(); ++i) {
        OpPlan &p = plans[i], &q = plans[i + 1];
        if (p.kind != CONV2D_OP_AVGPOOL || q.kind != CONV2D_OP_CONV || p.pool_by_next || q.pool_pw) continue;
        if (p.layout != CONV2D_LAYOUT_NHWC || p.dtype != q.dtype || !p.vec) continue;
        const ConvArgs &a = q.a;
        if (a.kh != 1 || a.kw != 1 || a.stride != 1 || a.pad != 0 || a.res || a.w_ohwi) continue;
        if (a.x != p.y || a.N != p.N || a.H != p.H / 2 || a.W != p.W / 2 || a.Cin != p.C) continue;
        if (q.plan.family != FAM_NHWC || q.plan.nh.splits != 1 || !poolpw_fits(a.Cin, a.Cout, q.dtype)) continue;
        const long long eb = dtype_bytes(q.dtype);
        const long long xb = (long long)p.N * p.H * p.W * p.C * eb, pb = (long long)a.M * a.Cin * eb;
        const long long yb = (long long)a.M * a.Cout * eb;
        if (xb >= (1ll << 31) || yb >= (1ll << 31) || !aligned16(a.y) || !aligned16(a.w)) continue;
        if (overlap(a.y, yb, p.x, xb) || overlap(a.y, yb, p.y, pb)) continue;
        PoolPwArgs pp{};
        pp.x = p.x;
        pp.w = a.w;
        pp.bias = a.bias;
        pp.alpha = a.alpha;
        pp.y = a.y;
        pp.p = p.y;
        pp.N = p.N;
        pp.H = p.H;
        pp.W = p.W;
        pp.OH = a.H;
        pp.OW = a.W;
        pp.Cin = a.Cin;
        pp.Cout = a.Cout;
        pp.act = a.act;
        p.pool_by_next = true;
        q.pool_pw = true;
        q.pp = pp;
    }
}

// A stem conv (3 -> 32 channels, stride 2) whose output is marked transient, followed by
// the stride-1 3x3 conv that reads it, runs as one kernel that never stores the first
// output (bit-identical to the two launches when the second would run on the halo
// kernel, its plan for such shapes).
void link_stem_pair(std::vector<OpPlan> &plans) {
    for (size_t i = 0; i + 1 < plans.size(); ++i) {
        OpPlan &p = plans[i], &q = plans[i + 1];
        if (p.kind != CONV2D_OP_CONV || q.kind != CONV2D_OP_CONV || !p.y_transient || p.pair_by_next || q.stem_pair)
            continue;
        if (p.layout != CONV2D_LAYOUT_NHWC || p.dtype != q.dtype || p.plan.family != FAM_STEM) continue;
        if (q.plan.family != FAM_HALO || q.pool_pw || !stem_pair_fits(p.a, q.a, q.dtype)) continue;
        const int eb = dtype_bytes(q.dtype);
        if (overlap(q.a.y, (long long)q.a.M * q.a.Cout * eb, p.a.x, (long long)p.a.N * p.a.H * p.a.W * 3 * eb)) continue;
        p.pair_by_next = true;
        q.stem_pair = true;
        q.pa = p.a;
    }
}

int check_stack(const conv2d_op *ops, int n, int layout, int dtype, size_t ws, std::vector<OpPlan> *plans,
                int *bad) {
    if (n < 0 || (n > 0 && !ops)) return set_error(CONV2D_EINVAL, "ops must hold n >= 0 entries");
    plans->resize((size_t)n);
    for (int i = 0; i < n; ++i) {
        int rc = check_op(ops[i], layout, dtype, ws, &(*plans)[(size_t)i]);
        if (rc) {
            if (bad) *bad = i;
            return set_error(rc, "op %d: %s", i, g_err.c_str());
        }
    }
    link_chains(*plans, ws);
    link_pool_pw(*plans);
    link_stem_pair(*plans);
    return CONV2D_OK;
}

// Host-side state the launches need (the CU count), fetched before any launch so that a
// captured stack makes no device query inside the capture.
int prepare_stack(const std::vector<OpPlan> &plans) {
    int cus = 0;
    return plans.empty() ? CONV2D_OK : device_cus(&cus);
}

int launch_op(const OpPlan &o, const Workspace &ws, hipStream_t st) {
    hipError_t e = hipSuccess;
    const bool nchw = o.layout == CONV2D_LAYOUT_NCHW;
    switch (o.kind) {
    case CONV2D_OP_CONV:
        if (o.pair_by_next) return CONV2D_OK;  // computed by the next op's kernel
        if (o.stem_pair) {
            int cus = 0;
            int rc = device_cus(&cus);
            if (rc) return rc;
            e = launch_stem_pair(o.pa, o.a, o.dtype, 3 * cus, st);
            return e == hipSuccess ? CONV2D_OK : hip_fail(e, "stem conv pair launch");
        }
        if (o.pool_pw) {
            e = launch_poolpw(o.pp, o.dtype, st);
            return e == hipSuccess ? CONV2D_OK : hip_fail(e, "avgpool2x2 + conv1x1 launch");
        }
        return launch_conv(o.a, o.plan, o.layout, o.dtype, ws, st);
    case CONV2D_OP_CONV_MAXPOOL: {
        const ConvArgs &a = o.a;
        if (o.pf.kind == POOL_FUSED_STEM) {
            e = launch_stem3_maxpool(a, a.y, o.dtype, st);
        } else if (o.pf.kind == POOL_FUSED_HALO) {
            int cus = 0;
            int rc = device_cus(&cus);
            if (rc) return rc;
            e = launch_halo3x3_maxpool(a, a.y, o.dtype, 2 * cus, st);
        } else {
            // the conv into the workspace, then the pool kernel
            ConvArgs b = a;
            b.y = ws.p;
            b.vec_out = true;
            int rc = launch_conv(b, o.pf.conv_plan, o.layout, o.dtype, Workspace{nullptr, 0}, st);
            if (rc) return rc;
            const int ve = 16 / dtype_bytes(o.dtype);
            const bool vec = !nchw && (a.Cout % ve) == 0 && aligned16(a.y);
            e = launch_maxpool(ws.p, a.y, a.N, a.OH, a.OW, a.Cout, nchw, o.dtype, vec, st);
        }
        if (e != hipSuccess) return hip_fail(e, "conv2d_fused_maxpool3x3s2 launch");
        return CONV2D_OK;
    }
    case CONV2D_OP_MAXPOOL:
        e = launch_maxpool(o.x, o.y, o.N, o.H, o.W, o.C, nchw, o.dtype, o.vec, st);
        return e == hipSuccess ? CONV2D_OK : hip_fail(e, "maxpool3x3s2 launch");
    case CONV2D_OP_AVGPOOL:
        if (o.pool_by_next) return CONV2D_OK;  // computed by the next op's kernel
        e = launch_avgpool(o.x, o.y, o.N, o.H, o.W, o.C, nchw, o.dtype, o.vec, st);
        return e == hipSuccess ? CONV2D_OK : hip_fail(e, "avgpool2x2 launch");
    case CONV2D_OP_COPY:
        e = launch_copy(o.x, o.y, o.bytes, st);
        return e == hipSuccess ? CONV2D_OK : hip_fail(e, "copy launch");
    case CONV2D_OP_DECONV: {
        if (!o.dp.mfma) {
            e = launch_deconv_direct(o.da, o.dtype, o.dp.out_f32, nchw, st);
            return e == hipSuccess ? CONV2D_OK : hip_fail(e, "conv_transpose4x4s2 launch");
        }
        DeconvArgs a = o.da;
        if (!o.dp.prepacked) {
            a.wp = ws.p;
            e = launch_deconv_pack(a.w, ws.p, a.Cin, a.Cout, a.CoP, o.dtype, st);
        }
        if (e == hipSuccess && o.dp.all) {
            if (o.dp.x_copy) {
                void *xs = ws.p + o.dp.x_off;
                e = launch_nchw_to_nhwc(a.x, xs, a.N, a.Cin, a.H * a.W, o.dtype, st);
                a.x = xs;
            }
            if (e == hipSuccess) e = launch_deconv_mfma_all(a, o.dtype, o.dp.out_f32, nchw, !o.dp.x_copy, st);
        } else if (e == hipSuccess) {
            e = launch_deconv_mfma(a, o.dtype, o.dp.out_f32, nchw, st);
        }
        return e == hipSuccess ? CONV2D_OK : hip_fail(e, "conv_transpose4x4s2 launch");
    }
    case CONV2D_OP_UPSAMPLE:
    case CONV2D_OP_CONCAT:
    case CONV2D_OP_UPSAMPLE_CONCAT:
        e = launch_concat(o.x, o.b, o.y, o.N, o.H, o.W, o.Ca, o.Cb, o.up, nchw, o.dtype, o.vec, st);
        return e == hipSuccess ? CONV2D_OK : hip_fail(e, "upsample/concat launch");
    default:
        return set_error(CONV2D_EINVAL, "unknown op kind %d", o.kind);
    }
}

int run_one(const conv2d_op &op, int layout, int dtype, void *stream, const Workspace &ws) {
    OpPlan o{};
    int rc = check_op(op, layout, dtype, ws.bytes, &o);
    if (rc) return rc;
    rc = launch_op(o, ws, static_cast<hipStream_t>(stream));
    return rc ? rc : set_ok();
}

int describe_op(const OpPlan &o, char *buf, int cap) {
    char tmp[200];
    switch (o.kind) {
    case CONV2D_OP_CONV:
        if (o.pair_by_next) {
            snprintf(tmp, sizeof tmp, "stem3x3_mfma %s (in the next op's kernel, output not stored)",
                     dtype_name(o.dtype));
            break;
        }
        if (o.stem_pair) {
            snprintf(tmp, sizeof tmp, "stem3x3+halo3x3_pair %s th8 co32 w4 (with the previous op)", dtype_name(o.dtype));
            break;
        }
        if (o.pool_pw) {
            snprintf(tmp, sizeof tmp, "avgpool2x2+conv1x1_nhwc %s %dx128 (with the previous op)",
                     dtype_name(o.dtype), o.a.Cin == 64 ? 64 : 32);
            break;
        }
        return describe(o.plan, o.layout, o.dtype, buf, cap);
    case CONV2D_OP_CONV_MAXPOOL:
        if (o.pf.kind == POOL_FUSED_STEM) {
            snprintf(tmp, sizeof tmp, "stem3x3_mfma %s fused with maxpool3x3s2", dtype_name(o.dtype));
        } else if (o.pf.kind == POOL_FUSED_HALO) {
            snprintf(tmp, sizeof tmp, "halo3x3_nhwc %s th4 co%d w4 fused with maxpool3x3s2", dtype_name(o.dtype),
                     o.a.Cout <= 32 ? 32 : 64);
        } else {
            char inner[160];
            describe(o.pf.conv_plan, o.layout, o.dtype, inner, sizeof inner);
            snprintf(tmp, sizeof tmp, "%s then maxpool3x3s2", inner);
        }
        break;
    case CONV2D_OP_MAXPOOL:
        snprintf(tmp, sizeof tmp, "maxpool3x3s2");
        break;
    case CONV2D_OP_AVGPOOL:
        snprintf(tmp, sizeof tmp, o.pool_by_next ? "avgpool2x2 (in the next op's kernel)" : "avgpool2x2");
        break;
    case CONV2D_OP_DECONV:
        if (o.dp.mfma)
            snprintf(tmp, sizeof tmp, "%s%sdeconv4x4s2_mfma%s_%s %s%s", o.dp.prepacked ? "" : "deconv4x4s2_pack+",
                     o.dp.all && o.dp.x_copy ? "to_nhwc+" : "", o.dp.all ? "_all" : "",
                     o.layout == CONV2D_LAYOUT_NCHW ? "nchw" : "nhwc", dtype_name(o.dtype),
                     o.dp.out_f32 ? " out f32" : "");
        else
            snprintf(tmp, sizeof tmp, "deconv4x4s2_direct %s%s", dtype_name(o.dtype), o.dp.out_f32 ? " out f32" : "");
        break;
    case CONV2D_OP_UPSAMPLE:
    case CONV2D_OP_CONCAT:
    case CONV2D_OP_UPSAMPLE_CONCAT:
        snprintf(tmp, sizeof tmp, "%s%s", o.kind == CONV2D_OP_UPSAMPLE ? "upsample2x" : o.up ? "upsample2x_concat" : "concat",
                 o.vec ? "_vec16" : "_scalar");
        break;
    default:
        snprintf(tmp, sizeof tmp, "copy");
        break;
    }
    int n = (int)strlen(tmp);
    if (buf && cap > 0) {
        strncpy(buf, tmp, (size_t)cap - 1);
        buf[cap - 1] = 0;
    }
    return n;
}

// Device buffers of one tuning run, freed on every path out.
struct TuneBuffers {
    void *p[6] = {};
    ~TuneBuffers() {
        for (void *q : p)
            if (q) (void)hipFree(q);
    }
};

int tune_run(int N, int H, int W, int Cin, int Cout, int kh, int kw, int stride, int pad, int act, int has_residual,
             int layout, int dtype, int reps, Plan *best_out, float *best_us) {
    if (reps < 1 || reps > 10000) return set_error(CONV2D_EINVAL, "conv2d_tune: reps must be in 1..10000");
    // validate the shape first with stand-in addresses (nothing is allocated for a bad call)
    {
        ConvArgs t{};
        const void *px = (const void *)(uintptr_t)0x100000000ull, *pw = (const void *)(uintptr_t)0x900000000ull;
        const void *py = (const void *)(uintptr_t)0x1100000000ull, *pr = (const void *)(uintptr_t)0x1900000000ull;
        const float *pa = (const float *)(uintptr_t)0x2100000000ull;
        int rc = check_conv(px, pw, nullptr, pa, has_residual ? pr : nullptr, py, N, H, W, Cin, Cout, kh, kw, stride, pad, act,
                            layout, dtype, &t);
        if (rc) return rc;
    }
    const int eb = dtype_bytes(dtype);
    const int OH = out_dim(H, kh, stride, pad), OW = out_dim(W, kw, stride, pad);
    const size_t sizes[6] = {(size_t)N * H * W * Cin * eb, (size_t)Cout * kh * kw * Cin * eb,
                             (size_t)N * OH * OW * Cout * eb, has_residual ? (size_t)N * OH * OW * Cout * eb : 0,
                             (size_t)Cout * 4, (size_t)Cout * 4};
    TuneBuffers b;
    for (int i = 0; i < 6; ++i) {
        if (!sizes[i]) continue;
        hipError_t e = hipMalloc(&b.p[i], sizes[i]);
        if (e != hipSuccess) return hip_fail(e, "conv2d_tune buffers");
        e = hipMemset(b.p[i], 0, sizes[i]);
        if (e != hipSuccess) return hip_fail(e, "conv2d_tune buffers");
    }
    ConvArgs a{};
    int rc = check_conv(b.p[0], b.p[1], (const float *)b.p[4], (const float *)b.p[5], b.p[3], b.p[2], N, H, W, Cin, Cout, kh, kw, stride,
                        pad, act, layout, dtype, &a);
    if (rc) return rc;
    a.bias = (const float *)b.p[4];
    if (a.act != CONV2D_ACT_PRELU) a.alpha = nullptr;
    // the candidates are the variants this thread's workspace allows (the same the
    // planner may later pick from for calls with that workspace)
    const Workspace ws = current_ws();
    const Plan def = make_plan_default(a, layout, dtype, ws.bytes);
    std::vector<Plan> cands;
    cands.push_back(def);
    if (def.family == FAM_NCHW_VIA_NHWC) {
        for (int tile = 0; tile < NHWC_TILE_COUNT; ++tile) {
            Plan c = def;
            c.nchw_hg = false;
            c.nh.tile = tile;
            cands.push_back(c);
        }
        if (hgemm_nchw_fits(a, layout, dtype)) {
            for (int cfg = 0; cfg < hgemm_cfg_count(); ++cfg)
                for (bool cf : {false, true}) {
                    if (!hgemm_cfg_ok(a, cfg, true)) continue;
                    Plan c = def;
                    c.nchw_hg = true;
                    c.hg.cfg = cfg;
                    c.hg.cfast = cf;
                    cands.push_back(c);
                }
        }
    } else if (def.family == FAM_NHWC || def.family == FAM_HALO || def.family == FAM_HALO_WS ||
               def.family == FAM_HGEMM) {
        if (hgemm_fits(a, layout, dtype)) {
            for (int cfg = 0; cfg < hgemm_cfg_count(); ++cfg)
                for (bool cf : {false, true}) {
                    if (!hgemm_cfg_ok(a, cfg)) continue;
                    Plan c{};
                    c.family = FAM_HGEMM;
                    c.hg.cfg = cfg;
                    c.hg.cfast = cf;
                    cands.push_back(c);
                }
        }
        if (halo_fits(a, layout, dtype) && a.Cin == 64 && def.family != FAM_HALO_WS) {
            Plan c{};
            c.family = FAM_HALO_WS;
            c.halo = plan_halo(a);
            cands.push_back(c);
        }
        if (halo_fits(a, layout, dtype)) {
            for (int th : {4, 8}) {
                if (!halo_th_ok(a, th)) continue;
                Plan c{};
                c.family = FAM_HALO;
                c.halo = plan_halo(a);
                c.halo.th = th;
                cands.push_back(c);
            }
        }
        for (int tile = 0; tile < NHWC_TILE_COUNT; ++tile)
            for (int sp : {1, 2, 3, 4}) {
                if (!splits_ok(a, sp, ws.bytes)) continue;
                Plan c{};
                c.family = FAM_NHWC;
                c.nh = plan_nhwc(a, ws.bytes);
                c.nh.tile = tile;
                c.nh.splits = sp;
                cands.push_back(c);
            }
    }
    // everything the launches need, fetched before timing
    int cus = 0;
    rc = device_cus(&cus);
    if (rc) return rc;
    hipStream_t st = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "conv2d_tune stream");
    hipEvent_t e0 = nullptr, e1 = nullptr;
    e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    int best = -1;
    float best_ms = 0.0f;
    for (size_t i = 0; i < cands.size() && e == hipSuccess; ++i) {
        for (int w = 0; w < 2 && rc == CONV2D_OK; ++w) rc = launch_conv(a, cands[i], layout, dtype, ws, st);
        if (rc) break;
        // the GPU idles while the host queues the timed launches (about 30 us of host
        // time each, more under a profiler), so host-side cost stays out of the timing
        e = launch_idle(std::min(4096, 8 + reps * 12), st);
        if (e != hipSuccess) break;
        e = hipEventRecord(e0, st);
        for (int r = 0; r < reps && rc == CONV2D_OK && e == hipSuccess; ++r)
            rc = launch_conv(a, cands[i], layout, dtype, ws, st);
        if (rc || e != hipSuccess) break;
        e = hipEventRecord(e1, st);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (e == hipSuccess && (best < 0 || ms < best_ms)) {
            best = (int)i;
            best_ms = ms;
        }
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    hipError_t es = hipStreamSynchronize(st);
    (void)hipStreamDestroy(st);
    if (rc) return rc;
    if (e != hipSuccess) return hip_fail(e, "conv2d_tune timing");
    if (es != hipSuccess) return hip_fail(es, "conv2d_tune");
    *best_out = cands[(size_t)best];
    *best_us = best_ms * 1e3f / (float)reps;
    // record the winner (only for the families the planner looks up)
    if (best_out->family == FAM_NHWC || best_out->family == FAM_HALO || best_out->family == FAM_HALO_WS ||
        best_out->family == FAM_NCHW_VIA_NHWC || best_out->family == FAM_HGEMM) {
        const std::string dev = device_tag();
        if (!dev.empty()) {
            TunedEntry t{best_out->family, best_out->nh.tile, best_out->nh.splits, best_out->halo.th};
            if (best_out->family == FAM_HGEMM) t = TunedEntry{FAM_HGEMM, best_out->hg.cfg, 1, best_out->hg.cfast ? 1 : 0};
            if (best_out->family == FAM_NCHW_VIA_NHWC && best_out->nchw_hg)
                t = TunedEntry{FAM_NCHW_VIA_NHWC, kNchwHgTile + best_out->hg.cfg, 1, best_out->hg.cfast ? 1 : 0};
            std::lock_guard<std::mutex> lock(g_tune_mu);
            g_tuned[tune_key(dev, a, layout, dtype)] = t;
            g_tuned_n.store((int)g_tuned.size(), std::memory_order_release);
        }
        best_out->tuned = true;
    }
    return CONV2D_OK;
}

}  // namespace

extern "C" {

int conv2d_abi_version(void) { return 10; }

const char *conv2d_last_error(void) { return g_err.c_str(); }

int conv2d_out_dim(int in, int k, int stride, int pad) { return out_dim(in, k, stride, pad); }

int conv2d_check_args(const void *x, const void *w, const float *bias, const float *alpha,
                      const void *residual, const void *y, int N, int H, int W, int Cin,
                      int Cout, int kh, int kw, int stride, int pad, int act, int layout,
                      int dtype) {
    ConvArgs a{};
    int rc = check_conv(x, w, bias, alpha, residual, y, N, H, W, Cin, Cout, kh, kw, stride, pad, act,
                        layout, dtype, &a);
    if (!rc && a.w_ohwi) rc = check_w_ohwi(a, make_plan(a, layout, dtype, current_ws().bytes));
    return rc ? rc : set_ok();
}

int conv2d_plan(int N, int H, int W, int Cin, int Cout, int kh, int kw, int stride, int pad,
                int act, int layout, int dtype, char *buf, int cap) {
    // Stand-in addresses (never dereferenced): aligned, non-overlapping.
    const void *px = (const void *)(uintptr_t)0x100000000ull;
    const void *pw = (const void *)(uintptr_t)0x900000000ull;
    const void *py = (const void *)(uintptr_t)0x1100000000ull;
    const float *pa = (const float *)(uintptr_t)0x1900000000ull;
    ConvArgs a{};
    int rc = check_conv(px, pw, nullptr, pa, nullptr, py, N, H, W, Cin, Cout, kh, kw, stride, pad, act,
                        layout, dtype, &a);
    if (rc) return rc;
    const Plan pl = make_plan(a, layout, dtype, current_ws().bytes);
    rc = check_w_ohwi(a, pl);
    if (rc) return rc;
    set_ok();
    return describe(pl, layout, dtype, buf, cap);
}

int conv2d_fused(const void *x, const void *w, const float *bias, const float *alpha,
                 const void *residual, void *y, int N, int H, int W, int Cin, int Cout, int kh,
                 int kw, int stride, int pad, int act, int layout, int dtype, void *stream) {
    const conv2d_op op{CONV2D_OP_CONV, x, w, bias, alpha, residual, y, N, H, W, Cin, Cout, kh, kw, stride, pad, act};
    return run_one(op, layout, dtype, stream, current_ws());
}

int conv2d_fused_maxpool3x3s2(const void *x, const void *w, const float *bias, const float *alpha, void *y,
                              int N, int H, int W, int Cin, int Cout, int kh, int kw, int stride, int pad,
                              int act, int layout, int dtype, void *stream) {
    const conv2d_op op{CONV2D_OP_CONV_MAXPOOL, x, w, bias, alpha, nullptr, y, N, H, W, Cin, Cout, kh, kw,
                       stride, pad, act};
    return run_one(op, layout, dtype, stream, current_ws());
}

int conv2d_fused_maxpool_plan(int N, int H, int W, int Cin, int Cout, int kh, int kw, int stride, int pad,
                              int act, int layout, int dtype, char *buf, int cap) {
    const void *px = (const void *)(uintptr_t)0x100000000ull;
    const void *pw = (const void *)(uintptr_t)0x900000000ull;
    void *py = (void *)(uintptr_t)0x1100000000ull;
    const float *pa = (const float *)(uintptr_t)0x1900000000ull;
    const conv2d_op op{CONV2D_OP_CONV_MAXPOOL, px, pw, nullptr, pa, nullptr, py, N, H, W, Cin, Cout, kh, kw,
                       stride, pad, act};
    OpPlan o{};
    int rc = check_op(op, layout, dtype, current_ws().bytes, &o);
    if (rc) return rc;
    set_ok();
    return describe_op(o, buf, cap);
}

int maxpool3x3s2(const void *x, void *y, int N, int H, int W, int C, int layout, int dtype,
                 void *stream) {
    const conv2d_op op{CONV2D_OP_MAXPOOL, x, nullptr, nullptr, nullptr, nullptr, y, N, H, W, C, C, 3, 3, 2, 1, 0};
    return run_one(op, layout, dtype, stream, current_ws());
}

int avgpool2x2(const void *x, void *y, int N, int H, int W, int C, int layout, int dtype,
               void *stream) {
    const conv2d_op op{CONV2D_OP_AVGPOOL, x, nullptr, nullptr, nullptr, nullptr, y, N, H, W, C, C, 2, 2, 2, 0, 0};
    return run_one(op, layout, dtype, stream, current_ws());
}

int conv_transpose4x4s2(const void *x, const void *w, const float *bias, const float *alpha, void *y, int N, int H,
                        int W, int Cin, int Cout, int act, int layout, int dtype, int out_dtype, void *stream) {
    OpPlan o{};
    o.kind = CONV2D_OP_DECONV;
    o.layout = layout;
    o.dtype = dtype;
    const Workspace ws = current_ws();
    int rc = check_deconv(x, w, bias, alpha, y, N, H, W, Cin, Cout, act, layout, dtype, out_dtype, ws.bytes, &o.da,
                          &o.dp);
    if (rc) return rc;
    rc = launch_op(o, ws, static_cast<hipStream_t>(stream));
    return rc ? rc : set_ok();
}

int conv_transpose4x4s2_packed_bytes(int Cin, int Cout, int dtype, size_t *bytes) {
    if (!bytes) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2_packed_bytes: bytes must not be null");
    if (Cin <= 0 || Cout <= 0) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2_packed_bytes: sizes must be positive");
    if (dtype != CONV2D_DTYPE_BF16 && dtype != CONV2D_DTYPE_F16)
        return set_error(CONV2D_EUNSUPPORTED, "conv_transpose4x4s2_packed_bytes: packing is for 16-bit weights");
    *bytes = deconv_packed_bytes(Cin, Cout, 2);
    return set_ok();
}

int conv_transpose4x4s2_pack(const void *w, void *wp, int Cin, int Cout, int dtype, void *stream) {
    if (!w || !wp) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2_pack: w and wp must not be null");
    if (Cin <= 0 || Cout <= 0) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2_pack: sizes must be positive");
    if (dtype != CONV2D_DTYPE_BF16 && dtype != CONV2D_DTYPE_F16)
        return set_error(CONV2D_EUNSUPPORTED, "conv_transpose4x4s2_pack: packing is for 16-bit weights");
    if ((Cin % 8) != 0) return set_error(CONV2D_EUNSUPPORTED, "conv_transpose4x4s2_pack: Cin must be a multiple of 8");
    const size_t wb = deconv_packed_bytes(Cin, Cout, 2);
    if (wb >= (1ull << 31) || 16ll * Cin * Cout > kMaxElems)
        return set_error(CONV2D_EUNSUPPORTED, "conv_transpose4x4s2_pack: packed weights of 2 GiB or more");
    if (!aligned16(wp)) return set_error(CONV2D_EINVAL, "conv_transpose4x4s2_pack: wp must be 16-byte aligned");
    if (overlap(wp, (long long)wb, w, 32ll * Cin * Cout))
        return set_error(CONV2D_EINVAL, "conv_transpose4x4s2_pack: wp overlaps w");
    hipError_t e = launch_deconv_pack(w, wp, Cin, Cout, (Cout + 31) / 32 * 32, dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "conv_transpose4x4s2_pack launch");
    return set_ok();
}

int conv_transpose4x4s2_prepacked(const void *x, const void *wp, const float *bias, const float *alpha, void *y, int N,
                                  int H, int W, int Cin, int Cout, int act, int layout, int dtype, int out_dtype,
                                  void *stream) {
    OpPlan o{};
    o.kind = CONV2D_OP_DECONV;
    o.layout = layout;
    o.dtype = dtype;
    const Workspace ws = current_ws();
    int rc = check_deconv(x, wp, bias, alpha, y, N, H, W, Cin, Cout, act, layout, dtype, out_dtype, ws.bytes, &o.da,
                          &o.dp, true);
    if (rc) return rc;
    rc = launch_op(o, ws, static_cast<hipStream_t>(stream));
    return rc ? rc : set_ok();
}

int conv_transpose4x4s2_plan(int N, int H, int W, int Cin, int Cout, int act, int layout, int dtype, int out_dtype,
                             char *buf, int cap) {
    OpPlan o{};
    o.kind = CONV2D_OP_DECONV;
    o.layout = layout;
    o.dtype = dtype;
    const void *px = (const void *)(uintptr_t)0x100000000ull;
    const void *pw = (const void *)(uintptr_t)0x900000000ull;
    const void *py = (const void *)(uintptr_t)0x1100000000ull;
    const float *pa = (const float *)(uintptr_t)0x1900000000ull;
    int rc = check_deconv(px, pw, nullptr, pa, py, N, H, W, Cin, Cout, act, layout, dtype, out_dtype,
                          current_ws().bytes, &o.da, &o.dp);
    if (rc) return rc;
    set_ok();
    return describe_op(o, buf, cap);
}

int upsample_nearest2x(const void *x, void *y, int N, int H, int W, int C, int layout, int dtype, void *stream) {
    const conv2d_op op{CONV2D_OP_UPSAMPLE, x, nullptr, nullptr, nullptr, nullptr, y, N, H, W, C, 0, 0, 0, 0, 0, 0};
    return run_one(op, layout, dtype, stream, current_ws());
}

int concat_channels(const void *a, const void *b, void *y, int N, int H, int W, int Ca, int Cb, int layout, int dtype,
                    void *stream) {
    const conv2d_op op{CONV2D_OP_CONCAT, a, nullptr, nullptr, nullptr, b, y, N, H, W, Ca, Cb, 0, 0, 0, 0, 0};
    return run_one(op, layout, dtype, stream, current_ws());
}

int upsample2x_concat(const void *a, const void *b, void *y, int N, int H, int W, int Ca, int Cb, int layout,
                      int dtype, void *stream) {
    const conv2d_op op{CONV2D_OP_UPSAMPLE_CONCAT, a, nullptr, nullptr, nullptr, b, y, N, H, W, Ca, Cb, 0, 0, 0, 0, 0};
    return run_one(op, layout, dtype, stream, current_ws());
}

int conv2d_tune(int N, int H, int W, int Cin, int Cout, int kh, int kw, int stride, int pad, int act, int has_residual,
                int layout, int dtype, int reps, float *best_us, char *buf, int cap) {
    Plan best{};
    float us = 0.0f;
    int rc = tune_run(N, H, W, Cin, Cout, kh, kw, stride, pad, act, has_residual, layout, dtype, reps, &best, &us);
    if (rc) return rc;
    if (best_us) *best_us = us;
    set_ok();
    return describe(best, layout, dtype, buf, cap);
}

int conv2d_tune_save(const char *path) {
    if (!path) return set_error(CONV2D_EINVAL, "conv2d_tune_save: path must not be null");
    std::map<std::string, TunedEntry> copy;
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        copy = g_tuned;
    }
    FILE *f = fopen(path, "w");
    if (!f) return set_error(CONV2D_EINVAL, "conv2d_tune_save: cannot open %s", path);
    fprintf(f, "# conv2d tuned plans v1: device|N|H|W|Cin|Cout|kh|kw|stride|pad|layout|dtype|residual family tile splits th\n");
    for (const auto &kv : copy)
        fprintf(f, "%s %d %d %d %d\n", kv.first.c_str(), kv.second.family, kv.second.tile, kv.second.splits,
                kv.second.th);
    const bool bad = ferror(f) != 0;
    if (fclose(f) != 0 || bad) return set_error(CONV2D_EINVAL, "conv2d_tune_save: write to %s failed", path);
    set_ok();
    return (int)copy.size();
}

int conv2d_tune_load(const char *path) {
    if (!path) return set_error(CONV2D_EINVAL, "conv2d_tune_load: path must not be null");
    FILE *f = fopen(path, "r");
    if (!f) return set_error(CONV2D_EINVAL, "conv2d_tune_load: cannot open %s", path);
    std::map<std::string, TunedEntry> add;
    char line[512];
    int lineno = 0;
    while (fgets(line, sizeof line, f)) {
        ++lineno;
        if (line[0] == '#' || line[0] == '\n' || line[0] == 0) continue;
        char key[256];
        TunedEntry t{};
        char extra[4];
        const int got = sscanf(line, "%255s %d %d %d %d %3s", key, &t.family, &t.tile, &t.splits, &t.th, extra);
        int bars = 0;
        for (const char *c = key; *c; ++c) bars += *c == '|';
        const bool ok = got == 5 && bars == 12 && ((t.family == FAM_NHWC && t.tile >= 0 && t.tile < NHWC_TILE_COUNT &&
                                                    t.splits >= 1 && t.splits <= 4) ||
                                                   (t.family == FAM_NCHW_VIA_NHWC && t.tile >= 0 &&
                                                    t.tile < NHWC_TILE_COUNT && t.splits == 1) ||
                                                   (t.family == FAM_NCHW_VIA_NHWC && t.tile >= kNchwHgTile &&
                                                    t.tile < kNchwHgTile + hgemm_cfg_count() && t.splits == 1 &&
                                                    (t.th == 0 || t.th == 1)) ||
                                                   (t.family == FAM_HALO && (t.th == 4 || t.th == 8)) ||
                                                   (t.family == FAM_HALO_WS && t.th == 4) ||
                                                   (t.family == FAM_HGEMM && t.tile >= 0 && t.tile < hgemm_cfg_count() &&
                                                    t.splits == 1 && (t.th == 0 || t.th == 1)));
        if (!ok) {
            fclose(f);
            return set_error(CONV2D_EINVAL, "conv2d_tune_load: %s line %d is not a tuned-plan record", path, lineno);
        }
        add[key] = t;
    }
    fclose(f);
    std::lock_guard<std::mutex> lock(g_tune_mu);
    for (const auto &kv : add) g_tuned[kv.first] = kv.second;
    g_tuned_n.store((int)g_tuned.size(), std::memory_order_release);
    set_ok();
    return (int)add.size();
}

int conv2d_tune_clear(void) {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_tuned.clear();
    g_tuned_n.store(0, std::memory_order_release);
    return set_ok();
}

int conv2d_weights_to_ohwi(const void *w, void *w2, int Cout, int Cin, int kh, int kw, int dtype, void *stream) {
    if (!w || !w2) return set_error(CONV2D_EINVAL, "conv2d_weights_to_ohwi: w and w2 must not be null");
    if (Cout <= 0 || Cin <= 0 || kh <= 0 || kw <= 0)
        return set_error(CONV2D_EINVAL, "conv2d_weights_to_ohwi: sizes must be positive");
    if (dtype != CONV2D_DTYPE_BF16 && dtype != CONV2D_DTYPE_F16)
        return set_error(CONV2D_EUNSUPPORTED, "conv2d_weights_to_ohwi: for the 16-bit types");
    const long long e = (long long)Cout * Cin * kh * kw;
    if (e > kMaxElems) return set_error(CONV2D_EUNSUPPORTED, "conv2d_weights_to_ohwi: too large");
    if (overlap(w2, e * 2, w, e * 2)) return set_error(CONV2D_EINVAL, "conv2d_weights_to_ohwi: w2 overlaps w");
    hipError_t er = launch_oihw_to_ohwi(w, w2, Cout, Cin, kh * kw, dtype, static_cast<hipStream_t>(stream));
    if (er != hipSuccess) return hip_fail(er, "conv2d_weights_to_ohwi launch");
    return set_ok();
}

int conv2d_stack_check(const conv2d_op *ops, int n, int layout, int dtype, int *bad_index) {
    if (bad_index) *bad_index = -1;
    std::vector<OpPlan> plans;
    int rc = check_stack(ops, n, layout, dtype, current_ws().bytes, &plans, bad_index);
    return rc ? rc : set_ok();
}

int conv2d_stack_plan(const conv2d_op *ops, int n, int layout, int dtype, int index, char *buf, int cap) {
    std::vector<OpPlan> plans;
    int bad = -1;
    int rc = check_stack(ops, n, layout, dtype, current_ws().bytes, &plans, &bad);
    if (rc) return rc;
    if (index < 0 || index >= n) return set_error(CONV2D_EINVAL, "op index %d outside the stack of %d", index, n);
    set_ok();
    return describe_op(plans[(size_t)index], buf, cap);
}

int conv2d_stack_run(const conv2d_op *ops, int n, int layout, int dtype, void *stream) {
    std::vector<OpPlan> plans;
    int bad = -1;
    const Workspace ws = current_ws();
    int rc = check_stack(ops, n, layout, dtype, ws.bytes, &plans, &bad);
    if (rc) return rc;
    rc = prepare_stack(plans);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int i = 0; i < n; ++i) {
        rc = launch_op(plans[(size_t)i], ws, st);
        if (rc) return set_error(rc, "op %d: %s", i, g_err.c_str());
    }
    return set_ok();
}

struct conv2d_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
    int ops;
};

int conv2d_stack_graph_create(const conv2d_op *ops, int n, int layout, int dtype, conv2d_graph **out) {
    if (!out) return set_error(CONV2D_EINVAL, "out must not be null");
    *out = nullptr;
    std::vector<OpPlan> plans;
    int bad = -1;
    // the graph keeps the workspace set now: its replays use that memory
    const Workspace ws = current_ws();
    int rc = check_stack(ops, n, layout, dtype, ws.bytes, &plans, &bad);
    if (rc) return rc;
    // everything that queries the device happens before the capture
    rc = prepare_stack(plans);
    if (rc) return rc;
    hipStream_t cs = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "capture stream");
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(cs);
        return hip_fail(e, "hipStreamBeginCapture");
    }
    int lrc = CONV2D_OK;
    std::string lerr;
    for (int i = 0; i < n && lrc == CONV2D_OK; ++i) {
        lrc = launch_op(plans[(size_t)i], ws, cs);
        if (lrc) lerr = "op " + std::to_string(i) + ": " + g_err;
    }
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(cs, &g);
    (void)hipStreamDestroy(cs);
    if (lrc) {
        if (g) (void)hipGraphDestroy(g);
        return set_error(lrc, "%s", lerr.c_str());
    }
    if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
    hipGraphExec_t x = nullptr;
    e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(g);
        return hip_fail(e, "hipGraphInstantiate");
    }
    conv2d_graph *h = new (std::nothrow) conv2d_graph{g, x, n};
    if (!h) {
        (void)hipGraphExecDestroy(x);
        (void)hipGraphDestroy(g);
        return set_error(CONV2D_EHIP, "out of host memory");
    }
    *out = h;
    return set_ok();
}

int conv2d_stack_graph_launch(conv2d_graph *g, void *stream) {
    if (!g) return set_error(CONV2D_EINVAL, "graph must not be null");
    hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
    return set_ok();
}

int conv2d_stack_graph_destroy(conv2d_graph *g) {
    if (!g) return set_ok();
    hipError_t e1 = hipGraphExecDestroy(g->exec);
    hipError_t e2 = hipGraphDestroy(g->graph);
    delete g;
    if (e1 != hipSuccess) return hip_fail(e1, "hipGraphExecDestroy");
    if (e2 != hipSuccess) return hip_fail(e2, "hipGraphDestroy");
    return set_ok();
}

}  // extern "C"

namespace {

// Scratch of conv2d_fused_noalloc, for callers that cannot allocate device memory: one
// copy of this array per GPU, held until the process ends. In host code its name is
// only a stand-in; the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and is the only form passed to kernels.
constexpr size_t kNoAllocScratchBytes = 16ull << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

char *g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int noalloc_scratch(Workspace *ws) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "conv2d_fused_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return set_error(CONV2D_EHIP, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_fail(e, "conv2d_fused_noalloc: hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = static_cast<char *>(ptr);
    }
    *ws = Workspace{g_scratch_ptr[dev], kNoAllocScratchBytes};
    return CONV2D_OK;
}

}  // namespace

extern "C" {

int conv2d_fused_noalloc(const void *x, const void *w, const float *bias, const float *alpha,
                         const void *residual, void *y, int N, int H, int W, int Cin, int Cout, int kh,
                         int kw, int stride, int pad, int act, int layout, int dtype, void *stream) {
    const conv2d_op op{CONV2D_OP_CONV, x, w, bias, alpha, residual, y, N, H, W, Cin, Cout, kh, kw, stride, pad, act};
    // the variant conv2d_fused takes with all the workspace it wants; its scratch must
    // fit the static array (nothing is launched otherwise)
    OpPlan o{};
    int rc = check_op(op, layout, dtype, kUnlimitedWs, &o);
    if (rc) return rc;
    const size_t need = ws_need(o);
    if (need > kNoAllocScratchBytes)
        return set_error(CONV2D_EUNSUPPORTED,
                         "conv2d_fused_noalloc: this layer's kernels need %zu bytes of scratch, more than the %zu "
                         "bytes of the library's static scratch; use conv2d_fused with a workspace",
                         need, kNoAllocScratchBytes);
    Workspace ws{};
    rc = noalloc_scratch(&ws);
    if (rc) return rc;
    return run_one(op, layout, dtype, stream, ws);
}

int conv2d_set_workspace(void *p, size_t bytes) {
    if (!p && bytes) return set_error(CONV2D_EINVAL, "conv2d_set_workspace: a null workspace must have 0 bytes");
    if (((uintptr_t)p & 255u) != 0) return set_error(CONV2D_EINVAL, "conv2d_set_workspace: p must be 256-byte aligned");
    const int dev = ws_slot();
    if (dev < 0 || dev >= kMaxDevices) return set_error(CONV2D_EHIP, "device index %d out of range", dev);
    g_ws[dev] = Workspace{static_cast<char *>(p), p ? bytes : 0};
    return CONV2D_OK;  // a setter: the thread's last error stays as it was
}

int conv2d_workspace_size(int N, int H, int W, int Cin, int Cout, int kh, int kw, int stride, int pad, int act,
                          int layout, int dtype, size_t *bytes) {
    if (!bytes) return set_error(CONV2D_EINVAL, "conv2d_workspace_size: bytes must not be null");
    const void *px = (const void *)(uintptr_t)0x100000000ull;
    const void *pw = (const void *)(uintptr_t)0x900000000ull;
    void *py = (void *)(uintptr_t)0x1100000000ull;
    const float *pa = (const float *)(uintptr_t)0x1900000000ull;
    const conv2d_op op{CONV2D_OP_CONV, px, pw, nullptr, pa, nullptr, py, N, H, W, Cin, Cout, kh, kw, stride, pad, act};
    OpPlan o{};
    int rc = check_op(op, layout, dtype, kUnlimitedWs, &o);
    if (rc) return rc;
    *bytes = ws_need(o);
    return set_ok();
}

int conv2d_stack_workspace_size(const conv2d_op *ops, int n, int layout, int dtype, size_t *bytes) {
    if (!bytes) return set_error(CONV2D_EINVAL, "conv2d_stack_workspace_size: bytes must not be null");
    std::vector<OpPlan> plans;
    int bad = -1;
    int rc = check_stack(ops, n, layout, dtype, kUnlimitedWs, &plans, &bad);
    if (rc) return rc;
    // chained convs use two halves, each holding an input or output copy; the other ops
    // use the workspace from its start
    size_t need = 0, half = 0;
    for (const OpPlan &o : plans) {
        if (o.kind == CONV2D_OP_CONV && (o.plan.chain_in || o.plan.chain_out)) {
            const int eb = dtype_bytes(o.dtype);
            half = std::max(half, round256((size_t)o.a.N * o.a.H * o.a.W * o.a.Cin * eb));
            half = std::max(half, round256((size_t)o.a.M * o.a.Cout * eb));
        } else {
            need = std::max(need, ws_need(o));
        }
    }
    *bytes = std::max(need, 2 * half);
    return set_ok();
}

}  // extern "C"
