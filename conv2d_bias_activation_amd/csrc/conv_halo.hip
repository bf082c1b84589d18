// 3x3 stride-1 pad-1 channel-last convolution for narrow layers (Cin 16/32/64,
// Cout <= 64) on CDNA4 matrix cores, with halo tiles.
//
// The GEMM is the one of the implicit-GEMM kernels (m = output pixel, k = (tap,
// input channel), n = output channel; inferencelayer page, `conv()` with its im2col
// and fused bias/activation epilogue), but the patch matrix is never gathered row by
// row: a workgroup stages the input pixels of a TH x 32 output tile plus a one-pixel
// border, (TH+2) x 34 pixels x Cin, in LDS once, and the nine taps read their A
// operands from that one copy at shifted pixel positions (the halo tiles of the
// WebGPU page's convolution shader). Input bytes move HBM -> LDS about
// (TH+2)*34/(TH*32) times instead of nine times.
//
//  * Weights stay in registers: with Cin <= 64 one wave's 32 output channels over
//    all 9*Cin k are 9*Cin/16 operand fragments of 4 VGPRs (144 VGPRs at Cin 64),
//    loaded once per workgroup.
//  * Workgroups are persistent: each walks tiles t = k*G + r (r its XCD-grouped
//    index among G), with the halo of tile k+2 loading into the buffer tile k just
//    released while tile k's epilogue and tile k+1's products run.
//  * The halo copy goes straight from memory into LDS (16-byte direct-to-LDS loads,
//    out-of-image pixels as out-of-range offsets that read zeros). A pixel takes
//    Cin/8 + 1 16-byte slots (the last one is padding), an odd number of 16-byte
//    bank groups, so the 16 consecutive pixels that a quarter-wave reads for one
//    operand fall in 16 distinct groups of the 64 banks, and every operand address
//    is the lane's base plus a compile-time offset.
#include "igemm_common.hpp"
#include "kernels.hpp"

namespace c2d {

namespace {

template <int N> __device__ __forceinline__ void halo_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void halo_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace

// CIN input channels (16, 32 or 64); TH output rows per tile (tiles are TH x 32);
// WN waves along the output channels (32 each), 8 / WN waves along the tile rows.
template <typename T, int CIN, int TH, int WN>
__global__ __launch_bounds__(512) void halo3x3_kernel(ConvArgs a, int tiles_w, int tiles_h, int ntiles) {
    constexpr int NW = 8;
    constexpr int WM = NW / WN;
    constexpr int FM = TH / WM;               // 32-pixel tile rows per wave
    static_assert(FM >= 1 && FM * WM == TH, "tile rows split evenly over the waves");
    constexpr int TW = 32, HW = TW + 2, HR = TH + 2;
    constexpr int CPX = CIN / 8;              // 16-byte chunks of channels per pixel
    static_assert(CPX == 2 || CPX == 4 || CPX == 8, "Cin 16, 32 or 64");
    constexpr int SPX = CPX + 1;              // 16-byte slots per pixel in LDS (odd)
    constexpr int PSTR = SPX * 16;            // pixel stride in LDS, bytes
    constexpr int NQ = HR * HW;               // halo pixels
    constexpr int NDW = (NQ * SPX + 64 * NW - 1) / (64 * NW);  // loads per lane per halo
    constexpr int HBUF = NDW * NW * 1024;
    constexpr int KC = CIN / 16;              // 16-wide k steps per tap
    constexpr int KS = 9 * KC;
    constexpr int WLD = 32 + 4;
    constexpr int SLICE = 16 * WLD * 4;
    __shared__ __attribute__((aligned(1024))) char hb0[HBUF];
    __shared__ __attribute__((aligned(1024))) char hb1[HBUF];
    __shared__ __attribute__((aligned(16))) char slices[NW * SLICE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int rl = lane & 31, hi = lane >> 5;
    const int H = a.H, W = a.W, Cout = a.Cout;

    // This wave's weights: output channel co = 32*wn + rl, k step s -> tap s / KC,
    // channels 16*(s % KC) + 8*hi .. +8 (the B operand layout).
    typedef typename Mfma32<T>::vec vec;
    vec bw[KS];
    {
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (uint32_t)((size_t)Cout * 9 * CIN * sizeof(T)));
        const int co = wn * 32 + rl;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint32_t off =
                co < Cout ? (uint32_t)((co * 9 + s / KC) * CIN + (s % KC) * 16 + hi * 8) * (uint32_t)sizeof(T) : kOOB;
            bw[s] = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off, 0, 0));
        }
    }

    // Tile order: G workgroups, the ones on one XCD (blockIdx % 8) take a contiguous
    // run of each round's G tiles, so neighbouring tiles share halo rows in one L2.
    const int G = gridDim.x;
    const int r = (G % 8) == 0 ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;

    const i32x4 rx = rsrc_words(a.x, (uint32_t)((size_t)a.N * H * W * CIN * sizeof(T)));
    // Halo of tile t into buf; a t past the last tile issues the same number of
    // loads with out-of-range offsets (no traffic), so the vmcnt waits stay exact.
    auto issue = [&](char *buf, int t) {
        const bool live = t < ntiles;
        const int tt = live ? t : 0;
        const int tx = tt % tiles_w, rr = tt / tiles_w;
        const int ty = rr % tiles_h, n = rr / tiles_h;
        const int oy0 = ty * TH, ox0 = tx * TW;
#pragma unroll
        for (int d = 0; d < NDW; ++d) {
            const int slot = (d * NW + wave) * 64 + lane;
            const int q = slot / SPX, c = slot - q * SPX;
            const int hy = q / HW, hx = q - hy * HW;
            const int iy = oy0 + hy - 1, ix = ox0 + hx - 1;
            const bool ok = live && c < CPX && q < NQ && (unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W;
            const uint32_t off = (uint32_t)(((n * H + iy) * W + ix) * CIN + c * 8) * (uint32_t)sizeof(T);
            dma_b128(rx, ok ? off : kOOB, lds_addr(buf + (d * NW + wave) * 1024));
        }
    };

    f32x16 acc[FM][1];
    auto compute = [&](const char *buf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][0][e] = 0.0f;
        // A operand of tile row wm*FM+i at k step s: pixel (row + ky, rl + kx) of the
        // halo, chunk 2*(s % KC) + hi.
        const char *base = buf + ((wm * FM) * HW + rl) * PSTR + hi * 16;
        auto read = [&](int s, vec(&fa)[FM]) {
            const int tap = s / KC, ky = tap / 3, kx = tap % 3;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const vec *>(base + ((i + ky) * HW + kx) * PSTR + (s % KC) * 32);
        };
        vec fa[2][FM];
        read(0, fa[0]);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s + 1 < KS) read(s + 1, fa[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FM; ++i) acc[i][0] = Mfma32<T>::run(fa[s & 1][i], bw[s], acc[i][0]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    float *slice = reinterpret_cast<float *>(slices + wave * SLICE);
    const uint32_t out_bytes = (uint32_t)((size_t)a.M * Cout * sizeof(T));

    // One tile. Its halo has landed for this wave (the wait in the previous tile's
    // epilogue, or the prologue's): barrier (so it has for every wave), products,
    // barrier (every wave is done reading buf), epilogue. Between the epilogue's loads
    // and its stores, wait for all of this wave's loads (the residual and bias, the
    // halo of tile k+1, which has had this tile's products to arrive) and refill buf
    // with tile k+2. Loads return in order, so issuing the refill only after that
    // wait keeps the epilogue's own loads from queueing behind it.
    auto tile = [&](char *buf, int k) {
        const int t = k * G + r;
        halo_barrier();
        compute(buf);
        halo_barrier();
        const int tx = t % tiles_w, rr = t / tiles_w;
        const int ty = rr % tiles_h, n = rr / tiles_h;
        const int oy0 = ty * TH + wm * FM, ox0 = tx * TW;
        wave_epilogue_nhwc32_rows<T, FM, 1, WLD>(
            acc, slice, a,
            [=](int lr) {
                const int oy = oy0 + lr / 32, ox = ox0 + lr % 32;
                return (oy < H && ox < W) ? (n * H + oy) * W + ox : -1;
            },
            wn * 32, lane, out_bytes, nullptr,
            [&] {
                halo_wait_vmcnt<0>();
                issue(buf, (k + 2) * G + r);
            });
    };
    issue(hb0, r);
    issue(hb1, G + r);
    halo_wait_vmcnt<0>();
    for (int k = 0; k * G + r < ntiles; k += 2) {
        tile(hb0, k);
        if ((k + 1) * G + r >= ntiles) break;
        tile(hb1, k + 1);
    }
    halo_wait_vmcnt<0>();
}

template <typename T, int CIN, int TH, int WN>
static hipError_t launch_halo_t(const ConvArgs &a, int grid_cap, hipStream_t st) {
    const int tiles_w = (a.W + 31) / 32, tiles_h = (a.H + TH - 1) / TH;
    const long long nt = (long long)a.N * tiles_w * tiles_h;
    if (nt > 0x7fffffffll) return hipErrorInvalidValue;
    const int ntiles = (int)nt;
    int grid = ntiles < grid_cap ? ntiles : grid_cap;
    if (grid > 8) grid -= grid % 8;
    hipLaunchKernelGGL((halo3x3_kernel<T, CIN, TH, WN>), dim3(grid), dim3(512), 0, st, a, tiles_w, tiles_h,
                       ntiles);
    return hipGetLastError();
}

template <typename T, int CIN>
static hipError_t launch_halo_c(const ConvArgs &a, const HaloPlan &p, hipStream_t st) {
    if (p.wn == 1) {
        if (p.th == 8) return launch_halo_t<T, CIN, 8, 1>(a, p.grid_cap, st);
        if constexpr (CIN <= 32)  // two (16+2) x 34-pixel halos of 64 channels exceed the LDS
            if (p.th == 16) return launch_halo_t<T, CIN, 16, 1>(a, p.grid_cap, st);
    } else if (p.wn == 2) {
        if (p.th == 4) return launch_halo_t<T, CIN, 4, 2>(a, p.grid_cap, st);
        if (p.th == 8) return launch_halo_t<T, CIN, 8, 2>(a, p.grid_cap, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_halo_d(const ConvArgs &a, const HaloPlan &p, hipStream_t st) {
    switch (a.Cin) {
    case 16: return launch_halo_c<T, 16>(a, p, st);
    case 32: return launch_halo_c<T, 32>(a, p, st);
    case 64: return launch_halo_c<T, 64>(a, p, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_halo3x3(const ConvArgs &a, int dtype, const HaloPlan &p, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_BF16: return launch_halo_d<bf16>(a, p, st);
    case CONV2D_DTYPE_F16: return launch_halo_d<f16>(a, p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace c2d
