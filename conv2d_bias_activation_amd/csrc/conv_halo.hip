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
//  * Weights stay in registers: one wave's 32 output channels over its share of the
//    9*Cin k are 9*Cin/(16*WK) operand fragments of 4 VGPRs (72 VGPRs at Cin 32, or
//    at Cin 64 with k split over a pair of waves). A workgroup copies the weights
//    into LDS once, in fragment order, and every wave reads its fragments from there.
//  * Workgroups are persistent: each walks tiles t = k*G + r (r its XCD-grouped
//    index among G), with the halo of tile k+2 loading into the buffer tile k just
//    released while tile k's epilogue and tile k+1's products run. Bias and slopes
//    stay in registers; a tile's residual loads go out before its products.
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
// WN waves along the output channels (32 each); WK waves along k (each takes CIN/WK
// of the input channels of every tap and the pair adds their sums through LDS);
// 8 / (WN * WK) waves along the tile rows.
template <typename T, int CIN, int TH, int WN, int WK>
__global__ __launch_bounds__(512) void halo3x3_kernel(ConvArgs a, int tiles_w, int tiles_h, int ntiles) {
    constexpr int NW = 8;
    constexpr int WM = NW / (WN * WK);
    constexpr int FM = TH / WM;               // 32-pixel tile rows per wave
    static_assert(WM >= 1 && FM >= 1 && FM * WM == TH, "tile rows split evenly over the waves");
    constexpr int TW = 32, HW = TW + 2, HR = TH + 2;
    constexpr int CPX = CIN / 8;              // 16-byte chunks of channels per pixel
    static_assert(CPX == 2 || CPX == 4 || CPX == 8, "Cin 16, 32 or 64");
    constexpr int SPX = CPX + 1;              // 16-byte slots per pixel in LDS (odd)
    constexpr int PSTR = SPX * 16;            // pixel stride in LDS, bytes
    constexpr int NQ = HR * HW;               // halo pixels
    constexpr int NDW = (NQ * SPX + 64 * NW - 1) / (64 * NW);  // loads per lane per halo
    constexpr int HBUF = NDW * NW * 1024;
    constexpr int KC = CIN / 16;              // 16-wide k steps per tap
    static_assert(KC % WK == 0, "k split");
    constexpr int KCW = KC / WK;              // of them per wave
    constexpr int KSW = 9 * KCW;              // k steps per wave
    constexpr int WBYTES = WN * WK * KSW * 1024;            // weights in operand order
    constexpr int NDWW = (WBYTES + NW * 1024 - 1) / (NW * 1024);
    constexpr int RING = cmax<2 * HBUF, NDWW * NW * 1024>::v;
    constexpr int NHW = 2 / WK;               // 16-row halves of each block this wave stores
    constexpr int NH = FM * NHW;
    constexpr int XCH = WK == 2 ? NW * FM * 2 * 1024 : 16;  // per wave: FM x 8 floats per lane
    constexpr int WLD = 32 + 4;
    constexpr int SLICE = 16 * WLD * 4;
    constexpr int VE = 8;                     // 16-bit values per 16-byte run
    __shared__ __attribute__((aligned(1024))) char ring[RING];
    __shared__ __attribute__((aligned(1024))) char xch[XCH];
    __shared__ __attribute__((aligned(16))) char slices[NW * SLICE];
    char *const hb0 = ring;
    char *const hb1 = ring + HBUF;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM, wk = (wave / WM) % WK, wn = wave / (WM * WK);
    const int rl = lane & 31, hi = lane >> 5;
    const int cc = lane & 3, rsub = lane >> 2;  // epilogue: 16-byte run cc of row rsub
    const int H = a.H, W = a.W, Cout = a.Cout;
    typedef typename Mfma32<T>::vec vec;

    // Weights, once per workgroup: staged in LDS in operand order ([wn][wk][k step]
    // [lane] x 16 bytes: output channel 32*wn + lane % 32, channels 8*(lane/32).. of
    // the wave's k step), then each wave takes its KSW fragments into registers.
    // Bias and slopes of the lane's epilogue run stay in registers too.
    const i32x4 rwt = rsrc_words(a.w, (uint32_t)((size_t)Cout * 9 * CIN * sizeof(T)));
#pragma unroll
    for (int d = 0; d < NDWW; ++d) {
        const int rest = d * NW + wave;
        const int sw = rest % KSW, wkk = (rest / KSW) % WK, wnn = rest / (KSW * WK);
        const int co = wnn * 32 + rl, tap = sw / KCW, ci = (wkk * KCW + sw % KCW) * 16 + hi * 8;
        const bool ok = wnn < WN && co < Cout;
        dma_b128(rwt, ok ? (uint32_t)((co * 9 + tap) * CIN + ci) * (uint32_t)sizeof(T) : kOOB,
                 lds_addr(ring + rest * 1024));
    }
    float bv[VE], av[VE];
    {
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.bias, a.bias ? (uint32_t)Cout * 4u : 0u);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.alpha, a.alpha ? (uint32_t)Cout * 4u : 0u);
        const int co = wn * 32 + cc * VE;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const uint32_t off = co + e < Cout ? (uint32_t)(co + e) * 4u : kOOB;
            bv[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (int)off, 0, 0));
            av[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, (int)off, 0, 0));
        }
    }
    halo_wait_vmcnt<0>();
    halo_barrier();
    vec bw[KSW];
#pragma unroll
    for (int sw = 0; sw < KSW; ++sw)
        bw[sw] = *reinterpret_cast<const vec *>(ring + (((wn * WK + wk) * KSW + sw) * 64 + lane) * 16);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): fragments in registers before the ring is reused
    halo_barrier();

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

    f32x16 acc[FM];
    auto compute = [&](const char *buf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
        // A operand of tile row wm*FM+i at the wave's k step sw: pixel (row + ky, rl + kx)
        // of the halo, 16-channel chunk wk*KCW + sw % KCW, 8-channel half hi.
        const char *base = buf + ((wm * FM) * HW + rl) * PSTR + hi * 16 + wk * KCW * 32;
        auto read = [&](int sw, vec(&fa)[FM]) {
            const int tap = sw / KCW, ky = tap / 3, kx = tap % 3;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const vec *>(base + ((i + ky) * HW + kx) * PSTR + (sw % KCW) * 32);
        };
        vec fa[2][FM];
        read(0, fa[0]);
#pragma unroll
        for (int sw = 0; sw < KSW; ++sw) {
            if (sw + 1 < KSW) read(sw + 1, fa[(sw + 1) & 1]);
            // keep the scheduler from sinking those reads below the products
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FM; ++i) acc[i] = Mfma32<T>::run(fa[sw & 1][i], bw[sw], acc[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Epilogue rows: the wave's q-th 16-row half (block i = q / NHW, half h) holds
    // pixels 16h + 0..15 of tile row wm*FM + i; a lane finishes row rsub of each half,
    // channels 32*wn + 8*cc .. +8.
    const bool has_res = a.res != nullptr, pre = a.res_before_act != 0;
    const uint32_t out_bytes = (uint32_t)((size_t)a.M * Cout * sizeof(T));
    const __amdgpu_buffer_rsrc_t rres = make_rsrc(a.res, has_res ? out_bytes : 0u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, out_bytes);
    const int co_run = wn * 32 + cc * VE;
    auto half_of = [&](int q) { return WK == 2 ? wk : q % NHW; };
    auto out_off = [&](int t, int q) -> uint32_t {
        const int tx = t % tiles_w, rr = t / tiles_w;
        const int ty = rr % tiles_h, n = rr / tiles_h;
        const int oy = ty * TH + wm * FM + q / NHW, ox = tx * TW + 16 * half_of(q) + rsub;
        return (oy < H && ox < W && co_run < Cout)
                   ? ((uint32_t)((n * H + oy) * W + ox) * (uint32_t)Cout + (uint32_t)co_run) * (uint32_t)sizeof(T)
                   : kOOB;
    };

    float *slice = reinterpret_cast<float *>(slices + wave * SLICE);
    float *mine = reinterpret_cast<float *>(xch + wave * (FM * 2 * 1024));
    const float *theirs = reinterpret_cast<const float *>(xch + (WK == 2 ? (wave + (wk ? -WM : WM)) : wave) * (FM * 2 * 1024));

    // One tile. Its halo has landed for this wave (the wait in the previous tile's
    // epilogue, or the prologue's): barrier (so it has for every wave), residual loads,
    // products, [hand the partner the half it stores,] barrier (every wave is done
    // reading buf), [add the partner's half,] epilogue. Between the epilogue's LDS
    // phase and its stores, wait for all of this wave's loads (the residual, and the
    // halo of tile k+1, which has had this tile's products to arrive) and refill buf
    // with tile k+2.
    auto tile = [&](char *buf, int k) {
        const int t = k * G + r;
        halo_barrier();
        uint32_t off[NH];
        u32x4 rv[NH];
#pragma unroll
        for (int q = 0; q < NH; ++q) {
            off[q] = out_off(t, q);
            rv[q] = has_res ? __builtin_amdgcn_raw_buffer_load_b128(rres, (int)off[q], 0, 0) : u32x4{0u, 0u, 0u, 0u};
        }
        compute(buf);
        if constexpr (WK == 2) {
            const int hs = 1 - wk;  // the half the partner stores
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    *reinterpret_cast<f32x4 *>(mine + ((i * 2 + u) * 64 + lane) * 4) =
                        f32x4{acc[i][8 * hs + 4 * u], acc[i][8 * hs + 4 * u + 1], acc[i][8 * hs + 4 * u + 2],
                              acc[i][8 * hs + 4 * u + 3]};
        }
        halo_barrier();
        if constexpr (WK == 2) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const f32x4 o = *reinterpret_cast<const f32x4 *>(theirs + ((i * 2 + u) * 64 + lane) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][8 * wk + 4 * u + e] += o[e];
                }
        }
        // LDS phase: each 16-row half through the wave's slice, back as 8-channel runs.
        float v[NH][VE];
#pragma unroll
        for (int q = 0; q < NH; ++q) {
            const int i = q / NHW, h = half_of(q);
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) slice[(g * 8 + hi * 4 + e) * WLD + rl] = acc[i][(2 * h + g) * 4 + e];
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int e = 0; e < VE; e += 4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(slice + rsub * WLD + cc * VE + e);
                v[q][e] = x[0];
                v[q][e + 1] = x[1];
                v[q][e + 2] = x[2];
                v[q][e + 3] = x[3];
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
        }
        halo_wait_vmcnt<0>();
        issue(buf, (k + 2) * G + r);
        auto finish = [&](auto act_tag) {
            constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
            for (int q = 0; q < NH; ++q) {
                T rt[VE], out[VE];
                __builtin_memcpy(rt, &rv[q], 16);
                epilogue_vec<T, ACT, VE>(v[q], bv, av, rt, has_res, pre, out);
                u32x4 o;
                __builtin_memcpy(&o, out, 16);
                __builtin_amdgcn_raw_buffer_store_b128(o, ry, (int)off[q], 0, 0);
            }
        };
        switch (a.act) {
        case CONV2D_ACT_RELU: finish(std::integral_constant<int, CONV2D_ACT_RELU>{}); break;
        case CONV2D_ACT_SILU: finish(std::integral_constant<int, CONV2D_ACT_SILU>{}); break;
        case CONV2D_ACT_PRELU: finish(std::integral_constant<int, CONV2D_ACT_PRELU>{}); break;
        default: finish(std::integral_constant<int, CONV2D_ACT_NONE>{}); break;
        }
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
    constexpr int WK = CIN == 64 ? 2 : 1;
    hipLaunchKernelGGL((halo3x3_kernel<T, CIN, TH, WN, WK>), dim3(grid), dim3(512), 0, st, a, tiles_w, tiles_h,
                       ntiles);
    return hipGetLastError();
}

// Tile heights per (Cin, waves along Cout): 64-channel layers split k over wave pairs,
// which leaves 2 (WN = 2) or 4 (WN = 1) waves along the tile rows.
template <typename T, int CIN>
static hipError_t launch_halo_c(const ConvArgs &a, const HaloPlan &p, hipStream_t st) {
    if constexpr (CIN == 64) {
        if (p.wn == 1 && p.th == 4) return launch_halo_t<T, CIN, 4, 1>(a, p.grid_cap, st);
        if (p.wn == 1 && p.th == 8) return launch_halo_t<T, CIN, 8, 1>(a, p.grid_cap, st);
        if (p.wn == 2 && p.th == 4) return launch_halo_t<T, CIN, 4, 2>(a, p.grid_cap, st);
    } else {
        if (p.wn == 1 && p.th == 8) return launch_halo_t<T, CIN, 8, 1>(a, p.grid_cap, st);
        if (p.wn == 1 && p.th == 16) return launch_halo_t<T, CIN, 16, 1>(a, p.grid_cap, st);
        if (p.wn == 2 && p.th == 4) return launch_halo_t<T, CIN, 4, 2>(a, p.grid_cap, st);
        if (p.wn == 2 && p.th == 8) return launch_halo_t<T, CIN, 8, 2>(a, p.grid_cap, st);
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
