// Channel-last implicit-GEMM convolution on CDNA4 matrix cores, pipelined.
//
// Same GEMM as the general kernel (m = output pixel, k = (tap, input channel),
// n = output channel; inferencelayer page, `conv()`: im2col + `enc_gemm3` with bias
// and activation in the epilogue), built for throughput on gfx950:
//
//  * K steps of 64: every thread moves whole 16-byte channel runs (8 x 16-bit) of
//    the patch matrix A and of the weight B with buffer loads. A padding tap, a row
//    past the last pixel or a column past the last channel gets an out-of-range
//    buffer offset, which the hardware answers with zeros: no branches in the loop.
//  * LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled by row (chunk
//    position p holds logical chunk p ^ (row % 8)), so neither the 16-byte stores
//    nor the matrix-core operand reads of 16 consecutive rows hit the same banks.
//  * The loads go straight from memory into LDS (buffer_load ... lds: each lane's
//    16 bytes land at the wave's LDS base + 16 * lane, which is exactly the swizzled
//    row layout above), through a ring of NS LDS stages with one barrier per step:
//    NS = 3 keeps two K steps in flight while the matrix cores work on a third.
//  * When Cin is a multiple of 64 the K loop takes the taps innermost, so the patch
//    rows of consecutive steps are the same pixels shifted by one tap and mostly
//    hit in the vector L1 cache.
//  * KG = 2 runs two wave groups per workgroup on alternate K steps (each with its own
//    half of every LDS stage) and adds the two fp32 accumulators through LDS at the
//    end: two waves per SIMD for layers with too few output tiles to put one
//    workgroup on every CU twice (ResNet stages 3-4), without a second pass.
#include <utility>

#include "igemm_common.hpp"
#include "kernels.hpp"

namespace c2d {

// s_waitcnt with only the vector-memory counter limited (expcnt and lgkmcnt at their
// maxima, so they impose no wait).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without a memory fence: the LDS data it publishes is complete
// either through the explicit vmcnt wait before it (direct-to-LDS loads) or because
// the readers' operands were consumed. The empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <typename T, int BM, int BN, int WGM, int WGN, int NS, int KG, bool TAP_INNER, bool SPLIT,
          bool NCHW_OUT>
__global__ __launch_bounds__(64 * WGM * WGN * KG, 8 / (WGM * WGN * KG)) void igemm_nhwc_kernel(
    ConvArgs a, int tiles_n, int steps_per_split, float *partials) {
    constexpr int NW = WGM * WGN;        // waves per K group (4 or 8)
    static_assert(KG == 1 || (KG == 2 && NW == 4), "two K groups of four waves");
    constexpr int BK = 64;               // k per step (elements)
    constexpr int ROWB = 128;            // bytes per LDS row (BK 16-bit values)
    constexpr int FM = BM / (32 * WGM);  // 32x32 blocks per wave along M
    constexpr int FN = BN / (32 * WGN);
    static_assert((NW == 4 || NW == 8) && FM >= 1 && FN >= 1, "4 or 8 waves");
    constexpr int RR = 8 * NW;           // rows per load round (8 per wave)
    static_assert(BM % RR == 0 && BN % RR == 0, "whole load rounds");
    static_assert(NS >= 2 && NS <= 6, "LDS stages");
    constexpr int LA = BM / RR;          // 16-byte A loads per thread per step
    constexpr int LB = BN / RR;
    constexpr int L = LA + LB;
    constexpr int STAGE = (BM + BN) * ROWB;  // one K group's half of a stage
    constexpr int STAGE_ALL = KG * STAGE;
    constexpr int WN = FN * 32;          // columns per wave
    constexpr int WLD = WN + 4;          // row stride of a wave's epilogue slice (floats)
    constexpr int SLICE = 16 * WLD * 4;  // bytes
    constexpr int SPS = STAGE_ALL / SLICE;  // slices per stage array
    static_assert(SPS * 2 >= NW, "epilogue slices fit in two stages");
    // KG = 2: group 1's accumulators pass through stage 1 while group 0's slices are in stage 0
    static_assert(KG == 1 || (SPS >= NW && NW * FM * FN * 16 * 64 * 4 <= STAGE_ALL), "K-group reduction fits");
    // One array per stage: distinct objects let the compiler see that the direct-to-LDS
    // loads into one stage never alias the operand reads from another, so it keeps the
    // explicit vmcnt waits instead of draining every load before each read.
    __shared__ __attribute__((aligned(1024))) char st0[STAGE_ALL];
    __shared__ __attribute__((aligned(1024))) char st1[STAGE_ALL];
    __shared__ __attribute__((aligned(1024))) char st2[NS > 2 ? STAGE_ALL : 16];
    __shared__ __attribute__((aligned(1024))) char st3[NS > 3 ? STAGE_ALL : 16];
    __shared__ __attribute__((aligned(1024))) char st4[NS > 4 ? STAGE_ALL : 16];
    __shared__ __attribute__((aligned(1024))) char st5[NS > 5 ? STAGE_ALL : 16];
    auto stage_ptr = [&](auto idx) -> char * {
        constexpr int I = decltype(idx)::value;
        if constexpr (I == 0) return st0;
        else if constexpr (I == 1) return st1;
        else if constexpr (I == 2) return st2;
        else if constexpr (I == 3) return st3;
        else if constexpr (I == 4) return st4;
        else return st5;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave_all / NW;           // K group: takes the steps s with s % KG == grp
    const int wave = wave_all - grp * NW;    // wave within its group
    const int wm = wave % WGM, wn = wave / WGM;
    const int gofs = grp * STAGE;            // the group's half of each stage

    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int m0 = (tile / tiles_n) * BM;
    const int n0 = (tile % tiles_n) * BN;

    const int H = a.H, W = a.W, Cin = a.Cin, kh = a.kh, kw = a.kw, K = a.K;
    const int OW = a.OW, OHW = a.OH * a.OW;
    // Split-K (gridDim.y slices): this workgroup takes K steps [s_begin, s_end).
    const int nsteps_all = (K + BK - 1) / BK;
    const int s_begin = blockIdx.y * steps_per_split;
    const int nsteps = max(0, min(nsteps_all, s_begin + steps_per_split) - s_begin);
    const int nsup = (nsteps + KG - 1) / KG;  // ring steps: KG K steps each, one per group
    const int s_first = s_begin + grp;        // this group's first K step

    const i32x4 rx = rsrc_words(a.x, (uint32_t)((size_t)a.N * H * W * Cin * sizeof(T)));
    const i32x4 rw = rsrc_words(a.w, (uint32_t)((size_t)a.Cout * K * sizeof(T)));

    // This thread's loads: rows (j*NW + wave)*8 + lrow, LDS chunk position pch (= the
    // lane's slot in the wave's 1 KiB), which holds the row's logical 16-byte chunk
    // c = pch ^ ((row / 2) % 8) (k offset 8c within the step; NW is even, so this is
    // the same for every j). With that swizzle the 16 rows read by one quarter-wave
    // occupy 16 distinct 16-byte bank groups.
    const int lrow = lane >> 3;
    const int pch = lane & 7;
    const int c = pch ^ ((wave * 4 + (lane >> 4)) & 7);

    int a_pix[LA], a_ih[LA], a_iw[LA];
    bool a_ok[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        int m = m0 + (j * NW + wave) * 8 + lrow;
        a_ok[j] = m < a.M;
        int mm = a_ok[j] ? m : 0;
        int n = mm / OHW, pix = mm - n * OHW;
        int oh = pix / OW, ow = pix - oh * OW;
        a_pix[j] = n * H * W;
        a_ih[j] = oh * a.stride - a.pad;
        a_iw[j] = ow * a.stride - a.pad;
    }
    int b_off[LB];
    bool b_ok[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        int co = n0 + (j * NW + wave) * 8 + lrow;
        b_ok[j] = co < a.Cout;
        b_off[j] = (b_ok[j] ? co : 0) * K;
    }

    // k state of this thread's chunk at the next step to load
    int ky, kx, ci;
    // Taps innermost: k step = (channel block cb, tap). Each row's byte offset at tap
    // (0, 0) and a mask of its taps that fall inside the image are fixed per thread;
    // a step then adds one wave-uniform offset, so a load costs a bit test, an add and
    // a select (the address arithmetic was most of the step's instruction stream).
    int cb = 0;
    int a_base[LA], b_base[LB];
    uint32_t a_mask[LA];
    if constexpr (TAP_INNER) {
        const int taps = kh * kw;
        cb = s_first / taps;
        const int tap = s_first - cb * taps;
        ky = tap / kw;
        kx = tap - ky * kw;
        ci = 0;
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            a_base[j] = ((a_pix[j] + a_ih[j] * W + a_iw[j]) * Cin + c * 8) * (int)sizeof(T);
            uint32_t mk = 0;
            for (int ty = 0; ty < kh; ++ty)
                for (int tx = 0; tx < kw; ++tx) {
                    const bool in = a_ok[j] && (unsigned)(a_ih[j] + ty) < (unsigned)H && (unsigned)(a_iw[j] + tx) < (unsigned)W;
                    mk |= (in ? 1u : 0u) << (ty * kw + tx);
                }
            a_mask[j] = mk;
        }
        // a weight row past Cout gets a base of 2^31 bytes: every offset from it is out of range
#pragma unroll
        for (int j = 0; j < LB; ++j) b_base[j] = b_ok[j] ? (b_off[j] + c * 8) * (int)sizeof(T) : (int)0x80000000u;
    } else {
        const int k = s_first * BK + c * 8;
        const int tap = k / Cin;
        ci = k - tap * Cin;
        ky = tap / kw;
        kx = tap - ky * kw;
    }

    // Issues one step's loads into LDS stage `stage`. A step past this slice (live
    // false) still issues them, with out-of-range offsets (no memory traffic), so every
    // step adds exactly L to the vector-memory counter and the waits below are exact.
    auto advance = [&]() {
        if constexpr (TAP_INNER) {
            if (++kx == kw) {
                kx = 0;
                if (++ky == kh) {
                    ky = 0;
                    ++cb;
                }
            }
        } else {
            ci += BK;
            while (ci >= Cin) {
                ci -= Cin;
                if (++kx == kw) {
                    kx = 0;
                    ++ky;
                }
            }
        }
    };
    auto issue = [&](char *stage, bool live) {
        char *sA = stage + gofs;
        char *sB = sA + BM * ROWB;
        if constexpr (TAP_INNER) {
            const int tap = ky * kw + kx;
            const bool kin = live && cb * BK < Cin;
            const int toff = ((ky * W + kx) * Cin + cb * BK) * (int)sizeof(T);
            const int koff = (tap * Cin + cb * BK) * (int)sizeof(T);
#pragma unroll
            for (int j = 0; j < LA; ++j) {
                const bool ok = kin && ((a_mask[j] >> tap) & 1u);
                dma_b128(rx, ok ? (uint32_t)(a_base[j] + toff) : kOOB, lds_addr(sA + (j * NW + wave) * 1024));
            }
#pragma unroll
            for (int j = 0; j < LB; ++j)
                dma_b128(rw, kin ? (uint32_t)(b_base[j] + koff) : kOOB, lds_addr(sB + (j * NW + wave) * 1024));
#pragma unroll
            for (int r = 0; r < KG; ++r) advance();
            return;
        }
        const bool kin = live && ky < kh;
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            int iy = a_ih[j] + ky, ix = a_iw[j] + kx;
            bool ok = a_ok[j] && kin && (unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W;
            uint32_t off = (uint32_t)((a_pix[j] + iy * W + ix) * Cin + ci) * (uint32_t)sizeof(T);
            dma_b128(rx, ok ? off : kOOB, lds_addr(sA + (j * NW + wave) * 1024));
        }
        const int kk = (ky * kw + kx) * Cin + ci;
#pragma unroll
        for (int j = 0; j < LB; ++j) {
            uint32_t off = (uint32_t)(b_off[j] + kk) * (uint32_t)sizeof(T);
            dma_b128(rw, (b_ok[j] && kin) ? off : kOOB, lds_addr(sB + (j * NW + wave) * 1024));
        }
#pragma unroll
        for (int r = 0; r < KG; ++r) advance();
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    typedef typename Mfma32<T>::vec vec;
    const int rl = lane & 31, kq = lane >> 5, sw = (rl >> 1) & 7;
    // One step's matrix-core work. The operand reads of sub-step ks+1 are issued
    // before the products of sub-step ks, so LDS latency overlaps the matrix cores.
    auto compute = [&](const char *stage) {
        const char *sA = stage + gofs;
        const char *sB = sA + BM * ROWB;
        vec fa[2][FM], fb[2][FN];
        auto read = [&](int ks, vec(&xa)[FM], vec(&xb)[FN]) {
            const int chunk = ((ks * 2 + kq) ^ sw) * 16;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                xa[i] = *reinterpret_cast<const vec *>(sA + (wm * FM * 32 + i * 32 + rl) * ROWB + chunk);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                xb[j] = *reinterpret_cast<const vec *>(sB + (wn * FN * 32 + j * 32 + rl) * ROWB + chunk);
        };
        read(0, fa[0], fb[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < 3) read(ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
            // keep the scheduler from sinking those reads below the products
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = Mfma32<T>::run(fa[ks & 1][i], fb[ks & 1][j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Ring of NS stages; step s lives in stage s % NS and is loaded NS-1 steps ahead.
    // One step: wait for this wave's loads of the step (the NS-2 younger steps stay in
    // flight), barrier (every wave's have landed and every wave is done with the
    // previous step's stage), matrix cores on this step, then refill the previous
    // step's stage with step s+NS-1 (so the matrix cores start right after the barrier).
    // With KG = 2 a ring step holds two K steps, one per group; a group whose K step is
    // past the slice loads zeros (live false) and adds zero products.
    auto step = [&](auto idx, int s) {
        constexpr int I = decltype(idx)::value;
        wait_vmcnt<(NS - 2) * L>();
        barrier_nofence();
        compute(stage_ptr(std::integral_constant<int, I>{}));
        issue(stage_ptr(std::integral_constant<int, (I + NS - 1) % NS>{}), KG * (s + NS - 1) + grp < nsteps);
    };
    [&]<int... I>(std::integer_sequence<int, I...>) {
        (issue(stage_ptr(std::integral_constant<int, I>{}), KG * I + grp < nsteps), ...);
    }(std::make_integer_sequence<int, NS - 1>{});
    for (int s0 = 0; s0 < nsup; s0 += NS) {
        bool done = false;
        [&]<int... I>(std::integer_sequence<int, I...>) {
            ((done = done || s0 + I >= nsup, done ? void() : step(std::integral_constant<int, I>{}, s0 + I)), ...);
        }(std::make_integer_sequence<int, NS>{});
    }
    wait_vmcnt<0>();
    __syncthreads();

    if constexpr (KG == 2) {
        // group 1 hands its accumulators to the wave of group 0 with the same output
        // block (lane-major floats: conflict-free), then leaves
        float *red = reinterpret_cast<float *>(st1) + wave * (FM * FN * 16 * 64) + lane;
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) red[((i * FN + j) * 16 + e) * 64] = acc[i][j][e];
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] += red[((i * FN + j) * 16 + e) * 64];
    }

    // Epilogue, each wave over its own rows through its slice of stage 0 (LDS phase,
    // then global phase; see wave_epilogue_nhwc32).
    float *slice = reinterpret_cast<float *>(wave < SPS ? st0 + wave * SLICE : st1 + (wave - SPS) * SLICE);
    const uint32_t out_bytes = (uint32_t)((size_t)a.M * a.Cout * sizeof(T));
    if constexpr (NCHW_OUT) {
        wave_epilogue_nchw32<T, FM, FN, WLD>(acc, slice, a, m0 + wm * FM * 32, n0 + wn * WN, lane, out_bytes);
        if (a.y2) {
            // the same values again, channel-last, for the next channel-first conv of a
            // stack (same epilogue arithmetic, so the copy equals y element for element)
            ConvArgs b = a;
            b.y = a.y2;
            b.res = nullptr;
            b.vec_out = 1;
            wave_epilogue_nhwc32<T, FM, FN, WLD>(acc, slice, b, m0 + wm * FM * 32, n0 + wn * WN, lane, out_bytes);
        }
    } else {
        float *part = SPLIT ? partials + (size_t)blockIdx.y * a.M * a.Cout : nullptr;
        wave_epilogue_nhwc32<T, FM, FN, WLD>(acc, slice, a, m0 + wm * FM * 32, n0 + wn * WN, lane, out_bytes,
                                             part);
    }
}

// Second pass of a split-K launch: per 16-byte output run, the fp32 slices are
// added in slice order (so the result does not depend on scheduling), then bias,
// residual and activation, and one rounding to T.
template <typename T>
__global__ __launch_bounds__(256) void splitk_epilogue_kernel(ConvArgs a, const float *partials,
                                                              int splits) {
    constexpr int VE = 16 / (int)sizeof(T);
    const int runs_per_row = a.Cout / VE;
    const long long total = (long long)a.M * runs_per_row;
    const size_t slice = (size_t)a.M * a.Cout;
    const T *__restrict__ res = static_cast<const T *>(a.res);
    T *__restrict__ y = static_cast<T *>(a.y);
    const bool has_res = res != nullptr, pre = a.res_before_act != 0;
    for (long long it = blockIdx.x * 256ll + threadIdx.x; it < total; it += (long long)gridDim.x * 256) {
        const int m = (int)(it / runs_per_row);
        const int co = (int)(it - (long long)m * runs_per_row) * VE;
        const size_t o = (size_t)m * a.Cout + co;
        float v[VE];
#pragma unroll
        for (int e = 0; e < VE; e += 4) {
            f32x4 t = *reinterpret_cast<const f32x4 *>(partials + o + e);
            v[e] = t[0];
            v[e + 1] = t[1];
            v[e + 2] = t[2];
            v[e + 3] = t[3];
        }
        for (int sidx = 1; sidx < splits; ++sidx) {
#pragma unroll
            for (int e = 0; e < VE; e += 4) {
                f32x4 t = *reinterpret_cast<const f32x4 *>(partials + sidx * slice + o + e);
                v[e] += t[0];
                v[e + 1] += t[1];
                v[e + 2] += t[2];
                v[e + 3] += t[3];
            }
        }
        float bv[VE], av[VE];
        T rv[VE], out[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            bv[e] = a.bias ? a.bias[co + e] : 0.0f;
            av[e] = a.alpha ? a.alpha[co + e] : 0.0f;
        }
        if (has_res) {
            u32x4 t = *reinterpret_cast<const u32x4 *>(res + o);
            __builtin_memcpy(rv, &t, 16);
        }
        switch (a.act) {
        case CONV2D_ACT_RELU:
            epilogue_vec<T, CONV2D_ACT_RELU, VE>(v, bv, av, rv, has_res, pre, out);
            break;
        case CONV2D_ACT_SILU:
            epilogue_vec<T, CONV2D_ACT_SILU, VE>(v, bv, av, rv, has_res, pre, out);
            break;
        case CONV2D_ACT_PRELU:
            epilogue_vec<T, CONV2D_ACT_PRELU, VE>(v, bv, av, rv, has_res, pre, out);
            break;
        default:
            epilogue_vec<T, CONV2D_ACT_NONE, VE>(v, bv, av, rv, has_res, pre, out);
            break;
        }
        u32x4 t;
        __builtin_memcpy(&t, out, 16);
        *reinterpret_cast<u32x4 *>(y + o) = t;
    }
}

namespace {

// Tile shapes: (BM, BN) per workgroup, waves WGM x WGN, LDS stages.
struct TileCfg {
    int bm, bn, wgm, wgn, ns, kg;
};
constexpr TileCfg kTiles[NHWC_TILE_COUNT] = {
    {256, 128, 4, 2, 2, 1},  // NHWC_TILE_256x128_W8
    {128, 128, 2, 2, 3, 1},  // NHWC_TILE_128x128
    {128, 64, 2, 2, 3, 1},   // NHWC_TILE_128x64
    {256, 64, 4, 2, 3, 1},   // NHWC_TILE_256x64_W8
    {256, 32, 4, 1, 3, 1},   // NHWC_TILE_256x32
    {64, 64, 2, 2, 3, 1},    // NHWC_TILE_64x64
    {128, 128, 2, 4, 3, 1},  // NHWC_TILE_128x128_W8
    {128, 256, 2, 4, 2, 1},  // NHWC_TILE_128x256_W8
    {64, 64, 2, 2, 6, 1},    // NHWC_TILE_64x64_D6
    {128, 64, 2, 2, 5, 1},   // NHWC_TILE_128x64_D5
    {128, 128, 2, 4, 4, 1},  // NHWC_TILE_128x128_W8_D4
    {64, 128, 2, 2, 5, 1},   // NHWC_TILE_64x128_D5
    {64, 64, 2, 2, 4, 1},    // NHWC_TILE_64x64_D4
    {256, 128, 4, 2, 3, 1},  // NHWC_TILE_256x128_W8_D3
    {64, 64, 2, 2, 3, 2},    // NHWC_TILE_64x64_K2
    {64, 64, 2, 2, 4, 2},    // NHWC_TILE_64x64_K2_D4
    {64, 64, 2, 2, 2, 2},    // NHWC_TILE_64x64_K2_D2 (64 KiB of LDS: two workgroups per CU)
};

template <typename T, int TILE>
hipError_t launch_t(const ConvArgs &a, const NhwcPlan &p, float *partials, hipStream_t st) {
    constexpr TileCfg c = kTiles[TILE];
    const long long tiles_m = (a.M + c.bm - 1) / c.bm;
    const int tiles_n = (a.Cout + c.bn - 1) / c.bn;
    if (tiles_m * tiles_n > 0x7fffffffll) return hipErrorInvalidValue;
    const int splits = p.splits > 1 ? p.splits : 1;
    const int nsteps = (a.K + 63) / 64;
    const int per = (nsteps + splits - 1) / splits;
    dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)splits);
    dim3 block(64 * c.wgm * c.wgn * c.kg);
    hipError_t e;
    if (p.nchw_out) {
        if (splits > 1) return hipErrorInvalidValue;  // split-K writes channel-last only
        if (p.tap_inner)
            e = launch_kernel(igemm_nhwc_kernel<T, c.bm, c.bn, c.wgm, c.wgn, c.ns, c.kg, true, false, true>, grid, block, 0,
                              st, a, tiles_n, per, partials);
        else
            e = launch_kernel(igemm_nhwc_kernel<T, c.bm, c.bn, c.wgm, c.wgn, c.ns, c.kg, false, false, true>, grid, block,
                              0, st, a, tiles_n, per, partials);
    } else if (p.tap_inner) {
        if (splits > 1)
            e = launch_kernel(igemm_nhwc_kernel<T, c.bm, c.bn, c.wgm, c.wgn, c.ns, c.kg, true, true, false>, grid, block, 0,
                              st, a, tiles_n, per, partials);
        else
            e = launch_kernel(igemm_nhwc_kernel<T, c.bm, c.bn, c.wgm, c.wgn, c.ns, c.kg, true, false, false>, grid, block,
                              0, st, a, tiles_n, per, partials);
    } else {
        if (splits > 1)
            e = launch_kernel(igemm_nhwc_kernel<T, c.bm, c.bn, c.wgm, c.wgn, c.ns, c.kg, false, true, false>, grid, block,
                              0, st, a, tiles_n, per, partials);
        else
            e = launch_kernel(igemm_nhwc_kernel<T, c.bm, c.bn, c.wgm, c.wgn, c.ns, c.kg, false, false, false>, grid, block,
                              0, st, a, tiles_n, per, partials);
    }
    if (e != hipSuccess || splits == 1) return e;
    constexpr int VE = 16 / (int)sizeof(T);
    long long runs = (long long)a.M * (a.Cout / VE);
    long long blocks = (runs + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    return launch_kernel(splitk_epilogue_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st, a,
                         (const float *)partials, splits);
}

template <typename T>
hipError_t launch_dtype(const ConvArgs &a, const NhwcPlan &p, float *partials, hipStream_t st) {
    switch (p.tile) {
    case 0: return launch_t<T, 0>(a, p, partials, st);
    case 1: return launch_t<T, 1>(a, p, partials, st);
    case 2: return launch_t<T, 2>(a, p, partials, st);
    case 3: return launch_t<T, 3>(a, p, partials, st);
    case 4: return launch_t<T, 4>(a, p, partials, st);
    case 5: return launch_t<T, 5>(a, p, partials, st);
    case 6: return launch_t<T, 6>(a, p, partials, st);
    case 7: return launch_t<T, 7>(a, p, partials, st);
    case 8: return launch_t<T, 8>(a, p, partials, st);
    case 9: return launch_t<T, 9>(a, p, partials, st);
    case 10: return launch_t<T, 10>(a, p, partials, st);
    case 11: return launch_t<T, 11>(a, p, partials, st);
    case 12: return launch_t<T, 12>(a, p, partials, st);
    case 13: return launch_t<T, 13>(a, p, partials, st);
    case 14: return launch_t<T, 14>(a, p, partials, st);
    case 15: return launch_t<T, 15>(a, p, partials, st);
    case 16: return launch_t<T, 16>(a, p, partials, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int nhwc_tile_bm(int tile) { return (tile >= 0 && tile < NHWC_TILE_COUNT) ? kTiles[tile].bm : 0; }
int nhwc_tile_bn(int tile) { return (tile >= 0 && tile < NHWC_TILE_COUNT) ? kTiles[tile].bn : 0; }
int nhwc_tile_waves(int tile) {
    return (tile >= 0 && tile < NHWC_TILE_COUNT) ? kTiles[tile].wgm * kTiles[tile].wgn * kTiles[tile].kg : 0;
}

hipError_t launch_igemm_nhwc(const ConvArgs &a, int dtype, const NhwcPlan &p, float *partials,
                             hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_BF16:
        return launch_dtype<bf16>(a, p, partials, st);
    case CONV2D_DTYPE_F16:
        return launch_dtype<f16>(a, p, partials, st);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace c2d
