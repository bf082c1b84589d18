// 3x3 stride-1 pad-1 channel-last convolution with 64 input channels and up to 64 output
// channels (the ResNet-D stage-1 convs) on CDNA4 matrix cores: halo tiles with
// specialised waves.
//
// The GEMM is the implicit-GEMM one of the other kernels (m = output pixel, k = (tap,
// input channel), n = output channel; inferencelayer page, `conv()`: im2col + GEMM with
// bias and activation in the epilogue); as in the halo kernel, a 4 x 32-pixel output
// tile reads its patches from one copy of its (4+2) x 34-pixel input halo in LDS (the
// halo tiles of the framecast page's convolution shader). What differs is who does
// what: a workgroup of 8 waves has
//
//  * four compute waves (one per SIMD) that hold their weights in registers for the
//    whole launch (32 output channels x all 576 k: 36 operand fragments, taken once from
//    a coalesced copy of the weights in LDS) and run only matrix-core products: each
//    takes two tile rows (64 pixels) x 32 channels, and hands its fp32 sums of tile s-1
//    to a tile in LDS while the products of tile s run;
//  * four loader/epilogue waves that keep the input halos coming (direct-to-LDS loads,
//    two tiles ahead into a ring of three halo buffers, with the tile-invariant address
//    arithmetic hoisted out of the loop), load the residual three tiles ahead into
//    registers, and run the epilogue of tile s-2 from the hand-off tile (bias, residual
//    before or after the activation, activation, one rounding, 16-byte stores of 8
//    channels).
//
// The two groups meet at one workgroup barrier per tile, so the matrix cores work on
// tile s while the hand-off of s-1, the epilogue of s-2 and the loads of tiles s+1, s+2
// proceed. The workgroups are persistent (one per CU) and walk tiles t = s*G + r. The
// last tile of a workgroup is not handed off: its compute waves run its epilogue
// straight from their registers (its residual loaded during the second half of its
// products) while the loader waves finish the one before, so the launch ends one
// epilogue after its last products instead of two hand-offs and two epilogues.
#include "igemm_common.hpp"
#include "kernels.hpp"

namespace c2d {

namespace {

template <int N> __device__ __forceinline__ void ws_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier after this wave's LDS accesses have completed (s_barrier does not
// wait for them); direct-to-LDS loads are published by the loaders' vmcnt waits.
__device__ __forceinline__ void ws_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

constexpr int kWsTH = 4, kWsTW = 32, kWsHR = kWsTH + 2, kWsHW = kWsTW + 2;

}  // namespace

template <typename T, int CIN>
__global__ __launch_bounds__(512, 1) void halo3x3_ws_kernel(ConvArgs a, int tiles_w, int tiles_h, int ntiles) {
    constexpr int CPX = CIN / 8;                 // 16-byte chunks of channels per pixel
    constexpr int SPX = CPX + 1;                 // 16-byte slots per pixel in LDS (odd)
    constexpr int PSTR = SPX * 16;               // pixel stride in a halo buffer
    constexpr int NQ = kWsHR * kWsHW;            // halo pixels
    constexpr int NCHUNK = (NQ * SPX + 63) / 64;  // 1 KiB load chunks per halo
    constexpr int HBUF = NCHUNK * 1024;
    constexpr int NLD = (NCHUNK + 3) / 4;        // loads per loader lane per halo
    constexpr int KC = CIN / 16;                 // 16-wide k steps per tap
    constexpr int KS = 9 * KC;                   // k steps
    constexpr int XPIX = 64 * 4 + 16;            // hand-off tile: 64 fp32 channels per pixel, padded
    constexpr int XBUF = kWsTH * kWsTW * XPIX;
    constexpr int NRES = 4;                      // 16-byte units per epilogue lane per tile
    // One LDS array: halo buffers 0..2, the two hand-off tiles, then a sink for the load
    // chunks past a halo. Until the end of step 0 the 64-channel weights (Cout x 9*CIN
    // elements) sit in the space from halo buffer 2 on, which nothing else uses before
    // step 1 (halo 2 is issued in step 1, the first hand-off happens in step 1); their
    // rows are padded to an odd number of 16-byte pieces (RPC), so the 32 rows that one
    // operand fragment reads start in 16 distinct bank groups per 16 lanes.
    constexpr int XOFF = 3 * HBUF, SINK = XOFF + 2 * XBUF, WOFF = 2 * HBUF;
    constexpr int LDS_BYTES = SINK + 1024;
    constexpr int RPC = 9 * CIN / 8 + 1;             // 16-byte pieces per padded weight row
    constexpr int WCHP = (64 * RPC + 63) / 64;       // 1 KiB load chunks of the padded weights
    constexpr int WLD = (WCHP + 7) / 8;              // of them per wave
    static_assert(LDS_BYTES <= 160 * 1024 && WOFF + WCHP * 1024 <= SINK, "LDS");
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
    typedef typename Mfma32<T>::vec vec;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool compute_wave = wave < 4;
    const int rl = lane & 31, hi = lane >> 5;
    const int H = a.H, W = a.W, Cout = a.Cout;

    // tiles of this workgroup: t = s*G + r, the workgroups of one XCD (blockIdx % 8) taking
    // a contiguous run of each round's tiles (neighbouring halos share rows in one L2)
    const int G = gridDim.x;
    const int r = (G % 8) == 0 ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
    const int nsteps = r < ntiles ? (ntiles - r + G - 1) / G : 0;  // tiles of this workgroup
    struct Geo {
        int n, oy0, ox0;
        bool live;
    };
    auto geo = [&](int s) -> Geo {
        const int t = s * G + r;
        const bool live = s < nsteps;
        const int tt = live ? t : 0;
        const int tx = tt % tiles_w, rr = tt / tiles_w;
        return Geo{rr / tiles_h, (rr % tiles_h) * kWsTH, tx * kWsTW, live};
    };

    // Weights: every wave copies its share of the [64][9*CIN] block (rows past Cout read
    // as zeros) into LDS with 16-byte direct-to-LDS loads, in padded rows; the compute
    // waves take their operand fragments from there into registers while they compute
    // tile 0, so no separate copy stands between the loads and the first products.
    {
        const i32x4 rw = rsrc_words(a.w, (uint32_t)((size_t)Cout * 9 * CIN * sizeof(T)));
#pragma unroll
        for (int d = 0; d < WLD; ++d) {
            const int chunk = d * 8 + wave;
            const int q = chunk * 64 + lane, row = q / RPC, pc = q % RPC;
            const bool ok = chunk < WCHP && pc < RPC - 1 && row < Cout;
            dma_b128(rw, ok ? (uint32_t)((row * 9 * CIN + pc * 8) * (int)sizeof(T)) : kOOB,
                     lds_addr(lds + (chunk < WCHP ? WOFF + chunk * 1024 : SINK)));
        }
    }
    const uint32_t out_bytes = (uint32_t)((size_t)a.M * Cout * sizeof(T));

    if (compute_wave) {
        // ---- compute waves: wave (wn, wm) = channels 32*wn.., tile rows 2*wm, 2*wm + 1 ----
        const int wn = wave & 1, wm = wave >> 1;
        ws_wait_vmcnt<0>();
        ws_barrier();  // weights and the first halo in LDS
        vec bw[KS];
        // this lane's weight row (channel 32*wn + rl), piece 2*ks + hi for k step ks
        const char *wrow = lds + WOFF + (32 * wn + rl) * RPC * 16 + hi * 16;
        f32x16 acc[2][2];  // two tiles' sums: one accumulating, the previous one handed off
        auto compute = [&](auto cur, auto first, int s, auto hook) {
            constexpr int C = decltype(cur)::value;
            constexpr bool FIRST = decltype(first)::value;  // tile 0: the weights come from LDS
            const char *buf = lds + (s % 3) * HBUF;
            // B operand of tile row 2*wm + i at k step ks: halo pixel (row + ky, rl + kx),
            // channels 16*kc + 8*hi ..
            const char *base = buf + ((2 * wm) * kWsHW + rl) * PSTR + hi * 16;
            auto read = [&](int ks, vec(&f)[2]) {
                const int tap = ks / KC, kc = ks % KC, ky = tap / 3, kx = tap % 3;
                if constexpr (FIRST) bw[ks] = *reinterpret_cast<const vec *>(wrow + ks * 32);
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    f[i] = *reinterpret_cast<const vec *>(base + ((i + ky) * kWsHW + kx) * PSTR + kc * 32);
            };
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[C][i][e] = 0.0f;
            constexpr int PF = 2;  // operand reads run PF k steps ahead of the products
            vec f[PF + 1][2];
#pragma unroll
            for (int ks = 0; ks < PF; ++ks) read(ks, f[ks]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + PF < KS) read(ks + PF, f[(ks + PF) % (PF + 1)]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 2; ++i) acc[C][i] = Mfma32<T>::run(bw[ks], f[ks % (PF + 1)][i], acc[C][i]);
                __builtin_amdgcn_sched_barrier(0);
                hook(ks);
            }
        };
        auto no_hook = [](int) {};
        // hand-off of tile s: lane (rl, hi) holds channels 32*wn + 8*g + 4*hi + 0..3 of pixel rl
        auto handoff = [&](auto prev, int s) {
            constexpr int C = decltype(prev)::value;
            char *x = lds + XOFF + (s & 1) * XBUF;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int p = (2 * wm + i) * kWsTW + rl;
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<f32x4 *>(x + p * XPIX + (32 * wn + 8 * g + 4 * hi) * 4) =
                        f32x4{acc[C][i][4 * g], acc[C][i][4 * g + 1], acc[C][i][4 * g + 2], acc[C][i][4 * g + 3]};
            }
        };
        // The last tile's epilogue runs here, from the registers: its residual (this lane's
        // two 8-channel runs of each of its two rows) is loaded during the second half of
        // its products, when the weight fragments of the first half are no longer needed.
        const bool has_res = a.res != nullptr;
        const __amdgpu_buffer_rsrc_t rres = make_rsrc(a.res, has_res ? out_bytes : 0u);
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, out_bytes);
        // byte offset of the run of row i (0, 1), channels 32*wn + 16*pp + 8*hi .. of the last tile
        auto last_off = [&](int i, int pp) -> uint32_t {
            const Geo gl = geo(nsteps - 1);
            const int oy = gl.oy0 + 2 * wm + i, ox = gl.ox0 + rl, co = 32 * wn + 16 * pp + 8 * hi;
            return (gl.live && oy < H && ox < W && co < Cout)
                       ? (uint32_t)(((gl.n * H + oy) * W + ox) * Cout + co) * (uint32_t)sizeof(T)
                       : kOOB;
        };
        u32x4 lres[2][2];
        auto res_hook = [&](int ks) {
            if (ks == KS / 2) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp)
                        lres[i][pp] =
                            __builtin_amdgcn_raw_buffer_load_b128(rres, (int)(has_res ? last_off(i, pp) : kOOB), 0, 0);
            }
        };
        auto swap_halves = [](u32x2 &lo, u32x2 &hi2) {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const auto r2 = __builtin_amdgcn_permlane32_swap(lo[d], hi2[d], false, false);
                lo[d] = r2[0];
                hi2[d] = r2[1];
            }
        };
        // lane (rl, hi) holds channels 32*wn + 8*q + 4*hi + 0..3 (q < 4) of pixel rl of each
        // row; one lane-half swap per pair of groups (2*pp, 2*pp + 1) leaves 8 consecutive
        // channels 32*wn + 16*pp + 8*hi .. per lane, stored as one 16-byte run
        auto last_epilogue = [&](auto cur) {
            constexpr int C = decltype(cur)::value;
            const __amdgpu_buffer_rsrc_t rbias = make_rsrc(a.bias, a.bias ? (uint32_t)Cout * 4u : 0u);
            const __amdgpu_buffer_rsrc_t ralpha = make_rsrc(a.alpha, a.alpha ? (uint32_t)Cout * 4u : 0u);
            float bq[16], aq[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int co = 32 * wn + 8 * q + 4 * hi;
                const uint32_t bo = co < Cout ? (uint32_t)co * 4u : kOOB;
                const f32x4 bv4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rbias, (int)bo, 0, 0));
                const f32x4 av4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ralpha, (int)bo, 0, 0));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bq[4 * q + e] = bv4[e];
                    aq[4 * q + e] = av4[e];
                }
            }
            const int mode = has_res ? (a.res_before_act ? 1 : 2) : 0;
            auto finish = [&](auto act_tag, auto res_tag) {
                constexpr int ACT = decltype(act_tag)::value;
                constexpr int RES = decltype(res_tag)::value;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        u32x2 q2[2];
                        u32x2 rq[2] = {u32x2{lres[i][pp][0], lres[i][pp][1]}, u32x2{lres[i][pp][2], lres[i][pp][3]}};
                        if constexpr (RES != 0) swap_halves(rq[0], rq[1]);
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int q = 2 * pp + h;
                            T rt[4], o4[4];
                            __builtin_memcpy(rt, &rq[h], 8);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float v = acc[C][i][4 * q + e] + bq[4 * q + e];
                                if constexpr (RES == 1) v += to_f32(rt[e]);
                                if constexpr (ACT == CONV2D_ACT_RELU) v = v > 0.0f ? v : 0.0f;
                                if constexpr (ACT == CONV2D_ACT_SILU) v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
                                if constexpr (ACT == CONV2D_ACT_PRELU) v = v >= 0.0f ? v : aq[4 * q + e] * v;
                                if constexpr (RES == 2) v += to_f32(rt[e]);
                                o4[e] = round_fp32<T>(v);
                            }
                            __builtin_memcpy(&q2[h], o4, 8);
                        }
                        swap_halves(q2[0], q2[1]);
                        __builtin_amdgcn_raw_buffer_store_b128(u32x4{q2[0][0], q2[0][1], q2[1][0], q2[1][1]}, ry,
                                                               (int)last_off(i, pp), 0, 0);
                    }
            };
            auto with_res = [&](auto act_tag) {
                switch (mode) {
                case 1: finish(act_tag, std::integral_constant<int, 1>{}); break;
                case 2: finish(act_tag, std::integral_constant<int, 2>{}); break;
                default: finish(act_tag, std::integral_constant<int, 0>{}); break;
                }
            };
            switch (a.act) {
            case CONV2D_ACT_RELU: with_res(std::integral_constant<int, CONV2D_ACT_RELU>{}); break;
            case CONV2D_ACT_SILU: with_res(std::integral_constant<int, CONV2D_ACT_SILU>{}); break;
            case CONV2D_ACT_PRELU: with_res(std::integral_constant<int, CONV2D_ACT_PRELU>{}); break;
            default: with_res(std::integral_constant<int, CONV2D_ACT_NONE>{}); break;
            }
        };
        // Step s (1 <= s < nsteps): the sums of tile s-1 go to the hand-off tile while the
        // products of tile s run (the LDS writes and the matrix cores overlap), then the
        // barrier. The last tile's sums stay in the registers for its epilogue below.
        auto step = [&](auto cur, int s) {
            constexpr int C = decltype(cur)::value;
            if (s >= 1 && s < nsteps) handoff(std::integral_constant<int, 1 - C>{}, s - 1);
            if (s < nsteps) compute(cur, std::false_type{}, s, no_hook);
            if (s < nsteps) ws_barrier();
        };
        // step 0: tile 0 (every workgroup has one), taking the weights into registers
        compute(std::integral_constant<int, 0>{}, std::true_type{}, 0, no_hook);
        ws_barrier();
        for (int s = 1; s <= nsteps; s += 2) {
            step(std::integral_constant<int, 1>{}, s);
            if (s + 1 > nsteps) break;
            step(std::integral_constant<int, 0>{}, s + 1);
        }
        res_hook(KS / 2);
        if ((nsteps - 1) & 1)
            last_epilogue(std::integral_constant<int, 1>{});
        else
            last_epilogue(std::integral_constant<int, 0>{});
        return;
    }

    // ---- loader / epilogue waves ----
    const int we = wave - 4;
    const int te = we * 64 + lane;   // 0..255
    const int c8 = te & 7;           // this lane's 8-channel group, the same in every unit
    const i32x4 rx = rsrc_words(a.x, (uint32_t)((size_t)a.N * H * W * CIN * sizeof(T)));
    const bool has_res = a.res != nullptr;
    const __amdgpu_buffer_rsrc_t rres = make_rsrc(a.res, has_res ? out_bytes : 0u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, out_bytes);
    float bv[8], av[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int co = 8 * c8 + e;
        bv[e] = a.bias && co < Cout ? a.bias[co] : 0.0f;
        av[e] = a.alpha && co < Cout ? a.alpha[co] : 0.0f;
    }
    // Tile-invariant parts of this lane's halo slots: pixel (hy, hx) of the halo and
    // channel chunk c, as an element offset from the tile's corner pixel (row oy0 - 1,
    // column ox0 - 1); kNoPix marks a padding slot (nothing to load).
    constexpr uint32_t kNoPix = 0xffffffffu;
    int h_rel[NLD];
    uint32_t h_yx[NLD];  // hy << 8 | hx
#pragma unroll
    for (int d = 0; d < NLD; ++d) {
        const int slot = (d * 4 + we) * 64 + lane;
        const int q = slot / SPX, c = slot - q * SPX;
        const int hy = q / kWsHW, hx = q - hy * kWsHW;
        const bool real = c < CPX && q < NQ;
        h_rel[d] = (hy * W + hx) * CIN + c * 8;
        h_yx[d] = real ? (uint32_t)(hy << 8 | hx) : kNoPix;
    }
    // the same for this lane's output units: pixel (py, px) of the tile (kNoPix for a
    // channel group past Cout)
    int u_rel[NRES];
    uint32_t u_yx[NRES];
    const bool c_ok = 8 * c8 < Cout;
#pragma unroll
    for (int j = 0; j < NRES; ++j) {
        const int p = (te + 256 * j) >> 3, py = p / kWsTW, px = p % kWsTW;
        u_rel[j] = (py * W + px) * Cout + 8 * c8;
        u_yx[j] = c_ok ? (uint32_t)(py << 8 | px) : kNoPix;
    }

    // Fast paths for tiles away from the image border (wave-uniform tests): a halo wholly
    // inside the image needs no test per slot and an output tile wholly inside none per
    // unit, only a base offset plus the lane's offset. For a slot or unit with nothing to
    // load or store that lane offset is 2^31: x and y hold fewer than 2^31 bytes, so
    // base + 2^31 lies past the buffer without wrapping (an out-of-range access).
    constexpr uint32_t kFar = 0x80000000u;
    uint32_t h_relb[NLD], u_relb[NRES];
#pragma unroll
    for (int d = 0; d < NLD; ++d) h_relb[d] = h_yx[d] == kNoPix ? kFar : (uint32_t)h_rel[d] * (uint32_t)sizeof(T);
#pragma unroll
    for (int j = 0; j < NRES; ++j) u_relb[j] = u_yx[j] == kNoPix ? kFar : (uint32_t)u_rel[j] * (uint32_t)sizeof(T);

    // the input halo of tile s into buffer s % 3; a step past the last tile still issues
    // its loads, with out-of-range offsets (no traffic), so every step's count is the same
    auto issue_halo = [&](int s) {
        const Geo g = geo(s);
        char *buf = lds + (s % 3) * HBUF;
        const int corner = ((g.n * H + g.oy0 - 1) * W + g.ox0 - 1) * CIN;
        const bool inside = g.live && g.oy0 >= 1 && g.oy0 + kWsTH + 1 <= H && g.ox0 >= 1 && g.ox0 + kWsTW + 1 <= W;
        if (inside) {
            const uint32_t cb = (uint32_t)corner * (uint32_t)sizeof(T);
#pragma unroll
            for (int d = 0; d < NLD; ++d) {
                const int chunk = d * 4 + we;
                char *dst = chunk < NCHUNK ? buf + chunk * 1024 : lds + SINK;
                dma_b128(rx, cb + h_relb[d], lds_addr(dst));
            }
            return;
        }
#pragma unroll
        for (int d = 0; d < NLD; ++d) {
            const int chunk = d * 4 + we;
            const int iy = g.oy0 - 1 + (int)(h_yx[d] >> 8), ix = g.ox0 - 1 + (int)(h_yx[d] & 0xff);
            const bool ok =
                g.live && h_yx[d] != kNoPix && (unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W;
            char *dst = chunk < NCHUNK ? buf + chunk * 1024 : lds + SINK;
            dma_b128(rx, ok ? (uint32_t)(corner + h_rel[d]) * (uint32_t)sizeof(T) : kOOB, lds_addr(dst));
        }
    };
    // byte offset in y (and the residual) of this lane's unit j of tile s, or an
    // out-of-range offset
    auto tile_inside = [&](const Geo &g) { return g.live && g.oy0 + kWsTH <= H && g.ox0 + kWsTW <= W; };
    auto tile_base = [&](const Geo &g) {
        return (uint32_t)(((g.n * H + g.oy0) * W + g.ox0) * Cout) * (uint32_t)sizeof(T);
    };
    auto unit_off = [&](const Geo &g, int j) -> uint32_t {
        const int oy = g.oy0 + (int)(u_yx[j] >> 8), ox = g.ox0 + (int)(u_yx[j] & 0xff);
        return (g.live && u_yx[j] != kNoPix && oy < H && ox < W)
                   ? (uint32_t)(((g.n * H + g.oy0) * W + g.ox0) * Cout + u_rel[j]) * (uint32_t)sizeof(T)
                   : kOOB;
    };
    // the offsets of all this lane's units of tile g
    auto unit_offs = [&](const Geo &g, uint32_t (&off)[NRES]) {
        if (tile_inside(g)) {
            const uint32_t tb = tile_base(g);
#pragma unroll
            for (int j = 0; j < NRES; ++j) off[j] = tb + u_relb[j];
        } else {
#pragma unroll
            for (int j = 0; j < NRES; ++j) off[j] = unit_off(g, j);
        }
    };
    u32x4 res[3][NRES];
    auto issue_res = [&](auto slot, int s) {
        constexpr int I = decltype(slot)::value;
        const Geo g = geo(s);
        uint32_t off[NRES];
        unit_offs(g, off);
#pragma unroll
        for (int j = 0; j < NRES; ++j)
            res[I][j] = __builtin_amdgcn_raw_buffer_load_b128(rres, (int)(has_res ? off[j] : kOOB), 0, 0);
    };
    auto epilogue = [&](auto slot, int s) {
        constexpr int I = decltype(slot)::value;
        const Geo g = geo(s);
        const char *x = lds + XOFF + (s & 1) * XBUF;
        const int mode = has_res ? (a.res_before_act ? 1 : 2) : 0;
        uint32_t off[NRES];
        unit_offs(g, off);
        auto finish = [&](auto act_tag, auto res_tag) {
            constexpr int ACT = decltype(act_tag)::value;
            constexpr int RES = decltype(res_tag)::value;
#pragma unroll
            for (int j = 0; j < NRES; ++j) {
                const int p = (te + 256 * j) >> 3;
                const f32x4 v0 = *reinterpret_cast<const f32x4 *>(x + p * XPIX + c8 * 32);
                const f32x4 v1 = *reinterpret_cast<const f32x4 *>(x + p * XPIX + c8 * 32 + 16);
                T rt[8], out[8];
                __builtin_memcpy(rt, &res[I][j], 16);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float v = (e < 4 ? v0[e] : v1[e - 4]) + bv[e];
                    if constexpr (RES == 1) v += to_f32(rt[e]);
                    if constexpr (ACT == CONV2D_ACT_RELU) v = v > 0.0f ? v : 0.0f;
                    if constexpr (ACT == CONV2D_ACT_SILU) v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
                    if constexpr (ACT == CONV2D_ACT_PRELU) v = v >= 0.0f ? v : av[e] * v;
                    if constexpr (RES == 2) v += to_f32(rt[e]);
                    out[e] = round_fp32<T>(v);
                }
                u32x4 o;
                __builtin_memcpy(&o, out, 16);
                __builtin_amdgcn_raw_buffer_store_b128(o, ry, (int)off[j], 0, 0);
            }
        };
        auto with_res = [&](auto act_tag) {
            switch (mode) {
            case 1: finish(act_tag, std::integral_constant<int, 1>{}); break;
            case 2: finish(act_tag, std::integral_constant<int, 2>{}); break;
            default: finish(act_tag, std::integral_constant<int, 0>{}); break;
            }
        };
        switch (a.act) {
        case CONV2D_ACT_RELU: with_res(std::integral_constant<int, CONV2D_ACT_RELU>{}); break;
        case CONV2D_ACT_SILU: with_res(std::integral_constant<int, CONV2D_ACT_SILU>{}); break;
        case CONV2D_ACT_PRELU: with_res(std::integral_constant<int, CONV2D_ACT_PRELU>{}); break;
        default: with_res(std::integral_constant<int, CONV2D_ACT_NONE>{}); break;
        }
    };

    // Start: the halo and residual of tile 0 go out behind this wave's weight chunks;
    // the weights and the halo land (barrier). Only what tile 0 needs is in flight, so
    // the start-up burst of every CU carries no more than that.
    issue_halo(0);
    issue_res(std::integral_constant<int, 0>{}, 0);
    ws_wait_vmcnt<NRES>();  // the weights and the halo of tile 0
    ws_barrier();
    // Step s: the epilogue of tile s-2, whose sums the compute waves handed off during
    // step s-1 (its residual went out three steps before); the halo of tile s+2 issued;
    // the residual of tile s+1 issued into the register slot that epilogue just freed;
    // then a wait that leaves only this step's loads and stores in flight, so the halo
    // of tile s+1 is in LDS before the barrier that starts its products.
    // Halo buffer s+2 = s-1 (mod 3): its products ended at the barrier that began step s.
    // The epilogue comes before the halo loads: the compiler, which cannot see those
    // direct-to-LDS loads, counts fewer loads younger than the residual than there are,
    // and its wait for the residual would otherwise also wait for this step's halo.
    // Steps 0 and 1 differ: buffer 2 holds the weights until the end of step 0, so step
    // 0 issues the halo of tile 1 and waits for it, and step 1 those of tiles 2 and 3.
    constexpr int STEP_OPS = NLD + NRES + NRES;
    auto no_stores = [&]() {
#pragma unroll
        for (int j = 0; j < NRES; ++j)  // the same count of stores, none of them live
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, ry, (int)kOOB, 0, 0);
    };
    no_stores();
    issue_halo(1);
    issue_res(std::integral_constant<int, 1>{}, 1);
    ws_wait_vmcnt<NRES>();  // the halo of tile 1
    ws_barrier();
    no_stores();
    issue_halo(2);
    issue_halo(3);
    issue_res(std::integral_constant<int, 2>{}, 2);
    ws_wait_vmcnt<NLD + NRES>();  // the halo of tile 2
    if (nsteps > 1) ws_barrier();
    // The loaders run the epilogues of tiles 0 .. nsteps-2 (the compute waves that of the
    // last tile), so step s issues the halo of tile s+2 and the residual of tile s+1 only
    // while those are still to come (s + 3 <= nsteps); after that its wait leaves only its
    // stores in flight (the halo of tile s+1, where it is a tile, came before them). The
    // last step, nsteps, has no barrier: the compute waves have reached their last one.
    auto step = [&](auto slot, int s) {
        constexpr int I = decltype(slot)::value;  // s % 3
        epilogue(std::integral_constant<int, (I + 1) % 3>{}, s - 2);
        if (s + 3 <= nsteps) {
            issue_halo(s + 2);
            issue_res(std::integral_constant<int, (I + 1) % 3>{}, s + 1);
            ws_wait_vmcnt<STEP_OPS>();
        } else {
            ws_wait_vmcnt<NRES>();
        }
        if (s < nsteps) ws_barrier();
    };
    for (int s = 2; s <= nsteps; s += 3) {
        step(std::integral_constant<int, 2>{}, s);
        if (s + 1 > nsteps) break;
        step(std::integral_constant<int, 0>{}, s + 1);
        if (s + 2 > nsteps) break;
        step(std::integral_constant<int, 1>{}, s + 2);
    }
    ws_wait_vmcnt<0>();  // no direct-to-LDS load outlives the workgroup
}

template <typename T>
static hipError_t launch_ws_t(const ConvArgs &a, int grid_cap, hipStream_t st) {
    const int tiles_w = (a.W + kWsTW - 1) / kWsTW, tiles_h = (a.H + kWsTH - 1) / kWsTH;
    const long long nt = (long long)a.N * tiles_w * tiles_h;
    if (nt > 0x7fffffffll) return hipErrorInvalidValue;
    const int ntiles = (int)nt;
    int grid = ntiles < grid_cap ? ntiles : grid_cap;
    if (grid > 8) grid -= grid % 8;
    return launch_kernel(halo3x3_ws_kernel<T, 64>, dim3(grid), dim3(512), 0, st, a, tiles_w, tiles_h, ntiles);
}

hipError_t launch_halo3x3_ws(const ConvArgs &a, int dtype, int grid_cap, hipStream_t st) {
    if (a.Cin != 64 || a.Cout > 64 || a.kh != 3 || a.kw != 3 || a.stride != 1 || a.pad != 1)
        return hipErrorInvalidValue;
    switch (dtype) {
    case CONV2D_DTYPE_BF16: return launch_ws_t<bf16>(a, grid_cap, st);
    case CONV2D_DTYPE_F16: return launch_ws_t<f16>(a, grid_cap, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace c2d
