// 3x3 stride-1 or stride-2 pad-1 channel-last convolution for wide layers (Cin a multiple of the K
// chunk, or of 8 for channel-first outputs; Cout a multiple of 8) on CDNA4 matrix cores: the implicit GEMM of the
// inferencelayer page's `conv()` (m = output pixel, k = (tap, input channel), n = output
// channel, fused bias + activation epilogue) with halo tiles in place of a per-tap
// patch gather, as in the framecast page's tiled convolution shader.
//
// A workgroup owns a TH x TW tile of output pixels and CB output channels. Its K loop
// runs over chunks of CK input channels. A chunk is the tile's input halo, (TH+2) x
// (TW+2) pixels x CK channels, plus the weights of all nine taps for those channels
// and the workgroup's output channels, both copied into an NS-stage LDS ring with
// direct-to-LDS loads, so each input pixel crosses the memory pipe once per chunk for
// all nine taps instead of nine times. LDS rows are the CK channels of one halo pixel
// or one (tap, output channel) weight row, 2*CK bytes, whose 16-byte pieces are
// permuted by an XOR of the row number (piece q of row r sits at q ^ ((r / (16/RS)) %
// RS), RS pieces per row), which the loads apply on the global side; 16 consecutive
// rows then start in 16 different bank groups (16 consecutive pixels that wrap a tile
// row skip the two halo columns and can still meet two-way conflicts; the layout of the
// second kernel below has none).
//
// Waves form a WP x WC grid: wave (wp, wc) computes the tile's 32-pixel blocks wp,
// wp + WP, ... for the FN 32-channel blocks wc*FN .. wc*FN + FN - 1, with 32x32x16
// products (weights the A operand, pixels the B operand), and runs the fused epilogue
// from registers: bias, residual before or after the activation, activation, one
// rounding, 16-byte stores of 8 channels (pairs of 4-channel groups joined across the
// wave halves by v_permlane32_swap).
//
// The second kernel (specialised waves) computes the same layer with loader waves that
// only copy and compute waves that only multiply, the K chunk split over the compute
// waves; it leads where one workgroup per CU has to carry a deep K (512 channels).
#include <utility>

#include "igemm_common.hpp"
#include "kernels.hpp"

namespace c2d {

namespace {

template <int N> __device__ __forceinline__ void hg_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier after this wave's LDS accesses have completed (s_barrier alone does
// not wait for them: a partial sum written just before it could still be in flight).
__device__ __forceinline__ void hg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

constexpr uint32_t kHgBad = 0x80000000u;  // offset of a load with nothing to fetch (past every tensor)

}  // namespace

// Compile-time geometry of one kernel variant.
template <int TH_, int TW_, int WP_, int WC_, int FN_, int NS_, int CK_, int PD_, int S_ = 1>
struct HgCfg {
    static constexpr int TH = TH_, TW = TW_, WP = WP_, WC = WC_, FN = FN_, NS = NS_, CK = CK_;
    static constexpr int PD = PD_;                     // k steps of operand reads ahead
    static constexpr int S = S_;                       // stride (1 or 2; pad 1)
    static constexpr int NW = WP * WC;                 // waves per workgroup
    static constexpr int P = TH * TW;                  // tile pixels
    static constexpr int NBLK = (P + 31) / 32;         // 32-pixel blocks of the tile
    static constexpr int NBW = (NBLK + WP - 1) / WP;   // blocks per wave (at most)
    static constexpr int CB = 32 * FN * WC;            // output channels per workgroup
    static constexpr int HW2 = S * (TW - 1) + 3;      // halo columns
    static constexpr int HR = (S * (TH - 1) + 3) * HW2;  // halo rows (pixels)
    static constexpr int WR = 9 * CB;                  // weight rows
    static constexpr int RS = CK / 8;                  // 16-byte pieces per row
    static constexpr int RB = 2 * CK;                  // bytes per row
    static constexpr int SWZ = 16 / RS;                // rows per step of the XOR pattern
    static constexpr int KS = CK / 16;                 // 16-deep k steps per tap
    static constexpr int HCH = (HR * RS + 63) / 64;    // 1 KiB loads of the halo
    static constexpr int WCH = (WR * RS + 63) / 64;    // 1 KiB loads of the weights
    static constexpr int NCH = HCH + WCH;
    static constexpr int NLD = (NCH + NW - 1) / NW;    // loads per wave per chunk
    static constexpr int WOFF = HCH * 1024;            // weights within a stage
    static constexpr int STAGE = NCH * 1024;
    static constexpr int SINK = NS * STAGE;            // landing place of the padding loads
    static constexpr int LDS = SINK + 1024;
    static_assert(CK == 16 || CK == 32 || CK == 64, "K chunk of 16, 32 or 64 channels");
    static_assert((NS - 2) * NLD < 64 && NS >= 2, "outstanding loads fit the counter");
    static_assert(PD >= 1 && PD < 9 * KS, "operand read-ahead within one chunk");
    static_assert(NBW * WP >= NBLK, "every pixel block has a wave");
    static_assert(LDS <= 160 * 1024, "LDS of one CU");
    static_assert(S == 1 || S == 2, "stride 1 or 2");
};

template <typename T, typename C, bool NCHW>
__global__ __launch_bounds__(64 * C::NW, 1) void hgemm3x3_kernel(ConvArgs a, HgemmGeo g) {
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
    typedef typename Mfma32<T>::vec vec;
    constexpr int NBW = C::NBW, FN = C::FN, KS = C::KS, RS = C::RS, RB = C::RB, NLD = C::NLD;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wp = wave % C::WP, wc = wave / C::WP;
    const int rl = lane & 31, hi = lane >> 5;
    const int H = a.H, W = a.W, Cin = a.Cin, Cout = a.Cout;
    const int OH = a.OH, OW = a.OW;

    // Tile of this workgroup. Workgroups go to the 8 XCDs round-robin (blockIdx % 8);
    // each XCD gets a contiguous run of tile ids, and consecutive ids vary the pixel
    // tile fastest (g.cfast == 0: the XCD shares weights) or the channel tile fastest
    // (g.cfast == 1: it shares halos), whichever keeps less data per XCD.
    const int G = gridDim.x, q8 = G / 8, r8 = G % 8, xcd = blockIdx.x % 8;
    const int t = xcd * q8 + (xcd < r8 ? xcd : r8) + blockIdx.x / 8;
    const int npt = g.ntiles_p;
    const int tc = g.cfast ? t % g.tiles_c : t / npt;
    const int tp = g.cfast ? t / g.tiles_c : t % npt;
    const int tx = tp % g.tiles_x, tq = tp / g.tiles_x;
    const int ty = tq % g.tiles_y, n = tq / g.tiles_y;
    const int oy0 = ty * C::TH, ox0 = tx * C::TW, co0 = tc * C::CB;

    // This thread's direct-to-LDS slots: load d of this wave is 1 KiB chunk d*NW + wave
    // of a stage (halo chunks, then weight chunks, then padding that goes to the sink),
    // lane l its 16-byte slot l. base[d] is the byte offset of the slot's data for
    // input-channel chunk 0 (chunk c adds c*CK elements), or kHgBad where there is
    // nothing to load (a halo pixel outside the image or past the halo, a weight row
    // past Cout or past the weights): such loads write zeros. The channel-first
    // instantiation also takes a Cin that is not a multiple of CK: its last chunk is
    // partial, and bit d of lastok says whether slot d's 8 channels lie inside it (the
    // others load zeros there, for the pixels and the weights alike, so the k steps past
    // Cin add zero products). The channel-last one needs whole chunks, which keeps its
    // copy path free of that test.
    constexpr bool PARTIAL = NCHW;
    uint32_t base[NLD];
    uint32_t lastok = 0;
    const int nfull = Cin / C::CK, crem = PARTIAL ? Cin - nfull * C::CK : 0;
#pragma unroll
    for (int d = 0; d < NLD; ++d) {
        const int ch = d * C::NW + wave;
        uint32_t b = kHgBad;
        int qv = 0;
        if (ch < C::HCH) {
            const int s = ch * 64 + lane, r = s / RS, pos = s % RS;
            qv = pos ^ ((r / C::SWZ) % RS);
            if (r < C::HR) {
                const int hy = r / C::HW2, hx = r % C::HW2;
                const int iy = C::S * oy0 - 1 + hy, ix = C::S * ox0 - 1 + hx;
                if ((unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W)
                    b = (uint32_t)((((n * H + iy) * W + ix) * Cin + qv * 8) * (int)sizeof(T));
            }
        } else if (ch < C::NCH) {
            const int s = (ch - C::HCH) * 64 + lane, r = s / RS, pos = s % RS;
            qv = pos ^ ((r / C::SWZ) % RS);
            if (r < C::WR) {
                const int tap = r / C::CB, co = co0 + r % C::CB;
                if (co < Cout) b = (uint32_t)((((co * 9 + tap) * Cin) + qv * 8) * (int)sizeof(T));
            }
        }
        base[d] = b;
        if (PARTIAL && qv * 8 < crem) lastok |= 1u << d;
    }
    const i32x4 rx = rsrc_words(a.x, (uint32_t)((size_t)a.N * H * W * Cin * sizeof(T)));
    const i32x4 rw = rsrc_words(a.w, (uint32_t)((size_t)Cout * 9 * Cin * sizeof(T)));
    const int nchunks = nfull + (crem != 0 ? 1 : 0);
    const uint32_t lds0 = lds_addr(lds);
    // Issues input-channel chunk c into stage st. A chunk past the last one issues the
    // same loads at out-of-range offsets, so that every chunk adds exactly NLD to this
    // wave's count of outstanding vector-memory operations.
    auto issue_one = [&](int c, int st, int d) {
        const int ch = d * C::NW + wave;
        const uint32_t dst = ch < C::NCH ? lds0 + st * C::STAGE + ch * 1024 : lds0 + C::SINK;
        uint32_t off;
        if constexpr (PARTIAL) {
            const bool live = c < nfull || (c < nchunks && ((lastok >> d) & 1u) != 0);
            off = (base[d] == kHgBad || !live) ? kHgBad : base[d] + (uint32_t)(c * C::CK * (int)sizeof(T));
        } else {
            const uint32_t cadd = c < nchunks ? (uint32_t)(c * C::CK * (int)sizeof(T)) : kHgBad;
            off = base[d] == kHgBad ? kHgBad : base[d] + cadd;
        }
        dma_b128(ch < C::HCH ? rx : rw, off, dst);
    };
    auto issue = [&](int c, int st) {
#pragma unroll
        for (int d = 0; d < NLD; ++d) issue_one(c, st, d);
    };

    // Operand offsets within a stage. B (pixels): lane rl of block b = wp + WP*i is tile
    // pixel p = 32*b + rl at halo row (py + ky)*HW2 + px + kx for tap (ky, kx); lanes of a
    // block past the tile read row 0 (their sums are never stored). A (weights): row
    // tap*CB + 32*(wc*FN + j) + rl. Lane half hi reads piece 2*ks + hi of the row.
    int nb = 0;  // blocks of this wave inside the tile
    uint32_t boff[NBW][9][KS];
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const int b = wp + C::WP * i;
        const int p = 32 * b + rl;
        const bool in = b < C::NBLK && p < C::P;
        const int py = in ? p / C::TW : 0, px = in ? p % C::TW : 0;
        nb += b < C::NBLK ? 1 : 0;
#pragma unroll
        for (int tap = 0; tap < 9; ++tap) {
            const int r = (C::S * py + tap / 3) * C::HW2 + C::S * px + tap % 3;
            const int sw = (r / C::SWZ) % RS;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) boff[i][tap][ks] = (uint32_t)(r * RB + (((2 * ks + hi) ^ sw) << 4));
        }
    }
    uint32_t aoff[KS];
    {
        const int sw = (rl / C::SWZ) % RS;  // the same for every row tap*CB + 32*(...) + rl
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            aoff[ks] = (uint32_t)(C::WOFF + (32 * wc * FN + rl) * RB + (((2 * ks + hi) ^ sw) << 4));
    }

    f32x16 acc[NBW][FN];
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // The products of one chunk held in stage `sb` (byte offset): 9 taps x KS k steps,
    // with the operand fragments of step s + PD read from LDS while step s multiplies
    // (PD + 1 fragment buffers; the scheduling barriers keep that order).
    constexpr int NSTEP = 9 * KS, PD = C::PD, NBF = PD + 1;
    static_assert(NLD <= NSTEP, "one copy per k step at most");
    auto load = [&](uint32_t sb, int s, vec (&fa)[FN], vec (&fb)[NBW]) {
        const char *L = lds;
        const int tap = s / KS, ks = s % KS;
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fa[j] = *reinterpret_cast<const vec *>(L + sb + aoff[ks] + (tap * C::CB + 32 * j) * RB);
#pragma unroll
        for (int i = 0; i < NBW; ++i)
            if (i < nb) fb[i] = *reinterpret_cast<const vec *>(L + sb + boff[i][tap][ks]);
    };
    // The products of a chunk also issue the copies of chunk nc into stage nst, spread
    // over the k steps (copy d after the products of step d*NSTEP/NLD), so the memory
    // pipe fills the stage while the matrix cores run instead of the wave stalling on a
    // burst of copies before its products.
    auto compute = [&](uint32_t sb, int nc, int nst) {
        vec fa[NBF][FN], fb[NBF][NBW];
#pragma unroll
        for (int s = 0; s < PD; ++s) load(sb, s, fa[s], fb[s]);
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            if (s + PD < NSTEP) load(sb, s + PD, fa[(s + PD) % NBF], fb[(s + PD) % NBF]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NBW; ++i)
                if (i < nb)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = Mfma32<T>::run(fa[s % NBF][j], fb[s % NBF][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int d = 0; d < NLD; ++d)
                if (d * NSTEP / NLD == s) issue_one(nc, nst, d);
        }
    };

    // Ring of NS stages: chunk c lives in stage c % NS and is issued NS-1 chunks ahead.
    // Per chunk: wait for this wave's loads of chunk c, barrier (every wave's loads of
    // it have landed, and every wave is done with chunk c-1, whose stage is refilled
    // next), then the products of chunk c, which issue chunk c+NS-1 into that stage as
    // they go.
    [&]<int... I>(std::integer_sequence<int, I...>) { (issue(I, I), ...); }(std::make_integer_sequence<int, C::NS - 1>{});
    int st = 0;
    for (int c = 0; c < nchunks; ++c) {
        hg_wait_vmcnt<(C::NS - 2) * NLD>();
        hg_barrier();
        const int nst = st == 0 ? C::NS - 1 : st - 1;  // (c + NS - 1) % NS
        compute((uint32_t)(st * C::STAGE), c + C::NS - 1, nst);
        st = st + 1 == C::NS ? 0 : st + 1;
    }
    hg_wait_vmcnt<0>();

    // Epilogue from registers. Block (i, j): lane (rl, hi) holds channels 8*q + 4*hi +
    // 0..3 (q < 4) of the block's 32, for pixel rl; one lane-half swap per pair of groups
    // (2*pp, 2*pp + 1) leaves lane (rl, hi) with 8 consecutive channels 16*pp + 8*hi..
    // (lanes 32..63 of the first group trade with lanes 0..31 of the second), stored as
    // one 16-byte run. With NCHW, y and the residual are channel-first instead: each
    // value is read and stored as one 16-bit element of its channel plane (before the
    // swap), and the same rounded values also go channel-last to y2 when it is set (the
    // input copy of the next channel-first conv of a stack).
    const uint32_t out_bytes = (uint32_t)((size_t)a.M * Cout * sizeof(T));
    const bool has_res = a.res != nullptr;
    const __amdgpu_buffer_rsrc_t rres = make_rsrc(a.res, has_res ? out_bytes : 0u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, out_bytes);
    const bool store_cl = !NCHW || a.y2 != nullptr;  // channel-last runs are stored
    const __amdgpu_buffer_rsrc_t rcl = NCHW ? make_rsrc(a.y2, a.y2 ? out_bytes : 0u) : ry;
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(a.bias, a.bias ? (uint32_t)Cout * 4u : 0u);
    const __amdgpu_buffer_rsrc_t ralpha = make_rsrc(a.alpha, a.alpha ? (uint32_t)Cout * 4u : 0u);
    const uint32_t plane = (uint32_t)OH * (uint32_t)OW;
    auto swap_halves = [](u32x2 &lo, u32x2 &hi2) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const auto r2 = __builtin_amdgcn_permlane32_swap(lo[d], hi2[d], false, false);
            lo[d] = r2[0];
            hi2[d] = r2[1];
        }
    };
    uint32_t off[NBW][FN][2];  // channel-last byte offsets of this lane's two 8-channel runs
    uint32_t opx[NBW];         // channel-first: the pixel's index within its plane, or kOOB
    u32x4 rv[NBW][FN][2];
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const int b = wp + C::WP * i;
        const int p = 32 * b + rl;
        const int py = p / C::TW, px = p % C::TW;
        const int oy = oy0 + py, ox = ox0 + px;
        const bool pin = b < C::NBLK && p < C::P && oy < OH && ox < OW;
        opx[i] = pin ? (uint32_t)(oy * OW + ox) : kOOB;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int co = co0 + 32 * (wc * FN + j) + 16 * pp + 8 * hi;
                off[i][j][pp] = (pin && co < Cout)
                                    ? ((uint32_t)((n * OH + oy) * OW + ox) * (uint32_t)Cout + (uint32_t)co) *
                                          (uint32_t)sizeof(T)
                                    : kOOB;
                rv[i][j][pp] = (has_res && !NCHW) ? __builtin_amdgcn_raw_buffer_load_b128(rres, (int)off[i][j][pp], 0, 0)
                                                  : u32x4{0u, 0u, 0u, 0u};
            }
    }
    const int mode = has_res ? (a.res_before_act ? 1 : 2) : 0;
    auto finish = [&](auto act_tag, auto res_tag) {
        constexpr int ACT = decltype(act_tag)::value;
        constexpr int RES = decltype(res_tag)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            // bias and slopes of this lane's channels: group q is 32*(wc*FN + j) + 8*q + 4*hi + 0..3
            float bq[16], aq[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int co = co0 + 32 * (wc * FN + j) + 8 * q + 4 * hi;
                const uint32_t bo = co < Cout ? (uint32_t)co * 4u : kOOB;
                // (whole-vector casts: this compiler's __builtin_bit_cast of a single
                // vector element reads element 0 whatever the index)
                const f32x4 bv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rbias, (int)bo, 0, 0));
                const f32x4 av = ACT == CONV2D_ACT_PRELU
                                     ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ralpha, (int)bo, 0, 0))
                                     : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bq[4 * q + e] = bv[e];
                    aq[4 * q + e] = av[e];
                }
            }
#pragma unroll
            for (int i = 0; i < NBW; ++i) {
                if (i >= nb) continue;
                // channel-first element offsets of group q (channel co0 + 32*(wc*FN+j) + 8*q + 4*hi + e
                // at offset oq[q] + e * plane elements), and the residual read from there
                uint32_t oq[4] = {kOOB, kOOB, kOOB, kOOB};
                T rn[16];
                if constexpr (NCHW) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int co = co0 + 32 * (wc * FN + j) + 8 * q + 4 * hi;  // co + 3 < Cout iff co < Cout
                        oq[q] = (opx[i] != kOOB && co < Cout) ? ((uint32_t)(n * Cout + co) * plane + opx[i]) : kOOB;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            uint16_t u = 0;
                            if constexpr (RES != 0)
                                u = __builtin_amdgcn_raw_buffer_load_b16(
                                    rres, (int)(oq[q] == kOOB ? kOOB : (oq[q] + (uint32_t)e * plane) * 2u), 0, 0);
                            __builtin_memcpy(&rn[4 * q + e], &u, 2);
                        }
                    }
                }
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    u32x2 q2[2];
                    u32x2 rq[2] = {u32x2{rv[i][j][pp][0], rv[i][j][pp][1]}, u32x2{rv[i][j][pp][2], rv[i][j][pp][3]}};
                    if constexpr (RES != 0 && !NCHW) swap_halves(rq[0], rq[1]);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int q = 2 * pp + h;
                        T rt[4], out[4];
                        if constexpr (NCHW)
                            __builtin_memcpy(rt, &rn[4 * q], 8);
                        else
                            __builtin_memcpy(rt, &rq[h], 8);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float v = acc[i][j][4 * q + e] + bq[4 * q + e];
                            if constexpr (RES == 1) v += to_f32(rt[e]);
                            if constexpr (ACT == CONV2D_ACT_RELU) v = v > 0.0f ? v : 0.0f;
                            if constexpr (ACT == CONV2D_ACT_SILU) v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
                            if constexpr (ACT == CONV2D_ACT_PRELU) v = v >= 0.0f ? v : aq[4 * q + e] * v;
                            if constexpr (RES == 2) v += to_f32(rt[e]);
                            out[e] = round_fp32<T>(v);
                            if constexpr (NCHW) {
                                uint16_t u;
                                __builtin_memcpy(&u, &out[e], 2);
                                __builtin_amdgcn_raw_buffer_store_b16(
                                    u, ry, (int)(oq[q] == kOOB ? kOOB : (oq[q] + (uint32_t)e * plane) * 2u), 0, 0);
                            }
                        }
                        __builtin_memcpy(&q2[h], out, 8);
                    }
                    if (store_cl) {
                        swap_halves(q2[0], q2[1]);
                        __builtin_amdgcn_raw_buffer_store_b128(u32x4{q2[0][0], q2[0][1], q2[1][0], q2[1][1]}, rcl,
                                                               (int)off[i][j][pp], 0, 0);
                    }
                }
            }
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
}

// ---- specialised waves, K split over the compute waves ----
//
// The same layer with the memory traffic and the products in different waves. Per
// 64-channel chunk, four loader waves copy the tile's halo and the chunk's weights (all
// nine taps, CB output channels) into a two-stage LDS ring with direct-to-LDS loads, so
// a wave that stalls on a full memory pipe is never one that feeds a matrix core. The
// chunk's four 16-deep k steps are split over the compute waves: compute wave w takes k
// step w % 4 of every chunk for the whole tile (all pixel blocks, all channel blocks), so
// one pixel fragment read from LDS feeds FN products and one weight fragment NBLK; the
// partial sums of the compute waves are added through LDS at the end. Both operands come
// from LDS; with TS = 2 the nine taps of a k step are split between two compute waves
// (even and odd taps), which share a SIMD: twice the waves reading LDS, the same LDS
// traffic and matrix-core work per SIMD. Halo pixel (hy, hx) and weight row (tap, co) take 128-byte slots whose
// 16-byte pieces are permuted by an XOR (((hy*TW + hx) >> 1) & 7 for the halo, (row >> 1)
// & 7 for the weights), applied on the global side of the copies; 16 consecutive
// output pixels or weight rows then read 16 different bank groups.
template <int TH_, int TW_, int FN_, int PD_, int TS_>
struct HgwCfg {
    static constexpr int TH = TH_, TW = TW_, FN = FN_, PD = PD_, TS = TS_;
    static constexpr int NCW = 4 * TS;                 // compute waves
    static constexpr int NWV = NCW + 4;                // waves per workgroup
    static constexpr int NTAP = (9 + TS - 1) / TS;     // taps of compute wave 0 (the most)
    static constexpr int CK = 64;
    static constexpr int P = TH * TW;
    static constexpr int NBLK = (P + 31) / 32;
    static constexpr int NU = NBLK * FN;
    static constexpr int CB = 32 * FN;
    static constexpr int HW2 = TW + 2;
    static constexpr int HR = (TH + 2) * HW2;
    static constexpr int WR = 9 * CB;
    static constexpr int HCH = (HR * 8 + 63) / 64;     // 1 KiB copies of the halo
    static constexpr int WCH = (WR * 8 + 63) / 64;     // 1 KiB copies of the weights
    static constexpr int NCH = HCH + WCH;
    static constexpr int NLD = (NCH + 3) / 4;          // copies per loader wave per chunk
    static constexpr int WOFF = HCH * 1024;
    static constexpr int STAGE = NCH * 1024;
    static constexpr int SINK = 2 * STAGE;
    static constexpr int RED = (NCW - 1) * NU * 4096;
    static constexpr int LDS = (SINK + 1024 > RED ? SINK + 1024 : RED);
    static_assert(TW % 2 == 0, "the bank pattern needs an even tile width");
    static_assert(LDS <= 160 * 1024, "LDS of one CU");
    static_assert(NLD < 64, "outstanding copies fit the counter");
    static_assert(TS == 1 || TS == 2, "taps split over one or two waves");
};

template <typename T, typename C>
__global__ __launch_bounds__(64 * C::NWV, 1) void hgemmws3x3_kernel(ConvArgs a, HgemmGeo g) {
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
    typedef typename Mfma32<T>::vec vec;
    constexpr int NBLK = C::NBLK, FN = C::FN, NLD = C::NLD;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool loader = wave >= C::NCW;
    constexpr int TS = C::TS, NCW = C::NCW;
    const int rl = lane & 31, hi = lane >> 5;
    const int H = a.H, W = a.W, Cin = a.Cin, Cout = a.Cout;

    const int G = gridDim.x, q8 = G / 8, r8 = G % 8, xcd = blockIdx.x % 8;
    const int t = xcd * q8 + (xcd < r8 ? xcd : r8) + blockIdx.x / 8;
    const int npt = g.ntiles_p;
    const int tc = g.cfast ? t % g.tiles_c : t / npt;
    const int tp = g.cfast ? t / g.tiles_c : t % npt;
    const int tx = tp % g.tiles_x, tq = tp / g.tiles_x;
    const int ty = tq % g.tiles_y, n = tq / g.tiles_y;
    const int oy0 = ty * C::TH, ox0 = tx * C::TW, co0 = tc * C::CB;
    const int nch = Cin / C::CK;
    const uint32_t lds0 = lds_addr(lds);

    if (loader) {
        // copy d of loader wave lw: 1 KiB chunk d*4 + lw of a stage (halo, weights, then
        // padding that lands in the sink); lane l its 16-byte slot l
        const int lw = wave - NCW;
        uint32_t base[NLD];
#pragma unroll
        for (int d = 0; d < NLD; ++d) {
            const int ch = d * 4 + lw;
            uint32_t b = kHgBad;
            if (ch < C::HCH) {
                const int s = ch * 64 + lane, L = s >> 3, pos = s & 7;
                if (L < C::HR) {
                    const int hy = L / C::HW2, hx = L % C::HW2;
                    const int qv = pos ^ (((hy * C::TW + hx) >> 1) & 7);
                    const int iy = oy0 - 1 + hy, ix = ox0 - 1 + hx;
                    if ((unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W)
                        b = (uint32_t)((((n * H + iy) * W + ix) * Cin + qv * 8) * (int)sizeof(T));
                }
            } else if (ch < C::NCH) {
                const int s = (ch - C::HCH) * 64 + lane, r = s >> 3, pos = s & 7;
                if (r < C::WR) {
                    const int qv = pos ^ ((r >> 1) & 7);
                    const int tap = r / C::CB, co = co0 + r % C::CB;
                    if (co < Cout) b = (uint32_t)((((co * 9 + tap) * Cin) + qv * 8) * (int)sizeof(T));
                }
            }
            base[d] = b;
        }
        const i32x4 rx = rsrc_words(a.x, (uint32_t)((size_t)a.N * H * W * Cin * sizeof(T)));
        const i32x4 rw = rsrc_words(a.w, (uint32_t)((size_t)Cout * 9 * Cin * sizeof(T)));
        auto issue = [&](int c, int st) {
            const uint32_t cadd = (uint32_t)(c * C::CK * (int)sizeof(T));
#pragma unroll
            for (int d = 0; d < NLD; ++d) {
                const int ch = d * 4 + lw;
                const uint32_t dst = ch < C::NCH ? lds0 + st * C::STAGE + ch * 1024 : lds0 + C::SINK;
                const uint32_t off = base[d] == kHgBad ? kHgBad : base[d] + cadd;
                dma_b128(ch < C::HCH ? rx : rw, off, dst);
            }
        };
        // chunk 0, then per chunk c: barrier (compute waves are done with chunk c-1's
        // stage), copy chunk c+1 into it, wait for the copies
        issue(0, 0);
        hg_wait_vmcnt<0>();
        hg_barrier();
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) {
                issue(c + 1, (c + 1) & 1);
                hg_wait_vmcnt<0>();
            }
            hg_barrier();
        }
        // the sums of the compute waves pass through LDS: one more barrier
        hg_barrier();
        return;
    }

    // compute wave w: k step ks = w % 4, taps th, th + TS, ... (th = w / 4); its ntap taps
    const int ks = wave % 4, th = wave / 4;
    const int ntap = (9 - th + TS - 1) / TS;
    // pixel fragment offsets (block i, the wave's tap u) and weight rows
    uint32_t boff[NBLK][C::NTAP];
#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
        const int p = 32 * i + rl;
        const bool in = p < C::P;
        const int py = in ? p / C::TW : 0, px = in ? p % C::TW : 0;
#pragma unroll
        for (int u = 0; u < C::NTAP; ++u) {
            const int tap = th + TS * u < 9 ? th + TS * u : 8;
            const int hy = py + tap / 3, hx = px + tap % 3;
            const int L = hy * C::HW2 + hx, q = 2 * ks + hi;
            boff[i][u] = (uint32_t)(L * 128 + ((q ^ (((hy * C::TW + hx) >> 1) & 7)) << 4));
        }
    }
    // weight row tap*CB + 32*j + rl: (row >> 1) & 7 == (rl >> 1) & 7 for every tap and j
    const uint32_t aoff = (uint32_t)(C::WOFF + rl * 128 + (((2 * ks + hi) ^ ((rl >> 1) & 7)) << 4));

    f32x16 acc[NBLK][FN];
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    auto compute = [&](int st) {
        const char *S = lds + st * C::STAGE;
        constexpr int NBF = C::PD + 1;
        vec fa[NBF][FN], fb[NBF][NBLK];
        // the wave's u-th tap (a wave with fewer taps repeats its last one's reads and
        // skips its products)
        auto rd = [&](int u, vec (&ra)[FN], vec (&rb)[NBLK]) {
            const int tap = th + TS * u < 9 ? th + TS * u : 8;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                ra[j] = *reinterpret_cast<const vec *>(S + aoff + (tap * C::CB + 32 * j) * 128);
#pragma unroll
            for (int i = 0; i < NBLK; ++i) rb[i] = *reinterpret_cast<const vec *>(S + boff[i][u]);
        };
        constexpr int NT = C::NTAP;
#pragma unroll
        for (int s = 0; s < C::PD && s < NT; ++s) rd(s, fa[s], fb[s]);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            if (u + C::PD < NT) rd(u + C::PD, fa[(u + C::PD) % NBF], fb[(u + C::PD) % NBF]);
            __builtin_amdgcn_sched_barrier(0);
            if (u < ntap) {
#pragma unroll
                for (int i = 0; i < NBLK; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = Mfma32<T>::run(fa[u % NBF][j], fb[u % NBF][i], acc[i][j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    hg_barrier();
    for (int c = 0; c < nch; ++c) {
        compute(c & 1);
        hg_barrier();
    }

    // Sum of the compute waves' partials: unit (32x32 block) v = i*FN + j is finished by
    // compute wave v % 4; the other NCW - 1 waves leave theirs in LDS, [unit][sender
    // slot][16 values][64 lanes] fp32.
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int v = i * FN + j, own = v % 4;
            if (own != wave) {
                const int slot = wave - (wave > own ? 1 : 0);
                float *dst = red + ((v * (NCW - 1) + slot) * 16) * 64 + lane;
#pragma unroll
                for (int e = 0; e < 16; ++e) dst[e * 64] = acc[i][j][e];
            }
        }
    hg_barrier();
    if (wave >= 4) return;
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int v = i * FN + j;
            if (v % 4 == wave) {
#pragma unroll
                for (int sl = 0; sl < NCW - 1; ++sl) {
                    const float *src = red + ((v * (NCW - 1) + sl) * 16) * 64 + lane;
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] += src[e * 64];
                }
            }
        }

    // Epilogue of this wave's units, as in the kernel above: block (i, j), lane (rl, hi)
    // holds channels 8*q + 4*hi + 0..3 (q < 4) of block j for pixel rl of block i.
    const uint32_t out_bytes = (uint32_t)((size_t)a.M * Cout * sizeof(T));
    const bool has_res = a.res != nullptr;
    const __amdgpu_buffer_rsrc_t rres = make_rsrc(a.res, has_res ? out_bytes : 0u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, out_bytes);
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(a.bias, a.bias ? (uint32_t)Cout * 4u : 0u);
    const __amdgpu_buffer_rsrc_t ralpha = make_rsrc(a.alpha, a.alpha ? (uint32_t)Cout * 4u : 0u);
    auto swap_halves = [](u32x2 &lo, u32x2 &hi2) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const auto r2 = __builtin_amdgcn_permlane32_swap(lo[d], hi2[d], false, false);
            lo[d] = r2[0];
            hi2[d] = r2[1];
        }
    };
    const int mode = has_res ? (a.res_before_act ? 1 : 2) : 0;
    auto finish = [&](auto act_tag, auto res_tag) {
        constexpr int ACT = decltype(act_tag)::value;
        constexpr int RES = decltype(res_tag)::value;
#pragma unroll
        for (int i = 0; i < NBLK; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if ((i * FN + j) % 4 != wave) continue;
                const int p = 32 * i + rl;
                const int py = p / C::TW, px = p % C::TW;
                const int oy = oy0 + py, ox = ox0 + px;
                const bool pin = p < C::P && oy < H && ox < W;
                uint32_t off[2];
                u32x4 rv[2];
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const int co = co0 + 32 * j + 16 * pp + 8 * hi;
                    off[pp] = (pin && co < Cout) ? ((uint32_t)((n * H + oy) * W + ox) * (uint32_t)Cout + (uint32_t)co) *
                                                       (uint32_t)sizeof(T)
                                                 : kOOB;
                    rv[pp] = RES != 0 ? __builtin_amdgcn_raw_buffer_load_b128(rres, (int)off[pp], 0, 0)
                                      : u32x4{0u, 0u, 0u, 0u};
                }
                float bq[16], aq[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int co = co0 + 32 * j + 8 * q + 4 * hi;
                    const uint32_t bo = co < Cout ? (uint32_t)co * 4u : kOOB;
                    // (whole-vector casts: this compiler's __builtin_bit_cast of a single
                    // vector element reads element 0 whatever the index)
                    const f32x4 bv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rbias, (int)bo, 0, 0));
                    const f32x4 av = ACT == CONV2D_ACT_PRELU
                                         ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ralpha, (int)bo, 0, 0))
                                         : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bq[4 * q + e] = bv[e];
                        aq[4 * q + e] = av[e];
                    }
                }
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    u32x2 q2[2];
                    u32x2 rq[2] = {u32x2{rv[pp][0], rv[pp][1]}, u32x2{rv[pp][2], rv[pp][3]}};
                    if constexpr (RES != 0) swap_halves(rq[0], rq[1]);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int q = 2 * pp + h;
                        T rt[4], out[4];
                        __builtin_memcpy(rt, &rq[h], 8);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float v = acc[i][j][4 * q + e] + bq[4 * q + e];
                            if constexpr (RES == 1) v += to_f32(rt[e]);
                            if constexpr (ACT == CONV2D_ACT_RELU) v = v > 0.0f ? v : 0.0f;
                            if constexpr (ACT == CONV2D_ACT_SILU) v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
                            if constexpr (ACT == CONV2D_ACT_PRELU) v = v >= 0.0f ? v : aq[4 * q + e] * v;
                            if constexpr (RES == 2) v += to_f32(rt[e]);
                            out[e] = round_fp32<T>(v);
                        }
                        __builtin_memcpy(&q2[h], out, 8);
                    }
                    swap_halves(q2[0], q2[1]);
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4{q2[0][0], q2[0][1], q2[1][0], q2[1][1]}, ry,
                                                           (int)off[pp], 0, 0);
                }
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
}

namespace {

// The variants, indexed by HgemmPlan::cfg (from MI355X timings of the ResNet stage 2-4
// layers: variant 0 leads at 40x40x256, variant 1 at 20x20x512).
typedef HgCfg<10, 10, 4, 1, 1, 2, 32, 2> HgV0;  // 100 px x 32 ch, two workgroups per CU
typedef HgwCfg<10, 10, 1, 1, 1> HgV1;           // specialised waves: 100 px x 32 ch
typedef HgwCfg<10, 10, 1, 1, 2> HgV2;           // the same, taps split over two waves
typedef HgCfg<16, 16, 4, 1, 2, 2, 32, 2> HgV3;  // 256 px x 64 ch
typedef HgCfg<10, 20, 4, 1, 1, 2, 32, 2> HgV4;  // 200 px x 32 ch (7 pixel blocks, 2 per wave)
typedef HgCfg<10, 20, 4, 1, 2, 2, 32, 2> HgV5;  // 200 px x 64 ch
// stride 2
typedef HgCfg<10, 10, 4, 1, 2, 2, 32, 2, 2> HgV6;  // 100 px x 64 ch
typedef HgCfg<10, 10, 4, 1, 1, 2, 32, 2, 2> HgV7;  // 100 px x 32 ch
typedef HgCfg<8, 16, 4, 1, 2, 2, 32, 2, 2> HgV8;   // 128 px x 64 ch
// 255 px (17 x 15: 8 pixel blocks, one of them one pixel short) x 32 ch: a 68 x 120 map
// of 240 channels (the IFNet block) in exactly 256 workgroups
typedef HgCfg<17, 15, 8, 1, 1, 2, 32, 2> HgV9;   // eight waves, one pixel block each
typedef HgCfg<17, 15, 4, 1, 1, 2, 32, 2> HgV10;  // four waves, two pixel blocks each
typedef HgCfg<17, 15, 8, 1, 1, 3, 32, 2> HgV11;  // the same in a three-stage ring
// stride 2, 100 px x 32 ch in a three-stage ring (copies issued two chunks ahead of
// their use; one workgroup per CU): leads on the first stage-4 conv (40x40x256 -> 512)
typedef HgCfg<10, 10, 4, 1, 1, 3, 32, 2, 2> HgV12;
constexpr int kHgVariants = 13;

template <typename C> long long hg_tiles(const ConvArgs &a) {
    return (long long)a.N * ((a.OW + C::TW - 1) / C::TW) * ((a.OH + C::TH - 1) / C::TH) *
           ((a.Cout + C::CB - 1) / C::CB);
}

template <typename C> constexpr int hg_stride() {
    if constexpr (requires { C::S; })
        return C::S;
    else
        return 1;
}

template <typename T, typename C> hipError_t launch_hgw_c(const ConvArgs &a, bool cfast, bool nchw, hipStream_t st) {
    if (nchw || (a.Cin % C::CK) != 0 || a.stride != 1 || a.OH != a.H || a.OW != a.W) return hipErrorInvalidValue;
    const long long tiles = hg_tiles<C>(a);
    if (tiles <= 0 || tiles > 0x7fffffffll) return hipErrorInvalidValue;
    HgemmGeo g{};
    g.tiles_x = (a.OW + C::TW - 1) / C::TW;
    g.tiles_y = (a.OH + C::TH - 1) / C::TH;
    g.tiles_c = (a.Cout + C::CB - 1) / C::CB;
    g.ntiles_p = a.N * g.tiles_x * g.tiles_y;
    g.cfast = cfast ? 1 : 0;
    return launch_kernel(hgemmws3x3_kernel<T, C>, dim3((unsigned)tiles), dim3(64 * C::NWV), 0, st, a, g);
}

template <typename T, typename C> hipError_t launch_hg_c(const ConvArgs &a, bool cfast, bool nchw, hipStream_t st) {
    if ((a.Cin % (nchw ? 8 : C::CK)) != 0 || a.stride != C::S || a.OH != (a.H - 1) / C::S + 1 ||
        a.OW != (a.W - 1) / C::S + 1)
        return hipErrorInvalidValue;
    const long long tiles = hg_tiles<C>(a);
    if (tiles <= 0 || tiles > 0x7fffffffll) return hipErrorInvalidValue;
    HgemmGeo g{};
    g.tiles_x = (a.OW + C::TW - 1) / C::TW;
    g.tiles_y = (a.OH + C::TH - 1) / C::TH;
    g.tiles_c = (a.Cout + C::CB - 1) / C::CB;
    g.ntiles_p = a.N * g.tiles_x * g.tiles_y;
    g.cfast = cfast ? 1 : 0;
    if (nchw) return launch_kernel(hgemm3x3_kernel<T, C, true>, dim3((unsigned)tiles), dim3(64 * C::NW), 0, st, a, g);
    return launch_kernel(hgemm3x3_kernel<T, C, false>, dim3((unsigned)tiles), dim3(64 * C::NW), 0, st, a, g);
}

template <typename T> hipError_t launch_hg_d(const ConvArgs &a, const HgemmPlan &p, bool nchw, hipStream_t st) {
    switch (p.cfg) {
    case 0: return launch_hg_c<T, HgV0>(a, p.cfast, nchw, st);
    case 1: return launch_hgw_c<T, HgV1>(a, p.cfast, nchw, st);
    case 2: return launch_hgw_c<T, HgV2>(a, p.cfast, nchw, st);
    case 3: return launch_hg_c<T, HgV3>(a, p.cfast, nchw, st);
    case 4: return launch_hg_c<T, HgV4>(a, p.cfast, nchw, st);
    case 5: return launch_hg_c<T, HgV5>(a, p.cfast, nchw, st);
    case 6: return launch_hg_c<T, HgV6>(a, p.cfast, nchw, st);
    case 7: return launch_hg_c<T, HgV7>(a, p.cfast, nchw, st);
    case 8: return launch_hg_c<T, HgV8>(a, p.cfast, nchw, st);
    case 9: return launch_hg_c<T, HgV9>(a, p.cfast, nchw, st);
    case 10: return launch_hg_c<T, HgV10>(a, p.cfast, nchw, st);
    case 11: return launch_hg_c<T, HgV11>(a, p.cfast, nchw, st);
    case 12: return launch_hg_c<T, HgV12>(a, p.cfast, nchw, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int hgemm_cfg_count() { return kHgVariants; }

bool hgemm_cfg_info(int cfg, const ConvArgs &a, HgemmInfo *o) {
    auto fill = [&](auto c) {
        typedef decltype(c) C;
        o->ck = C::CK;
        o->th = C::TH;
        o->tw = C::TW;
        o->cb = C::CB;
        if constexpr (requires { C::NWV; }) {
            o->waves = C::NWV;
            o->ws = true;
        } else {
            o->waves = C::NW;
            o->ws = false;
        }
        o->lds = C::LDS;
        o->stride = hg_stride<C>();
        o->tiles = hg_tiles<C>(a);
        return true;
    };
    switch (cfg) {
    case 0: return fill(HgV0{});
    case 1: return fill(HgV1{});
    case 2: return fill(HgV2{});
    case 3: return fill(HgV3{});
    case 4: return fill(HgV4{});
    case 5: return fill(HgV5{});
    case 6: return fill(HgV6{});
    case 7: return fill(HgV7{});
    case 8: return fill(HgV8{});
    case 9: return fill(HgV9{});
    case 10: return fill(HgV10{});
    case 11: return fill(HgV11{});
    case 12: return fill(HgV12{});
    default: return false;
    }
}

hipError_t launch_hgemm3x3(const ConvArgs &a, int dtype, const HgemmPlan &p, bool nchw_out, hipStream_t st) {
    if (a.kh != 3 || a.kw != 3 || (a.stride != 1 && a.stride != 2) || a.pad != 1 || (a.Cout % 8) != 0 ||
        (!nchw_out && !a.vec_out) || (nchw_out && a.y2 && (reinterpret_cast<uintptr_t>(a.y2) & 15) != 0))
        return hipErrorInvalidValue;
    switch (dtype) {
    case CONV2D_DTYPE_BF16: return launch_hg_d<bf16>(a, p, nchw_out, st);
    case CONV2D_DTYPE_F16: return launch_hg_d<f16>(a, p, nchw_out, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace c2d
