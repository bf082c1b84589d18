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
//  * Weights stay in registers: one wave's 32*FN output channels over its share of the
//    9*Cin k are 9*Cin*FN/(16*WK) operand fragments of 4 VGPRs (72 per 32 channels at
//    Cin 32, or at Cin 64 with k split over a pair of waves). A workgroup copies the
//    weights into LDS once, in fragment order and in chunks the size of the halo
//    buffers, and every wave reads its fragments from there. With FN = 2 every pixel
//    operand read from LDS feeds two products.
//  * 4-wave workgroups run two to a CU: their tiles drift out of step, so one's
//    epilogue (vector-memory and VALU bound) overlaps the other's products.
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

// Workgroup barrier. s_barrier alone does not wait for the wave's own LDS writes
// (ds_write) to land, so lgkmcnt(0) comes first: the partial sums that a k-split
// pair exchanges and the pooled rows are complete for every wave that passes it.
// Direct-to-LDS loads are published by the explicit vmcnt waits instead.
__device__ __forceinline__ void halo_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace

// CIN input channels (16, 32 or 64); TH output rows per tile (tiles are TH x 32);
// FN 32-channel output blocks per wave (the workgroup covers 32*FN channels); WK
// waves along k (each takes CIN/WK of the input channels of every tap and the pair
// adds their sums through LDS); NW / WK waves along the tile rows.
//
// POOL: the 3x3 stride-2 pad-1 max pool of the output is written instead of the
// output (p.y, [N, PH, PW, Cout]); TH = 4, one tile row per wave, no k split, no
// residual. A tile is 4 conv rows 4ty.. by 32 conv columns 30tx - 1.. (columns
// overlap by two, so pooled column 15tx + c is centred on lane 2c + 1 of every row,
// c < 15) and gives pooled rows 2ty and 2ty + 1: rows 4ty-1..4ty+1 and 4ty+1..4ty+3.
// Each workgroup walks one run of tiles down the image (ty = seg*L .. seg*L + L - 1),
// carrying the activated, column-maxed last row of a tile in LDS into the next; a run
// that does not start at the top first computes the last row of the tile above
// (one wave's products). The max is taken on the rounded values, columns left to right
// within a row, then the rows top to bottom, each step keeping the running value unless
// the next is strictly greater: the taps in row-major order, as the pool kernel takes
// them, so the result equals pooling the stored conv output bit for bit (NaN included).
struct HaloPool {
    void *y;
    int PH, PW;
    int seg_len;  // tiles per run
    int segs;     // runs per column of tiles
};

template <typename T, int CIN, int TH, int FN, int WK, int NW, bool POOL>
__global__ __launch_bounds__(64 * NW, 8 / NW) void halo3x3_kernel(ConvArgs a, int tiles_w, int tiles_h, int ntiles,
                                                                  HaloPool pl) {
    constexpr int WM = NW / WK;
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
    constexpr int WUNITS = WK * KSW * FN;     // weights in operand order, 1 KiB units
    constexpr int RING = 2 * HBUF;            // two halo buffers; weights pass through in chunks
    constexpr int CUNITS = RING / 1024;       // units per chunk
    constexpr int NCH = (WUNITS + CUNITS - 1) / CUNITS;
    static_assert(CUNITS % NW == 0, "whole chunks per wave");
    constexpr int NDWW = CUNITS / NW;         // loads per lane per chunk
    constexpr int NG = 4 / WK;                // 4-channel groups of each block this wave stores
    constexpr int NP = NG / 2;                // pairs of them: one 16-byte store per lane
    constexpr int XBYTES = FM * FN * 2 * 1024;  // per wave: 8 floats per lane per block
    constexpr int XCH = WK == 2 ? NW * XBYTES : 16;
    static_assert(!POOL || (TH == 4 && FM == 1 && WK == 1), "pooled tiles: 4 rows, one per wave");
    // POOL: six rows of [64 lanes][FN * 32 values] in T: the tile's rows 0..2 and two
    // carry rows (the last row of the tile before and of this one), by tile parity
    constexpr int PROW = FN * 2 * 1024;
    constexpr int PROWB = POOL ? 6 * PROW : 0;
    // One array holds the two halo buffers and the pooled rows. When the weights fit in
    // it above halo buffer 0 (ONE_PASS), they are staged there in one go while the first
    // halo loads; otherwise they pass through the halo buffers in chunks first.
    constexpr int WTOP = RING + PROWB;
    constexpr int NDW1 = (WUNITS + NW - 1) / NW;     // weight loads per lane in one pass
    constexpr int WBASE = WTOP - NDW1 * NW * 1024;  // the one-pass weights (loads past WUNITS
                                                    // land at the top and are not read)
    constexpr bool ONE_PASS = WBASE >= HBUF;
    __shared__ __attribute__((aligned(1024))) char ring[WTOP];
    __shared__ __attribute__((aligned(1024))) char xch[XCH];
    __shared__ __attribute__((aligned(16))) float bal[2][32 * FN];  // bias, slopes (0 past Cout)
    char *const hb0 = ring;
    char *const hb1 = ring + HBUF;
    char *const prow = ring + RING;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM, wk = wave / WM;
    const int rl = lane & 31, hi = lane >> 5;
    const int H = a.H, W = a.W, Cout = a.Cout;
    typedef typename Mfma32<T>::vec vec;

    // Weights, once per workgroup: staged in LDS in operand order ([wk][k step][block j]
    // [lane] x 16 bytes: output channel 32*j + lane % 32, channels 8*(lane/32).. of the
    // wave's k step), then each wave takes its KSW*FN fragments into registers.
    // The weights are the A operand and the pixels the B operand, so the sums come
    // out with output channels along the rows: lane (rl, hi) holds channels
    // 32*j + 8*g + 4*hi + 0..3, g < 4, of pixel rl, and the epilogue stores 4-channel
    // runs straight from registers. The accumulators start from the bias; bias and
    // slopes sit in a small LDS table.
    const i32x4 rwt = rsrc_words(a.w, (uint32_t)((size_t)Cout * 9 * CIN * sizeof(T)));
    auto stage_chunk = [&](int c) {
#pragma unroll
        for (int d = 0; d < NDWW; ++d) {
            const int slot = d * NW + wave, u = c * CUNITS + slot;
            const int j = u % FN, sw = (u / FN) % KSW, wkk = u / (FN * KSW);
            const int co = j * 32 + rl, tap = sw / KCW, ci = (wkk * KCW + sw % KCW) * 16 + hi * 8;
            const bool ok = u < WUNITS && co < Cout;
            dma_b128(rwt, ok ? (uint32_t)((co * 9 + tap) * CIN + ci) * (uint32_t)sizeof(T) : kOOB,
                     lds_addr(ring + slot * 1024));
        }
    };
    // the wave stores channel groups g = g0 .. g0+NG-1 of each block (all four, or its
    // half for k-split pairs)
    const int g0 = WK == 2 ? 2 * wk : 0;
    if (threadIdx.x < 32 * FN) {
        const int co = threadIdx.x;
        bal[0][co] = a.bias && co < Cout ? a.bias[co] : 0.0f;
        bal[1][co] = a.alpha && co < Cout ? a.alpha[co] : 0.0f;
    }
    vec bw[KSW][FN];
    // all weights in one pass into [WBASE, WTOP)
    auto stage_all = [&]() {
#pragma unroll
        for (int d = 0; d < NDW1; ++d) {
            const int u = d * NW + wave;
            const int j = u % FN, sw = (u / FN) % KSW, wkk = u / (FN * KSW);
            const int co = j * 32 + rl, tap = sw / KCW, ci = (wkk * KCW + sw % KCW) * 16 + hi * 8;
            const bool ok = u < WUNITS && co < Cout;
            dma_b128(rwt, ok ? (uint32_t)((co * 9 + tap) * CIN + ci) * (uint32_t)sizeof(T) : kOOB,
                     lds_addr(ring + WBASE + u * 1024));
        }
    };
    auto take_weights = [&](const char *from, int c) {
#pragma unroll
        for (int sw = 0; sw < KSW; ++sw)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int u = (wk * KSW + sw) * FN + j - c * CUNITS;
                if (ONE_PASS || NCH == 1 || (u >= 0 && u < CUNITS))
                    bw[sw][j] = *reinterpret_cast<const vec *>(from + (u * 64 + lane) * 16);
            }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): fragments in registers before the space is reused
    };

    // Tile order: G workgroups, the ones on one XCD (blockIdx % 8) take a contiguous
    // run of each round's G tiles, so neighbouring tiles share halo rows in one L2.
    // POOL: workgroup = one run of tiles down one column of tiles.
    const int G = gridDim.x;
    const int r = (G % 8) == 0 ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
    struct Geo {
        int n, oy0, ox0;
        bool live;  // a tile of this workgroup
        bool pool;  // POOL: writes pooled rows (else only the carry row)
    };
    auto geo = [&](int k) -> Geo {
        if constexpr (!POOL) {
            const int t = k * G + r;
            const bool live = t < ntiles;
            const int tt = live ? t : 0;
            const int tx = tt % tiles_w, rr = tt / tiles_w;
            const int ty = rr % tiles_h, n = rr / tiles_h;
            return Geo{n, ty * TH, tx * TW, live, false};
        } else {
            const int seg = blockIdx.x % pl.segs, rest = blockIdx.x / pl.segs;
            const int tx = rest % tiles_w, n = rest / tiles_w;
            const int first = seg * pl.seg_len - (seg > 0 ? 1 : 0);
            const int end = (seg + 1) * pl.seg_len < tiles_h ? (seg + 1) * pl.seg_len : tiles_h;
            const int ty = first + k;
            const bool live = ty < end;
            return Geo{n, (live ? ty : first) * TH, tx * 30 - 1, live, !(seg > 0 && k == 0)};
        }
    };

    const i32x4 rx = rsrc_words(a.x, (uint32_t)((size_t)a.N * H * W * CIN * sizeof(T)));
    // Halo of the workgroup's tile k into buf; a k past its last tile issues the same
    // number of loads with out-of-range offsets (no traffic), so the vmcnt waits stay exact.
    auto issue = [&](char *buf, int k) {
        const Geo g = geo(k);
        const bool live = g.live;
        const int n = g.n, oy0 = g.oy0, ox0 = g.ox0;
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

    f32x16 acc[FM][FN];
    auto compute = [&](const char *buf) {
        // start from the bias (the first wave of a k-split pair), lane (rl, hi): channels
        // 32*j + 8*g + 4*hi + 0..3 in elements 4g..4g+3
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            f32x16 b0;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 bq = (WK == 1 || wk == 0) ? *reinterpret_cast<const f32x4 *>(&bal[0][j * 32 + 8 * g + 4 * hi])
                                                      : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int e = 0; e < 4; ++e) b0[4 * g + e] = bq[e];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) acc[i][j] = b0;
        }
        // B operand of tile row wm*FM+i at the wave's k step sw: pixel (row + ky, rl + kx)
        // of the halo, 16-channel chunk wk*KCW + sw % KCW, 8-channel half hi.
        const char *base = buf + ((wm * FM) * HW + rl) * PSTR + hi * 16 + wk * KCW * 32;
        auto read = [&](int sw, vec(&fa)[FM]) {
            const int tap = sw / KCW, ky = tap / 3, kx = tap % 3;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const vec *>(base + ((i + ky) * HW + kx) * PSTR + (sw % KCW) * 32);
        };
        // operand reads run PF k steps ahead of the products
        constexpr int PF = 2;
        vec fa[PF + 1][FM];
#pragma unroll
        for (int sw = 0; sw < PF && sw < KSW; ++sw) read(sw, fa[sw]);
#pragma unroll
        for (int sw = 0; sw < KSW; ++sw) {
            if (sw + PF < KSW) read(sw + PF, fa[(sw + PF) % (PF + 1)]);
            // keep the scheduler from sinking those reads below the products
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = Mfma32<T>::run(bw[sw][j], fa[sw % (PF + 1)][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Epilogue: block (i, j) is tile row wm*FM + i, channels 32*j..; lane (rl, hi)
    // holds pixel rl of the row, 4 channels 32*j + 8*g + 4*hi.. for each of its groups
    // g. After the math, one lane-half swap per pair of groups (2p, 2p+1) (lanes 32..63
    // of group 2p trade with lanes 0..31 of group 2p+1, v_permlane32_swap) leaves lane
    // (rl, hi) with 8 consecutive channels 32*j + 16*p + 8*hi.. of its pixel, stored in
    // one 16-byte access; the residual is loaded in that layout and swapped back. The
    // residual mode (none / added before / after the activation) and the activation
    // are template arguments of the store loop.
    const bool has_res = a.res != nullptr;
    const int res_mode = has_res ? (a.res_before_act ? 1 : 2) : 0;
    const uint32_t out_bytes = (uint32_t)((size_t)a.M * Cout * sizeof(T));
    const __amdgpu_buffer_rsrc_t rres = make_rsrc(a.res, has_res ? out_bytes : 0u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, out_bytes);
    const int p0 = g0 / 2;
    auto out_off = [&](const Geo &g, int i, int j, int pp) -> uint32_t {
        const int oy = g.oy0 + wm * FM + i, ox = g.ox0 + rl;
        const int co = j * 32 + 16 * (p0 + pp) + 8 * hi;
        return (g.live && oy < H && ox < W && co < Cout)
                   ? ((uint32_t)((g.n * H + oy) * W + ox) * (uint32_t)Cout + (uint32_t)co) * (uint32_t)sizeof(T)
                   : kOOB;
    };
    // lanes 32..63 of lo trade with lanes 0..31 of hi, for each of the two dwords
    auto swap_halves = [](u32x2 &lo, u32x2 &hi2) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const auto r2 = __builtin_amdgcn_permlane32_swap(lo[d], hi2[d], false, false);
            lo[d] = r2[0];
            hi2[d] = r2[1];
        }
    };

    // POOL epilogue of tile k: this wave's conv row, activated, -inf outside the conv
    // output, maxed with its left and right neighbour columns (lanes rl -/+ 1 of the
    // same half) and rounded, goes to LDS row wm (the last wave's to the carry row of
    // tile k + 1); then the even waves max the carry row of tile k with rows 0 and 1
    // into pooled row 2ty, the odd waves rows 1, 2 and the new carry into pooled row
    // 2ty + 1, each wave half of the channels.
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(pl.y, POOL ? (uint32_t)((size_t)a.N * pl.PH * pl.PW * Cout * sizeof(T)) : 0u);
    auto prow_at = [&](int row, int q) -> char * { return prow + row * PROW + (q * 64 + lane) * 16; };
    // ReLU: every activated value is +0 or positive and never NaN (x > 0 ? x : 0), so
    // the first largest of a window equals the plain maximum and the bit patterns of
    // these T values order like 16-bit unsigned integers: two channels at a time with
    // v_pk_max_u16, and 0 in place of -inf outside the conv output (every pooled window
    // holds a valid value, which is at least +0). The same bits as the general path.
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    auto pmax = [](uint32_t x, uint32_t y) {
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, x),
                                                                      __builtin_bit_cast(u16x2, y)));
    };
    typedef T t2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    auto pool_rows_relu = [&](const Geo &tg, int k) {
        const int oy = tg.oy0 + wm, ox = tg.ox0 + rl;
        const bool valid = (unsigned)oy < (unsigned)H && (unsigned)ox < (unsigned)W;
        // ReLU and the conv-output mask in one compare: x > thr ? x : 0
        const float thr = valid ? 0.0f : __builtin_inff();
        const int row = wm == WM - 1 ? 4 + ((k + 1) & 1) : wm;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            uint32_t pk[8];
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                const float x0 = acc[0][j][2 * e2], x1 = acc[0][j][2 * e2 + 1];
                // one rounding of each fp32 value to T (a pair conversion, round to nearest even)
                const t2 t = __builtin_convertvector(f32x2{x0 > thr ? x0 : 0.0f, x1 > thr ? x1 : 0.0f}, t2);
                const uint32_t c = __builtin_bit_cast(uint32_t, t);
                // neighbour columns by whole-wave DPP shifts (lanes 0 and 63, never the centre
                // of a pooled column, read 0)
                const uint32_t l = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, 0x138, 0xf, 0xf, true);
                const uint32_t r = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, 0x130, 0xf, 0xf, true);
                pk[e2] = pmax(pmax(l, c), r);
            }
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
                *reinterpret_cast<u32x4 *>(prow_at(row, j * 2 + pp)) =
                    u32x4{pk[4 * pp], pk[4 * pp + 1], pk[4 * pp + 2], pk[4 * pp + 3]};
        }
        halo_barrier();
        if (!tg.pool) return;
        const int odd = wave & 1, qh = wave >> 1;
        const int r0 = odd ? 1 : 4 + (k & 1), r1 = odd ? 2 : 0, r2 = odd ? 4 + ((k + 1) & 1) : 1;
        const int py = tg.oy0 / 2 + odd, px = (tg.ox0 + 1) / 2 + (rl - 1) / 2;
        const bool store = (rl & 1) && rl < 30 && px < pl.PW && py < pl.PH;
#pragma unroll
        for (int qq = 0; qq < FN; ++qq) {
            const int q = qh * FN + qq, j = q >> 1, pp = q & 1;
            const u32x4 v0 = *reinterpret_cast<const u32x4 *>(prow_at(r0, q));
            const u32x4 v1 = *reinterpret_cast<const u32x4 *>(prow_at(r1, q));
            const u32x4 v2 = *reinterpret_cast<const u32x4 *>(prow_at(r2, q));
            u32x2 qq2[2] = {u32x2{pmax(pmax(v0[0], v1[0]), v2[0]), pmax(pmax(v0[1], v1[1]), v2[1])},
                            u32x2{pmax(pmax(v0[2], v1[2]), v2[2]), pmax(pmax(v0[3], v1[3]), v2[3])}};
            swap_halves(qq2[0], qq2[1]);
            const int co = j * 32 + 16 * pp + 8 * hi;
            const uint32_t off = (store && co < Cout)
                                     ? ((uint32_t)((tg.n * pl.PH + py) * pl.PW + px) * (uint32_t)Cout +
                                        (uint32_t)co) * (uint32_t)sizeof(T)
                                     : kOOB;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{qq2[0][0], qq2[0][1], qq2[1][0], qq2[1][1]}, rp, (int)off,
                                                   0, 0);
        }
    };
    auto pool_rows = [&](const Geo &tg, int k) {
        const int oy = tg.oy0 + wm, ox = tg.ox0 + rl;
        const bool valid = (unsigned)oy < (unsigned)H && (unsigned)ox < (unsigned)W;
        auto act_all = [&](auto act_tag) {
            constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float x = acc[0][j][e];
                    if constexpr (ACT == CONV2D_ACT_RELU) x = x > 0.0f ? x : 0.0f;
                    if constexpr (ACT == CONV2D_ACT_SILU) x = x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
                    if constexpr (ACT == CONV2D_ACT_PRELU) {
                        const float al = bal[1][j * 32 + 8 * (e / 4) + 4 * hi + (e % 4)];
                        x = x >= 0.0f ? x : al * x;
                    }
                    acc[0][j][e] = valid ? x : -__builtin_inff();
                }
        };
        switch (a.act) {
        case CONV2D_ACT_RELU: act_all(std::integral_constant<int, CONV2D_ACT_RELU>{}); break;
        case CONV2D_ACT_SILU: act_all(std::integral_constant<int, CONV2D_ACT_SILU>{}); break;
        case CONV2D_ACT_PRELU: act_all(std::integral_constant<int, CONV2D_ACT_PRELU>{}); break;
        default: act_all(std::integral_constant<int, CONV2D_ACT_NONE>{}); break;
        }
        const int row = wm == WM - 1 ? 4 + ((k + 1) & 1) : wm;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            T q[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                // rounded first, as the pool of the stored conv output sees it; then the
                // first largest of (left, centre, right) from -inf, as `v > best` over the
                // taps in row-major order (NaN never wins; of equal zeros the first stays).
                // Through a scalar: this compiler lowers a bit cast applied directly to a
                // vector element as a read of element 0.
                // The neighbours come from whole-wave DPP shifts (lane i reads lane i-1, resp.
                // i+1; lanes 0 and 63 keep their own value), VALU moves with no LDS round trip.
                const float c = to_f32(round_fp32<T>(acc[0][j][e]));
                const int v = __builtin_bit_cast(int, c);
                const float l = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(v, v, 0x138, 0xf, 0xf, false));
                const float rgt = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(v, v, 0x130, 0xf, 0xf, false));
                q[e] = from_f32<T>(first_max3(l, c, rgt));
            }
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                u32x4 w4;
                __builtin_memcpy(&w4, &q[8 * pp], 16);
                *reinterpret_cast<u32x4 *>(prow_at(row, j * 2 + pp)) = w4;
            }
        }
        halo_barrier();
        if (!tg.pool) return;
        // pooled row 2ty + (wave & 1): carry-in, rows 0, 1 (even) or rows 1, 2, carry-out
        // (odd); the wave takes half of its 2*FN 8-channel quads
        const int odd = wave & 1, qh = wave >> 1;
        const int r0 = odd ? 1 : 4 + (k & 1), r1 = odd ? 2 : 0, r2 = odd ? 4 + ((k + 1) & 1) : 1;
        const int py = tg.oy0 / 2 + odd, px = (tg.ox0 + 1) / 2 + (rl - 1) / 2;
        const bool store = (rl & 1) && rl < 30 && px < pl.PW && py < pl.PH;
#pragma unroll
        for (int qq = 0; qq < FN; ++qq) {
            const int q = qh * FN + qq, j = q >> 1, pp = q & 1;
            const u32x4 v0 = *reinterpret_cast<const u32x4 *>(prow_at(r0, q));
            const u32x4 v1 = *reinterpret_cast<const u32x4 *>(prow_at(r1, q));
            const u32x4 v2 = *reinterpret_cast<const u32x4 *>(prow_at(r2, q));
            T t0[8], t1[8], t2[8], m[8];
            __builtin_memcpy(t0, &v0, 16);
            __builtin_memcpy(t1, &v1, 16);
            __builtin_memcpy(t2, &v2, 16);
            // The rows top to bottom, first largest as above. Compared in fp32 behind an
            // empty asm: left to itself, this compiler turned an f16 max of this shape into
            // v_max3_f16 and then packed two results with a plain OR, as if the instruction
            // cleared the upper 16 bits of its destination, which it does not.
            auto wide = [](T v) {
                float f = to_f32(v);
                asm volatile("" : "+v"(f));
                return f;
            };
#pragma unroll
            for (int e = 0; e < 8; ++e) m[e] = from_f32<T>(first_max3(wide(t0[e]), wide(t1[e]), wide(t2[e])));
            // groups 2pp, 2pp+1 (4 channels each) -> 8 consecutive channels per lane half
            u32x2 qq2[2];
            __builtin_memcpy(&qq2[0], &m[0], 8);
            __builtin_memcpy(&qq2[1], &m[4], 8);
            swap_halves(qq2[0], qq2[1]);
            const int co = j * 32 + 16 * pp + 8 * hi;
            const uint32_t off = (store && co < Cout)
                                     ? ((uint32_t)((tg.n * pl.PH + py) * pl.PW + px) * (uint32_t)Cout +
                                        (uint32_t)co) * (uint32_t)sizeof(T)
                                     : kOOB;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{qq2[0][0], qq2[0][1], qq2[1][0], qq2[1][1]}, rp, (int)off,
                                                   0, 0);
        }
    };

    float *mine = reinterpret_cast<float *>(xch + wave * XBYTES);
    const float *theirs = reinterpret_cast<const float *>(xch + (WK == 2 ? (wave + (wk ? -WM : WM)) : wave) * XBYTES);

    // One tile. Its halo has landed for this wave (the wait in the previous tile's
    // epilogue, or the prologue's): barrier (so it has for every wave), residual loads,
    // products, [hand the partner the channel groups it stores,] barrier (every wave
    // is done reading buf), [add the partner's sums,] wait for all of this wave's
    // loads (the residual, and the halo of tile k+1, which has had this tile's
    // products to arrive), refill buf with tile k+2, epilogue and stores.
    auto tile = [&](char *buf, int k) {
        const Geo tg = geo(k);
        halo_barrier();
        uint32_t off[FM][FN][NP];
        u32x4 rv[FM][FN][NP];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) {
                    off[i][j][pp] = out_off(tg, i, j, pp);
                    rv[i][j][pp] = (!POOL && has_res) ? __builtin_amdgcn_raw_buffer_load_b128(rres, (int)off[i][j][pp], 0, 0)
                                                      : u32x4{0u, 0u, 0u, 0u};
                }
        // a carry-only tile needs the last row alone
        if (!POOL || tg.pool || wm == WM - 1) compute(buf);
        if constexpr (WK == 2) {
            const int hs = 1 - wk;  // the channel groups (2hs, 2hs+1) the partner stores
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        *reinterpret_cast<f32x4 *>(mine + (((i * FN + j) * 2 + u) * 64 + lane) * 4) =
                            f32x4{acc[i][j][8 * hs + 4 * u], acc[i][j][8 * hs + 4 * u + 1],
                                  acc[i][j][8 * hs + 4 * u + 2], acc[i][j][8 * hs + 4 * u + 3]};
        }
        halo_barrier();
        if constexpr (WK == 2) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const f32x4 o =
                            *reinterpret_cast<const f32x4 *>(theirs + (((i * FN + j) * 2 + u) * 64 + lane) * 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[i][j][8 * wk + 4 * u + e] += o[e];
                    }
        }
        halo_wait_vmcnt<0>();
        issue(buf, k + 2);
        if constexpr (POOL) {
            if (a.act == CONV2D_ACT_RELU)
                pool_rows_relu(tg, k);
            else
                pool_rows(tg, k);
            return;
        }
        auto finish = [&](auto act_tag, auto res_tag) {
            constexpr int ACT = decltype(act_tag)::value;
            constexpr int RES = decltype(res_tag)::value;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int pp = 0; pp < NP; ++pp) {
                        u32x2 q[2];  // the pair's two groups, 4 channels each, packed
                        u32x2 rq[2] = {u32x2{rv[i][j][pp][0], rv[i][j][pp][1]}, u32x2{rv[i][j][pp][2], rv[i][j][pp][3]}};
                        if constexpr (RES != 0) swap_halves(rq[0], rq[1]);
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int g = 2 * pp + h;  // group within the wave's share
                            T rt[4], out[4];
                            __builtin_memcpy(rt, &rq[h], 8);
                            f32x4 al{0.0f, 0.0f, 0.0f, 0.0f};
                            if constexpr (ACT == CONV2D_ACT_PRELU)
                                al = *reinterpret_cast<const f32x4 *>(&bal[1][j * 32 + 8 * (g0 + g) + 4 * hi]);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float x = acc[i][j][4 * (g0 + g) + e];
                                if constexpr (RES == 1) x += to_f32(rt[e]);
                                if constexpr (ACT == CONV2D_ACT_RELU) x = x > 0.0f ? x : 0.0f;
                                if constexpr (ACT == CONV2D_ACT_SILU) x = x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
                                if constexpr (ACT == CONV2D_ACT_PRELU) x = x >= 0.0f ? x : al[e] * x;
                                if constexpr (RES == 2) x += to_f32(rt[e]);
                                out[e] = round_fp32<T>(x);
                            }
                            __builtin_memcpy(&q[h], out, 8);
                        }
                        swap_halves(q[0], q[1]);
                        __builtin_amdgcn_raw_buffer_store_b128(u32x4{q[0][0], q[0][1], q[1][0], q[1][1]}, ry,
                                                               (int)off[i][j][pp], 0, 0);
                    }
        };
        auto with_res = [&](auto act_tag) {
            switch (res_mode) {
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
    if constexpr (ONE_PASS) {
        // the first halo beside the weights; the weights land (barrier), go into
        // registers (barrier); then the second halo
        issue(hb0, 0);
        stage_all();
        halo_wait_vmcnt<0>();
        halo_barrier();
        take_weights(ring + WBASE, 0);
        halo_barrier();
    } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            stage_chunk(c);
            halo_wait_vmcnt<0>();
            halo_barrier();
            take_weights(ring, c);
            halo_barrier();
        }
    }
    if constexpr (POOL) {
        // the carry into a run's first tile: the row above the image, a value no pooled
        // value loses to: -inf, or +0 for the ReLU path (its 16-bit integer order puts
        // -inf above every positive value)
        if (wm == 0) {
            const float none = a.act == CONV2D_ACT_RELU ? 0.0f : -__builtin_inff();
            T ninf[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ninf[e] = from_f32<T>(none);
            u32x4 w4;
            __builtin_memcpy(&w4, ninf, 16);
#pragma unroll
            for (int q = 0; q < 2 * FN; ++q) *reinterpret_cast<u32x4 *>(prow_at(4, q)) = w4;
        }
    }
    if constexpr (!ONE_PASS) issue(hb0, 0);
    issue(hb1, 1);
    if constexpr (!ONE_PASS) halo_wait_vmcnt<0>();
    for (int k = 0; geo(k).live; k += 2) {
        tile(hb0, k);
        if (!geo(k + 1).live) break;
        tile(hb1, k + 1);
    }
    halo_wait_vmcnt<0>();
}

template <typename T, int CIN, int TH, int FN, int NW>
static hipError_t launch_halo_t(const ConvArgs &a, int grid_cap, hipStream_t st) {
    const int tiles_w = (a.W + 31) / 32, tiles_h = (a.H + TH - 1) / TH;
    const long long nt = (long long)a.N * tiles_w * tiles_h;
    if (nt > 0x7fffffffll) return hipErrorInvalidValue;
    const int ntiles = (int)nt;
    int grid = ntiles < grid_cap ? ntiles : grid_cap;
    if (grid > 8) grid -= grid % 8;
    constexpr int WK = CIN == 64 ? 2 : 1;
    return launch_kernel(halo3x3_kernel<T, CIN, TH, FN, WK, NW, false>, dim3(grid), dim3(64 * NW), 0, st, a,
                         tiles_w, tiles_h, ntiles, HaloPool{});
}

// Pooled variant: runs of seg_len tiles, about two workgroups per CU (grid_cap slots).
template <typename T, int CIN, int FN>
static hipError_t launch_halo_pool_t(const ConvArgs &a, void *y, int grid_cap, hipStream_t st) {
    HaloPool pl{};
    pl.y = y;
    pl.PH = (a.OH - 1) / 2 + 1;
    pl.PW = (a.OW - 1) / 2 + 1;
    const int tiles_w = (pl.PW + 14) / 15, tiles_h = (pl.PH + 1) / 2;
    const long long cols = (long long)a.N * tiles_w;
    // as many runs as fit the slots (a run that starts below the top adds one carry row)
    const long long runs_per_col = cols >= grid_cap ? 1 : grid_cap / cols;
    long long len = (tiles_h + runs_per_col - 1) / runs_per_col;
    if (len < 2) len = 2;
    if (len > tiles_h) len = tiles_h;
    pl.seg_len = (int)len;
    pl.segs = (int)((tiles_h + len - 1) / len);
    const long long grid = cols * pl.segs;
    if (grid > 0x7fffffffll || (long long)a.N * a.H * a.W * CIN >= (1ll << 30)) return hipErrorInvalidValue;
    return launch_kernel(halo3x3_kernel<T, CIN, 4, FN, 1, 4, true>, dim3((unsigned)grid), dim3(256), 0, st, a,
                         tiles_w, tiles_h, 0, pl);
}

// Tile heights per (Cin, output blocks per wave, waves): 64-channel layers split k
// over wave pairs, which leaves NW/2 waves along the tile rows (NW otherwise); two
// 32-channel output blocks per wave only with one tile row per wave (registers).
// 4-wave workgroups run two to a CU (p.grid_cap counts workgroups).
template <typename T, int CIN, int NW>
static hipError_t launch_halo_w(const ConvArgs &a, const HaloPlan &p, hipStream_t st) {
    constexpr int WM = CIN == 64 ? NW / 2 : NW;
    if (p.fn == 1 && p.th == WM) return launch_halo_t<T, CIN, WM, 1, NW>(a, p.grid_cap, st);
    if (p.fn == 1 && p.th == 2 * WM) return launch_halo_t<T, CIN, 2 * WM, 1, NW>(a, p.grid_cap, st);
    if (p.fn == 2 && p.th == WM) return launch_halo_t<T, CIN, WM, 2, NW>(a, p.grid_cap, st);
    return hipErrorInvalidValue;
}

template <typename T, int CIN>
static hipError_t launch_halo_c(const ConvArgs &a, const HaloPlan &p, hipStream_t st) {
    if (p.waves == 8) return launch_halo_w<T, CIN, 8>(a, p, st);
    if (p.waves == 4) return launch_halo_w<T, CIN, 4>(a, p, st);
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

template <typename T>
static hipError_t launch_halo_pool_d(const ConvArgs &a, void *y, int grid_cap, hipStream_t st) {
    const bool fn1 = a.Cout <= 32;
    switch (a.Cin) {
    case 16: return fn1 ? launch_halo_pool_t<T, 16, 1>(a, y, grid_cap, st) : launch_halo_pool_t<T, 16, 2>(a, y, grid_cap, st);
    case 32: return fn1 ? launch_halo_pool_t<T, 32, 1>(a, y, grid_cap, st) : launch_halo_pool_t<T, 32, 2>(a, y, grid_cap, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_halo3x3_maxpool(const ConvArgs &a, void *y, int dtype, int grid_cap, hipStream_t st) {
    if (a.res) return hipErrorInvalidValue;
    switch (dtype) {
    case CONV2D_DTYPE_BF16: return launch_halo_pool_d<bf16>(a, y, grid_cap, st);
    case CONV2D_DTYPE_F16: return launch_halo_pool_d<f16>(a, y, grid_cap, st);
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
