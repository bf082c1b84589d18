// 3x3 convolution of a 3-channel channel-last 16-bit image (the stem conv of the
// inferencelayer page's `encoder_maps`: stride 2, pad 1) on CDNA4 matrix cores.
//
// K = 27 is too thin for a tiled GEMM, and on the vector ALUs the 27 x Cout fp32
// multiply-adds per pixel would cost more than moving the image and the feature map.
// Here one 32x32x16 product pair covers 32 pixels x 32 output channels:
//
//  * K is laid out as the three 9-value image rows of the 3x3x3 patch (ky, then kx
//    and channel, which is how both the image row and the OHWI weight row are stored):
//    step 0 takes values 0..7 of patch row 0 (lanes 0-31) and of row 1 (lanes 32-63),
//    step 1 values 0..7 of row 2 and, in lanes 32-63, the three leftover values 8 of
//    rows 0-2 and five zeros. Weights are the A operand (built once per lane in that
//    order), pixels the B operand.
//  * A workgroup stages the input rows that its output rows need, whole, in LDS
//    (16-byte loads, zero rows for padding, a zero pixel in front for the left pad).
//    A lane's 8 consecutive values start 2-byte aligned, so it reads 5 dwords of the
//    row and shifts them together in pairs (v_alignbit).
//  * The epilogue is the channel-last one of the halo kernel: the accumulators start
//    from the bias, channel groups are paired by a lane-half swap and stored as
//    8-channel 16-byte runs.
#include "igemm_common.hpp"
#include "kernels.hpp"

namespace c2d {

// B operands of one 32-pixel block from three staged input rows (row0, row0 + rstr,
// row0 + 2*rstr), the patch row starting at byte base + sh/8 of each. Lanes 0-31 take
// values 0..7 of rows 0 and 2; lanes 32-63 values 0..7 of row 1 and values 8 of rows
// 0-2. Each lane reads only the dwords it uses (five for its first operand; five of row
// 2, or the one dword holding value 8 of each row, for its second).
template <typename V>
__device__ __forceinline__ void stem_operands(const char *row0, int rstr, int base, int sh, int hi, V (&xb)[2]) {
    const uint32_t *s0 = reinterpret_cast<const uint32_t *>(row0 + hi * rstr + base);
    uint32_t d[5], e[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) d[i] = s0[i];
    // second operand: lanes 0-31 dwords 0..4 of row 2; lanes 32-63 dword 4 of rows 0, 1, 2
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int off = hi ? (i < 3 ? i : 2) * rstr + 16 : 2 * rstr + 4 * i;
        e[i] = *reinterpret_cast<const uint32_t *>(row0 + base + off);
    }
    uint32_t b0[4], b1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b0[i] = __builtin_amdgcn_alignbit(d[i + 1], d[i], sh);
        b1[i] = __builtin_amdgcn_alignbit(e[i + 1], e[i], sh);
    }
    const uint32_t v8_0 = (e[0] >> sh) & 0xffffu, v8_1 = (e[1] >> sh) & 0xffffu, v8_2 = (e[2] >> sh) & 0xffffu;
    b1[0] = hi ? (v8_0 | (v8_1 << 16)) : b1[0];
    b1[1] = hi ? v8_2 : b1[1];
    b1[2] = hi ? 0u : b1[2];
    b1[3] = hi ? 0u : b1[3];
    __builtin_memcpy(&xb[0], b0, 16);
    __builtin_memcpy(&xb[1], b1, 16);
}

// FN 32-channel output blocks (Cout <= 32*FN); RB output rows per workgroup; S stride.
template <typename T, int FN, int RB, int S>
__global__ __launch_bounds__(256) void stem3_kernel(ConvArgs a, int rstr) {
    constexpr int NW = 4;
    constexpr int RS = (RB - 1) * S + 3;  // input rows staged
    extern __shared__ __attribute__((aligned(16))) char srow[];  // [RS][rstr] bytes
    __shared__ __attribute__((aligned(16))) float bal[2][32 * FN];
    typedef typename Mfma32<T>::vec vec;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rl = lane & 31, hi = lane >> 5;
    const int H = a.H, W = a.W, OH = a.OH, OW = a.OW, Cout = a.Cout;
    const int rows_per_img = (OH + RB - 1) / RB;
    const int n = blockIdx.x / rows_per_img;
    const int oy0 = (blockIdx.x - n * rows_per_img) * RB;

    // Weights as the A operand: lane (co = 32j + rl, hi), step 0: values 0..7 of patch
    // row hi; step 1: values 0..7 of row 2 (hi = 0) or value 8 of rows 0, 1, 2 (hi = 1).
    vec wa[2][FN];
    {
        const T *w = static_cast<const T *>(a.w);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int co = j * 32 + rl;
            T v0[8], v1[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v0[e] = co < Cout ? w[co * 27 + hi * 9 + e] : from_f32<T>(0.0f);
                const int k1 = hi == 0 ? 18 + e : (e < 3 ? e * 9 + 8 : -1);
                v1[e] = (co < Cout && k1 >= 0) ? w[co * 27 + k1] : from_f32<T>(0.0f);
            }
            __builtin_memcpy(&wa[0][j], v0, 16);
            __builtin_memcpy(&wa[1][j], v1, 16);
        }
    }
    if (threadIdx.x < 32 * FN) {
        const int co = threadIdx.x;
        bal[0][co] = a.bias && co < Cout ? a.bias[co] : 0.0f;
        bal[1][co] = a.alpha && co < Cout ? a.alpha[co] : 0.0f;
    }

    // Stage input rows iy = oy0*S - 1 + r, r < RS: LDS row r = [16 zero bytes][W x 6
    // bytes][zeros up to rstr]; the pixel at column ix starts at byte 16 + 6*ix.
    // Eight loads per thread go out before their LDS writes (unconditional, with an
    // out-of-range offset for padding), so a workgroup waits for one load latency per
    // round instead of one per load.
    {
        const int row_bytes = W * 6;
        const int chunks = rstr / 16, total = RS * chunks;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)((size_t)a.N * H * row_bytes));
        for (int i0 = threadIdx.x; i0 < total; i0 += 8 * 256) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + 256 * u, r = i / chunks, c = i - r * chunks;
                const int iy = oy0 * S - 1 + r;
                const int b = c * 16 - 16;  // byte within the image row
                const bool ok = i < total && b >= 0 && b < row_bytes && (unsigned)iy < (unsigned)H;
                v[u] = __builtin_amdgcn_raw_buffer_load_b128(
                    rx, ok ? (int)((size_t)(n * H + iy) * row_bytes + b) : (int)kOOB, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + 256 * u, r = i / chunks, c = i - r * chunks;
                if (i < total) *reinterpret_cast<u32x4 *>(srow + r * rstr + c * 16) = v[u];
            }
        }
    }
    __syncthreads();

    const uint32_t out_bytes = (uint32_t)((size_t)a.M * Cout * sizeof(T));
    const bool has_res = a.res != nullptr;
    const int res_mode = has_res ? (a.res_before_act ? 1 : 2) : 0;
    const __amdgpu_buffer_rsrc_t rres = make_rsrc(a.res, has_res ? out_bytes : 0u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, out_bytes);
    auto swap_halves = [](u32x2 &lo, u32x2 &hi2) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const auto r2 = __builtin_amdgcn_permlane32_swap(lo[d], hi2[d], false, false);
            lo[d] = r2[0];
            hi2[d] = r2[1];
        }
    };

    const int tasks_w = (OW + 31) / 32;
    for (int task = wave; task < RB * tasks_w; task += NW) {
        const int rr = task / tasks_w, ox0 = (task - rr * tasks_w) * 32;
        const int oy = oy0 + rr, ox = ox0 + rl;
        if (oy >= OH) break;
        // The 9 values of patch row ky sit at bytes 16 + 6*(ox*S - 1) .. +18 of staged row
        // rr*S + ky; read the 5 dwords from the one below that offset and shift. Lanes
        // past the row end read the last pixel's patch (their outputs are not stored).
        const int byte = 16 + 6 * ((ox < OW ? ox : OW - 1) * S - 1);
        const int base = byte & ~3, sh = (byte & 3) * 8;
        vec xb[2];
        stem_operands(srow + rr * S * rstr, rstr, base, sh, hi, xb);
        f32x16 acc[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 bq = *reinterpret_cast<const f32x4 *>(&bal[0][j * 32 + 8 * g + 4 * hi]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[j][4 * g + e] = bq[e];
            }
            acc[j] = Mfma32<T>::run(wa[0][j], xb[0], acc[j]);
            acc[j] = Mfma32<T>::run(wa[1][j], xb[1], acc[j]);
        }
        // Epilogue: lane (rl, hi) holds channels 32j + 8g + 4hi.. of pixel ox; pairs of
        // groups become 8-channel runs 32j + 16p + 8hi.. after the lane-half swap.
        const bool live = oy < OH && ox < OW;
        uint32_t off[FN][2];
        u32x4 rv[FN][2];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int co = j * 32 + 16 * pp + 8 * hi;
                off[j][pp] = (live && co < Cout)
                                 ? ((uint32_t)((n * OH + oy) * OW + ox) * (uint32_t)Cout + (uint32_t)co) *
                                       (uint32_t)sizeof(T)
                                 : kOOB;
                rv[j][pp] = has_res ? __builtin_amdgcn_raw_buffer_load_b128(rres, (int)off[j][pp], 0, 0)
                                    : u32x4{0u, 0u, 0u, 0u};
            }
        auto finish = [&](auto act_tag, auto res_tag) {
            constexpr int ACT = decltype(act_tag)::value;
            constexpr int RES = decltype(res_tag)::value;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    u32x2 q[2];
                    u32x2 rq[2] = {u32x2{rv[j][pp][0], rv[j][pp][1]}, u32x2{rv[j][pp][2], rv[j][pp][3]}};
                    if constexpr (RES != 0) swap_halves(rq[0], rq[1]);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int g = 2 * pp + h;
                        T rt[4], out[4];
                        __builtin_memcpy(rt, &rq[h], 8);
                        f32x4 al{0.0f, 0.0f, 0.0f, 0.0f};
                        if constexpr (ACT == CONV2D_ACT_PRELU)
                            al = *reinterpret_cast<const f32x4 *>(&bal[1][j * 32 + 8 * g + 4 * hi]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float x = acc[j][4 * g + e];
                            if constexpr (RES == 1) x += to_f32(rt[e]);
                            if constexpr (ACT == CONV2D_ACT_RELU) x = __builtin_fmaxf(x, 0.0f);
                            if constexpr (ACT == CONV2D_ACT_SILU) x = x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
                            if constexpr (ACT == CONV2D_ACT_PRELU) x = x >= 0.0f ? x : al[e] * x;
                            if constexpr (RES == 2) x += to_f32(rt[e]);
                            out[e] = round_fp32<T>(x);
                        }
                        __builtin_memcpy(&q[h], out, 8);
                    }
                    swap_halves(q[0], q[1]);
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4{q[0][0], q[0][1], q[1][0], q[1][1]}, ry,
                                                           (int)off[j][pp], 0, 0);
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
    }
}

// The same convolution followed by a 3x3 stride-2 pad-1 max pool, written as one
// kernel that stores only the pooled map (the stem conv + max-pool step of the
// inferencelayer page's `encoder_maps`). Workgroup: one pooled row py of one image
// and 4 column groups (one per wave). A group covers 32 conv columns c0 = 30g - 1 ..
// c0 + 31 of the three conv rows 2py-1 .. 2py+1 (six products per 32 channels); lane
// rl = 2k+1 (k < 15) is the centre of pooled column 15g + k, so every pool window lies
// inside one group (groups overlap by two columns). Each conv row is activated and
// rounded to T; its columns rl-1, rl, rl+1 (DPP wave shifts) are maxed left to right, then
// the rows top to bottom, each step keeping the running value unless the next is
// strictly greater: the taps in row-major order with the pool kernel's comparison, so
// the result equals pooling the stored conv output bit for bit (NaN skipped, an all-NaN
// window -inf, the first of equal zeros kept). Taps outside the conv map count as -inf.
template <typename T, int FN, int S>
__global__ __launch_bounds__(256) void stem3_pool_kernel(ConvArgs a, int PH, int PW, int groups, int rstr,
                                                         int ixs_step) {
    constexpr int NW = 4;
    constexpr int RS = 2 * S + 3;  // input rows staged
    extern __shared__ __attribute__((aligned(16))) char srow[];  // [RS][rstr] bytes
    __shared__ __attribute__((aligned(16))) float bal[2][32 * FN];
    typedef typename Mfma32<T>::vec vec;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rl = lane & 31, hi = lane >> 5;
    const int H = a.H, W = a.W, OH = a.OH, OW = a.OW, Cout = a.Cout;
    const int segs = (groups + NW - 1) / NW;
    const int seg = blockIdx.x % segs, py = (blockIdx.x / segs) % PH, n = blockIdx.x / (segs * PH);
    const int g = seg * NW + wave;

    vec wa[2][FN];
    {
        const T *w = static_cast<const T *>(a.w);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int co = j * 32 + rl;
            T v0[8], v1[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v0[e] = co < Cout ? w[co * 27 + hi * 9 + e] : from_f32<T>(0.0f);
                const int k1 = hi == 0 ? 18 + e : (e < 3 ? e * 9 + 8 : -1);
                v1[e] = (co < Cout && k1 >= 0) ? w[co * 27 + k1] : from_f32<T>(0.0f);
            }
            __builtin_memcpy(&wa[0][j], v0, 16);
            __builtin_memcpy(&wa[1][j], v1, 16);
        }
    }
    if (threadIdx.x < 32 * FN) {
        const int co = threadIdx.x;
        bal[0][co] = a.bias && co < Cout ? a.bias[co] : 0.0f;
        bal[1][co] = a.alpha && co < Cout ? a.alpha[co] : 0.0f;
    }

    // Stage input rows iy = (2py-1)*S - 1 + r, r < RS, from column ixs = 120*S*seg - 8 on
    // (a multiple of 8 pixels, so the copy moves aligned 16-byte chunks; 8 columns before
    // the segment's first patch column): column ix sits at byte 6*(ix - ixs) of LDS row r,
    // and columns outside the image (padding) read as zero.
    const int ixs = seg * ixs_step - 8;
    {
        const int row_bytes = W * 6;
        const int chunks = rstr / 16, total = RS * chunks;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)((size_t)a.N * H * row_bytes));
        for (int i0 = threadIdx.x; i0 < total; i0 += 8 * 256) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + 256 * u, r = i / chunks, c = i - r * chunks;
                const int iy = (2 * py - 1) * S - 1 + r;
                const int b = ixs * 6 + c * 16;  // byte within the image row
                const bool ok = i < total && b >= 0 && b < row_bytes && (unsigned)iy < (unsigned)H;
                v[u] = __builtin_amdgcn_raw_buffer_load_b128(
                    rx, ok ? (int)((size_t)(n * H + iy) * row_bytes + b) : (int)kOOB, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + 256 * u, r = i / chunks, c = i - r * chunks;
                if (i < total) *reinterpret_cast<u32x4 *>(srow + r * rstr + c * 16) = v[u];
            }
        }
    }
    __syncthreads();
    if (g >= groups) return;

    const int c0 = 30 * g - 1;
    const int cc = c0 + rl;                  // this lane's conv column
    const bool col_ok = cc >= 0 && cc < OW;
    const int ccr = cc < 0 ? 0 : (cc < OW ? cc : OW - 1);  // column read for the patch
    const int byte = 6 * (ccr * S - 1 - ixs);
    const int base = byte & ~3, sh = (byte & 3) * 8;
    float best[FN][16];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) best[j][e] = -__builtin_inff();
    auto act_max = [&](auto act_tag, const f32x16 (&acc)[FN], bool ok) {
        constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float x = acc[j][e];
                if constexpr (ACT == CONV2D_ACT_RELU) x = __builtin_fmaxf(x, 0.0f);
                if constexpr (ACT == CONV2D_ACT_SILU) x = x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
                if constexpr (ACT == CONV2D_ACT_PRELU) {
                    const float al = bal[1][j * 32 + 8 * (e / 4) + 4 * hi + (e % 4)];
                    x = x >= 0.0f ? x : al * x;
                }
                // through a scalar: this compiler lowers a bit cast applied directly to a
                // vector element as a read of element 0
                const float c = ok ? to_f32(round_fp32<T>(x)) : -__builtin_inff();
                const int v = __builtin_bit_cast(int, c);
                // neighbours by whole-wave DPP shifts: lane i reads lane i-1, resp. i+1
                // (lanes 0 and 63 keep their own value)
                const float l = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(v, v, 0x138, 0xf, 0xf, false));
                const float r = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(v, v, 0x130, 0xf, 0xf, false));
                const float m = first_max3(l, c, r);
                best[j][e] = m > best[j][e] ? m : best[j][e];
            }
    };
#pragma unroll
    for (int dr = 0; dr < 3; ++dr) {
        const int oy = 2 * py - 1 + dr;
        const bool row_ok = oy >= 0 && oy < OH;
        const int r0 = (dr + (row_ok ? 0 : (oy < 0 ? 1 : -1))) * S;  // a clamped row when out of range
        vec xb[2];
        stem_operands(srow + r0 * rstr, rstr, base, sh, hi, xb);
        f32x16 acc[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 bq = *reinterpret_cast<const f32x4 *>(&bal[0][j * 32 + 8 * gq + 4 * hi]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[j][4 * gq + e] = bq[e];
            }
            acc[j] = Mfma32<T>::run(wa[0][j], xb[0], acc[j]);
            acc[j] = Mfma32<T>::run(wa[1][j], xb[1], acc[j]);
        }
        const bool ok = row_ok && col_ok;
        switch (a.act) {
        case CONV2D_ACT_RELU: act_max(std::integral_constant<int, CONV2D_ACT_RELU>{}, acc, ok); break;
        case CONV2D_ACT_SILU: act_max(std::integral_constant<int, CONV2D_ACT_SILU>{}, acc, ok); break;
        case CONV2D_ACT_PRELU: act_max(std::integral_constant<int, CONV2D_ACT_PRELU>{}, acc, ok); break;
        default: act_max(std::integral_constant<int, CONV2D_ACT_NONE>{}, acc, ok); break;
        }
    }
    // pooled column of this lane (odd lanes below 30 are window centres)
    const int px = 15 * g + (rl - 1) / 2;
    const bool store = (rl & 1) && rl < 30 && px < PW;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, (uint32_t)((size_t)a.N * PH * PW * Cout * sizeof(T)));
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            u32x2 q[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                T out[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = from_f32<T>(best[j][4 * (2 * pp + h) + e]);
                __builtin_memcpy(&q[h], out, 8);
            }
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const auto r2 = __builtin_amdgcn_permlane32_swap(q[0][d], q[1][d], false, false);
                q[0][d] = r2[0];
                q[1][d] = r2[1];
            }
            const int co = j * 32 + 16 * pp + 8 * hi;
            const uint32_t off = (store && co < Cout)
                                     ? ((uint32_t)((n * PH + py) * PW + px) * (uint32_t)Cout + (uint32_t)co) *
                                           (uint32_t)sizeof(T)
                                     : kOOB;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{q[0][0], q[0][1], q[1][0], q[1][1]}, ry, (int)off, 0, 0);
        }
}

// Two 3x3 convs in one kernel, the first one's output never stored: a 3-channel image
// through a stride-2 conv to 32 channels (the stem conv above), then a stride-1 conv of
// that map to at most 32 channels (the second conv of the inferencelayer page's
// `encoder_maps` stem; a stack hands this pair over when the first output is marked
// transient). Persistent workgroups of 4 waves walk 8 x 32 output tiles of the second
// conv. Per tile: the image window its input halo needs (21 rows x 69 columns) is
// staged in LDS; the waves compute the first conv on the 10 x 34 halo pixels (the stem
// kernel's two 32x32x16 products per 32 pixels, accumulators from the bias, activation,
// one rounding; pixels outside the first conv's map are the second conv's zero padding)
// and write them to a halo buffer in the layout of the halo kernel; then the second
// conv's products read the halo (weights in registers, the same k order and
// accumulation as the halo kernel), while the next tile's image rows go straight from
// memory into the staging buffer (direct-to-LDS loads, which hold no registers; the
// first tile's go out before the weights are read, so the two latencies overlap). Both
// convs round exactly as the two kernels do, so the output equals the two launches bit
// for bit. Three workgroups per CU (measured on MI355X at 4 x 640 x 640: 22.2 us against
// 23.8 with two, and 27.8 for the two launches, when the rows went through registers).
struct StemPairGeo {
    int tiles_w, tiles_h, ntiles;
};

// Waits until at most N of this wave's vector-memory operations are outstanding. The
// count is only meaningful if every store written before the wait is issued before it,
// so the compiler may not move memory operations across it.
template <int N> __device__ __forceinline__ void pair_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}

// Workgroup barrier after this wave's LDS accesses have completed; direct-to-LDS loads
// are published by the explicit vmcnt waits before it.
__device__ __forceinline__ void pair_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <typename T>
__global__ __launch_bounds__(256, 3) void stem_pair_kernel(ConvArgs a1, ConvArgs a2, StemPairGeo tg) {
    constexpr int NW = 4, TH = 8, TW = 32, FM = 2;     // tile rows, columns; rows per wave
    constexpr int HR = TH + 2, HW = TW + 2, NQ = HR * HW;  // halo of the second conv
    constexpr int PSTR = 80;                          // halo pixel: 32 channels + one pad slot
    constexpr int NB1 = (NQ + 31) / 32;               // 32-pixel blocks of the first conv
    constexpr int RSW = 2 * TH + 5;                   // image rows staged per tile
    constexpr int RSTR = 448;                         // bytes per staged image row (69 pixels + slack)
    constexpr int CPR = RSTR / 16;                    // 16-byte chunks per staged row
    constexpr int NSL = (RSW * CPR + 255) / 256;      // staging loads per thread
    constexpr int KSW = 18;                           // second conv: 9 taps x 2 chunks of 16 channels
    // the staged window takes whole 4 KiB rounds of direct-to-LDS loads (the slots past
    // its RSW rows hold zeros that nothing reads)
    constexpr int SBYTES = NSL * 256 * 16, HBYTES = NQ * PSTR;
    static_assert(SBYTES >= RSW * RSTR && RSTR == CPR * 16, "staged rows are contiguous 16-byte slots");
    static_assert(HBYTES >= KSW * 1024, "the weight staging fits the halo buffer");
    __shared__ __attribute__((aligned(16))) char srow[SBYTES];
    __shared__ __attribute__((aligned(1024))) char halo[HBYTES];
    __shared__ __attribute__((aligned(16))) float bal[4][32];  // bias and slopes of both convs
    typedef typename Mfma32<T>::vec vec;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rl = lane & 31, hi = lane >> 5;
    const int H = a1.H, W = a1.W, OH = a1.OH, OW = a1.OW;  // image; the first conv's map
    const int C2 = a2.Cout;

    // tiles t = k*G + r, the workgroups of one XCD taking a contiguous run of each whole
    // round; the tiles of a last, partial round go to workgroups by launch order instead
    // (blockIdx % 8 round-robins the XCDs), so its few tiles spread over all XCDs and
    // CUs rather than doubling up on the CUs of one
    const int G = gridDim.x;
    const int r = (G % 8) == 0 ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
    struct Geo {
        int n, oy0, ox0;
        bool live;
    };
    auto geo = [&](int k) -> Geo {
        const int t = k * G + ((k + 1) * G > tg.ntiles ? (int)blockIdx.x : r);
        const bool live = t < tg.ntiles;
        const int tt = live ? t : 0;
        const int tx = tt % tg.tiles_w, rr = tt / tg.tiles_w;
        return Geo{rr / tg.tiles_h, (rr % tg.tiles_h) * TH, tx * TW, live};
    };
    // Image window of a tile: rows 2*oy0 - 3 + j (j < RSW), the row bytes from win0 on
    // (16-byte aligned, at or before column 2*ox0 - 3), chunks outside the image zero.
    // It goes straight into srow (direct-to-LDS loads: slot i = 16-byte chunk i % CPR of
    // row i / CPR); every thread issues NSL loads, so each wave's count is the same.
    const int row_bytes = W * 6;
    const i32x4 rx = rsrc_words(a1.x, (uint32_t)((size_t)a1.N * H * row_bytes));
    auto win0 = [](int ox0) {  // byte of column 2*ox0 - 3 rounded down to 16 (floor for negatives)
        const int b = 6 * (2 * ox0 - 3);
        return b >= 0 ? b & ~15 : -((-b + 15) & ~15);
    };
    auto stage = [&](const Geo &g) {
#pragma unroll
        for (int d = 0; d < NSL; ++d) {
            const int i = threadIdx.x + 256 * d;
            const int j = i / CPR, c = i - j * CPR;
            const int iy = 2 * g.oy0 - 3 + j, b = win0(g.ox0) + 16 * c;
            const bool ok = g.live && i < RSW * CPR && (unsigned)iy < (unsigned)H && b >= 0 && b < row_bytes;
            dma_b128(rx, ok ? (uint32_t)((size_t)(g.n * H + iy) * row_bytes + b) : kOOB,
                     lds_addr(srow + (256 * d + 64 * wave) * 16));
        }
    };
    // the first tile's window goes out before the weights, so the two latencies overlap
    stage(geo(0));

    // first conv's weights as A operands (the stem kernel's layout: step 0 values 0..7 of
    // patch row hi, step 1 values 0..7 of row 2 or value 8 of rows 0..2)
    vec wa[2];
    {
        const T *w = static_cast<const T *>(a1.w);
        T v0[8], v1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v0[e] = w[rl * 27 + hi * 9 + e];
            const int k1 = hi == 0 ? 18 + e : (e < 3 ? e * 9 + 8 : -1);
            v1[e] = k1 >= 0 ? w[rl * 27 + k1] : from_f32<T>(0.0f);
        }
        __builtin_memcpy(&wa[0], v0, 16);
        __builtin_memcpy(&wa[1], v1, 16);
    }
    if (threadIdx.x < 32) {
        const int co = threadIdx.x;
        bal[0][co] = a1.bias ? a1.bias[co] : 0.0f;
        bal[1][co] = a1.alpha ? a1.alpha[co] : 0.0f;
        bal[2][co] = a2.bias && co < C2 ? a2.bias[co] : 0.0f;
        bal[3][co] = a2.alpha && co < C2 ? a2.alpha[co] : 0.0f;
    }
    // second conv's weights in operand order ([k step][lane] x 16 bytes: output channel
    // rl, input channels 16*(k step % 2) + 8*hi .. of tap k step / 2), staged once in the
    // halo buffer, then into registers
    vec bw[KSW];
    {
        const __amdgpu_buffer_rsrc_t rw2 = make_rsrc(a2.w, (uint32_t)((size_t)C2 * 9 * 32 * sizeof(T)));
#pragma unroll
        for (int d = 0; d < (KSW * 64 + 255) / 256; ++d) {
            const int u = threadIdx.x + 256 * d;  // (k step, lane) slot
            const int sw = u / 64, ln = u % 64, co = ln % 32, h2 = ln / 32;
            const bool ok = sw < KSW && co < C2;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                rw2, ok ? (int)(((co * 9 + sw / 2) * 32 + (sw % 2) * 16 + h2 * 8) * (int)sizeof(T)) : (int)kOOB, 0, 0);
            if (sw < KSW) *reinterpret_cast<u32x4 *>(halo + u * 16) = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int sw = 0; sw < KSW; ++sw) bw[sw] = *reinterpret_cast<const vec *>(halo + (sw * 64 + lane) * 16);


    const uint32_t out_bytes = (uint32_t)((size_t)a2.M * C2 * sizeof(T));
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a2.y, out_bytes);
    auto swap_halves = [](u32x2 &lo, u32x2 &hi2) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const auto r2 = __builtin_amdgcn_permlane32_swap(lo[d], hi2[d], false, false);
            lo[d] = r2[0];
            hi2[d] = r2[1];
        }
    };
    // the activations as the two kernels write them (their ReLU forms differ for -0)
    auto act1_of = [](auto act_tag, float x, float al) {  // the stem kernel's
        constexpr int ACT = decltype(act_tag)::value;
        if constexpr (ACT == CONV2D_ACT_RELU) x = __builtin_fmaxf(x, 0.0f);
        if constexpr (ACT == CONV2D_ACT_SILU) x = x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
        if constexpr (ACT == CONV2D_ACT_PRELU) x = x >= 0.0f ? x : al * x;
        return x;
    };
    auto act2_of = [](auto act_tag, float x, float al) {  // the halo kernel's
        constexpr int ACT = decltype(act_tag)::value;
        if constexpr (ACT == CONV2D_ACT_RELU) x = x > 0.0f ? x : 0.0f;
        if constexpr (ACT == CONV2D_ACT_SILU) x = x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
        if constexpr (ACT == CONV2D_ACT_PRELU) x = x >= 0.0f ? x : al * x;
        return x;
    };

    // First conv on the halo pixels of tile g (staged window in srow) into `halo`.
    auto first_conv = [&](auto act_tag, const Geo &g) {
        const int off0 = 6 * (2 * g.ox0 - 3) - win0(g.ox0);  // byte of window column 0 in a staged row
        for (int b = wave; b < NB1; b += NW) {
            const int q = 32 * b + rl, qc = q < NQ ? q : NQ - 1;
            const int hy = qc / HW, hx = qc - hy * HW;
            const int r1 = g.oy0 - 1 + hy, c1 = g.ox0 - 1 + hx;
            const bool inmap = (unsigned)r1 < (unsigned)OH && (unsigned)c1 < (unsigned)OW;
            const int byte = off0 + 12 * hx;
            vec xb[2];
            stem_operands(srow + 2 * hy * RSTR, RSTR, byte & ~3, (byte & 3) * 8, hi, xb);
            f32x16 acc;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 bq = *reinterpret_cast<const f32x4 *>(&bal[0][8 * gq + 4 * hi]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[4 * gq + e] = bq[e];
            }
            acc = Mfma32<T>::run(wa[0], xb[0], acc);
            acc = Mfma32<T>::run(wa[1], xb[1], acc);
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                u32x2 qv[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int gq = 2 * pp + h;
                    f32x4 al{0.0f, 0.0f, 0.0f, 0.0f};
                    if constexpr (decltype(act_tag)::value == CONV2D_ACT_PRELU)
                        al = *reinterpret_cast<const f32x4 *>(&bal[1][8 * gq + 4 * hi]);
                    T o4[4];
                    // rounded on every lane, then zeroed outside the map (a select, not a
                    // branch per value around the rounding's fence)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const T v = round_fp32<T>(act1_of(act_tag, acc[4 * gq + e], al[e]));
                        o4[e] = inmap ? v : from_f32<T>(0.0f);
                    }
                    __builtin_memcpy(&qv[h], o4, 8);
                }
                swap_halves(qv[0], qv[1]);
                // lane (rl, hi): channels 16*pp + 8*hi .. of halo pixel q
                if (q < NQ)
                    *reinterpret_cast<u32x4 *>(halo + q * PSTR + (2 * pp + hi) * 16) =
                        u32x4{qv[0][0], qv[0][1], qv[1][0], qv[1][1]};
            }
        }
    };

    // Second conv's products of the tile (rows FM*wave, FM*wave + 1) and its epilogue.
    auto second_conv = [&](auto act_tag, const Geo &g) {
        f32x16 acc[FM];
        {
            f32x16 b0;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 bq = *reinterpret_cast<const f32x4 *>(&bal[2][8 * gq + 4 * hi]);
#pragma unroll
                for (int e = 0; e < 4; ++e) b0[4 * gq + e] = bq[e];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) acc[i] = b0;
        }
        const char *base = halo + ((wave * FM) * HW + rl) * PSTR + hi * 16;
        auto read = [&](int sw, vec(&fa)[FM]) {
            const int tap = sw / 2, ky = tap / 3, kx = tap % 3;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const vec *>(base + ((i + ky) * HW + kx) * PSTR + (sw % 2) * 32);
        };
        constexpr int PF = 2;
        vec fa[PF + 1][FM];
#pragma unroll
        for (int sw = 0; sw < PF; ++sw) read(sw, fa[sw]);
#pragma unroll
        for (int sw = 0; sw < KSW; ++sw) {
            if (sw + PF < KSW) read(sw + PF, fa[(sw + PF) % (PF + 1)]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FM; ++i) acc[i] = Mfma32<T>::run(bw[sw], fa[sw % (PF + 1)][i], acc[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int oy = g.oy0 + wave * FM + i, ox = g.ox0 + rl;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int co = 16 * pp + 8 * hi;
                const uint32_t off = (g.live && oy < OH && ox < OW && co < C2)
                                         ? ((uint32_t)((g.n * OH + oy) * OW + ox) * (uint32_t)C2 + (uint32_t)co) *
                                               (uint32_t)sizeof(T)
                                         : kOOB;
                u32x2 qv[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int gq = 2 * pp + h;
                    f32x4 al{0.0f, 0.0f, 0.0f, 0.0f};
                    if constexpr (decltype(act_tag)::value == CONV2D_ACT_PRELU)
                        al = *reinterpret_cast<const f32x4 *>(&bal[3][8 * gq + 4 * hi]);
                    T o4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o4[e] = round_fp32<T>(act2_of(act_tag, acc[i][4 * gq + e], al[e]));
                    __builtin_memcpy(&qv[h], o4, 8);
                }
                swap_halves(qv[0], qv[1]);
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{qv[0][0], qv[0][1], qv[1][0], qv[1][1]}, ry, (int)off, 0,
                                                       0);
            }
        }
    };

    // The second conv's epilogue issues FM * 2 stores per lane after the next window's
    // loads; waiting until no more than those are outstanding leaves the window landed.
    constexpr int NSTORE = FM * 2;
    auto run = [&](auto act1_tag, auto act2_tag) {
        Geo g = geo(0);
        // the first window has landed (this wave's loads; the barrier: every wave's),
        // and the weight fragments are in registers (lgkmcnt(0) in the barrier) before
        // the first tile's halo overwrites their staging
        pair_wait_vmcnt<0>();
        pair_barrier();
        for (int k = 0; g.live; ++k) {
            first_conv(act1_tag, g);
            pair_barrier();  // halo complete; every wave done with the staged window
            const Geo gn = geo(k + 1);
            stage(gn);
            second_conv(act2_tag, g);
            pair_wait_vmcnt<NSTORE>();
            pair_barrier();  // next window staged; every wave done reading the halo
            g = gn;
        }
        pair_wait_vmcnt<0>();  // no direct-to-LDS load outlives the workgroup
    };
    auto with_act2 = [&](auto act1_tag) {
        switch (a2.act) {
        case CONV2D_ACT_RELU: run(act1_tag, std::integral_constant<int, CONV2D_ACT_RELU>{}); break;
        case CONV2D_ACT_SILU: run(act1_tag, std::integral_constant<int, CONV2D_ACT_SILU>{}); break;
        case CONV2D_ACT_PRELU: run(act1_tag, std::integral_constant<int, CONV2D_ACT_PRELU>{}); break;
        default: run(act1_tag, std::integral_constant<int, CONV2D_ACT_NONE>{}); break;
        }
    };
    switch (a1.act) {
    case CONV2D_ACT_RELU: with_act2(std::integral_constant<int, CONV2D_ACT_RELU>{}); break;
    case CONV2D_ACT_SILU: with_act2(std::integral_constant<int, CONV2D_ACT_SILU>{}); break;
    case CONV2D_ACT_PRELU: with_act2(std::integral_constant<int, CONV2D_ACT_PRELU>{}); break;
    default: with_act2(std::integral_constant<int, CONV2D_ACT_NONE>{}); break;
    }
}

bool stem_pair_fits(const ConvArgs &a1, const ConvArgs &a2, int dtype) {
    return (dtype == CONV2D_DTYPE_BF16 || dtype == CONV2D_DTYPE_F16) && a1.Cin == 3 && a1.kh == 3 && a1.kw == 3 &&
           a1.stride == 2 && a1.pad == 1 && a1.Cout == 32 && !a1.res && (a1.W % 8) == 0 && a1.W <= 3000 &&
           a2.x == a1.y && a2.N == a1.N && a2.H == a1.OH && a2.W == a1.OW && a2.Cin == 32 && a2.kh == 3 && a2.kw == 3 &&
           a2.stride == 1 && a2.pad == 1 && !a2.res && a2.Cout <= 32 && (a2.Cout % 8) == 0 && a2.vec_out &&
           (long long)a1.N * a1.H * a1.W * 6 < (1ll << 31) && (long long)a2.M * a2.Cout * 2 < (1ll << 31);
}

hipError_t launch_stem_pair(const ConvArgs &a1, const ConvArgs &a2, int dtype, int grid_cap, hipStream_t st) {
    if (!stem_pair_fits(a1, a2, dtype) || grid_cap <= 0) return hipErrorInvalidValue;
    StemPairGeo tg{};
    tg.tiles_w = (a2.OW + 31) / 32;
    tg.tiles_h = (a2.OH + 7) / 8;
    const long long nt = (long long)a2.N * tg.tiles_w * tg.tiles_h;
    if (nt <= 0 || nt > 0x7fffffffll) return hipErrorInvalidValue;
    tg.ntiles = (int)nt;
    int grid = tg.ntiles < grid_cap ? tg.ntiles : grid_cap;
    if (grid > 8) grid -= grid % 8;
    if (dtype == CONV2D_DTYPE_BF16)
        return launch_kernel(stem_pair_kernel<bf16>, dim3(grid), dim3(256), 0, st, a1, a2, tg);
    return launch_kernel(stem_pair_kernel<f16>, dim3(grid), dim3(256), 0, st, a1, a2, tg);
}

template <typename T, int FN, int S>
static hipError_t launch_stem_pool_t(const ConvArgs &a, void *y, hipStream_t st) {
    constexpr int RS = 2 * S + 3;
    const int PH = (a.OH - 1) / 2 + 1, PW = (a.OW - 1) / 2 + 1;
    const int groups = (PW + 14) / 15;
    const int segs = (groups + 3) / 4;
    // a segment of 4 groups covers conv columns 120*seg - 1 .. 120*seg + 120, i.e. input
    // columns (120*seg - 1)*S - 1 .. (120*seg + 120)*S + 1; staging starts 8 columns
    // before 120*S*seg and reads 20 bytes from each patch row's first dword
    const int ixs_step = 120 * S;  // a multiple of 8
    const int rstr = (6 * (120 * S + 16) + 16 + 15) / 16 * 16;
    const size_t smem = (size_t)RS * rstr;
    const long long blocks = (long long)a.N * PH * segs;
    if (blocks * 256 > 0xffffffffll || smem > 64 * 1024) return hipErrorInvalidValue;
    ConvArgs b = a;
    b.y = y;
    return launch_kernel(stem3_pool_kernel<T, FN, S>, dim3((unsigned)blocks), dim3(256), smem, st, b, PH, PW,
                         groups, rstr, ixs_step);
}

template <typename T>
static hipError_t launch_stem_pool_d(const ConvArgs &a, void *y, hipStream_t st) {
    const int fn = a.Cout <= 32 ? 1 : 2;
    if (a.stride == 2) return fn == 1 ? launch_stem_pool_t<T, 1, 2>(a, y, st) : launch_stem_pool_t<T, 2, 2>(a, y, st);
    return fn == 1 ? launch_stem_pool_t<T, 1, 1>(a, y, st) : launch_stem_pool_t<T, 2, 1>(a, y, st);
}

hipError_t launch_stem3_maxpool(const ConvArgs &a, void *y, int dtype, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_BF16: return launch_stem_pool_d<bf16>(a, y, st);
    case CONV2D_DTYPE_F16: return launch_stem_pool_d<f16>(a, y, st);
    case CONV2D_DTYPE_F32: return launch_stem3_f32_maxpool(a, y, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int FN, int S>
static hipError_t launch_stem_t(const ConvArgs &a, hipStream_t st) {
    constexpr int RB = 2;
    constexpr int RS = (RB - 1) * S + 3;
    // 16 zero bytes, the row, and the right pad pixel plus the dword read past it
    const int rstr = ((16 + a.W * 6 + 8) + 15) / 16 * 16;
    const size_t smem = (size_t)RS * rstr;
    if (smem > 96 * 1024) return hipErrorInvalidValue;
    const long long blocks = (long long)a.N * ((a.OH + RB - 1) / RB);
    if (blocks > 0x7fffffffll) return hipErrorInvalidValue;
    return launch_kernel(stem3_kernel<T, FN, RB, S>, dim3((unsigned)blocks), dim3(256), smem, st, a, rstr);
}

template <typename T>
static hipError_t launch_stem_d(const ConvArgs &a, hipStream_t st) {
    const int fn = a.Cout <= 32 ? 1 : 2;
    if (a.stride == 2) return fn == 1 ? launch_stem_t<T, 1, 2>(a, st) : launch_stem_t<T, 2, 2>(a, st);
    return fn == 1 ? launch_stem_t<T, 1, 1>(a, st) : launch_stem_t<T, 2, 1>(a, st);
}

hipError_t launch_stem3(const ConvArgs &a, int dtype, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_BF16: return launch_stem_d<bf16>(a, st);
    case CONV2D_DTYPE_F16: return launch_stem_d<f16>(a, st);
    case CONV2D_DTYPE_F32: return launch_stem3_f32(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace c2d
