// The stem conv of the inferencelayer page's `encoder_maps` (3x3 over a 3-channel
// channel-last image, stride 1 or 2, pad 1) in fp32 storage on CDNA4 matrix cores, and
// the same conv followed by the 3x3 stride-2 pad-1 max pool in one kernel that writes
// only the pooled map.
//
// The products use v_mfma_f32_32x32x2_f32: 32 output channels (A operand, the weights)
// by 32 pixels (B operand), two k values per instruction, K = 27 padded to 28 (14
// instructions per block). k follows the OHWI weight row, k = 9*ky + 3*kx + c. Lane
// (rl, hi) holds A[rl][hi] and B[hi][rl] of each instruction; the 16 results of lane
// (rl, hi) are channels 8*(e/4) + 4*hi + e%4 of pixel rl. The accumulators start from
// the bias, and both kernels build every pixel's sum in the same order, so the pooled
// map equals pooling the plain kernel's output bit for bit.
//
// A workgroup stages the input rows it needs in LDS (16-byte copies of whole pixel
// triples, zeros outside the image); a lane reads its 14 B values as single floats.
#include "igemm_common.hpp"
#include "kernels.hpp"

namespace c2d {

namespace {

__device__ __forceinline__ f32x16 mfma32x2(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// A operands of channel block j: lane (rl, hi), step s: w[co][2s + hi] (0 past k = 26
// or co >= Cout).
template <int FN>
__device__ __forceinline__ void stem_f32_weights(const ConvArgs &a, int rl, int hi, float (&wa)[FN][14]) {
    const float *w = static_cast<const float *>(a.w);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int co = 32 * j + rl;
#pragma unroll
        for (int s = 0; s < 14; ++s) {
            const int k = 2 * s + hi;
            wa[j][s] = (co < a.Cout && k < 27) ? w[co * 27 + k] : 0.0f;
        }
    }
}

// LDS float offset of k value 2s + hi of a patch whose top-left input pixel is at
// column ix0 (relative to the staged origin) of staged row r0: row (r0 + ky) of `rf`
// floats, 3 floats per pixel.
__device__ __forceinline__ int stem_f32_koff(int s, int hi, int rf) {
    const int k = 2 * s + hi < 27 ? 2 * s + hi : 26;  // the padding step reads a real value times a zero weight
    const int ky = k / 9, kx = (k % 9) / 3, c = k % 3;
    return ky * rf + 3 * kx + c;
}

// The 14 products of one block: acc += W x patch; `pix` is the patch origin's float
// offset in LDS.
template <int FN>
__device__ __forceinline__ void stem_f32_block(const float *sx, int pix, int hi, int rf, const float (&wa)[FN][14],
                                               f32x16 (&acc)[FN]) {
    float xb[14];
#pragma unroll
    for (int s = 0; s < 14; ++s) xb[s] = sx[pix + stem_f32_koff(s, hi, rf)];
#pragma unroll
    for (int s = 0; s < 14; ++s)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[j] = mfma32x2(wa[j][s], xb[s], acc[j]);
}

// Bias (and PReLU slopes) of this lane's channels: e -> 32j + 8*(e/4) + 4*hi + e%4.
template <int FN>
__device__ __forceinline__ void stem_f32_bias(const ConvArgs &a, int hi, float (&bq)[FN][16], float (&aq)[FN][16]) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int co = 32 * j + 8 * (e / 4) + 4 * hi + (e % 4);
            bq[j][e] = (a.bias && co < a.Cout) ? a.bias[co] : 0.0f;
            aq[j][e] = (a.alpha && co < a.Cout) ? a.alpha[co] : 0.0f;
        }
}

template <int ACT> __device__ __forceinline__ float stem_f32_act(float x, float al) {
    if constexpr (ACT == CONV2D_ACT_RELU) x = x > 0.0f ? x : 0.0f;
    if constexpr (ACT == CONV2D_ACT_SILU) x = x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
    if constexpr (ACT == CONV2D_ACT_PRELU) x = x >= 0.0f ? x : al * x;
    return x;
}

// Copies input rows iy0 .. iy0 + nrows - 1, columns ix0 .. ix0 + ncols - 1 (ix0 and
// ncols multiples of 4), into LDS rows of rf floats; zeros outside the image.
__device__ __forceinline__ void stem_f32_stage(const ConvArgs &a, int n, int iy0, int nrows, int ix0, int ncols,
                                               int rf, float *sx) {
    const int H = a.H, W = a.W;
    const int chunks = ncols * 3 / 4;  // 16-byte chunks per staged row
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)((size_t)a.N * H * W * 12));
    // eight loads per thread in flight before their LDS writes (unconditional, with an
    // out-of-range offset for padding): one load latency per round
    const int total = nrows * chunks, step = (int)blockDim.x;
    for (int i0 = threadIdx.x; i0 < total; i0 += 8 * step) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + step * u, r = i / chunks, c = i - r * chunks;
            const int iy = iy0 + r;
            const int fl = ix0 * 3 + c * 4;  // float within the image row (may be negative)
            const bool ok = i < total && (unsigned)iy < (unsigned)H && fl >= 0 && fl < W * 3;
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(
                rx, ok ? (int)(((size_t)(n * H + iy) * W * 3 + fl) * 4) : (int)kOOB, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + step * u, r = i / chunks, c = i - r * chunks;
            if (i < total) *reinterpret_cast<u32x4 *>(sx + r * rf + c * 4) = v[u];
        }
    }
}

}  // namespace

// Plain conv: one workgroup per output row; each wave takes 32-pixel column blocks.
template <int FN, int S>
__global__ __launch_bounds__(256) void stem3_f32_kernel(ConvArgs a, int rf) {
    extern __shared__ __attribute__((aligned(16))) float sx[];  // [3][rf]: columns -4 ..
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rl = lane & 31, hi = lane >> 5;
    const int OH = a.OH, OW = a.OW, Cout = a.Cout;
    const int n = blockIdx.x / OH, oy = blockIdx.x - n * OH;

    float wa[FN][14], bq[FN][16], aq[FN][16];
    stem_f32_weights<FN>(a, rl, hi, wa);
    stem_f32_bias<FN>(a, hi, bq, aq);
    // staged row r = input row oy*S - 1 + r; float 3*(ix + 4) + c holds column ix
    stem_f32_stage(a, n, oy * S - 1, 3, -4, rf / 3, rf, sx);
    __syncthreads();

    const bool has_res = a.res != nullptr;
    const int res_mode = has_res ? (a.res_before_act ? 1 : 2) : 0;
    const uint32_t out_bytes = (uint32_t)((size_t)a.M * Cout * 4);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, out_bytes);
    const __amdgpu_buffer_rsrc_t rres = make_rsrc(a.res, has_res ? out_bytes : 0u);
    const int nblk = (OW + 31) / 32;
    for (int cb = wave; cb < nblk; cb += 4) {
        const int ox = cb * 32 + rl;
        const int oxr = ox < OW ? ox : OW - 1;
        f32x16 acc[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] = bq[j][e];
        stem_f32_block<FN>(sx, 3 * (oxr * S - 1 + 4), hi, rf, wa, acc);
        auto finish = [&](auto act_tag, auto res_tag) {
            constexpr int ACT = decltype(act_tag)::value;
            constexpr int RES = decltype(res_tag)::value;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int co = 32 * j + 8 * q + 4 * hi;
                    const uint32_t off = (ox < OW && co < Cout)
                                             ? ((uint32_t)((n * OH + oy) * OW + ox) * (uint32_t)Cout + (uint32_t)co) * 4u
                                             : kOOB;
                    f32x4 r4 = RES != 0 ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rres, (int)off, 0, 0))
                                        : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    f32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float v = acc[j][4 * q + e];
                        if constexpr (RES == 1) v += r4[e];
                        v = stem_f32_act<ACT>(v, aq[j][4 * q + e]);
                        if constexpr (RES == 2) v += r4[e];
                        o[e] = v;
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), ry, (int)off, 0, 0);
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

// Conv + max pool: workgroup = one pooled row py of one image and a segment of 4
// column groups, one per wave. Group g covers conv columns 30g - 1 .. 30g + 30 of the
// conv rows 2py - 1 .. 2py + 1; lane rl = 2k + 1 (k < 15) is the centre of pooled
// column 15g + k, so every window lies inside one group. Each conv row is activated,
// its columns rl - 1, rl, rl + 1 (DPP wave shifts) maxed left to right, then the rows top to
// bottom, each step keeping the running value unless the next is strictly greater: the
// pool kernel's comparison in row-major tap order (NaN skipped, an all-NaN window gives
// -inf, the first of equal zeros kept); taps outside the conv map count as -inf.
template <int FN, int S>
__global__ __launch_bounds__(256) void stem3_f32_pool_kernel(ConvArgs a, int PH, int PW, int groups, int rf) {
    constexpr int RS = 2 * S + 3;
    extern __shared__ __attribute__((aligned(16))) float sx[];  // [RS][rf]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rl = lane & 31, hi = lane >> 5;
    const int OH = a.OH, OW = a.OW, Cout = a.Cout;
    const int segs = (groups + 3) / 4;
    const int seg = blockIdx.x % segs, py = (blockIdx.x / segs) % PH, n = blockIdx.x / (segs * PH);
    const int g = seg * 4 + wave;

    float wa[FN][14], bq[FN][16], aq[FN][16];
    stem_f32_weights<FN>(a, rl, hi, wa);
    stem_f32_bias<FN>(a, hi, bq, aq);
    // the segment's conv columns 120 seg - 1 .. 120 seg + 120 read input columns
    // (120 seg - 1) S - 1 .. (120 seg + 120) S + 1; staging starts at ixs = 120 S seg - 4
    const int ixs = 120 * S * seg - 4;
    stem_f32_stage(a, n, (2 * py - 1) * S - 1, RS, ixs, rf / 3, rf, sx);
    __syncthreads();
    if (g >= groups) return;

    const int cc = 30 * g - 1 + rl;  // this lane's conv column
    const bool col_ok = cc >= 0 && cc < OW;
    const int ccr = cc < 0 ? 0 : (cc < OW ? cc : OW - 1);
    const int pix = 3 * (ccr * S - 1 - ixs);
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
                const float c = ok ? stem_f32_act<ACT>(acc[j][e], aq[j][e]) : -__builtin_inff();
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
        f32x16 acc[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] = bq[j][e];
        stem_f32_block<FN>(sx, r0 * rf + pix, hi, rf, wa, acc);
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
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, (uint32_t)((size_t)a.N * PH * PW * Cout * 4));
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int co = 32 * j + 8 * q + 4 * hi;
            const uint32_t off = (store && co < Cout)
                                     ? ((uint32_t)((n * PH + py) * PW + px) * (uint32_t)Cout + (uint32_t)co) * 4u
                                     : kOOB;
            const f32x4 o = {best[j][4 * q], best[j][4 * q + 1], best[j][4 * q + 2], best[j][4 * q + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), ry, (int)off, 0, 0);
        }
}

namespace {

template <int FN, int S> hipError_t launch_stem_f32_t(const ConvArgs &a, hipStream_t st) {
    // staged row: columns -4 .. W + 3 (the right pad pixel and one past), 3 floats each
    const int rf = (a.W + 8) * 3;
    const size_t smem = (size_t)3 * rf * 4;
    const long long blocks = (long long)a.N * a.OH;
    if (smem > 64 * 1024 || blocks > 0x7fffffffll) return hipErrorInvalidValue;
    return launch_kernel(stem3_f32_kernel<FN, S>, dim3((unsigned)blocks), dim3(256), smem, st, a, rf);
}

template <int FN, int S> hipError_t launch_stem_f32_pool_t(const ConvArgs &a, void *y, hipStream_t st) {
    constexpr int RS = 2 * S + 3;
    const int PH = (a.OH - 1) / 2 + 1, PW = (a.OW - 1) / 2 + 1;
    const int groups = (PW + 14) / 15;
    const int segs = (groups + 3) / 4;
    // staged columns: ixs .. ixs + 120 S + 8 (a segment's patch columns and margins)
    const int rf = (120 * S + 8) * 3;
    const size_t smem = (size_t)RS * rf * 4;
    const long long blocks = (long long)a.N * PH * segs;
    if (smem > 64 * 1024 || blocks > 0x7fffffffll) return hipErrorInvalidValue;
    ConvArgs b = a;
    b.y = y;
    return launch_kernel(stem3_f32_pool_kernel<FN, S>, dim3((unsigned)blocks), dim3(256), smem, st, b, PH, PW,
                         groups, rf);
}

}  // namespace

hipError_t launch_stem3_f32(const ConvArgs &a, hipStream_t st) {
    const int fn = a.Cout <= 32 ? 1 : 2;
    if (a.stride == 2) return fn == 1 ? launch_stem_f32_t<1, 2>(a, st) : launch_stem_f32_t<2, 2>(a, st);
    return fn == 1 ? launch_stem_f32_t<1, 1>(a, st) : launch_stem_f32_t<2, 1>(a, st);
}

hipError_t launch_stem3_f32_maxpool(const ConvArgs &a, void *y, hipStream_t st) {
    const int fn = a.Cout <= 32 ? 1 : 2;
    if (a.stride == 2) return fn == 1 ? launch_stem_f32_pool_t<1, 2>(a, y, st) : launch_stem_f32_pool_t<2, 2>(a, y, st);
    return fn == 1 ? launch_stem_f32_pool_t<1, 1>(a, y, st) : launch_stem_f32_pool_t<2, 1>(a, y, st);
}

}  // namespace c2d
