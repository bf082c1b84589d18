// The ResNet-D shortcut of a downsampling block in one kernel: the 2x2 stride-2 average
// pool of the block input (inferencelayer page, AVGPOOL_SRC: ((x00 + x01) + x10) + x11
// then x 0.25 in fp32, one rounding) and the 1x1 convolution of the pooled map
// (inferencelayer page, `conv()` with a 1x1 kernel: a GEMM over the input channels, bias
// and activation in the epilogue), channel-last, 16-bit storage.
//
// A workgroup owns TM pooled pixels and TN output channels with the whole K (Cin) in
// LDS. While it stages its pixel operand it computes the pool: each thread reads the
// four 16-byte input vectors of one (pooled pixel, 8-channel) item, adds them in the pool
// kernel's order, rounds once and writes the result both to LDS and (the workgroups of
// the first channel tile) to the pooled map, which the stack still defines as an
// output. The weights are staged beside it. Products: 32x32x16 matrix-core steps over k
// in increasing order from a zero accumulator, the bias added in the epilogue, one
// rounding: the arithmetic of the general GEMM on these shapes, so the outputs equal a
// pool call followed by a conv call bit for bit.
//
// LDS rows are the Cin channels of one pixel or one output channel, RS = Cin/8 16-byte
// pieces; piece q of row r sits at q ^ (r % 8), so the 32 rows one operand fragment
// reads fall on distinct bank groups per eight lanes.
#include "igemm_common.hpp"
#include "kernels.hpp"

namespace c2d {

template <typename T, int TM, int TN, int CIN>
__global__ __launch_bounds__(256, 1) void poolpw_kernel(PoolPwArgs a) {
    constexpr int RS = CIN / 8;              // 16-byte pieces per row
    constexpr int KS = CIN / 16;             // 16-deep k steps
    constexpr int MB = TM / 32, NB = TN / 32;
    constexpr int NBW = MB * NB / 4;         // 32x32 blocks per wave
    static_assert(MB * NB % 4 == 0 && NBW >= 1, "blocks split evenly over four waves");
    static_assert(RS >= 8, "at least 64 input channels");
    constexpr int ABYTES = TM * CIN * (int)sizeof(T), BBYTES = TN * CIN * (int)sizeof(T);
    static_assert(ABYTES + BBYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) char lds[ABYTES + BBYTES];
    char *const As = lds;            // pooled pixels
    char *const Bs = lds + ABYTES;   // weights
    typedef typename Mfma32<T>::vec vec;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rl = lane & 31, hi = lane >> 5;
    const int H = a.H, W = a.W, OH = a.OH, OW = a.OW, Cout = a.Cout;
    const int M = a.N * OH * OW;
    const int tn = blockIdx.x % a.tiles_n, tm = blockIdx.x / a.tiles_n;
    const int m0 = tm * TM, n0 = tn * TN;
    auto piece = [](int r, int q) { return r * RS + (q ^ (r & 7)); };

    // All loads go out before any is used (whole unrolled loops of compile-time length),
    // so the workgroup pays the memory latency once.
    constexpr int NWI = TN * RS / 256, NAI = TM * RS / 256;  // weight and pixel items per thread
    static_assert(TN * RS % 256 == 0 && TM * RS % 256 == 0, "whole items per thread");
    // weights: row r = output channel n0 + r (zeros past Cout)
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (uint32_t)((size_t)Cout * CIN * sizeof(T)));
    u32x4 wv[NWI];
#pragma unroll
    for (int k = 0; k < NWI; ++k) {
        const int it = tid + 256 * k, r = it / RS, q = it % RS, co = n0 + r;
        wv[k] = __builtin_amdgcn_raw_buffer_load_b128(
            rw, (int)(co < Cout ? (uint32_t)((co * CIN + q * 8) * (int)sizeof(T)) : kOOB), 0, 0);
    }
    // pooled pixels: row p = pooled pixel m0 + p (zeros past M)
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)((size_t)a.N * H * W * CIN * sizeof(T)));
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.p, a.p ? (uint32_t)((size_t)M * CIN * sizeof(T)) : 0u);
    const bool write_p = a.p != nullptr && tn == 0;
    const uint32_t dx = (uint32_t)(CIN * (int)sizeof(T)), dy = (uint32_t)(W * CIN * (int)sizeof(T));
    u32x4 xv[NAI][4];
    uint32_t pout[NAI];
#pragma unroll
    for (int k = 0; k < NAI; ++k) {
        const int it = tid + 256 * k, p = it / RS, q = it % RS, m = m0 + p;
        uint32_t o00 = kOOB;
        pout[k] = kOOB;
        if (m < M) {
            const int n = m / (OH * OW), rem = m - n * OH * OW, oh = rem / OW, ow = rem - oh * OW;
            o00 = (uint32_t)((((n * H + 2 * oh) * W + 2 * ow) * CIN + q * 8) * (int)sizeof(T));
            pout[k] = (uint32_t)((m * CIN + q * 8) * (int)sizeof(T));
        }
        xv[k][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)o00, 0, 0);
        xv[k][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(o00 == kOOB ? kOOB : o00 + dx), 0, 0);
        xv[k][2] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(o00 == kOOB ? kOOB : o00 + dy), 0, 0);
        xv[k][3] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(o00 == kOOB ? kOOB : o00 + dy + dx), 0, 0);
    }
#pragma unroll
    for (int k = 0; k < NWI; ++k) {
        const int it = tid + 256 * k, r = it / RS, q = it % RS;
        *reinterpret_cast<u32x4 *>(Bs + piece(r, q) * 16) = wv[k];
    }
#pragma unroll
    for (int k = 0; k < NAI; ++k) {
        const int it = tid + 256 * k, p = it / RS, q = it % RS;
        T t00[8], t01[8], t10[8], t11[8], out[8];
        __builtin_memcpy(t00, &xv[k][0], 16);
        __builtin_memcpy(t01, &xv[k][1], 16);
        __builtin_memcpy(t10, &xv[k][2], 16);
        __builtin_memcpy(t11, &xv[k][3], 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float s = to_f32(t00[e]) + to_f32(t01[e]);
            s = s + to_f32(t10[e]);
            s = s + to_f32(t11[e]);
            out[e] = from_f32<T>(s * 0.25f);
        }
        u32x4 o;
        __builtin_memcpy(&o, out, 16);
        *reinterpret_cast<u32x4 *>(As + piece(p, q) * 16) = o;
        if (write_p) __builtin_amdgcn_raw_buffer_store_b128(o, rp, (int)pout[k], 0, 0);
    }
    __syncthreads();

    // products: block b = wave + 4*i is pixel block b % MB, channel block b / MB; the
    // weights are the A operand (rows = channels), the pixels the B operand
    f32x16 acc[NBW];
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int b = wave + 4 * i, mb = b % MB, nb = b / MB;
            const vec fa = *reinterpret_cast<const vec *>(Bs + piece(32 * nb + rl, 2 * ks + hi) * 16);
            const vec fb = *reinterpret_cast<const vec *>(As + piece(32 * mb + rl, 2 * ks + hi) * 16);
            acc[i] = Mfma32<T>::run(fa, fb, acc[i]);
        }
    }

    // epilogue: lane (rl, hi) of block (mb, nb) holds channels 32*nb + 8*g + 4*hi + 0..3,
    // g < 4, of pixel 32*mb + rl; one lane-half swap per pair of groups leaves 8
    // consecutive channels per lane for one 16-byte store
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, (uint32_t)((size_t)M * Cout * sizeof(T)));
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(a.bias, a.bias ? (uint32_t)Cout * 4u : 0u);
    const __amdgpu_buffer_rsrc_t ralpha = make_rsrc(a.alpha, a.alpha ? (uint32_t)Cout * 4u : 0u);
    const int act = a.act;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const int b = wave + 4 * i, mb = b % MB, nb = b / MB;
        const int m = m0 + 32 * mb + rl;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            u32x2 q2[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int g = 2 * pp + h;
                const int co = n0 + 32 * nb + 8 * g + 4 * hi;
                const uint32_t bo = co < Cout ? (uint32_t)co * 4u : kOOB;
                const f32x4 bv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rbias, (int)bo, 0, 0));
                const f32x4 av = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ralpha, (int)bo, 0, 0));
                T out[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = acc[i][4 * g + e] + bv[e];
                    if (act == CONV2D_ACT_RELU) v = v > 0.0f ? v : 0.0f;
                    if (act == CONV2D_ACT_SILU) v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
                    if (act == CONV2D_ACT_PRELU) v = v >= 0.0f ? v : av[e] * v;
                    out[e] = round_fp32<T>(v);
                }
                __builtin_memcpy(&q2[h], out, 8);
            }
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const auto r2 = __builtin_amdgcn_permlane32_swap(q2[0][d], q2[1][d], false, false);
                q2[0][d] = r2[0];
                q2[1][d] = r2[1];
            }
            const int co = n0 + 32 * nb + 16 * pp + 8 * hi;
            const uint32_t off = (m < M && co < Cout) ? (uint32_t)(((size_t)m * Cout + co) * sizeof(T)) : kOOB;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{q2[0][0], q2[0][1], q2[1][0], q2[1][1]}, ry, (int)off, 0, 0);
        }
    }
}

namespace {

template <typename T, int TM, int TN, int CIN>
hipError_t launch_pp(PoolPwArgs a, hipStream_t st) {
    const long long M = (long long)a.N * a.OH * a.OW;
    a.tiles_n = (a.Cout + TN - 1) / TN;
    const long long grid = (M + TM - 1) / TM * a.tiles_n;
    if (grid <= 0 || grid > 0x7fffffffll) return hipErrorInvalidValue;
    return launch_kernel(poolpw_kernel<T, TM, TN, CIN>, dim3((unsigned)grid), dim3(256), 0, st, a);
}

// Tile: 32 pixels x 128 channels for every input width. Each workgroup lives for one
// tile (its loads all go out at once), so the launch is bound by that latency, and more,
// smaller tiles finish sooner (measured on MI355X at the ResNet-D shortcut shapes, 4 x
// 160^2 x 64 -> 128: 6.7 us against 7.6 with 64 x 128 and 7.8 with 64 x 64; 128 and 256
// input channels 5.8 and 6.2 us, the best of the shapes tried).
template <typename T> hipError_t launch_pp_t(const PoolPwArgs &a, hipStream_t st) {
    switch (a.Cin) {
    case 64: return launch_pp<T, 32, 128, 64>(a, st);
    case 128: return launch_pp<T, 32, 128, 128>(a, st);
    case 256: return launch_pp<T, 32, 128, 256>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool poolpw_fits(int Cin, int Cout, int dtype) {
    return (dtype == CONV2D_DTYPE_BF16 || dtype == CONV2D_DTYPE_F16) && (Cin == 64 || Cin == 128 || Cin == 256) &&
           Cout % 8 == 0 && Cout > 0;
}

hipError_t launch_poolpw(const PoolPwArgs &a, int dtype, hipStream_t st) {
    if (!poolpw_fits(a.Cin, a.Cout, dtype) || a.OH != a.H / 2 || a.OW != a.W / 2 || a.OH < 1 || a.OW < 1)
        return hipErrorInvalidValue;
    switch (dtype) {
    case CONV2D_DTYPE_BF16: return launch_pp_t<bf16>(a, st);
    case CONV2D_DTYPE_F16: return launch_pp_t<f16>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace c2d
