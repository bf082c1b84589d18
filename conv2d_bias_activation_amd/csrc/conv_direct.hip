// Direct convolution on the vector ALUs, for layers with few input channels.
//
// With Cin = 3 (the image stem of the inferencelayer page's `encoder_maps`, and the
// 7-channel first conv of the framecast page's graph) a GEMM has K = 27: too thin
// for matrix cores and dominated by reading the image and writing the feature map.
// Each thread computes one output pixel for a block of COB output channels with
// fp32 FMAs. The block's weights, widened to fp32, are staged once per input-channel
// chunk in LDS in [tap][ci][co] order, so that every lane of a wave reads the same
// 16 bytes (an LDS broadcast) for four output channels at a time.
// This kernel also serves any shape the matrix-core path does not take.
#include "common.hpp"
#include "kernels.hpp"

namespace c2d {

template <typename T, int COB, bool NCHW>
__global__ __launch_bounds__(256) void direct_kernel(ConvArgs a, int cic) {
    extern __shared__ float sw[];  // [kh*kw][cic][COB]
    const T *__restrict__ x = static_cast<const T *>(a.x);
    const T *__restrict__ w = static_cast<const T *>(a.w);
    const int H = a.H, W = a.W, Cin = a.Cin, kh = a.kh, kw = a.kw;
    const int taps = kh * kw;
    const int OHW = a.OH * a.OW;
    const int co0 = blockIdx.y * COB;
    const int m = blockIdx.x * 256 + threadIdx.x;
    const bool live = m < a.M;
    const int mm = live ? m : 0;
    const int n = mm / OHW, pix = mm - n * OHW;
    const int oh = pix / a.OW, ow = pix - oh * a.OW;
    const int ih0 = oh * a.stride - a.pad, iw0 = ow * a.stride - a.pad;

    float acc[COB];
#pragma unroll
    for (int j = 0; j < COB; ++j) acc[j] = 0.0f;

    for (int c0 = 0; c0 < Cin; c0 += cic) {
        const int cc_n = min(cic, Cin - c0);
        __syncthreads();
        // stage weights: sw[(tap*cic + cc)*COB + j] = w[co0+j][ci=c0+cc][tap]
        const int total = taps * cc_n * COB;
        for (int i = threadIdx.x; i < total; i += 256) {
            int j = i % COB;
            int r = i / COB;
            int cc = r % cc_n;
            int tap = r / cc_n;
            int co = co0 + j;
            float v = 0.0f;
            if (co < a.Cout) {
                size_t off = NCHW ? ((size_t)co * Cin + c0 + cc) * taps + tap
                                  : ((size_t)co * taps + tap) * Cin + c0 + cc;
                v = to_f32(w[off]);
            }
            sw[(tap * cic + cc) * COB + j] = v;
        }
        __syncthreads();
        if (!live) continue;
        for (int ky = 0; ky < kh; ++ky) {
            const int iy = ih0 + ky;
            if ((unsigned)iy >= (unsigned)H) continue;
            for (int kx = 0; kx < kw; ++kx) {
                const int ix = iw0 + kx;
                if ((unsigned)ix >= (unsigned)W) continue;
                const float *wt = sw + (ky * kw + kx) * cic * COB;
                for (int cc = 0; cc < cc_n; ++cc) {
                    const int ci = c0 + cc;
                    const float xv = to_f32(NCHW ? x[(((size_t)n * Cin + ci) * H + iy) * W + ix]
                                                 : x[(((size_t)n * H + iy) * W + ix) * Cin + ci]);
                    const f32x4 *w4 = reinterpret_cast<const f32x4 *>(wt + cc * COB);
#pragma unroll
                    for (int j4 = 0; j4 < COB / 4; ++j4) {
                        f32x4 ww = w4[j4];
                        acc[4 * j4 + 0] = __builtin_fmaf(xv, ww[0], acc[4 * j4 + 0]);
                        acc[4 * j4 + 1] = __builtin_fmaf(xv, ww[1], acc[4 * j4 + 1]);
                        acc[4 * j4 + 2] = __builtin_fmaf(xv, ww[2], acc[4 * j4 + 2]);
                        acc[4 * j4 + 3] = __builtin_fmaf(xv, ww[3], acc[4 * j4 + 3]);
                    }
                }
            }
        }
    }
    if (!live) return;

    const T *__restrict__ res = static_cast<const T *>(a.res);
    T *__restrict__ y = static_cast<T *>(a.y);
    const bool has_res = res != nullptr, pre = a.res_before_act != 0;
    constexpr int VE = 16 / (int)sizeof(T);
    if (!NCHW && a.vec_out && (a.Cout % VE) == 0 && co0 + COB <= a.Cout) {
        size_t o = (size_t)m * a.Cout + co0;
#pragma unroll
        for (int v = 0; v < COB / VE; ++v) {
            T rv[VE], out[VE];
            if (has_res) {
                u32x4 t = *reinterpret_cast<const u32x4 *>(res + o + v * VE);
                __builtin_memcpy(rv, &t, 16);
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                int j = v * VE + e, co = co0 + j;
                float b = a.bias ? a.bias[co] : 0.0f;
                float al = a.alpha ? a.alpha[co] : 0.0f;
                float r = has_res ? to_f32(rv[e]) : 0.0f;
                out[e] = round_fp32<T>(epilogue(acc[j], b, al, r, has_res, a.act, pre));
            }
            u32x4 t;
            __builtin_memcpy(&t, out, 16);
            *reinterpret_cast<u32x4 *>(y + o + v * VE) = t;
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < COB; ++j) {
        int co = co0 + j;
        if (co >= a.Cout) break;
        size_t o = NCHW ? ((size_t)n * a.Cout + co) * OHW + pix : (size_t)m * a.Cout + co;
        float b = a.bias ? a.bias[co] : 0.0f;
        float al = a.alpha ? a.alpha[co] : 0.0f;
        float r = has_res ? to_f32(res[o]) : 0.0f;
        y[o] = round_fp32<T>(epilogue(acc[j], b, al, r, has_res, a.act, pre));
    }
}

template <typename T, bool NCHW>
static hipError_t launch_direct_t(const ConvArgs &a, hipStream_t st) {
    constexpr int COB = 32;
    const int taps = a.kh * a.kw;
    // LDS budget for the staged weights: 32 KiB.
    int cic = (32 * 1024 / 4) / (taps * COB);
    if (cic < 1) return hipErrorInvalidValue;
    if (cic > a.Cin) cic = a.Cin;
    size_t smem = (size_t)taps * cic * COB * sizeof(float);
    dim3 grid((a.M + 255) / 256, (a.Cout + COB - 1) / COB);
    return launch_kernel(direct_kernel<T, COB, NCHW>, grid, dim3(256), smem, st, a, cic);
}

hipError_t launch_direct(const ConvArgs &a, int dtype, bool nchw, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_F32:
        return nchw ? launch_direct_t<float, true>(a, st) : launch_direct_t<float, false>(a, st);
    case CONV2D_DTYPE_BF16:
        return nchw ? launch_direct_t<bf16, true>(a, st) : launch_direct_t<bf16, false>(a, st);
    case CONV2D_DTYPE_F16:
        return nchw ? launch_direct_t<f16, true>(a, st) : launch_direct_t<f16, false>(a, st);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace c2d
