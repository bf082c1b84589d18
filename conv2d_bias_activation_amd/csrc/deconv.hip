// Transposed convolution, 4x4 kernel, stride 2, pad 1: the ConvTranspose2d that ends
// an IFNet block on the framecast page (`wgslDeconv`). Input pixel (iy, ix) with tap
// (ky, kx) adds x * w[ci][co][ky][kx] to output (2*iy - 1 + ky, 2*ix - 1 + kx); then
// bias and the activation.
//
// Seen from an output pixel (2j + py, 2i + px), only the taps with ky of parity
// 1 - py and kx of parity 1 - px land on it, two per axis: each of the four output
// parity classes (py, px) is a 2x2 stride-1 convolution over the input, tap (ty, tx)
// reading input pixel (j - 1 + py + ty, i - 1 + px + tx) with weight
// w[ci][co][3 - py - 2*ty][3 - px - 2*tx]. The matrix-core kernel runs exactly that:
// the weights are first repacked (once per call, into the library scratch) to
// wp[class][co][tap][ci] with ci contiguous, so each class is a GEMM with K = 4*Cin
// whose B operand rows are 16-byte runs; a workgroup stages three input rows of a
// 34-pixel strip once and its four waves (one per class) read shifted views of it.
#include "common.hpp"
#include "igemm_common.hpp"
#include "kernels.hpp"

namespace c2d {

namespace {

constexpr int DC_TW = 32;           // input columns per tile: 64 output columns, 2 output rows
constexpr int DC_KC = 32;           // input channels per staged chunk
constexpr int DC_SPX = DC_TW + 2;   // staged columns i0 - 1 .. i0 + 32
constexpr int DC_PS = 40;           // LDS elements per staged pixel: 80 bytes, an odd number of
                                    // 16-byte slots, so 32 lanes reading 32 pixels hit distinct banks
constexpr int DC_BUF = 3 * DC_SPX * DC_PS;
constexpr int DC_VECS = 3 * DC_SPX * (DC_KC / 8);  // 16-byte vectors per staged chunk (408)
constexpr int DC_OLD = 2 * DC_TW + 2;              // output tile row in LDS: 64 columns + 2 pad

template <typename TO> __device__ __forceinline__ TO out_cast(float v) { return from_f32<TO>(v); }

}  // namespace

// w[ci][co][ky][kx] -> wp[cls][co][t][ci], cls = 2*py + px, t = 2*ty + tx, with
// ky = 3 - py - 2*ty and kx = 3 - px - 2*tx; rows co >= Cout (up to CoP) are zero.
template <typename T>
__global__ __launch_bounds__(256) void deconv_pack_kernel(const T *__restrict__ w, T *__restrict__ wp, int Cin,
                                                          int Cout, int CoP) {
    const long long total = 16ll * CoP * Cin;
    for (long long i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
        const int ci = (int)(i % Cin);
        long long r = i / Cin;
        const int t = (int)(r & 3);
        r >>= 2;
        const int co = (int)(r % CoP);
        const int cls = (int)(r / CoP);
        const int py = cls >> 1, px = cls & 1, ty = t >> 1, tx = t & 1;
        const int ky = 3 - py - 2 * ty, kx = 3 - px - 2 * tx;
        wp[i] = co < Cout ? w[((size_t)ci * Cout + co) * 16 + ky * 4 + kx] : from_f32<T>(0.0f);
    }
}

// Channel-last 16-bit input (Cin % 8 == 0, 16-byte aligned), packed weights. Block: 4
// waves, wave = parity class; tile = input row j of image n, input columns i0 .. i0+31,
// output channels co0 .. co0+31 (blockIdx.y).
template <typename T, typename TO, bool NCHW_OUT>
__global__ __launch_bounds__(256) void deconv_mfma_kernel(DeconvArgs a) {
    typedef typename Mfma32<T>::vec vec;
    __shared__ __attribute__((aligned(16))) T sx[2][DC_BUF];
    __shared__ float so[32][2][DC_OLD];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int py = wv >> 1, px = wv & 1;
    const int H = a.H, W = a.W, Cin = a.Cin, Cout = a.Cout;
    const int tiles_w = (W + DC_TW - 1) / DC_TW;
    int t = blockIdx.x;
    const int ib = t % tiles_w;
    t /= tiles_w;
    const int j = t % H, n = t / H;
    const int i0 = ib * DC_TW;
    const int co0 = blockIdx.y * 32;
    const T *__restrict__ x = static_cast<const T *>(a.x);

    // staging of one chunk: 3 rows x 34 pixels x 4 vectors of 8 channels, zero outside
    // the image and past Cin
    u32x4 st[2];
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = tid + 256 * q;
            const int r = idx / (DC_SPX * 4), rem = idx - r * (DC_SPX * 4);
            const int p = rem >> 2, cv = rem & 3;
            const int iy = j - 1 + r, ix = i0 - 1 + p, ci = c0 + cv * 8;
            const bool ok = idx < DC_VECS && (unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W && ci < Cin;
            st[q] = ok ? *reinterpret_cast<const u32x4 *>(x + (((size_t)n * H + iy) * W + ix) * Cin + ci)
                       : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = tid + 256 * q;
            if (idx < DC_VECS) {
                const int r = idx / (DC_SPX * 4), rem = idx - r * (DC_SPX * 4);
                const int p = rem >> 2, cv = rem & 3;
                *reinterpret_cast<u32x4 *>(&sx[buf][(r * DC_SPX + p) * DC_PS + cv * 8]) = st[q];
            }
        }
    };

    const int col = lane & 31, kq = (lane >> 5) * 8;
    const T *__restrict__ wrow =
        static_cast<const T *>(a.wp) + ((size_t)((2 * py + px) * a.CoP + co0 + col) * 4) * Cin;
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

    const int nch = (Cin + DC_KC - 1) / DC_KC;
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int c0 = c * DC_KC;
        if (c + 1 < nch) load_chunk(c0 + DC_KC);
        vec bw[4][2];
#pragma unroll
        for (int tp = 0; tp < 4; ++tp)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ci = c0 + h * 16 + kq;
                u32x4 v = ci < Cin ? *reinterpret_cast<const u32x4 *>(wrow + tp * Cin + ci) : u32x4{0u, 0u, 0u, 0u};
                __builtin_memcpy(&bw[tp][h], &v, 16);
            }
        const T *sb = sx[c & 1];
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) {
            const int ty = tp >> 1, tx = tp & 1;
            const T *pa = sb + ((py + ty) * DC_SPX + col + px + tx) * DC_PS + kq;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                vec av;
                __builtin_memcpy(&av, pa + h * 16, 16);
                acc = Mfma32<T>::run(av, bw[tp][h], acc);
            }
        }
        if (c + 1 < nch) store_chunk((c + 1) & 1);
        __syncthreads();
    }

    // epilogue: lane holds output channel co0 + col for the class pixels
    // p = 8*(i/4) + 4*(lane/32) + i%4; activated fp32 values go to an LDS tile
    // [channel][output row][output column] and leave in coalesced runs
    const int co = co0 + col;
    const float bv = (a.bias && co < Cout) ? a.bias[co] : 0.0f;
    const float av = (a.alpha && co < Cout) ? a.alpha[co] : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int p = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        so[col][py][2 * p + px] = activate(a.act, acc[i] + bv, av);
    }
    __syncthreads();
    TO *__restrict__ y = static_cast<TO *>(a.y);
    const int OH = 2 * H, OW = 2 * W;
    const int oc0 = 2 * i0;
    if constexpr (NCHW_OUT) {
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int e = tid + 256 * it;
            const int oc = e & 63, r = (e >> 6) & 1, cl = e >> 7;
            if (co0 + cl < Cout && oc0 + oc < OW)
                y[(((size_t)n * Cout + co0 + cl) * OH + 2 * j + r) * OW + oc0 + oc] = out_cast<TO>(so[cl][r][oc]);
        }
    } else {
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int e = tid + 256 * it;
            const int cl = e & 31, oc = (e >> 5) & 63, r = e >> 11;
            if (co0 + cl < Cout && oc0 + oc < OW)
                y[(((size_t)n * OH + 2 * j + r) * OW + oc0 + oc) * Cout + co0 + cl] = out_cast<TO>(so[cl][r][oc]);
        }
    }
}

// Any layout and storage type: one thread per output, the gather over the (at most)
// four contributing taps and all input channels, weights read in the caller's layout.
template <typename T, typename TO, bool NCHW>
__global__ __launch_bounds__(256) void deconv_direct_kernel(DeconvArgs a) {
    const int H = a.H, W = a.W, Cin = a.Cin, Cout = a.Cout, OH = 2 * H, OW = 2 * W;
    const long long total = (long long)a.N * OH * OW * Cout;
    const T *__restrict__ x = static_cast<const T *>(a.x);
    const T *__restrict__ w = static_cast<const T *>(a.w);
    TO *__restrict__ y = static_cast<TO *>(a.y);
    for (long long it = blockIdx.x * 256ll + threadIdx.x; it < total; it += (long long)gridDim.x * 256) {
        int n, co, oy, ox;
        if (NCHW) {
            ox = (int)(it % OW);
            long long q = it / OW;
            oy = (int)(q % OH);
            q /= OH;
            co = (int)(q % Cout);
            n = (int)(q / Cout);
        } else {
            co = (int)(it % Cout);
            long long q = it / Cout;
            ox = (int)(q % OW);
            q /= OW;
            oy = (int)(q % OH);
            n = (int)(q / OH);
        }
        const int py = oy & 1, px = ox & 1, j = oy >> 1, i = ox >> 1;
        float acc = 0.0f;
        for (int ty = 0; ty < 2; ++ty) {
            const int iy = j - 1 + py + ty;
            if ((unsigned)iy >= (unsigned)H) continue;
            const int ky = 3 - py - 2 * ty;
            for (int tx = 0; tx < 2; ++tx) {
                const int ix = i - 1 + px + tx;
                if ((unsigned)ix >= (unsigned)W) continue;
                const int kx = 3 - px - 2 * tx;
                const T *wc = w + (size_t)co * 16 + ky * 4 + kx;
                if (NCHW) {
                    const T *xc = x + (size_t)n * Cin * H * W + (size_t)iy * W + ix;
                    for (int ci = 0; ci < Cin; ++ci)
                        acc += to_f32(xc[(size_t)ci * H * W]) * to_f32(wc[(size_t)ci * Cout * 16]);
                } else {
                    const T *xc = x + (((size_t)n * H + iy) * W + ix) * Cin;
                    for (int ci = 0; ci < Cin; ++ci) acc += to_f32(xc[ci]) * to_f32(wc[(size_t)ci * Cout * 16]);
                }
            }
        }
        const float bv = a.bias ? a.bias[co] : 0.0f;
        const float av = a.alpha ? a.alpha[co] : 0.0f;
        y[it] = out_cast<TO>(activate(a.act, acc + bv, av));
    }
}

template <typename T>
static hipError_t pack_t(const void *w, void *wp, int Cin, int Cout, int CoP, hipStream_t st) {
    const long long total = 16ll * CoP * Cin;
    long long blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    return launch_kernel(deconv_pack_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const T *>(w),
                         static_cast<T *>(wp), Cin, Cout, CoP);
}

hipError_t launch_deconv_pack(const void *w, void *wp, int Cin, int Cout, int CoP, int dtype, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_BF16:
        return pack_t<bf16>(w, wp, Cin, Cout, CoP, st);
    case CONV2D_DTYPE_F16:
        return pack_t<f16>(w, wp, Cin, Cout, CoP, st);
    default:
        return hipErrorInvalidValue;
    }
}

template <typename T, typename TO>
static hipError_t mfma_t(const DeconvArgs &a, bool nchw_out, hipStream_t st) {
    const long long tiles = (long long)a.N * a.H * ((a.W + DC_TW - 1) / DC_TW);
    dim3 grid((unsigned)tiles, (unsigned)(a.CoP / 32));
    if (nchw_out) return launch_kernel(deconv_mfma_kernel<T, TO, true>, grid, dim3(256), 0, st, a);
    return launch_kernel(deconv_mfma_kernel<T, TO, false>, grid, dim3(256), 0, st, a);
}

hipError_t launch_deconv_mfma(const DeconvArgs &a, int dtype, bool out_f32, bool nchw_out, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_BF16:
        return out_f32 ? mfma_t<bf16, float>(a, nchw_out, st) : mfma_t<bf16, bf16>(a, nchw_out, st);
    case CONV2D_DTYPE_F16:
        return out_f32 ? mfma_t<f16, float>(a, nchw_out, st) : mfma_t<f16, f16>(a, nchw_out, st);
    default:
        return hipErrorInvalidValue;
    }
}

template <typename T, typename TO>
static hipError_t direct_t(const DeconvArgs &a, bool nchw, hipStream_t st) {
    const long long total = (long long)a.N * 4 * a.H * a.W * a.Cout;
    long long blocks = (total + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (nchw) return launch_kernel(deconv_direct_kernel<T, TO, true>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return launch_kernel(deconv_direct_kernel<T, TO, false>, dim3((unsigned)blocks), dim3(256), 0, st, a);
}

hipError_t launch_deconv_direct(const DeconvArgs &a, int dtype, bool out_f32, bool nchw, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_F32:
        return direct_t<float, float>(a, nchw, st);
    case CONV2D_DTYPE_BF16:
        return out_f32 ? direct_t<bf16, float>(a, nchw, st) : direct_t<bf16, bf16>(a, nchw, st);
    case CONV2D_DTYPE_F16:
        return out_f32 ? direct_t<f16, float>(a, nchw, st) : direct_t<f16, f16>(a, nchw, st);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace c2d
