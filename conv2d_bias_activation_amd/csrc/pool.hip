// 3x3/s2/p1 max pool and 2x2/s2 average pool (inferencelayer page, `MAXPOOL_SRC`
// and `AVGPOOL_SRC`). Both only move data: each output reads its window once and is
// written once, so the kernels are laid out for coalesced 16-byte accesses along
// channels (channel-last) or along the row (channel-first).
//
// Max: the largest in-range tap, compared in fp32 after an exact widening, so the
// stored value is bit-identical to an input (the first largest in row-major tap
// order; an all-NaN window gives -inf). Average: ((x00 + x01) + x10) + x11 in fp32,
// in that order, then times 0.25 and one rounding to the storage type.
#include "common.hpp"
#include "kernels.hpp"

namespace c2d {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buffer_rsrc_bytes(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

template <typename T> struct Vec16 {
    static constexpr int n = 16 / (int)sizeof(T);
    T v[16 / sizeof(T)];
};

template <typename T> __device__ __forceinline__ Vec16<T> load16(const T *p) {
    Vec16<T> r;
    u32x4 t = *reinterpret_cast<const u32x4 *>(p);
    __builtin_memcpy(r.v, &t, 16);
    return r;
}
template <typename T> __device__ __forceinline__ void store16(T *p, const Vec16<T> &r) {
    u32x4 t;
    __builtin_memcpy(&t, r.v, 16);
    *reinterpret_cast<u32x4 *>(p) = t;
}

// channel-last: blockIdx.y is an output row (n, oh), threads walk its (pixel, 16-byte
// channel vector) items; the nine taps are buffer loads (an out-of-image tap gets an
// out-of-range offset and is then ignored by the compare), all in flight together.
template <typename T>
__global__ __launch_bounds__(256) void maxpool_nhwc_vec(const T *__restrict__ x, T *__restrict__ y,
                                                        int N, int H, int W, int C, int OH, int OW) {
    constexpr int VE = Vec16<T>::n;
    const int CV = C / VE;
    const int item = blockIdx.x * 256 + threadIdx.x;
    if (item >= OW * CV) return;
    const int row = blockIdx.y;  // n * OH + oh
    const int n = row / OH, oh = row - n * OH;
    const int ow = item / CV, cv = item - ow * CV;
    const __amdgpu_buffer_rsrc_t rx = make_buffer_rsrc_bytes(x, (uint32_t)((size_t)N * H * W * C * sizeof(T)));
    u32x4 v[9];
    bool ok[9];
#pragma unroll
    for (int dy = 0; dy < 3; ++dy)
#pragma unroll
        for (int dx = 0; dx < 3; ++dx) {
            const int iy = 2 * oh + dy - 1, ix = 2 * ow + dx - 1;
            const bool in = (unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W;
            const uint32_t off = in ? (uint32_t)(((n * H + iy) * W + ix) * C + cv * VE) * (uint32_t)sizeof(T)
                                    : 0xFFFFFFF0u;
            v[dy * 3 + dx] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
            ok[dy * 3 + dx] = in;
        }
    float best[VE];
    Vec16<T> out;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        best[e] = -__builtin_inff();
        out.v[e] = from_f32<T>(-__builtin_inff());
    }
#pragma unroll
    for (int t = 0; t < 9; ++t) {
        T tv[VE];
        __builtin_memcpy(tv, &v[t], 16);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const float f = to_f32(tv[e]);
            const bool take = ok[t] && f > best[e];
            best[e] = take ? f : best[e];
            out.v[e] = take ? tv[e] : out.v[e];
        }
    }
    store16(y + ((size_t)row * OW + ow) * C + cv * VE, out);
}

// any layout, one thread per output element (channel-first: consecutive threads
// walk along the output row)
template <typename T, bool NCHW>
__global__ __launch_bounds__(256) void maxpool_scalar(const T *__restrict__ x, T *__restrict__ y,
                                                      int N, int H, int W, int C, int OH, int OW) {
    const long long total = (long long)N * OH * OW * C;
    for (long long it = blockIdx.x * 256ll + threadIdx.x; it < total; it += (long long)gridDim.x * 256) {
        int n, c, oh, ow;
        if (NCHW) {
            ow = (int)(it % OW);
            long long q = it / OW;
            oh = (int)(q % OH);
            q /= OH;
            c = (int)(q % C);
            n = (int)(q / C);
        } else {
            c = (int)(it % C);
            long long q = it / C;
            ow = (int)(q % OW);
            q /= OW;
            oh = (int)(q % OH);
            n = (int)(q / OH);
        }
        float best = -__builtin_inff();
        T out = from_f32<T>(-__builtin_inff());
        for (int dy = 0; dy < 3; ++dy) {
            int iy = 2 * oh + dy - 1;
            if ((unsigned)iy >= (unsigned)H) continue;
            for (int dx = 0; dx < 3; ++dx) {
                int ix = 2 * ow + dx - 1;
                if ((unsigned)ix >= (unsigned)W) continue;
                size_t off = NCHW ? (((size_t)n * C + c) * H + iy) * W + ix
                                  : (((size_t)n * H + iy) * W + ix) * C + c;
                T v = x[off];
                float f = to_f32(v);
                if (f > best) {
                    best = f;
                    out = v;
                }
            }
        }
        y[it] = out;
    }
}

// channel-last: blockIdx.y is an output row (n, oh), threads walk its (pixel, 16-byte
// channel vector) items (the window is always inside the image: OH = H/2, OW = W/2).
template <typename T>
__global__ __launch_bounds__(256) void avgpool_nhwc_vec(const T *__restrict__ x, T *__restrict__ y,
                                                        int N, int H, int W, int C, int OH, int OW) {
    constexpr int VE = Vec16<T>::n;
    const int CV = C / VE;
    const int item = blockIdx.x * 256 + threadIdx.x;
    if (item >= OW * CV) return;
    const int row = blockIdx.y;  // n * OH + oh
    const int n = row / OH, oh = row - n * OH;
    const int ow = item / CV, cv = item - ow * CV;
    const T *b = x + ((size_t)(n * H + 2 * oh) * W + 2 * ow) * C + cv * VE;
    Vec16<T> v00 = load16(b), v01 = load16(b + C);
    Vec16<T> v10 = load16(b + (size_t)W * C), v11 = load16(b + (size_t)W * C + C);
    Vec16<T> out;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        float s = to_f32(v00.v[e]) + to_f32(v01.v[e]);
        s = s + to_f32(v10.v[e]);
        s = s + to_f32(v11.v[e]);
        out.v[e] = from_f32<T>(s * 0.25f);
    }
    store16(y + ((size_t)row * OW + ow) * C + cv * VE, out);
}

template <typename T, bool NCHW>
__global__ __launch_bounds__(256) void avgpool_scalar(const T *__restrict__ x, T *__restrict__ y,
                                                      int N, int H, int W, int C, int OH, int OW) {
    const long long total = (long long)N * OH * OW * C;
    for (long long it = blockIdx.x * 256ll + threadIdx.x; it < total; it += (long long)gridDim.x * 256) {
        int n, c, oh, ow;
        if (NCHW) {
            ow = (int)(it % OW);
            long long q = it / OW;
            oh = (int)(q % OH);
            q /= OH;
            c = (int)(q % C);
            n = (int)(q / C);
        } else {
            c = (int)(it % C);
            long long q = it / C;
            ow = (int)(q % OW);
            q /= OW;
            oh = (int)(q % OH);
            n = (int)(q / OH);
        }
        size_t b, dx, dy;
        if (NCHW) {
            b = (((size_t)n * C + c) * H + 2 * oh) * W + 2 * ow;
            dx = 1;
            dy = W;
        } else {
            b = (((size_t)n * H + 2 * oh) * W + 2 * ow) * C + c;
            dx = C;
            dy = (size_t)W * C;
        }
        float s = to_f32(x[b]) + to_f32(x[b + dx]);
        s = s + to_f32(x[b + dy]);
        s = s + to_f32(x[b + dy + dx]);
        y[it] = from_f32<T>(s * 0.25f);
    }
}

static unsigned pool_grid(long long items) {
    long long g = (items + 255) / 256;
    const long long cap = 256 * 64;  // enough waves to fill 256 CUs; the loop strides the rest
    return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

template <typename T>
static hipError_t maxpool_t(const void *x, void *y, int N, int H, int W, int C, bool nchw,
                            bool vec, hipStream_t st) {
    int OH = (H - 1) / 2 + 1, OW = (W - 1) / 2 + 1;
    const T *xp = static_cast<const T *>(x);
    T *yp = static_cast<T *>(y);
    // the vector kernel takes one output row per grid row and 32-bit byte offsets
    if (!nchw && vec && (long long)N * OH <= 65535 && (long long)N * H * W * C * (long long)sizeof(T) < (1ll << 31)) {
        const int per_row = OW * (C / Vec16<T>::n);
        return launch_kernel(maxpool_nhwc_vec<T>, dim3((unsigned)((per_row + 255) / 256), (unsigned)(N * OH)),
                             dim3(256), 0, st, xp, yp, N, H, W, C, OH, OW);
    } else if (nchw) {
        return launch_kernel(maxpool_scalar<T, true>, dim3(pool_grid((long long)N * OH * OW * C)), dim3(256), 0,
                             st, xp, yp, N, H, W, C, OH, OW);
    } else {
        return launch_kernel(maxpool_scalar<T, false>, dim3(pool_grid((long long)N * OH * OW * C)), dim3(256), 0,
                             st, xp, yp, N, H, W, C, OH, OW);
    }
}

template <typename T>
static hipError_t avgpool_t(const void *x, void *y, int N, int H, int W, int C, bool nchw,
                            bool vec, hipStream_t st) {
    int OH = H / 2, OW = W / 2;
    const T *xp = static_cast<const T *>(x);
    T *yp = static_cast<T *>(y);
    if (!nchw && vec && (long long)N * OH <= 65535 && OW > 0) {
        const int per_row = OW * (C / Vec16<T>::n);
        return launch_kernel(avgpool_nhwc_vec<T>, dim3((unsigned)((per_row + 255) / 256), (unsigned)(N * OH)),
                             dim3(256), 0, st, xp, yp, N, H, W, C, OH, OW);
    } else if (nchw) {
        return launch_kernel(avgpool_scalar<T, true>, dim3(pool_grid((long long)N * OH * OW * C)), dim3(256), 0,
                             st, xp, yp, N, H, W, C, OH, OW);
    } else {
        return launch_kernel(avgpool_scalar<T, false>, dim3(pool_grid((long long)N * OH * OW * C)), dim3(256), 0,
                             st, xp, yp, N, H, W, C, OH, OW);
    }
}

hipError_t launch_maxpool(const void *x, void *y, int N, int H, int W, int C, bool nchw, int dtype,
                          bool vec, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_F32:
        return maxpool_t<float>(x, y, N, H, W, C, nchw, vec, st);
    case CONV2D_DTYPE_BF16:
        return maxpool_t<bf16>(x, y, N, H, W, C, nchw, vec, st);
    case CONV2D_DTYPE_F16:
        return maxpool_t<f16>(x, y, N, H, W, C, nchw, vec, st);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_avgpool(const void *x, void *y, int N, int H, int W, int C, bool nchw, int dtype,
                          bool vec, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_F32:
        return avgpool_t<float>(x, y, N, H, W, C, nchw, vec, st);
    case CONV2D_DTYPE_BF16:
        return avgpool_t<bf16>(x, y, N, H, W, C, nchw, vec, st);
    case CONV2D_DTYPE_F16:
        return avgpool_t<f16>(x, y, N, H, W, C, nchw, vec, st);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace c2d
