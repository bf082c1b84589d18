// Nearest-neighbour 2x upsample and per-pixel channel concat, the data-movement steps
// of the inferencelayer page's CCFM neck (`UPSAMPLE_SRC`, `CONCAT_SRC`): the top-down
// path upsamples a lateral conv's output and concatenates it, channels first, with a
// backbone map. One kernel does all three calls:
//
//   y[n, oy, ox, c] = c < Ca ? a[n, oy >> up, ox >> up, c] : b[n, oy, ox, c - Ca]
//
// with up = 1 for an upsample (Cb = 0, no b) or the fused upsample + concat, and
// up = 0 for a plain concat. Fusing the two saves writing the upsampled map and
// reading it back (4 * |a| bytes each way). Values are copied, never converted.
#include "common.hpp"
#include "kernels.hpp"

namespace c2d {

// channel-last, 16-byte vectors: Ca and Cb multiples of the vector, pointers aligned.
// Grid rows walk the output rows (n, oy); threads walk a row's (pixel, vector) items.
template <typename T>
__global__ __launch_bounds__(256) void cat_nhwc_vec(const T *__restrict__ a, const T *__restrict__ b,
                                                    T *__restrict__ y, int rows, int H, int W, int Ca, int Cb,
                                                    int up) {
    constexpr int VE = 16 / (int)sizeof(T);
    const int CVa = Ca / VE, CV = (Ca + Cb) / VE;
    const int item = blockIdx.x * 256 + threadIdx.x;
    if (item >= W * CV) return;
    const int ox = item / CV, cv = item - ox * CV;
    for (int row = blockIdx.y; row < rows; row += gridDim.y) {
        const int n = row / H, oy = row - n * H;
        const T *src;
        if (cv < CVa) {
            const int ah = H >> up, aw = W >> up;
            src = a + (((size_t)n * ah + (oy >> up)) * aw + (ox >> up)) * Ca + (size_t)cv * VE;
        } else {
            src = b + ((size_t)row * W + ox) * Cb + (size_t)(cv - CVa) * VE;
        }
        *reinterpret_cast<u32x4 *>(y + ((size_t)row * W + ox) * (Ca + Cb) + (size_t)cv * VE) =
            *reinterpret_cast<const u32x4 *>(src);
    }
}

// channel-first planes: plane (n, c) of y is plane c of a (upsampled when up) or plane
// c - Ca of b. With up == 0 and H*W a multiple of the vector (aligned pointers), each
// thread moves 16 bytes; otherwise one element.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void cat_nchw(const T *__restrict__ a, const T *__restrict__ b, T *__restrict__ y,
                                                int planes, int H, int W, int Ca, int Cb, int up) {
    constexpr int VE = VEC ? 16 / (int)sizeof(T) : 1;
    const int C = Ca + Cb;
    const int HW = H * W;
    const int items = HW / VE;
    for (int plane = blockIdx.y; plane < planes; plane += gridDim.y)  // plane = n * C + c
    for (int item = blockIdx.x * 256 + threadIdx.x; item < items; item += gridDim.x * 256) {
        const int n = plane / C, c = plane - n * C;
        T *yp = y + (size_t)plane * HW;
        if constexpr (VEC) {
            const T *src = c < Ca ? a + ((size_t)n * Ca + c) * HW : b + ((size_t)n * Cb + (c - Ca)) * HW;
            reinterpret_cast<u32x4 *>(yp)[item] = reinterpret_cast<const u32x4 *>(src)[item];
        } else {
            const int oy = item / W, ox = item - oy * W;
            T v;
            if (c < Ca) {
                const int ah = H >> up, aw = W >> up;
                v = a[(((size_t)n * Ca + c) * ah + (oy >> up)) * aw + (ox >> up)];
            } else {
                v = b[((size_t)n * Cb + (c - Ca)) * HW + item];
            }
            yp[item] = v;
        }
    }
}

// any channel count, channel-last: one element per thread
template <typename T>
__global__ __launch_bounds__(256) void cat_nhwc_scalar(const T *__restrict__ a, const T *__restrict__ b,
                                                       T *__restrict__ y, int rows, int H, int W, int Ca, int Cb,
                                                       int up) {
    const int C = Ca + Cb;
    for (int row = blockIdx.y; row < rows; row += gridDim.y)
    for (int item = blockIdx.x * 256 + threadIdx.x; item < W * C; item += gridDim.x * 256) {
        const int n = row / H, oy = row - n * H;
        const int ox = item / C, c = item - ox * C;
        T v;
        if (c < Ca) {
            const int ah = H >> up, aw = W >> up;
            v = a[(((size_t)n * ah + (oy >> up)) * aw + (ox >> up)) * Ca + c];
        } else {
            v = b[((size_t)row * W + ox) * Cb + (c - Ca)];
        }
        y[(size_t)row * W * C + item] = v;
    }
}

template <typename T>
static hipError_t cat_t(const void *a, const void *b, void *y, int N, int H, int W, int Ca, int Cb, int up,
                        bool nchw, bool vec, hipStream_t st) {
    const T *pa = static_cast<const T *>(a);
    const T *pb = static_cast<const T *>(b);
    T *py = static_cast<T *>(y);
    const int C = Ca + Cb;
    // grid rows are capped at 65535 (the kernels stride over the rest)
    auto gy = [](int rows) { return (unsigned)(rows < 65535 ? rows : 65535); };
    if (!nchw) {
        const int rows = N * H;
        if (vec) {
            const int items = W * (C / (16 / (int)sizeof(T)));
            dim3 grid((unsigned)((items + 255) / 256), gy(rows));
            return launch_kernel(cat_nhwc_vec<T>, grid, dim3(256), 0, st, pa, pb, py, rows, H, W, Ca, Cb, up);
        }
        int bx = (W * C + 255) / 256;
        if (bx > 64) bx = 64;
        return launch_kernel(cat_nhwc_scalar<T>, dim3((unsigned)bx, gy(rows)), dim3(256), 0, st, pa, pb, py, rows, H,
                             W, Ca, Cb, up);
    }
    const int planes = N * C;
    const int items = vec ? H * W / (16 / (int)sizeof(T)) : H * W;
    int bx = (items + 255) / 256;
    if (bx > 64) bx = 64;
    dim3 grid((unsigned)bx, gy(planes));
    if (vec) return launch_kernel(cat_nchw<T, true>, grid, dim3(256), 0, st, pa, pb, py, planes, H, W, Ca, Cb, up);
    return launch_kernel(cat_nchw<T, false>, grid, dim3(256), 0, st, pa, pb, py, planes, H, W, Ca, Cb, up);
}

hipError_t launch_concat(const void *a, const void *b, void *y, int N, int H, int W, int Ca, int Cb, bool up,
                         bool nchw, int dtype, bool vec, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_F32:
        return cat_t<float>(a, b, y, N, H, W, Ca, Cb, up ? 1 : 0, nchw, vec, st);
    case CONV2D_DTYPE_BF16:
        return cat_t<bf16>(a, b, y, N, H, W, Ca, Cb, up ? 1 : 0, nchw, vec, st);
    case CONV2D_DTYPE_F16:
        return cat_t<f16>(a, b, y, N, H, W, Ca, Cb, up ? 1 : 0, nchw, vec, st);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace c2d
