// Shared device helpers of the fused conv2d library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#include "../../include/conv2d_fused.h"

namespace c2d {

// Launches kernel k and returns that launch's own status, not the thread's sticky last
// error (which can still hold an earlier, unrelated failure of the host program).
template <typename... P>
inline hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, size_t smem, hipStream_t st,
                                std::type_identity_t<P>... args) {
    void *ptrs[] = {static_cast<void *>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, ptrs, smem, st);
}

typedef __bf16 bf16;
typedef _Float16 f16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Everything a conv kernel needs, passed by value.
struct ConvArgs {
    const void *x;
    const void *w;
    const float *bias;   // may be null
    const float *alpha;  // may be null unless PReLU
    const void *res;     // may be null
    void *y;
    int N, H, W, Cin, Cout, kh, kw, stride, pad, OH, OW;
    int M;    // N*OH*OW output pixels (GEMM rows)
    int K;    // Cin*kh*kw (GEMM depth)
    int act;  // CONV2D_ACT_* (low byte only)
    int res_before_act;
    int w_ohwi;  // channel-first layer whose weights are given channel-last (OHWI)
    int vec_out;  // y and residual are 16-byte aligned
    void *y2;     // channel-first output: also written channel-last here (no residual), or null
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(f16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
// Casts to the 16-bit types round to nearest-even (gfx950 v_cvt_pk_bf16_f32 and
// v_cvt_f16_f32 under the default rounding mode).
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float v) { return (f16)v; }

// x, the fp32 result of an epilogue, rounded once to T. The empty asm makes x an fp32
// value first: otherwise this compiler may fold a multiply that produced x into the
// conversion (v_fma_mix*), rounding the exact product to T instead of the fp32 product,
// which can differ in the last place from another kernel's epilogue of the same sums.
// Epilogues whose outputs must match bit for bit (a fused conv + pool and the two-call
// path) all round through here.
template <typename T> __device__ __forceinline__ T round_fp32(float x) {
    asm volatile("" : "+v"(x));
    return from_f32<T>(x);
}

// Activation of the epilogue: ReLU, SiLU v/(1+exp(-v)) or per-channel PReLU.
__device__ __forceinline__ float activate(int act, float v, float alpha) {
    switch (act) {
    case CONV2D_ACT_RELU:
        return v > 0.0f ? v : 0.0f;
    case CONV2D_ACT_SILU:
        // exp(-v) overflows to +inf for v < -88, giving v * 0 = -0: the exact value
        // there is below 1e-36 in magnitude.
        return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
    case CONV2D_ACT_PRELU:
        return v >= 0.0f ? v : alpha * v;
    default:
        return v;
    }
}

// The same activation with the code fixed at compile time, for epilogues that select it
// once (a switch outside the loop over their values) rather than per value.
template <int ACT> __device__ __forceinline__ float activate_c(float v, float alpha) {
    if constexpr (ACT == CONV2D_ACT_RELU) return v > 0.0f ? v : 0.0f;
    if constexpr (ACT == CONV2D_ACT_SILU) return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
    if constexpr (ACT == CONV2D_ACT_PRELU) return v >= 0.0f ? v : alpha * v;
    return v;
}

// bias, residual (before or after the activation) and activation of one output.
__device__ __forceinline__ float epilogue(float acc, float bias, float alpha, float r,
                                          bool has_res, int act, bool res_before) {
    float v = acc + bias;
    if (has_res && res_before) v += r;
    v = activate(act, v, alpha);
    if (has_res && !res_before) v += r;
    return v;
}

// The max pool's comparison (inferencelayer page, `MAXPOOL_SRC`: `v > best` from the
// padding value): of a, b, c taken in that order, starting from -inf, a later value
// replaces the running one only when strictly greater, so NaN is skipped, three NaN give
// -inf, and of equal values (-0 and +0) the first stays.
__device__ __forceinline__ float first_max3(float a, float b, float c) {
    float m = -__builtin_inff();
    m = a > m ? a : m;
    m = b > m ? b : m;
    m = c > m ? c : m;
    return m;
}

// Maps a hardware workgroup id to a logical tile id so that each of the 8 XCDs
// (which take workgroups round-robin and each own an L2) runs one contiguous run
// of logical tiles, which then share input rows and weights in that L2.
__device__ __forceinline__ int xcd_remap(int g, int total) {
    const int nx = 8;
    int q = total / nx, r = total % nx;
    int x = g % nx, i = g / nx;
    return x * q + (x < r ? x : r) + i;
}

}  // namespace c2d
