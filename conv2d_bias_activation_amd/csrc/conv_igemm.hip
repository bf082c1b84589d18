// Implicit-GEMM convolution on CDNA4 matrix cores (MFMA), general shapes.
//
// The layer is a GEMM C[m, co] = sum_k A[m, k] * B[k, co] with m an output pixel
// (n, oh, ow), k a (tap, input channel) pair and B the weight (inferencelayer page,
// `conv()`: im2col then `enc_gemm3` with bias + activation in the epilogue). Here
// the im2col matrix A is never written: each K step gathers its BM x 32 slice of
// patches straight from the input into LDS (zero for out-of-range taps), the
// weight slice [BN x 32] is read as stored, and matrix-core instructions consume
// both from LDS. The epilogue (bias, residual, activation, rounding) runs on the
// fp32 accumulators after a pass through LDS that makes the output stores
// coalesced.
//
// K order follows the weight layout so that B is a plain row-major [Cout][K]
// matrix: channel-last (OHWI) weights give k = (ky*kw + kx)*Cin + ci, the pages'
// (dy, dx, c) order; channel-first (OIHW) weights give k = (ci*kh + ky)*kw + kx.
#include "igemm_common.hpp"
#include "kernels.hpp"

namespace c2d {


// T: storage type. BM x BN tile per 256-thread workgroup, waves arranged WGM x WGN.
// NCHW: channel-first layout. AVEC: channel-last with Cin a multiple of the 16-byte
// vector, so each (pixel, tap) channel run is loaded 16 bytes at a time.
// BVEC: K a multiple of the vector, so weight rows load 16 bytes at a time.
template <typename T, int BM, int BN, int WGM, int WGN, bool NCHW, bool AVEC, bool BVEC>
__global__ __launch_bounds__(256) void igemm_kernel(ConvArgs a, int tiles_n) {
    constexpr int BK = 32;
    constexpr int VE = 16 / (int)sizeof(T);
    constexpr int KPL = Mfma<T>::KPL;
    constexpr int KSTEP = 4 * KPL;
    constexpr int FM = BM / (16 * WGM);
    constexpr int FN = BN / (16 * WGN);
    static_assert(FM >= 1 && FN >= 1 && WGM * WGN == 4, "tile shape");
    constexpr int LDK = BK + VE;  // padded LDS row, in elements
    constexpr int STAGE = (BM + BN) * LDK;
    constexpr int LDC = BN + 4;
    constexpr int SMEM = cmax<2 * STAGE * (int)sizeof(T), BM * LDC * 4>::v;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];
    T *sAB = reinterpret_cast<T *>(smem);
    float *sC = reinterpret_cast<float *>(smem);

    const T *__restrict__ x = static_cast<const T *>(a.x);
    const T *__restrict__ w = static_cast<const T *>(a.w);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wm = wid % WGM, wn = wid / WGM;

    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int m0 = (tile / tiles_n) * BM;
    const int n0 = (tile % tiles_n) * BN;

    const int H = a.H, W = a.W, Cin = a.Cin, kh = a.kh, kw = a.kw;
    const int OHW = a.OH * a.OW;
    const int K = a.K;
    const int nsteps = (K + BK - 1) / BK;

    // ---------------- A (patch) loader state ----------------
    constexpr int KV = BK / VE;              // 16-byte vectors per A/B row slice
    constexpr int NAV = (BM * KV + 255) / 256;
    constexpr int NAS = (BM * BK + 255) / 256;
    // vector path (channel-last): fixed k-vector column per thread
    const int kv = tid % KV;
    int a_img[NAV], a_ih[NAV], a_iw[NAV];
    bool a_ok[NAV];
    int ci_s = 0, kx_s = 0, ky_s = 0;
    // scalar path: fixed row per thread
    int s_img = 0, s_ih = 0, s_iw = 0;
    bool s_ok = false;
    if constexpr (AVEC) {
#pragma unroll
        for (int v = 0; v < NAV; ++v) {
            int idx = tid + v * 256;
            int m = m0 + idx / KV;
            a_ok[v] = idx < BM * KV && m < a.M;
            int mm = a_ok[v] ? m : 0;
            int n = mm / OHW, pix = mm - n * OHW;
            int oh = pix / a.OW, ow = pix - oh * a.OW;
            a_img[v] = n * H * W * Cin;
            a_ih[v] = oh * a.stride - a.pad;
            a_iw[v] = ow * a.stride - a.pad;
        }
        int k = kv * VE;
        int tap = k / Cin;
        ci_s = k - tap * Cin;
        ky_s = tap / kw;
        kx_s = tap - ky_s * kw;
    } else {
        int m = m0 + tid % BM;
        s_ok = m < a.M;
        int mm = s_ok ? m : 0;
        int n = mm / OHW, pix = mm - n * OHW;
        int oh = pix / a.OW, ow = pix - oh * a.OW;
        s_img = NCHW ? n * Cin * H * W : n * H * W * Cin;
        s_ih = oh * a.stride - a.pad;
        s_iw = ow * a.stride - a.pad;
    }

    constexpr int NBV = (BN * KV + 255) / 256;
    constexpr int NBS = (BN * BK + 255) / 256;
    u32x4 ra[AVEC ? NAV : 1];
    T rs[AVEC ? 1 : NAS];
    u32x4 rb[BVEC ? NBV : 1];
    T rbs[BVEC ? 1 : NBS];

    auto load_global = [&](int step) {
        const int k0 = step * BK;
        if constexpr (AVEC) {
            const bool kin = ky_s < kh;
#pragma unroll
            for (int v = 0; v < NAV; ++v) {
                int iy = a_ih[v] + ky_s, ix = a_iw[v] + kx_s;
                bool ok = a_ok[v] && kin && (unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W;
                u32x4 z = {0u, 0u, 0u, 0u};
                ra[v] = ok ? *reinterpret_cast<const u32x4 *>(x + a_img[v] + (iy * W + ix) * Cin + ci_s)
                           : z;
            }
            ci_s += BK;
            while (ci_s >= Cin) {
                ci_s -= Cin;
                if (++kx_s == kw) {
                    kx_s = 0;
                    ++ky_s;
                }
            }
        } else {
            const int taps = kh * kw;
#pragma unroll
            for (int e = 0; e < NAS; ++e) {
                int kcol = tid / BM + e * (256 / BM);
                int k = k0 + kcol;
                T v = from_f32<T>(0.0f);
                if (s_ok && k < K) {
                    int ci, ky, kx;
                    if constexpr (NCHW) {
                        ci = k / taps;
                        int r = k - ci * taps;
                        ky = r / kw;
                        kx = r - ky * kw;
                    } else {
                        int tap = k / Cin;
                        ci = k - tap * Cin;
                        ky = tap / kw;
                        kx = tap - ky * kw;
                    }
                    int iy = s_ih + ky, ix = s_iw + kx;
                    if ((unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W)
                        v = NCHW ? x[s_img + (ci * H + iy) * W + ix]
                                 : x[s_img + (iy * W + ix) * Cin + ci];
                }
                rs[e] = v;
            }
        }
        if constexpr (BVEC) {
#pragma unroll
            for (int v = 0; v < NBV; ++v) {
                int idx = tid + v * 256;
                int col = idx / KV, kk = k0 + (idx % KV) * VE;
                bool ok = idx < BN * KV && n0 + col < a.Cout && kk < K;
                u32x4 z = {0u, 0u, 0u, 0u};
                rb[v] = ok ? *reinterpret_cast<const u32x4 *>(w + (size_t)(n0 + col) * K + kk) : z;
            }
        } else {
#pragma unroll
            for (int e = 0; e < NBS; ++e) {
                int idx = tid + e * 256;
                int col = idx / BK, kk = k0 + idx % BK;
                bool ok = idx < BN * BK && n0 + col < a.Cout && kk < K;
                rbs[e] = ok ? w[(size_t)(n0 + col) * K + kk] : from_f32<T>(0.0f);
            }
        }
    };

    auto store_lds = [&](int buf) {
        T *sA = sAB + buf * STAGE;
        T *sB = sA + BM * LDK;
        if constexpr (AVEC) {
#pragma unroll
            for (int v = 0; v < NAV; ++v) {
                int idx = tid + v * 256;
                if (idx < BM * KV)
                    *reinterpret_cast<u32x4 *>(sA + (idx / KV) * LDK + kv * VE) = ra[v];
            }
        } else {
#pragma unroll
            for (int e = 0; e < NAS; ++e) {
                int kcol = tid / BM + e * (256 / BM);
                sA[(tid % BM) * LDK + kcol] = rs[e];
            }
        }
        if constexpr (BVEC) {
#pragma unroll
            for (int v = 0; v < NBV; ++v) {
                int idx = tid + v * 256;
                if (idx < BN * KV)
                    *reinterpret_cast<u32x4 *>(sB + (idx / KV) * LDK + (idx % KV) * VE) = rb[v];
            }
        } else {
#pragma unroll
            for (int e = 0; e < NBS; ++e) {
                int idx = tid + e * 256;
                if (idx < BN * BK) sB[(idx / BK) * LDK + idx % BK] = rbs[e];
            }
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    typedef typename Mfma<T>::vec vec;
    auto compute = [&](int buf) {
        const T *sA = sAB + buf * STAGE;
        const T *sB = sA + BM * LDK;
#pragma unroll
        for (int ks = 0; ks < BK / KSTEP; ++ks) {
            vec fa[FM], fb[FN];
            const int kof = ks * KSTEP + (lane >> 4) * KPL;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const vec *>(sA + (wm * FM * 16 + i * 16 + (lane & 15)) * LDK + kof);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[j] = *reinterpret_cast<const vec *>(sB + (wn * FN * 16 + j * 16 + (lane & 15)) * LDK + kof);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = Mfma<T>::run(fa[i], fb[j], acc[i][j]);
        }
    };

    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        const bool more = s + 1 < nsteps;
        if (more) load_global(s + 1);
        compute(s & 1);
        if (more) store_lds((s + 1) & 1);
        __syncthreads();
    }

    // ---------------- epilogue ----------------
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int row = wm * FM * 16 + i * 16 + (lane >> 4) * 4 + r;
                int col = wn * FN * 16 + j * 16 + (lane & 15);
                sC[row * LDC + col] = acc[i][j][r];
            }
    __syncthreads();

    store_tile<T, BM, BN, LDC, NCHW>(sC, a, m0, n0, tid);
}

template <typename T, int BM, int BN, int WGM, int WGN, bool NCHW, bool AVEC, bool BVEC>
static hipError_t launch_igemm_t(const ConvArgs &a, hipStream_t st) {
    int tiles_m = (a.M + BM - 1) / BM;
    int tiles_n = (a.Cout + BN - 1) / BN;
    long long g = (long long)tiles_m * tiles_n;
    if (g > 0x7fffffff) return hipErrorInvalidValue;
    return launch_kernel(igemm_kernel<T, BM, BN, WGM, WGN, NCHW, AVEC, BVEC>, dim3((unsigned)g), dim3(256), 0, st,
                         a, tiles_n);
}

template <typename T, int BM, int BN, int WGM, int WGN>
static hipError_t launch_igemm_tile(const ConvArgs &a, bool nchw, bool avec, bool bvec,
                                    hipStream_t st) {
    if (nchw) {
        if (bvec) return launch_igemm_t<T, BM, BN, WGM, WGN, true, false, true>(a, st);
        return launch_igemm_t<T, BM, BN, WGM, WGN, true, false, false>(a, st);
    }
    if (avec) return launch_igemm_t<T, BM, BN, WGM, WGN, false, true, true>(a, st);
    if (bvec) return launch_igemm_t<T, BM, BN, WGM, WGN, false, false, true>(a, st);
    return launch_igemm_t<T, BM, BN, WGM, WGN, false, false, false>(a, st);
}

template <typename T>
static hipError_t launch_igemm_dtype(const ConvArgs &a, const IgemmPlan &p, hipStream_t st) {
    switch (p.tile) {
    case IGEMM_TILE_128x128:
        return launch_igemm_tile<T, 128, 128, 2, 2>(a, p.nchw, p.avec, p.bvec, st);
    case IGEMM_TILE_128x64:
        return launch_igemm_tile<T, 128, 64, 2, 2>(a, p.nchw, p.avec, p.bvec, st);
    case IGEMM_TILE_64x64:
        return launch_igemm_tile<T, 64, 64, 2, 2>(a, p.nchw, p.avec, p.bvec, st);
    case IGEMM_TILE_256x32:
        return launch_igemm_tile<T, 256, 32, 4, 1>(a, p.nchw, p.avec, p.bvec, st);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_igemm(const ConvArgs &a, int dtype, const IgemmPlan &p, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_BF16:
        return launch_igemm_dtype<bf16>(a, p, st);
    case CONV2D_DTYPE_F16:
        return launch_igemm_dtype<f16>(a, p, st);
    case CONV2D_DTYPE_F32:
        return launch_igemm_dtype<float>(a, p, st);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace c2d
