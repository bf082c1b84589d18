// Pieces shared by the matrix-core convolution kernels.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace c2d {

// One 16x16 output block per instruction; every lane holds KPL consecutive k of
// one A row (lane % 16) and one B column (lane % 16); lane / 16 picks which KPL-run
// of the instruction's 4*KPL k values. The fp32 result: lane holds rows
// 4*(lane/16) + i, i < 4, of column lane % 16.
template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
    static constexpr int KPL = 8;
    typedef __bf16 vec __attribute__((ext_vector_type(8)));
    __device__ static f32x4 run(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<f16> {
    static constexpr int KPL = 8;
    typedef _Float16 vec __attribute__((ext_vector_type(8)));
    __device__ static f32x4 run(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static constexpr int KPL = 1;
    typedef float vec;
    __device__ static f32x4 run(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// 32x32 output block per instruction, K = 16 (gfx950: twice the rate of the
// 16x16x32 form). A operand: lane holds A[lane % 32][8*(lane/32) .. +8]; B operand:
// B[8*(lane/32) .. +8][lane % 32]; the 16 fp32 results of lane l are rows
// 8*(i/4) + 4*(l/32) + (i%4), i < 16, of column l % 32.
template <typename T> struct Mfma32;
template <> struct Mfma32<bf16> {
    typedef __bf16 vec __attribute__((ext_vector_type(8)));
    __device__ static f32x16 run(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma32<f16> {
    typedef _Float16 vec __attribute__((ext_vector_type(8)));
    __device__ static f32x16 run(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <int A, int B> struct cmax { static constexpr int v = A > B ? A : B; };

// Epilogue of a BM x BN output tile whose fp32 sums sit in LDS (sC, row stride LDC,
// rows = output pixels m0.., columns = output channels n0..): bias, residual,
// activation and one rounding to T, stored with 16-byte accesses where the layout
// allows (channel-last: along channels; channel-first: along pixels of one plane).
template <typename T, int BM, int BN, int LDC, bool NCHW>
__device__ __forceinline__ void store_tile(const float *sC, const ConvArgs &a, int m0, int n0,
                                           int tid) {
    constexpr int VE = 16 / (int)sizeof(T);
    const int OHW = a.OH * a.OW;
    const T *__restrict__ res = static_cast<const T *>(a.res);
    T *__restrict__ y = static_cast<T *>(a.y);
    const bool has_res = res != nullptr;
    const bool pre = a.res_before_act != 0;
    const int act = a.act;
    const int Cout = a.Cout;

    if constexpr (!NCHW) {
        if ((Cout % VE) == 0 && a.vec_out) {
            // Each thread keeps one 16-byte column chunk for all its rows: the bias and
            // slopes are read once and all residual loads are issued before the math.
            constexpr int CV = BN / VE;
            static_assert(256 % CV == 0, "column chunks per row divide the block");
            constexpr int RSTEP = 256 / CV;
            constexpr int NIT = (BM + RSTEP - 1) / RSTEP;
            const int cv = tid % CV, row0 = tid / CV;
            const int co = n0 + cv * VE;
            if (co < Cout) {
                float bv[VE], av[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    bv[e] = a.bias ? a.bias[co + e] : 0.0f;
                    av[e] = a.alpha ? a.alpha[co + e] : 0.0f;
                }
                u32x4 rr[NIT];
#pragma unroll
                for (int it = 0; it < NIT; ++it) {
                    const int row = row0 + it * RSTEP, m = m0 + row;
                    rr[it] = u32x4{0u, 0u, 0u, 0u};
                    if (has_res && row < BM && m < a.M)
                        rr[it] = *reinterpret_cast<const u32x4 *>(res + (size_t)m * Cout + co);
                }
#pragma unroll
                for (int it = 0; it < NIT; ++it) {
                    const int row = row0 + it * RSTEP, m = m0 + row;
                    if (row >= BM || m >= a.M) continue;
                    T rv[VE], out[VE];
                    __builtin_memcpy(rv, &rr[it], 16);
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        float r = has_res ? to_f32(rv[e]) : 0.0f;
                        out[e] = round_fp32<T>(epilogue(sC[row * LDC + cv * VE + e], bv[e], av[e], r, has_res, act, pre));
                    }
                    u32x4 t;
                    __builtin_memcpy(&t, out, 16);
                    *reinterpret_cast<u32x4 *>(y + (size_t)m * Cout + co) = t;
                }
            }
        } else {
            for (int it = tid; it < BM * BN; it += 256) {
                int row = it / BN, col = it % BN;
                int m = m0 + row, co = n0 + col;
                if (m >= a.M || co >= Cout) continue;
                size_t o = (size_t)m * Cout + co;
                float b = a.bias ? a.bias[co] : 0.0f;
                float al = a.alpha ? a.alpha[co] : 0.0f;
                float r = has_res ? to_f32(res[o]) : 0.0f;
                y[o] = round_fp32<T>(epilogue(sC[row * LDC + col], b, al, r, has_res, act, pre));
            }
        }
    } else {
        constexpr int RV = BM / VE;
        const bool plane_aligned = (OHW % VE) == 0 && a.vec_out;
        for (int it = tid; it < BN * RV; it += 256) {
            int col = it / RV, rv = it % RV;
            int co = n0 + col, mb = m0 + rv * VE;
            if (co >= Cout || mb >= a.M) continue;
            float b = a.bias ? a.bias[co] : 0.0f;
            float al = a.alpha ? a.alpha[co] : 0.0f;
            int n = mb / OHW, pix = mb - n * OHW;
            size_t o = ((size_t)n * Cout + co) * OHW + pix;
            if (plane_aligned && (pix % VE) == 0 && mb + VE <= a.M) {
                // the VE pixels are consecutive in one plane and 16-byte aligned
                T rvv[VE];
                if (has_res) {
                    u32x4 t = *reinterpret_cast<const u32x4 *>(res + o);
                    __builtin_memcpy(rvv, &t, 16);
                }
                T out[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    float r = has_res ? to_f32(rvv[e]) : 0.0f;
                    out[e] = round_fp32<T>(epilogue(sC[(rv * VE + e) * LDC + col], b, al, r, has_res, act, pre));
                }
                u32x4 t;
                __builtin_memcpy(&t, out, 16);
                *reinterpret_cast<u32x4 *>(y + o) = t;
            } else {
                for (int e = 0; e < VE; ++e) {
                    int m = mb + e;
                    if (m >= a.M) break;
                    int n2 = m / OHW, pix2 = m - n2 * OHW;
                    size_t o2 = ((size_t)n2 * Cout + co) * OHW + pix2;
                    float r = has_res ? to_f32(res[o2]) : 0.0f;
                    y[o2] = round_fp32<T>(epilogue(sC[(rv * VE + e) * LDC + col], b, al, r, has_res, act, pre));
                }
            }
        }
    }
}

// Fused epilogue of one wave's (FM*16) x (FN*16) accumulator block, channel-last
// output. acc holds the 16x16 matrix-core layout (lane: rows 4*(lane/16) + r of
// column lane % 16 of every block); `slice` is the wave's own 16 x WLD floats of LDS.
// Block row by block row, the sums go through the slice so that each lane reads
// back a 16-byte run along the output channels: bias and slopes are loaded once per
// lane, residuals and outputs move 16 bytes at a time. Rows mrow0.., columns ncol0...
template <typename T, int FM, int FN, int WLD>
__device__ __forceinline__ void wave_epilogue_nhwc(const f32x4 (&acc)[FM][FN], float *slice,
                                                   const ConvArgs &a, int mrow0, int ncol0,
                                                   int lane) {
    constexpr int VE = 16 / (int)sizeof(T);
    constexpr int WN = FN * 16;
    constexpr int CPR = WN / VE;  // 16-byte runs per row
    static_assert(64 % CPR == 0, "runs per row divide the wave");
    constexpr int RPP = 64 / CPR;  // rows per pass of the wave
    constexpr int NP = (16 + RPP - 1) / RPP;
    const T *__restrict__ res = static_cast<const T *>(a.res);
    T *__restrict__ y = static_cast<T *>(a.y);
    const bool has_res = res != nullptr, pre = a.res_before_act != 0;
    const int act = a.act, Cout = a.Cout;
    const int rl = lane & 15, kq = lane >> 4;
    const int cc = lane % CPR, rsub = lane / CPR;
    const int co = ncol0 + cc * VE;
    const bool vec = a.vec_out && (Cout % VE) == 0;
    float bv[VE], av[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        const bool in = co + e < Cout;
        bv[e] = (a.bias && in) ? a.bias[co + e] : 0.0f;
        av[e] = (a.alpha && in) ? a.alpha[co + e] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) slice[(kq * 4 + r) * WLD + j * 16 + rl] = acc[i][j][r];
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's slice writes are done
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = rsub + p * RPP;
            const int m = mrow0 + i * 16 + row;
            if (row >= 16 || m >= a.M || co >= Cout) continue;
            const float *src = slice + row * WLD + cc * VE;
            const size_t o = (size_t)m * Cout + co;
            if (vec) {
                T rv[VE], out[VE];
                if (has_res) {
                    u32x4 t = *reinterpret_cast<const u32x4 *>(res + o);
                    __builtin_memcpy(rv, &t, 16);
                }
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    float r = has_res ? to_f32(rv[e]) : 0.0f;
                    out[e] = round_fp32<T>(epilogue(src[e], bv[e], av[e], r, has_res, act, pre));
                }
                u32x4 t;
                __builtin_memcpy(&t, out, 16);
                *reinterpret_cast<u32x4 *>(y + o) = t;
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    if (co + e >= Cout) break;
                    float r = has_res ? to_f32(res[o + e]) : 0.0f;
                    y[o + e] = round_fp32<T>(epilogue(src[e], bv[e], av[e], r, has_res, act, pre));
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
    }
}

// VE-wide epilogue with the activation fixed at compile time (the caller switches on
// the runtime code once, outside the element loops).
template <typename T, int ACT, int VE>
__device__ __forceinline__ void epilogue_vec(const float *v, const float *bv, const float *av,
                                             const T *rv, bool has_res, bool pre, T *out) {
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        float x = v[e] + bv[e];
        const float r = has_res ? to_f32(rv[e]) : 0.0f;
        x += pre ? r : 0.0f;
        if (ACT == CONV2D_ACT_RELU) x = x > 0.0f ? x : 0.0f;
        if (ACT == CONV2D_ACT_SILU) x = x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
        if (ACT == CONV2D_ACT_PRELU) x = x >= 0.0f ? x : av[e] * x;
        x += pre ? 0.0f : r;
        out[e] = round_fp32<T>(x);
    }
}

// Raw buffer descriptors (untyped, stride 0; word 3 as used by gfx9-family GPUs). An
// access whose offset lies past `bytes` does nothing: loads return zeros and stores
// are dropped. A null base with 0 bytes gives a descriptor that reads only zeros.
constexpr uint32_t kOOB = 0xFFFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

// The same descriptor as four words, for the direct-to-LDS load below.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void *p, uint32_t bytes) {
    const uint64_t a = (uint64_t)p;
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Direct-to-LDS 16-byte buffer load: lane i's 16 bytes from `voff` land at LDS address
// lds + 16*i (lds must be wave-uniform). Issued as inline assembly so that the
// compiler, which cannot tell which LDS bytes such a load writes, does not drain every
// outstanding load before each later LDS read: the caller owns the vmcnt waits and
// barriers that order these loads before the reads of their data.
// The compiler also does not see that this is a vector-memory instruction reading the
// descriptor SGPRs and M0, so it inserts none of the wait states that such a read needs
// after a VALU write of those SGPRs (5 on gfx9: an SGPR spill reloaded by v_readlane
// just before made the load use a stale descriptor) or after an SALU write of M0 (1):
// the s_nop 4 in front provides them.
__device__ __forceinline__ void dma_b128(i32x4 rsrc, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}

// Fused epilogue of one wave's (FM*32) x (FN*32) block of 32x32 matrix-core
// accumulators, channel-last output (rows mrow0.. are pixels, columns ncol0.. output
// channels). Phase 1 touches only LDS: 16 rows at a time go through the wave's
// `slice` (16 x WLD floats) and come back as VE-wide runs along the channels, kept
// in registers. Phase 2 touches only global memory, with buffer instructions whose
// out-of-range offsets the hardware ignores, so there are no per-element branches:
// bias and slopes once per lane, then every residual load, then the math and the
// 16-byte stores, all in flight together. `out_bytes` bounds y (and the residual).
// With `part` non-null the wave stores its fp32 sums there instead ([M][Cout] fp32,
// one K slice of a split-K launch) and applies nothing; a separate pass adds the
// slices and runs the epilogue.
//
// `rowof(r)` maps the wave's local row r (0 <= r < FM*32) to its output pixel m, or -1
// for a row that has no pixel (past the end of the map or of a tile row). `mid()` runs
// after every global load of the epilogue has been issued and before the first store.
template <typename T, int FM, int FN, int WLD, typename RowOf, typename Mid>
__device__ __forceinline__ void wave_epilogue_nhwc32_rows(const f32x16 (&acc)[FM][FN], float *slice,
                                                          const ConvArgs &a, RowOf rowof, int ncol0,
                                                          int lane, uint32_t out_bytes, float *part,
                                                          Mid mid) {
    constexpr int VE = 16 / (int)sizeof(T);
    constexpr int WN = FN * 32;
    constexpr int CPR = WN / VE;  // VE-wide runs per row
    static_assert(64 % CPR == 0 && CPR <= 16, "runs per row");
    constexpr int RPP = 64 / CPR;  // rows per pass of the wave (>= 4)
    constexpr int NP = 16 / RPP;   // passes per 16 rows
    static_assert(16 % RPP == 0, "passes cover 16 rows");
    constexpr int NH = FM * 2;     // 16-row halves
    const int col = lane & 31, hi = lane >> 5;
    const int cc = lane % CPR, rsub = lane / CPR;

    float v[NH][NP][VE];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 2; ++g)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        slice[(g * 8 + hi * 4 + r) * WLD + j * 32 + col] = acc[i][j][(2 * h + g) * 4 + r];
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's slice writes landed
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const float *src = slice + (rsub + p * RPP) * WLD + cc * VE;
#pragma unroll
                for (int e = 0; e < VE; e += 4) {
                    f32x4 t = *reinterpret_cast<const f32x4 *>(src + e);
                    v[i * 2 + h][p][e] = t[0];
                    v[i * 2 + h][p][e + 1] = t[1];
                    v[i * 2 + h][p][e + 2] = t[2];
                    v[i * 2 + h][p][e + 3] = t[3];
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
        }

    const int Cout = a.Cout;
    const int co = ncol0 + cc * VE;
    if (part) {
        // split-K slice: raw fp32 sums (only used when Cout % VE == 0)
        mid();
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(part, (uint32_t)((size_t)a.M * Cout * 4));
#pragma unroll
        for (int q = 0; q < NH; ++q)
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int m = rowof(q * 16 + rsub + p * RPP);
                const uint32_t o = (m >= 0 && co < Cout) ? ((uint32_t)m * (uint32_t)Cout + (uint32_t)co) * 4u : kOOB;
#pragma unroll
                for (int e = 0; e < VE; e += 4) {
                    u32x4 t = __builtin_bit_cast(u32x4, f32x4{v[q][p][e], v[q][p][e + 1], v[q][p][e + 2], v[q][p][e + 3]});
                    __builtin_amdgcn_raw_buffer_store_b128(t, rp, (int)(o == kOOB ? kOOB : o + e * 4u), 0, 0);
                }
            }
        return;
    }
    const bool has_res = a.res != nullptr, pre = a.res_before_act != 0;
    const bool vec = a.vec_out && (Cout % VE) == 0;
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(a.bias, a.bias ? (uint32_t)Cout * 4u : 0u);
    const __amdgpu_buffer_rsrc_t ralpha = make_rsrc(a.alpha, a.alpha ? (uint32_t)Cout * 4u : 0u);
    const __amdgpu_buffer_rsrc_t rres = make_rsrc(a.res, has_res ? out_bytes : 0u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, out_bytes);
    float bv[VE], av[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        const uint32_t off = co + e < Cout ? (uint32_t)(co + e) * 4u : kOOB;
        bv[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rbias, (int)off, 0, 0));
        av[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ralpha, (int)off, 0, 0));
    }
    // element offset of each run (or kOOB past the last pixel / channel)
    uint32_t off[NH][NP];
#pragma unroll
    for (int q = 0; q < NH; ++q)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int m = rowof(q * 16 + rsub + p * RPP);
            off[q][p] = (m >= 0 && co < Cout) ? ((uint32_t)m * (uint32_t)Cout + (uint32_t)co) * (uint32_t)sizeof(T)
                                              : kOOB;
        }
    T rv[NH][NP][VE];
#pragma unroll
    for (int q = 0; q < NH; ++q)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (vec) {
                u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rres, (int)off[q][p], 0, 0);
                __builtin_memcpy(rv[q][p], &t, 16);
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const uint32_t o = (off[q][p] != kOOB && co + e < Cout) ? off[q][p] + e * (uint32_t)sizeof(T) : kOOB;
                    uint16_t u = 0;
                    if constexpr (sizeof(T) == 2) u = __builtin_amdgcn_raw_buffer_load_b16(rres, (int)o, 0, 0);
                    __builtin_memcpy(&rv[q][p][e], &u, sizeof(T));
                }
            }
        }
    mid();
    auto finish = [&](auto act_tag) {
        constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
        for (int q = 0; q < NH; ++q)
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                T out[VE];
                epilogue_vec<T, ACT, VE>(v[q][p], bv, av, rv[q][p], has_res, pre, out);
                if (vec) {
                    u32x4 t;
                    __builtin_memcpy(&t, out, 16);
                    __builtin_amdgcn_raw_buffer_store_b128(t, ry, (int)off[q][p], 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        const uint32_t o = (off[q][p] != kOOB && co + e < Cout) ? off[q][p] + e * (uint32_t)sizeof(T) : kOOB;
                        uint16_t u;
                        __builtin_memcpy(&u, &out[e], 2);
                        __builtin_amdgcn_raw_buffer_store_b16(u, ry, (int)o, 0, 0);
                    }
                }
            }
    };
    switch (a.act) {
    case CONV2D_ACT_RELU:
        finish(std::integral_constant<int, CONV2D_ACT_RELU>{});
        break;
    case CONV2D_ACT_SILU:
        finish(std::integral_constant<int, CONV2D_ACT_SILU>{});
        break;
    case CONV2D_ACT_PRELU:
        finish(std::integral_constant<int, CONV2D_ACT_PRELU>{});
        break;
    default:
        finish(std::integral_constant<int, CONV2D_ACT_NONE>{});
        break;
    }
}

// Rows mrow0, mrow0+1, ... of the GEMM (pixels in order); rows at or past M have none.
template <typename T, int FM, int FN, int WLD>
__device__ __forceinline__ void wave_epilogue_nhwc32(const f32x16 (&acc)[FM][FN], float *slice,
                                                     const ConvArgs &a, int mrow0, int ncol0,
                                                     int lane, uint32_t out_bytes,
                                                     float *part = nullptr) {
    const int M = a.M;
    wave_epilogue_nhwc32_rows<T, FM, FN, WLD>(
        acc, slice, a, [=](int r) { return mrow0 + r < M ? mrow0 + r : -1; }, ncol0, lane, out_bytes, part,
        [] {});
}

// The same epilogue for channel-first output (y and the residual are [N][Cout][OH*OW]):
// each lane reads back one output channel over 8 consecutive pixels, which are one
// 16-byte run of an output plane when OH*OW is a multiple of 8 (runs start at pixels
// that are multiples of 8, so they never cross a plane). Otherwise every element is
// addressed on its own.
template <typename T, int FM, int FN, int WLD>
__device__ __forceinline__ void wave_epilogue_nchw32(const f32x16 (&acc)[FM][FN], float *slice,
                                                     const ConvArgs &a, int mrow0, int ncol0,
                                                     int lane, uint32_t out_bytes) {
    static_assert(sizeof(T) == 2, "16-bit storage");
    constexpr int WN = FN * 32;
    constexpr int NH = FM * 2;
    const int col = lane & 31, hi = lane >> 5;
    float v[NH][FN][8];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 2; ++g)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        slice[(g * 8 + hi * 4 + r) * WLD + j * 32 + col] = acc[i][j][(2 * h + g) * 4 + r];
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int t = 0; t < FN; ++t) {
                const int idx = lane + 64 * t, c = idx % WN, rg = idx / WN;
#pragma unroll
                for (int r = 0; r < 8; ++r) v[i * 2 + h][t][r] = slice[(rg * 8 + r) * WLD + c];
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
        }

    const bool has_res = a.res != nullptr, pre = a.res_before_act != 0;
    const int Cout = a.Cout, OHW = a.OH * a.OW;
    const bool vec = a.vec_out && (OHW % 8) == 0;
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(a.bias, a.bias ? (uint32_t)Cout * 4u : 0u);
    const __amdgpu_buffer_rsrc_t ralpha = make_rsrc(a.alpha, a.alpha ? (uint32_t)Cout * 4u : 0u);
    const __amdgpu_buffer_rsrc_t rres = make_rsrc(a.res, has_res ? out_bytes : 0u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, out_bytes);
    float bv[FN], av[FN];
    uint32_t off[NH][FN];
    T rv[NH][FN][8];
#pragma unroll
    for (int t = 0; t < FN; ++t) {
        const int idx = lane + 64 * t, co = ncol0 + idx % WN;
        const uint32_t bo = co < Cout ? (uint32_t)co * 4u : kOOB;
        bv[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rbias, (int)bo, 0, 0));
        av[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ralpha, (int)bo, 0, 0));
    }
#pragma unroll
    for (int q = 0; q < NH; ++q)
#pragma unroll
        for (int t = 0; t < FN; ++t) {
            const int idx = lane + 64 * t, co = ncol0 + idx % WN;
            const int m = mrow0 + q * 16 + (idx / WN) * 8;
            const int n = m / OHW, pix = m - n * OHW;
            off[q][t] = (m < a.M && co < Cout)
                            ? (((uint32_t)n * (uint32_t)Cout + (uint32_t)co) * (uint32_t)OHW + (uint32_t)pix) * 2u
                            : kOOB;
            if (vec) {
                u32x4 tt = __builtin_amdgcn_raw_buffer_load_b128(rres, (int)off[q][t], 0, 0);
                __builtin_memcpy(rv[q][t], &tt, 16);
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int mr = m + r, nr = mr / OHW, pr = mr - nr * OHW;
                    const uint32_t o = (mr < a.M && co < Cout)
                        ? (((uint32_t)nr * (uint32_t)Cout + (uint32_t)co) * (uint32_t)OHW + (uint32_t)pr) * 2u
                        : kOOB;
                    uint16_t u = __builtin_amdgcn_raw_buffer_load_b16(rres, (int)o, 0, 0);
                    __builtin_memcpy(&rv[q][t][r], &u, 2);
                }
            }
        }
    auto finish = [&](auto act_tag) {
        constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
        for (int q = 0; q < NH; ++q)
#pragma unroll
            for (int t = 0; t < FN; ++t) {
                float b8[8], a8[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    b8[r] = bv[t];
                    a8[r] = av[t];
                }
                T out[8];
                epilogue_vec<T, ACT, 8>(v[q][t], b8, a8, rv[q][t], has_res, pre, out);
                if (vec) {
                    u32x4 tt;
                    __builtin_memcpy(&tt, out, 16);
                    __builtin_amdgcn_raw_buffer_store_b128(tt, ry, (int)off[q][t], 0, 0);
                } else {
                    const int idx = lane + 64 * t, co = ncol0 + idx % WN;
                    const int m = mrow0 + q * 16 + (idx / WN) * 8;
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const int mr = m + r, nr = mr / OHW, pr = mr - nr * OHW;
                        const uint32_t o = (mr < a.M && co < Cout)
                            ? (((uint32_t)nr * (uint32_t)Cout + (uint32_t)co) * (uint32_t)OHW + (uint32_t)pr) * 2u
                            : kOOB;
                        uint16_t u;
                        __builtin_memcpy(&u, &out[r], 2);
                        __builtin_amdgcn_raw_buffer_store_b16(u, ry, (int)o, 0, 0);
                    }
                }
            }
    };
    switch (a.act) {
    case CONV2D_ACT_RELU:
        finish(std::integral_constant<int, CONV2D_ACT_RELU>{});
        break;
    case CONV2D_ACT_SILU:
        finish(std::integral_constant<int, CONV2D_ACT_SILU>{});
        break;
    case CONV2D_ACT_PRELU:
        finish(std::integral_constant<int, CONV2D_ACT_PRELU>{});
        break;
    default:
        finish(std::integral_constant<int, CONV2D_ACT_NONE>{});
        break;
    }
}

}  // namespace c2d
