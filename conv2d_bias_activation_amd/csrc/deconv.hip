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
// each class is a GEMM with K = 4*Cin over 64-channel chunks. The weights are first
// repacked (once per call, into the library scratch) in the order in which the kernel's
// lanes take them as MFMA B operands, so that each wave-wide weight load reads one
// contiguous kilobyte; a workgroup stages the input rows its tile's taps reach (the
// tile's one or two rows and one above and below) over a 34-pixel strip once, and its
// four waves (one per class) read shifted views of it.
#include <type_traits>

#include "common.hpp"
#include "igemm_common.hpp"
#include "kernels.hpp"

namespace c2d {

namespace {

constexpr int DC_TW = 32;           // input columns per tile
constexpr int DC_MR = 2;            // input rows per tile: a wave's 32-pixel blocks that share each weight load
constexpr int DC_ROWS = DC_MR + 2;  // staged rows j0 - 1 .. j0 + DC_MR
constexpr int DC_KC = 64;           // input channels per staged chunk
constexpr int DC_SPX = DC_TW + 2;   // staged columns i0 - 1 .. i0 + 32
constexpr int DC_PS = DC_KC + 8;    // LDS elements per staged pixel: 144 bytes, an odd number of
                                    // 16-byte slots, so 32 lanes reading 32 pixels hit distinct banks
constexpr int DC_BUF = DC_ROWS * DC_SPX * DC_PS;
constexpr int DC_VECS = DC_ROWS * DC_SPX * (DC_KC / 8);  // 16-byte vectors per chunk, channel-last (1088)
constexpr int DC_VQ = (DC_VECS + 255) / 256;             // per thread (5)
constexpr int DC_ELEMS = DC_ROWS * DC_SPX * DC_KC;       // elements per chunk, channel-first (8704)
constexpr int DC_EQ = (DC_ELEMS + 255) / 256;            // per thread (34)
constexpr int DC_KS = DC_KC / 16;                   // 16-deep MFMA steps per tap and chunk
// Staging lanes past the chunk's last vector or element store into a pad after the
// buffer, so every lane stores and no load is sunk into a branch (where its wait would
// be vmcnt(0)).
constexpr int DC_PAD = (256 * DC_VQ - DC_VECS) * 8 > 256 * DC_EQ - DC_ELEMS ? (256 * DC_VQ - DC_VECS) * 8
                                                                             : 256 * DC_EQ - DC_ELEMS;
constexpr int DC_BUFA = DC_BUF + DC_PAD;  // allocated elements per buffer
constexpr int DC_OLD = 2 * DC_TW + 2;               // output tile row in LDS: 64 columns + 2 pad
// output tile in LDS: per channel 2*DC_MR rows of DC_OLD floats plus one word, so the
// channel stride (265 words) is odd and the 32 lanes that hold 32 channels of one pixel
// write and read 32 different banks
constexpr int DC_OCS = 2 * DC_MR * DC_OLD + 1;

template <typename TO> __device__ __forceinline__ TO out_cast(float v) { return from_f32<TO>(v); }

// Buffer resource over `bytes` bytes: a load at an offset past the end returns zero, so
// padding taps and channel tails are loads like any other (no branch around them, which
// would make the compiler wait for every load in flight at the join).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_bytes(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOob = 0xFFFFFFF0u;  // an offset past the end of any buffer under 2^31 bytes

}  // namespace

// w[ci][co][ky][kx] -> wp in MFMA operand order: for class cls = 2*py + px, 32-channel
// output block cob, 64-channel input chunk c, tap t = 2*ty + tx (ky = 3 - py - 2*ty,
// kx = 3 - px - 2*tx) and 16-deep step ks, one 1 KiB run of 64 lanes x 8 channels:
// lane (h << 5) | col holds w[ci][co] for co = 32*cob + col and
// ci = 64*c + 16*ks + 8*h .. +8. Channels past Cin and outputs past Cout are zero, so
// the kernel's weight loads need no bounds. One thread per (co, ci) pair of the padded
// ranges reads that pair's 16 contiguous taps.
template <typename T>
__global__ __launch_bounds__(256) void deconv_pack_kernel(const T *__restrict__ w, T *__restrict__ wp, int Cin,
                                                          int Cout, int CoP, int CinP) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= CoP * CinP) return;
    const int ci = i % CinP, co = i / CinP;
    const bool in = ci < Cin && co < Cout;
    T tap[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) tap[k] = in ? w[((size_t)ci * Cout + co) * 16 + k] : from_f32<T>(0.0f);
    const int cob = co >> 5, col = co & 31;
    const int c = ci >> 6, ks = (ci >> 4) & 3, h = (ci >> 3) & 1, e = ci & 7;
    const int nch = CinP >> 6, ncob = CoP >> 5;
#pragma unroll
    for (int cls = 0; cls < 4; ++cls)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int py = cls >> 1, px = cls & 1, ty = t >> 1, tx = t & 1;
            const int ky = 3 - py - 2 * ty, kx = 3 - px - 2 * tx;
            const size_t run = (((size_t)(cls * ncob + cob) * nch + c) * 4 + t) * 4 + ks;
            wp[run * 512 + ((h << 5) | col) * 8 + e] = tap[ky * 4 + kx];
        }
}

// 16-bit input with Cin % 8 == 0 (channel-last: 16-byte aligned; channel-first: read
// straight from the planes and transposed while staging), packed weights. Block: 4
// waves, wave = parity class; tile = input rows j0, j0 + 1 of image n, input columns
// i0 .. i0+31, output channels co0 .. co0+31 (blockIdx.y): each wave computes two
// 32-pixel blocks (one per input row) with every weight operand it loads. The K loop
// runs over 64-channel chunks with the next chunk's input and weight loads in flight
// during the current chunk's products.
template <typename T, typename TO, bool NCHW>
__global__ __launch_bounds__(256) void deconv_mfma_kernel(DeconvArgs a) {
    typedef typename Mfma32<T>::vec vec;
    __shared__ __attribute__((aligned(16))) T sx[2][DC_BUFA];
    __shared__ float so[32 * DC_OCS];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int py = wv >> 1, px = wv & 1;
    const int H = a.H, W = a.W, Cin = a.Cin, Cout = a.Cout;
    const int tiles_w = (W + DC_TW - 1) / DC_TW;
    int t = blockIdx.x;
    const int ib = t % tiles_w;
    t /= tiles_w;
    const int tiles_h = (H + DC_MR - 1) / DC_MR;
    const int j0 = (t % tiles_h) * DC_MR, n = t / tiles_h;
    const int i0 = ib * DC_TW;
    const int co0 = blockIdx.y * 32;
    const T *__restrict__ x = static_cast<const T *>(a.x);

    // staging registers of one chunk: 4 rows x 34 pixels x 64 channels, zero outside the
    // image and past Cin
    u32x4 sv[NCHW ? 1 : DC_VQ];
    T se[NCHW ? DC_EQ : 1];
    const __amdgpu_buffer_rsrc_t rx = rsrc_bytes(x, a.x_bytes);
    auto load_chunk = [&](int c0) {
        if constexpr (NCHW) {
            // element e: pixel fastest (coalesced along the plane row), then row, channel
#pragma unroll
            for (int q = 0; q < DC_EQ; ++q) {
                const int e = tid + 256 * q;
                const int p = e % DC_SPX, rc = e / DC_SPX;
                const int r = rc % DC_ROWS, cl = rc / DC_ROWS;
                const int iy = j0 - 1 + r, ix = i0 - 1 + p, ci = c0 + cl;
                const bool ok = e < DC_ELEMS && (unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W && ci < Cin;
                const uint32_t off = ok ? ((((uint32_t)n * Cin + ci) * H + iy) * W + ix) * 2u : kOob;
                const unsigned short v = __builtin_amdgcn_raw_buffer_load_b16(rx, (int)off, 0, 0);
                __builtin_memcpy(&se[q], &v, 2);
            }
        } else {
#pragma unroll
            for (int q = 0; q < DC_VQ; ++q) {
                const int idx = tid + 256 * q;
                const int r = idx / (DC_SPX * 8), rem = idx - r * (DC_SPX * 8);
                const int p = rem >> 3, cv = rem & 7;
                const int iy = j0 - 1 + r, ix = i0 - 1 + p, ci = c0 + cv * 8;
                const bool ok = idx < DC_VECS && (unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W && ci < Cin;
                const uint32_t off = ok ? ((((uint32_t)n * H + iy) * W + ix) * Cin + ci) * 2u : kOob;
                sv[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
            }
        }
    };
    auto store_chunk = [&](int buf) {
        if constexpr (NCHW) {
#pragma unroll
            for (int q = 0; q < DC_EQ; ++q) {
                const int e = tid + 256 * q;
                const int p = e % DC_SPX, rc = e / DC_SPX;
                const int r = rc % DC_ROWS, cl = rc / DC_ROWS;
                sx[buf][e < DC_ELEMS ? (r * DC_SPX + p) * DC_PS + cl : DC_BUF + (e - DC_ELEMS)] = se[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < DC_VQ; ++q) {
                const int idx = tid + 256 * q;
                const int r = idx / (DC_SPX * 8), rem = idx - r * (DC_SPX * 8);
                const int p = rem >> 3, cv = rem & 7;
                const int at = idx < DC_VECS ? (r * DC_SPX + p) * DC_PS + cv * 8 : DC_BUF + (idx - DC_VECS) * 8;
                *reinterpret_cast<u32x4 *>(&sx[buf][at]) = sv[q];
            }
        }
    };

    const int col = lane & 31, kq = (lane >> 5) * 8;
    // B operands of one chunk: tap tp, 16-deep step ks; this lane's 16 bytes of each
    // 1 KiB run (the past-the-end prefetch after the last chunk reads zero)
    const __amdgpu_buffer_rsrc_t rw = rsrc_bytes(a.wp, a.wp_bytes);
    const int nchp = (Cin + DC_KC - 1) / DC_KC;
    const uint32_t wbase = (uint32_t)(((2 * py + px) * (a.CoP >> 5) + blockIdx.y) * nchp) * (16u * 1024u) + lane * 16u;
    u32x4 bw[4 * DC_KS];
    auto load_b = [&](int c) {
        const uint32_t cb = wbase + (uint32_t)c * (16u * 1024u);
#pragma unroll
        for (int i = 0; i < 4 * DC_KS; ++i)
            bw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(c < nchp ? cb + i * 1024u : kOob), 0, 0);
    };
    f32x16 acc[DC_MR];
#pragma unroll
    for (int m = 0; m < DC_MR; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;

    const int nch = (Cin + DC_KC - 1) / DC_KC;
    load_chunk(0);
    load_b(0);
    store_chunk(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int c0 = c * DC_KC;
        // this chunk's weights leave the prefetch registers before the next loads land
        // there; the next chunk's loads are issued unconditionally (past the last chunk
        // every channel is out of range and reads zero)
        vec bcur[4 * DC_KS];
#pragma unroll
        for (int i = 0; i < 4 * DC_KS; ++i) __builtin_memcpy(&bcur[i], &bw[i], 16);
        load_chunk(c0 + DC_KC);
        load_b(c + 1);
        const T *sb = sx[c & 1];
        // consecutive products alternate between the two pixel blocks' accumulators, so
        // each waits on the one two instructions back rather than the one just issued
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) {
            const int ty = tp >> 1, tx = tp & 1;
#pragma unroll
            for (int ks = 0; ks < DC_KS; ++ks)
#pragma unroll
                for (int m = 0; m < DC_MR; ++m) {
                    vec av;
                    __builtin_memcpy(&av, sb + ((m + py + ty) * DC_SPX + col + px + tx) * DC_PS + kq + ks * 16, 16);
                    acc[m] = Mfma32<T>::run(av, bcur[tp * DC_KS + ks], acc[m]);
                }
        }
        store_chunk((c + 1) & 1);
        __syncthreads();
    }

    // epilogue: lane holds output channel co0 + col for the class pixels
    // p = 8*(i/4) + 4*(lane/32) + i%4; activated fp32 values go to an LDS tile
    // [channel][output row][output column] and leave in coalesced runs
    const int co = co0 + col;
    const float bv = (a.bias && co < Cout) ? a.bias[co] : 0.0f;
    const float av = (a.alpha && co < Cout) ? a.alpha[co] : 0.0f;
    // the activation is chosen once, outside the loop over the 32 values
    auto epi = [&](auto actc) {
        constexpr int ACT = decltype(actc)::value;
#pragma unroll
        for (int m = 0; m < DC_MR; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int p = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                so[col * DC_OCS + (2 * m + py) * DC_OLD + 2 * p + px] = activate_c<ACT>(acc[m][i] + bv, av);
            }
    };
    switch (a.act) {
    case CONV2D_ACT_RELU: epi(std::integral_constant<int, CONV2D_ACT_RELU>{}); break;
    case CONV2D_ACT_SILU: epi(std::integral_constant<int, CONV2D_ACT_SILU>{}); break;
    case CONV2D_ACT_PRELU: epi(std::integral_constant<int, CONV2D_ACT_PRELU>{}); break;
    default: epi(std::integral_constant<int, CONV2D_ACT_NONE>{}); break;
    }
    __syncthreads();
    // output rows 2*j0 .. 2*j0 + 2*DC_MR - 1 (local row lr), columns 2*i0 .. +63
    TO *__restrict__ y = static_cast<TO *>(a.y);
    const int OH = 2 * H, OW = 2 * W;
    const int oc0 = 2 * i0, or0 = 2 * j0;
    if constexpr (NCHW) {
#pragma unroll 4
        for (int it = 0; it < 16 * DC_MR; ++it) {
            const int e = tid + 256 * it;
            const int oc = e & 63, lr = (e >> 6) & (2 * DC_MR - 1), cl = e / (128 * DC_MR);
            if (co0 + cl < Cout && oc0 + oc < OW && or0 + lr < OH)
                y[(((size_t)n * Cout + co0 + cl) * OH + or0 + lr) * OW + oc0 + oc] = out_cast<TO>(so[cl * DC_OCS + lr * DC_OLD + oc]);
        }
    } else {
#pragma unroll 4
        for (int it = 0; it < 16 * DC_MR; ++it) {
            const int e = tid + 256 * it;
            const int cl = e & 31, oc = (e >> 5) & 63, lr = e >> 11;
            if (co0 + cl < Cout && oc0 + oc < OW && or0 + lr < OH)
                y[(((size_t)n * OH + or0 + lr) * OW + oc0 + oc) * Cout + co0 + cl] = out_cast<TO>(so[cl * DC_OCS + lr * DC_OLD + oc]);
        }
    }
}

// 16-bit input with Cin % 8 == 0 and Cin <= 256, packed weights: the same tiles and
// products as deconv_mfma_kernel, but the whole strip (4 rows x 34 pixels x every input
// channel) is staged in LDS at once with 16-byte loads, so a workgroup waits for one
// round of input loads instead of one per 64-channel chunk. The input is channel-last
// (16-byte aligned; for a channel-first layer, its channel-last copy) or, with NCHW_IN,
// the caller's channel-first planes (W % 8 == 0, 16-byte aligned), transposed while they
// are staged. y channel-first (NCHW_OUT) or channel-last.
constexpr int DA_CMAX = 256;                                  // input channels staged at most
constexpr int DA_PSMAX = DA_CMAX + 8;                         // LDS elements per pixel at most
// channel-first staging: 8-pixel segments i0-8+8s (s < 6) cover the strip's pixels i0-1 .. i0+32
constexpr int DA_NSEG = 6;

template <typename T, typename TO, bool NCHW_OUT, bool NCHW_IN, int MR>
__global__ __launch_bounds__(256) void deconv_mfma_all_kernel(DeconvArgs a) {
    // MR input rows per tile (2, or 1 when the 2-row tiles leave CUs idle); ROWS staged rows
    constexpr int ROWS = MR + 2;
    constexpr int OCS = 2 * MR * DC_OLD + 1;  // epilogue tile channel stride (odd)
    constexpr int VQ = (ROWS * DC_SPX * (DA_CMAX / 8) + 255) / 256;  // 16-byte vectors per thread (17 at MR 2)
    constexpr int PQ = (DA_CMAX / 2 * ROWS * DA_NSEG + 255) / 256;   // plane work items per thread (12 at MR 2)
    typedef typename Mfma32<T>::vec vec;
    // the staged strip; its tail also receives the stores of lanes past the last vector
    __shared__ __attribute__((aligned(16))) T sx[ROWS * DC_SPX * DA_PSMAX + 256 * 8];
    __shared__ float so[32 * OCS];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int py = wv >> 1, px = wv & 1;
    const int H = a.H, W = a.W, Cin = a.Cin, Cout = a.Cout;
    const int tiles_w = (W + DC_TW - 1) / DC_TW;
    int t = blockIdx.x;
    const int ib = t % tiles_w;
    t /= tiles_w;
    const int tiles_h = (H + MR - 1) / MR;
    const int j0 = (t % tiles_h) * MR, n = t / tiles_h;
    const int i0 = ib * DC_TW;
    const int co0 = blockIdx.y * 32;
    const int nchp = (Cin + DC_KC - 1) / DC_KC;
    const int CinP = nchp * DC_KC;        // staged channels: zero past Cin
    const int PS = CinP + 8;              // LDS elements per pixel (an odd number of 16-byte slots)
    const int CV = CinP / 8;              // 16-byte vectors per pixel
    const int nvec = ROWS * DC_SPX * CV;

    // every input load of the strip in flight at once (out-of-range offsets read zero)
    const __amdgpu_buffer_rsrc_t rx = rsrc_bytes(a.x, a.x_bytes);
    u32x4 sv[NCHW_IN ? 1 : VQ];
    // channel-first: work item (channel pair cp, strip row r, segment sg) loads 8 pixels
    // of both planes of the pair; a segment lies wholly inside or outside the image row
    u32x4 pv0[NCHW_IN ? PQ : 1], pv1[NCHW_IN ? PQ : 1];
    const int nitems = CinP / 2 * ROWS * DA_NSEG;
    if constexpr (NCHW_IN) {
#pragma unroll
        for (int q = 0; q < PQ; ++q) {
            const int idx = tid + 256 * q;
            const int sg = idx % DA_NSEG, r = (idx / DA_NSEG) % ROWS, ci = 2 * (idx / (DA_NSEG * ROWS));
            const int iy = j0 - 1 + r, ix = i0 - 8 + 8 * sg;
            const bool ok = idx < nitems && (unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W && ci < Cin;
            const uint32_t off = ok ? ((((uint32_t)n * Cin + ci) * H + iy) * W + ix) * 2u : kOob;
            pv0[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
            pv1[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(ok ? off + (uint32_t)H * W * 2u : kOob), 0, 0);
        }
    } else {
#pragma unroll
        for (int q = 0; q < VQ; ++q) {
            const int idx = tid + 256 * q;
            const int pr = idx / CV, cv = idx - pr * CV;     // pixel of the strip, channel vector
            const int r = pr / DC_SPX, p = pr - r * DC_SPX;
            const int iy = j0 - 1 + r, ix = i0 - 1 + p, ci = cv * 8;
            const bool ok = idx < nvec && (unsigned)iy < (unsigned)H && (unsigned)ix < (unsigned)W && ci < Cin;
            const uint32_t off = ok ? ((((uint32_t)n * H + iy) * W + ix) * Cin + ci) * 2u : kOob;
            sv[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
        }
    }
    // weight operands of chunk 0
    const __amdgpu_buffer_rsrc_t rw = rsrc_bytes(a.wp, a.wp_bytes);
    const int col = lane & 31, kq = (lane >> 5) * 8;
    const uint32_t wbase = (uint32_t)(((2 * py + px) * (a.CoP >> 5) + blockIdx.y) * nchp) * (16u * 1024u) + lane * 16u;
    u32x4 bw[4 * DC_KS];
    auto load_b = [&](int c) {
        const uint32_t cb = wbase + (uint32_t)c * (16u * 1024u);
#pragma unroll
        for (int i = 0; i < 4 * DC_KS; ++i)
            bw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(c < nchp ? cb + i * 1024u : kOob), 0, 0);
    };
    load_b(0);
    if constexpr (NCHW_IN) {
        // pixel k of segment sg is strip pixel p = 8 sg + k - 7; the pair's two values go
        // to LDS as one 4-byte word (ci even, PS even)
#pragma unroll
        for (int q = 0; q < PQ; ++q) {
            const int idx = tid + 256 * q;
            if (idx >= nitems) continue;
            const int sg = idx % DA_NSEG, r = (idx / DA_NSEG) % ROWS, ci = 2 * (idx / (DA_NSEG * ROWS));
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int p = 8 * sg + k - 7;
                if (p < 0 || p >= DC_SPX) continue;
                const uint32_t lo = (pv0[q][k >> 1] >> (16 * (k & 1))) & 0xffffu;
                const uint32_t hi = (pv1[q][k >> 1] >> (16 * (k & 1))) & 0xffffu;
                *reinterpret_cast<uint32_t *>(&sx[(r * DC_SPX + p) * PS + ci]) = lo | (hi << 16);
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < VQ; ++q) {
            const int idx = tid + 256 * q;
            const int pr = idx / CV, cv = idx - pr * CV;
            const int at = idx < nvec ? pr * PS + cv * 8 : ROWS * DC_SPX * DA_PSMAX + tid * 8;
            *reinterpret_cast<u32x4 *>(&sx[at]) = sv[q];
        }
    }
    __syncthreads();

    f32x16 acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;
    for (int c = 0; c < nchp; ++c) {
        vec bcur[4 * DC_KS];
#pragma unroll
        for (int i = 0; i < 4 * DC_KS; ++i) __builtin_memcpy(&bcur[i], &bw[i], 16);
        load_b(c + 1);
        const int c0 = c * DC_KC;
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) {
            const int ty = tp >> 1, tx = tp & 1;
#pragma unroll
            for (int ks = 0; ks < DC_KS; ++ks)
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    vec av;
                    __builtin_memcpy(&av, &sx[((m + py + ty) * DC_SPX + col + px + tx) * PS + c0 + kq + ks * 16], 16);
                    acc[m] = Mfma32<T>::run(av, bcur[tp * DC_KS + ks], acc[m]);
                }
        }
    }

    const int co = co0 + col;
    const float bv = (a.bias && co < Cout) ? a.bias[co] : 0.0f;
    const float av = (a.alpha && co < Cout) ? a.alpha[co] : 0.0f;
    auto epi = [&](auto actc) {
        constexpr int ACT = decltype(actc)::value;
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int p = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                so[col * OCS + (2 * m + py) * DC_OLD + 2 * p + px] = activate_c<ACT>(acc[m][i] + bv, av);
            }
    };
    switch (a.act) {
    case CONV2D_ACT_RELU: epi(std::integral_constant<int, CONV2D_ACT_RELU>{}); break;
    case CONV2D_ACT_SILU: epi(std::integral_constant<int, CONV2D_ACT_SILU>{}); break;
    case CONV2D_ACT_PRELU: epi(std::integral_constant<int, CONV2D_ACT_PRELU>{}); break;
    default: epi(std::integral_constant<int, CONV2D_ACT_NONE>{}); break;
    }
    __syncthreads();
    TO *__restrict__ y = static_cast<TO *>(a.y);
    const int OH = 2 * H, OW = 2 * W;
    const int oc0 = 2 * i0, or0 = 2 * j0;
    if constexpr (NCHW_OUT) {
#pragma unroll 4
        for (int it = 0; it < 16 * MR; ++it) {
            const int e = tid + 256 * it;
            const int oc = e & 63, lr = (e >> 6) & (2 * MR - 1), cl = e / (128 * MR);
            if (co0 + cl < Cout && oc0 + oc < OW && or0 + lr < OH)
                y[(((size_t)n * Cout + co0 + cl) * OH + or0 + lr) * OW + oc0 + oc] = out_cast<TO>(so[cl * OCS + lr * DC_OLD + oc]);
        }
    } else {
#pragma unroll 4
        for (int it = 0; it < 16 * MR; ++it) {
            const int e = tid + 256 * it;
            const int cl = e & 31, oc = (e >> 5) & 63, lr = e >> 11;
            if (co0 + cl < Cout && oc0 + oc < OW && or0 + lr < OH)
                y[(((size_t)n * OH + or0 + lr) * OW + oc0 + oc) * Cout + co0 + cl] = out_cast<TO>(so[cl * OCS + lr * DC_OLD + oc]);
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
    const int CinP = (Cin + DC_KC - 1) / DC_KC * DC_KC;
    const long long total = (long long)CoP * CinP;
    return launch_kernel(deconv_pack_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                         static_cast<const T *>(w), static_cast<T *>(wp), Cin, Cout, CoP, CinP);
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
static hipError_t mfma_t(const DeconvArgs &a, bool nchw, hipStream_t st) {
    const long long tiles = (long long)a.N * ((a.H + DC_MR - 1) / DC_MR) * ((a.W + DC_TW - 1) / DC_TW);
    dim3 grid((unsigned)tiles, (unsigned)(a.CoP / 32));
    if (nchw) return launch_kernel(deconv_mfma_kernel<T, TO, true>, grid, dim3(256), 0, st, a);
    return launch_kernel(deconv_mfma_kernel<T, TO, false>, grid, dim3(256), 0, st, a);
}

hipError_t launch_deconv_mfma(const DeconvArgs &a, int dtype, bool out_f32, bool nchw, hipStream_t st) {
    switch (dtype) {
    case CONV2D_DTYPE_BF16:
        return out_f32 ? mfma_t<bf16, float>(a, nchw, st) : mfma_t<bf16, bf16>(a, nchw, st);
    case CONV2D_DTYPE_F16:
        return out_f32 ? mfma_t<f16, float>(a, nchw, st) : mfma_t<f16, f16>(a, nchw, st);
    default:
        return hipErrorInvalidValue;
    }
}

template <typename T, typename TO, int MR>
static hipError_t mfma_all_mr(const DeconvArgs &a, bool nchw_in, hipStream_t st) {
    const long long tiles = (long long)a.N * ((a.H + MR - 1) / MR) * ((a.W + DC_TW - 1) / DC_TW);
    dim3 grid((unsigned)tiles, (unsigned)(a.CoP / 32));
    if (nchw_in) return launch_kernel(deconv_mfma_all_kernel<T, TO, true, true, MR>, grid, dim3(256), 0, st, a);
    return launch_kernel(deconv_mfma_all_kernel<T, TO, true, false, MR>, grid, dim3(256), 0, st, a);
}

// One-row tiles when two-row tiles would leave CUs idle (the IFNet deconv: 136 two-row
// tiles for 256 CUs); those workgroups fit two to a CU (smaller strip and epilogue tile).
template <typename T, typename TO>
static hipError_t mfma_all_t(const DeconvArgs &a, bool nchw_in, hipStream_t st) {
    const long long tiles2 = (long long)a.N * ((a.H + 1) / 2) * ((a.W + DC_TW - 1) / DC_TW) * (a.CoP / 32);
    if (tiles2 < 256) return mfma_all_mr<T, TO, 1>(a, nchw_in, st);
    return mfma_all_mr<T, TO, 2>(a, nchw_in, st);
}

hipError_t launch_deconv_mfma_all(const DeconvArgs &a, int dtype, bool out_f32, bool nchw_out, bool nchw_in,
                                  hipStream_t st) {
    // channel-first layers only; the planes are read directly only when 8-pixel segments are aligned
    if (a.Cin > DA_CMAX || (a.Cin % 8) != 0 || !nchw_out || (nchw_in && (a.W % 8) != 0)) return hipErrorInvalidValue;
    switch (dtype) {
    case CONV2D_DTYPE_BF16:
        return out_f32 ? mfma_all_t<bf16, float>(a, nchw_in, st) : mfma_all_t<bf16, bf16>(a, nchw_in, st);
    case CONV2D_DTYPE_F16:
        return out_f32 ? mfma_all_t<f16, float>(a, nchw_in, st) : mfma_all_t<f16, f16>(a, nchw_in, st);
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
