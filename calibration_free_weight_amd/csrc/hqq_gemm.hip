// hqq_gemm.hip -- the linear layer of an HQQ-quantized weight on gfx950:
// Y[M, N] = X[M, K] . W_r^T, with W_r the binary16 reconstruction of the packed axis-1
// quantized weight [N, K] ("HQQ - Half-Quadratic Quantization" usage guide, section "HQQLinear
// layer": the layer computes with the dequantized weight). Each weight is reconstructed as
// binary16((q - zero) * scale) in binary32, exactly as hqq_dequantize writes it; products of
// two binary16 values are exact in binary32 and accumulate in binary32; Y is stored binary16.
//
// Two paths:
//  * M <= 8 (decode): one wave per output row streams the row's packed codes (32 per lane per
//    step), reconstructs them in registers and accumulates every X row against them; a wave
//    reduction ends the row. HBM-bound on the packed weight.
//  * larger M: 64 x 128 output tiles per 256-thread block; each K step of 64 stages the X tile
//    and the reconstructed binary16 W tile in LDS and runs the v_mfma_f32_16x16x32_f16 matrix
//    cores (each wave a 32 x 64 sub-tile: 2 x 4 accumulators of 16 x 16).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "hqq_internal.h"

namespace hqq {
namespace {

typedef uint32_t g4u __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float g_h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ uint16_t g_f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

struct QW {                      // a packed axis-1 quantized weight [N, K]
    const uint8_t *packed;
    const uint16_t *scale;
    const void *zero;
    const uint16_t *meta;        // 8-bit zero meta {step, base}, or nullptr
    int64_t N, K;
    int g_log2, zero_bits;
};

// Codes k0 .. k0+31 of row n (k0 a multiple of 16; codes past K read as 0 and are never
// used). NB in {1, 2, 4, 8}: a row starts on a byte (K is a multiple of 16), so the 32 codes
// are the NB words at byte (n*K + k0)*NB/8, read as words when aligned (whole words only
// inside the row's bytes). NB = 3: ten codes per word, extracted one by one.
template <int NB>
__device__ __forceinline__ void load_codes32(const QW &w, int64_t n, int64_t k0, uint32_t (&q)[32])
{
    const int64_t c0 = n * w.K + k0;
    const int valid = w.K - k0 < 32 ? (int)(w.K - k0) : 32;
    if constexpr (NB == 3) {
        const uint32_t *wd = reinterpret_cast<const uint32_t *>(w.packed);
#pragma unroll
        for (int i = 0; i < 32; ++i)
            q[i] = i < valid ? (wd[(c0 + i) / 10] >> (3 * (int)((c0 + i) % 10))) & 7u : 0u;
    } else {
        const int64_t b0 = c0 * NB / 8;
        const int nbytes = valid * NB / 8;
        uint32_t words[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) words[i] = 0;
        if ((b0 & 3) == 0 && nbytes == 4 * NB) {
            const uint32_t *p = reinterpret_cast<const uint32_t *>(w.packed + b0);
#pragma unroll
            for (int i = 0; i < NB; ++i) words[i] = p[i];
        } else {
            for (int i = 0; i < nbytes; ++i) words[i >> 2] |= (uint32_t)w.packed[b0 + i] << (8 * (i & 3));
        }
        constexpr uint32_t mask = (1u << NB) - 1u;
        constexpr int per = 32 / NB;             // codes per word
#pragma unroll
        for (int i = 0; i < 32; ++i) q[i] = (words[i / per] >> (NB * (i % per))) & mask;
    }
}

// Zero of group gi in binary32: the binary16 zero, or zq*step + base (one fused rounding)
__device__ __forceinline__ float zero_of(const QW &w, int64_t gi, float m0, float m1)
{
    return w.zero_bits == 16 ? g_h2f(static_cast<const uint16_t *>(w.zero)[gi])
                             : fmaf((float)static_cast<const uint8_t *>(w.zero)[gi], m0, m1);
}

// 32 codes of row n from k0 to binary16 pairs (16 words), as hqq_dequantize writes them.
template <int NB>
__device__ __forceinline__ void recon32(const QW &w, int64_t n, int64_t k0, float m0, float m1,
                                        uint32_t (&out)[16])
{
    uint32_t q[32];
    load_codes32<NB>(w, n, k0, q);
    const int64_t gpr = w.K >> w.g_log2;
#pragma unroll
    for (int c = 0; c < 4; ++c) {               // 8 codes never straddle a group (g >= 16)
        if (k0 + 8 * c >= w.K) {
#pragma unroll
            for (int i = 0; i < 4; ++i) out[4 * c + i] = 0;
            continue;
        }
        const int64_t gi = n * gpr + ((k0 + 8 * c) >> w.g_log2);
        const float zf = zero_of(w, gi, m0, m1), s = g_h2f(w.scale[gi]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[4 * c + i] = (uint32_t)g_f2h(((float)q[8 * c + 2 * i] - zf) * s) |
                             (uint32_t)g_f2h(((float)q[8 * c + 2 * i + 1] - zf) * s) << 16;
    }
}

// ---------------------------------------------------------------------------------------
// M <= 8: one wave per output row; MB X rows at most (the launch picks 1, 2, 4 or 8).
// ---------------------------------------------------------------------------------------
constexpr int kSkinnyM = 8;

template <int NB, int MB>
__global__ void __launch_bounds__(256) gemv_kernel(const uint16_t *__restrict__ X, int M, QW w,
                                                   uint16_t *__restrict__ Y)
{
    constexpr int IT = 2;                        // steps of 32 codes per lane in flight
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= w.N) return;                        // whole wave
    const float m0 = w.meta ? g_h2f(w.meta[0]) : 0.0f, m1 = w.meta ? g_h2f(w.meta[1]) : 0.0f;
    const int64_t gpr = w.K >> w.g_log2;
    float acc[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = 0.0f;
    for (int64_t kb = (int64_t)lane * 32; kb < w.K; kb += 64 * 32 * IT) {
        // every load of the IT steps first: codes, per-group scale and zero, and X (M = 1)
        uint32_t q[IT][32];
        float zf[IT][4], sc[IT][4];
        g4u xv[IT][4];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int64_t k0 = kb + (int64_t)it * 64 * 32;
            if (k0 >= w.K) break;
            load_codes32<NB>(w, n, k0, q[it]);
            if (w.g_log2 >= 5) {                 // the 32 codes lie in one group
                const int64_t gi = n * gpr + (k0 >> w.g_log2);
                const float z = zero_of(w, gi, m0, m1), sv = g_h2f(w.scale[gi]);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    zf[it][c] = z;
                    sc[it][c] = sv;
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t kk = k0 + 8 * c < w.K ? k0 + 8 * c : k0;
                    const int64_t gi = n * gpr + (kk >> w.g_log2);
                    zf[it][c] = zero_of(w, gi, m0, m1);
                    sc[it][c] = g_h2f(w.scale[gi]);
                }
            }
            if constexpr (MB == 1) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    xv[it][c] = k0 + 8 * c < w.K ? *reinterpret_cast<const g4u *>(X + k0 + 8 * c)
                                                 : g4u{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int64_t k0 = kb + (int64_t)it * 64 * 32;
            if (k0 >= w.K) break;
            const int valid = w.K - k0 < 32 ? (int)(w.K - k0) : 32;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (8 * c >= valid) break;
                h2 wp[4];                        // binary16 weight pairs
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    wp[i] = __builtin_bit_cast(
                        h2, (uint32_t)g_f2h(((float)q[it][8 * c + 2 * i] - zf[it][c]) * sc[it][c]) |
                                (uint32_t)g_f2h(((float)q[it][8 * c + 2 * i + 1] - zf[it][c]) * sc[it][c]) << 16);
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    if (m >= M) break;
                    const g4u x = MB == 1 ? xv[it][c]
                                          : *reinterpret_cast<const g4u *>(X + (int64_t)m * w.K + k0 + 8 * c);
                    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
                    // two exact binary16 products per step into the binary32 sum
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[m] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, xs[i]), wp[i], acc[m], false);
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        if (m >= M) break;
        float v = acc[m];
#pragma unroll
        for (int off = 32; off >= 1; off /= 2) v += __shfl_xor(v, off);
        if (lane == 0) Y[(int64_t)m * w.N + n] = g_f2h(v);
    }
}

// ---------------------------------------------------------------------------------------
// Larger M: MFMA tiles.
// ---------------------------------------------------------------------------------------
constexpr int BM = 64, BN = 128, BK = 64, LP = BK + 8;   // LDS row pitch (halves)

// The raw inputs of one K step for this thread: 16 halves of X (two 16-byte loads) and the
// packed codes, scale and zero of 32 weights; loaded a step ahead, consumed into LDS.
template <int NB>
struct Stage {
    g4u x0, x1;
    uint32_t q[32];                  // the codes
    float zf[4], s[4];
    bool wv;
};

template <int NB>
__device__ __forceinline__ void stage_load(const uint16_t *X, int64_t M, const QW &w, int64_t m0,
                                           int64_t n0, int64_t k0, float zs, float zb, int t,
                                           Stage<NB> &st)
{
    {
        const int r = t >> 2, c = (t & 3) * 16;
        const int64_t m = m0 + r, k = k0 + c;
        st.x0 = g4u{0, 0, 0, 0};
        st.x1 = g4u{0, 0, 0, 0};
        if (m < M && k < w.K) {                  // K is a multiple of 16: whole chunks
            const g4u *p = reinterpret_cast<const g4u *>(X + m * w.K + k);
            st.x0 = p[0];
            st.x1 = p[1];
        }
    }
    const int r = t >> 1, c = (t & 1) * 32;
    const int64_t n = n0 + r, k = k0 + c;
    st.wv = n < w.N && k < w.K;
    if (st.wv) {
        load_codes32<NB>(w, n, k, st.q);
        const int64_t gpr = w.K >> w.g_log2;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int64_t kk = k + 8 * cc < w.K ? k + 8 * cc : k;
            const int64_t gi = n * gpr + (kk >> w.g_log2);
            st.zf[cc] = zero_of(w, gi, zs, zb);
            st.s[cc] = g_h2f(w.scale[gi]);
        }
    }
}

template <int NB>
__device__ __forceinline__ void stage_store(const Stage<NB> &st, const QW &w, int64_t k0, int t,
                                            uint16_t *xs, uint16_t *ws)
{
    {
        const int r = t >> 2, c = (t & 3) * 16;
        *reinterpret_cast<g4u *>(&xs[r * LP + c]) = st.x0;
        *reinterpret_cast<g4u *>(&xs[r * LP + c + 8]) = st.x1;
    }
    const int r = t >> 1, c = (t & 1) * 32;
    const uint32_t (&q)[32] = st.q;
    uint32_t out[16];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = st.wv && k0 + c + 8 * cc < w.K;
            out[4 * cc + i] =
                ok ? (uint32_t)g_f2h(((float)q[8 * cc + 2 * i] - st.zf[cc]) * st.s[cc]) |
                         (uint32_t)g_f2h(((float)q[8 * cc + 2 * i + 1] - st.zf[cc]) * st.s[cc]) << 16
                   : 0u;
        }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<g4u *>(&ws[r * LP + c + 8 * i]) =
            g4u{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
}

template <int NB>
__global__ void __launch_bounds__(256) gemm_mfma_kernel(const uint16_t *__restrict__ X, int64_t M,
                                                        QW w, uint16_t *__restrict__ Y)
{
    __shared__ __attribute__((aligned(16))) uint16_t xs[BM * LP];
    __shared__ __attribute__((aligned(16))) uint16_t ws[BN * LP];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;     // 32-row, 64-column sub-tile of the wave
    const int64_t tiles_n = (w.N + BN - 1) / BN;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM, n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
    const float zs = w.meta ? g_h2f(w.meta[0]) : 0.0f, zb = w.meta ? g_h2f(w.meta[1]) : 0.0f;
    f4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    // Software pipeline: the next K step's global loads are in flight during this step's
    // matrix-core work; they are reconstructed into LDS after it.
    Stage<NB> st;
    stage_load<NB>(X, M, w, m0, n0, 0, zs, zb, t, st);
    for (int64_t k0 = 0; k0 < w.K; k0 += BK) {
        stage_store<NB>(st, w, k0, t, xs, ws);
        __syncthreads();
        if (k0 + BK < w.K) stage_load<NB>(X, M, w, m0, n0, k0 + BK, zs, zb, t, st);
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            const int kk = ks + 8 * (lane >> 4);
            h8 a[2], b[4];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const h8 *>(&xs[(32 * wm + 16 * i + (lane & 15)) * LP + kk]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const h8 *>(&ws[(64 * wn + 16 * j + (lane & 15)) * LP + kk]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // D[row][col] of a 16 x 16 tile: lane holds rows 4*(lane/16) .. +3 of column lane%16
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + 32 * wm + 16 * i + 4 * (lane >> 4) + e;
                const int64_t n = n0 + 64 * wn + 16 * j + (lane & 15);
                if (m < M && n < w.N) Y[m * w.N + n] = g_f2h(acc[i][j][e]);
            }
}

template <int NB>
void launch_nb(const uint16_t *X, int64_t M, const QW &w, uint16_t *Y, hipStream_t stream)
{
    const dim3 block(256);
    if (M <= kSkinnyM) {
        const dim3 grid((unsigned)((w.N + 3) / 4));
        if (M == 1) hipLaunchKernelGGL((gemv_kernel<NB, 1>), grid, block, 0, stream, X, (int)M, w, Y);
        else if (M == 2) hipLaunchKernelGGL((gemv_kernel<NB, 2>), grid, block, 0, stream, X, (int)M, w, Y);
        else if (M <= 4) hipLaunchKernelGGL((gemv_kernel<NB, 4>), grid, block, 0, stream, X, (int)M, w, Y);
        else hipLaunchKernelGGL((gemv_kernel<NB, 8>), grid, block, 0, stream, X, (int)M, w, Y);
    } else {
        const int64_t blocks = ((M + BM - 1) / BM) * ((w.N + BN - 1) / BN);
        hipLaunchKernelGGL((gemm_mfma_kernel<NB>), dim3((unsigned)blocks), block, 0, stream, X, M, w, Y);
    }
}

}  // namespace

hipError_t launch_gemm(const uint16_t *X, int64_t M, const uint8_t *packed, const uint16_t *scale,
                       const void *zero, const uint16_t *zero_meta, int64_t N, int64_t K,
                       int nbits, int g, int zero_bits, uint16_t *Y, hipStream_t stream)
{
    if (M == 0 || N == 0) return hipSuccess;
    int lg = 0;
    while ((1 << lg) < g) ++lg;
    const QW w{packed, scale, zero, zero_bits == 8 ? zero_meta : nullptr, N, K, lg, zero_bits};
    switch (nbits) {
    case 1: launch_nb<1>(X, M, w, Y, stream); break;
    case 2: launch_nb<2>(X, M, w, Y, stream); break;
    case 3: launch_nb<3>(X, M, w, Y, stream); break;
    case 4: launch_nb<4>(X, M, w, Y, stream); break;
    case 8: launch_nb<8>(X, M, w, Y, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hqq
