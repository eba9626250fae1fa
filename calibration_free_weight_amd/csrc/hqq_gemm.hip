// hqq_gemm.hip -- the linear layer of an HQQ-quantized weight on gfx950:
// Y[M, N] = X[M, K] . W_r^T, with W_r the binary16 reconstruction of the packed axis-1
// quantized weight [N, K] ("HQQ - Half-Quadratic Quantization" usage guide, section "HQQLinear
// layer": the layer computes with the dequantized weight). Each weight is reconstructed as
// binary16((q - zero) * scale) in binary32, exactly as hqq_dequantize writes it; products of
// two binary16 values are exact in binary32 and accumulate in binary32; Y is stored binary16.
//
// Paths by M:
//  * M = 1 (decode): a wave takes two output rows and streams their packed codes (32 per lane
//    per chunk), reconstructs them in registers and accumulates the X row against them with
//    v_dot2; a wave reduction ends each row.
//  * 2 <= M <= 64 (skinny): the weight streams once; a block owns 16 weight rows, its waves
//    split K, and each lane reconstructs its v_mfma_f32_16x16x32_f16 B fragment per step.
//  * M > 64 with a workspace: W_r is written once into the workspace as binary16 and a plain
//    binary16 MFMA GEMM (double-buffered LDS, XCD-aware tile order) reads it.
//  * M > 64 without one: the skinny kernel on slices of 64 rows.
//  * Packed buffers the fast kernels cannot read word-wise (unaligned): the original kernels,
//    one wave per output row for M <= 8 and, above that, 64 x 128 output tiles per block that
//    stage the X tile and the reconstructed binary16 W tile in LDS for the matrix cores.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <vector>

#include "hqq_internal.h"

namespace hqq {
namespace {

typedef uint32_t g4u __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float g_h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
// binary32 -> binary16, round to nearest even, of an already rounded binary32 value. The
// empty asm hides how f was computed: otherwise the compiler folds a binary32 multiply or fma
// feeding the conversion into one mixed-precision instruction (v_fma_mixlo_f16) that rounds
// the exact result to binary16 once, which differs from rounding to binary32 first whenever
// the binary32 value is a binary16 tie.
__device__ __forceinline__ uint16_t g_f2h(float f)
{
    asm("" : "+v"(f));
    return __half_as_ushort(__float2half_rn(f));
}
// Two such conversions packed into one word (a in the low half): one v_cvt_pk_f16_f32, which
// the compiler does not always form from two single conversions joined by shifts.
typedef float g2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t g_f2h2(float a, float b)
{
    asm("" : "+v"(a), "+v"(b));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(g2f{a, b}, h2));
}

struct QW {                      // a packed axis-1 quantized weight [N, K]
    const uint8_t *packed;
    const uint16_t *scale;
    const void *zero;
    const uint16_t *meta;        // 8-bit zero meta {step, base}, or nullptr
    int64_t N, K;
    int g_log2, zero_bits;
};

// Weights that read the same X, multiplied by one launch of the decode or skinny kernel: the
// grid is the weights' grids one after another, and a block finds its weight by its index.
constexpr int kMaxSet = 8;
struct QWSet {
    QW w[kMaxSet];
    uint16_t *Y[kMaxSet];
    uint32_t b0[kMaxSet + 1];    // first block of each weight; b0[n] = all blocks
    int n;
};
// The block's weight, and blk turned into the block's index among that weight's blocks.
__device__ __forceinline__ int set_pick(const QWSet &s, uint32_t &blk)
{
    int i = 0;
    while (i + 1 < s.n && blk >= s.b0[i + 1]) ++i;
    blk -= s.b0[i];
    return i;
}

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
            out[4 * c + i] = g_f2h2(((float)q[8 * c + 2 * i] - zf) * s, ((float)q[8 * c + 2 * i + 1] - zf) * s);
    }
}

// ---------------------------------------------------------------------------------------
// Fallback for M <= 8 (3-bit at M = 1, packed buffers that are not word-aligned): one wave
// per output row; MB X rows at most (the launch picks 1, 2, 4 or 8).
// ---------------------------------------------------------------------------------------
constexpr int kSkinnyM = 8;
#ifndef HQQ_SKINNY_LO
#define HQQ_SKINNY_LO 1
#endif
constexpr int kSkinnyLo = HQQ_SKINNY_LO;  // M above this (up to 64): the matrix-core skinny kernel
#ifndef HQQ_GEMV_ROWS
#define HQQ_GEMV_ROWS 2
#endif
constexpr int kGemvRows = HQQ_GEMV_ROWS;  // rows per wave of the M = 1 decode kernel
constexpr int kWsM = 64;         // the reconstruct-once path (with a workspace) above this M
#ifndef HQQ_GEMM_DEPTH
#define HQQ_GEMM_DEPTH 2
#endif
constexpr int kDepth = HQQ_GEMM_DEPTH;   // K steps of loads in flight in the binary16 GEMM
#ifndef HQQ_GEMM_BM
#define HQQ_GEMM_BM 0
#endif
constexpr int kBM16 = HQQ_GEMM_BM;       // output rows per block of the binary16 GEMM (0: chosen)
#ifndef HQQ_GEMM_KS
#define HQQ_GEMM_KS 2
#endif
constexpr int kSplitK = HQQ_GEMM_KS;     // wave groups splitting each K step
constexpr int64_t kMaxWsK = int64_t(1) << 22;   // 32-bit buffer offsets over 128 rows of K

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
                        h2, g_f2h2(((float)q[it][8 * c + 2 * i] - zf[it][c]) * sc[it][c], ((float)q[it][8 * c + 2 * i + 1] - zf[it][c]) * sc[it][c]));
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

// M = 1 (and M <= 8 in the rare shapes the skinny kernel does not take), bit widths 1, 2, 4, 8
// with K*nbits a multiple of 32 and a 4-byte aligned packed buffer: each wave takes R
// consecutive rows (R > 1 for one X row: the lane's X values are
// loaded once and used for every row). A lane takes chunks of 32 codes, 2048 codes apart.
// Everything is read with buffer loads from wave-uniform bases; an offset past the end of a
// buffer reads zero, so chunks past K (X = 0: they add nothing) and rows past N need no
// branches. The codes of a 32-bit word are split into byte planes (one mask per plane) and
// each byte converted by v_cvt_f32_ubyte.
template <int NB>
__device__ __forceinline__ void plane_codes(const uint32_t (&wd)[NB], float (&c)[32])
{
    constexpr int P = 8 / NB;                   // planes per word
    constexpr uint32_t m = ((1u << NB) - 1u) * 0x01010101u;
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int p = 0; p < P; ++p) {
            uint32_t pl = (wd[i] >> (NB * p)) & m;
            if constexpr (NB < 8) asm("" : "+v"(pl));   // keep the plane: one byte convert per code
#pragma unroll
            for (int b = 0; b < 4; ++b) c[i * (32 / NB) + b * P + p] = (float)((pl >> (8 * b)) & 0xFFu);
        }
}

template <int NB>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&wd)[NB])
{
    if constexpr (NB == 1) {
        wd[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    } else if constexpr (NB == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        wd[0] = v[0];
        wd[1] = v[1];
    } else if constexpr (NB == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) wd[i] = v[i];
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wd[i] = v[i];
            wd[4 + i] = u[i];
        }
    }
}

// A buffer resource over [base, base + bytes) (clamped below 2^31). Base and size must be
// wave-uniform; both pass through readfirstlane, because 64-bit compares and selects on the
// way can leave them in VGPRs, and a resource in VGPRs makes every load through it a
// waterfall loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int nr = __builtin_amdgcn_readfirstlane((int)(bytes < 0x7FFFFFF0 ? bytes : 0x7FFFFFF0));
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(hi << 32 | lo), (short)0,
                                             nr, 0x00020000);
}

template <int NB, int MB, int R, int ZB, int ITV = 0>
__global__ void __launch_bounds__(256) gemv2_kernel(const uint16_t *__restrict__ X, int M,
                                                    QWSet set)
{
    uint32_t blk = blockIdx.x;
    const int wi = set_pick(set, blk);
    const QW w = set.w[wi];
    uint16_t *__restrict__ const Y = set.Y[wi];
    constexpr int zb = ZB / 8;                   // bytes per stored zero
    constexpr uint32_t kOut = 0x80000000u;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int64_t n0 = ((int64_t)blk * 4 + wave) * R;
    if (n0 >= w.N) return;                       // whole wave
    const int64_t rows = w.N - n0 < R ? w.N - n0 : R;
    const int64_t rb = w.K * NB / 8;             // packed bytes per row (a multiple of 4)
    const int64_t gpr = w.K >> w.g_log2;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(w.packed + n0 * rb, rows * rb);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.scale + n0 * gpr, rows * gpr * 2);
    const __amdgpu_buffer_rsrc_t rz =
        make_rsrc(static_cast<const uint8_t *>(w.zero) + n0 * gpr * zb, rows * gpr * zb);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (int64_t)M * w.K * 2);
    const float m0 = w.meta ? g_h2f(w.meta[0]) : 0.0f, m1 = w.meta ? g_h2f(w.meta[1]) : 0.0f;
    const int gsh = w.g_log2;
    float acc[MB][R];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

    constexpr int IT = ITV ? ITV : (MB >= 4 ? 1 : 2);   // chunks per lane in flight
    const int64_t steps = (w.K + 2047) >> 11;    // chunks of the row per lane (some past K)
    for (int64_t j0 = 0; j0 < steps; j0 += IT) {
        uint32_t wd[IT][R][NB];
        uint16_t sv[IT][R][2], zv[IT][R][2];
        g4u xv[IT][MB][4];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int64_t k = ((j0 + it) * 64 + lane) * 32;
            const bool in = k < w.K;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                load_words<NB>(rp, in ? (uint32_t)(r * rb + k * NB / 8) : kOut, wd[it][r]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {       // the groups of codes 0-15 and 16-31
                    const uint32_t gi = (uint32_t)(r * gpr + ((k + 16 * h) >> gsh));
                    sv[it][r][h] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, in ? gi * 2 : kOut, 0, 0);
                    if constexpr (zb == 2)
                        zv[it][r][h] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rz, in ? gi * 2 : kOut, 0, 0);
                    else
                        zv[it][r][h] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b8(rz, in ? gi : kOut, 0, 0);
                }
            }
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    // each 8-code piece masked on its own: with K % 32 == 16 a chunk's second
                    // half lies past the row, and its X must read zero (the weights there
                    // may belong to the next row)
                    const bool inx = m < M && k + 8 * c < w.K;
                    const uint32_t off = inx ? (uint32_t)((m * w.K + k + 8 * c) * 2) : kOut;
                    xv[it][m][c] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
                }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float c[32];
                plane_codes<NB>(wd[it][r], c);
                float zf[2], sc[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if constexpr (zb == 2) zf[h] = g_h2f(zv[it][r][h]);
                    else zf[h] = fmaf((float)zv[it][r][h], m0, m1);
                    sc[h] = g_h2f(sv[it][r][h]);
                }
#pragma unroll
                for (int q = 0; q < 16; ++q) {      // pairs of codes
                    const int h = q >> 3;
                    const h2 wp = __builtin_bit_cast(
                        h2, g_f2h2((c[2 * q] - zf[h]) * sc[h], (c[2 * q + 1] - zf[h]) * sc[h]));
#pragma unroll
                    for (int m = 0; m < MB; ++m) {
                        const uint32_t xw = xv[it][m][q >> 2][q & 3];
                        acc[m][r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, xw), wp, acc[m][r], false);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        if (m >= M) break;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float v = acc[m][r];
#pragma unroll
            for (int off = 32; off >= 1; off /= 2) v += __shfl_xor(v, off);
            if (lane == 0 && r < rows) Y[(int64_t)m * w.N + n0 + r] = g_f2h(v);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Fallback for M > 8 with a packed buffer that is not word-aligned: LDS-staged MFMA tiles.
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
                ok ? g_f2h2(((float)q[8 * cc + 2 * i] - st.zf[cc]) * st.s[cc], ((float)q[8 * cc + 2 * i + 1] - st.zf[cc]) * st.s[cc])
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

// ---------------------------------------------------------------------------------------
// Larger M with a workspace: W_r is reconstructed once into binary16 (HBM-bound), then a
// plain binary16 matrix-core GEMM reads it. The fused kernel above reconstructs each weight
// tile once per 64-row block of X, which dominates once there are several such blocks.
// ---------------------------------------------------------------------------------------

// Reconstruction as a flat map: with groups along rows and g | K, code i (row-major) belongs
// to group i / g, so W_r[i] = binary16((q_i - zero[i/g]) * scale[i/g]) needs no row
// arithmetic. A unit is 8 consecutive codes (one 16-byte store; g >= 16, so one group); units
// are lane-contiguous, so each load and store instruction of a wave covers one contiguous
// range. Each thread takes U units, a grid apart, with all their loads issued first.
constexpr int kReconU = 4;

template <int NB>
__device__ __forceinline__ void unit_codes(const uint8_t *packed, int64_t u, uint32_t (&q)[8])
{
    if constexpr (NB == 3) {                     // ten codes per 32-bit word
        const uint32_t *wd = reinterpret_cast<const uint32_t *>(packed);
        const int64_t c0 = u * 8, w0 = c0 / 10;
        const int j = (int)(c0 - w0 * 10);
        const uint32_t a = wd[w0], b = j > 2 ? wd[w0 + 1] : 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int p = j + i;
            q[i] = (p < 10 ? a >> (3 * p) : b >> (3 * (p - 10))) & 7u;
        }
    } else {
        uint32_t lo, hi = 0;                     // the unit's NB bytes
        if constexpr (NB == 1) lo = packed[u];
        else if constexpr (NB == 2) lo = reinterpret_cast<const uint16_t *>(packed)[u];
        else if constexpr (NB == 4) lo = reinterpret_cast<const uint32_t *>(packed)[u];
        else {
            const uint2 v = reinterpret_cast<const uint2 *>(packed)[u];
            lo = v.x;
            hi = v.y;
        }
        constexpr uint32_t mask = (1u << NB) - 1u;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            q[i] = NB == 8 ? ((i < 4 ? lo : hi) >> (8 * (i & 3))) & mask : (lo >> (NB * i)) & mask;
    }
}

// AX0: groups run down columns instead (hqq_dequantize of an axis-0 weight with cols a
// multiple of 8): the unit's 8 codes lie in one row and belong to 8 consecutive groups of the
// [rows/g, cols] per-group arrays. NT: nontemporal (streaming) stores, for an output that is
// not read again soon (hqq_dequantize; the GEMM's workspace is read right after and is
// better left in the caches).
template <int NB, bool AX0, bool NT>
__global__ void __launch_bounds__(256) recon_kernel(QW w, int64_t n, int64_t cols,
                                                   uint16_t *__restrict__ Wr)
{
    constexpr int U = kReconU;
    constexpr int ZS = AX0 ? 8 : 1;              // scale/zero pairs per unit
    const int64_t units = n >> 3, T = (int64_t)gridDim.x * 256;
    const float m0 = w.meta ? g_h2f(w.meta[0]) : 0.0f, m1 = w.meta ? g_h2f(w.meta[1]) : 0.0f;
    for (int64_t u0 = (int64_t)blockIdx.x * 256 + threadIdx.x; u0 < units; u0 += T * U) {
        uint32_t q[U][8];
        float zf[U][ZS], sc[U][ZS];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t u = u0 + k * T;
            if (u >= units) break;
            unit_codes<NB>(w.packed, u, q[k]);
            int64_t gi;
            if constexpr (AX0) {
                const int64_t row = (u * 8) / cols;
                gi = (row >> w.g_log2) * cols + (u * 8 - row * cols);
            } else {
                gi = (u * 8) >> w.g_log2;
            }
#pragma unroll
            for (int e = 0; e < ZS; ++e) {
                zf[k][e] = zero_of(w, gi + e, m0, m1);
                sc[k][e] = g_h2f(w.scale[gi + e]);
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t u = u0 + k * T;
            if (u >= units) break;
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int a = AX0 ? 2 * i : 0, b = AX0 ? 2 * i + 1 : 0;
                o[i] = g_f2h2(((float)q[k][2 * i] - zf[k][a]) * sc[k][a], ((float)q[k][2 * i + 1] - zf[k][b]) * sc[k][b]);
            }
            const g4u v{o[0], o[1], o[2], o[3]};
            if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<g4u *>(Wr + u * 8));
            else *reinterpret_cast<g4u *>(Wr + u * 8) = v;
        }
    }
}

template <int NB>
void launch_recon_nb(const QW &w, int64_t n, int64_t cols, int axis, bool nt, uint16_t *out,
                     hipStream_t stream)
{
    const int64_t per_block = 256 * kReconU;
    const int64_t rb = (n / 8 + per_block - 1) / per_block;
    const dim3 grid((unsigned)(rb < 65536 ? rb : 65536)), block(256);
    if (axis == 0)
        hipLaunchKernelGGL((recon_kernel<NB, true, true>), grid, block, 0, stream, w, n, cols, out);
    else if (nt)
        hipLaunchKernelGGL((recon_kernel<NB, false, true>), grid, block, 0, stream, w, n, cols, out);
    else
        hipLaunchKernelGGL((recon_kernel<NB, false, false>), grid, block, 0, stream, w, n, cols, out);
}

#ifndef HQQ_GEMM_SWZ
#define HQQ_GEMM_SWZ 1
#endif
// LDS layout of the binary16 GEMM's tiles: rows of BK halves (8 chunks of 16 bytes), chunk c
// of row r stored at chunk c ^ f(r), f(r) = (r/2) ^ 4*(r%2). A matrix-core operand read
// (lanes 0..15 read one chunk of rows r0..r0+15) and a row store (8 lanes per row) then touch
// distinct banks whether the LDS serves 8 or 16 lanes of a 16-byte access per cycle.
constexpr int kRow16 = HQQ_GEMM_SWZ ? BK : LP;          // row pitch (halves)
__device__ __forceinline__ int lds_pos(int r, int c)
{
    if constexpr (HQQ_GEMM_SWZ) return r * BK + ((c ^ (((r >> 1) ^ ((r & 1) << 2)) & 7)) << 3);
    else return r * LP + c * 8;
}

// Y[M, N] = X[M, K] . Wr[N, K]^T, all binary16 row-major, binary32 accumulation.
// BMT x 128 output tiles per block of 256*KS threads: KS groups of four waves, each wave a
// BMT/2 x 64 sub-tile; group g takes the 32-wide k slices g, g + KS, ... of every K step of
// 64, and the groups' sums are added at the end (KS = 2 gives two waves per SIMD for the same
// LDS traffic, so one wave's LDS and barrier waits overlap the other's matrix-core work).
// K steps go through two LDS buffers; the global loads run D steps ahead in a ring of
// register sets (a block is latency-bound on its loads otherwise); each step stores the next
// step's set into the other LDS buffer (one barrier per step). Blocks are spread so that each
// XCD takes a contiguous range of tiles, n-major with the row tiles of one weight tile
// adjacent: that tile is then fetched into one L2.
template <int BMT, int D, int KS>
__global__ void __launch_bounds__(256 * KS) gemm_f16_kernel(const uint16_t *__restrict__ X,
                                                            int64_t M,
                                                            const uint16_t *__restrict__ Wr,
                                                            int64_t N, int64_t K,
                                                            uint16_t *__restrict__ Y)
{
    constexpr int NT = 256 * KS;
    constexpr int TI = BMT / 32;                 // 16-row MFMA tiles per wave
    constexpr int XL = BMT * BK / 8 / NT;        // 16-byte X chunks per thread per step
    constexpr int WL = BN * BK / 8 / NT;         // 16-byte W chunks per thread per step
    static_assert(XL >= 1 && WL >= 1 && BK % (32 * KS) == 0, "tile split");
    // two buffers of the X tile, then two of the W tile; at the end, group 1's sums
    constexpr int kLds = 2 * (BMT + BN) * kRow16;
    static_assert(KS == 1 || 256 * TI * 16 * 4 <= kLds * 2, "reduction fits the LDS");
    __shared__ __attribute__((aligned(16))) uint16_t lds[kLds];
    auto xs = [&](int buf) { return lds + buf * BMT * kRow16; };
    auto ws = [&](int buf) { return lds + 2 * BMT * kRow16 + buf * BN * kRow16; };
    const int t = threadIdx.x, lane = t & 63, wave = (t >> 6) & 3, grp = t >> 8;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t tiles_m = (M + BMT - 1) / BMT;
    int64_t b = blockIdx.x;
    const int64_t per = gridDim.x / 8;
    if (b < per * 8) b = (b % 8) * per + b / 8;
    const int64_t m0 = (b % tiles_m) * BMT, n0 = (b / tiles_m) * BN;

    f4 acc[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    // Buffer loads over the block's rows: an offset at or past the record count returns
    // zeros, so rows past M or N, columns past K and whole steps past the end need no
    // branches, and every load of the ring stays countable by the wait counters.
    const uint32_t kOut = 0x80000000u;
    auto rsrc = [](const uint16_t *base, int64_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0,
                                                 (int)(bytes < 0x7FFFFFF0 ? bytes : 0x7FFFFFF0),
                                                 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t rx = rsrc(X + m0 * K, (M - m0) * K * 2);
    const __amdgpu_buffer_rsrc_t rw = rsrc(Wr + n0 * K, (N - n0) * K * 2);
    const int col = (t & 7) * 8;                 // the thread's 8 columns of every chunk
    uint32_t xo[XL], wo[WL];                     // byte offsets of the chunks at k = 0
#pragma unroll
    for (int c = 0; c < XL; ++c) xo[c] = (uint32_t)((((t + NT * c) >> 3) * K + col) * 2);
#pragma unroll
    for (int c = 0; c < WL; ++c) wo[c] = (uint32_t)((((t + NT * c) >> 3) * K + col) * 2);
    g4u xr[D][XL], wr[D][WL];
    auto load = [&](int64_t k0, g4u (&xv)[XL], g4u (&wv)[WL]) {
        const bool in = col < K - k0;            // k < K implies k + 8 <= K
        const uint32_t kb = (uint32_t)(k0 * 2);
#pragma unroll
        for (int c = 0; c < XL; ++c)
            xv[c] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? xo[c] + kb : kOut, 0, 0);
#pragma unroll
        for (int c = 0; c < WL; ++c)
            wv[c] = __builtin_amdgcn_raw_buffer_load_b128(rw, in ? wo[c] + kb : kOut, 0, 0);
    };
    auto store = [&](int buf, const g4u (&xi)[XL], const g4u (&wi)[WL]) {
#pragma unroll
        for (int c = 0; c < XL; ++c) {
            const int idx = t + NT * c;
            *reinterpret_cast<g4u *>(xs(buf) + lds_pos(idx >> 3, idx & 7)) = xi[c];
        }
#pragma unroll
        for (int c = 0; c < WL; ++c) {
            const int idx = t + NT * c;
            *reinterpret_cast<g4u *>(ws(buf) + lds_pos(idx >> 3, idx & 7)) = wi[c];
        }
    };

    // Ring invariant at the top of step kt: LDS buffer kt&1 holds step kt; register set
    // (kt + i) % D holds step kt + i for 1 <= i < D (loads in flight); set kt % D is free.
    // The loop runs whole rings of D steps: steps past the end hold zeros and add nothing.
    const int64_t nk = (K + BK - 1) / BK;
#pragma unroll
    for (int d = 0; d < D; ++d) load((int64_t)d * BK, xr[d], wr[d]);
    store(0, xr[0], wr[0]);
    __syncthreads();
    for (int64_t kt0 = 0; kt0 < nk; kt0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t kt = kt0 + d;
            const int cur = (d & 1) ^ (int)(kt0 & 1);   // = kt & 1
            load((kt + D) * BK, xr[d], wr[d]);
#pragma unroll
            for (int s = 0; s < BK / 32 / KS; ++s) {
                const int ch = (s * KS + grp) * 4 + (lane >> 4);   // the lane's 16-byte chunk
                h8 a[TI], bv[4];
#pragma unroll
                for (int i = 0; i < TI; ++i)
                    a[i] = *reinterpret_cast<const h8 *>(xs(cur) + lds_pos(BMT / 2 * wm + 16 * i + (lane & 15), ch));
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bv[j] = *reinterpret_cast<const h8 *>(ws(cur) + lds_pos(64 * wn + 16 * j + (lane & 15), ch));
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bv[j], acc[i][j], 0, 0, 0);
            }
            store(cur ^ 1, xr[(d + 1) % D], wr[(d + 1) % D]);
            __syncthreads();
        }
    }
    if constexpr (KS == 2) {
        // group 1 hands its sums to group 0 through the (now idle) LDS buffers
        float *red = reinterpret_cast<float *>(lds);
        const int slot = wave * 64 + lane;
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) red[((i * 4 + j) * 4 + e) * 256 + slot] = acc[i][j][e];
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] += red[((i * 4 + j) * 4 + e) * 256 + slot];
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + BMT / 2 * wm + 16 * i + 4 * (lane >> 4) + e;
                const int64_t n = n0 + 64 * wn + 16 * j + (lane & 15);
                if (m < M && n < N) Y[m * N + n] = g_f2h(acc[i][j][e]);
            }
}

// 2 <= M <= 64: the weight streams once and the matrix cores take the products. A block owns
// 16 weight rows (N) and all of M (MT tiles of 16 rows); its ST waves take the 32-wide K steps
// w, w + ST, ... and add their sums through LDS at the end, in wave order. Per step a lane
// reconstructs 8 consecutive codes of its row (exactly the v_mfma_f32_16x16x32_f16 B fragment
// it holds) with its X fragments. Loads run D steps ahead in a ring of raw slots (code words,
// scale, zero, X), loaded in a coalescing lane order and moved to the fragment lanes by
// ds_bpermute when used; the loop runs whole rings. Rows past N and steps past K read
// clamped (valid) units: past K their X reads zero through the buffer resource, past N their
// outputs are never stored, so the loads need no branches.
template <int NB>
struct RawUnit {                                 // the 32-bit words holding 8 codes
    static constexpr int W = NB == 3 || NB == 8 ? 2 : 1;
    uint32_t w[W];
    uint32_t j;                                  // 3-bit: position of the first code in w[0]
};

template <int NB>
__device__ __forceinline__ void raw_unit(const uint8_t *packed, int64_t u, int64_t n_words,
                                         RawUnit<NB> &r)
{
    if constexpr (NB == 3) {
        const uint32_t *wd = reinterpret_cast<const uint32_t *>(packed);
        const int64_t c0 = u * 8, w0 = c0 / 10;
        r.j = (uint32_t)(c0 - w0 * 10);
        r.w[0] = wd[w0];
        r.w[1] = wd[w0 + 1 < n_words ? w0 + 1 : w0];
    } else if constexpr (NB == 8) {
        const uint2 v = reinterpret_cast<const uint2 *>(packed)[u];
        r.w[0] = v.x;
        r.w[1] = v.y;
    } else if constexpr (NB == 4) {
        r.w[0] = reinterpret_cast<const uint32_t *>(packed)[u];
    } else if constexpr (NB == 2) {
        r.w[0] = reinterpret_cast<const uint16_t *>(packed)[u];
    } else {
        r.w[0] = packed[u];
    }
}

template <int NB>
__device__ __forceinline__ void raw_codes(const RawUnit<NB> &r, float (&c)[8])
{
    if constexpr (NB == 3) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t p = r.j + i;
            c[i] = (float)((p < 10 ? r.w[0] >> (3 * p) : r.w[1] >> (3 * (p - 10))) & 7u);
        }
    } else if constexpr (NB == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = (float)((r.w[i >> 2] >> (8 * (i & 3))) & 0xFFu);
    } else {
        constexpr int P = 8 / NB;                // planes; byte b of plane p: code b*P + p
        constexpr uint32_t m = ((1u << NB) - 1u) * 0x01010101u;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            uint32_t pl = (r.w[0] >> (NB * p)) & m;
            asm("" : "+v"(pl));                  // one byte convert per code
#pragma unroll
            for (int b = 0; b < 8 / P; ++b) c[b * P + p] = (float)((pl >> (8 * b)) & 0xFFu);
        }
    }
}

template <int NB, int MT, int ZB>
struct SkinnySlot {
    RawUnit<NB> u;
    uint32_t sv, zv;                             // raw binary16 scale; raw zero
    g4u xa[MT];
};

template <int NB, int MT, int ZB>
__global__ void __launch_bounds__(512) gemm_skinny_kernel(const uint16_t *__restrict__ X,
                                                          int64_t M, QWSet set)
{
    uint32_t blk = blockIdx.x;
    const int wi = set_pick(set, blk);
    const QW w = set.w[wi];
    uint16_t *__restrict__ const Y = set.Y[wi];
    constexpr uint32_t kOut = 0x80000000u;
    constexpr int ST = 8, D = 4;                 // waves per block; steps of loads in flight
    __shared__ float red[(ST - 1) * MT * 4 * 64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = (int64_t)blk * 16;
    // MFMA fragment layout: lane t holds row t % 16, k-piece t / 16 (8 k) of a step. Loads
    // use lane l = 4 * row + piece instead, so 4 neighbouring lanes read one contiguous run
    // (the fragment layout puts neighbours in different rows, and the texture addresser
    // then handles almost every lane as its own access); ds_bpermute moves the data over.
    const int lr = lane >> 2, lp = lane & 3;      // loading lane's row and piece
    const int src = ((lane & 15) * 4 + (lane >> 4)) * 4;   // byte address of the source lane
    const int64_t nl = n0 + lr < w.N ? n0 + lr : w.N - 1;   // loading row (clamped)
    const int64_t gpr = w.K >> w.g_log2;
    const int64_t n_words = (w.N * w.K + 9) / 10;   // 3-bit words
    const float m0 = w.meta ? g_h2f(w.meta[0]) : 0.0f, m1 = w.meta ? g_h2f(w.meta[1]) : 0.0f;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, M * w.K * 2);
    uint32_t xrow[MT];                           // byte offsets of the loading lane's X rows
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = 16 * mt + lr < M ? 16 * mt + lr : M - 1;
        xrow[mt] = (uint32_t)(m * w.K * 2);
    }
    f4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f4{0.f, 0.f, 0.f, 0.f};

    const int64_t steps = (w.K + 31) >> 5;
    using Slot = SkinnySlot<NB, MT, ZB>;
    auto load = [&](int64_t s, Slot &r) {
        const int64_t kx = s * 32 + 8 * lp;      // loading lane's k
        const bool inx = s < steps && kx < w.K;
        const int64_t kc = inx ? kx : 0;
        raw_unit<NB>(w.packed, (nl * w.K + kc) >> 3, n_words, r.u);
        const int64_t gi = nl * gpr + (kc >> w.g_log2);
        r.sv = w.scale[gi];
        if constexpr (ZB == 16) r.zv = static_cast<const uint16_t *>(w.zero)[gi];
        else r.zv = static_cast<const uint8_t *>(w.zero)[gi];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            r.xa[mt] = __builtin_amdgcn_raw_buffer_load_b128(rx, inx ? xrow[mt] + (uint32_t)(kx * 2) : kOut, 0, 0);
    };
    auto perm = [&](uint32_t v) { return (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v); };
    auto step = [&](const Slot &r0) {
        Slot r;                                  // the fragment lane's codes and X
#pragma unroll
        for (int i = 0; i < RawUnit<NB>::W; ++i) r.u.w[i] = perm(r0.u.w[i]);
        if constexpr (NB == 3) r.u.j = perm(r0.u.j);
        r.sv = perm(r0.sv);
        r.zv = perm(r0.zv);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            r.xa[mt] = g4u{perm(r0.xa[mt].x), perm(r0.xa[mt].y), perm(r0.xa[mt].z), perm(r0.xa[mt].w)};
        float c[8];
        raw_codes<NB>(r.u, c);
        const float sc = g_h2f((uint16_t)r.sv);
        const float zf = ZB == 16 ? g_h2f((uint16_t)r.zv) : fmaf((float)r.zv, m0, m1);
        uint32_t bw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            bw[i] = g_f2h2((c[2 * i] - zf) * sc, (c[2 * i + 1] - zf) * sc);
        const h8 b = __builtin_bit_cast(h8, g4u{bw[0], bw[1], bw[2], bw[3]});
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, r.xa[mt]), b, acc[mt], 0, 0, 0);
    };
    Slot ring[D];
#pragma unroll
    for (int d = 0; d < D; ++d) load(wave + (int64_t)d * ST, ring[d]);
    for (int64_t s0 = wave; s0 < steps; s0 += (int64_t)D * ST) {
#pragma unroll
        for (int d = 0; d < D; ++d) {            // steps past the end add zeros
            step(ring[d]);
            load(s0 + (int64_t)(d + D) * ST, ring[d]);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[(((wave - 1) * MT + mt) * 4 + e) * 64 + lane] = acc[mt][e];
    }
    __syncthreads();
    if (wave > 0) return;
    const int64_t n = n0 + (lane & 15);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = acc[mt][e];
#pragma unroll
            for (int v2 = 0; v2 < ST - 1; ++v2) v += red[((v2 * MT + mt) * 4 + e) * 64 + lane];
            const int64_t m = 16 * mt + 4 * (lane >> 4) + e;
            if (m < M && n < w.N) Y[m * w.N + n] = g_f2h(v);
        }
}

// Launches a kernel over the weights w[0..n) (outputs Y[0..n)), up to kMaxSet per launch:
// blocks(w) is a weight's grid, go(grid, set) the launch.
template <typename B, typename L>
void launch_sets(const QW *w, uint16_t *const *Y, int n, B blocks, L go)
{
    for (int o = 0; o < n; o += kMaxSet) {
        QWSet set{};
        uint32_t total = 0;
        for (int i = o; i < n && i < o + kMaxSet; ++i) {
            set.w[set.n] = w[i];
            set.Y[set.n] = Y[i];
            set.b0[set.n] = total;
            total += (uint32_t)blocks(w[i]);
            ++set.n;
        }
        set.b0[set.n] = total;
        if (total > 0) go(dim3(total), set);
    }
}

template <int NB, int ZB>
void launch_skinny_zb(const uint16_t *X, int64_t M, const QW *w, uint16_t *const *Y, int n,
                      hipStream_t stream)
{
    const dim3 block(512);
    auto blocks = [](const QW &q) { return (q.N + 15) / 16; };
    launch_sets(w, Y, n, blocks, [&](dim3 grid, const QWSet &set) {
        if (M <= 16) hipLaunchKernelGGL((gemm_skinny_kernel<NB, 1, ZB>), grid, block, 0, stream, X, M, set);
        else if (M <= 32) hipLaunchKernelGGL((gemm_skinny_kernel<NB, 2, ZB>), grid, block, 0, stream, X, M, set);
        else if (M <= 48) hipLaunchKernelGGL((gemm_skinny_kernel<NB, 3, ZB>), grid, block, 0, stream, X, M, set);
        else hipLaunchKernelGGL((gemm_skinny_kernel<NB, 4, ZB>), grid, block, 0, stream, X, M, set);
    });
}

template <int NB>
void launch_skinny(const uint16_t *X, int64_t M, const QW *w, uint16_t *const *Y, int n,
                   hipStream_t stream)
{
    if (w[0].zero_bits == 8) launch_skinny_zb<NB, 8>(X, M, w, Y, n, stream);
    else launch_skinny_zb<NB, 16>(X, M, w, Y, n, stream);
}

template <int NB, int ZB>
void launch_gemv2(const uint16_t *X, int64_t M, const QW *w, uint16_t *const *Y, int n,
                  hipStream_t stream)
{
    const dim3 block(256);
    const int64_t K = w[0].K;
    if (M == 1) {
        constexpr int R = kGemvRows;
        auto blocks = [](const QW &q) { return (q.N + 4 * R - 1) / (4 * R); };
        // rows of more than two chunks per lane keep three in flight (the 11008-wide rows of
        // an MLP down projection then take two load rounds instead of three; six were slower)
        launch_sets(w, Y, n, blocks, [&](dim3 grid, const QWSet &set) {
            if (((K + 2047) >> 11) > 2)
                hipLaunchKernelGGL((gemv2_kernel<NB, 1, R, ZB, 3>), grid, block, 0, stream, X, (int)M, set);
            else
                hipLaunchKernelGGL((gemv2_kernel<NB, 1, R, ZB>), grid, block, 0, stream, X, (int)M, set);
        });
        return;
    }
    auto blocks = [](const QW &q) { return (q.N + 3) / 4; };
    launch_sets(w, Y, n, blocks, [&](dim3 grid, const QWSet &set) {
        if (M == 2) hipLaunchKernelGGL((gemv2_kernel<NB, 2, 1, ZB>), grid, block, 0, stream, X, (int)M, set);
        else if (M <= 4) hipLaunchKernelGGL((gemv2_kernel<NB, 4, 1, ZB>), grid, block, 0, stream, X, (int)M, set);
        else hipLaunchKernelGGL((gemv2_kernel<NB, 8, 1, ZB>), grid, block, 0, stream, X, (int)M, set);
    });
}

// Y = X . Wr^T for a binary16 Wr [N, K] (K a multiple of 8, at most kMaxWsK).
void launch_f16(const uint16_t *X, int64_t M, const uint16_t *Wr, int64_t N, int64_t K,
                uint16_t *Y, hipStream_t stream)
{
    // 128-row tiles halve the LDS and L2 traffic per flop; 64-row tiles when the larger ones
    // would not give every CU two blocks
    const int64_t tn = (N + BN - 1) / BN;
    const bool tall = kBM16 == 128 || (kBM16 == 0 && ((M + 127) / 128) * tn >= 512);
    if (tall)
        hipLaunchKernelGGL((gemm_f16_kernel<128, kDepth, kSplitK>),
                           dim3((unsigned)(((M + 127) / 128) * tn)), dim3(256 * kSplitK), 0,
                           stream, X, M, Wr, N, K, Y);
    else
        hipLaunchKernelGGL((gemm_f16_kernel<64, kDepth, kSplitK>),
                           dim3((unsigned)(((M + 63) / 64) * tn)), dim3(256 * kSplitK), 0,
                           stream, X, M, Wr, N, K, Y);
}

// The kernel a weight takes for M rows of X (and a workspace Wr, or none).
enum GemmPath { kPathRecon, kPathSkinny, kPathGemv2, kPathGemv, kPathTiles };
template <int NB>
GemmPath path_of(const QW &w, int64_t M, const uint16_t *Wr)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(w.packed);
    if (M > kWsM && Wr && recon_fits(w.packed, NB, w.K, 1, Wr)) return kPathRecon;
    if (M > kSkinnyLo && 64 * w.K * 2 < 0x7FFFFFF0 &&
        (pa & (NB == 8 ? 7 : NB == 1 ? 0 : NB == 2 ? 1 : 3)) == 0)
        return kPathSkinny;
    if (M <= kSkinnyM && NB != 3 && (w.K * NB) % 32 == 0 && (pa & 3) == 0 &&
        M * w.K * 2 < 0x7FFFFFF0 && 4 * (w.K * NB / 8) < 0x7FFFFFF0)
        return kPathGemv2;
    return M <= kSkinnyM ? kPathGemv : kPathTiles;
}

// Weights w[0..n) of one bit width and one K, all multiplied by the same X. Those that take
// the skinny or decode kernel share launches (by zero storage); the others go one by one,
// reusing the workspace Wr in turn.
template <int NB>
void launch_nb(const uint16_t *X, int64_t M, const QW *w, uint16_t *const *Y, int n, uint16_t *Wr,
               hipStream_t stream)
{
    const int64_t K = w[0].K;
    for (const int zb : {8, 16}) {
        for (const GemmPath pth : {kPathSkinny, kPathGemv2}) {
            std::vector<QW> sw;
            std::vector<uint16_t *> sy;
            for (int i = 0; i < n; ++i)
                if (w[i].zero_bits == zb && path_of<NB>(w[i], M, Wr) == pth) {
                    sw.push_back(w[i]);
                    sy.push_back(Y[i]);
                }
            if (sw.empty()) continue;
            const int m = (int)sw.size();
            if (pth == kPathSkinny) {
                // up to 64 rows per launch; more rows (no workspace) in slices of 64
                std::vector<uint16_t *> ys(m);
                for (int64_t m0 = 0; m0 < M; m0 += 64) {
                    for (int j = 0; j < m; ++j) ys[j] = sy[j] + m0 * sw[j].N;
                    launch_skinny<NB>(X + m0 * K, M - m0 < 64 ? M - m0 : 64, sw.data(), ys.data(), m,
                                      stream);
                }
            } else if (zb == 8) {
                launch_gemv2<NB, 8>(X, M, sw.data(), sy.data(), m, stream);
            } else {
                launch_gemv2<NB, 16>(X, M, sw.data(), sy.data(), m, stream);
            }
        }
    }
    const dim3 block(256);
    for (int i = 0; i < n; ++i) {
        const QW &q = w[i];
        uint16_t *const y = Y[i];
        switch (path_of<NB>(q, M, Wr)) {
        case kPathRecon:
            launch_recon_nb<NB>(q, q.N * K, K, 1, false, Wr, stream);   // N*K: a multiple of 16
            launch_f16(X, M, Wr, q.N, K, y, stream);
            break;
        case kPathGemv: {
            const dim3 grid((unsigned)((q.N + 3) / 4));
            if (M == 1) hipLaunchKernelGGL((gemv_kernel<NB, 1>), grid, block, 0, stream, X, (int)M, q, y);
            else if (M == 2) hipLaunchKernelGGL((gemv_kernel<NB, 2>), grid, block, 0, stream, X, (int)M, q, y);
            else if (M <= 4) hipLaunchKernelGGL((gemv_kernel<NB, 4>), grid, block, 0, stream, X, (int)M, q, y);
            else hipLaunchKernelGGL((gemv_kernel<NB, 8>), grid, block, 0, stream, X, (int)M, q, y);
            break;
        }
        case kPathTiles: {
            const int64_t blocks = ((M + BM - 1) / BM) * ((q.N + BN - 1) / BN);
            hipLaunchKernelGGL((gemm_mfma_kernel<NB>), dim3((unsigned)blocks), block, 0, stream, X, M, q, y);
            break;
        }
        default:
            break;                               // launched above
        }
    }
}

}  // namespace

bool recon_fits(const void *packed, int nbits, int64_t cols, int axis, const void *out)
{
    const uintptr_t p = reinterpret_cast<uintptr_t>(packed);
    const int word = nbits == 8 ? 8 : nbits == 3 ? 4 : nbits;   // bytes per 8-code load
    return (reinterpret_cast<uintptr_t>(out) & 15) == 0 && (p & (word - 1)) == 0 &&
           (axis == 1 || cols % 8 == 0);
}

hipError_t launch_recon(const uint8_t *packed, const uint16_t *scale, const void *zero,
                        const uint16_t *zero_meta, int64_t rows, int64_t cols, int nbits, int g,
                        int zero_bits, int axis, uint16_t *out, hipStream_t stream)
{
    const int64_t n = rows * cols;
    if (n == 0) return hipSuccess;
    int lg = 0;
    while ((1 << lg) < g) ++lg;
    const QW w{packed, scale, zero, zero_bits == 8 ? zero_meta : nullptr, rows, cols, lg, zero_bits};
    switch (nbits) {
    case 1: launch_recon_nb<1>(w, n, cols, axis, true, out, stream); break;
    case 2: launch_recon_nb<2>(w, n, cols, axis, true, out, stream); break;
    case 3: launch_recon_nb<3>(w, n, cols, axis, true, out, stream); break;
    case 4: launch_recon_nb<4>(w, n, cols, axis, true, out, stream); break;
    case 8: launch_recon_nb<8>(w, n, cols, axis, true, out, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= kWsM || N <= 0 || K <= 0 || K > kMaxWsK) return 0;
    return ((size_t)N * (size_t)K * 2 + 255) & ~(size_t)255;
}

bool gemm_f16_fits(int64_t N, int64_t K) { return N > 0 && K > 0 && K % 8 == 0 && K <= kMaxWsK; }

hipError_t launch_gemm_f16(const uint16_t *X, int64_t M, const uint16_t *Wr, int64_t N, int64_t K,
                           uint16_t *Y, hipStream_t stream)
{
    launch_f16(X, M, Wr, N, K, Y, stream);
    return hipGetLastError();
}

namespace {

// Y = 0 for an empty sum (K = 0): the weight buffers may be empty or null then, so no
// multiplying kernel may run (a fill kernel rather than a memset, so that the call can be
// captured into a graph).
__global__ void __launch_bounds__(256) zero_kernel(uint16_t *__restrict__ Y, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        Y[i] = 0;
}

void launch_zero(uint16_t *Y, int64_t n, hipStream_t stream)
{
    if (n <= 0) return;
    int64_t b = (n + 255) / 256;
    if (b > 4096) b = 4096;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)b), dim3(256), 0, stream, Y, n);
}

}  // namespace

hipError_t launch_gemm(const uint16_t *X, int64_t M, const uint8_t *packed, const uint16_t *scale,
                       const void *zero, const uint16_t *zero_meta, int64_t N, int64_t K,
                       int nbits, int g, int zero_bits, uint16_t *Y, uint16_t *Wr,
                       hipStream_t stream)
{
    if (M == 0 || N == 0) return hipSuccess;
    if (K == 0) {
        launch_zero(Y, M * N, stream);
        return hipGetLastError();
    }
    int lg = 0;
    while ((1 << lg) < g) ++lg;
    const QW w{packed, scale, zero, zero_bits == 8 ? zero_meta : nullptr, N, K, lg, zero_bits};
    switch (nbits) {
    case 1: launch_nb<1>(X, M, &w, &Y, 1, Wr, stream); break;
    case 2: launch_nb<2>(X, M, &w, &Y, 1, Wr, stream); break;
    case 3: launch_nb<3>(X, M, &w, &Y, 1, Wr, stream); break;
    case 4: launch_nb<4>(X, M, &w, &Y, 1, Wr, stream); break;
    case 8: launch_nb<8>(X, M, &w, &Y, 1, Wr, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_multi(const uint16_t *X, int64_t M, int64_t K, const GemmWeight *ws, int n,
                             uint16_t *Wr, hipStream_t stream)
{
    if (M == 0) return hipSuccess;
    for (const int nbits : {1, 2, 3, 4, 8}) {
        std::vector<QW> w;
        std::vector<uint16_t *> Y;
        for (int i = 0; i < n; ++i) {
            const GemmWeight &g = ws[i];
            if (g.nbits != nbits || g.N == 0) continue;
            int lg = 0;
            while ((1 << lg) < g.group_size) ++lg;
            w.push_back(QW{g.packed, g.scale, g.zero, g.zero_bits == 8 ? g.zero_meta : nullptr, g.N,
                           K, lg, g.zero_bits});
            Y.push_back(g.Y);
        }
        if (w.empty()) continue;
        const int m = (int)w.size();
        if (K == 0) {
            for (int i = 0; i < m; ++i) launch_zero(Y[i], M * w[i].N, stream);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            continue;
        }
        switch (nbits) {
        case 1: launch_nb<1>(X, M, w.data(), Y.data(), m, Wr, stream); break;
        case 2: launch_nb<2>(X, M, w.data(), Y.data(), m, Wr, stream); break;
        case 3: launch_nb<3>(X, M, w.data(), Y.data(), m, Wr, stream); break;
        case 4: launch_nb<4>(X, M, w.data(), Y.data(), m, Wr, stream); break;
        default: launch_nb<8>(X, M, w.data(), Y.data(), m, Wr, stream); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace hqq
