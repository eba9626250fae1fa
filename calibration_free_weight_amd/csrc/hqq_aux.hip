// hqq_aux.hip -- zero-point requantization, dequantization, pack and unpack for gfx950.
//
// Packed layout (the pages list the bit widths 8/4/3/2/1 and give no layout; the containers
// are this library's choice): a flat code stream in memory order,
// code k of a container in bits [nbits*k, nbits*k + nbits); uint8 containers for 8/4/2/1
// bits, little-endian uint32 containers of ten 3-bit codes with bits 30-31 zero.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <type_traits>

#include "hqq_internal.h"

namespace hqq {
namespace {

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
// binary32 -> binary16, round to nearest even, of an already rounded binary32 value. The
// empty asm hides how f was computed: otherwise the compiler folds a binary32 multiply or fma
// feeding the conversion into one mixed-precision instruction (v_fma_mixlo_f16) that rounds
// the exact result to binary16 once, which differs from rounding to binary32 first whenever
// the binary32 value is a binary16 tie.
__device__ __forceinline__ uint16_t f2h(float f)
{
    asm("" : "+v"(f));
    return __half_as_ushort(__float2half_rn(f));
}

// ---------------------------------------------------------------------------------------
// After the solve, per batch: 8-bit zero-points and the 3-bit words shared by two groups.
//
// 8-bit zero-point [techreport.ngo, "Half-Quadratic Quantization of Large Machine Learning
// Models", section "Benchmark results / Llama-2": the zero-point is quantized to 8 bit with
// no further grouping or optimisation]. One min-max affine uint8 round-to-nearest quantizer
// over all zeros of the tensor, on the grid of its stored binary16 pair:
//   step = binary16((zmax - zmin)/255) (1 if that is 0), base = binary16(zmin),
//   zq = clamp(rne((z - base)/step), 0, 255), meta = {step, base}; read back zq*step + base.
// The solver leaves each tensor's (zmin, zmax) as order-preserving integer keys, in
// kMinmaxSlots copies that this kernel reduces once per job.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float unkey(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// A block takes kFinishRounds rounds of 256 x kFinishPerThread items; in a round a thread
// takes kFinishPerThread items 256 apart and issues all their loads before any store, so
// the memory latency is paid once per round rather than once per item.
constexpr int kFinishPerThread = 8;
constexpr int kFinishRounds = 2;
constexpr int64_t kFinishPerBlock = 256 * kFinishPerThread * kFinishRounds;

// One job's view for the finish kernel, held in registers: the kernel's stores cannot then
// force the job descriptor to be reloaded for every item.
struct FinishJob {
    const float *zero32;
    uint8_t *zq;
    uint16_t *meta;
    const uint2 *stash;
    uint32_t *packed;
    int64_t item0, end;
    uint32_t g;
    uint16_t h_step, h_base;
    float step, basef;
};

__device__ __forceinline__ FinishJob finish_job(const DevJob &J, int64_t end, uint32_t kmin,
                                                uint32_t kmax)
{
    FinishJob f;
    f.zero32 = J.zero32;
    f.zq = J.zq;
    f.meta = J.meta;
    f.stash = J.stash;
    f.packed = reinterpret_cast<uint32_t *>(J.packed);
    f.item0 = J.item0;
    f.end = end;
    f.g = (uint32_t)J.g;
    const float zmin = unkey(kmin), zmax = unkey(kmax);
    f.h_step = f2h((zmax - zmin) / 255.0f);
    f.step = h2f(f.h_step);
    if (!(f.step > 0.0f)) {
        f.h_step = 0x3c00;                          // binary16 1.0
        f.step = 1.0f;
    }
    f.h_base = f2h(zmin);
    f.basef = h2f(f.h_base);
    return f;
}

// The 8-bit code of a zero on the tensor's grid.
__device__ __forceinline__ uint8_t zero_code(const FinishJob &f, float z)
{
    const float v = rintf((z - f.basef) / f.step);
    return (uint8_t)fminf(fmaxf(v, 0.0f), 255.0f);
}

// Group i's 3-bit code stream starts inside a 10-code word that group i - 1 ends in.
__device__ __forceinline__ bool shares_word(const FinishJob &f, uint32_t i)
{
    return i >= 1 && ((i % 10u) * (f.g % 10u)) % 10u != 0;
}

__device__ __forceinline__ void finish_item(const FinishJob &f, int64_t item)
{
    const uint32_t i = (uint32_t)(item - f.item0);  // a group index (< 2^32 per tensor)
    if (f.zq) {
        f.zq[i] = zero_code(f, f.zero32[i]);
        if (i == 0) {
            f.meta[0] = f.h_step;
            f.meta[1] = f.h_base;
        }
    }
    if (f.stash && shares_word(f, i)) {
        const int64_t w = (int64_t)i * f.g / 10;
        f.packed[w] = f.stash[i - 1].x | f.stash[i].y;
    }
}

// One round of kFinishPerThread items that all belong to job f: every load first, then the
// codes and the joined words.
__device__ __forceinline__ void finish_round(const FinishJob &f, int64_t item)
{
    constexpr int P = kFinishPerThread;
    uint32_t i[P];
#pragma unroll
    for (int k = 0; k < P; ++k) i[k] = (uint32_t)(item + 256 * k - f.item0);
    if (f.zq) {
        float z[P];
#pragma unroll
        for (int k = 0; k < P; ++k) z[k] = __builtin_nontemporal_load(f.zero32 + i[k]);
#pragma unroll
        for (int k = 0; k < P; ++k) f.zq[i[k]] = zero_code(f, z[k]);
        if (i[0] == 0) {
            f.meta[0] = f.h_step;
            f.meta[1] = f.h_base;
        }
    }
    if (f.stash) {
        uint32_t word[P];
        bool join[P];
#pragma unroll
        for (int k = 0; k < P; ++k) {
            join[k] = shares_word(f, i[k]);
            word[k] = join[k] ? f.stash[i[k] - 1].x | f.stash[i[k]].y : 0u;
        }
#pragma unroll
        for (int k = 0; k < P; ++k)
            if (join[k]) f.packed[(int64_t)i[k] * f.g / 10] = word[k];
    }
}

__global__ void __launch_bounds__(256) finish_kernel(const DevJob *table, int n_jobs,
                                                     int64_t n_items)
{
    __shared__ int job_sh;
    __shared__ uint32_t grid_sh[2];                 // job_sh's (min, max) keys, reduced
    const int64_t base = (int64_t)blockIdx.x * kFinishPerBlock;
    if (threadIdx.x < 64) {
        // The last job with item0 <= base: the first wave tests 64 jobs per step, with
        // independent loads (item0 rises with the job index).
        int last = 0;
        for (int j0 = 0; j0 < n_jobs; j0 += 64) {
            const int j = j0 + (int)threadIdx.x;
            const uint64_t m = __ballot(j < n_jobs && table[j].item0 <= base);
            if (m == 0) break;
            last = j0 + 63 - __builtin_clzll(m);
            if (m != ~0ull) break;
        }
        // The first wave then reduces that job's key copies once for the block (one per lane).
        uint32_t kmin = 0xffffffffu, kmax = 0u;
        if (table[last].zq && threadIdx.x < kMinmaxSlots) {
            kmin = table[last].minmax[kMinmaxStride * threadIdx.x];
            kmax = table[last].minmax[kMinmaxStride * threadIdx.x + 1];
        }
        for (int d = 32; d >= 1; d >>= 1) {
            kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, d));
            kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d));
        }
        if (threadIdx.x == 0) {
            job_sh = last;
            grid_sh[0] = kmin;
            grid_sh[1] = kmax;
        }
    }
    __syncthreads();
    const int j0 = job_sh;
    const FinishJob f0 =
        finish_job(table[j0], j0 + 1 < n_jobs ? table[j0 + 1].item0 : n_items, grid_sh[0], grid_sh[1]);
    int j = j0;
    for (int r = 0; r < kFinishRounds; ++r) {
        const int64_t rbase = base + (int64_t)r * 256 * kFinishPerThread;
        if (rbase + 256 * kFinishPerThread <= f0.end) {   // the whole round in the first job
            finish_round(f0, rbase + threadIdx.x);
            continue;
        }
        for (int k = 0; k < kFinishPerThread; ++k) {
            const int64_t item = rbase + (int64_t)k * 256 + threadIdx.x;
            if (item >= n_items) break;
            if (item < f0.end) {
                finish_item(f0, item);
                continue;
            }
            // a later job in this block: its descriptor and key copies straight from memory
            while (j + 1 < n_jobs && table[j + 1].item0 <= item) ++j;
            uint32_t kmin = 0xffffffffu, kmax = 0u;
            if (table[j].zq)
                for (int p = 0; p < kMinmaxSlots; ++p) {
                    kmin = min(kmin, table[j].minmax[kMinmaxStride * p]);
                    kmax = max(kmax, table[j].minmax[kMinmaxStride * p + 1]);
                }
            const FinishJob fj =
                finish_job(table[j], j + 1 < n_jobs ? table[j + 1].item0 : n_items, kmin, kmax);
            finish_item(fj, item);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Code extraction helpers
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t get_code(const uint8_t *packed, int64_t k, int nbits)
{
    if (nbits == 3) {
        uint32_t w = reinterpret_cast<const uint32_t *>(packed)[k / 10];
        return (w >> (3 * (int)(k % 10))) & 7u;
    }
    const int64_t bit = k * nbits;
    return (uint32_t)(packed[bit >> 3] >> (bit & 7)) & ((1u << nbits) - 1u);
}

// Dequantize [usage guide "HQQ - Half-Quadratic Quantization", section "HQQLinear layer",
// dequantize()]: W_r = binary16((q - zero) * scale). One thread per 16 codes (3 bits: per
// 10-code word).
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t *packed,
                                                      const uint16_t *scale, const void *zero,
                                                      const uint16_t *meta, int64_t n,
                                                      int nbits, int g, int zero_bits,
                                                      int64_t cols, int axis, uint16_t *out)
{
    const int per = nbits == 3 ? 10 : 16;
    const int64_t chunks = (n + per - 1) / per;
    float m0 = 0.0f, m1 = 0.0f;
    if (zero_bits == 8) {
        m0 = h2f(meta[0]);
        m1 = h2f(meta[1]);
    }
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t k0 = c * per;
        for (int j = 0; j < per; ++j) {
            const int64_t k = k0 + j;
            if (k >= n) break;
            // axis 1: group k/g; axis 0: group (row/g, col) of a [rows/g, cols] array
            const int64_t gi = axis == 1 ? k / g : (k / cols / g) * cols + k % cols;
            const float zf = zero_bits == 16
                                 ? h2f(reinterpret_cast<const uint16_t *>(zero)[gi])
                                 : fmaf((float)reinterpret_cast<const uint8_t *>(zero)[gi], m0, m1);
            const float v = ((float)get_code(packed, k, nbits) - zf) * h2f(scale[gi]);
            out[k] = f2h(v);
        }
    }
}

// Pack: one thread per container group (16 codes = 2*nbits bytes, or one 3-bit word).
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t *codes, int64_t n, int nbits,
                                                   uint8_t *packed)
{
    const uint32_t mask = (1u << nbits) - 1u;
    if (nbits == 3) {
        const int64_t words = (n + 9) / 10;
        for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words;
             w += (int64_t)gridDim.x * blockDim.x) {
            uint32_t word = 0;
            for (int k = 0; k < 10; ++k) {
                const int64_t c = w * 10 + k;
                if (c < n) word |= (codes[c] & mask) << (3 * k);
            }
            reinterpret_cast<uint32_t *>(packed)[w] = word;
        }
        return;
    }
    const int64_t nbytes = (n * nbits + 7) / 8;
    const int64_t chunks = (n + 15) / 16;
    for (int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ch < chunks;
         ch += (int64_t)gridDim.x * blockDim.x) {
        uint32_t bits[4] = {0u, 0u, 0u, 0u};      // 16 codes * nbits <= 128 bits
        for (int j = 0; j < 16; ++j) {
            const int64_t c = ch * 16 + j;
            if (c >= n) break;
            const int bit = j * nbits;
            bits[bit >> 5] |= (codes[c] & mask) << (bit & 31);
        }
        const int64_t b0 = ch * 2 * nbits;         // first byte of this chunk
        for (int b = 0; b < 2 * nbits; ++b) {
            if (b0 + b >= nbytes) break;
            packed[b0 + b] = (uint8_t)(bits[b >> 2] >> (8 * (b & 3)));
        }
    }
}

__global__ void __launch_bounds__(256) unpack_kernel(const uint8_t *packed, int64_t n,
                                                     int nbits, uint8_t *codes)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n;
         k += (int64_t)gridDim.x * blockDim.x)
        codes[k] = (uint8_t)get_code(packed, k, nbits);
}

// ---------------------------------------------------------------------------------------
// 8-bit scales [techreport.ngo, "Half-Quadratic Quantization of Large Machine Learning
// Models", section "Benchmark results / Llama-2", note on the HQQ_g16_s row: that
// variant also stores its scales on 8-bit grids, one per 128 scales]. Each run of SG consecutive binary16
// scales gets the min-max affine uint8 rule of the 8-bit zero-point:
//   step = binary16((vmax - vmin)/255) (1 if that is 0), base = binary16(vmin),
//   q = clamp(rne((v - base)/step), 0, 255), meta[2m..2m+1] = {step, base} of run m.
// A lane holds 8 consecutive scales (one 16-byte load), so LPG = SG/8 neighbouring lanes
// of one wave hold a run and reduce its min / max with LPG-wide butterflies. HBM-bound: it
// reads 2 B and writes 1 B per scale plus 4 B per run.
// ---------------------------------------------------------------------------------------
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

constexpr int kScaleUnroll = 4;                 // 512-scale tiles in flight per wave

template <int LPG>
__global__ void __launch_bounds__(256) scale_requant_kernel(const uint16_t *__restrict__ scale,
                                                            int64_t n, uint8_t *__restrict__ sq,
                                                            uint16_t *__restrict__ meta)
{
    constexpr int SG = 8 * LPG, U = kScaleUnroll;
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t n_waves = (int64_t)gridDim.x * 4;
    // The loop bound is per wave: every lane of a wave runs the butterflies together.
    for (int64_t t0 = wave * U; t0 * 512 < n; t0 += n_waves * U) {
        v4u w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {           // all loads first
            const int64_t e0 = ((t0 + u) * 64 + lane) * 8;
            if (e0 + 8 <= n) {
                w[u] = *reinterpret_cast<const v4u *>(scale + e0);
            } else {                            // a ragged end: absent scales read as NaN
                uint32_t h[4] = {0x7e007e00u, 0x7e007e00u, 0x7e007e00u, 0x7e007e00u};
                for (int i = 0; i < 8 && e0 + i < n; ++i)
                    h[i >> 1] = (h[i >> 1] & (i & 1 ? 0x0000ffffu : 0xffff0000u)) |
                                (uint32_t)scale[e0 + i] << (16 * (i & 1));
                w[u] = v4u{h[0], h[1], h[2], h[3]};
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e0 = ((t0 + u) * 64 + lane) * 8;
            const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = h2f((uint16_t)(i & 1 ? ws[i >> 1] >> 16 : ws[i >> 1]));
            float vmin = INFINITY, vmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; ++i) {      // fminf / fmaxf skip the NaN of absent scales
                vmin = fminf(vmin, v[i]);
                vmax = fmaxf(vmax, v[i]);
            }
#pragma unroll
            for (int off = LPG / 2; off >= 1; off /= 2) {
                vmin = fminf(vmin, __shfl_xor(vmin, off));
                vmax = fmaxf(vmax, __shfl_xor(vmax, off));
            }
            if (e0 >= n) continue;              // no scale here (the butterflies are done)
            uint16_t h_step = f2h((vmax - vmin) / 255.0f);
            float step = h2f(h_step);
            if (!(step > 0.0f)) {
                h_step = 0x3c00;                // binary16 1.0
                step = 1.0f;
            }
            const uint16_t h_base = f2h(vmin);
            const float base = h2f(h_base);
            // The code is rne of the binary32 quotient (v - base)/step, clamped to [0, 255].
            // Quotient by the correctly rounded reciprocal and one fused correction: within a
            // few ulps of the binary32 quotient (x >= 0, step a normal binary32 number, no
            // overflow), so both round to the same integer unless the quotient is within
            // 2^-14 (at least 4 ulps below 256) of a half-integer; those take the division.
            const float rcp = 1.0f / step;
            float q[8];
            bool near = false;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = v[i] - base;
                const float q0 = x * rcp;
                q[i] = fmaf(fmaf(-q0, step, x), rcp, q0);
                near |= fabsf(fabsf(q[i] - rintf(q[i])) - 0.5f) <= 0x1p-14f;
            }
            if (near) {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = (v[i] - base) / step;
            }
            // v_cvt_pk_u8_f32: round half to even, saturate to [0, 255]
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo = __builtin_amdgcn_cvt_pk_u8_f32(q[i], i, lo);
                hi = __builtin_amdgcn_cvt_pk_u8_f32(q[i + 4], i, hi);
            }
            if (e0 + 8 <= n) {
                *reinterpret_cast<v2u *>(sq + e0) = v2u{lo, hi};
            } else {
                for (int i = 0; i < 8 && e0 + i < n; ++i)
                    sq[e0 + i] = (uint8_t)((i < 4 ? lo : hi) >> (8 * (i & 3)));
            }
            if (lane % LPG == 0)
                reinterpret_cast<uint32_t *>(meta)[e0 / SG] =
                    (uint32_t)h_step | (uint32_t)h_base << 16;
        }
    }
}

// Read-back of 8-bit scales: binary16(fma(q, step, base)) in binary32, 8 scales per lane,
// kScaleUnroll chunks in flight per thread.
__global__ void __launch_bounds__(256) scale_dequant_kernel(const uint8_t *__restrict__ sq,
                                                            const uint16_t *__restrict__ meta,
                                                            int64_t n, int sg_log2,
                                                            uint16_t *__restrict__ out)
{
    constexpr int U = kScaleUnroll;
    const int64_t T = (int64_t)gridDim.x * 256;
    for (int64_t c0 = (int64_t)blockIdx.x * 256 + threadIdx.x; c0 * 8 < n; c0 += T * U) {
        v2u w[U];
        uint32_t mm[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e0 = (c0 + u * T) * 8;
            w[u] = v2u{0u, 0u};
            mm[u] = 0;
            if (e0 + 8 <= n) w[u] = *reinterpret_cast<const v2u *>(sq + e0);
            if (e0 < n) mm[u] = reinterpret_cast<const uint32_t *>(meta)[e0 >> sg_log2];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e0 = (c0 + u * T) * 8;
            if (e0 >= n) break;
            const float step = h2f((uint16_t)mm[u]), base = h2f((uint16_t)(mm[u] >> 16));
            if (e0 + 8 <= n) {
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t b = i < 2 ? w[u].x : w[u].y;
                    const int sh = 16 * (i & 1);
                    o[i] = (uint32_t)f2h(fmaf((float)((b >> sh) & 0xffu), step, base)) |
                           (uint32_t)f2h(fmaf((float)((b >> (sh + 8)) & 0xffu), step, base)) << 16;
                }
                *reinterpret_cast<v4u *>(out + e0) = v4u{o[0], o[1], o[2], o[3]};
            } else {
                for (int i = 0; i < 8 && e0 + i < n; ++i)
                    out[e0 + i] = f2h(fmaf((float)sq[e0 + i], step, base));
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Transposes of row-major [R, C] arrays to [C, R] (axis-0 grouping runs the group solver on
// the transposed weights and writes its outputs back in the tensor's order). One launch
// serves a list of arrays (the tensors of a batch): its 64 x 64 tiles are numbered across
// the list, and each block finds its array by binary search. Reads and writes are whole
// 64-element tile rows.
// ---------------------------------------------------------------------------------------
enum XSub { kXGen16, kXWhole16, kXGen8, kXCodes1, kXCodes2, kXCodes4, kXCodes8, kXWide1,
            kXWide2, kXWide4, kXWide8, kXNib4 };

struct XTaskDev {
    const void *src;
    void *dst;
    int64_t R, C, tile0;
    int sub;
};
constexpr int kXTasks = 48;
struct XArgs {
    XTaskDev t[kXTasks];
    int n;
    int64_t tiles;
};

template <typename T>
__device__ void xtile_generic(const T *__restrict__ src, int64_t R, int64_t C, T *__restrict__ dst,
                              int64_t r0, int64_t c0, T (*tile)[65])
{
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int64_t r = r0 + ty + 4 * k, c = c0 + tx;
        if (r < R && c < C) tile[ty + 4 * k][tx] = src[r * C + c];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int64_t c = c0 + ty + 4 * k, r = r0 + tx;
        if (r < R && c < C) dst[c * R + r] = tile[tx][ty + 4 * k];
    }
}

// binary16, whole tiles (R and C multiples of 64): 8-byte loads and stores, 16 threads per
// 128-byte tile row.
__device__ void xtile_whole16(const uint16_t *__restrict__ src, int64_t R, int64_t C,
                              uint16_t *__restrict__ dst, int64_t r0, int64_t c0,
                              uint16_t (*tile)[68])
{
    const int q = threadIdx.x & 15, w = threadIdx.x >> 4;    // 4-element quad, row
    v2u in[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        in[k] = *reinterpret_cast<const v2u *>(src + (r0 + w + 16 * k) * C + c0 + 4 * q);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint16_t *row = &tile[w + 16 * k][4 * q];
        row[0] = (uint16_t)in[k].x;
        row[1] = (uint16_t)(in[k].x >> 16);
        row[2] = (uint16_t)in[k].y;
        row[3] = (uint16_t)(in[k].y >> 16);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = w + 16 * k;                              // output row = input column
        const v2u o = {(uint32_t)tile[4 * q][c] | (uint32_t)tile[4 * q + 1][c] << 16,
                       (uint32_t)tile[4 * q + 2][c] | (uint32_t)tile[4 * q + 3][c] << 16};
        *reinterpret_cast<v2u *>(dst + (c0 + c) * R + r0 + 4 * q) = o;
    }
}

// Packed NB-bit codes of [C, R] (row-major stream) to the packed stream of [R, C], for NB in
// {1, 2, 4, 8} when every row of both streams starts on a byte (R*NB, C*NB multiples of 8);
// WIDE: on a 4-byte boundary (multiples of 32), moved as 32-bit words. Here R, C and the
// tile origin (r0, c0) are those of the output.
template <int NB, bool WIDE>
__device__ void xtile_codes(const uint8_t *__restrict__ src, int64_t R, int64_t C,
                            uint8_t *__restrict__ dst, int64_t r0, int64_t c0,
                            uint8_t (*tile)[65])
{
    using W = typename std::conditional<WIDE, uint32_t, uint8_t>::type;
    constexpr int PER = 8 * (int)sizeof(W) / NB;   // codes per word
    constexpr int RB = 64 / PER;                // words per 64-code tile row
    // source row c (output column c) holds output rows r0.. as RB words
    for (int e = threadIdx.x; e < 64 * RB; e += 256) {
        const int cc = e / RB, b = e % RB;
        const int64_t c = c0 + cc, r = r0 + (int64_t)b * PER;
        if (c < C && r < R) {
            const uint32_t v = reinterpret_cast<const W *>(src)[(c * R + r) * NB / 8 / sizeof(W)];
#pragma unroll
            for (int u = 0; u < PER; ++u) tile[cc][b * PER + u] = (v >> (NB * u)) & ((1u << NB) - 1u);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * RB; e += 256) {
        const int rr = e / RB, b = e % RB;
        const int64_t r = r0 + rr, c = c0 + (int64_t)b * PER;
        if (r < R && c < C) {
            uint32_t v = 0;
#pragma unroll
            for (int u = 0; u < PER; ++u) v |= (uint32_t)tile[b * PER + u][rr] << (NB * u);
            reinterpret_cast<W *>(dst)[(r * C + c) * NB / 8 / sizeof(W)] = (W)v;
        }
    }
}

// 4-bit codes with R and C multiples of 8 (the usual case): 128 x 128 output tiles. Each
// thread loads an 8 x 8 block of codes as eight 32-bit words (one per source row), transposes
// it in registers in three swap stages (16-, 8- and 4-bit fields), and writes the eight
// output words to LDS; the output rows then leave as 16-byte stores (4-byte ones when C is
// not a multiple of 32). A wave's loads are 64-byte runs of four source rows.
__device__ __forceinline__ void swap_fields(uint32_t &a, uint32_t &b, int sh, uint32_t keep)
{
    const uint32_t na = (a & keep) | ((b << sh) & ~keep);
    const uint32_t nb = ((a >> sh) & keep) | (b & ~keep);
    a = na;
    b = nb;
}

__device__ void xtile_nib4(const uint8_t *__restrict__ src, int64_t R, int64_t C,
                           uint8_t *__restrict__ dst, int64_t r0, int64_t c0, uint32_t *tile)
{
    constexpr int P = 17;                       // LDS row pitch in words (16 + 1)
    const int t = threadIdx.x, rb = t & 15, cb = t >> 4;
    const int64_t r = r0 + rb * 8, c = c0 + cb * 8;
    uint32_t w[8];
    if (r < R && c < C) {                       // R, C multiples of 8: blocks are whole
        const uint32_t *s32 = reinterpret_cast<const uint32_t *>(src);
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = s32[((c + j) * R + r) >> 3];
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = 0u;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) swap_fields(w[j], w[j + 4], 16, 0x0000FFFFu);
#pragma unroll
    for (int j = 0; j < 8; j += 4) {
        swap_fields(w[j], w[j + 2], 8, 0x00FF00FFu);
        swap_fields(w[j + 1], w[j + 3], 8, 0x00FF00FFu);
    }
#pragma unroll
    for (int j = 0; j < 8; j += 2) swap_fields(w[j], w[j + 1], 4, 0x0F0F0F0Fu);
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[(rb * 8 + i) * P + cb] = w[i];   // output row r + i
    __syncthreads();
    const bool wide = C % 32 == 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int u = t + 256 * h, rr = u >> 2, q = u & 3;
        const int64_t orow = r0 + rr, oc = c0 + 32 * q;
        if (orow >= R || oc >= C) continue;
        uint32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = tile[rr * P + 4 * q + k];
        uint32_t *d32 = reinterpret_cast<uint32_t *>(dst + ((orow * C + oc) >> 1));
        if (wide) {
            *reinterpret_cast<uint4 *>(d32) = uint4{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (oc + 8 * k < C) d32[k] = v[k];
        }
    }
}

__global__ void __launch_bounds__(256) xpose_kernel(XArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[64 * 68];
    for (int64_t tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
        int lo = 0, hi = a.n - 1;               // last task whose first tile <= tile
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.t[mid].tile0 <= tile) lo = mid;
            else hi = mid - 1;
        }
        const XTaskDev T = a.t[lo];
        // tiles cover the output for codes ([R, C]) and the input otherwise ([R, C] -> [C, R]);
        // 128 x 128 for 4-bit codes in whole 8 x 8 blocks, 64 x 64 otherwise
        const int ts = T.sub == kXNib4 ? 128 : 64;
        const int64_t lt = tile - T.tile0, tc = (T.C + ts - 1) / ts;
        const int64_t r0 = (lt / tc) * ts, c0 = (lt % tc) * ts;
        const uint8_t *s8 = static_cast<const uint8_t *>(T.src);
        uint8_t *d8 = static_cast<uint8_t *>(T.dst);
        auto t8 = reinterpret_cast<uint8_t (*)[65]>(lds);
        switch (T.sub) {
        case kXGen16:
            xtile_generic(static_cast<const uint16_t *>(T.src), T.R, T.C,
                          static_cast<uint16_t *>(T.dst), r0, c0,
                          reinterpret_cast<uint16_t (*)[65]>(lds));
            break;
        case kXWhole16:
            xtile_whole16(static_cast<const uint16_t *>(T.src), T.R, T.C,
                          static_cast<uint16_t *>(T.dst), r0, c0,
                          reinterpret_cast<uint16_t (*)[68]>(lds));
            break;
        case kXGen8: xtile_generic(s8, T.R, T.C, d8, r0, c0, t8); break;
        case kXCodes1: xtile_codes<1, false>(s8, T.R, T.C, d8, r0, c0, t8); break;
        case kXCodes2: xtile_codes<2, false>(s8, T.R, T.C, d8, r0, c0, t8); break;
        case kXCodes4: xtile_codes<4, false>(s8, T.R, T.C, d8, r0, c0, t8); break;
        case kXCodes8: xtile_codes<8, false>(s8, T.R, T.C, d8, r0, c0, t8); break;
        case kXWide1: xtile_codes<1, true>(s8, T.R, T.C, d8, r0, c0, t8); break;
        case kXWide2: xtile_codes<2, true>(s8, T.R, T.C, d8, r0, c0, t8); break;
        case kXWide4: xtile_codes<4, true>(s8, T.R, T.C, d8, r0, c0, t8); break;
        case kXNib4: xtile_nib4(s8, T.R, T.C, d8, r0, c0, reinterpret_cast<uint32_t *>(lds)); break;
        default: xtile_codes<8, true>(s8, T.R, T.C, d8, r0, c0, t8); break;
        }
        __syncthreads();                        // the tile buffer is reused by the next tile
    }
}

unsigned grid_for(int64_t items, int per_block)
{
    int64_t b = (items + per_block - 1) / per_block;
    if (b > 65536) b = 65536;
    return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_finish(const DevJob *table, int n_jobs, int64_t n_items, hipStream_t stream)
{
    if (n_items == 0 || n_jobs == 0) return hipSuccess;
    const int64_t blocks = (n_items + kFinishPerBlock - 1) / kFinishPerBlock;
    hipLaunchKernelGGL(finish_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, table, n_jobs,
                       n_items);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *packed, const uint16_t *scale, const void *zero,
                          const uint16_t *meta, int64_t n, int nbits, int g, int zero_bits,
                          int64_t cols, int axis, uint16_t *out, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const int per = nbits == 3 ? 10 : 16;
    hipLaunchKernelGGL(dequant_kernel, dim3(grid_for((n + per - 1) / per, 256)), dim3(256), 0,
                       stream, packed, scale, zero, meta, n, nbits, g, zero_bits, cols, axis,
                       out);
    return hipGetLastError();
}

hipError_t launch_pack(const uint8_t *codes, int64_t n, int nbits, uint8_t *packed,
                       hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const int per = nbits == 3 ? 10 : 16;
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for((n + per - 1) / per, 256)), dim3(256), 0,
                       stream, codes, n, nbits, packed);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t n, int nbits, uint8_t *codes,
                         hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, packed, n,
                       nbits, codes);
    return hipGetLastError();
}

hipError_t launch_scale_requant(const uint16_t *scale, int64_t n, int scale_group, uint8_t *sq,
                                uint16_t *meta, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const dim3 grid(grid_for((n + 511) / 512 / kScaleUnroll * 64, 256)), block(256);
    switch (scale_group) {
    case 8: hipLaunchKernelGGL(scale_requant_kernel<1>, grid, block, 0, stream, scale, n, sq, meta); break;
    case 16: hipLaunchKernelGGL(scale_requant_kernel<2>, grid, block, 0, stream, scale, n, sq, meta); break;
    case 32: hipLaunchKernelGGL(scale_requant_kernel<4>, grid, block, 0, stream, scale, n, sq, meta); break;
    case 64: hipLaunchKernelGGL(scale_requant_kernel<8>, grid, block, 0, stream, scale, n, sq, meta); break;
    case 128: hipLaunchKernelGGL(scale_requant_kernel<16>, grid, block, 0, stream, scale, n, sq, meta); break;
    case 256: hipLaunchKernelGGL(scale_requant_kernel<32>, grid, block, 0, stream, scale, n, sq, meta); break;
    case 512: hipLaunchKernelGGL(scale_requant_kernel<64>, grid, block, 0, stream, scale, n, sq, meta); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_scale_dequant(const uint8_t *sq, const uint16_t *meta, int64_t n,
                                int scale_group, uint16_t *out, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    int lg = 0;
    while ((1 << lg) < scale_group) ++lg;
    hipLaunchKernelGGL(scale_dequant_kernel, dim3(grid_for((n + 7) / 8 / kScaleUnroll, 256)), dim3(256), 0,
                       stream, sq, meta, n, lg, out);
    return hipGetLastError();
}

bool codes_transpose_fused(int nbits, int64_t R, int64_t C)
{
    return nbits != 3 && (R * nbits) % 8 == 0 && (C * nbits) % 8 == 0;
}

hipError_t launch_transposes(const XTask *tasks, int n, hipStream_t stream)
{
    auto al = [](const void *p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; };
    for (int o = 0; o < n; o += kXTasks) {
        XArgs a{};
        int64_t tiles = 0;
        for (int i = o; i < n && i < o + kXTasks; ++i) {
            const XTask &t = tasks[i];
            if (t.R == 0 || t.C == 0) continue;
            XTaskDev d{t.src, t.dst, t.R, t.C, tiles, 0};
            if (t.kind == kX16) {
                const bool whole = t.R % 64 == 0 && t.C % 64 == 0 && al(t.src, 8) && al(t.dst, 8);
                d.sub = whole ? kXWhole16 : kXGen16;
            } else if (t.kind == kX8) {
                d.sub = kXGen8;
            } else {
                if (!codes_transpose_fused(t.nbits, t.R, t.C)) return hipErrorInvalidValue;
                const bool wide = (t.R * t.nbits) % 32 == 0 && (t.C * t.nbits) % 32 == 0 &&
                                  al(t.src, 4) && al(t.dst, 4);
                const int lg = t.nbits == 1 ? 0 : t.nbits == 2 ? 1 : t.nbits == 4 ? 2 : 3;
                d.sub = (wide ? kXWide1 : kXCodes1) + lg;
                if (t.nbits == 4 && t.R % 8 == 0 && t.C % 8 == 0 && al(t.src, 4) &&
                    al(t.dst, t.C % 32 == 0 ? 16 : 4))
                    d.sub = kXNib4;
            }
            const int ts = d.sub == kXNib4 ? 128 : 64;
            tiles += ((t.R + ts - 1) / ts) * ((t.C + ts - 1) / ts);
            a.t[a.n++] = d;
        }
        a.tiles = tiles;
        if (a.n == 0) continue;
        const unsigned grid = (unsigned)(tiles < 65536 ? tiles : 65536);
        hipLaunchKernelGGL(xpose_kernel, dim3(grid), dim3(256), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace hqq
