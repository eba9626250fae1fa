// hqq_aux.hip -- zero-point requantization, dequantization, pack and unpack for gfx950.
//
// Packed layout (the pages name only the containers): a flat code stream in memory order,
// code k of a container in bits [nbits*k, nbits*k + nbits); uint8 containers for 8/4/2/1
// bits, little-endian uint32 containers of ten 3-bit codes with bits 30-31 zero.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "hqq_internal.h"

namespace hqq {
namespace {

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

// ---------------------------------------------------------------------------------------
// After the solve, per batch: 8-bit zero-points and the 3-bit words shared by two groups.
//
// 8-bit zero-point [techreport.ngo, "Half-Quadratic Quantization of Large Machine Learning
// Models", section "Benchmark results / Llama-2": the zero-point is quantized to 8 bit with
// no further grouping or optimisation]. One min-max affine uint8 round-to-nearest quantizer
// over all zeros of the tensor, on the grid of its stored binary16 pair:
//   step = binary16((zmax - zmin)/255) (1 if that is 0), base = binary16(zmin),
//   zq = clamp(rne((z - base)/step), 0, 255), meta = {step, base}; read back zq*step + base.
// The solver leaves each tensor's (zmin, zmax) as order-preserving integer keys.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float unkey(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

constexpr int kFinishPerThread = 8;

__global__ void __launch_bounds__(256) finish_kernel(const DevJob *table, int n_jobs,
                                                     int64_t n_items)
{
    __shared__ int job_sh;
    const int64_t base = (int64_t)blockIdx.x * 256 * kFinishPerThread;
    if (threadIdx.x == 0) {
        int lo = 0, hi = n_jobs - 1;                // last job with item0 <= base
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (table[mid].item0 <= base) lo = mid;
            else hi = mid - 1;
        }
        job_sh = lo;
    }
    __syncthreads();
    int j = job_sh;
    for (int r = 0; r < kFinishPerThread; ++r) {
        const int64_t item = base + (int64_t)r * 256 + threadIdx.x;
        if (item >= n_items) break;
        while (j + 1 < n_jobs && table[j + 1].item0 <= item) ++j;
        const DevJob &J = table[j];
        const int64_t i = item - J.item0;
        if (J.zq) {
            const float zmin = unkey(J.minmax[0]), zmax = unkey(J.minmax[1]);
            uint16_t h_step = f2h((zmax - zmin) / 255.0f);
            float step = h2f(h_step);
            if (!(step > 0.0f)) {
                h_step = 0x3c00;                    // binary16 1.0
                step = 1.0f;
            }
            const uint16_t h_base = f2h(zmin);
            const float v = rintf((J.zero32[i] - h2f(h_base)) / step);
            J.zq[i] = (uint8_t)fminf(fmaxf(v, 0.0f), 255.0f);
            if (i == 0) {
                J.meta[0] = h_step;
                J.meta[1] = h_base;
            }
        }
        if (J.stash && i >= 1 && (i * J.g) % 10 != 0) {
            const int64_t w = i * J.g / 10;
            reinterpret_cast<uint32_t *>(J.packed)[w] = J.stash[i - 1].x | J.stash[i].y;
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
                                                      uint16_t *out)
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
            const int64_t gi = k / g;
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
    const int64_t per_block = 256 * kFinishPerThread;
    const int64_t blocks = (n_items + per_block - 1) / per_block;
    hipLaunchKernelGGL(finish_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, table, n_jobs,
                       n_items);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *packed, const uint16_t *scale, const void *zero,
                          const uint16_t *meta, int64_t n, int nbits, int g, int zero_bits,
                          uint16_t *out, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const int per = nbits == 3 ? 10 : 16;
    hipLaunchKernelGGL(dequant_kernel, dim3(grid_for((n + per - 1) / per, 256)), dim3(256), 0,
                       stream, packed, scale, zero, meta, n, nbits, g, zero_bits, out);
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

}  // namespace hqq
