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
// 8-bit zero-point [techreport.ngo, "Half-Quadratic Quantization of Large Machine Learning
// Models", section "Benchmark results / Llama-2": the zero-point is quantized to 8 bit with
// no further grouping or optimisation]. One min-max affine uint8 round-to-nearest quantizer
// over all zeros of the tensor, on the grid of its stored binary16 pair:
//   step = binary16((zmax - zmin)/255) (1 if that is 0), base = binary16(zmin),
//   zq = clamp(rne((z - base)/step), 0, 255), meta = {step, base}; read back zq*step + base.
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) zero_minmax_kernel(const float2 *partials, int64_t n,
                                                           float4 *quant, uint16_t *meta)
{
    __shared__ float2 red[16];
    float lo = INFINITY, hi = -INFINITY;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        float2 p = partials[i];
        lo = fminf(lo, p.x);
        hi = fmaxf(hi, p.y);
    }
    for (int o = 1; o < 64; o <<= 1) {
        lo = fminf(lo, __shfl_xor(lo, o));
        hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(lo, hi);
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) {
            lo = fminf(lo, red[w].x);
            hi = fmaxf(hi, red[w].y);
        }
        uint16_t h_step = f2h((hi - lo) / 255.0f);
        float step = h2f(h_step);
        if (!(step > 0.0f)) {
            h_step = 0x3c00;                        // binary16 1.0
            step = 1.0f;
        }
        const uint16_t h_base = f2h(lo);
        *quant = make_float4(step, h2f(h_base), lo, hi);
        meta[0] = h_step;
        meta[1] = h_base;
    }
}

__global__ void __launch_bounds__(256) zero_quant_kernel(const float *z, int64_t n,
                                                         const float4 *quant, uint8_t *zq)
{
    const float4 qp = *quant;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v = rintf((z[i] - qp.y) / qp.x);
        zq[i] = (uint8_t)fminf(fmaxf(v, 0.0f), 255.0f);
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

hipError_t launch_zero_requant(const float *zero32, int64_t n_groups, const float2 *partials,
                               int64_t n_partials, float4 *quant, uint8_t *zq, uint16_t *meta,
                               hipStream_t stream)
{
    if (n_groups == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_minmax_kernel, dim3(1), dim3(1024), 0, stream, partials,
                       n_partials, quant, meta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(zero_quant_kernel, dim3(grid_for(n_groups, 256 * 4)), dim3(256), 0,
                       stream, zero32, n_groups, (const float4 *)quant, zq);
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
