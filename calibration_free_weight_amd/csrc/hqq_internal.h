// hqq_internal.h -- declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hqq {

constexpr int kMaxIters = 254;      // passes are counted in uint8 (1..iters+1)

// Arguments of one solver launch (one tensor).
struct SolveArgs {
    const uint16_t *W;              // binary16 bits, n_groups * G elements
    int64_t n_groups;
    float p, beta0, kappa;
    int iters, early_stop;
    uint8_t *packed;                // packed code stream
    uint16_t *scale;                // binary16 [n_groups]
    uint16_t *zero16;               // binary16 zeros (zero_bits == 16) or nullptr
    float *zero32;                  // binary32 zero staging (zero_bits == 8) or nullptr
    uint8_t *passes;                // nullable
    float2 *partials;               // per-block (min, max) of zero32, or nullptr
};

// Number of blocks the solver launch uses for n_groups groups of size g at nbits.
int64_t solve_blocks(int64_t n_groups, int g, int nbits);

hipError_t launch_solve(const SolveArgs &a, int nbits, int g, hipStream_t stream);

// 8-bit zero requantization: reduce the solver's per-block partials to the tensor's
// (zmin, zmax), derive the affine uint8 quantizer and the binary16 meta pair, then quantize.
hipError_t launch_zero_requant(const float *zero32, int64_t n_groups, const float2 *partials,
                               int64_t n_partials, float4 *quant, uint8_t *zq,
                               uint16_t *meta, hipStream_t stream);

hipError_t launch_dequant(const uint8_t *packed, const uint16_t *scale, const void *zero,
                          const uint16_t *meta, int64_t n, int nbits, int g, int zero_bits,
                          uint16_t *out, hipStream_t stream);

hipError_t launch_pack(const uint8_t *codes, int64_t n, int nbits, uint8_t *packed,
                       hipStream_t stream);

hipError_t launch_unpack(const uint8_t *packed, int64_t n, int nbits, uint8_t *codes,
                         hipStream_t stream);

}  // namespace hqq
