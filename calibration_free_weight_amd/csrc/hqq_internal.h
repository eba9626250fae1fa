// hqq_internal.h -- declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hqq {

constexpr int kMaxIters = 254;      // passes are counted in uint8 (1..iters+1)
// Copies of each tensor's (min, max) of the binary32 zeros: many small waves updating one
// pair of words with atomics serialise on its cache line, so each wave takes the pair of its
// slot, one slot per 128-byte line, and the requant kernel reduces the copies.
constexpr int kMinmaxSlots = 64;
constexpr int kMinmaxStride = 32;   // uint32 words between slots

// One tensor as the device kernels see it (the job table lives in the caller's workspace).
struct DevJob {
    const uint16_t *W;          // binary16 weights, n_groups * g elements
    uint8_t *packed;            // packed code stream
    uint16_t *scale;            // binary16 [n_groups]
    uint16_t *zero16;           // binary16 zeros, or nullptr for 8-bit zeros
    float *zero32;              // binary32 zero staging for 8-bit zeros, or nullptr
    uint8_t *passes;            // nullable
    uint2 *stash;               // 3-bit: partial boundary words per group, or nullptr
    uint32_t *minmax;           // 8-bit zeros: kMinmaxSlots pairs of order-preserving keys
                                // {min, max}, kMinmaxStride words apart; a wave updates the
                                // pair of its slot
    uint8_t *zq;                // 8-bit zeros out
    uint16_t *meta;             // 8-bit zeros: binary16 {step, base} out
    int64_t n_groups;
    int64_t tile0;              // first tile of this job in its launch class
    int64_t item0;              // first item of this job in the finish kernel's index space
    int32_t nbits, g;
};

// One persistent solver launch: jobs that share nbits, g and the solver parameters.
struct StreamArgs {
    const DevJob *jobs;         // this class's jobs, ordered by tile0
    int n_jobs;
    int64_t n_tiles;
    float p, beta0, kappa;
    int iters, early_stop;
    uint32_t *counter;          // tile claim counter, zero before the launch
    uint32_t chunk;             // tiles per claim
    uint32_t *status;           // bit 0 set by a wave that ran out of its step budget
    int64_t budget0;            // a wave's loop-step budget at start
    int64_t budget_tile;        // and what each tile it takes in adds
};

// Sets the calling thread's hqq_last_error() text and returns `status` (for entry points
// defined outside hqq_api.hip).
int report_error(int status, const char *msg);

// Diagnostic settings of the solver launches. Step budget of the waves: 0 selects the
// default (a bound the schedule never reaches); a positive value replaces the starting
// budget and stops its growth per tile. Pass layout: 0 chosen by size, 1 wide, 2 narrow.
void set_solver_debug(int64_t steps, int layout);
int64_t step_budget();
int solver_layout();

constexpr int kFillJobs = 24;   // job descriptors per table-fill launch (kernel arguments)
struct FillArgs {
    DevJob jobs[kFillJobs];
    int n, offset;
    uint32_t *counters;         // zeroed by the launch with offset 0
    int n_counters;
};

// Launch configuration of the solver for one class.
int64_t tiles_for(int64_t n_groups, int g);
hipError_t launch_fill(const FillArgs &f, DevJob *table, hipStream_t stream);
hipError_t launch_stream(const StreamArgs &a, int nbits, int g, hipStream_t stream);
// 8-bit zeros (per job min/max from the solver, then uint8 codes + meta) and 3-bit boundary
// words, over all jobs of a batch: items [0, n_items) map to jobs by DevJob::item0.
hipError_t launch_finish(const DevJob *table, int n_jobs, int64_t n_items, hipStream_t stream);

hipError_t launch_dequant(const uint8_t *packed, const uint16_t *scale, const void *zero,
                          const uint16_t *meta, int64_t n, int nbits, int g, int zero_bits,
                          int64_t cols, int axis, uint16_t *out, hipStream_t stream);

// Transposes of row-major arrays, many per launch. kX16 / kX8: [R, C] -> [C, R] of 2- or
// 1-byte elements. kXCodes: the packed nbits-bit code stream of a [C, R] array -> that of
// [R, C] (R, C of the output), only when codes_transpose_fused(nbits, R, C): 8/4/2/1 bits
// with every row starting on a byte.
enum XKind { kX16, kX8, kXCodes };
struct XTask {
    const void *src;
    void *dst;
    int64_t R, C;
    XKind kind;
    int nbits;
};
bool codes_transpose_fused(int nbits, int64_t R, int64_t C);
hipError_t launch_transposes(const XTask *tasks, int n, hipStream_t stream);

// Y[M, N] = X[M, K] . W_r^T for a packed axis-1 quantized weight [N, K] (binary16 X, Y).
// Flat reconstruction of a packed weight into binary16 (hqq_dequantize's fast path): needs
// recon_fits (16-byte aligned output, packed aligned to one 8-code load, and for axis 0 cols
// a multiple of 8); n = rows*cols is then a multiple of 8.
bool recon_fits(const void *packed, int nbits, int64_t cols, int axis, const void *out);
hipError_t launch_recon(const uint8_t *packed, const uint16_t *scale, const void *zero,
                        const uint16_t *zero_meta, int64_t rows, int64_t cols, int nbits, int g,
                        int zero_bits, int axis, uint16_t *out, hipStream_t stream);
// Y = X . Wr^T with a binary16 Wr [N, K] on the matrix cores; gemm_f16_fits(N, K) must hold
bool gemm_f16_fits(int64_t N, int64_t K);
hipError_t launch_gemm_f16(const uint16_t *X, int64_t M, const uint16_t *Wr, int64_t N, int64_t K,
                           uint16_t *Y, hipStream_t stream);
// Wr: binary16 [N, K] workspace of gemm_workspace_bytes(M, N, K) bytes, or nullptr
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const uint16_t *X, int64_t M, const uint8_t *packed, const uint16_t *scale,
                       const void *zero, const uint16_t *zero_meta, int64_t N, int64_t K,
                       int nbits, int g, int zero_bits, uint16_t *Y, uint16_t *Wr,
                       hipStream_t stream);
// Several weights [N_i, K] multiplied by the same X (each exactly as launch_gemm would): the
// weights that take the decode or skinny kernels share launches. Wr as in launch_gemm, large
// enough for every weight that uses it (used in turn).
struct GemmWeight {
    const uint8_t *packed;
    const uint16_t *scale;
    const void *zero;
    const uint16_t *zero_meta;
    int64_t N;
    int nbits, group_size, zero_bits;
    uint16_t *Y;
};
hipError_t launch_gemm_multi(const uint16_t *X, int64_t M, int64_t K, const GemmWeight *w, int n,
                             uint16_t *Wr, hipStream_t stream);

// 8-bit scales: scale_group a power of two in [8, 512]; buffers 16-byte aligned (meta 4).
hipError_t launch_scale_requant(const uint16_t *scale, int64_t n, int scale_group, uint8_t *sq,
                                uint16_t *meta, hipStream_t stream);
hipError_t launch_scale_dequant(const uint8_t *sq, const uint16_t *meta, int64_t n,
                                int scale_group, uint16_t *out, hipStream_t stream);

hipError_t launch_pack(const uint8_t *codes, int64_t n, int nbits, uint8_t *packed,
                       hipStream_t stream);

hipError_t launch_unpack(const uint8_t *packed, int64_t n, int nbits, uint8_t *codes,
                         hipStream_t stream);

}  // namespace hqq
