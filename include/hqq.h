/*
 * hqq.h -- C ABI of the MI355X (gfx950) HQQ weight quantizer.
 *
 * The method: Half-Quadratic Quantization, a calibration-free weight quantizer. Per group of
 * `group_size` consecutive weights of a row it fixes the min-max scale, then optimises the
 * zero-point by half-quadratic splitting of an lp (p < 1) reconstruction loss: a generalized
 * soft-threshold of the residual alternates with a closed-form average for the zero, with
 * beta growing by kappa each iteration, for about 20 iterations with early stopping.
 * Sources:
 *   [TR] techreport.ngo, "Half-Quadratic Quantization of Large Machine Learning Models",
 *        sections "Outlier-aware optimization without gradients" (the solver) and
 *        "Benchmark results / Llama-2" (p = 0.7, beta = 1, kappa = 1.01, 20 iterations with
 *        early stopping; zero-point quantized to 8 bit without grouping or optimisation).
 *   [SK] "HQQ - Half-Quadratic Quantization" usage guide, sections "Core concepts /
 *        Quantization configuration" (nbits, group_size, axis) and "HQQLinear layer"
 *        (W_q, scale, zero, dequantize()).
 *
 * Conventions common to every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller. The library allocates no
 *    memory and keeps no state between calls; scratch space is the caller's `workspace`.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue work on it and
 *    never synchronise (the one exception, hqq_batch_check, says so); a device fault
 *    surfaces at the caller's next synchronisation.
 *  - Arguments are validated on the host before any HIP call. A rejected call returns a
 *    non-zero hqq_status, enqueues nothing and leaves a message in hqq_last_error().
 *  - Inputs must be finite; results for NaN/Inf weights are unspecified.
 *  - Calls are reentrant; concurrent calls need distinct workspaces and outputs.
 *  - Layouts: W is binary16, row-major [rows, cols], contiguous. With axis = 1 a group is
 *    `group_size` consecutive elements of a row, so the tensor is a flat array of
 *    n_groups = rows*cols/group_size contiguous groups, numbered in memory order. With
 *    axis = 0 a group is `group_size` consecutive elements of a column: group (b, j) is
 *    W[b*g .. b*g+g-1][j], and per-group outputs (scale, zero, passes) form a row-major
 *    [rows/g, cols] array (group (b, j) at b*cols + j). Either way the codes keep W's
 *    row-major order.
 *  - Packed codes. The pages list the bit widths 8/4/3/2/1 [SK "HQQ - Half-Quadratic
 *    Quantization", introduction] and give no storage layout; this one is the library's
 *    choice. One flat stream in memory order; code k of a container occupies bits
 *    [nbits*k, nbits*k + nbits). 8/4/2/1-bit codes fill uint8 containers (1/2/4/8 per byte);
 *    3-bit codes fill little-endian uint32 containers, 10 per word, bits 30-31 zero.
 *    Unused trailing bits are zero. Size: hqq_packed_bytes(rows*cols, nbits).
 *  - Reconstruction: W_r = (q - zero) * scale, where `scale` stores 1/s for the solver's
 *    quantizer multiplier s and `zero` the solver's zero-point (binary16), or for 8-bit
 *    zeros zero = zq * zero_meta[0] + zero_meta[1] with one binary16 pair per tensor.
 */
#ifndef HQQ_H
#define HQQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hqq_status {
    HQQ_OK = 0,
    HQQ_ERR_ARG = 1,         /* invalid argument (null, misaligned, out of range)       */
    HQQ_ERR_UNSUPPORTED = 2, /* valid for the method but not built (e.g. group_size 8)    */
    HQQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than hqq_workspace_bytes()  */
    HQQ_ERR_DEVICE = 4       /* a HIP call failed; see hqq_last_error()                  */
} hqq_status;

/* One tensor and its quantizer parameters (the single-tensor call is a batch of one).
 * Field meanings are those of hqq_quantize below. */
typedef struct hqq_job {
    const void *W;           /* binary16 [rows, cols], 16-byte aligned                     */
    int64_t rows, cols;
    int nbits;               /* 1, 2, 3, 4 or 8 [SK "Quantization configuration"]          */
    int group_size;          /* 16, 32, 64, 128 or 256; divides cols (axis 1) or rows (0)  */
    int axis;                /* 1: groups along rows; 0: down columns (see Layouts)        */
    float p, beta, kappa;    /* lp exponent (0 < p <= 1), initial beta, beta growth [TR]   */
    int iters;               /* 0..254 half-quadratic iterations; 0 = min-max RTN          */
    int early_stop;          /* 1: stop a group when its error rises; 0: run all iters     */
    int zero_bits;           /* 16: binary16 zeros; 8: uint8 zeros + per-tensor meta [TR]  */
    void *packed;            /* out: hqq_packed_bytes(rows*cols, nbits) bytes, 16-B aligned */
    void *scale;             /* out: binary16 [n_groups]                                    */
    void *zero;              /* out: binary16 [n_groups] or uint8 [n_groups]                */
    void *zero_meta;         /* out: binary16 [2] when zero_bits == 8, else NULL            */
    uint8_t *passes;         /* out, nullable: evaluations run per group (instrumentation)  */
} hqq_job;

/* Bytes of the packed code stream (the layout under "Packed codes" above, for the pages'
 * bit widths 8/4/3/2/1 [SK introduction]) for n_codes codes of nbits bits, 0 for any other
 * nbits or n_codes < 0: ceil(n*nbits/8) for 8/4/2/1 bits, 4*ceil(n/10) for 3 bits. Host
 * only; never fails otherwise. */
size_t hqq_packed_bytes(int64_t n_codes, int nbits);

/* Workspace bytes hqq_quantize_batch needs for these jobs (host array): the device copy of
 * the job table and its work counters, binary32 zero staging and per-tensor (min, max) for
 * 8-bit zero requantization, the words that 3-bit groups share, and for each axis-0 job a
 * transposed copy of its weights and outputs (about 2 + nbits/8 bytes per weight); 0 if
 * every tensor is empty. Returns SIZE_MAX if a job is invalid; the quantize call then reports why. */
size_t hqq_workspace_bytes(const hqq_job *jobs, int n_jobs);

/* Quantize one tensor [TR "Outlier-aware optimization without gradients"].
 * Per group: s = qmax/(max - min), z0 = -min*s (binary32), then up to `iters` iterations of
 *   W_e = sign(r)*max(|r| - |r|^(p-1)/beta, 0), r = W - (q - z)/s  (generalized soft-threshold)
 *   z   = mean(q - (W - W_e)*s)                                      (closed-form zero update)
 *   beta = beta*kappa, q = clamp(round(W*s + z), 0, 2^nbits - 1)
 * keeping the iterate with the lowest mean |W - (q - z)/s| and stopping when it rises
 * (early_stop). Per-element arithmetic is exact; the zero is rounded to binary32 at each
 * update. Outputs: packed codes, scale = binary16(1/s), zero (see hqq_job), passes.
 * workspace: device buffer (256-byte aligned) of at least hqq_workspace_bytes() for this one
 * job (it holds the device job table; NULL only for an empty tensor). With zero_bits == 8
 * its first 4*n_groups bytes hold, after the call, the binary32 zeros the solver returned
 * (before 8-bit requantization; for axis 0 in column-major group order, j*(rows/g) + b). */
hqq_status hqq_quantize(const void *W, int64_t rows, int64_t cols, int nbits, int group_size,
                        int axis, float p, float beta, float kappa, int iters, int early_stop,
                        int zero_bits, void *packed, void *scale, void *zero, void *zero_meta,
                        uint8_t *passes, void *workspace, size_t workspace_bytes, void *stream);

/* hqq_quantize without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as hqq_quantize; it calls no hipMalloc, hipFree or
 * allocating library routine. Its scratch is one static device array of 64 MiB that every
 * GPU the library runs on holds until the process ends; the tensor's hqq_workspace_bytes()
 * must fit it (every tensor of the model-shaped stacks at axis 1 does; axis 0 takes about
 * 2 + nbits/8 bytes per weight), else HQQ_ERR_WORKSPACE and nothing is enqueued. All calls
 * on one GPU share that array and the next call overwrites it: calls that overlap on one GPU
 * (concurrent streams, or threads) race and must be ordered by the caller. */
hqq_status hqq_quantize_noalloc(const void *W, int64_t rows, int64_t cols, int nbits,
                                int group_size, int axis, float p, float beta, float kappa,
                                int iters, int early_stop, int zero_bits, void *packed,
                                void *scale, void *zero, void *zero_meta, uint8_t *passes,
                                void *stream);

/* Quantize several tensors with one launch sequence (e.g. every linear layer of a model
 * stack). `jobs` is a host array, read during the call only; every job is validated first.
 * Jobs may mix nbits and group sizes; each job's output is what hqq_quantize writes. */
hqq_status hqq_quantize_batch(const hqq_job *jobs, int n_jobs, void *workspace,
                              size_t workspace_bytes, void *stream);

/* The two steps of hqq_quantize_batch, callable separately (e.g. to time them apart).
 * hqq_solve_batch runs the group solver for every job: it writes packed codes, scale,
 * passes and, for zero_bits == 16, the binary16 zeros; for zero_bits == 8 it leaves the
 * binary32 zeros and their per-tensor reduction inputs in the workspace.
 * hqq_requant_batch then quantizes those zeros to 8 bit [TR "Benchmark results / Llama-2"]
 * and writes zero and zero_meta, joins the 3-bit words two groups share, and writes every
 * output of axis-0 jobs (solved in transposed order) back in the tensor's order. It must be
 * given the same jobs and workspace, after hqq_solve_batch on the same stream. */
hqq_status hqq_solve_batch(const hqq_job *jobs, int n_jobs, void *workspace,
                           size_t workspace_bytes, void *stream);
hqq_status hqq_requant_batch(const hqq_job *jobs, int n_jobs, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Completion check of the last solve on a workspace. Every solver wave bounds its loop
 * steps by a budget the schedule never reaches, so that a defect ends the launch instead of
 * hanging it; a wave that runs out sets a status word in the workspace (cleared by the next
 * solve on that workspace) and leaves some groups of the batch unwritten. This call takes
 * the same jobs and workspace as the solve, waits for `stream` to complete (it is the one
 * synchronising call of this library), and returns HQQ_ERR_DEVICE with a message when the
 * flag is set or the stream reports an error, HQQ_OK otherwise. Argument errors as for
 * hqq_quantize_batch. */
hqq_status hqq_batch_check(const hqq_job *jobs, int n_jobs, const void *workspace,
                           size_t workspace_bytes, void *stream);

/* Diagnostic hook for tests; the settings apply to every solver launch made afterwards, by
 * any thread. step_budget > 0 gives each solver wave a fixed budget of that many loop steps
 * (0 restores the default): with a small budget the solver ends early, every wave still
 * exits normally, and hqq_batch_check reports the incomplete batch. pass_layout selects the
 * solver kernel: 0 by the size of the batch (the default), 1 the persistent solver with one
 * lane per group (wide), 2 the persistent solver with several lanes per group (narrow), 3 the
 * lockstep solver (one wave per tile; the default for small batches); results are identical,
 * only the speed differs. */
void hqq_debug_solver(int64_t step_budget, int pass_layout);

/* Quantize a batch whose weights live in HOST memory, for stacks larger than the device
 * memory [SK "Common issues": when quantization runs out of memory, load the layers one after
 * another; TR "Speed: from hours to minutes": each weight crosses to the GPU once]. jobs[i].W is a host pointer (allocate it pinned, e.g. with
 * hipHostMalloc, for the copy to overlap the solve; pageable memory works but serialises);
 * every output pointer is a device pointer, as for hqq_quantize_batch, with the same results.
 * Consecutive jobs are cut into chunks whose weights fit half of `staging` (a device buffer,
 * 256-byte aligned; each tensor takes 2*rows*cols bytes rounded up to 256): chunk k is
 * copied into half k % 2 on `copy_stream` while chunk k-1 is solved on `stream`.
 * `workspace` must hold hqq_streamed_workspace_bytes(jobs, n_jobs, staging_bytes). The
 * call enqueues only (it creates five HIP events and releases them before returning); the
 * host weights must stay valid and unchanged until `stream` has completed the work. A
 * tensor larger than half the staging buffer -> HQQ_ERR_WORKSPACE. copy_stream may equal
 * stream (no overlap). The first copy into each half waits for all work enqueued on
 * `stream` before the call, so consecutive calls may share one staging buffer. */
hqq_status hqq_quantize_streamed(const hqq_job *jobs, int n_jobs, void *staging,
                                 size_t staging_bytes, void *workspace, size_t workspace_bytes,
                                 void *stream, void *copy_stream);

/* Workspace bytes hqq_quantize_streamed needs with a staging buffer of staging_bytes (the
 * largest chunk's batch workspace); SIZE_MAX if a job is invalid or does not fit. */
size_t hqq_streamed_workspace_bytes(const hqq_job *jobs, int n_jobs, size_t staging_bytes);

/* Reconstruct binary16 weights [SK "HQQLinear layer", dequantize()]:
 * W_out = binary16((q - zero_f) * scale), zero_f the binary16 zero or, for zero_bits == 8,
 * zq * zero_meta[0] + zero_meta[1] (one fused rounding), with each element's group found
 * by `axis`. Same layouts as hqq_quantize. */
hqq_status hqq_dequantize(const void *packed, const void *scale, const void *zero,
                          const void *zero_meta, int64_t rows, int64_t cols, int nbits,
                          int group_size, int axis, int zero_bits, void *W_out, void *stream);

/* 8-bit scales [TR "Benchmark results / Llama-2", the note on the HQQ_g16_s row: that
 * variant also stores its scales on 8-bit grids, one per 128 scales]. Quantizes n binary16 scales (e.g. the `scale`
 * output of hqq_quantize, one per weight group, in group order) in runs of `scale_group`
 * consecutive scales (the last run shorter when scale_group does not divide n). Each run m
 * gets the min-max affine uint8 rule of 8-bit zeros, with no optimisation:
 *   step = binary16((vmax - vmin)/255) (1 if that is 0), base = binary16(vmin),
 *   scale_q[i] = clamp(rne((v_i - base)/step), 0, 255)       (binary32 operations),
 *   scale_meta[2m] = step, scale_meta[2m + 1] = base.
 * The weight codes are not re-derived. scale: binary16 [n], 16-byte aligned; scale_q:
 * uint8 [n], 8-byte aligned; scale_meta: binary16 [2*ceil(n/scale_group)], 4-byte aligned.
 * scale_group: a power of two in [8, 512] (128 on the pages). n = 0 does nothing. */
hqq_status hqq_requant_scales(const void *scale, int64_t n, int scale_group, uint8_t *scale_q,
                              void *scale_meta, void *stream);

/* Read back 8-bit scales as binary16 scales for hqq_dequantize:
 * scale_out[i] = binary16(fma(scale_q[i], step, base)) with run i/scale_group's pair, the
 * fma in binary32. Same layouts as hqq_requant_scales; scale_out is 16-byte aligned. */
hqq_status hqq_dequantize_scales(const uint8_t *scale_q, const void *scale_meta, int64_t n,
                                 int scale_group, void *scale_out, void *stream);

/* The linear layer of a quantized weight [SK "HQQLinear layer": the layer computes with the
 * dequantized weight]: Y[M, N] = X[M, K] . W_r^T, where W_r [N, K] is exactly what
 * hqq_dequantize reconstructs from an axis-1 quantized weight (rows N, cols K, same packed /
 * scale / zero / zero_meta layouts); products of binary16 values are accumulated in binary32
 * (in any order) and Y is rounded to binary16. X: binary16 row-major [M, K], 16-byte aligned;
 * Y: binary16 row-major [M, N]. Up to M = 64 the packed weight streams once per call (M = 1
 * on the vector units, 2..64 on the matrix cores); larger M without a workspace streams it
 * once per 64 rows of X.
 * workspace (optional, device, 16-byte aligned, caller-owned): with M > 64 and at least
 * hqq_gemm_workspace_bytes(M, N, K) bytes, W_r is reconstructed once into it and a plain
 * binary16 matrix-core GEMM reads it (the faster choice for large M); NULL keeps the
 * streaming kernels. A non-NULL workspace that is too small is HQQ_ERR_WORKSPACE. Its
 * contents are scratch; calls that share one race. Packed buffers that are not 4-byte
 * aligned (8 bytes at 8 bits) take slower fallback kernels, with or without a workspace.
 * K = 0 (an empty sum) writes Y = 0; X, packed, scale, zero and zero_meta may then be NULL.
 * M = 0 or N = 0 does nothing. */
hqq_status hqq_gemm(const void *X, int64_t M, const void *packed, const void *scale,
                    const void *zero, const void *zero_meta, int64_t N, int64_t K, int nbits,
                    int group_size, int zero_bits, void *Y, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Workspace bytes for hqq_gemm's reconstruct-once path: 2*N*K rounded up to 256 for M > 64,
 * else 0 (no workspace is used). */
size_t hqq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* One weight of hqq_gemm_multi: hqq_gemm's per-weight arguments, and its output. */
typedef struct hqq_gemm_weight {
    const void *packed;      /* packed codes of the axis-1 quantized weight [N, K] */
    const void *scale;       /* binary16 [N*K/group_size] */
    const void *zero;        /* binary16, or uint8 with zero_bits == 8 */
    const void *zero_meta;   /* binary16 {step, base} with zero_bits == 8, else ignored */
    int64_t N;               /* rows of the weight = columns of its Y */
    int nbits;               /* 1, 2, 3, 4 or 8 */
    int group_size;          /* 16, 32, 64, 128 or 256 */
    int zero_bits;           /* 16 or 8 */
    void *Y;                 /* binary16 row-major [M, N] */
} hqq_gemm_weight;

/* Several linear layers that read one input [SK "HQQLinear layer", as hqq_gemm]: for each
 * weight i, Y_i = X . W_r,i^T, bit for bit what hqq_gemm(X, M, weight i, K, Y_i) writes (the
 * same kernel computes each weight's outputs the same way). Weights that share a bit width
 * and zero storage and take the streaming kernels (M <= 64, word-aligned packed buffers)
 * are multiplied by shared launches, up to eight weights each, so that layers such as an
 * attention block's q, k and v projections, or an MLP's gate and up projections, fill the
 * GPU together rather than one after another; the others are launched one by one. Every
 * weight is [N_i, K] with the same K; X as in hqq_gemm; the Y_i must not overlap each other
 * or X. n_weights = 0, M = 0 or N_i = 0 do nothing for those weights; K = 0 writes Y_i = 0
 * (X and the weight buffers may then be NULL). workspace: as in
 * hqq_gemm, at least the largest hqq_gemm_workspace_bytes(M, N_i, K), used by one weight
 * after another; too small is HQQ_ERR_WORKSPACE. Argument errors name the weight; nothing is
 * launched when any weight is invalid. Nothing is allocated on the device. */
hqq_status hqq_gemm_multi(const void *X, int64_t M, int64_t K, const hqq_gemm_weight *weights,
                          int n_weights, void *workspace, size_t workspace_bytes, void *stream);

/* The same layer in two steps [SK "HQQLinear layer": the layer computes with the dequantized
 * weight]: given Wr, the binary16 weight [N, K] that hqq_dequantize wrote, Y[M, N] = X[M, K] .
 * Wr^T with binary32 sums (any order) rounded to binary16, on the matrix-core kernel of
 * hqq_gemm's reconstruct-once path (for the same Wr, the two give identical Y). For callers
 * that keep Wr resident and multiply it many times, so the reconstruction is paid once.
 * X and Wr: binary16 row-major, 16-byte aligned; Y: binary16 row-major [M, N],
 * 2-byte aligned. K: a positive multiple of 8, at most 2^22, else HQQ_ERR_ARG. M = 0 or N = 0
 * does nothing. Nothing is allocated; the call only enqueues on `stream`. */
hqq_status hqq_gemm_f16(const void *X, int64_t M, const void *Wr, int64_t N, int64_t K, void *Y,
                        void *stream);

/* The bit-packing of the quantized weight W_q [SK "HQQLinear layer": W_q holds the packed
 * codes; bit widths 8/4/3/2/1 from its introduction], standalone: pack n_codes uint8 codes
 * (device, each < 2^nbits) into the layout under "Packed codes" above. `packed` (device,
 * caller-owned) must be 16-byte aligned and hold hqq_packed_bytes(n_codes, nbits) bytes; the
 * unused bits of the last container are written as zero and nothing past it is touched.
 * Codes >= 2^nbits are masked to their low nbits bits. nbits outside {1,2,3,4,8},
 * n_codes < 0, null pointers or a misaligned `packed` -> HQQ_ERR_ARG; n_codes = 0 does
 * nothing. Enqueues one kernel on `stream`. */
hqq_status hqq_pack(const uint8_t *codes, int64_t n_codes, int nbits, void *packed,
                    void *stream);

/* Inverse of hqq_pack [same passages]: reads hqq_packed_bytes(n_codes, nbits) bytes of
 * `packed` (device; 4-byte aligned for 3 bits) and writes n_codes uint8 codes (device,
 * caller-owned) in stream order. Argument errors as for hqq_pack. */
hqq_status hqq_unpack(const void *packed, int64_t n_codes, int nbits, uint8_t *codes,
                      void *stream);

/* Static text for a status code. */
const char *hqq_status_string(hqq_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char *hqq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HQQ_H */
