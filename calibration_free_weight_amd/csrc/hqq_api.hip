// hqq_api.hip -- the C ABI declared in include/hqq.h: argument validation (on the host,
// before any HIP call), workspace planning and kernel dispatch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "hqq.h"
#include "hqq_internal.h"

namespace {

thread_local std::string g_last_error;

hqq_status fail(hqq_status s, const std::string &msg)
{
    g_last_error = msg;
    return s;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool valid_bits(int nbits) { return nbits == 1 || nbits == 2 || nbits == 3 || nbits == 4 || nbits == 8; }
bool built_group(int g) { return g == 16 || g == 32 || g == 64 || g == 128 || g == 256; }

size_t packed_bytes(int64_t n, int nbits)
{
    if (n < 0 || !valid_bits(nbits)) return 0;
    if (nbits == 3) return (size_t)(4 * ((n + 9) / 10));
    return (size_t)((n * nbits + 7) / 8);
}

std::string job_name(int i) { return i < 0 ? std::string("") : "job " + std::to_string(i) + ": "; }

// Shape and parameter checks shared by quantize and dequantize.
hqq_status check_layout(int64_t rows, int64_t cols, int nbits, int group_size, int axis,
                        const std::string &who)
{
    if (rows < 0 || cols < 0) return fail(HQQ_ERR_ARG, who + "rows and cols must be >= 0");
    if (rows > 0 && cols > (int64_t(1) << 40) / rows)
        return fail(HQQ_ERR_ARG, who + "rows*cols too large");
    if (!valid_bits(nbits)) return fail(HQQ_ERR_ARG, who + "nbits must be 1, 2, 3, 4 or 8");
    if (axis == 0)
        return fail(HQQ_ERR_UNSUPPORTED, who + "axis=0 (groups down columns) is not built");
    if (axis != 1) return fail(HQQ_ERR_ARG, who + "axis must be 0 or 1");
    if (group_size <= 0) return fail(HQQ_ERR_ARG, who + "group_size must be > 0");
    if (cols % group_size != 0) return fail(HQQ_ERR_ARG, who + "group_size must divide cols");
    if (!built_group(group_size))
        return fail(HQQ_ERR_UNSUPPORTED, who + "group_size must be 16, 32, 64, 128 or 256");
    return HQQ_OK;
}

hqq_status check_job(const hqq_job &j, int idx)
{
    const std::string who = job_name(idx);
    hqq_status st = check_layout(j.rows, j.cols, j.nbits, j.group_size, j.axis, who);
    if (st != HQQ_OK) return st;
    if (!(std::isfinite(j.p) && j.p > 0.0f && j.p <= 1.0f))
        return fail(HQQ_ERR_ARG, who + "p must satisfy 0 < p <= 1");
    if (!(std::isfinite(j.beta) && j.beta > 0.0f)) return fail(HQQ_ERR_ARG, who + "beta must be > 0");
    if (!(std::isfinite(j.kappa) && j.kappa > 0.0f))
        return fail(HQQ_ERR_ARG, who + "kappa must be > 0");
    if (j.iters < 0 || j.iters > hqq::kMaxIters)
        return fail(HQQ_ERR_ARG, who + "iters must be in [0, 254]");
    if (j.early_stop != 0 && j.early_stop != 1)
        return fail(HQQ_ERR_ARG, who + "early_stop must be 0 or 1");
    if (j.zero_bits != 8 && j.zero_bits != 16)
        return fail(HQQ_ERR_ARG, who + "zero_bits must be 8 or 16");
    if (j.rows * j.cols == 0) return HQQ_OK;
    if (!j.W || !j.packed || !j.scale || !j.zero)
        return fail(HQQ_ERR_ARG, who + "W, packed, scale and zero must be non-null");
    if (j.zero_bits == 8 && !j.zero_meta)
        return fail(HQQ_ERR_ARG, who + "zero_meta must be non-null when zero_bits == 8");
    if (!aligned(j.W, 16)) return fail(HQQ_ERR_ARG, who + "W must be 16-byte aligned");
    if (!aligned(j.packed, 16)) return fail(HQQ_ERR_ARG, who + "packed must be 16-byte aligned");
    if (!aligned(j.scale, 2)) return fail(HQQ_ERR_ARG, who + "scale must be 2-byte aligned");
    if (j.zero_bits == 16 && !aligned(j.zero, 2))
        return fail(HQQ_ERR_ARG, who + "zero must be 2-byte aligned");
    if (j.zero_bits == 8 && !aligned(j.zero_meta, 2))
        return fail(HQQ_ERR_ARG, who + "zero_meta must be 2-byte aligned");
    return HQQ_OK;
}

// Workspace of one job: binary32 zero staging, the solver's per-block (min, max) and the
// derived quantizer, each section 256-byte aligned. Nothing for binary16 zeros.
size_t job_workspace(const hqq_job &j)
{
    if (j.zero_bits != 8 || j.rows * j.cols == 0) return 0;
    const int64_t ng = j.rows * j.cols / j.group_size;
    const int64_t nb = hqq::solve_blocks(ng, j.group_size, j.nbits);
    return round_up(sizeof(float) * (size_t)ng) + round_up(sizeof(float2) * (size_t)nb) +
           round_up(sizeof(float4));
}

hqq_status device_fail(hipError_t e, const std::string &what)
{
    return fail(HQQ_ERR_DEVICE, what + ": " + hipGetErrorString(e));
}

struct JobWs {
    float *zero32 = nullptr;
    float2 *partials = nullptr;
    float4 *quant = nullptr;
};

JobWs job_ws(const hqq_job &j, char *ws)
{
    JobWs r;
    if (j.zero_bits != 8 || j.rows * j.cols == 0) return r;
    const int64_t ng = j.rows * j.cols / j.group_size;
    const int64_t nb = hqq::solve_blocks(ng, j.group_size, j.nbits);
    r.zero32 = reinterpret_cast<float *>(ws);
    r.partials = reinterpret_cast<float2 *>(ws + round_up(sizeof(float) * (size_t)ng));
    r.quant = reinterpret_cast<float4 *>(ws + round_up(sizeof(float) * (size_t)ng) +
                                         round_up(sizeof(float2) * (size_t)nb));
    return r;
}

hqq_status solve_job(const hqq_job &j, char *ws, hipStream_t stream)
{
    const int64_t n = j.rows * j.cols;
    if (n == 0) return HQQ_OK;
    hqq::SolveArgs a{};
    a.W = static_cast<const uint16_t *>(j.W);
    a.n_groups = n / j.group_size;
    a.p = j.p;
    a.beta0 = j.beta;
    a.kappa = j.kappa;
    a.iters = j.iters;
    a.early_stop = j.early_stop;
    a.packed = static_cast<uint8_t *>(j.packed);
    a.scale = static_cast<uint16_t *>(j.scale);
    a.passes = j.passes;
    const JobWs w = job_ws(j, ws);
    if (j.zero_bits == 8) {
        a.zero32 = w.zero32;
        a.partials = w.partials;
    } else {
        a.zero16 = static_cast<uint16_t *>(j.zero);
    }
    hipError_t e = hqq::launch_solve(a, j.nbits, j.group_size, stream);
    if (e != hipSuccess) return device_fail(e, "solver launch");
    return HQQ_OK;
}

hqq_status requant_job(const hqq_job &j, char *ws, hipStream_t stream)
{
    const int64_t n = j.rows * j.cols;
    if (n == 0 || j.zero_bits != 8) return HQQ_OK;
    const int64_t ng = n / j.group_size;
    const JobWs w = job_ws(j, ws);
    hipError_t e = hqq::launch_zero_requant(w.zero32, ng, w.partials,
                                            hqq::solve_blocks(ng, j.group_size, j.nbits),
                                            w.quant, static_cast<uint8_t *>(j.zero),
                                            static_cast<uint16_t *>(j.zero_meta), stream);
    if (e != hipSuccess) return device_fail(e, "zero requantization launch");
    return HQQ_OK;
}

// Validates every job and the workspace; nothing is enqueued on failure.
hqq_status check_batch(const hqq_job *jobs, int n_jobs, void *workspace, size_t workspace_bytes)
{
    if (n_jobs < 0) return fail(HQQ_ERR_ARG, "n_jobs must be >= 0");
    if (n_jobs > 0 && !jobs) return fail(HQQ_ERR_ARG, "jobs must be non-null");
    size_t need = 0;
    for (int i = 0; i < n_jobs; ++i) {
        hqq_status st = check_job(jobs[i], n_jobs > 1 ? i : -1);
        if (st != HQQ_OK) return st;
        need += job_workspace(jobs[i]);
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(HQQ_ERR_WORKSPACE, "workspace must hold " + std::to_string(need) + " bytes");
    if (need > 0 && !aligned(workspace, kAlign))
        return fail(HQQ_ERR_ARG, "workspace must be 256-byte aligned");
    return HQQ_OK;
}

enum Phase { kSolve = 1, kRequant = 2 };

hqq_status run_batch(const hqq_job *jobs, int n_jobs, void *workspace, size_t workspace_bytes,
                     void *stream, int phases)
{
    hqq_status st = check_batch(jobs, n_jobs, workspace, workspace_bytes);
    if (st != HQQ_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (phases & kSolve) {
        char *ws = static_cast<char *>(workspace);
        for (int i = 0; i < n_jobs; ++i) {
            st = solve_job(jobs[i], ws, s);
            if (st != HQQ_OK) return st;
            ws += job_workspace(jobs[i]);
        }
    }
    if (phases & kRequant) {
        char *ws = static_cast<char *>(workspace);
        for (int i = 0; i < n_jobs; ++i) {
            st = requant_job(jobs[i], ws, s);
            if (st != HQQ_OK) return st;
            ws += job_workspace(jobs[i]);
        }
    }
    g_last_error.clear();
    return HQQ_OK;
}

}  // namespace

extern "C" {

size_t hqq_packed_bytes(int64_t n_codes, int nbits) { return packed_bytes(n_codes, nbits); }

size_t hqq_workspace_bytes(const hqq_job *jobs, int n_jobs)
{
    if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return SIZE_MAX;
    size_t total = 0;
    for (int i = 0; i < n_jobs; ++i) {
        if (check_job(jobs[i], i) != HQQ_OK) return SIZE_MAX;
        total += job_workspace(jobs[i]);
    }
    return total;
}

hqq_status hqq_quantize_batch(const hqq_job *jobs, int n_jobs, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    return run_batch(jobs, n_jobs, workspace, workspace_bytes, stream, kSolve | kRequant);
}

hqq_status hqq_solve_batch(const hqq_job *jobs, int n_jobs, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    return run_batch(jobs, n_jobs, workspace, workspace_bytes, stream, kSolve);
}

hqq_status hqq_requant_batch(const hqq_job *jobs, int n_jobs, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    return run_batch(jobs, n_jobs, workspace, workspace_bytes, stream, kRequant);
}

hqq_status hqq_quantize(const void *W, int64_t rows, int64_t cols, int nbits, int group_size,
                        int axis, float p, float beta, float kappa, int iters, int early_stop,
                        int zero_bits, void *packed, void *scale, void *zero, void *zero_meta,
                        uint8_t *passes, void *workspace, size_t workspace_bytes, void *stream)
{
    hqq_job j;
    j.W = W;
    j.rows = rows;
    j.cols = cols;
    j.nbits = nbits;
    j.group_size = group_size;
    j.axis = axis;
    j.p = p;
    j.beta = beta;
    j.kappa = kappa;
    j.iters = iters;
    j.early_stop = early_stop;
    j.zero_bits = zero_bits;
    j.packed = packed;
    j.scale = scale;
    j.zero = zero;
    j.zero_meta = zero_meta;
    j.passes = passes;
    return hqq_quantize_batch(&j, 1, workspace, workspace_bytes, stream);
}

hqq_status hqq_dequantize(const void *packed, const void *scale, const void *zero,
                          const void *zero_meta, int64_t rows, int64_t cols, int nbits,
                          int group_size, int axis, int zero_bits, void *W_out, void *stream)
{
    hqq_status st = check_layout(rows, cols, nbits, group_size, axis, "");
    if (st != HQQ_OK) return st;
    if (zero_bits != 8 && zero_bits != 16) return fail(HQQ_ERR_ARG, "zero_bits must be 8 or 16");
    const int64_t n = rows * cols;
    if (n == 0) return HQQ_OK;
    if (!packed || !scale || !zero || !W_out)
        return fail(HQQ_ERR_ARG, "packed, scale, zero and W_out must be non-null");
    if (zero_bits == 8 && !zero_meta)
        return fail(HQQ_ERR_ARG, "zero_meta must be non-null when zero_bits == 8");
    if (nbits == 3 && !aligned(packed, 4)) return fail(HQQ_ERR_ARG, "packed must be 4-byte aligned");
    if (!aligned(scale, 2) || !aligned(W_out, 2) || (zero_bits == 16 && !aligned(zero, 2)) ||
        (zero_bits == 8 && !aligned(zero_meta, 2)))
        return fail(HQQ_ERR_ARG, "binary16 buffers must be 2-byte aligned");
    hipError_t e = hqq::launch_dequant(static_cast<const uint8_t *>(packed),
                                       static_cast<const uint16_t *>(scale), zero,
                                       static_cast<const uint16_t *>(zero_meta), n, nbits,
                                       group_size, zero_bits, static_cast<uint16_t *>(W_out),
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "dequantize launch");
    g_last_error.clear();
    return HQQ_OK;
}

hqq_status hqq_pack(const uint8_t *codes, int64_t n_codes, int nbits, void *packed, void *stream)
{
    if (!valid_bits(nbits)) return fail(HQQ_ERR_ARG, "nbits must be 1, 2, 3, 4 or 8");
    if (n_codes < 0) return fail(HQQ_ERR_ARG, "n_codes must be >= 0");
    if (n_codes == 0) return HQQ_OK;
    if (!codes || !packed) return fail(HQQ_ERR_ARG, "codes and packed must be non-null");
    if (!aligned(packed, 16)) return fail(HQQ_ERR_ARG, "packed must be 16-byte aligned");
    hipError_t e = hqq::launch_pack(codes, n_codes, nbits, static_cast<uint8_t *>(packed),
                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "pack launch");
    g_last_error.clear();
    return HQQ_OK;
}

hqq_status hqq_unpack(const void *packed, int64_t n_codes, int nbits, uint8_t *codes,
                      void *stream)
{
    if (!valid_bits(nbits)) return fail(HQQ_ERR_ARG, "nbits must be 1, 2, 3, 4 or 8");
    if (n_codes < 0) return fail(HQQ_ERR_ARG, "n_codes must be >= 0");
    if (n_codes == 0) return HQQ_OK;
    if (!codes || !packed) return fail(HQQ_ERR_ARG, "codes and packed must be non-null");
    if (nbits == 3 && !aligned(packed, 4)) return fail(HQQ_ERR_ARG, "packed must be 4-byte aligned");
    hipError_t e = hqq::launch_unpack(static_cast<const uint8_t *>(packed), n_codes, nbits,
                                      codes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "unpack launch");
    g_last_error.clear();
    return HQQ_OK;
}

const char *hqq_status_string(hqq_status s)
{
    switch (s) {
    case HQQ_OK: return "ok";
    case HQQ_ERR_ARG: return "invalid argument";
    case HQQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case HQQ_ERR_WORKSPACE: return "workspace too small";
    case HQQ_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

const char *hqq_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
