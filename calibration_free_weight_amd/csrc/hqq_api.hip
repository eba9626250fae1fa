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
    if (axis != 0 && axis != 1) return fail(HQQ_ERR_ARG, who + "axis must be 0 or 1");
    if (group_size <= 0) return fail(HQQ_ERR_ARG, who + "group_size must be > 0");
    if (axis == 1 && cols % group_size != 0)
        return fail(HQQ_ERR_ARG, who + "group_size must divide cols (axis 1)");
    if (axis == 0 && rows % group_size != 0)
        return fail(HQQ_ERR_ARG, who + "group_size must divide rows (axis 0)");
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
    if (j.rows * j.cols / j.group_size >= (int64_t(1) << 32))
        return fail(HQQ_ERR_ARG, who + "at most 2^32 - 1 groups per tensor");
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

hqq_status device_fail(hipError_t e, const std::string &what)
{
    return fail(HQQ_ERR_DEVICE, what + ": " + hipGetErrorString(e));
}

// ---- batch plan ---------------------------------------------------------------------------
// Non-empty jobs are grouped into launch classes (same nbits, group size and solver
// parameters); each class is one persistent solver launch over its jobs' tiles. Workspace:
//   binary32 zero staging of every 8-bit-zero job (first, so a one-job call finds its zeros
//   at offset 0), the 3-bit boundary stash of every 3-bit job, per-job (min, max) keys, the
//   device job table and one tile counter per class; each section 256-byte aligned.
// An axis-0 job runs the group solver on its transposed weights ([cols, rows], whose rows
// hold the column runs); the solver's outputs, in that order, are written back in the
// tensor's order after the solve.
struct Axis0 {
    const hqq_job *src;
    uint16_t *wt;          // transposed weights; after the solve, 2n bytes of code staging
    uint8_t *packed_t;     // packed codes of the transposed tensor
    uint16_t *scale_t;     // [cols, rows/g]
    void *zero_t;          // binary16 or uint8 [cols, rows/g]
    uint8_t *passes_t;     // or nullptr
};

struct Plan {
    std::vector<hqq::DevJob> table;      // in class order
    std::vector<Axis0> ax0;
    std::vector<int> first;              // first table index of each class
    std::vector<int64_t> tiles;          // tiles of each class
    std::vector<const hqq_job *> src;    // host job of each table entry
    int64_t n_items = 0;                 // finish-kernel items
    size_t bytes = 0;
    size_t off_table = 0, off_counters = 0;
};

bool same_class(const hqq_job &a, const hqq_job &b)
{
    return a.nbits == b.nbits && a.group_size == b.group_size && a.p == b.p && a.beta == b.beta &&
           a.kappa == b.kappa && a.iters == b.iters && a.early_stop == b.early_stop;
}

// Builds the plan; with ws == nullptr only the sizes are computed.
void make_plan(const hqq_job *jobs, int n_jobs, char *ws, Plan &P)
{
    std::vector<int> order;
    std::vector<bool> used(n_jobs, false);
    for (int i = 0; i < n_jobs; ++i) {
        if (used[i] || jobs[i].rows * jobs[i].cols == 0) continue;
        P.first.push_back((int)order.size());
        for (int j = i; j < n_jobs; ++j) {
            if (!used[j] && jobs[j].rows * jobs[j].cols != 0 && same_class(jobs[i], jobs[j])) {
                used[j] = true;
                order.push_back(j);
            }
        }
    }
    const int n = (int)order.size();
    size_t off = 0;
    std::vector<size_t> z_off(n), s_off(n);
    for (int t = 0; t < n; ++t) {
        const hqq_job &j = jobs[order[t]];
        const int64_t ng = j.rows * j.cols / j.group_size;
        z_off[t] = off;
        if (j.zero_bits == 8) off += round_up(sizeof(float) * (size_t)ng);
    }
    for (int t = 0; t < n; ++t) {
        const hqq_job &j = jobs[order[t]];
        const int64_t ng = j.rows * j.cols / j.group_size;
        s_off[t] = off;
        if (j.nbits == 3) off += round_up(sizeof(uint2) * (size_t)ng);
    }
    std::vector<size_t> a_off(n);
    for (int t = 0; t < n; ++t) {
        const hqq_job &j = jobs[order[t]];
        if (j.axis != 0) continue;
        const int64_t nw = j.rows * j.cols, ng = nw / j.group_size;
        a_off[t] = off;
        off += round_up(2 * (size_t)nw) + round_up(packed_bytes(nw, j.nbits)) +
               round_up(2 * (size_t)ng) + round_up((j.zero_bits == 16 ? 2 : 1) * (size_t)ng) +
               (j.passes ? round_up((size_t)ng) : 0);
    }
    const size_t off_mm = off;
    off += round_up(sizeof(uint32_t) * hqq::kMinmaxStride * hqq::kMinmaxSlots *
                    (size_t)(n > 0 ? n : 1));
    P.off_table = off;
    off += round_up(sizeof(hqq::DevJob) * (size_t)(n > 0 ? n : 1));
    P.off_counters = off;                // one tile counter per class, then the status word
    off += round_up(sizeof(uint32_t) * (P.first.size() + 1));
    P.bytes = n > 0 ? off : 0;
    P.first.push_back(n);
    int64_t item = 0;
    for (size_t c = 0; c + 1 < P.first.size(); ++c) {
        int64_t tile = 0;
        for (int t = P.first[c]; t < P.first[c + 1]; ++t) {
            const hqq_job &j = jobs[order[t]];
            const int64_t ng = j.rows * j.cols / j.group_size;
            hqq::DevJob d{};
            d.W = static_cast<const uint16_t *>(j.W);
            d.packed = static_cast<uint8_t *>(j.packed);
            d.scale = static_cast<uint16_t *>(j.scale);
            d.passes = j.passes;
            d.n_groups = ng;
            d.tile0 = tile;
            d.nbits = j.nbits;
            d.g = j.group_size;
            d.item0 = item;
            if (ws && j.axis == 0) {
                const int64_t nw = j.rows * j.cols;
                Axis0 a{};
                a.src = &j;
                char *p = ws + a_off[t];
                a.wt = reinterpret_cast<uint16_t *>(p);
                p += round_up(2 * (size_t)nw);
                a.packed_t = reinterpret_cast<uint8_t *>(p);
                p += round_up(packed_bytes(nw, j.nbits));
                a.scale_t = reinterpret_cast<uint16_t *>(p);
                p += round_up(2 * (size_t)ng);
                a.zero_t = p;
                p += round_up((j.zero_bits == 16 ? 2 : 1) * (size_t)ng);
                a.passes_t = j.passes ? reinterpret_cast<uint8_t *>(p) : nullptr;
                d.W = a.wt;
                d.packed = a.packed_t;
                d.scale = a.scale_t;
                d.passes = a.passes_t;
                P.ax0.push_back(a);
            }
            if (ws) {
                const bool t0 = j.axis == 0;
                if (j.zero_bits == 8) {
                    d.zero32 = reinterpret_cast<float *>(ws + z_off[t]);
                    d.minmax = reinterpret_cast<uint32_t *>(ws + off_mm) +
                               hqq::kMinmaxStride * hqq::kMinmaxSlots * t;
                    d.zq = static_cast<uint8_t *>(t0 ? P.ax0.back().zero_t : j.zero);
                    d.meta = static_cast<uint16_t *>(j.zero_meta);
                } else {
                    d.zero16 = static_cast<uint16_t *>(t0 ? P.ax0.back().zero_t : j.zero);
                }
                if (j.nbits == 3) d.stash = reinterpret_cast<uint2 *>(ws + s_off[t]);
            }
            if (j.zero_bits == 8 || j.nbits == 3) item += ng;
            tile += hqq::tiles_for(ng, j.group_size);
            P.table.push_back(d);
            P.src.push_back(&j);
        }
        P.tiles.push_back(tile);
    }
    P.n_items = item;
}

size_t batch_workspace(const hqq_job *jobs, int n_jobs)
{
    Plan P;
    make_plan(jobs, n_jobs, nullptr, P);
    return P.bytes;
}

// Validates every job and the workspace; nothing is enqueued on failure.
hqq_status check_batch(const hqq_job *jobs, int n_jobs, void *workspace, size_t workspace_bytes)
{
    if (n_jobs < 0) return fail(HQQ_ERR_ARG, "n_jobs must be >= 0");
    if (n_jobs > 0 && !jobs) return fail(HQQ_ERR_ARG, "jobs must be non-null");
    if (n_jobs > 65535) return fail(HQQ_ERR_ARG, "at most 65535 jobs per batch");
    for (int i = 0; i < n_jobs; ++i) {
        hqq_status st = check_job(jobs[i], n_jobs > 1 ? i : -1);
        if (st != HQQ_OK) return st;
    }
    const size_t need = batch_workspace(jobs, n_jobs);
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
    char *ws = static_cast<char *>(workspace);
    Plan P;
    make_plan(jobs, n_jobs, ws, P);
    const int n = (int)P.table.size();
    if (n == 0) {
        g_last_error.clear();
        return HQQ_OK;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hqq::DevJob *table = reinterpret_cast<hqq::DevJob *>(ws + P.off_table);
    uint32_t *counters = reinterpret_cast<uint32_t *>(ws + P.off_counters);
    const int n_classes = (int)P.first.size() - 1;
    if (phases & kSolve) {
        if (!P.ax0.empty()) {                    // the column runs become rows
            std::vector<hqq::XTask> x;
            for (const Axis0 &a : P.ax0)
                x.push_back({a.src->W, a.wt, a.src->rows, a.src->cols, hqq::kX16, 0});
            hipError_t e = hqq::launch_transposes(x.data(), (int)x.size(), s);
            if (e != hipSuccess) return device_fail(e, "axis-0 transpose launch");
        }
        for (int o = 0; o < n; o += hqq::kFillJobs) {
            hqq::FillArgs f{};
            f.n = n - o < hqq::kFillJobs ? n - o : hqq::kFillJobs;
            f.offset = o;
            f.counters = counters;
            f.n_counters = n_classes + 1;
            for (int i = 0; i < f.n; ++i) f.jobs[i] = P.table[o + i];
            hipError_t e = hqq::launch_fill(f, table, s);
            if (e != hipSuccess) return device_fail(e, "job table launch");
        }
        for (int c = 0; c < n_classes; ++c) {
            const hqq_job &j = *P.src[P.first[c]];
            hqq::StreamArgs a{};
            a.jobs = table + P.first[c];
            a.n_jobs = P.first[c + 1] - P.first[c];
            a.n_tiles = P.tiles[c];
            a.p = j.p;
            a.beta0 = j.beta;
            a.kappa = j.kappa;
            a.iters = j.iters;
            a.early_stop = j.early_stop;
            a.counter = counters + c;
            a.status = counters + n_classes;
            hipError_t e = hqq::launch_stream(a, j.nbits, j.group_size, s);
            if (e != hipSuccess) return device_fail(e, "solver launch");
        }
    }
    if (phases & kRequant) {
        hipError_t e = hqq::launch_finish(table, n, P.n_items, s);
        if (e != hipSuccess) return device_fail(e, "zero requantization launch");
        // axis-0 outputs back in the tensor's order: packed codes in one pass where every
        // row starts on a byte (else unpacked, transposed and packed), and the per-group
        // [cols, rows/g] arrays; the transposes of all jobs share launches
        std::vector<hqq::XTask> x;
        for (const Axis0 &a : P.ax0) {
            const hqq_job &j = *a.src;
            const int64_t nw = j.rows * j.cols, nb = j.rows / j.group_size;
            if (hqq::codes_transpose_fused(j.nbits, j.rows, j.cols)) {
                x.push_back({a.packed_t, j.packed, j.rows, j.cols, hqq::kXCodes, j.nbits});
            } else {                             // 3-bit words, or rows not byte-aligned
                uint8_t *ct = reinterpret_cast<uint8_t *>(a.wt), *c = ct + nw;
                e = hqq::launch_unpack(a.packed_t, nw, j.nbits, ct, s);
                if (e == hipSuccess) {
                    const hqq::XTask t{ct, c, j.cols, j.rows, hqq::kX8, 0};
                    e = hqq::launch_transposes(&t, 1, s);
                }
                if (e == hipSuccess)
                    e = hqq::launch_pack(c, nw, j.nbits, static_cast<uint8_t *>(j.packed), s);
                if (e != hipSuccess) return device_fail(e, "axis-0 code write-back launch");
            }
            x.push_back({a.scale_t, j.scale, j.cols, nb, hqq::kX16, 0});
            x.push_back({a.zero_t, j.zero, j.cols, nb, j.zero_bits == 16 ? hqq::kX16 : hqq::kX8, 0});
            if (a.passes_t) x.push_back({a.passes_t, j.passes, j.cols, nb, hqq::kX8, 0});
        }
        if (!x.empty()) {
            e = hqq::launch_transposes(x.data(), (int)x.size(), s);
            if (e != hipSuccess) return device_fail(e, "axis-0 write-back launch");
        }
    }
    g_last_error.clear();
    return HQQ_OK;
}

// ---- host-streamed batches ----------------------------------------------------------------
// Consecutive jobs are cut into chunks whose weights fit half of the staging buffer (each
// tensor at a 256-byte aligned offset); chunk k is copied into half k % 2.
struct Chunk {
    int first, count;
};

hqq_status make_chunks(const hqq_job *jobs, int n_jobs, size_t staging_bytes,
                       std::vector<Chunk> &out)
{
    const size_t half = staging_bytes / 2 / kAlign * kAlign;
    size_t used = 0;
    int first = 0;
    for (int i = 0; i < n_jobs; ++i) {
        const size_t b = round_up(2 * (size_t)(jobs[i].rows * jobs[i].cols));
        if (b > half)
            return fail(HQQ_ERR_WORKSPACE, job_name(i) + "its weights (" + std::to_string(b) +
                                               " bytes) exceed half the staging buffer");
        if (used + b > half) {
            out.push_back({first, i - first});
            first = i;
            used = 0;
        }
        used += b;
    }
    if (n_jobs > first) out.push_back({first, n_jobs - first});
    return HQQ_OK;
}

size_t streamed_workspace(const hqq_job *jobs, const std::vector<Chunk> &chunks)
{
    size_t need = 0;
    for (const Chunk &c : chunks) {
        const size_t b = batch_workspace(jobs + c.first, c.count);
        need = b > need ? b : need;
    }
    return need;
}

}  // namespace

int hqq::report_error(int status, const char *msg)
{
    g_last_error = msg;
    return status;
}

extern "C" {

size_t hqq_packed_bytes(int64_t n_codes, int nbits) { return packed_bytes(n_codes, nbits); }

size_t hqq_workspace_bytes(const hqq_job *jobs, int n_jobs)
{
    if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return SIZE_MAX;
    if (n_jobs > 65535) return SIZE_MAX;
    for (int i = 0; i < n_jobs; ++i)
        if (check_job(jobs[i], i) != HQQ_OK) return SIZE_MAX;
    return batch_workspace(jobs, n_jobs);
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

hqq_status hqq_batch_check(const hqq_job *jobs, int n_jobs, const void *workspace,
                           size_t workspace_bytes, void *stream)
{
    hqq_status st = check_batch(jobs, n_jobs, const_cast<void *>(workspace), workspace_bytes);
    if (st != HQQ_OK) return st;
    Plan P;
    make_plan(jobs, n_jobs, nullptr, P);
    if (P.table.empty()) {
        g_last_error.clear();
        return HQQ_OK;
    }
    const int n_classes = (int)P.first.size() - 1;
    const uint32_t *status =
        reinterpret_cast<const uint32_t *>(static_cast<const char *>(workspace) + P.off_counters) +
        n_classes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t flag = 0;
    hipError_t e = hipMemcpyAsync(&flag, status, sizeof(flag), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return device_fail(e, "batch check");
    if (flag & 1u)
        return fail(HQQ_ERR_DEVICE, "the solver ran out of its step budget: some groups of this "
                                    "batch were not written");
    g_last_error.clear();
    return HQQ_OK;
}

void hqq_debug_solver(int64_t step_budget, int pass_layout)
{
    hqq::set_solver_debug(step_budget, pass_layout);
}

size_t hqq_streamed_workspace_bytes(const hqq_job *jobs, int n_jobs, size_t staging_bytes)
{
    if (n_jobs < 0 || (n_jobs > 0 && !jobs) || n_jobs > 65535) return SIZE_MAX;
    for (int i = 0; i < n_jobs; ++i)
        if (check_job(jobs[i], i) != HQQ_OK) return SIZE_MAX;
    std::vector<Chunk> chunks;
    if (make_chunks(jobs, n_jobs, staging_bytes, chunks) != HQQ_OK) return SIZE_MAX;
    return streamed_workspace(jobs, chunks);
}

hqq_status hqq_quantize_streamed(const hqq_job *jobs, int n_jobs, void *staging,
                                 size_t staging_bytes, void *workspace, size_t workspace_bytes,
                                 void *stream, void *copy_stream)
{
    if (n_jobs < 0) return fail(HQQ_ERR_ARG, "n_jobs must be >= 0");
    if (n_jobs > 0 && !jobs) return fail(HQQ_ERR_ARG, "jobs must be non-null");
    if (n_jobs > 65535) return fail(HQQ_ERR_ARG, "at most 65535 jobs per batch");
    for (int i = 0; i < n_jobs; ++i) {
        hqq_status st = check_job(jobs[i], n_jobs > 1 ? i : -1);
        if (st != HQQ_OK) return st;
    }
    std::vector<Chunk> chunks;
    hqq_status st = make_chunks(jobs, n_jobs, staging_bytes, chunks);
    if (st != HQQ_OK) return st;
    bool any = false;
    for (int i = 0; i < n_jobs; ++i) any = any || jobs[i].rows * jobs[i].cols > 0;
    if (!any) {
        g_last_error.clear();
        return HQQ_OK;
    }
    if (!staging || !aligned(staging, kAlign))
        return fail(HQQ_ERR_ARG, "staging must be non-null and 256-byte aligned");
    const size_t need = streamed_workspace(jobs, chunks);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(HQQ_ERR_WORKSPACE, "workspace must hold " + std::to_string(need) + " bytes");
    if (need > 0 && !aligned(workspace, kAlign))
        return fail(HQQ_ERR_ARG, "workspace must be 256-byte aligned");

    hipStream_t s = static_cast<hipStream_t>(stream), cs = static_cast<hipStream_t>(copy_stream);
    // copied[h]: half h holds its chunk; consumed[h]: the solve of half h's chunk is done;
    // entry: all work enqueued on `stream` before this call (a previous call's solves may
    // still read either half)
    hipEvent_t copied[2] = {nullptr, nullptr}, consumed[2] = {nullptr, nullptr}, entry = nullptr;
    hipError_t e = hipEventCreateWithFlags(&entry, hipEventDisableTiming);
    for (int h = 0; h < 2 && e == hipSuccess; ++h) {
        e = hipEventCreateWithFlags(&copied[h], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&consumed[h], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipEventRecord(entry, s);
    auto release = [&]() {                       // safe while recorded work is pending
        for (int h = 0; h < 2; ++h) {
            if (copied[h]) (void)hipEventDestroy(copied[h]);
            if (consumed[h]) (void)hipEventDestroy(consumed[h]);
        }
        if (entry) (void)hipEventDestroy(entry);
    };
    if (e != hipSuccess) {
        release();
        return device_fail(e, "event creation");
    }
    const size_t half = staging_bytes / 2 / kAlign * kAlign;
    std::vector<hqq_job> local;
    for (size_t k = 0; k < chunks.size() && st == HQQ_OK; ++k) {
        const Chunk &c = chunks[k];
        const int h = (int)(k % 2);
        char *dst = static_cast<char *>(staging) + h * half;
        if (k >= 2) e = hipStreamWaitEvent(cs, consumed[h], 0);   // chunk k-2 left this half
        else e = hipStreamWaitEvent(cs, entry, 0);                  // earlier work left it
        local.assign(jobs + c.first, jobs + c.first + c.count);
        size_t off = 0;
        for (int i = 0; i < c.count && e == hipSuccess; ++i) {
            const size_t b = 2 * (size_t)(local[i].rows * local[i].cols);
            if (b > 0) e = hipMemcpyAsync(dst + off, local[i].W, b, hipMemcpyHostToDevice, cs);
            local[i].W = dst + off;
            off += round_up(b);
        }
        if (e == hipSuccess) e = hipEventRecord(copied[h], cs);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, copied[h], 0);
        if (e != hipSuccess) {
            st = device_fail(e, "weight upload");
            break;
        }
        st = run_batch(local.data(), c.count, workspace, workspace_bytes, stream, kSolve | kRequant);
        if (st == HQQ_OK) {
            e = hipEventRecord(consumed[h], s);
            if (e != hipSuccess) st = device_fail(e, "event record");
        }
    }
    release();
    if (st == HQQ_OK) g_last_error.clear();
    return st;
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
    // the flat, coalesced kernel when the alignments allow, else the element-wise one
    const bool flat = hqq::recon_fits(packed, nbits, cols, axis, W_out);
    hipError_t e =
        flat ? hqq::launch_recon(static_cast<const uint8_t *>(packed),
                                 static_cast<const uint16_t *>(scale), zero,
                                 static_cast<const uint16_t *>(zero_meta), rows, cols, nbits,
                                 group_size, zero_bits, axis, static_cast<uint16_t *>(W_out),
                                 static_cast<hipStream_t>(stream))
             : hqq::launch_dequant(static_cast<const uint8_t *>(packed),
                                   static_cast<const uint16_t *>(scale), zero,
                                   static_cast<const uint16_t *>(zero_meta), n, nbits,
                                   group_size, zero_bits, cols, axis,
                                   static_cast<uint16_t *>(W_out),
                                   static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "dequantize launch");
    g_last_error.clear();
    return HQQ_OK;
}

static hqq_status check_scale_group(int scale_group)
{
    if (scale_group < 8 || scale_group > 512 || (scale_group & (scale_group - 1)) != 0)
        return fail(HQQ_ERR_ARG, "scale_group must be a power of two in [8, 512]");
    return HQQ_OK;
}

hqq_status hqq_requant_scales(const void *scale, int64_t n, int scale_group, uint8_t *scale_q,
                              void *scale_meta, void *stream)
{
    if (n < 0) return fail(HQQ_ERR_ARG, "n must be >= 0");
    hqq_status st = check_scale_group(scale_group);
    if (st != HQQ_OK) return st;
    if (n == 0) return HQQ_OK;
    if (!scale || !scale_q || !scale_meta)
        return fail(HQQ_ERR_ARG, "scale, scale_q and scale_meta must be non-null");
    if (!aligned(scale, 16) || !aligned(scale_q, 8) || !aligned(scale_meta, 4))
        return fail(HQQ_ERR_ARG, "scale must be 16-, scale_q 8- and scale_meta 4-byte aligned");
    hipError_t e = hqq::launch_scale_requant(static_cast<const uint16_t *>(scale), n, scale_group,
                                             scale_q, static_cast<uint16_t *>(scale_meta),
                                             static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "scale requant launch");
    g_last_error.clear();
    return HQQ_OK;
}

hqq_status hqq_dequantize_scales(const uint8_t *scale_q, const void *scale_meta, int64_t n,
                                 int scale_group, void *scale_out, void *stream)
{
    if (n < 0) return fail(HQQ_ERR_ARG, "n must be >= 0");
    hqq_status st = check_scale_group(scale_group);
    if (st != HQQ_OK) return st;
    if (n == 0) return HQQ_OK;
    if (!scale_q || !scale_meta || !scale_out)
        return fail(HQQ_ERR_ARG, "scale_q, scale_meta and scale_out must be non-null");
    if (!aligned(scale_q, 8) || !aligned(scale_meta, 4) || !aligned(scale_out, 16))
        return fail(HQQ_ERR_ARG, "scale_q must be 8-, scale_meta 4- and scale_out 16-byte aligned");
    hipError_t e = hqq::launch_scale_dequant(scale_q, static_cast<const uint16_t *>(scale_meta), n,
                                             scale_group, static_cast<uint16_t *>(scale_out),
                                             static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "scale dequantize launch");
    g_last_error.clear();
    return HQQ_OK;
}

size_t hqq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    return hqq::gemm_workspace_bytes(M, N, K);
}

namespace {
// Argument checks of one weight of hqq_gemm / hqq_gemm_multi (M > 0, N > 0).
hqq_status check_gemm_weight(const void *packed, const void *scale, const void *zero,
                             const void *zero_meta, int64_t N, int64_t K, int nbits,
                             int group_size, int zero_bits, const void *Y, const char *what)
{
    hqq_status st = check_layout(N, K, nbits, group_size, 1, what);
    if (st != HQQ_OK) return st;
    if (zero_bits != 8 && zero_bits != 16)
        return fail(HQQ_ERR_ARG, std::string(what) + "zero_bits must be 8 or 16");
    if (!Y || (K > 0 && (!packed || !scale || !zero)))
        return fail(HQQ_ERR_ARG, std::string(what) + "Y, packed, scale and zero must be non-null");
    if (zero_bits == 8 && K > 0 && !zero_meta)
        return fail(HQQ_ERR_ARG, std::string(what) + "zero_meta must be non-null when zero_bits == 8");
    if (!aligned(Y, 2) || !aligned(scale, 2) || (zero_bits == 16 && !aligned(zero, 2)) ||
        (zero_bits == 8 && !aligned(zero_meta, 2)))
        return fail(HQQ_ERR_ARG, std::string(what) + "binary16 buffers must be 2-byte aligned");
    if (nbits == 3 && !aligned(packed, 4))
        return fail(HQQ_ERR_ARG, std::string(what) + "packed must be 4-byte aligned");
    return HQQ_OK;
}
}  // namespace

hqq_status hqq_gemm(const void *X, int64_t M, const void *packed, const void *scale,
                    const void *zero, const void *zero_meta, int64_t N, int64_t K, int nbits,
                    int group_size, int zero_bits, void *Y, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    hqq_status st = check_layout(N, K, nbits, group_size, 1, "");
    if (st != HQQ_OK) return st;
    if (M < 0) return fail(HQQ_ERR_ARG, "M must be >= 0");
    if (M > 0 && K > (int64_t(1) << 40) / M) return fail(HQQ_ERR_ARG, "M*K too large");
    if (zero_bits != 8 && zero_bits != 16) return fail(HQQ_ERR_ARG, "zero_bits must be 8 or 16");
    if (M == 0 || N == 0) return HQQ_OK;
    if (!X && K > 0) return fail(HQQ_ERR_ARG, "X, Y, packed, scale and zero must be non-null");
    st = check_gemm_weight(packed, scale, zero, zero_meta, N, K, nbits, group_size, zero_bits, Y, "");
    if (st != HQQ_OK) return st;
    if (K > 0 && !aligned(X, 16)) return fail(HQQ_ERR_ARG, "X must be 16-byte aligned");
    const size_t need = hqq::gemm_workspace_bytes(M, N, K);
    if (workspace && need > 0 && workspace_bytes < need)
        return fail(HQQ_ERR_WORKSPACE, "workspace smaller than hqq_gemm_workspace_bytes(M, N, K)");
    if (workspace && !aligned(workspace, 16))
        return fail(HQQ_ERR_ARG, "workspace must be 16-byte aligned");
    hipError_t e = hqq::launch_gemm(static_cast<const uint16_t *>(X), M,
                                    static_cast<const uint8_t *>(packed),
                                    static_cast<const uint16_t *>(scale), zero,
                                    static_cast<const uint16_t *>(zero_meta), N, K, nbits,
                                    group_size, zero_bits, static_cast<uint16_t *>(Y),
                                    need > 0 ? static_cast<uint16_t *>(workspace) : nullptr,
                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "gemm launch");
    g_last_error.clear();
    return HQQ_OK;
}

hqq_status hqq_gemm_multi(const void *X, int64_t M, int64_t K, const hqq_gemm_weight *weights,
                          int n_weights, void *workspace, size_t workspace_bytes, void *stream)
{
    if (M < 0 || K < 0 || n_weights < 0) return fail(HQQ_ERR_ARG, "M, K and n_weights must be >= 0");
    if (M > 0 && K > (int64_t(1) << 40) / M) return fail(HQQ_ERR_ARG, "M*K too large");
    if (n_weights > 0 && !weights) return fail(HQQ_ERR_ARG, "weights must be non-null");
    size_t need = 0;
    std::vector<hqq::GemmWeight> ws;
    for (int i = 0; i < n_weights; ++i) {
        const hqq_gemm_weight &w = weights[i];
        const std::string what = "weight " + std::to_string(i) + ": ";
        hqq_status st = check_layout(w.N, K, w.nbits, w.group_size, 1, what.c_str());
        if (st != HQQ_OK) return st;
        if (w.zero_bits != 8 && w.zero_bits != 16)
            return fail(HQQ_ERR_ARG, what + "zero_bits must be 8 or 16");
        if (M == 0 || w.N == 0) continue;
        st = check_gemm_weight(w.packed, w.scale, w.zero, w.zero_meta, w.N, K, w.nbits,
                               w.group_size, w.zero_bits, w.Y, what.c_str());
        if (st != HQQ_OK) return st;
        const size_t nd = hqq::gemm_workspace_bytes(M, w.N, K);
        need = nd > need ? nd : need;
        ws.push_back(hqq::GemmWeight{static_cast<const uint8_t *>(w.packed),
                                     static_cast<const uint16_t *>(w.scale), w.zero,
                                     static_cast<const uint16_t *>(w.zero_meta), w.N, w.nbits,
                                     w.group_size, w.zero_bits, static_cast<uint16_t *>(w.Y)});
    }
    if (ws.empty()) {
        g_last_error.clear();
        return HQQ_OK;
    }
    if (!X && K > 0) return fail(HQQ_ERR_ARG, "X must be non-null");
    if (K > 0 && !aligned(X, 16)) return fail(HQQ_ERR_ARG, "X must be 16-byte aligned");
    if (workspace && need > 0 && workspace_bytes < need)
        return fail(HQQ_ERR_WORKSPACE,
                    "workspace smaller than the largest hqq_gemm_workspace_bytes(M, N_i, K)");
    if (workspace && !aligned(workspace, 16))
        return fail(HQQ_ERR_ARG, "workspace must be 16-byte aligned");
    hipError_t e = hqq::launch_gemm_multi(static_cast<const uint16_t *>(X), M, K, ws.data(),
                                          (int)ws.size(),
                                          need > 0 ? static_cast<uint16_t *>(workspace) : nullptr,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "gemm launch");
    g_last_error.clear();
    return HQQ_OK;
}

hqq_status hqq_gemm_f16(const void *X, int64_t M, const void *Wr, int64_t N, int64_t K, void *Y,
                        void *stream)
{
    if (M < 0 || N < 0 || K < 0) return fail(HQQ_ERR_ARG, "M, N and K must be >= 0");
    if (M == 0 || N == 0) return HQQ_OK;
    if (!hqq::gemm_f16_fits(N, K))
        return fail(HQQ_ERR_ARG, "K must be a positive multiple of 8 and at most 2^22");
    if (M > (int64_t(1) << 40) / K) return fail(HQQ_ERR_ARG, "M*K too large");
    if (!X || !Wr || !Y) return fail(HQQ_ERR_ARG, "X, Wr and Y must be non-null");
    if (!aligned(X, 16) || !aligned(Wr, 16)) return fail(HQQ_ERR_ARG, "X and Wr must be 16-byte aligned");
    if (!aligned(Y, 2)) return fail(HQQ_ERR_ARG, "Y must be 2-byte aligned");
    hipError_t e = hqq::launch_gemm_f16(static_cast<const uint16_t *>(X), M,
                                        static_cast<const uint16_t *>(Wr), N, K,
                                        static_cast<uint16_t *>(Y), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "gemm_f16 launch");
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
