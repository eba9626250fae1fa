// hqq_stream.hip -- the HQQ group solver for gfx950: persistent waves streaming groups
// through an LDS pool.
//
// Method [techreport.ngo, "Half-Quadratic Quantization of Large Machine Learning Models",
// section "Outlier-aware optimization without gradients"; parameters from its section
// "Benchmark results / Llama-2"]: per group of G consecutive weights, fix the min-max scale
// s and optimise the zero-point z by half-quadratic splitting of an lp (p < 1) loss -- a
// generalized soft-threshold of the residual (sub-problem 1) alternating with a closed-form
// average for z (sub-problem 2), beta growing by kappa per iteration, and an early stop when
// the mean |W - W_r| rises.
//
// Arithmetic contract (the library's documented semantics): s, z and beta are binary32;
// every per-element quantity is exact -- u = x*s + z, the code q = clamp(rne(u)), the
// residual u - q and the group sums S = sum|u - q|, Q = sum q and x*s -- and each zero update
// rounds its exact value once to binary32. Exact values make ties in the stop test real ties.
//
// How the kernel meets that contract fast:
//  * Passes run in binary32 (v_fma_mix on the binary16 weights). A binary32 u differs from
//    the exact one by at most half an ulp, 2^(NBITS-25) for u < 2^NBITS, so a code can only
//    be wrong when |u - rne(u)| is within that of 1/2: the pass tracks D = max|u - rne(u)|
//    and hands the group to the exact path when D >= kThr. Otherwise Q is exact and S is
//    within g*2^(NBITS-24) plus its own summation error of the exact sum, so a stop decision
//    is certain unless the two sums are that close; near ties also go to the exact path.
//  * The exact path evaluates in binary64, where x*s (11 x 24 significant bits) and x*s + z
//    are exact. It also computes the zero update with a live shrink (W_e != 0), which only
//    happens when max|r| = D/s exceeds beta^(-1/(2-p)).
//  * The zero update without shrink is (Q - sum x*s)/G with sum x*s exact in binary64
//    (computed once per group), rounded once to binary32.
//  * A group whose new zero equals the accepted one, with the shrink dead for every later
//    beta, is at an exact fixed point: every later iteration repeats it, so it finishes.
//
// Scheduling: one wave per workgroup, persistent. The wave claims tiles (GPI consecutive
// groups of one tensor; 64 lanes x E weights) from a global counter, prefetches the next tile
// into registers, and keeps up to NS = 3*GPI groups resident in LDS: a ring of active groups
// (each pass takes up to GPI of them, so lanes stay busy while groups stop at different
// iterations), a list of finished groups (epilogue in batches of GPI), a list of groups that
// need the exact path (also batched) and a free list. K = G/E lanes hold one group.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "hqq_internal.h"

namespace hqq {
namespace {

enum : uint8_t { kActive = 0, kFinished = 1, kExact = 2 };
enum : uint8_t { kDecide = 1, kShrink = 2 };         // exact-path work (flags bits 1-2)
typedef _Float16 h2v __attribute__((ext_vector_type(2)));   // two binary16 weights

// Global-address-space view of a pointer: global_* instructions count only against vmcnt,
// whereas flat ones also hold lgkmcnt and would make LDS waits wait for memory.
template <typename T> __device__ __forceinline__ __attribute__((address_space(1))) T *gbl(T *p)
{
    return (__attribute__((address_space(1))) T *)p;
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t atomic_add_g(uint32_t *p, uint32_t v)
{
    return __hip_atomic_fetch_add(gbl(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_min_g(uint32_t *p, uint32_t v)
{
    __hip_atomic_fetch_min(gbl(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_max_g(uint32_t *p, uint32_t v)
{
    __hip_atomic_fetch_max(gbl(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float h2f(uint32_t h) { return __half2float(__ushort_as_half((uint16_t)h)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

template <int CTRL> __device__ __forceinline__ float dppf(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL> __device__ __forceinline__ double dppd(double v)
{
    const uint64_t b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, false);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
// Butterflies within the K lanes of a group: lane xor 1, xor 2 (quad permutes), then half-row
// and row mirrors, each pairing lanes of two already-reduced halves; wave-wide steps beyond.
#define HQQ_RED(T, DPP, OP)                                                                   \
    template <int K> __device__ __forceinline__ T OP##_k(T v)                                 \
    {                                                                                         \
        if (K >= 2) v = OP(v, DPP<0xb1>(v));                                                  \
        if (K >= 4) v = OP(v, DPP<0x4e>(v));                                                  \
        if (K >= 8) v = OP(v, DPP<0x141>(v));                                                 \
        if (K >= 16) v = OP(v, DPP<0x140>(v));                                                \
        if (K >= 32) v = OP(v, __shfl_xor(v, 16));                                            \
        if (K >= 64) v = OP(v, __shfl_xor(v, 32));                                            \
        return v;                                                                             \
    }
__device__ __forceinline__ float addf(float a, float b) { return a + b; }
__device__ __forceinline__ double addd(double a, double b) { return a + b; }
__device__ __forceinline__ float maxf(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float minf(float a, float b) { return fminf(a, b); }
HQQ_RED(float, dppf, addf)
HQQ_RED(double, dppd, addd)
HQQ_RED(float, dppf, maxf)
HQQ_RED(float, dppf, minf)
#undef HQQ_RED

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Order-preserving map of binary32 onto uint32 (for atomic min/max of the zeros).
__device__ __forceinline__ uint32_t fkey(float f)
{
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ double shrink(double r, double pm1, double beta)
{
    if (r == 0.0) return 0.0;
    const double a = fabs(r);
    const double m = fmax(a - pow(a, pm1) / beta, 0.0);
    return r > 0.0 ? m : -m;
}

template <int NBITS, int G>
struct Cfg {
    static constexpr int E = G >= 32 ? 32 : 16;     // weights per lane
    static constexpr int K = G / E;                 // lanes per group
    static constexpr int GPI = 64 / K;              // groups per pass
    static constexpr int NS = 3 * GPI;              // resident groups
    static constexpr int RC = NS <= 64 ? 64 : (NS <= 128 ? 128 : 256);   // ring capacity
    static constexpr int W = E / 2;                 // packed binary16 pairs per lane
    static constexpr float QMAX = (float)((1 << NBITS) - 1);
    // A binary32 code can disagree with the exact one only if |u - rne(u)| >= kThr.
    static constexpr float kThr = 0.5f - (float)(1.0 / (1 << (24 - NBITS)));
    // Bound on |S_binary32 - S_exact| from the per-element rounding (G halves of an ulp, x2).
    static constexpr double kElemErr = (double)G / (double)(1 << (24 - NBITS));
};

// Binary32 evaluation of one lane's E weights at zero z: S = sum|u - q|, Q = sum q,
// D = max |u - rne(u)| (before any clamp).
template <int NBITS, int G, bool CLAMP>
__device__ __forceinline__ void eval_fast(const uint32_t (&xr)[Cfg<NBITS, G>::W], float s, float z,
                                          float &S, float &Q, float &D)
{
    using C = Cfg<NBITS, G>;
    float s0 = 0.f, s1 = 0.f, q0 = 0.f, q1 = 0.f, d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int i = 0; i < C::W; ++i) {
        const float u0 = fmaf(h2f(xr[i] & 0xffffu), s, z);
        const float u1 = fmaf(h2f(xr[i] >> 16), s, z);
        const float r0 = rintf(u0), r1 = rintf(u1);
        if (CLAMP) {
            const float c0 = __builtin_amdgcn_fmed3f(r0, 0.f, C::QMAX);
            const float c1 = __builtin_amdgcn_fmed3f(r1, 0.f, C::QMAX);
            s0 += fabsf(u0 - c0);
            s1 += fabsf(u1 - c1);
            q0 += c0;
            q1 += c1;
        } else {
            s0 += fabsf(u0 - r0);
            s1 += fabsf(u1 - r1);
            q0 += r0;
            q1 += r1;
        }
        d0 = fmaxf(d0, fabsf(u0 - r0));
        d1 = fmaxf(d1, fabsf(u1 - r1));
    }
    S = s0 + s1;
    Q = q0 + q1;
    D = fmaxf(d0, d1);
}

struct Exact {
    double S, Q, D;
};

// Exact (binary64) evaluation of one lane's E weights (binary16, in LDS) at zero z. Rare:
// a rolled loop, so it adds few registers to the binary32 path.
template <int NBITS, int G>
__device__ __forceinline__ Exact eval_exact(const uint16_t *x, float s, float z)
{
    using C = Cfg<NBITS, G>;
    const double sd = s, zd = z, qm = C::QMAX;
    double s_ = 0.0, q_ = 0.0, d_ = 0.0;
#pragma unroll 1
    for (int i = 0; i < C::E; ++i) {
        const double u = fma((double)h2f(x[i]), sd, zd);
        const double c = fmin(fmax(rint(u), 0.0), qm);
        const double e = fabs(u - c);
        s_ += e;
        q_ += c;
        d_ = fmax(d_, e);
    }
    return Exact{s_, q_, d_};
}

template <int NBITS, int G>
__global__ void __launch_bounds__(64) stream_kernel(StreamArgs a,
                                                    const DevJob *__restrict__ jobs)
{
    using C = Cfg<NBITS, G>;
    constexpr int E = C::E, K = C::K, GPI = C::GPI, NS = C::NS, W = C::W, RM = C::RC - 1;
    static_assert(NS <= 255, "slot indices are bytes");

    // Pool of resident groups: weights and per-group state (one array per field).
    __shared__ __attribute__((aligned(16))) uint16_t xs[NS * G];
    __shared__ float st_z[NS];         // candidate zero (next evaluation)
    __shared__ float st_zb[NS];        // accepted zero
    __shared__ float st_s[NS];         // quantizer multiplier
    __shared__ float st_beta[NS];      // beta of the next shrink
    __shared__ float st_Qb[NS];        // accepted sum of codes
    __shared__ float st_Db[NS];        // accepted max |u - q|
    __shared__ double st_Sb[NS];       // accepted sum |u - q|
    __shared__ double st_sxs[NS];      // exact sum x*s
    __shared__ uint32_t st_mnmx[NS];   // binary16 min (low half) and max (high half)
    __shared__ uint32_t st_gidx[NS];   // group index within its tensor
    __shared__ uint16_t st_job[NS];    // job index within the launch class
    __shared__ uint8_t st_t[NS];       // index of the next zero update (1-based)
    __shared__ uint8_t st_fl[NS];      // bit 0: Sb/Db exact; bits 1-2: exact-path work
    __shared__ uint8_t rings[4 * C::RC];   // slot rings: active, finished, exact-pending, free
    uint8_t *const ring_act = rings, *const ring_fin = rings + C::RC,
                   *const ring_exq = rings + 2 * C::RC, *const ring_free = rings + 3 * C::RC;
    __shared__ float tau[kMaxIters];
    __shared__ uint8_t stage[NBITS == 3 ? 64 * E : 4];

    const int lane = threadIdx.x;
    const int k = lane / K;                      // group within a pass
    const int sub = lane % K;                    // part of the group
    const bool leader = sub == 0;

    // Dead-zone thresholds: the shrink of iteration t uses beta_{t-1} = beta0*kappa^(t-1)
    // (binary32 products in order) and maps r to 0 iff |r| <= beta^(-1/(2-p)).
    for (int t = lane; t < a.iters; t += 64) {
        float b = a.beta0;
        for (int i = 0; i < t; ++i) b = b * a.kappa;
        tau[t] = (float)pow((double)b, -1.0 / (2.0 - (double)a.p));
    }
    for (int i = lane; i < NS; i += 64) ring_free[i] = (uint8_t)i;
    __syncthreads();
    const float tau_min = a.iters > 0 ? tau[a.iters - 1] * (1.0f - 4e-6f) : 0.0f;
    const double pm1 = (double)a.p - 1.0;

    uint32_t act_h = 0, act_n = 0, fin_h = 0, fin_n = 0, exq_h = 0, exq_n = 0, fre_h = 0, fre_n = NS;

    // ---- tile claiming and prefetch -------------------------------------------------------
    int64_t tile = 0, tile_end = 0;
    int cur_job = 0;
    bool pf_ok = false;
    int pf_job = 0, pf_nv = 0;
    int64_t pf_g0 = 0;
    u32x4 pf[E / 8];                             // prefetched weights of the next tile

    auto prefetch = [&]() {
        if (tile >= tile_end) {
            uint32_t base = 0;
            if (lane == 0) base = atomic_add_g(a.counter, a.chunk);
            base = uniform(base);
            if ((int64_t)base >= a.n_tiles) {
                pf_ok = false;
#pragma unroll
                for (int i = 0; i < E / 8; ++i) pf[i] = u32x4{0u, 0u, 0u, 0u};
                return;
            }
            tile = base;
            tile_end = (int64_t)base + a.chunk < a.n_tiles ? (int64_t)base + a.chunk : a.n_tiles;
        }
        // job of this tile (jobs are ordered by tile0); wave-uniform, so scalar loads
        while (cur_job + 1 < a.n_jobs && jobs[cur_job + 1].tile0 <= tile)
            cur_job = (int)uniform((uint32_t)cur_job + 1);
        while (jobs[cur_job].tile0 > tile) cur_job = (int)uniform((uint32_t)cur_job - 1);
        const DevJob &J = jobs[cur_job];
        const int64_t g0 = (tile - J.tile0) * GPI;
        const int64_t left = J.n_groups - g0;
        pf_nv = (int)uniform((uint32_t)(left < GPI ? left : GPI));
        pf_g0 = g0;
        pf_job = cur_job;
        // The next tile's weights stay in flight in registers until INIT uses them. Every
        // lane loads (lanes past a ragged end re-read the tile's first group), so the old
        // register contents are dead when the loads are issued.
        const int64_t gl = g0 + (k < pf_nv ? k : 0);
        const u32x4 *src = reinterpret_cast<const u32x4 *>(J.W + gl * G + sub * E);
#pragma unroll
        for (int i = 0; i < E / 8; ++i) pf[i] = gbl(const_cast<u32x4 *>(src))[i];
        pf_ok = true;
        ++tile;
    };

    // ---- queue pushes (one entry per group, by its leader lane) -------------------------
    auto push = [&](bool valid, uint8_t out, uint8_t slot) {
        const uint64_t m_act = __ballot(valid && leader && out == kActive);
        const uint64_t m_fin = __ballot(valid && leader && out == kFinished);
        const uint64_t m_exq = __ballot(valid && leader && out == kExact);
        if (valid && leader) {
            if (out == kActive) ring_act[(act_h + act_n + lanes_below(m_act)) & RM] = slot;
            else if (out == kFinished) ring_fin[(fin_h + fin_n + lanes_below(m_fin)) & RM] = slot;
            else ring_exq[(exq_h + exq_n + lanes_below(m_exq)) & RM] = slot;
        }
        act_n += (uint32_t)__builtin_popcountll(m_act);
        fin_n += (uint32_t)__builtin_popcountll(m_fin);
        exq_n += (uint32_t)__builtin_popcountll(m_exq);
    };

    // ---- after an accepted evaluation (zb, Qb, Db, sbx already current in registers):
    //      the next zero, or finished / exact path. Writes the fields it changes.
    auto advance = [&](uint8_t slot, float s, float zb, float Qb, float Db, bool sbx) -> uint8_t {
        const int t = st_t[slot];
        if (t > a.iters) return kFinished;
        // Dead zone of the shrink: max|r| = max|u - q|/s <= beta^(-1/(2-p)), tested with a
        // relative margin of 4e-6 that covers the binary32 rounding of the products. The
        // smallest threshold (the last beta) decides most groups at once, for this and every
        // later iteration.
        const float dmax = sbx ? Db : Db + (0.5f - C::kThr);
        const bool dead_all = dmax <= tau_min * s;
        if (!dead_all && !(dmax <= tau[t - 1] * (s * (1.0f - 4e-6f)))) {
            if (leader) st_fl[slot] = (uint8_t)((sbx ? 1 : 0) | (kShrink << 1));
            return kExact;                           // the shrink may move residuals
        }
        const float zn = (float)(((double)Qb - st_sxs[slot]) * (1.0 / G));
        if (zn == zb && dead_all) {                  // exact fixed point
            if (leader) st_zb[slot] = zn;
            return kFinished;
        }
        if (leader) {
            st_z[slot] = zn;
            st_beta[slot] = st_beta[slot] * a.kappa;
            st_t[slot] = (uint8_t)(t + 1);
        }
        return kActive;
    };

    int mm_job = -1;                             // running zero (min, max) of one tensor
    float mm_lo = INFINITY, mm_hi = -INFINITY;
    auto flush_minmax = [&]() {
        if (mm_job >= 0 && lane == 0) {
            atomic_min_g(jobs[mm_job].minmax, fkey(mm_lo));
            atomic_max_g(jobs[mm_job].minmax + 1, fkey(mm_hi));
        }
    };

    prefetch();

    while (true) {
        if (pf_ok && act_n < GPI && fre_n >= GPI) {
            // ================= INIT: a prefetched tile enters the pool =================
            const int nv = pf_nv;
            const bool valid = k < nv;
            uint8_t slot = 0;
            if (valid) slot = ring_free[(fre_h + k) & RM];
            fre_h = (fre_h + nv) & RM;
            fre_n -= nv;
            uint8_t out = kFinished;
            if (valid) {
                uint32_t xr[W];
                u32x4 *dst = reinterpret_cast<u32x4 *>(xs + slot * G + sub * E);
#pragma unroll
                for (int i = 0; i < E / 8; ++i) {
                    const u32x4 v = pf[i];
                    dst[i] = v;
                    xr[4 * i] = v.x;
                    xr[4 * i + 1] = v.y;
                    xr[4 * i + 2] = v.z;
                    xr[4 * i + 3] = v.w;
                }
                // min / max on binary16 pairs, then across the group
                h2v hmn = __builtin_bit_cast(h2v, xr[0]), hmx = hmn;
#pragma unroll
                for (int i = 1; i < W; ++i) {
                    const h2v h = __builtin_bit_cast(h2v, xr[i]);
                    hmn = __builtin_elementwise_min(hmn, h);
                    hmx = __builtin_elementwise_max(hmx, h);
                }
                float mn = fminf((float)hmn.x, (float)hmn.y);
                float mx = fmaxf((float)hmx.x, (float)hmx.y);
                mn = minf_k<K>(mn);
                mx = maxf_k<K>(mx);
                const float rng = mx - mn;
                const float s = rng > 0.0f ? C::QMAX / rng : 1.0f;
                const float z0 = 0.0f - mn * s;      // +0 when min is a zero of either sign
                const double sd = s;
                double sxs = 0.0;
#pragma unroll
                for (int i = 0; i < 2 * W; ++i)
                    sxs = fma((double)h2f(i & 1 ? xr[i >> 1] >> 16 : xr[i >> 1] & 0xffffu), sd, sxs);
                sxs = addd_k<K>(sxs);
                float S, Q, D;
                eval_fast<NBITS, G, false>(xr, s, z0, S, Q, D);
                S = addf_k<K>(S);
                Q = addf_k<K>(Q);
                D = maxf_k<K>(D);
                double Sb = S;
                bool sbx = false;
                if (D >= C::kThr) {                  // a code may differ from the exact one
                    const Exact x0 = eval_exact<NBITS, G>(xs + slot * G + sub * E, s, z0);
                    Sb = addd_k<K>(x0.S);
                    Q = (float)addd_k<K>(x0.Q);
                    D = (float)maxf_k<K>((float)x0.D);
                    sbx = true;
                }
                if (leader) {
                    st_z[slot] = z0;
                    st_zb[slot] = z0;
                    st_s[slot] = s;
                    st_beta[slot] = a.beta0;
                    st_Qb[slot] = Q;
                    st_Db[slot] = D;
                    st_Sb[slot] = Sb;
                    st_sxs[slot] = sxs;
                    st_mnmx[slot] = (uint32_t)f2h(mn) | ((uint32_t)f2h(mx) << 16);
                    st_gidx[slot] = (uint32_t)(pf_g0 + k);
                    st_job[slot] = (uint16_t)pf_job;
                    st_t[slot] = 1;
                    st_fl[slot] = sbx ? 1 : 0;
                }
                out = advance(slot, s, z0, Q, D, sbx);
            }
            push(valid, out, slot);
            prefetch();
            continue;
        }

        if (fin_n >= GPI || (fin_n > 0 && act_n < GPI && (fre_n < GPI || !pf_ok))) {
            // ================= EPILOGUE: codes, packing, scale / zero ===================
            // One tensor per batch (descriptor in scalar registers); groups of another tensor
            // go back to the finished list for a later batch.
            const int n = fin_n < GPI ? (int)fin_n : GPI;
            bool valid = k < n;
            uint8_t slot = 0;
            if (valid) slot = ring_fin[(fin_h + k) & RM];
            fin_h = (fin_h + n) & RM;
            fin_n -= n;
            uint32_t job = 0;
            if (valid) job = st_job[slot];
            const uint32_t job0 = uniform(job);      // lane 0 always holds a group
            const bool later = valid && job != job0;
            const uint64_t m_later = __ballot(later && leader);
            if (later && leader) ring_fin[(fin_h + fin_n + lanes_below(m_later)) & RM] = slot;
            fin_n += (uint32_t)__builtin_popcountll(m_later);
            valid = valid && !later;
            const DevJob &J = jobs[job0];
            float zb = 0.f;
            uint32_t code[E];
            uint32_t gidx = 0;
            if (valid) {
                zb = st_zb[slot];
                const float s = st_s[slot];
                gidx = st_gidx[slot];
                const uint16_t *xl = xs + slot * G + sub * E;
                uint32_t xr[W];
#pragma unroll
                for (int i = 0; i < E / 8; ++i) {
                    const uint4 v = reinterpret_cast<const uint4 *>(xl)[i];
                    xr[4 * i] = v.x;
                    xr[4 * i + 1] = v.y;
                    xr[4 * i + 2] = v.z;
                    xr[4 * i + 3] = v.w;
                }
                uint32_t near = 0;                   // codes next to a rounding boundary
#pragma unroll
                for (int i = 0; i < E; ++i) {
                    const uint32_t h = i & 1 ? xr[i >> 1] >> 16 : xr[i >> 1] & 0xffffu;
                    const float u = fmaf(h2f(h), s, zb);
                    const float r = rintf(u);
                    near |= (fabsf(u - r) >= C::kThr ? 1u : 0u) << i;
                    code[i] = (uint32_t)__builtin_amdgcn_fmed3f(r, 0.f, C::QMAX);
                }
                if (near) {                          // exact codes there (binary64)
#pragma unroll 1
                    for (int i = 0; i < E; ++i) {
                        if (near >> i & 1u) {
                            const double u = fma((double)h2f(xl[i]), (double)s, (double)zb);
                            const uint32_t c = (uint32_t)fmin(fmax(rint(u), 0.0), (double)C::QMAX);
#pragma unroll
                            for (int j = 0; j < E; ++j)
                                if (j == i) code[j] = c;
                        }
                    }
                }
                const int64_t e0 = (int64_t)gidx * G + sub * E;   // first weight of this lane
                if constexpr (NBITS == 8) {
                    auto dst = gbl(reinterpret_cast<u32x4 *>(J.packed + e0));
#pragma unroll
                    for (int i = 0; i < E / 16; ++i) {
                        u32x4 o;
                        o.x = code[16 * i] | code[16 * i + 1] << 8 | code[16 * i + 2] << 16 | code[16 * i + 3] << 24;
                        o.y = code[16 * i + 4] | code[16 * i + 5] << 8 | code[16 * i + 6] << 16 | code[16 * i + 7] << 24;
                        o.z = code[16 * i + 8] | code[16 * i + 9] << 8 | code[16 * i + 10] << 16 | code[16 * i + 11] << 24;
                        o.w = code[16 * i + 12] | code[16 * i + 13] << 8 | code[16 * i + 14] << 16 | code[16 * i + 15] << 24;
                        dst[i] = o;
                    }
                } else if constexpr (NBITS == 4 || NBITS == 2 || NBITS == 1) {
                    constexpr int PER = 32 / NBITS;       // codes per 32-bit word
                    constexpr int NW = E / PER > 0 ? E / PER : 1;
                    uint32_t w[NW];
#pragma unroll
                    for (int i = 0; i < NW; ++i) w[i] = 0;
#pragma unroll
                    for (int i = 0; i < E; ++i) w[i / PER] |= code[i] << (NBITS * (i % PER));
                    uint8_t *dst = J.packed + e0 * NBITS / 8;
                    if constexpr (E * NBITS == 128)
                        *gbl(reinterpret_cast<u32x4 *>(dst)) = u32x4{w[0], w[1], w[2], w[3]};
                    else if constexpr (E * NBITS == 64)
                        *gbl(reinterpret_cast<u32x2 *>(dst)) = u32x2{w[0], w[1]};
                    else if constexpr (E * NBITS == 32)
                        *gbl(reinterpret_cast<uint32_t *>(dst)) = w[0];
                    else
                        *gbl(reinterpret_cast<uint16_t *>(dst)) = (uint16_t)w[0];
                }
                if (leader) {
                    gbl(J.scale)[gidx] = f2h(1.0f / s);
                    if (J.zero16) gbl(J.zero16)[gidx] = f2h(zb);
                    if (J.zero32) gbl(J.zero32)[gidx] = zb;
                    // evaluations run = index of the next update when the group stops
                    if (J.passes) gbl(J.passes)[gidx] = st_t[slot];
                }
                if constexpr (NBITS == 3) {
#pragma unroll
                    for (int i = 0; i < E; ++i) stage[lane * E + i] = (uint8_t)code[i];
                }
            }
            if constexpr (NBITS == 3) {
                // Flat 10-code words: words wholly inside the group are written here; a word
                // shared with a neighbouring group goes to the stash (joined after the solve).
                __syncthreads();
                if (valid) {
                    const int64_t c0 = (int64_t)gidx * G;          // first code of the group
                    const int64_t c1 = c0 + G;                      // one past the last
                    const int64_t ncode = J.n_groups * G;
                    const int64_t w0 = c0 / 10, w1 = (c1 - 1) / 10;
                    auto out = gbl(reinterpret_cast<uint32_t *>(J.packed));
                    for (int64_t w = w0 + sub; w <= w1; w += K) {
                        uint32_t word = 0;
#pragma unroll
                        for (int c = 0; c < 10; ++c) {
                            const int64_t ci = w * 10 + c;
                            if (ci >= c0 && ci < c1)
                                word |= (uint32_t)stage[k * G + (int)(ci - c0)] << (3 * c);
                        }
                        const bool head = w * 10 < c0;                  // shared with group-1
                        const bool tail = w * 10 + 10 > c1 && c1 < ncode; // shared with group+1
                        uint32_t *st2 = reinterpret_cast<uint32_t *>(J.stash + gidx);
                        if (head) gbl(st2)[1] = word;
                        else if (tail) gbl(st2)[0] = word;
                        else out[w] = word;
                    }
                }
                __syncthreads();
            }
            // Per-tensor (min, max) of the binary32 zeros for the 8-bit requantization: a
            // running pair per wave, flushed with atomics only when the tensor changes (all
            // waves work on the same tensor at once, so per-batch atomics would serialise).
            if (J.minmax) {
                float lo = valid ? zb : INFINITY, hi = valid ? zb : -INFINITY;
                lo = __builtin_bit_cast(float, uniform(__float_as_uint(minf_k<64>(lo))));
                hi = __builtin_bit_cast(float, uniform(__float_as_uint(maxf_k<64>(hi))));
                if ((int)job0 != mm_job) {
                    flush_minmax();
                    mm_job = (int)job0;
                    mm_lo = lo;
                    mm_hi = hi;
                } else {
                    mm_lo = fminf(mm_lo, lo);
                    mm_hi = fmaxf(mm_hi, hi);
                }
            }
            const uint64_t m_done = __ballot(valid && leader);
            if (valid && leader) ring_free[(fre_h + fre_n + lanes_below(m_done)) & RM] = slot;
            fre_n += (uint32_t)__builtin_popcountll(m_done);
            continue;
        }

        if (exq_n >= GPI || (exq_n > 0 && act_n < GPI && (fre_n < GPI || !pf_ok))) {
            // ================= EXACT: binary64 decisions and shrink updates ==============
            const int n = exq_n < GPI ? (int)exq_n : GPI;
            const bool valid = k < n;
            uint8_t slot = 0;
            if (valid) slot = ring_exq[(exq_h + k) & RM];
            exq_h = (exq_h + n) & RM;
            exq_n -= n;
            uint8_t out = kFinished;
            if (valid) {
                const uint16_t *xl = xs + slot * G + sub * E;
                const float s = st_s[slot];
                const uint8_t fl = st_fl[slot];
                if ((fl >> 1) == kDecide) {
                    const float z = st_z[slot];
                    const Exact xn = eval_exact<NBITS, G>(xl, s, z);
                    const double S = addd_k<K>(xn.S);
                    const float Q = (float)addd_k<K>(xn.Q);
                    const float D = maxf_k<K>((float)xn.D);
                    double Sb = st_Sb[slot];
                    if (!(fl & 1)) Sb = addd_k<K>(eval_exact<NBITS, G>(xl, s, st_zb[slot]).S);
                    if (!a.early_stop || S <= Sb) {
                        if (leader) {
                            st_zb[slot] = z;
                            st_Sb[slot] = S;
                            st_Qb[slot] = Q;
                            st_Db[slot] = D;
                            st_fl[slot] = 1;
                        }
                        out = advance(slot, s, z, Q, D, true);
                    } else {
                        out = kFinished;
                    }
                } else {
                    // zero update with the shrink live: z = mean(q - (x - W_e)*s), W_e from
                    // the residual r = x - W_r = (u - q)/s of the accepted iterate.
                    const double sd = s, zd = st_zb[slot], qm = C::QMAX;
                    const double beta = st_beta[slot];
                    double acc = 0.0;
#pragma unroll 1
                    for (int i = 0; i < E; ++i) {
                        const double xv = h2f(xl[i]);
                        const double u = fma(xv, sd, zd);
                        const double c = fmin(fmax(rint(u), 0.0), qm);
                        const double we = shrink((u - c) / sd, pm1, beta);
                        acc += c - (xv - we) * sd;
                    }
                    acc = addd_k<K>(acc);
                    if (leader) {
                        st_z[slot] = (float)(acc * (1.0 / G));
                        st_beta[slot] = st_beta[slot] * a.kappa;
                        st_t[slot] = (uint8_t)(st_t[slot] + 1);
                        st_fl[slot] = fl & 1;
                    }
                    out = kActive;
                }
            }
            push(valid, out, slot);
            continue;
        }

        if (act_n > 0) {
            // ================= PASS: evaluate up to GPI active groups =====================
            const int n = act_n < GPI ? (int)act_n : GPI;
            const bool valid = k < n;
            uint8_t slot = 0;
            if (valid) slot = ring_act[(act_h + k) & RM];
            act_h = (act_h + n) & RM;
            act_n -= n;
            uint32_t xr[W];
            float z = 0.f, s = 1.f, Sb = 0.f;
            uint8_t fl = 0;
            bool clampfree = true;
            if (valid) {
                z = st_z[slot];
                s = st_s[slot];
                Sb = (float)st_Sb[slot];
                fl = st_fl[slot];
                const uint32_t mm = st_mnmx[slot];
                const uint4 *src = reinterpret_cast<const uint4 *>(xs + slot * G + sub * E);
#pragma unroll
                for (int i = 0; i < E / 8; ++i) {
                    const uint4 v = src[i];
                    xr[4 * i] = v.x;
                    xr[4 * i + 1] = v.y;
                    xr[4 * i + 2] = v.z;
                    xr[4 * i + 3] = v.w;
                }
                const float ulo = fmaf(h2f(mm & 0xffffu), s, z);
                const float uhi = fmaf(h2f(mm >> 16), s, z);
                clampfree = ulo >= -0.5f && uhi < C::QMAX + 0.5f;
            }
            const bool any_clamp = __ballot(valid && !clampfree) != 0;
            uint8_t out = kFinished;
            if (valid) {
                float S, Q, D;
                if (any_clamp) eval_fast<NBITS, G, true>(xr, s, z, S, Q, D);
                else eval_fast<NBITS, G, false>(xr, s, z, S, Q, D);
                S = addf_k<K>(S);
                Q = addf_k<K>(Q);
                D = maxf_k<K>(D);
                bool accept = false;
                if (D >= C::kThr) {
                    if (leader) st_fl[slot] = (uint8_t)((fl & 1) | (kDecide << 1));
                    out = kExact;
                } else if (!a.early_stop) {
                    accept = true;
                } else {
                    // |S - S_exact| bounds (binary32 sums: G half-ulps of u plus the relative
                    // summation error; clamped elements may sit above 2^NBITS where the ulp is
                    // larger, so a clamped pass takes a wider bound). The margins are far above
                    // the binary32 rounding of this comparison itself.
                    const float em = any_clamp ? 4.0f * (float)C::kElemErr : (float)C::kElemErr;
                    const float m = em + S * 0x1p-18f +
                                    ((fl & 1) ? 0x1p-18f * Sb : 4.0f * (float)C::kElemErr + Sb * 0x1p-18f);
                    if (S > Sb + m) out = kFinished;
                    else if (S < Sb - m) accept = true;
                    else {
                        if (leader) st_fl[slot] = (uint8_t)((fl & 1) | (kDecide << 1));
                        out = kExact;
                    }
                }
                if (accept) {
                    if (leader) {
                        st_zb[slot] = z;
                        st_Sb[slot] = S;
                        st_Qb[slot] = Q;
                        st_Db[slot] = D;
                        st_fl[slot] = 0;
                    }
                    out = advance(slot, s, z, Q, D, false);
                }
            }
            push(valid, out, slot);
            continue;
        }
        break;
    }
    flush_minmax();
}

template <int NBITS, int G>
hipError_t launch_one(const StreamArgs &args, hipStream_t stream)
{
    if (args.n_tiles == 0) return hipSuccess;
    StreamArgs a = args;
    // Persistent grid: as many single-wave workgroups as the LDS pool lets the CUs hold; tiles
    // are claimed in chunks small enough to balance the waves (about 16 claims per wave).
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            cus = v;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stream_kernel<NBITS, G>, 64, 0) !=
            hipSuccess || per_cu <= 0)
        per_cu = 4;
    const int64_t waves = (int64_t)cus * per_cu;
    int64_t chunk = a.n_tiles / (waves * 16);
    chunk = chunk < 1 ? 1 : (chunk > 32 ? 32 : chunk);
    a.chunk = (uint32_t)chunk;
    const int64_t claims = (a.n_tiles + chunk - 1) / chunk;
    const int64_t grid = waves < claims ? waves : claims;
    hipLaunchKernelGGL((stream_kernel<NBITS, G>), dim3((unsigned)grid), dim3(64), 0, stream, a,
                       a.jobs);
    return hipGetLastError();
}

template <int NBITS>
hipError_t launch_bits(const StreamArgs &a, int g, hipStream_t stream)
{
    switch (g) {
    case 16: return launch_one<NBITS, 16>(a, stream);
    case 32: return launch_one<NBITS, 32>(a, stream);
    case 64: return launch_one<NBITS, 64>(a, stream);
    case 128: return launch_one<NBITS, 128>(a, stream);
    case 256: return launch_one<NBITS, 256>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

__global__ void fill_kernel(FillArgs f, DevJob *table)
{
    const int i = threadIdx.x;
    if (i < f.n) {
        const DevJob j = f.jobs[i];
        table[f.offset + i] = j;
        if (j.minmax) {
            j.minmax[0] = 0xffffffffu;
            j.minmax[1] = 0u;
        }
    }
    if (f.offset == 0)
        for (int c = i; c < f.n_counters; c += blockDim.x) f.counters[c] = 0u;
}

}  // namespace

int64_t tiles_for(int64_t n_groups, int g)
{
    const int E = g >= 32 ? 32 : 16;
    const int64_t gpi = 64 / (g / E);
    return (n_groups + gpi - 1) / gpi;
}

hipError_t launch_fill(const FillArgs &f, DevJob *table, hipStream_t stream)
{
    hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(64), 0, stream, f, table);
    return hipGetLastError();
}

hipError_t launch_stream(const StreamArgs &a, int nbits, int g, hipStream_t stream)
{
    switch (nbits) {
    case 1: return launch_bits<1>(a, g, stream);
    case 2: return launch_bits<2>(a, g, stream);
    case 3: return launch_bits<3>(a, g, stream);
    case 4: return launch_bits<4>(a, g, stream);
    case 8: return launch_bits<8>(a, g, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hqq
