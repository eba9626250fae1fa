// hqq_stream.hip -- the HQQ group solver for gfx950: persistent waves in which every lane owns
// one group, its weights held in registers from the first evaluation to the last.
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
// Scheduling (one wave per workgroup, persistent):
//  * PASS: each lane (a lane pair for G = 256) holds one group's weights in VGPRs together
//    with its solver state, evaluates it at its candidate zero and takes the stop / accept /
//    next-zero decision itself. No data moves between lanes and nothing touches memory.
//  * A group that finishes, or whose decision needs the exact path, leaves its lane for a
//    staging slot in LDS; the lane takes a ready group from LDS in its place. When both
//    exist they exchange (in place with LDS atomic swaps for a group held by one lane, through
//    a spare slot for one spread over a lane pair), so the pool can never block.
//  * Work that is cheaper across lanes runs in batches of GB groups with KB lanes per group
//    (EB weights per lane): INIT (a prefetched tile of GB groups: min/max, s, z0, exact
//    sum x*s, the tile's scales stored; the groups become ready), EXACT (binary64 decisions
//    and shrink updates) and EPILOGUE (codes of the accepted zero, packing, zero stores).
//  * The next tile's weights are in flight in registers while the wave works.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "hqq_internal.h"

namespace hqq {
namespace {

enum : uint32_t { kEmpty = 0, kActive = 1, kHoldFin = 2, kHoldExq = 3 };   // a lane's group
// Group flags: bit 0 Sb/Db exact, bits 1-2 exact-path work, bit 3 first evaluation pending.
enum : uint8_t { kSbExact = 1, kFirst = 8 };
enum : uint8_t { kDecide = 1, kShrink = 2 };

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

// Packed binary16 min / max issued directly: through the builtins every loaded operand is first
// quieted (a max of it with itself, one more instruction per pair), which changes only a
// signalling NaN, and weights are finite by contract.
__device__ __forceinline__ uint32_t pk_min_h(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ uint32_t pk_max_h(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Min and max of a group's weights: a tree over the lane's binary16 pairs, then one packed
// word {min, -max} reduced over the K lanes of the group (one packed min per step serves both).
template <int W, int K>
__device__ __forceinline__ void group_min_max(const uint32_t (&xb)[W], float &mn, float &mx)
{
    static_assert(W >= 2 && (W & (W - 1)) == 0, "pairs per lane: a power of two");
    uint32_t lo[W / 2], hi[W / 2];
#pragma unroll
    for (int i = 0; i < W / 2; ++i) {
        lo[i] = pk_min_h(xb[2 * i], xb[2 * i + 1]);
        hi[i] = pk_max_h(xb[2 * i], xb[2 * i + 1]);
    }
#pragma unroll
    for (int w = W / 4; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) {
            lo[i] = pk_min_h(lo[2 * i], lo[2 * i + 1]);
            hi[i] = pk_max_h(hi[2 * i], hi[2 * i + 1]);
        }
    // a = {min of the low halves, max of the low halves}, b the same of the high halves
    const uint32_t a = __builtin_amdgcn_perm(hi[0], lo[0], 0x05040100u);
    const uint32_t b = __builtin_amdgcn_perm(hi[0], lo[0], 0x07060302u);
    uint32_t v;
    asm("v_pk_min_f16 %0, %1, %2 neg_lo:[0,0] neg_hi:[1,1]" : "=v"(v) : "v"(a), "v"(b));
    if (K >= 2) v = pk_min_h(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));
    if (K >= 4) v = pk_min_h(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));
    if (K >= 8) v = pk_min_h(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
    if (K >= 16) v = pk_min_h(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
    if (K >= 32) v = pk_min_h(v, (uint32_t)__shfl_xor((int)v, 16));
    if (K >= 64) v = pk_min_h(v, (uint32_t)__shfl_xor((int)v, 32));
    mn = h2f(v & 0xffffu);
    mx = -h2f(v >> 16);
}

// Sum x*s over a lane's E weights in binary64. Every product is exact; the sum is exact
// unless the group's weights span more than about 2^11 in magnitude, and within an ulp of
// binary64 then. Four chains keep the adds independent.
template <int W>
__device__ __forceinline__ double lane_sum_xs(const uint32_t (&xb)[W], double sd)
{
    static_assert(W % 2 == 0, "pairs per lane: even");
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < W; ++i) {
        acc[(2 * i) & 3] = fma((double)h2f(xb[i] & 0xffffu), sd, acc[(2 * i) & 3]);
        acc[(2 * i + 1) & 3] = fma((double)h2f(xb[i] >> 16), sd, acc[(2 * i + 1) & 3]);
    }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}
// Another lane's value (ds_bpermute from lane src), binary32 or binary64.
__device__ __forceinline__ float bperm_f(int src, float v)
{
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}
__device__ __forceinline__ double bperm_d(int src, double v)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)(b >> 32));
    return __longlong_as_double((long long)((uint64_t)hi << 32 | lo));
}
// Sum of a lane's weights in binary64, for tiles whose weights all lie below 1/(2L) in
// magnitude: v_dot2 against {1, 1} adds a binary16 pair and a running binary32 sum, and chains
// of L pairs stay exact, since every partial sum is a multiple of 2^-24 below 1, which
// binary32 holds (checked on the GPU: all 822,083,584 pairs below 1/2 with a zero addend, and
// random chains of 2, 4 and 8 pairs, subnormals included). The chain sums add exactly in
// binary64 (below 2^23 units of 2^-24). s * (this sum) then rounds the exact sum x*s once, so
// it equals lane_sum_xs's result wherever that one is exact.
template <int W, int L>
__device__ __forceinline__ double lane_sum_x(const uint32_t (&xb)[W])
{
    static_assert(W % L == 0, "whole chains");
    constexpr int NC = W / L, NA = NC < 4 ? NC : 4;
    typedef _Float16 hh2 __attribute__((ext_vector_type(2)));
    const hh2 one = {(_Float16)1.0f, (_Float16)1.0f};
    double acc[NA];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        float p = __builtin_amdgcn_fdot2(__builtin_bit_cast(hh2, xb[c * L]), one, 0.0f, false);
#pragma unroll
        for (int l = 1; l < L; ++l)
            p = __builtin_amdgcn_fdot2(__builtin_bit_cast(hh2, xb[c * L + l]), one, p, false);
        acc[c % NA] = c < NA ? (double)p : acc[c % NA] + (double)p;
    }
    if constexpr (NA == 4) return (acc[0] + acc[1]) + (acc[2] + acc[3]);
    else if constexpr (NA == 2) return acc[0] + acc[1];
    else return acc[0];
}
// A lane's binary64 sum of x for a tile whose largest magnitude am (wave-uniform choice) is
// below 1/2, with the longest exact chains am allows.
template <int W>
__device__ __forceinline__ double lane_sum_x_tile(const uint32_t (&xb)[W], float am)
{
    if (__ballot(am >= 0.25f)) return lane_sum_x<W, 1>(xb);
    if constexpr (W % 4 == 0) {
        if (__ballot(am >= 0.125f)) return lane_sum_x<W, 2>(xb);
        return lane_sum_x<W, 4>(xb);
    } else if constexpr (W % 2 == 0) {
        return lane_sum_x<W, 2>(xb);
    } else {
        return lane_sum_x<W, 1>(xb);
    }
}
// LDS atomic swap of 8 bytes (ds_wrxchg_rtn_b64): stores v, returns the old contents.
__device__ __forceinline__ uint64_t xchg_l(uint64_t *p, uint64_t v)
{
    return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint64_t pack2(float a, float b)
{
    return (uint64_t)__float_as_uint(a) | (uint64_t)__float_as_uint(b) << 32;
}
__device__ __forceinline__ uint64_t pack2(float a, uint32_t b) { return (uint64_t)__float_as_uint(a) | (uint64_t)b << 32; }
__device__ __forceinline__ uint64_t pack2(uint32_t a, uint32_t b) { return (uint64_t)a | (uint64_t)b << 32; }
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }
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

// pow for the rare paths (the shrink and its dead-zone threshold). Out of line: inlined, its
// constants would be hoisted into registers for the whole solver loop.
__device__ __attribute__((noinline)) double pow_ool(double a, double e) { return pow(a, e); }

__device__ __forceinline__ double shrink(double r, double pm1, double beta)
{
    if (r == 0.0) return 0.0;
    const double a = fabs(r);
    const double m = fmax(a - pow_ool(a, pm1) / beta, 0.0);
    return r > 0.0 ? m : -m;
}


// Solver state of a group in a staging slot, as three 16-byte records (one LDS array each, so a
// group moves with three 128-bit accesses). meta packs the flags (bits 0-7), the index of the
// next zero update (8-15) and the tensor (16-31).
struct alignas(16) SlotA {
    float s, z, zb, Db;      // quantizer multiplier, candidate zero, accepted zero, its max|u-q|
};
struct alignas(16) SlotB {
    float beta;              // beta of the next shrink
    uint32_t mnmx;           // binary16 min (low half) and max (high half)
    uint32_t gidx;           // group index within its tensor
    uint32_t meta;
};
struct alignas(16) SlotC {
    double Sb;               // accepted sum |u - q|
    double X;                // exact sum x*s
};
__device__ __forceinline__ uint32_t meta_fl(uint32_t m) { return m & 0xffu; }
__device__ __forceinline__ uint32_t meta_t(uint32_t m) { return (m >> 8) & 0xffu; }
__device__ __forceinline__ uint32_t meta_job(uint32_t m) { return m >> 16; }
__device__ __forceinline__ uint32_t with_fl(uint32_t m, uint32_t fl) { return (m & ~0xffu) | fl; }

// Pass layouts. Wide (the default): a lane owns a group (a lane pair when G = 256), which
// keeps the pass free of cross-lane reductions. Narrow: several lanes share a group (16
// weights each up to g64, 32 above; 4 lanes at g64 and g128), for tensors too small to give
// every lane of the machine several groups: a pass then takes a quarter of the time, so the
// last groups of a launch, which decide its length, finish sooner.
template <int G> constexpr int wide_ep() { return G <= 128 ? G : 128; }
template <int G> constexpr int narrow_ep() { return G <= 16 ? G : (G <= 64 ? 16 : 32); }

template <int NBITS, int G, int EP_ = wide_ep<G>()>
struct Cfg {
    // Pass layout: KP lanes per group, EP weights per lane.
    static constexpr int EP = EP_;
    static constexpr int KP = G / EP;               // lanes per group in a pass
    static constexpr int WP = EP / 2;               // binary16 pairs per lane
    static constexpr bool NARROW = EP < wide_ep<G>();
    // Batch layout (INIT, EXACT, EPILOGUE): KB lanes per group, EB weights per lane.
    static constexpr int EB = G >= 32 ? 32 : 16;
    static constexpr int KB = G / EB;
    static constexpr int GB = 64 / KB;              // groups per batch (one tile)
    static constexpr int WB = EB / 2;
    static constexpr int NC = G / 8;                // 16-byte chunks per group
    // Waves per SIMD the registers allow, and the staging slots that fit that many waves'
    // LDS: 160 KB per compute unit, taken per wave in blocks of 1280 bytes (measured: 12,584
    // bytes per wave let 12 waves share a compute unit, 13,032 only 11), holds each slot's
    // weights and 48 bytes of state, the rings and the 3-bit code stage; at most three
    // batches of slots.
    // (3-bit g32 stays at three: its code stage leaves fewer slots than four waves need.)
    // The narrow layout holds 8 or 16 weight registers per lane and runs four waves (three
    // for 3-bit g32 and g256, whose slot pools would not fit four).
    static constexpr int WAVES =
        NARROW ? (NBITS == 3 && (G == 32 || G >= 256) ? 3 : 4)
               : ((G <= 16 || (G == 32 && NBITS != 3)) ? 4 : (G <= 128 ? 3 : 2));
    static constexpr int RC = GB >= 32 ? 128 : 64;  // ring capacity
    static constexpr int LDS_WAVE = 163840 / (4 * WAVES) / 1280 * 1280;
    static constexpr int LDS_FREE = LDS_WAVE - 4 * RC - (NBITS == 3 ? 64 * EB : 0) - 128;
    // How groups move between lanes and slots. A group held by one lane (g16-g128 in the wide
    // layout) swaps in place with LDS atomic exchanges: half the swaps, measured 10-13 % faster
    // at g16-g64 and 12 % at g128. Groups spread over several lanes (g256, the narrow layout)
    // move with 16-byte stores and loads through free slots and a spare slot.
    static constexpr bool XCHG = KP == 1;
    static_assert(!XCHG || KP == 1, "in-place swaps move one lane per group");
    // one more column of weights (for an odd stride) comes out of the budget first, and with
    // the spare slot two whole slots
    static constexpr int NS_FIT = (LDS_FREE - (XCHG ? 2 * G : 2 * (2 * G + 48))) / (2 * G + 48);
#ifdef HQQ_STRESS_SLOTS
    // stress build for the tests: a pool of one batch plus a few slots, so that free slots
    // are scarce and holders often swap in place or wait
    static constexpr int NS = GB + HQQ_STRESS_SLOTS;
#else
    static constexpr int NS = NS_FIT < 3 * GB ? NS_FIT : 3 * GB;   // staging slots
#endif
    static constexpr int NSP = XCHG ? NS : NS + 1;  // slots including the spare
    static constexpr int CS = NSP | 1;              // chunk stride: odd, at least NSP
    static_assert(NS >= GB + 4 && NS <= RC, "staging slots");
    static constexpr float QMAX = (float)((1 << NBITS) - 1);
    // A binary32 code can disagree with the exact one only if |u - rne(u)| >= kThr.
    static constexpr float kThr = 0.5f - (float)(1.0 / (1 << (24 - NBITS)));
    // Bound on |S_binary32 - S_exact| from the per-element rounding (G halves of an ulp, x2).
    static constexpr double kElemErr = (double)G / (double)(1 << (24 - NBITS));
};

// Binary32 evaluation of N binary16 pairs at zero z, for a group whose codes cannot leave
// [0, 2^NBITS - 1] (the caller checks the group's min and max; clamping groups take the exact
// path): S = sum|u - q|, T = sum(u - q) and D = max|u - q| with q = rne(u). The code sum
// follows from T without a sum of its own: sum q = sum u - T, and sum u differs from the
// exact sum x*s + G*z by at most G half-ulps of u, far below 1/2, so
// Q = rne(sum x*s + G*z - T) is exact.
template <int NBITS, int N>
__device__ __forceinline__ void eval_fast(const uint32_t (&xr)[N], float s, float z, float &S,
                                          float &T, float &D)
{
    float s0 = 0.f, s1 = 0.f, t0 = 0.f, t1 = 0.f, d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float u0 = fmaf(h2f(xr[i] & 0xffffu), s, z);
        const float u1 = fmaf(h2f(xr[i] >> 16), s, z);
        const float e0 = u0 - rintf(u0), e1 = u1 - rintf(u1);
        s0 += fabsf(e0);
        s1 += fabsf(e1);
        t0 += e0;
        t1 += e1;
        d0 = fmaxf(d0, fabsf(e0));
        d1 = fmaxf(d1, fabsf(e1));
    }
    S = s0 + s1;
    T = t0 + t1;
    D = fmaxf(d0, d1);
    // S and T are read only on some outcomes of the decision; without this the compiler sinks
    // their sums into those branches and keeps every residual of the lane alive until then.
    asm volatile("" : "+v"(S), "+v"(T), "+v"(D));
}

// LDS position (in binary16 elements) of 16-byte chunk c of staging slot j, chunk-major with
// a stride of CS chunks: a lane walks its slot at a constant stride (immediate offsets),
// lanes reading the same chunk of different slots touch neighbouring 16-byte words, and with
// CS odd the lanes that read consecutive quarters of one group land in different banks.
template <int CS>
__device__ __forceinline__ int chunk_at(int j, int c)
{
    return (c * CS + j) << 3;
}

struct Exact {
    double S, Q, D;
};

// Exact (binary64) evaluation of one batch lane's EB weights (chunks c0.. of slot j) at zero
// z. Rare: a rolled loop over the 16-byte chunks (one LDS read each), so it adds few
// registers to the binary32 path; the binary64 sums are exact in any order. CLAMP false when
// no weight of the group can leave the code range at z or zb (the caller checks the extreme
// weights), so rint(u) is the code; SB true adds the exact S at a second zero zb in the same
// loop (returned in sb), sharing the loads and the conversions of the weights.
template <class C, bool CLAMP, bool SB>
__device__ __forceinline__ Exact eval_exact_t(const uint16_t *xs, int j, int c0, float s, float z,
                                              float zb, double &sb)
{
    const double sd = s, zd = z, zbd = zb, qm = C::QMAX;
    double s_ = 0.0, q_ = 0.0, d_ = 0.0, sb_ = 0.0;
#pragma unroll 1
    for (int c = 0; c < C::EB / 8; ++c) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(xs + chunk_at<C::CS>(j, c0 + c));
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t h = i & 1 ? w4[i >> 1] >> 16 : w4[i >> 1] & 0xffffu;
            const double x = h2f(h);
            const double u = fma(x, sd, zd);
            const double c2 = CLAMP ? fmin(fmax(rint(u), 0.0), qm) : rint(u);
            const double e = fabs(u - c2);
            s_ += e;
            q_ += c2;
            d_ = fmax(d_, e);
            if constexpr (SB) {
                const double ub = fma(x, sd, zbd);
                sb_ += fabs(ub - (CLAMP ? fmin(fmax(rint(ub), 0.0), qm) : rint(ub)));
            }
        }
    }
    sb = sb_;
    return Exact{s_, q_, d_};
}

// What follows an accepted evaluation (zb, Qb, Db current; sbx: Db is exact): the next zero,
// the end of the group, or the exact path for a zero update whose shrink may be live.
enum : uint8_t { kNext = 0, kDone = 1, kNeedShrink = 2 };
struct Advance {
    uint8_t out;
    float zn;
};
template <class C>
__device__ __forceinline__ Advance advance_core(int t, int iters, float s, float zb, float Qb,
                                                float Db, bool sbx, double X, float beta,
                                                float tau_min, double tau_exp)
{
    constexpr int G = C::KB * C::EB;
    if (t > iters) return Advance{kDone, zb};
    // Dead zone of the shrink: max|r| = max|u - q|/s <= beta^(-1/(2-p)), tested with a
    // relative margin of 4e-6 that covers the binary32 rounding of the products. The
    // smallest threshold (the last beta) decides most groups at once, for this and every
    // later iteration.
    const float dmax = sbx ? Db : Db + (0.5f - C::kThr);
    const bool dead_all = dmax <= tau_min * s;
    if (!dead_all) {
        // this iteration's threshold, from the group's beta (beta0*kappa^(t-1))
        const float tau_t = (float)pow_ool((double)beta, tau_exp);
        if (!(dmax <= tau_t * (s * (1.0f - 4e-6f)))) return Advance{kNeedShrink, zb};
    }
    const float zn = (float)(((double)Qb - X) * (1.0 / G));
    if (zn == zb && dead_all) return Advance{kDone, zn};   // exact fixed point
    return Advance{kNext, zn};
}

template <int NBITS, int G, int EPL>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(Cfg<NBITS, G, EPL>::WAVES)))
stream_kernel(StreamArgs a, const DevJob *__restrict__ jobs)
{
    using C = Cfg<NBITS, G, EPL>;
    constexpr int KP = C::KP, WP = C::WP, EB = C::EB, KB = C::KB, GB = C::GB, WB = C::WB;
    constexpr int NS = C::NS, RM = C::RC - 1;
    static_assert(NS <= 255, "slot indices are bytes");
    constexpr int kSpare = NS;                   // the spare slot (in no ring), g > 64 only

    // Staging slots (and the spare): weights and per-group state (one array per field).
    __shared__ __attribute__((aligned(16))) uint16_t xs[C::CS * G];
    __shared__ SlotA st_a[C::NSP];
    __shared__ SlotB st_b[C::NSP];
    __shared__ SlotC st_c[C::NSP];
    __shared__ uint8_t rings[4 * C::RC];   // slot rings: ready, finished, exact-pending, free
    uint8_t *const ring_rdy = rings, *const ring_fin = rings + C::RC,
                   *const ring_exq = rings + 2 * C::RC, *const ring_free = rings + 3 * C::RC;
    __shared__ __attribute__((aligned(4))) uint8_t stage[NBITS == 3 ? 64 * EB : 4];

    const int lane = threadIdx.x;
    // batch layout
    const int k = lane / KB;                     // group within a batch
    const int sub = lane % KB;                   // part of the group
    const bool bleader = sub == 0;
    // pass layout
    const int part = lane % KP;
    const bool pleader = part == 0;
    const int pbase = lane - part;               // the group's first lane

    // Dead zone of the shrink: iteration t uses beta_{t-1} = beta0*kappa^(t-1) (binary32
    // products in order) and maps r to 0 iff |r| <= beta^(-1/(2-p)). The smallest threshold
    // (the last iteration's) settles most groups for every iteration at once.
    const double tau_exp = -1.0 / (2.0 - (double)a.p);
    float beta_last = a.beta0;
    for (int i = 1; i < a.iters; ++i) beta_last = beta_last * a.kappa;
    const float tau_min = __builtin_bit_cast(
        float, uniform(__float_as_uint(
                   a.iters > 0 ? (float)pow_ool((double)beta_last, tau_exp) * (1.0f - 4e-6f) : 0.0f)));
    for (int i = lane; i < NS; i += 64) ring_free[i] = (uint8_t)i;
    __syncthreads();
    const double pm1 = (double)a.p - 1.0;

    uint32_t rdy_h = 0, rdy_n = 0, fin_h = 0, fin_n = 0, exq_h = 0, exq_n = 0, fre_h = 0, fre_n = NS;

    // ---- the lane's group (pass layout) ---------------------------------------------------
    uint32_t xr[WP];
#pragma unroll
    for (int i = 0; i < WP; ++i) xr[i] = 0u;
    float g_s = 1.f, g_z = 0.f, g_zb = 0.f, g_Db = 0.f, g_beta = 0.f;
    double g_Sb = 0.0, g_X = 0.0;
    uint32_t g_mnmx = 0, g_gidx = 0, g_meta = 0;  // meta: flags, next update index, tensor
    uint32_t status = kEmpty;

    // ---- tile claiming and prefetch (batch layout) ----------------------------------------
    int64_t tile = 0, tile_end = 0;
    int cur_job = 0;
    bool pf_ok = false;
    int pf_job = 0, pf_nv = 0;
    int64_t pf_g0 = 0;
    u32x4 pf[EB / 8];                            // prefetched weights of the next tile

    // Claims the next tile and issues its loads. The loads are issued on every call (past the
    // last tile they re-read the first group of the launch, which is never used), so the
    // prefetch registers have a single definition in the loop and stay in place: a join
    // between a loaded and an unloaded version would copy them, and a copy waits for the loads.
    auto prefetch = [&]() {
        bool ok = true;
        if (tile >= tile_end) {
            uint32_t base = 0;
            if (lane == 0) base = atomic_add_g(a.counter, a.chunk);
            base = uniform(base);
            ok = (int64_t)base < a.n_tiles;
            tile = base;
            tile_end = (int64_t)base + a.chunk < a.n_tiles ? (int64_t)base + a.chunk : a.n_tiles;
        }
        const uint16_t *src_w = jobs[0].W;
        int64_t g0 = 0;
        if (ok) {
            // job of this tile (jobs are ordered by tile0); wave-uniform, so scalar loads
            while (cur_job + 1 < a.n_jobs && jobs[cur_job + 1].tile0 <= tile)
                cur_job = (int)uniform((uint32_t)cur_job + 1);
            while (jobs[cur_job].tile0 > tile) cur_job = (int)uniform((uint32_t)cur_job - 1);
            const DevJob &J = jobs[cur_job];
            g0 = (tile - J.tile0) * GB;
            const int64_t left = J.n_groups - g0;
            pf_nv = (int)uniform((uint32_t)(left < GB ? left : GB));
            pf_g0 = g0;
            pf_job = cur_job;
            src_w = J.W;
            ++tile;
        } else {
            pf_nv = 1;                           // the dummy load reads group 0 of job 0
        }
        pf_ok = ok;
        // Every lane loads (lanes past a ragged end re-read the tile's first group). The loads
        // stay below the last use of the previous tile's registers, so the two share registers.
        __builtin_amdgcn_sched_barrier(0);
        const int64_t gl = g0 + (k < pf_nv ? k : 0);
        const u32x4 *src = reinterpret_cast<const u32x4 *>(src_w + gl * G + sub * EB);
#pragma unroll
        for (int i = 0; i < EB / 8; ++i) pf[i] = gbl(const_cast<u32x4 *>(src))[i];
    };

    // Rank of this lane's group among the groups whose leading lane is set in m.
    auto group_rank = [&](uint64_t m, int first_lane) -> uint32_t {
        return (uint32_t)lanes_below(m & ~(1ull << first_lane));
    };

    // Pushes slot j of each batch group onto the ring its outcome names (leaders only).
    auto push_batch = [&](bool valid, uint8_t out, uint8_t j) {
        const uint64_t m_rdy = __ballot(valid && bleader && out == kNext);
        const uint64_t m_fin = __ballot(valid && bleader && out == kDone);
        const uint64_t m_exq = __ballot(valid && bleader && out == kNeedShrink);
        if (valid && bleader) {
            if (out == kNext) ring_rdy[(rdy_h + rdy_n + lanes_below(m_rdy)) & RM] = j;
            else if (out == kDone) ring_fin[(fin_h + fin_n + lanes_below(m_fin)) & RM] = j;
            else ring_exq[(exq_h + exq_n + lanes_below(m_exq)) & RM] = j;
        }
        rdy_n += (uint32_t)__builtin_popcountll(m_rdy);
        fin_n += (uint32_t)__builtin_popcountll(m_fin);
        exq_n += (uint32_t)__builtin_popcountll(m_exq);
    };

    // Batch version of the advance step, on slot j (fields written by the group's leader).
    auto advance_slot = [&](uint8_t j, float s, float zb, float Qb, float Db, bool sbx) -> uint8_t {
        const uint32_t m = st_b[j].meta;
        const int t = (int)meta_t(m);
        const Advance ad = advance_core<C>(t, a.iters, s, zb, Qb, Db, sbx, st_c[j].X,
                                                  st_b[j].beta, tau_min, tau_exp);
        if (bleader) {
            if (ad.out == kDone) st_a[j].zb = ad.zn;
            else if (ad.out == kNeedShrink) st_b[j].meta = with_fl(m, (sbx ? kSbExact : 0) | (kShrink << 1));
            else {
                st_a[j].z = ad.zn;
                st_b[j].beta = st_b[j].beta * a.kappa;
                st_b[j].meta = m + (1u << 8);
            }
        }
        return ad.out;
    };

    // Solver state of a group in a slot (read by every lane of the group, written by its
    // first lane) and in the lane's registers.
    struct GroupState {
        SlotA a;
        SlotB b;
        SlotC c;
    };
    auto load_state = [&](int j) -> GroupState { return GroupState{st_a[j], st_b[j], st_c[j]}; };
    auto put_state = [&](int j, const GroupState &n) {
        st_a[j] = n.a;
        st_b[j] = n.b;
        st_c[j] = n.c;
    };
    auto cur_state = [&]() -> GroupState {
        return GroupState{SlotA{g_s, g_z, g_zb, g_Db}, SlotB{g_beta, g_mnmx, g_gidx, g_meta},
                          SlotC{g_Sb, g_X}};
    };
    // Swaps the state in slot j with n (LDS atomic swaps, 8 bytes each); returns the old state.
    auto xchg_state = [&](int j, const GroupState &n) -> GroupState {
        uint64_t *pa = reinterpret_cast<uint64_t *>(&st_a[j]);
        uint64_t *pb = reinterpret_cast<uint64_t *>(&st_b[j]);
        uint64_t *pc = reinterpret_cast<uint64_t *>(&st_c[j]);
        const uint64_t a0 = xchg_l(pa, pack2(n.a.s, n.a.z)), a1 = xchg_l(pa + 1, pack2(n.a.zb, n.a.Db));
        const uint64_t b0 = xchg_l(pb, pack2(n.b.beta, n.b.mnmx)), b1 = xchg_l(pb + 1, pack2(n.b.gidx, n.b.meta));
        const uint64_t c0 = xchg_l(pc, __double_as_longlong(n.c.Sb)), c1 = xchg_l(pc + 1, __double_as_longlong(n.c.X));
        return GroupState{SlotA{lo_f(a0), hi_f(a0), lo_f(a1), hi_f(a1)},
                          SlotB{lo_f(b0), (uint32_t)(b0 >> 32), (uint32_t)b1, (uint32_t)(b1 >> 32)},
                          SlotC{__longlong_as_double(c0), __longlong_as_double(c1)}};
    };
    auto set_state = [&](const GroupState &n) {
        g_s = n.a.s;
        g_z = n.a.z;
        g_zb = n.a.zb;
        g_Db = n.a.Db;
        g_beta = n.b.beta;
        g_mnmx = n.b.mnmx;
        g_gidx = n.b.gidx;
        g_meta = n.b.meta;
        g_Sb = n.c.Sb;
        g_X = n.c.X;
    };

    // Per-tensor (min, max) of the binary32 zeros for the 8-bit requantization: a running pair
    // per lane for the tensor the wave's batches currently belong to, reduced over the wave and
    // flushed with atomics only when that tensor changes (all waves work on the same tensors
    // at once, so atomics per batch would serialise).
    int mm_job = -1;
    float mm_lo = INFINITY, mm_hi = -INFINITY;
    auto flush_minmax = [&]() {
        if (mm_job >= 0) {
            const float lo = minf_k<64>(mm_lo), hi = maxf_k<64>(mm_hi);
            if (lane == 0) {
                uint32_t *mm = jobs[mm_job].minmax + kMinmaxStride * (blockIdx.x % kMinmaxSlots);
                atomic_min_g(mm, fkey(lo));
                atomic_max_g(mm + 1, fkey(hi));
            }
        }
        mm_lo = INFINITY;
        mm_hi = -INFINITY;
    };

    // ================= EPILOGUE: codes, packing, scale / zero of up to GB finished groups
    auto epilogue = [&]() {
        __builtin_amdgcn_s_setprio(0);
        // One tensor per batch (descriptor in scalar registers); groups of another tensor
        // go back to the finished list for a later batch.
        const int n = fin_n < GB ? (int)fin_n : GB;
        bool valid = k < n;
        uint8_t j = 0;
        if (valid) j = ring_fin[(fin_h + k) & RM];
        fin_h = (fin_h + n) & RM;
        fin_n -= n;
        uint32_t job = 0;
        if (valid) job = meta_job(st_b[j].meta);
        const uint32_t job0 = uniform(job);      // lane 0 always holds a group
        const bool later = valid && job != job0;
        const uint64_t m_later = __ballot(later && bleader);
        if (later && bleader) ring_fin[(fin_h + fin_n + lanes_below(m_later)) & RM] = j;
        fin_n += (uint32_t)__builtin_popcountll(m_later);
        valid = valid && !later;
        const DevJob &J = jobs[job0];
        float zb = 0.f;
        uint32_t gidx = 0;
        if (valid) {
            const SlotA sa = st_a[j];
            zb = sa.zb;
            const float s = sa.s;
            gidx = st_b[j].gidx;
            const int64_t e0 = (int64_t)gidx * G + sub * EB;   // first weight of this lane
            // Packs this lane's EB codes and stores them, a 16-byte chunk of weights at a
            // time. val(h) maps a weight's binary16 bits to either its exact code or a u whose
            // code is rne(u) in [0, 2^NBITS - 1]: v_cvt_pk_u8_f32 rounds half to even and
            // saturates to [0, 255], so either way it yields the code. Byte b of plane m of
            // word q holds code PER*q + PL*b + m, so plane m shifts by NBITS*m (3-bit codes:
            // one per byte, joined into words below).
            auto emit = [&](auto val) {
                constexpr int PL = NBITS == 3 ? 1 : 8 / NBITS;   // planes
                constexpr int BY = EB / PL < 4 ? EB / PL : 4;    // bytes per word
                constexpr int PER = BY * PL;           // codes per word
                constexpr int NW = EB / PER;
                uint32_t pl[NW][PL];
#pragma unroll
                for (int q = 0; q < NW; ++q)
#pragma unroll
                    for (int m = 0; m < PL; ++m) pl[q][m] = 0u;
#pragma unroll
                for (int c = 0; c < EB / 8; ++c) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(xs + chunk_at<C::CS>(j, sub * (EB / 8) + c));
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int i = 8 * c + e;
                        const uint32_t h = e & 1 ? w4[e >> 1] >> 16 : w4[e >> 1] & 0xffffu;
                        const int q = i / PER, m = i % PL, b = (i % PER) / PL;
                        pl[q][m] = __builtin_amdgcn_cvt_pk_u8_f32(val(h), b, pl[q][m]);
                    }
                }
                uint32_t w[NW];
#pragma unroll
                for (int q = 0; q < NW; ++q) {
                    uint32_t word = pl[q][0];
#pragma unroll
                    for (int m = 1; m < PL; ++m) word |= pl[q][m] << (NBITS * m);
                    w[q] = word;
                }
                if constexpr (NBITS == 3) {
#pragma unroll
                    for (int q = 0; q < NW; ++q)
                        *reinterpret_cast<uint32_t *>(stage + lane * EB + 4 * q) = w[q];
                } else {
                    uint8_t *dst = J.packed + e0 * NBITS / 8;
                    if constexpr (BY == 2)             // 16 one-bit codes
                        *gbl(reinterpret_cast<uint16_t *>(dst)) = (uint16_t)w[0];
                    else if constexpr (NW == 4)
                        *gbl(reinterpret_cast<u32x4 *>(dst)) = u32x4{w[0], w[1], w[2], w[3]};
                    else if constexpr (NW == 2)
                        *gbl(reinterpret_cast<u32x2 *>(dst)) = u32x2{w[0], w[1]};
                    else if constexpr (NW == 1)
                        *gbl(reinterpret_cast<uint32_t *>(dst)) = w[0];
                    else {
#pragma unroll
                        for (int q = 0; q < NW / 4; ++q)
                            gbl(reinterpret_cast<u32x4 *>(dst))[q] =
                                u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
                    }
                }
            };
            // The accepted evaluation ran in binary32 with the same operations (so its D
            // bounds these codes: none is next to a rounding boundary and none clamps)
            // or in binary64; exact codes only if D was near 1/2.
            if (sa.Db < C::kThr - (float)(1.0 / (1 << (24 - NBITS)))) {
                emit([&](uint32_t h) { return fmaf(h2f(h), s, zb); });
            } else {
                emit([&](uint32_t h) {
                    const double u = fma((double)h2f(h), (double)s, (double)zb);
                    return (float)fmin(fmax(rint(u), 0.0), (double)C::QMAX);
                });
            }
            if (bleader) {
                if (J.zero16) gbl(J.zero16)[gidx] = f2h(zb);
                if (J.zero32) gbl(J.zero32)[gidx] = zb;
                // evaluations run = index of the next update when the group stops
                if (J.passes) gbl(J.passes)[gidx] = (uint8_t)meta_t(st_b[j].meta);
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
                for (int64_t w = w0 + sub; w <= w1; w += KB) {
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
        if (J.minmax) {
            if ((int)job0 != mm_job) {
                flush_minmax();
                mm_job = (int)job0;
            }
            if (valid) {
                mm_lo = fminf(mm_lo, zb);
                mm_hi = fmaxf(mm_hi, zb);
            }
        }
        const uint64_t m_done = __ballot(valid && bleader);
        if (valid && bleader) ring_free[(fre_h + fre_n + lanes_below(m_done)) & RM] = j;
        fre_n += (uint32_t)__builtin_popcountll(m_done);
    };

    // A bound on loop steps that the schedule never reaches (every step moves at least one
    // group forward): a defect ends the launch instead of hanging it, and the wave that runs
    // out sets the launch's status flag so that the host can report incomplete outputs.
    // 32-bit (scalar compares; the host's budgets stay far below 2^31 per wave, and the
    // per-tile additions saturate).
    int32_t budget = (int32_t)(a.budget0 < 0x40000000 ? a.budget0 : 0x40000000);
    const int32_t budget_tile = (int32_t)(a.budget_tile < 0x40000000 ? a.budget_tile : 0x40000000);
    bool ran_out = false;

    prefetch();

    // The outer loop takes one prefetched tile in per turn (INIT); the inner loop does all
    // other work. Only the outer loop touches the prefetch registers, so they keep one place.
    bool done = false, epi_first = false;
    while (!done) {
        while (true) {
            // Wave priority: the step choice and SWAP are short chains of LDS round trips
            // that decide what a wave does next; raised, they issue as soon as their data
            // returns, while the arithmetic phases (PASS, EXACT, EPILOGUE, INIT) of the
            // SIMD's other waves fill the gaps. Measured 1-5 % faster than one level.
            __builtin_amdgcn_s_setprio(1);
            if (--budget <= 0) {
                ran_out = true;
                done = true;
                break;
            }
            const bool lead = pleader;
            const bool holder = status == kHoldFin || status == kHoldExq;
            const uint64_t m_hold = __ballot(holder && lead);
            const uint64_t m_empty = __ballot(status == kEmpty && lead);
            const uint32_t n_hold = (uint32_t)__builtin_popcountll(m_hold);
            const uint32_t n_empty = (uint32_t)__builtin_popcountll(m_empty);

            // A tile comes in first when the ready groups cannot fill the lanes about to need
            // one and the free slots take the tile and every holder that needs a free slot
            // (with in-place swaps, those the ready groups and the tile's cannot take): one
            // swap then serves them all.
            // (fre_n >= GB + max(n_hold - partners, 0), written without a saturating
            // subtraction, which has only a vector form)
            const uint32_t partners = C::XCHG ? rdy_n + GB : 0u;
            if (pf_ok && rdy_n < n_empty + n_hold &&
                fre_n + (n_hold < partners ? n_hold : partners) >= GB + n_hold)
                break;   // INIT

            if ((n_hold > 0 && (rdy_n > 0 || fre_n > 0)) || (n_empty > 0 && rdy_n > 0)) {
                // ================= SWAP: groups leave lanes for slots and enter from slots ====
                // Every lane moves through one slot, so the weight registers have a single load
                // site (no copies at joins).
                if constexpr (C::XCHG) {
                    // In place: a holder swaps its group with a ready one through the ready
                    // group's slot (LDS atomic exchanges), so the exchange needs no free slot.
                    // Holders left without a ready group swap into free slots; lanes without a
                    // group swap the remaining ready groups out of theirs.
                    const uint32_t n_xc = n_hold < rdy_n ? n_hold : rdy_n;
                    const uint32_t n_left = n_hold - n_xc;
                    const uint32_t n_out = n_left < fre_n ? n_left : fre_n;
                    const uint32_t n_in = n_empty < rdy_n - n_xc ? n_empty : rdy_n - n_xc;
                    const uint32_t rk_h = group_rank(m_hold, pbase);
                    const uint32_t rk_e = group_rank(m_empty, pbase);
                    const bool xc_l = holder && rk_h < n_xc;
                    const bool out_l = holder && rk_h >= n_xc && rk_h < n_xc + n_out;
                    const bool in_l = status == kEmpty && rk_e < n_in;
                    const bool st = xc_l || out_l, ld = xc_l || in_l;
                    int j = 0;
                    if (xc_l) j = ring_rdy[(rdy_h + rk_h) & RM];
                    if (out_l) j = ring_free[(fre_h + rk_h - n_xc) & RM];
                    if (in_l) j = ring_rdy[(rdy_h + n_xc + rk_e) & RM];
                    if (st || ld) {
                        // Every moving lane exchanges its registers with slot j (LDS atomic swaps):
                        // a lane that only loads writes don't-care values into a slot that becomes
                        // free, a lane that only stores reads don't-care values and becomes empty.
    #pragma unroll
                        for (int c = 0; c < WP / 4; ++c) {
                            uint64_t *p = reinterpret_cast<uint64_t *>(xs + chunk_at<C::CS>(j, part * (WP / 4) + c));
                            const uint64_t lo = xchg_l(p, (uint64_t)xr[4 * c] | (uint64_t)xr[4 * c + 1] << 32);
                            const uint64_t hi = xchg_l(p + 1, (uint64_t)xr[4 * c + 2] | (uint64_t)xr[4 * c + 3] << 32);
                            xr[4 * c] = (uint32_t)lo;
                            xr[4 * c + 1] = (uint32_t)(lo >> 32);
                            xr[4 * c + 2] = (uint32_t)hi;
                            xr[4 * c + 3] = (uint32_t)(hi >> 32);
                        }
                        set_state(xchg_state(j, cur_state()));
                    }
                    // rings: stored groups go to finished / exact-pending; the slots of groups
                    // loaded into empty lanes become free
                    const bool to_fin = st && status == kHoldFin;
                    const uint64_t m_f = __ballot(to_fin && lead);
                    const uint64_t m_x = __ballot(st && !to_fin && lead);
                    const uint64_t m_fr = __ballot(in_l && lead);
                    if (st && lead) {
                        if (to_fin) ring_fin[(fin_h + fin_n + lanes_below(m_f)) & RM] = (uint8_t)j;
                        else ring_exq[(exq_h + exq_n + lanes_below(m_x)) & RM] = (uint8_t)j;
                    }
                    rdy_h = (rdy_h + n_xc + n_in) & RM;
                    rdy_n -= n_xc + n_in;
                    fre_h = (fre_h + n_out) & RM;
                    fre_n -= n_out;
                    if (in_l && lead) ring_free[(fre_h + fre_n + lanes_below(m_fr)) & RM] = (uint8_t)j;
                    fre_n += (uint32_t)__builtin_popcountll(m_fr);
                    fin_n += (uint32_t)__builtin_popcountll(m_f);
                    exq_n += (uint32_t)__builtin_popcountll(m_x);
                    if (ld) status = kActive;
                    else if (out_l) status = kEmpty;
                } else {
                    // Through free slots: holders store their group in a free slot; lanes left
                    // without a group load a ready one. When no slot is free, one holder
                    // exchanges its group with a ready one through the spare slot: the ready
                    // group is copied there, the holder's group takes its slot, and the holder
                    // loads from the spare like any other lane.
                    const uint32_t n_out = n_hold < fre_n ? n_hold : fre_n;
                    const uint32_t n_x = (n_out < n_hold && fre_n == 0 && rdy_n > 0) ? 1u : 0u;
                    const uint32_t rk_h = group_rank(m_hold, pbase);
                    const bool out_l = holder && rk_h < n_out;
                    const bool exch_l = n_x > 0 && holder && rk_h == n_out;
                    const bool no_group = status == kEmpty || out_l;
                    const uint64_t m_ng = __ballot(no_group && lead);
                    const uint32_t n_ng = (uint32_t)__builtin_popcountll(m_ng);
                    const uint32_t n_in = n_ng < rdy_n - n_x ? n_ng : rdy_n - n_x;
                    const uint32_t rk_n = group_rank(m_ng, pbase);
                    const bool in_l = no_group && rk_n < n_in;
                    const bool st = out_l || exch_l, ld = in_l || exch_l;
                    int jo = 0, ji = 0;
                    if (out_l) jo = ring_free[(fre_h + rk_h) & RM];
                    if (exch_l) jo = ring_rdy[rdy_h & RM];
                    if (in_l) ji = ring_rdy[(rdy_h + n_x + rk_n) & RM];
                    if (exch_l) ji = kSpare;
                    if (n_x > 0 && exch_l) {             // the ready group moves to the spare slot
    #pragma unroll
                        for (int c = 0; c < WP / 4; ++c) {
                            const int off = part * (WP / 4) + c;
                            const u32x4 v = *reinterpret_cast<const u32x4 *>(xs + chunk_at<C::CS>(jo, off));
                            *reinterpret_cast<u32x4 *>(xs + chunk_at<C::CS>(kSpare, off)) = v;
                        }
                        const GroupState ns = load_state(jo);
                        if (lead) put_state(kSpare, ns);
                    }
                    if (st) {
    #pragma unroll
                        for (int c = 0; c < WP / 4; ++c)
                            *reinterpret_cast<u32x4 *>(xs + chunk_at<C::CS>(jo, part * (WP / 4) + c)) =
                                u32x4{xr[4 * c], xr[4 * c + 1], xr[4 * c + 2], xr[4 * c + 3]};
                        if (lead) put_state(jo, cur_state());
                    }
                    if (ld) {
    #pragma unroll
                        for (int c = 0; c < WP / 4; ++c) {
                            const u32x4 v = *reinterpret_cast<const u32x4 *>(xs + chunk_at<C::CS>(ji, part * (WP / 4) + c));
                            xr[4 * c] = v.x;
                            xr[4 * c + 1] = v.y;
                            xr[4 * c + 2] = v.z;
                            xr[4 * c + 3] = v.w;
                        }
                        set_state(load_state(ji));
                    }
                    // rings: stored groups go to finished / exact-pending; the slots of loaded
                    // groups become free
                    const bool stored = st;
                    const bool to_fin = stored && status == kHoldFin;
                    const uint64_t m_f = __ballot(to_fin && lead);
                    const uint64_t m_x = __ballot(stored && !to_fin && lead);
                    const uint64_t m_fr = __ballot(in_l && lead);
                    if (stored && lead) {
                        if (to_fin) ring_fin[(fin_h + fin_n + lanes_below(m_f)) & RM] = (uint8_t)jo;
                        else ring_exq[(exq_h + exq_n + lanes_below(m_x)) & RM] = (uint8_t)jo;
                    }
                    rdy_h = (rdy_h + n_x + n_in) & RM;
                    rdy_n -= n_x + n_in;
                    fre_h = (fre_h + n_out) & RM;
                    fre_n -= n_out;
                    if (in_l && lead) ring_free[(fre_h + fre_n + lanes_below(m_fr)) & RM] = (uint8_t)ji;
                    fre_n += (uint32_t)__builtin_popcountll(m_fr);
                    fin_n += (uint32_t)__builtin_popcountll(m_f);
                    exq_n += (uint32_t)__builtin_popcountll(m_x);
                    if (ld) status = kActive;
                    else if (out_l) status = kEmpty;
                }
                continue;
            }

            const uint32_t n_act = (uint32_t)__builtin_popcountll(__ballot(status == kActive && lead));
            const bool can_init = pf_ok && fre_n >= GB;
            const bool idle = n_act == 0;            // no pass possible now

            if (fin_n >= GB || (fin_n > 0 && idle && !can_init && rdy_n == 0 && exq_n == 0)) {
                // When a tile is wanted as well, the epilogue runs in the outer loop after the
                // tile's wait and frees the slots the tile takes.
                if (pf_ok && fin_n >= GB && (rdy_n < n_empty + n_hold || idle)) {
                    epi_first = true;
                    break;
                }
                epilogue();
                continue;
            }

            // A full batch, or whatever is pending once the wave is idle or has no tile left
            // to claim: from then on a waiting group lengthens the wave's tail, so it should
            // not wait for the other lanes' groups to finish first.
            if (exq_n >= GB || (exq_n > 0 && (idle || !pf_ok) && rdy_n == 0)) {
                // ================= EXACT: binary64 decisions and shrink updates ==============
                __builtin_amdgcn_s_setprio(0);
                const int n = exq_n < GB ? (int)exq_n : GB;
                const bool valid = k < n;
                uint8_t j = 0;
                if (valid) j = ring_exq[(exq_h + k) & RM];
                exq_h = (exq_h + n) & RM;
                exq_n -= n;
                uint8_t out = kDone;
                if (valid) {
                    const SlotA sa = st_a[j];
                    const float s = sa.s;
                    const uint32_t m = st_b[j].meta;
                    const uint32_t fl = meta_fl(m);
                    const int c0 = sub * (EB / 8);
                    if (((fl >> 1) & 3) == kDecide) {
                        const float z = sa.z;
                        // S at the accepted zero as well, where only its binary32 value is kept
                        const bool need_sb = !(fl & kFirst) && !(fl & kSbExact);
                        // u of the group's extreme weights (exact in binary64; u rises with x)
                        // at both zeros: inside (-1/2, QMAX + 1/2), no code clamps
                        const uint32_t mm = st_b[j].mnmx;
                        const double sd = s, lo = h2f(mm & 0xffffu), hi = h2f(mm >> 16);
                        const double ul = fmin(fma(lo, sd, (double)z), fma(lo, sd, (double)sa.zb));
                        const double uh = fmax(fma(hi, sd, (double)z), fma(hi, sd, (double)sa.zb));
                        const bool inr = ul > -0.5 && uh < C::QMAX + 0.5;
                        const bool clamp_any = __ballot(!inr) != 0, sb_any = __ballot(need_sb) != 0;
                        double sbx = 0.0;
                        Exact xn;
                        if (!clamp_any) {
                            if (sb_any) xn = eval_exact_t<C, false, true>(xs, j, c0, s, z, sa.zb, sbx);
                            else xn = eval_exact_t<C, false, false>(xs, j, c0, s, z, sa.zb, sbx);
                        } else {
                            if (sb_any) xn = eval_exact_t<C, true, true>(xs, j, c0, s, z, sa.zb, sbx);
                            else xn = eval_exact_t<C, true, false>(xs, j, c0, s, z, sa.zb, sbx);
                        }
                        const double S = addd_k<KB>(xn.S);
                        const float Q = (float)addd_k<KB>(xn.Q);
                        const float D = maxf_k<KB>((float)xn.D);
                        double Sb = st_c[j].Sb;
                        if (need_sb) Sb = addd_k<KB>(sbx);
                        if ((fl & kFirst) || !a.early_stop || S <= Sb) {
                            if (bleader) {
                                st_a[j].zb = z;
                                st_a[j].Db = D;
                                st_c[j].Sb = S;
                                st_b[j].meta = with_fl(m, kSbExact);
                            }
                            out = advance_slot(j, s, z, Q, D, true);
                        } else {
                            out = kDone;
                        }
                    } else {
                        // zero update with the shrink live: z = mean(q - (x - W_e)*s), W_e from
                        // the residual r = x - W_r = (u - q)/s of the accepted iterate.
                        const double sd = s, zd = sa.zb, qm = C::QMAX;
                        const double beta = st_b[j].beta;
                        double acc = 0.0;
#pragma unroll 1
                        for (int i = 0; i < EB; ++i) {
                            const double xv = h2f(xs[chunk_at<C::CS>(j, c0 + (i >> 3)) + (i & 7)]);
                            const double u = fma(xv, sd, zd);
                            const double c = fmin(fmax(rint(u), 0.0), qm);
                            const double we = shrink((u - c) / sd, pm1, beta);
                            acc += c - (xv - we) * sd;
                        }
                        acc = addd_k<KB>(acc);
                        if (bleader) {
                            st_a[j].z = (float)(acc * (1.0 / G));
                            st_b[j].beta = (float)beta * a.kappa;
                            st_b[j].meta = with_fl(m + (1u << 8), fl & kSbExact);
                        }
                        out = kNext;
                    }
                }
                push_batch(valid, out, j);
                continue;
            }

            if (can_init && (rdy_n < n_empty + n_hold || idle)) break;   // INIT, below

            if (!idle) {
                // ================= PASS: every lane with a group evaluates it ================
                {
                    // Codes stay in range when the group's extreme weights do: u of the min (max)
                    // weight at least -1/2 (below 2^NBITS - 1/2). A binary32 bound that is off by
                    // its rounding puts that weight next to a rounding boundary, where the D test
                    // below hands the group to the exact path anyway. Groups that may clamp (about
                    // one evaluation in 10^5) take the exact path. (Selects, not a branch: a join
                    // here made the compiler copy the lane's state.)
                    const float ulo = fmaf(h2f(g_mnmx & 0xffffu), g_s, g_z);
                    const float uhi = fmaf(h2f(g_mnmx >> 16), g_s, g_z);
                    const bool clamp = status == kActive && !(ulo >= -0.5f && uhi < C::QMAX + 0.5f);
                    g_meta = clamp ? with_fl(g_meta, (meta_fl(g_meta) & (kSbExact | kFirst)) | (kDecide << 1))
                                   : g_meta;
                    status = clamp ? (uint32_t)kHoldExq : status;
                }
                __builtin_amdgcn_s_setprio(0);
                {
                    // Every lane runs the evaluation (the wave issues it for its active lanes
                    // anyway); lanes without an active group keep their state through the
                    // selects below. A branch here made the compiler keep the lane's state in
                    // two register sets and copy between them on every loop turn.
                    const bool act = status == kActive;
                    float S, T, D;
                    eval_fast<NBITS, WP>(xr, g_s, g_z, S, T, D);
                    if (KP > 1) {              // butterflies: every lane of the group gets
                        S = addf_k<KP>(S);     // the same sums, so all take the same decision
                        T = addf_k<KP>(T);
                        D = maxf_k<KP>(D);
                    }
                    const float Q = (float)rint(fma((double)G, (double)g_z, g_X) - (double)T);
                    // The decision (the batch path's, written with selects: the branches of
                    // the nested form made the compiler copy the lane's state at every join).
                    // |S - S_exact| bounds: binary32 sums, G half-ulps of u plus the relative
                    // summation error; the margins are far above the binary32 rounding of the
                    // comparison itself.
                    const uint32_t fl = meta_fl(g_meta);
                    const bool first = fl & kFirst;
                    const float Sb = (float)g_Sb;
                    const float m = (float)C::kElemErr + S * 0x1p-18f +
                                    ((fl & kSbExact) ? 0x1p-18f * Sb
                                                       : 4.0f * (float)C::kElemErr + Sb * 0x1p-18f);
                    const bool guard = act && D >= C::kThr;           // to the exact path
                    const bool plain = first || !a.early_stop;        // accepted unseen
                    const bool rise = act && !guard && !plain && S > Sb + m;   // the error rose
                    const bool accept = act && !guard && (plain || S < Sb - m);
                    const bool undecided = act && !guard && !plain && !rise && !accept;
                    // advance of an accepted evaluation (advance_core's steps with zb = z)
                    const int t = (int)meta_t(g_meta);
                    const bool over = t > a.iters;
                    const float dmax = D + (0.5f - C::kThr);
                    const bool dead_all = dmax <= tau_min * g_s;
                    bool live = false;                                // the shrink is live
                    if (accept && !over && !dead_all) {
                        const float tau_t = (float)pow_ool((double)g_beta, tau_exp);
                        live = !(dmax <= tau_t * (g_s * (1.0f - 4e-6f)));
                    }
                    const float zn = (float)(((double)Q - g_X) * (1.0 / G));
                    const bool fixed = !over && !live && zn == g_z && dead_all;
                    const bool fin = accept && (over || fixed);
                    const bool nxt = accept && !over && !live && !fixed;
                    const bool shr = accept && live;
                    const uint32_t acc_meta = with_fl(g_meta, 0);
                    uint32_t meta = g_meta;
                    meta = guard ? with_fl(g_meta, (fl & (kSbExact | kFirst)) | (kDecide << 1)) : meta;
                    meta = undecided ? with_fl(g_meta, (fl & kSbExact) | (kDecide << 1)) : meta;
                    meta = fin ? acc_meta : meta;
                    meta = shr ? with_fl(acc_meta, kShrink << 1) : meta;
                    meta = nxt ? acc_meta + (1u << 8) : meta;
                    g_meta = meta;
                    g_zb = accept ? (fixed ? zn : g_z) : g_zb;
                    g_Sb = accept ? (double)S : g_Sb;
                    g_Db = accept ? D : g_Db;
                    g_beta = nxt ? g_beta * a.kappa : g_beta;
                    g_z = nxt ? zn : g_z;
                    status = (guard || undecided || shr) ? (uint32_t)kHoldExq
                             : (rise || fin)              ? (uint32_t)kHoldFin
                                                          : status;
                }
                continue;
            }

            done = true;                             // nothing left: every ring and lane is empty
            break;
        }
        if (done) break;
        // Loads and stores share one completion counter, retired in order: a wait for the
        // tile issued after an epilogue's stores would wait for those too. So the tile is
        // waited for here, before any store of this turn, and INIT itself waits for nothing.
#pragma unroll
        for (int i = 0; i < EB / 8; ++i) asm volatile("" : "+v"(pf[i]));
        if (epi_first) {
            epi_first = false;
            epilogue();
            if (fre_n < GB) continue;            // finished groups of a later tensor stayed
        }
        // ================= INIT: a prefetched tile becomes ready groups ===============
        __builtin_amdgcn_s_setprio(0);
        budget = budget > 0x7fffffff - budget_tile ? 0x7fffffff : budget + budget_tile;
        const int nv = pf_nv;
        const bool valid = k < nv;
        uint8_t j = 0;
        if (valid) j = ring_free[(fre_h + k) & RM];
        fre_h = (fre_h + nv) & RM;
        fre_n -= nv;
        if (valid) {
            uint32_t xb[WB];
#pragma unroll
            for (int i = 0; i < EB / 8; ++i) {
                const u32x4 v = pf[i];
                *reinterpret_cast<u32x4 *>(xs + chunk_at<C::CS>(j, sub * (EB / 8) + i)) = v;
                xb[4 * i] = v.x;
                xb[4 * i + 1] = v.y;
                xb[4 * i + 2] = v.z;
                xb[4 * i + 3] = v.w;
            }
            float mn, mx;
            group_min_max<WB, KB>(xb, mn, mx);
            const float rng = mx - mn;
            const float s = rng > 0.0f ? C::QMAX / rng : 1.0f;
            const float z0 = 0.0f - mn * s;      // +0 when min is a zero of either sign
            // with every weight of the tile below 1/2 (most tiles), x*s summed as s * sum x
            const float am = fmaxf(-mn, mx);
            double sxs;
            if (__ballot(am >= 0.5f)) sxs = addd_k<KB>(lane_sum_xs<WB>(xb, (double)s));
            else sxs = (double)s * addd_k<KB>(lane_sum_x_tile<WB>(xb, am));
            if (bleader) {
                // The scale is fixed from here on: the tile's scales are stored now, one
                // contiguous run per tile, rather than one by one as groups finish.
                gbl(jobs[pf_job].scale)[pf_g0 + k] = f2h(1.0f / s);
                st_a[j] = SlotA{s, z0, z0, 0.f};
                float beta0 = a.beta0;
                asm volatile("" : "+s"(beta0));     // kept in a scalar register until here
                st_b[j] = SlotB{beta0, (uint32_t)f2h(mn) | ((uint32_t)f2h(mx) << 16),
                                (uint32_t)(pf_g0 + k), (uint32_t)pf_job << 16 | 1u << 8 | kFirst};
                st_c[j] = SlotC{0.0, sxs};
            }
        }
        push_batch(valid, kNext, j);
        prefetch();
    }
    flush_minmax();
    if (ran_out && lane == 0)   // set after the loop: inside it the atomic costs registers
        __hip_atomic_fetch_or(gbl(a.status), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exact (binary64) evaluation of a lane's EB weights held in registers at zero z (the
// lockstep kernel's form of eval_exact_t).
template <class C, int WB>
__device__ __forceinline__ Exact eval_exact_regs(const uint32_t (&xb)[WB], float s, float z)
{
    const double sd = s, zd = z, qm = C::QMAX;
    double s_ = 0.0, q_ = 0.0, d_ = 0.0;
    // two words (four weights) per turn: a register array indexed in a rolled loop costs an
    // indexed move per index, and the binary64 sums are exact in any order
#pragma unroll 1
    for (int w = 0; w < WB; w += 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t v = xb[w + (i >> 1)];
            const uint32_t h = i & 1 ? v >> 16 : v & 0xffffu;
            const double u = fma((double)h2f(h), sd, zd);
            const double c = fmin(fmax(rint(u), 0.0), qm);
            const double e = fabs(u - c);
            s_ += e;
            q_ += c;
            d_ = fmax(d_, e);
        }
    }
    return Exact{s_, q_, d_};
}

// eval_exact_regs at z, and in the same loop the exact error sum at a second zero zb (each
// sum in the same order as eval_exact_regs would take it).
template <class C, int WB>
__device__ __forceinline__ Exact eval_exact2_regs(const uint32_t (&xb)[WB], float s, float z,
                                                  float zb, double &Sb_out)
{
    const double sd = s, zd = z, zbd = zb, qm = C::QMAX;
    double s_ = 0.0, q_ = 0.0, d_ = 0.0, sb_ = 0.0;
#pragma unroll 1
    for (int w = 0; w < WB; w += 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t v = xb[w + (i >> 1)];
            const double x = (double)h2f(i & 1 ? v >> 16 : v & 0xffffu);
            const double u = fma(x, sd, zd);
            const double c = fmin(fmax(rint(u), 0.0), qm);
            const double e = fabs(u - c);
            s_ += e;
            q_ += c;
            d_ = fmax(d_, e);
            const double ub = fma(x, sd, zbd);
            const double cb = fmin(fmax(rint(ub), 0.0), qm);
            sb_ += fabs(ub - cb);
        }
    }
    Sb_out = sb_;
    return Exact{s_, q_, d_};
}

// Lockstep solver for classes too small to keep the persistent waves busy (a single layer,
// say). One wave per tile of GB groups in the batch layout (KB lanes per group, EB weights
// per lane, held in registers): every group of the tile is iterated in place, each loop turn
// taking one step of each unfinished group -- a binary32 evaluation, an exact (binary64)
// decision, or a zero update with a live shrink -- until all are done, then packed and
// stored. No staging slots, rings or swaps: lanes whose group finished early idle, which
// costs less than the persistent scheduler's latency when each wave has only a few tiles.
// Every decision is the persistent kernel's, so the results are identical.
enum : uint8_t { kStepFast = 0, kStepExact = 1, kStepShrink = 2, kStepDone = 3 };

template <int NBITS, int G, int EBL>
__global__ void __launch_bounds__(64) lockstep_kernel(StreamArgs a, const DevJob *__restrict__ jobs)
{
    using C = Cfg<NBITS, G>;
    // EBL weights per lane: the batch layout's EB, or more (fewer lanes per group, more groups
    // per tile) for a class of one tensor, whose tiles need not line up with the plan's
    constexpr int EB = EBL, KB = G / EB, GB = 64 / KB, WB = EB / 2;
    __shared__ __attribute__((aligned(4))) uint8_t stage[NBITS == 3 ? 64 * EB : 4];
    __shared__ __attribute__((aligned(16))) uint32_t xl[64 * WB];   // the wave's weights, lane-major
    __shared__ int lead_of[64];                                      // spread rounds: slot -> leader
    const int lane = threadIdx.x;
    const int k = lane / KB, sub = lane % KB;
    const bool bleader = sub == 0;
    const int64_t tile = blockIdx.x;
    // the tile's job (jobs ordered by tile0; wave-uniform search)
    int lo = 0, hi = a.n_jobs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (jobs[mid].tile0 <= tile) lo = mid;
        else hi = mid - 1;
    }
    const DevJob &J = jobs[(int)uniform((uint32_t)lo)];
    const int64_t g0 = (tile - J.tile0) * GB;
    const int64_t left = J.n_groups - g0;
    const int nv = (int)(left < GB ? left : GB);
    const bool valid = k < nv;
    const int64_t gidx = g0 + (valid ? k : 0);      // lanes past a ragged end re-read group g0
    uint32_t xb[WB];
    {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(J.W + gidx * G + sub * EB);
#pragma unroll
        for (int i = 0; i < EB / 8; ++i) {
            const u32x4 v = gbl(const_cast<u32x4 *>(src))[i];
            xb[4 * i] = v.x;
            xb[4 * i + 1] = v.y;
            xb[4 * i + 2] = v.z;
            xb[4 * i + 3] = v.w;
        }
    }
    // An LDS copy of the weights for the turns that spread groups over the whole wave (the
    // weights never change, so it is written once): group g of the tile, led by lane L = g*KB,
    // holds words L*WB .. L*WB + G/2 - 1 in element order.
#pragma unroll
    for (int i = 0; i < WB / 4; ++i)
        *reinterpret_cast<u32x4 *>(xl + lane * WB + 4 * i) =
            u32x4{xb[4 * i], xb[4 * i + 1], xb[4 * i + 2], xb[4 * i + 3]};
    __syncthreads();
    // Dead zone of the shrink (as in the persistent kernel).
    const double tau_exp = -1.0 / (2.0 - (double)a.p);
    float beta_last = a.beta0;
    for (int i = 1; i < a.iters; ++i) beta_last = beta_last * a.kappa;
    const float tau_min = __builtin_bit_cast(
        float, uniform(__float_as_uint(
                   a.iters > 0 ? (float)pow_ool((double)beta_last, tau_exp) * (1.0f - 4e-6f) : 0.0f)));
    const double pm1 = (double)a.p - 1.0;

    // ---- INIT: min / max on binary16 pairs, s, z0, exact sum x*s ----
    float mn, mx;
    group_min_max<WB, KB>(xb, mn, mx);
    const float rng = mx - mn;
    const float s = rng > 0.0f ? C::QMAX / rng : 1.0f;
    const double sd = s;
    const float am = fmaxf(-mn, mx);                               // as in the persistent INIT
    double X;
    if (__ballot(am >= 0.5f)) X = addd_k<KB>(lane_sum_xs<WB>(xb, sd));
    else X = sd * addd_k<KB>(lane_sum_x_tile<WB>(xb, am));
    if (valid && bleader) gbl(J.scale)[gidx] = f2h(1.0f / s);
    // binary32 range test of the fast path: u of the extreme weights stays in range
    const float umn = mn, umx = mx;

    float z = 0.0f - mn * s, zb = z, Db = 0.0f, beta = a.beta0;
    double Sb = 0.0;
    int t = 1;
    bool first = true, sbexact = false;
    uint8_t step = valid ? kStepFast : kStepDone;
    int64_t budget = a.budget0 + a.budget_tile;
    bool ran_out = false;

    // the decision after an exact evaluation (S, Q, D at z; Sbx the accepted error)
    auto exact_decide = [&](double S, float Q, float D, double Sbx) {
        if (first || !a.early_stop || S <= Sbx) {
            zb = z;
            Db = D;
            Sb = S;
            first = false;
            sbexact = true;
            const Advance ad = advance_core<C>(t, a.iters, s, z, Q, D, true, X, beta, tau_min,
                                               tau_exp);
            if (ad.out == kDone) {
                zb = ad.zn;
                step = kStepDone;
            } else if (ad.out == kNeedShrink) {
                step = kStepShrink;
            } else {
                z = ad.zn;
                beta = beta * a.kappa;
                ++t;
                step = kStepFast;
            }
        } else {
            step = kStepDone;
        }
    };

    // Binary32 evaluation of the groups in the fast step, spread over the whole wave when
    // few of them are left (mf: their leader lanes, nf of them): WPL = 4*R weights per lane,
    // read from the LDS copy four at a time, and LPG = G/WPL lanes per group; the q-th group
    // takes lanes q*LPG .. q*LPG+LPG-1. R and LPG are wave-uniform run-time values, so one
    // code path serves every width. Every lane of such a group receives its S, T and D. The
    // sums add in another order than eval_fast's, in chains no longer than its, so the margins
    // below cover them alike; D is a maximum and Q depends on T only through rne, far from a
    // half, so both come out the same.
    auto spread_eval = [&](uint64_t mf, int nf, int R, int lg, float &S, float &T, float &D) {
        const int LPG = 1 << lg;
        const int slot = lane >> lg, part = lane & (LPG - 1);
        if ((mf >> lane) & 1ull) lead_of[__builtin_popcountll(mf & ((1ull << lane) - 1ull))] = lane;
        __syncthreads();
        const int lead = slot < nf ? lead_of[slot] : 0;   // idle slots evaluate lane 0's group
        const float sv = bperm_f(lead, s), zv = bperm_f(lead, z);
        const uint32_t *src = xl + lead * WB + part * 2 * R;
        float sp = 0.0f, tp = 0.0f, dp = 0.0f;
#pragma unroll 1
        for (int r = 0; r < R; ++r) {
            const u32x2 v = *reinterpret_cast<const u32x2 *>(src + 2 * r);
            const uint32_t xr[2] = {v.x, v.y};
            float sr, tr, dr;
            eval_fast<NBITS, 2>(xr, sv, zv, sr, tr, dr);
            sp += sr;
            tp += tr;
            dp = fmaxf(dp, dr);
        }
        // butterflies within the LPG lanes of a slot (uniform branches)
        if (lg >= 1) { sp += dppf<0xb1>(sp); tp += dppf<0xb1>(tp); dp = fmaxf(dp, dppf<0xb1>(dp)); }
        if (lg >= 2) { sp += dppf<0x4e>(sp); tp += dppf<0x4e>(tp); dp = fmaxf(dp, dppf<0x4e>(dp)); }
        if (lg >= 3) { sp += dppf<0x141>(sp); tp += dppf<0x141>(tp); dp = fmaxf(dp, dppf<0x141>(dp)); }
        if (lg >= 4) { sp += dppf<0x140>(sp); tp += dppf<0x140>(tp); dp = fmaxf(dp, dppf<0x140>(dp)); }
        if (lg >= 5) {
            sp += __shfl_xor(sp, 16);
            tp += __shfl_xor(tp, 16);
            dp = fmaxf(dp, __shfl_xor(dp, 16));
        }
        if (lg >= 6) {
            sp += __shfl_xor(sp, 32);
            tp += __shfl_xor(tp, 32);
            dp = fmaxf(dp, __shfl_xor(dp, 32));
        }
        const int src_lane = __builtin_popcountll(mf & ((1ull << (lane - sub)) - 1ull)) << lg;
        S = bperm_f(src_lane, sp);
        T = bperm_f(src_lane, tp);
        D = bperm_f(src_lane, dp);
    };

    for (;;) {
        // The weights pass an empty asm at the top of every turn, so their binary32 forms are
        // not loop-invariant: the evaluation converts on the fly (v_fma_mix) rather than the
        // compiler holding all EB converted weights across the loop (32 more registers, one
        // wave fewer per SIMD at EB = 32).
#pragma unroll
        for (int i = 0; i < WB; ++i) asm volatile("" : "+v"(xb[i]));
        if (!__ballot(step != kStepDone)) break;
        if (--budget <= 0) {
            ran_out = true;
            break;
        }
        {
            const float ulo = fmaf(umn, s, z), uhi = fmaf(umx, s, z);
            const bool clamp = step == kStepFast && !(ulo >= -0.5f && uhi < C::QMAX + 0.5f);
            step = clamp ? (uint8_t)kStepExact : step;           // may clamp
        }
        // ---- binary32 evaluation; the decision as in the persistent kernel, with selects ----
        // A turn with few groups in the fast step spreads them over the wave (4 to 32
        // weights per lane, fewer than EB); otherwise each group's own lanes evaluate it.
        float S = 0.0f, T = 0.0f, D = 0.0f;
        bool spread = false;
        {
            const uint64_t mf = __ballot(step == kStepFast && bleader);
            const int nf = __builtin_popcountll(mf);
            // the fewest weights per lane (4, 8, 16 or 32, fewer than EB) that fit nf groups
            int R = 0;
            if (nf > 0 && EB > 4 && nf * G <= 64 * 4) R = 1;
            else if (nf > 0 && EB > 8 && nf * G <= 64 * 8) R = 2;
            else if (nf > 0 && EB > 16 && nf * G <= 64 * 16) R = 4;
            else if (nf > 0 && EB > 32 && nf * G <= 64 * 32) R = 8;
            if (R > 0) {
                // lanes per group: G / (4 R), a power of two
                const int lg = __builtin_ctz((unsigned)G) - 2 - __builtin_ctz((unsigned)R);
                spread_eval(mf, nf, R, lg, S, T, D);
                spread = true;
            }
        }
        if (step == kStepFast) {
            if (!spread) {
                eval_fast<NBITS, WB>(xb, s, z, S, T, D);
                if (KB > 1) {
                    S = addf_k<KB>(S);
                    T = addf_k<KB>(T);
                    D = maxf_k<KB>(D);
                }
            }
            const float Q = (float)rint(fma((double)G, (double)z, X) - (double)T);
            const float Sb32 = (float)Sb;
            const float m = (float)C::kElemErr + S * 0x1p-18f +
                            (sbexact ? 0x1p-18f * Sb32 : 4.0f * (float)C::kElemErr + Sb32 * 0x1p-18f);
            const bool guard = D >= C::kThr;
            const bool plain = first || !a.early_stop;
            const bool rise = !guard && !plain && S > Sb32 + m;
            const bool accept = !guard && (plain || S < Sb32 - m);
            const bool undecided = !guard && !plain && !rise && !accept;
            const bool over = t > a.iters;
            const float dmax = D + (0.5f - C::kThr);
            const bool dead_all = dmax <= tau_min * s;
            bool live = false;
            if (accept && !over && !dead_all) {
                const float tau_t = (float)pow_ool((double)beta, tau_exp);
                live = !(dmax <= tau_t * (s * (1.0f - 4e-6f)));
            }
            const float zn = (float)(((double)Q - X) * (1.0 / G));
            const bool fixed = !over && !live && zn == z && dead_all;
            const bool fin = accept && (over || fixed);
            const bool nxt = accept && !over && !live && !fixed;
            zb = accept ? (fixed ? zn : z) : zb;
            Sb = accept ? (double)S : Sb;
            Db = accept ? D : Db;
            first = (accept || undecided) ? false : first;
            sbexact = accept ? false : sbexact;
            beta = nxt ? beta * a.kappa : beta;
            t = nxt ? t + 1 : t;
            z = nxt ? zn : z;
            step = (guard || undecided) ? (uint8_t)kStepExact
                   : (rise || fin)      ? (uint8_t)kStepDone
                   : (accept && live)   ? (uint8_t)kStepShrink
                                        : step;
        }
        // ---- exact decision (binary64), for the groups the fast path could not settle; the
        //      accepted error is re-evaluated exactly (at zb) when the fast path accepted it.
        //      Groups of 16 and 32 weights (one lane each) sum their errors element by
        //      element, in the oracle's order, which fixes the result even where a sum rounds.
        if (G < 64 && __ballot(step == kStepExact)) {
            const bool any_sbx = __ballot(step == kStepExact && !first && !sbexact) != 0;
            if (step == kStepExact) {
                double sbx_l = 0.0;
                const Exact xn = any_sbx ? eval_exact2_regs<C, WB>(xb, s, z, zb, sbx_l)
                                         : eval_exact_regs<C, WB>(xb, s, z);
                double Sbx = Sb;
                if (!first && !sbexact) Sbx = sbx_l;
                exact_decide(xn.S, (float)xn.Q, (float)xn.D, Sbx);
            }
        } else if (G >= 64 && __ballot(step == kStepExact)) {
            // Groups of 64 or more weights already sum in another order than the oracle's
            // in their binary32 turns (over several lanes in the plan's layout), relying on
            // the sums being exact (they are unless a group's range is extreme, the oracle's
            // own precision reading). A turn has few such groups, so
            // their weights are spread over the whole wave first (through LDS; LPG lanes of
            // four weights per group, NPC groups per round): the binary64 loop then takes
            // four weights per lane instead of EB.
            constexpr int LPG = G / 4, NPC = 64 / LPG;
            const bool any_sbx = __ballot(step == kStepExact && !first && !sbexact) != 0;
            const int slot = lane / LPG, part = lane % LPG;
            uint64_t m_left = __ballot(step == kStepExact && bleader);
            while (m_left) {
                // this round: the next NPC waiting groups; slot q holds the q-th (leader lane L)
                uint64_t m_round = 0;
                int lead = 0;
                for (int q = 0; q < NPC && m_left; ++q) {
                    const int L = __builtin_ctzll(m_left);
                    m_left &= m_left - 1;
                    m_round |= 1ull << L;
                    lead = slot == q ? L : lead;
                }
                // the slot's group: s and zeros from its leader, four weights from LDS (group g
                // sits at words g*G/2 = L*WB; slots without a group compute unused values)
                const double sd = bperm_f(lead, s), zd = bperm_f(lead, z), zbd = bperm_f(lead, zb);
                const double qm = C::QMAX;
                const u32x2 v = *reinterpret_cast<const u32x2 *>(xl + lead * WB + 2 * part);
                double se = 0.0, qe = 0.0, de = 0.0, sbe = 0.0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = e < 2 ? v.x : v.y;
                    const double x = (double)h2f(e & 1 ? w >> 16 : w & 0xffffu);
                    const double u = fma(x, sd, zd);
                    const double c = fmin(fmax(rint(u), 0.0), qm);
                    const double d = fabs(u - c);
                    se += d;
                    qe += c;
                    de = fmax(de, d);
                    if (any_sbx) {
                        const double ub = fma(x, sd, zbd);
                        const double cb = fmin(fmax(rint(ub), 0.0), qm);
                        sbe += fabs(ub - cb);
                    }
                }
                se = addd_k<LPG>(se);
                qe = addd_k<LPG>(qe);
                const float dm = maxf_k<LPG>((float)de);
                if (any_sbx) sbe = addd_k<LPG>(sbe);
                // back to the lanes of each group of the round (every lane of a slot holds the
                // sums)
                const int my_lead = lane - sub;
                const bool mine = step == kStepExact && ((m_round >> my_lead) & 1ull);
                const int src = __builtin_popcountll(m_round & ((1ull << my_lead) - 1ull)) * LPG;
                const double S = bperm_d(src, se);
                const float Q = (float)bperm_d(src, qe);
                const float D = bperm_f(src, dm);
                const double Sbe = any_sbx ? bperm_d(src, sbe) : 0.0;
                if (!mine) continue;
                double Sbx = Sb;
                if (!first && !sbexact) Sbx = Sbe;
                exact_decide(S, Q, D, Sbx);
            }
        }
        // ---- zero update with the shrink live: z = mean(q - (x - W_e)*s), W_e from the
        //      residual r = x - W_r = (u - q)/s of the accepted iterate ----
        if (__ballot(step == kStepShrink)) {
            if (step == kStepShrink) {
                const double zd = zb, qm = C::QMAX, bd = beta;
                double acc = 0.0;
#pragma unroll 1
                for (int w = 0; w < WB; w += 2) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t v = xb[w + (i >> 1)];
                        const double xv = h2f(i & 1 ? v >> 16 : v & 0xffffu);
                        const double u = fma(xv, sd, zd);
                        const double c = fmin(fmax(rint(u), 0.0), qm);
                        const double we = shrink((u - c) / sd, pm1, bd);
                        acc += c - (xv - we) * sd;
                    }
                }
                acc = addd_k<KB>(acc);
                z = (float)(acc * (1.0 / G));
                beta = (float)bd * a.kappa;
                ++t;
                first = false;
                step = kStepFast;
            }
        }
    }

    // ---- EPILOGUE: codes of the accepted zero, packed; zero and count stores ----
    const int64_t e0 = gidx * G + sub * EB;
    auto emit = [&](auto val) {
        constexpr int PL = NBITS == 3 ? 1 : 8 / NBITS;   // planes
        constexpr int BY = EB / PL < 4 ? EB / PL : 4;    // bytes per word
        constexpr int PER = BY * PL;                     // codes per word
        constexpr int NW = EB / PER;
        uint32_t pl[NW][PL];
#pragma unroll
        for (int q = 0; q < NW; ++q)
#pragma unroll
            for (int m = 0; m < PL; ++m) pl[q][m] = 0u;
#pragma unroll
        for (int i = 0; i < EB; ++i) {
            const uint32_t h = i & 1 ? xb[i >> 1] >> 16 : xb[i >> 1] & 0xffffu;
            const int q = i / PER, m = i % PL, b = (i % PER) / PL;
            pl[q][m] = __builtin_amdgcn_cvt_pk_u8_f32(val(h), b, pl[q][m]);
        }
        uint32_t w[NW];
#pragma unroll
        for (int q = 0; q < NW; ++q) {
            uint32_t word = pl[q][0];
#pragma unroll
            for (int m = 1; m < PL; ++m) word |= pl[q][m] << (NBITS * m);
            w[q] = word;
        }
        if constexpr (NBITS == 3) {
#pragma unroll
            for (int q = 0; q < NW; ++q) *reinterpret_cast<uint32_t *>(stage + lane * EB + 4 * q) = w[q];
        } else if (valid) {
            uint8_t *dst = J.packed + e0 * NBITS / 8;
            if constexpr (BY == 2)
                *gbl(reinterpret_cast<uint16_t *>(dst)) = (uint16_t)w[0];
            else if constexpr (NW == 4)
                *gbl(reinterpret_cast<u32x4 *>(dst)) = u32x4{w[0], w[1], w[2], w[3]};
            else if constexpr (NW == 2)
                *gbl(reinterpret_cast<u32x2 *>(dst)) = u32x2{w[0], w[1]};
            else if constexpr (NW == 1)
                *gbl(reinterpret_cast<uint32_t *>(dst)) = w[0];
            else {
#pragma unroll
                for (int q = 0; q < NW / 4; ++q)
                    gbl(reinterpret_cast<u32x4 *>(dst))[q] =
                        u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
            }
        }
    };
    // the accepted evaluation's D bounds these codes (as in the persistent kernel's epilogue)
    if (Db < C::kThr - (float)(1.0 / (1 << (24 - NBITS)))) {
        emit([&](uint32_t h) { return fmaf(h2f(h), s, zb); });
    } else {
        emit([&](uint32_t h) {
            // the empty asm keeps the compiler from reusing INIT's binary64 conversions of
            // the weights here, which would keep all of them live through the loop
            asm volatile("" : "+v"(h));
            const double u = fma((double)h2f(h), (double)s, (double)zb);
            return (float)fmin(fmax(rint(u), 0.0), (double)C::QMAX);
        });
    }
    if constexpr (NBITS == 3) {
        // flat 10-code words wholly inside a group are written here; a word shared with a
        // neighbouring group goes to the stash (joined after the solve)
        __syncthreads();
        if (valid) {
            const int64_t c0 = gidx * G, c1 = c0 + G, ncode = J.n_groups * G;
            const int64_t w0 = c0 / 10, w1 = (c1 - 1) / 10;
            auto out = gbl(reinterpret_cast<uint32_t *>(J.packed));
            for (int64_t w = w0 + sub; w <= w1; w += KB) {
                uint32_t word = 0;
#pragma unroll
                for (int c = 0; c < 10; ++c) {
                    const int64_t ci = w * 10 + c;
                    if (ci >= c0 && ci < c1) word |= (uint32_t)stage[k * G + (int)(ci - c0)] << (3 * c);
                }
                const bool head = w * 10 < c0;
                const bool tail = w * 10 + 10 > c1 && c1 < ncode;
                uint32_t *st2 = reinterpret_cast<uint32_t *>(J.stash + gidx);
                if (head) gbl(st2)[1] = word;
                else if (tail) gbl(st2)[0] = word;
                else out[w] = word;
            }
        }
    }
    if (valid && bleader) {
        if (J.zero16) gbl(J.zero16)[gidx] = f2h(zb);
        if (J.zero32) gbl(J.zero32)[gidx] = zb;
        if (J.passes) gbl(J.passes)[gidx] = (uint8_t)t;
    }
    if (J.minmax) {                          // the tensor's (min, max) of the binary32 zeros
        const float lo_z = minf_k<64>(valid ? zb : INFINITY);
        const float hi_z = maxf_k<64>(valid ? zb : -INFINITY);
        if (lane == 0) {
            uint32_t *mm = J.minmax + kMinmaxStride * (blockIdx.x % kMinmaxSlots);
            atomic_min_g(mm, fkey(lo_z));
            atomic_max_g(mm + 1, fkey(hi_z));
        }
    }
    if (ran_out && lane == 0)
        __hip_atomic_fetch_or(gbl(a.status), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NBITS, int G, int EBL>
hipError_t launch_lockstep_eb(StreamArgs a, hipStream_t stream)
{
    constexpr int GB = 64 / (G / EBL);
    const int64_t fixed = step_budget();
    // every loop turn advances at least one group by one step; a group takes at most
    // 2*(iters + 1) evaluations and updates plus its exact decisions
    a.budget0 = fixed > 0 ? fixed : 8 * (int64_t)(a.iters + 4) * GB;
    a.budget_tile = 0;
    hipLaunchKernelGGL((lockstep_kernel<NBITS, G, EBL>), dim3((unsigned)a.n_tiles), dim3(64), 0,
                       stream, a, a.jobs);
    return hipGetLastError();
}

template <int NBITS, int G>
hipError_t launch_lockstep(StreamArgs a, hipStream_t stream)
{
    using C = Cfg<NBITS, G>;
    // A class of one tensor at g64 runs one lane per group (GB2 = 64 groups per tile, twice
    // the plan's GB): each turn's decision then serves twice the groups, and the registers
    // still allow four waves per SIMD (at g128 and g256 they would not). Its last tile still
    // starts inside the tensor, since the plan's last tile holds a group.
    constexpr int EB2 = G == 64 ? 64 : C::EB, GB2 = 64 / (G / EB2);
    if (EB2 != C::EB && a.n_jobs == 1) {
        a.n_tiles = (a.n_tiles * C::GB + GB2 - 1) / GB2;
        return launch_lockstep_eb<NBITS, G, EB2>(a, stream);
    }
    return launch_lockstep_eb<NBITS, G, C::EB>(a, stream);
}

template <int NBITS, int G, int EPL>
hipError_t launch_layout(StreamArgs a, int cus, hipStream_t stream)
{
    using C = Cfg<NBITS, G, EPL>;
    const int64_t fixed = step_budget();
    a.budget0 = fixed > 0 ? fixed : 1024;
    a.budget_tile = fixed > 0 ? 0 : 8 * (int64_t)(a.iters + 4) * C::GB;
    // Persistent grid: as many single-wave workgroups as the LDS pool lets the CUs hold; tiles
    // are claimed in chunks small enough to balance the waves (about 16 claims per wave).
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stream_kernel<NBITS, G, EPL>, 64, 0) !=
            hipSuccess || per_cu <= 0)
        per_cu = 4;
    const int64_t waves = (int64_t)cus * per_cu;
    int64_t chunk = a.n_tiles / (waves * 16);
    chunk = chunk < 1 ? 1 : (chunk > 32 ? 32 : chunk);
    a.chunk = (uint32_t)chunk;
    const int64_t claims = (a.n_tiles + chunk - 1) / chunk;
    const int64_t grid = waves < claims ? waves : claims;
    hipLaunchKernelGGL((stream_kernel<NBITS, G, EPL>), dim3((unsigned)grid), dim3(64), 0, stream,
                       a, a.jobs);
    return hipGetLastError();
}

template <int NBITS, int G>
hipError_t launch_one(const StreamArgs &a, hipStream_t stream)
{
    if (a.n_tiles == 0) return hipSuccess;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            cus = v;
    }
    // Lockstep when the class's groups would give each lane of the persistent grid (up to 12
    // waves of 64 lanes per compute unit) fewer than about four; else the persistent solver.
    const int64_t groups = a.n_tiles * Cfg<NBITS, G>::GB;
    const int mode = solver_layout();
    if (mode == 3 || (mode == 0 && groups < 4 * (int64_t)cus * 12 * 64))
        return launch_lockstep<NBITS, G>(a, stream);
    if constexpr (narrow_ep<G>() != wide_ep<G>())
        if (mode == 2) return launch_layout<NBITS, G, narrow_ep<G>()>(a, cus, stream);
    return launch_layout<NBITS, G, wide_ep<G>()>(a, cus, stream);
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
            for (int p = 0; p < kMinmaxSlots; ++p) {
                j.minmax[kMinmaxStride * p] = 0xffffffffu;
                j.minmax[kMinmaxStride * p + 1] = 0u;
            }
        }
    }
    if (f.offset == 0)
        for (int c = i; c < f.n_counters; c += blockDim.x) f.counters[c] = 0u;
}

std::atomic<int64_t> g_step_budget{0};
std::atomic<int> g_layout{0};

}  // namespace

void set_solver_debug(int64_t steps, int layout)
{
    g_step_budget.store(steps > 0 ? steps : 0);
    g_layout.store(layout >= 1 && layout <= 3 ? layout : 0);
}
int64_t step_budget() { return g_step_budget.load(); }
int solver_layout() { return g_layout.load(); }

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
