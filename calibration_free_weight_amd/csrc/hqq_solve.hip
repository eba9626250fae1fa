// hqq_solve.hip -- the HQQ group solver for gfx950.
//
// Method [techreport.ngo, "Half-Quadratic Quantization of Large Machine Learning Models",
// section "Outlier-aware optimization without gradients"; parameters from its section
// "Benchmark results / Llama-2"]: per group of G consecutive weights, fix the min-max scale
// s and optimise the zero-point z by half-quadratic splitting of an lp (p < 1) loss --
// a generalized soft-threshold of the residual (sub-problem 1) alternating with a
// closed-form average for z (sub-problem 2), beta growing by kappa per iteration, early
// stop when the reconstruction error rises.
//
// Arithmetic contract (identical to the library's documented semantics): s, z and beta are
// binary32; each per-element quantity -- u = x*s + z, the code q = clamp(rne(u)), the
// residual u - q, and the group sums of |u - q|, q and x*s -- is formed exactly in binary64
// (x is binary16, so x*s has at most 35 significant bits and x*s + z fits in binary64 for
// any group whose range is not extreme). Exact sums do not depend on summation order, so the
// parallel reductions below give the same values as a sequential loop, and ties in the
// early-stop test are real ties. Each zero update rounds its exact value once to binary32.
//
// Layout: a wave owns 64 lanes x 16 consecutive weights = 1024 weights; K = G/16 lanes hold
// one group (lanes l..l+K-1 hold its elements in order), so a wave holds 64/K groups and
// its loads and packed stores are contiguous. Group reductions are butterflies over the K
// lanes. A block is 4 waves (5 for 3-bit codes, so that a block's 5120 codes fill whole
// 10-code words).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "hqq_internal.h"

namespace hqq {
namespace {

constexpr int kElems = 16;          // weights per lane
constexpr int kTauTab = kMaxIters;  // shrink thresholds per iteration

template <int NBITS> struct Shape {
    static constexpr int waves = NBITS == 3 ? 5 : 4;
    static constexpr int threads = waves * 64;
};

template <int K> __device__ __forceinline__ double sum_k(double v)
{
#pragma unroll
    for (int o = 1; o < K; o <<= 1) v += __shfl_xor(v, o);
    return v;
}
template <int K> __device__ __forceinline__ float min_k(float v)
{
#pragma unroll
    for (int o = 1; o < K; o <<= 1) v = fminf(v, __shfl_xor(v, o));
    return v;
}
template <int K> __device__ __forceinline__ float max_k(float v)
{
#pragma unroll
    for (int o = 1; o < K; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
template <int K> __device__ __forceinline__ double max_kd(double v)
{
#pragma unroll
    for (int o = 1; o < K; o <<= 1) v = fmax(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

// Generalized soft-threshold (sub-problem 1): sign(r) * max(|r| - |r|^(p-1)/beta, 0), 0 at r = 0.
__device__ __forceinline__ double shrink(double r, double pm1, double beta)
{
    if (r == 0.0) return 0.0;
    double a = fabs(r);
    double m = fmax(a - pow(a, pm1) / beta, 0.0);
    return r > 0.0 ? m : -m;
}

template <int NBITS, int G>
__global__ void __launch_bounds__(Shape<NBITS>::threads) solve_kernel(SolveArgs a)
{
    constexpr int K = G / kElems;           // lanes per group
    constexpr int GPW = 64 / K;             // groups per wave
    constexpr int WAVES = Shape<NBITS>::waves;
    constexpr int GPB = GPW * WAVES;        // groups per block
    constexpr double QMAX = (double)((1 << NBITS) - 1);

    __shared__ double tau_tab[kTauTab];
    __shared__ uint8_t code_lds[NBITS == 3 ? WAVES * 64 * kElems : 1];
    __shared__ float2 red_lds[WAVES];

    // Shrink thresholds: at iteration t the shrink uses beta_{t-1} = beta0 * kappa^(t-1)
    // (binary32 products in order), and W_e = 0 exactly when |r| <= beta^(-1/(2-p)).
    for (int t = threadIdx.x; t < a.iters; t += blockDim.x) {
        float b = a.beta0;
        for (int i = 0; i < t; ++i) b = b * a.kappa;
        tau_tab[t] = pow((double)b, -1.0 / (2.0 - (double)a.p));
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane % K;
    const int64_t group = ((int64_t)blockIdx.x * WAVES + wave) * GPW + lane / K;
    const bool valid = group < a.n_groups;

    double x[kElems];
    if (valid) {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.W + group * G + sub * kElems);
        uint4 v0 = src[0], v1 = src[1];
        uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[2 * i] = (double)h2f((uint16_t)(w[i] & 0xffffu));
            x[2 * i + 1] = (double)h2f((uint16_t)(w[i] >> 16));
        }
    } else {
#pragma unroll
        for (int j = 0; j < kElems; ++j) x[j] = 0.0;
    }

    // Min-max initialisation (binary32 operations).
    float mn = (float)x[0], mx = (float)x[0];
#pragma unroll
    for (int j = 1; j < kElems; ++j) {
        mn = fminf(mn, (float)x[j]);
        mx = fmaxf(mx, (float)x[j]);
    }
    mn = min_k<K>(mn);
    mx = max_k<K>(mx);
    const float rng = mx - mn;
    const float s = rng > 0.0f ? (float)QMAX / rng : 1.0f;
    const double sd = (double)s;
    const float z0 = -(mn * s);

    // sum_j x_j * s, exact.
    double sxs = 0.0;
#pragma unroll
    for (int j = 0; j < kElems; ++j) sxs = fma(x[j], sd, sxs);
    sxs = sum_k<K>(sxs);

    // One evaluation at zero z: S = sum |u - q|, Q = sum q, D = max |u - q|.
    auto evaluate = [&](float z, double &S, double &Q, double &D) {
        const double zd = (double)z;
        double s0 = 0.0, s1 = 0.0, q0 = 0.0, q1 = 0.0, d0 = 0.0;
#pragma unroll
        for (int j = 0; j < kElems; j += 2) {
            double u0 = fma(x[j], sd, zd), u1 = fma(x[j + 1], sd, zd);
            double c0 = fmin(fmax(rint(u0), 0.0), QMAX);
            double c1 = fmin(fmax(rint(u1), 0.0), QMAX);
            double e0 = fabs(u0 - c0), e1 = fabs(u1 - c1);
            s0 += e0;
            s1 += e1;
            q0 += c0;
            q1 += c1;
            d0 = fmax(d0, fmax(e0, e1));
        }
        S = sum_k<K>(s0 + s1);
        Q = sum_k<K>(q0 + q1);
        D = max_kd<K>(d0);
    };

    double S_best, Q_best, D_best;
    evaluate(z0, S_best, Q_best, D_best);
    float zb = z0;
    float beta = a.beta0;
    int np = 1;
    bool active = valid && a.iters > 0;
    const double pm1 = (double)a.p - 1.0;
    const double tau_last = a.iters > 0 ? tau_tab[a.iters - 1] : 0.0;

    for (int t = 1; t <= a.iters; ++t) {
        if (!__any(active)) break;
        if (active) {
            // Sub-problem 1 is the zero map when every residual |r| = |u - q|/s sits in the
            // shrink's dead zone; then sub-problem 2 reduces to (sum q - sum x*s)/G.
            const double rmax = D_best / sd;
            const bool dead = rmax <= tau_tab[t - 1] * (1.0 - 1e-6);
            float zn;
            if (dead) {
                zn = (float)((Q_best - sxs) * (1.0 / G));
            } else {
                const double zd = (double)zb;
                double acc = 0.0;
#pragma unroll
                for (int j = 0; j < kElems; ++j) {
                    double u = fma(x[j], sd, zd);
                    double c = fmin(fmax(rint(u), 0.0), QMAX);
                    double we = shrink((u - c) / sd, pm1, (double)beta);
                    acc += c - (x[j] - we) * sd;
                }
                zn = (float)(sum_k<K>(acc) * (1.0 / G));
            }
            beta = beta * a.kappa;
            // Exact fixed point: the same zero again, and the shrink stays dead for every
            // remaining beta, so every later iteration would repeat this one. (zn may be
            // +0 where zb is -0; the iteration accepts zn, so keep it.)
            if (dead && zn == zb && rmax <= tau_last * (1.0 - 1e-6)) {
                zb = zn;
                active = false;
            } else {
                double S, Q, D;
                evaluate(zn, S, Q, D);
                ++np;
                if (a.early_stop && S > S_best) {
                    active = false;
                } else {
                    zb = zn;
                    S_best = S;
                    Q_best = Q;
                    D_best = D;
                }
            }
        }
    }

    // Epilogue: codes of the accepted zero, packed; scale, zero and passes per group.
    uint32_t q[kElems];
    {
        const double zd = (double)zb;
#pragma unroll
        for (int j = 0; j < kElems; ++j)
            q[j] = (uint32_t)fmin(fmax(rint(fma(x[j], sd, zd)), 0.0), QMAX);
    }
    if (valid) {
        const int64_t e0 = group * G + sub * kElems;   // first element of this lane
        if constexpr (NBITS == 8) {
            uint4 o;
            o.x = q[0] | q[1] << 8 | q[2] << 16 | q[3] << 24;
            o.y = q[4] | q[5] << 8 | q[6] << 16 | q[7] << 24;
            o.z = q[8] | q[9] << 8 | q[10] << 16 | q[11] << 24;
            o.w = q[12] | q[13] << 8 | q[14] << 16 | q[15] << 24;
            *reinterpret_cast<uint4 *>(a.packed + e0) = o;
        } else if constexpr (NBITS == 4) {
            uint2 o = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) o.x |= q[j] << (4 * j);
#pragma unroll
            for (int j = 0; j < 8; ++j) o.y |= q[8 + j] << (4 * j);
            *reinterpret_cast<uint2 *>(a.packed + e0 / 2) = o;
        } else if constexpr (NBITS == 2) {
            uint32_t o = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) o |= q[j] << (2 * j);
            *reinterpret_cast<uint32_t *>(a.packed + e0 / 4) = o;
        } else if constexpr (NBITS == 1) {
            uint32_t o = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) o |= q[j] << j;
            *reinterpret_cast<uint16_t *>(a.packed + e0 / 8) = (uint16_t)o;
        }
        if (sub == 0) {
            a.scale[group] = f2h(1.0f / s);
            if (a.zero16) a.zero16[group] = f2h(zb);
            if (a.zero32) a.zero32[group] = zb;
            if (a.passes) a.passes[group] = (uint8_t)np;
        }
    }
    if constexpr (NBITS == 3) {
        // 5 waves x 1024 codes = 512 whole words per full block: stage the codes in LDS so
        // that each 10-code word has exactly one writer.
#pragma unroll
        for (int j = 0; j < kElems; ++j) code_lds[threadIdx.x * kElems + j] = (uint8_t)q[j];
        __syncthreads();
        const int64_t g0 = (int64_t)blockIdx.x * GPB;
        const int64_t ng = a.n_groups - g0 < GPB ? a.n_groups - g0 : GPB;
        const int n = (int)(ng * G);
        const int nw = (n + 9) / 10;
        uint32_t *out = reinterpret_cast<uint32_t *>(a.packed) + g0 * G / 10;
        for (int w = threadIdx.x; w < nw; w += blockDim.x) {
            uint32_t word = 0;
#pragma unroll
            for (int k = 0; k < 10; ++k) {
                int c = w * 10 + k;
                if (c < n) word |= (uint32_t)code_lds[c] << (3 * k);
            }
            out[w] = word;
        }
    }
    if (a.partials) {
        // Block (min, max) of the binary32 zeros, for the per-tensor 8-bit requantization.
        float lo = valid ? zb : INFINITY, hi = valid ? zb : -INFINITY;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            lo = fminf(lo, __shfl_xor(lo, o));
            hi = fmaxf(hi, __shfl_xor(hi, o));
        }
        if (lane == 0) red_lds[wave] = make_float2(lo, hi);
        __syncthreads();
        if (threadIdx.x == 0) {
            float2 r = red_lds[0];
            for (int w = 1; w < WAVES; ++w) {
                r.x = fminf(r.x, red_lds[w].x);
                r.y = fmaxf(r.y, red_lds[w].y);
            }
            a.partials[blockIdx.x] = r;
        }
    }
}

template <int NBITS, int G>
hipError_t launch_one(const SolveArgs &a, hipStream_t stream)
{
    const int64_t blocks = solve_blocks(a.n_groups, G, NBITS);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((solve_kernel<NBITS, G>), dim3((unsigned)blocks),
                       dim3(Shape<NBITS>::threads), 0, stream, a);
    return hipGetLastError();
}

template <int NBITS>
hipError_t launch_bits(const SolveArgs &a, int g, hipStream_t stream)
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

}  // namespace

int64_t solve_blocks(int64_t n_groups, int g, int nbits)
{
    const int64_t gpb = (int64_t)(64 / (g / kElems)) * (nbits == 3 ? 5 : 4);
    return (n_groups + gpb - 1) / gpb;
}

hipError_t launch_solve(const SolveArgs &a, int nbits, int g, hipStream_t stream)
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
