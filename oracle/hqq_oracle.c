/*
 * hqq_oracle.c -- plain, slow, single-threaded CPU oracle of the HQQ solver.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg load this file's library. The GPU library neither links
 * nor includes it, and the two share no code, header, table or helper.
 *
 * Sources (web pages, cited by title and section):
 *   [TR] techreport.ngo, "Half-Quadratic Quantization of Large Machine Learning Models":
 *        section "Outlier-aware optimization without gradients" (weight-only lp objective
 *        with p < 1, fixed scale, zero-point optimised by half-quadratic splitting with an
 *        auxiliary variable W_e; sub-problem 1 = generalized soft-thresholding, sub-problem 2
 *        = an average over the group axis; about 20 iterations);
 *        section "Benchmark results", sub-section "Llama-2" (p = 0.7, beta = 1,
 *        kappa = 1.01, 20 iterations with early stopping; zero-point quantized to 8 bit with
 *        no further grouping or optimisation).
 *   [SK] "HQQ - Half-Quadratic Quantization" usage guide (skill4agent / labsco.ai copies),
 *        section "Core concepts / Quantization configuration" (nbits, group_size, axis) and
 *        section "HQQLinear layer" (outputs W_q, scale, zero; dequantize()).
 *
 * Where the pages leave a step open, the reading taken is stated at that step.
 *
 * Arithmetic: the solver state (scale, zero, beta) is IEEE-754 binary32 and every
 * per-element quantity is evaluated exactly in binary64 (see "Precision reading" below).
 * One rounding per written operation (the build uses -O2 -ffp-contract=off, no fast-math);
 * fma / fmaf only where a step says so; every sum is taken sequentially in index order.
 * Inputs must be finite (asserted).
 *
 * Parity pins for every function here live in the test suite. The regime with no closed
 * form (a live shrink, W_e != 0) is pinned trace for trace against an independent exact
 * re-statement of the iteration (exact rationals, |r|^(p-1) in 60-digit decimal arithmetic).
 */
#include <assert.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* IEEE-754 binary16 <-> binary32, written out from the format's definition.             */
/* ------------------------------------------------------------------------------------ */

/* binary16 -> binary32. Exact for every finite value (binary32 holds all of them). */
float hqo_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0x1f) {
        v = mant ? NAN : INFINITY;
    } else if (expo == 0) {
        v = ldexp((double)mant, -24);               /* subnormal: mant * 2^-24 */
    } else {
        v = ldexp((double)(1024 + mant), expo - 25); /* (1 + mant/1024) * 2^(expo-15) */
    }
    return (float)(sign ? -v : v);
}

/* binary32 -> binary16, round to nearest, ties to even. */
uint16_t hqo_float_to_half(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1): the leading bit has weight 2^(e-1) */
    int lead = e - 1;
    if (lead < -14) lead = -14;                     /* below the normal range: subnormal step */
    double quantum = ldexp(1.0, lead - 10);         /* binary16 spacing in this binade */
    double r = nearbyint(a / quantum);              /* exact division by 2^k; RNE rounding */
    double v = r * quantum;
    if (v >= 65536.0) return (uint16_t)(sign | 0x7c00); /* beyond 65504 after rounding: inf */
    /* Encode v, which is now exactly representable. */
    if (v < ldexp(1.0, -14)) {                      /* subnormal (or the smallest normal) */
        return (uint16_t)(sign | (uint16_t)nearbyint(ldexp(v, 24)));
    }
    frexp(v, &e);
    int expo = e - 1 + 15;
    uint16_t mant = (uint16_t)nearbyint(ldexp(v, 10 - (e - 1)) - 1024.0);
    return (uint16_t)(sign | (uint16_t)(expo << 10) | mant);
}

/* ------------------------------------------------------------------------------------ */
/* Solver steps                                                                          */
/*                                                                                      */
/* Precision reading. The pages run the solver "in half precision" on their GPU, i.e.   */
/* binary16 weights in and out. Here the solver's state -- the scale s, the zero z and  */
/* beta -- is binary32, and each per-element quantity is evaluated exactly:             */
/*   x*s + z for a binary16 x and binary32 s, z has at most ~50 significant bits, so a  */
/*   binary64 fused multiply-add returns it exactly; so are q - x*s, the residual        */
/*   x*s + z - q and their sums over a group (at most ~53 bits) for any weights whose    */
/*   group range is not extreme.                                                         */
/* Why: the early-stop test compares two reconstruction errors, and the error is        */
/* piecewise linear in z with flat pieces, so exact ties are common (0.5-4 % of stop    */
/* decisions on the synthetic weights); any rounded evaluation would settle them by     */
/* rounding noise. Evaluated exactly, a tie is a tie and is not a rise.                  */
/* Each update of the zero rounds the exact value once to binary32.                      */
/* ------------------------------------------------------------------------------------ */

/* Sub-problem 1 [TR, "Outlier-aware optimization without gradients"]: the proximal step of
 * the lp loss, which the page names the generalized soft-thresholding operator:
 *     W_e = sign(r) * max(|r| - |r|^(p-1) / beta, 0).
 * Reading: at r = 0 the power |r|^(p-1) is infinite for p < 1; the operator's limit there is
 * 0, which is what this returns. Evaluated in binary64. */
double hqo_shrink(double r, float p, float beta)
{
    if (r == 0.0) return 0.0;
    double a = fabs(r);
    double t = a - pow(a, (double)p - 1.0) / (double)beta;
    double m = fmax(t, 0.0);
    return r > 0.0 ? m : -m;
}

/* Sub-problem 2 [TR, same section]: with the scale s held fixed, the zero-point that best
 * fits the shrunk target is an average over the group:
 *     z = mean_j ( q_j - (x_j - W_e,j) * s ),
 * the minimiser of sum_j ((q_j - z)/s - (x_j - W_e,j))^2 over z. Summed in binary64 (exact
 * when every W_e,j is 0) and rounded once to binary32. */
float hqo_zero_update(const double *x, const double *q, const double *we, float s, int g)
{
    double acc = 0.0;
    for (int j = 0; j < g; ++j) {
        double target = x[j] - we[j];
        double term = q[j] - target * (double)s;
        acc = acc + term;
    }
    return (float)(acc / (double)g);
}

/* One evaluation of the quantizer at zero-point z (the quantize / reconstruct half of an
 * iteration): u = x*s + z, q = clamp(round-half-even(u), 0, qmax), and the reconstruction
 * W_r = (q - z)/s. Its error term |x_j - W_r,j| equals |x_j*s + z - q_j| / s; the numerator
 * is exact in binary64, so the function returns the exact sum
 *     S(z) = sum_j |x_j*s + z - q_j|,
 * and the page's mean error is S / (g*s). Within a group s is fixed, so comparing S compares
 * the errors. The residual r_j = x_j - W_r,j (needed by the shrink) is returned as
 * (x_j*s + z - q_j)/s, one binary64 rounding. */
double hqo_eval(const double *x, int g, float s, float z, int qmax, double *q, double *r)
{
    double S = 0.0;
    for (int j = 0; j < g; ++j) {
        double u = fma(x[j], (double)s, (double)z);
        double c = nearbyint(u);                    /* default mode: ties to even */
        c = fmin(fmax(c, 0.0), (double)qmax);
        if (c == 0.0) c = 0.0;                      /* a code is never -0 */
        q[j] = c;
        double d = u - c;
        r[j] = d / (double)s;
        S = S + fabs(d);
    }
    return S;
}

/* Min-max affine initialisation of one group. Reading (the pages do not spell out the
 * start point): scale s = qmax / (max - min) and zero z = 0 - min * s, binary32 operations,
 * so iteration 0 is plain round-to-nearest; a constant group (max == min) takes s = 1,
 * z = -min. The zero is not rounded to an integer or clamped: it is the continuous variable
 * the solver optimises [TR]. */
void hqo_init(const double *x, int g, int qmax, float *s_out, float *z_out)
{
    float mn = (float)x[0], mx = (float)x[0];
    for (int j = 1; j < g; ++j) {
        mn = fminf(mn, (float)x[j]);
        mx = fmaxf(mx, (float)x[j]);
    }
    float rng = mx - mn;
    float s = rng > 0.0f ? (float)qmax / rng : 1.0f;
    *s_out = s;
    *z_out = 0.0f - mn * s;                         /* +0 (not -0) when min is a zero */
}

enum { HQO_MAX_G = 4096 };

/* Full solver for one group of g weights (binary16 values held exactly as double).
 *
 * Steps, in the order the pages give them [TR "Outlier-aware optimization without
 * gradients"; parameters from TR "Benchmark results / Llama-2"]:
 *   init (min-max), evaluate at z0 -> accepted iterate 0 (plain RTN when iters == 0);
 *   for t = 1..iters:
 *     r = x - W_r of the accepted iterate; W_e = shrink(r; p, beta)   (sub-problem 1)
 *     z_new = mean(q - (x - W_e) * s)                                   (sub-problem 2)
 *     beta = beta * kappa                                               (binary32)
 *     evaluate at z_new
 *     early stop: if the error rose (strictly), stop and keep the previous iterate;
 *     otherwise accept it.
 * Readings: the stop test is per group, on the mean absolute reconstruction error; a tie
 * is not a rise; the codes returned are those of the accepted (best) iterate. Without
 * early stopping every iterate is accepted and the last one is returned.
 *
 * Outputs: codes[g], *s_out (quantizer multiplier s), *z_out (accepted zero), *passes
 * (number of evaluations, 1..iters+1), *last_change (last t at which the accepted zero
 * changed, 0 if never), *shrink_active (1 if any W_e was non-zero), *stopped (1 if the
 * loop ended on a rise of the error) and, when trace_S is not
 * NULL, S of every evaluation in trace_S[0..passes-1] with trace_acc[k] = 1 when evaluation
 * k was accepted. Returns the accepted mean error S / (g*s). */
double hqo_solve_group(const double *x, int g, int nbits, float p, float beta0, float kappa,
                       int iters, int early_stop, uint8_t *codes, float *s_out, float *z_out,
                       int *passes, int *last_change, int *shrink_active, int *stopped,
                       double *trace_S, uint8_t *trace_acc)
{
    assert(g >= 1 && g <= HQO_MAX_G);
    for (int j = 0; j < g; ++j) assert(isfinite(x[j]));
    const int qmax = (1 << nbits) - 1;
    double q[HQO_MAX_G], r[HQO_MAX_G], qn[HQO_MAX_G], rn[HQO_MAX_G], we[HQO_MAX_G];
    float s, z;
    hqo_init(x, g, qmax, &s, &z);
    double S_best = hqo_eval(x, g, s, z, qmax, q, r);
    int np = 1, lc = 0, act = 0, rose = 0;
    if (trace_S) { trace_S[0] = S_best; trace_acc[0] = 1; }
    float beta = beta0;
    for (int t = 1; t <= iters; ++t) {
        for (int j = 0; j < g; ++j) {
            we[j] = hqo_shrink(r[j], p, beta);
            if (we[j] != 0.0) act = 1;
        }
        float z_new = hqo_zero_update(x, q, we, s, g);
        beta = beta * kappa;
        double S_new = hqo_eval(x, g, s, z_new, qmax, qn, rn);
        if (trace_S) { trace_S[np] = S_new; trace_acc[np] = 0; }
        np += 1;
        if (early_stop && S_new > S_best) {
            rose = 1;
            break;
        }
        if (trace_S) trace_acc[np - 1] = 1;
        if (z_new != z) lc = t;
        z = z_new;
        S_best = S_new;
        memcpy(q, qn, sizeof(double) * (size_t)g);
        memcpy(r, rn, sizeof(double) * (size_t)g);
    }
    for (int j = 0; j < g; ++j) codes[j] = (uint8_t)q[j];
    *s_out = s;
    *z_out = z;
    if (passes) *passes = np;
    if (last_change) *last_change = lc;
    if (shrink_active) *shrink_active = act;
    if (stopped) *stopped = rose;
    return S_best / ((double)g * (double)s);
}

/* Solve n_groups consecutive groups of a flat binary16 array (groups along axis 1 of a
 * row-major [rows, cols] tensor with cols % g == 0 are exactly this: consecutive runs of g
 * elements [SK "Core concepts / Quantization configuration"]).
 *
 * Per group it writes: codes (g bytes), scale = binary16(1/s) -- the stored scale multiplies
 * (q - zero) to reconstruct, so dequantisation is (q - zero) * scale -- and the accepted
 * zero as float (zero_f32). Instrumentation arrays may be NULL. */
void hqo_solve_groups(const uint16_t *w, int64_t n_groups, int g, int nbits, float p,
                      float beta, float kappa, int iters, int early_stop, uint8_t *codes,
                      uint16_t *scale, float *zero_f32, float *s_f32, uint8_t *passes,
                      uint8_t *last_change, uint8_t *shrink_active, uint8_t *stopped)
{
    double x[HQO_MAX_G];
    for (int64_t i = 0; i < n_groups; ++i) {
        const uint16_t *wg = w + i * (int64_t)g;
        for (int j = 0; j < g; ++j) x[j] = (double)hqo_half_to_float(wg[j]);
        float s, z;
        int np, lc, act, rose;
        hqo_solve_group(x, g, nbits, p, beta, kappa, iters, early_stop,
                        codes + i * (int64_t)g, &s, &z, &np, &lc, &act, &rose, NULL, NULL);
        scale[i] = hqo_float_to_half(1.0f / s);
        zero_f32[i] = z;
        if (s_f32) s_f32[i] = s;
        if (passes) passes[i] = (uint8_t)np;
        if (last_change) last_change[i] = (uint8_t)lc;
        if (shrink_active) shrink_active[i] = (uint8_t)act;
        if (stopped) stopped[i] = (uint8_t)rose;
    }
}

/* One min-max affine uint8 round-to-nearest quantizer over n binary32 values, on the grid
 * of its stored binary16 pair (the rule of both 8-bit zeros and 8-bit scales below):
 *   step = binary16((vmax - vmin) / 255)   (1 if that is 0: all values equal),
 *   base = binary16(vmin),
 *   q    = clamp(round-half-even((v - base) / step), 0, 255)   (binary32 operations),
 * meta = {step, base}; a value reads back as q * step + base. Quantizing against the stored
 * pair (not the unrounded one) keeps the read-back within half a step. */
void hqo_u8_affine(const float *v, int64_t n, uint8_t *q, uint16_t *meta)
{
    float vmin = v[0], vmax = v[0];
    for (int64_t i = 1; i < n; ++i) {
        vmin = fminf(vmin, v[i]);
        vmax = fmaxf(vmax, v[i]);
    }
    uint16_t h_step = hqo_float_to_half((vmax - vmin) / 255.0f);
    float step = hqo_half_to_float(h_step);
    if (!(step > 0.0f)) {
        h_step = 0x3c00;                            /* binary16 1.0 */
        step = 1.0f;
    }
    uint16_t h_base = hqo_float_to_half(vmin);
    float base = hqo_half_to_float(h_base);
    for (int64_t i = 0; i < n; ++i) {
        float c = nearbyintf((v[i] - base) / step);
        c = fminf(fmaxf(c, 0.0f), 255.0f);
        q[i] = (uint8_t)c;
    }
    meta[0] = h_step;
    meta[1] = h_base;
}

/* Zero-point storage.
 * 16-bit: zero = binary16(z).
 * 8-bit [TR "Benchmark results / Llama-2": the zero-point goes to 8 bit with no extra
 * grouping and no optimisation]. Reading: one hqo_u8_affine quantizer over all zeros of the
 * tensor; meta = {step, base}. */
void hqo_zero_requant(const float *z, int64_t n, uint8_t *zq, uint16_t *meta)
{
    hqo_u8_affine(z, n, zq, meta);
}

/* 8-bit scales [TR "Benchmark results / Llama-2", the note on the HQQ_g16_s row of the
 * Llama-2 table: that variant also stores its scales on 8-bit grids, one per 128 scales].
 * Reading: the stored binary16 scales of a tensor (one per weight group, in group order)
 * are cut into consecutive groups of `group` values, the last one shorter when group does
 * not divide n; each gets its own hqo_u8_affine quantizer, like the zero-point ("without
 * optimisation"), and meta[2m], meta[2m+1] = {step, base} of group m. The codes of the
 * weights are not re-derived with the quantized scale. */
void hqo_scale_requant(const uint16_t *scale, int64_t n, int group, uint8_t *sq, uint16_t *meta)
{
    float v[4096];
    assert(group >= 1 && group <= 4096);
    for (int64_t g0 = 0, m = 0; g0 < n; g0 += group, ++m) {
        int64_t len = n - g0 < group ? n - g0 : group;
        for (int64_t i = 0; i < len; ++i) v[i] = hqo_half_to_float(scale[g0 + i]);
        hqo_u8_affine(v, len, sq + g0, meta + 2 * m);
    }
}

/* Read-back of 8-bit scales as binary16 scales for reconstruction: one binary32 fused
 * multiply-add q * step + base, rounded to binary16. */
void hqo_scale_dequant(const uint8_t *sq, const uint16_t *meta, int64_t n, int group,
                       uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        int64_t m = i / group;
        float step = hqo_half_to_float(meta[2 * m]);
        float base = hqo_half_to_float(meta[2 * m + 1]);
        out[i] = hqo_float_to_half(fmaf((float)sq[i], step, base));
    }
}

void hqo_zero_to_half(const float *z, int64_t n, uint16_t *zh)
{
    for (int64_t i = 0; i < n; ++i) zh[i] = hqo_float_to_half(z[i]);
}

/* ------------------------------------------------------------------------------------ */
/* Packed code layout. Reading: the pages list the bit widths 8/4/3/2/1 and give no layout, */
/* so the containers are this build's choice. A flat stream of codes in row-major order;   */
/* code k of a container occupies bits [nbits*k, nbits*k + nbits). 8/4/2/1-bit codes fill  */
/* uint8 containers (1/2/4/8 per byte); 3-bit codes fill little-endian uint32 containers,  */
/* 10 per word, bits 30-31 zero. Unused trailing bits are zero.                            */
/* ------------------------------------------------------------------------------------ */

size_t hqo_packed_bytes(int64_t n, int nbits)
{
    if (nbits == 3) return (size_t)(4 * ((n + 9) / 10));
    return (size_t)((n * nbits + 7) / 8);
}

void hqo_pack(const uint8_t *codes, int64_t n, int nbits, uint8_t *out)
{
    size_t nb = hqo_packed_bytes(n, nbits);
    memset(out, 0, nb);
    for (int64_t k = 0; k < n; ++k) {
        uint32_t c = codes[k];
        assert(c < (1u << nbits));
        if (nbits == 3) {
            int64_t word = k / 10;
            int bit = 3 * (int)(k % 10);
            uint32_t v = c << bit;
            for (int b = 0; b < 4; ++b) out[4 * word + b] |= (uint8_t)(v >> (8 * b));
        } else {
            int64_t bitpos = k * nbits;
            out[bitpos / 8] |= (uint8_t)(c << (bitpos % 8));
        }
    }
}

void hqo_unpack(const uint8_t *packed, int64_t n, int nbits, uint8_t *codes)
{
    uint32_t mask = (1u << nbits) - 1u;
    for (int64_t k = 0; k < n; ++k) {
        if (nbits == 3) {
            int64_t word = k / 10;
            uint32_t v = 0;
            for (int b = 0; b < 4; ++b) v |= (uint32_t)packed[4 * word + b] << (8 * b);
            codes[k] = (uint8_t)((v >> (3 * (k % 10))) & mask);
        } else {
            int64_t bitpos = k * nbits;
            codes[k] = (uint8_t)((packed[bitpos / 8] >> (bitpos % 8)) & mask);
        }
    }
}

/* Stored zero of group i as float: the binary16 value, or zq * meta[0] + meta[1] (fused). */
static float stored_zero(const void *zero, const uint16_t *meta, int zero_bits, int64_t i)
{
    if (zero_bits == 16) return hqo_half_to_float(((const uint16_t *)zero)[i]);
    float m0 = hqo_half_to_float(meta[0]), m1 = hqo_half_to_float(meta[1]);
    return fmaf((float)((const uint8_t *)zero)[i], m0, m1);
}

/* Dequantize [SK "HQQLinear layer", dequantize()]: W_r = (q - zero) * scale, rounded to
 * binary16. n is the element count, g the group size. */
void hqo_dequantize(const uint8_t *codes, const uint16_t *scale, const void *zero,
                    const uint16_t *meta, int64_t n, int g, int zero_bits, uint16_t *out)
{
    for (int64_t k = 0; k < n; ++k) {
        int64_t i = k / g;
        float zf = stored_zero(zero, meta, zero_bits, i);
        float sf = hqo_half_to_float(scale[i]);
        float v = ((float)codes[k] - zf) * sf;
        out[k] = hqo_float_to_half(v);
    }
}

/* Per-tensor reconstruction mean squared error from the stored (binary16 / uint8) metadata,
 * before the final binary16 rounding of the reconstruction: mean of (w - (q - zero)*scale)^2,
 * each residual formed in binary32, squares summed in binary64. */
double hqo_mse(const uint16_t *w, const uint8_t *codes, const uint16_t *scale, const void *zero,
               const uint16_t *meta, int64_t n, int g, int zero_bits)
{
    double acc = 0.0;
    for (int64_t k = 0; k < n; ++k) {
        int64_t i = k / g;
        float zf = stored_zero(zero, meta, zero_bits, i);
        float sf = hqo_half_to_float(scale[i]);
        float r = hqo_half_to_float(w[k]) - ((float)codes[k] - zf) * sf;
        acc += (double)r * (double)r;
    }
    return n > 0 ? acc / (double)n : 0.0;
}
