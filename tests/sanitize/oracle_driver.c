/* Drives every function of the CPU oracle over edge cases, for a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer (test infrastructure; compiled together with the oracle's
 * source as one translation unit). Exit status 0 and "oracle driver: ok" when nothing fired. */
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/hqq_oracle.c"

static uint32_t lcg_state = 12345u;
static uint32_t lcg(void)
{
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return lcg_state;
}

/* binary16 bits of a weight: mostly small values, some outliers, zeros of both signs,
 * subnormals and the largest finite values */
static uint16_t weight_bits(int kind)
{
    float v = ((float)(lcg() >> 8) / 16777216.0f - 0.5f) * 0.08f;
    switch (kind) {
    case 1: if (lcg() % 64 == 0) v *= 400.0f; break;          /* outliers */
    case 2: v = (lcg() & 1) ? 0.0f : -0.0f; break;           /* zeros */
    case 3: v = (float)((int)(lcg() % 2047) - 1023) * 5.9604645e-8f; break;   /* subnormals */
    case 4: v = (lcg() & 1) ? 65504.0f : -65504.0f; break;   /* extremes */
    case 5: v = 0.375f; break;                               /* constant */
    default: break;
    }
    return hqo_float_to_half(v);
}

int main(void)
{
    const int bits[] = {1, 2, 3, 4, 8};
    const int gs[] = {1, 2, 16, 64, 256, HQO_MAX_G};
    for (int bi = 0; bi < 5; ++bi)
        for (int gi = 0; gi < 6; ++gi)
            for (int kind = 0; kind < 6; ++kind) {
                const int g = gs[gi], nbits = bits[bi];
                const int64_t ng = g >= 256 ? 2 : 5, n = ng * g;
                uint16_t *w = malloc(sizeof(uint16_t) * (size_t)n);
                uint8_t *codes = malloc((size_t)n), *codes2 = malloc((size_t)n);
                uint16_t *scale = malloc(sizeof(uint16_t) * (size_t)ng);
                float *z = malloc(sizeof(float) * (size_t)ng), *s = malloc(sizeof(float) * (size_t)ng);
                uint8_t *pa = malloc((size_t)ng), *lc = malloc((size_t)ng), *act = malloc((size_t)ng);
                uint8_t *st = malloc((size_t)ng), *zq = malloc((size_t)ng);
                uint16_t meta[2], *zh = malloc(sizeof(uint16_t) * (size_t)ng);
                uint16_t *out = malloc(sizeof(uint16_t) * (size_t)n);
                for (int64_t i = 0; i < n; ++i) w[i] = weight_bits(kind);
                const float betas[] = {1.0f, 1e4f};
                for (int k = 0; k < 2; ++k) {
                    const int iters = k == 0 ? 20 : (g <= 16 ? 254 : 3);
                    hqo_solve_groups(w, ng, g, nbits, 0.7f, betas[k], 1.01f, iters, k == 0,
                                     codes, scale, z, s, pa, lc, act, st);
                }
                hqo_solve_groups(w, ng, g, nbits, 1.0f, 1.0f, 1.01f, 0, 1, codes, scale, z,
                                 NULL, NULL, NULL, NULL, NULL);
                hqo_zero_requant(z, ng, zq, meta);
                hqo_zero_to_half(z, ng, zh);
                size_t nb = hqo_packed_bytes(n, nbits);
                uint8_t *packed = malloc(nb > 0 ? nb : 1);
                hqo_pack(codes, n, nbits, packed);
                hqo_unpack(packed, n, nbits, codes2);
                for (int64_t i = 0; i < n; ++i)
                    if (codes2[i] != codes[i]) { fprintf(stderr, "pack round trip\n"); return 1; }
                hqo_dequantize(codes, scale, zh, NULL, n, g, 16, out);
                hqo_dequantize(codes, scale, zq, meta, n, g, 8, out);
                (void)hqo_mse(w, codes, scale, zh, NULL, n, g, 16);
                (void)hqo_mse(w, codes, scale, zq, meta, n, g, 8);
                uint8_t *sq = malloc((size_t)ng);
                uint16_t *smeta = malloc(sizeof(uint16_t) * 2 * (size_t)ng), *sback = malloc(sizeof(uint16_t) * (size_t)ng);
                for (int sg = 1; sg <= 128; sg *= 8) {
                    hqo_scale_requant(scale, ng, sg, sq, smeta);
                    hqo_scale_dequant(sq, smeta, ng, sg, sback);
                }
                free(w); free(codes); free(codes2); free(scale); free(z); free(s); free(pa);
                free(lc); free(act); free(st); free(zq); free(zh); free(out); free(packed);
                free(sq); free(smeta); free(sback);
            }
    /* conversions over every binary16 pattern and a spread of binary32 values */
    for (uint32_t h = 0; h < 65536; ++h) (void)hqo_half_to_float((uint16_t)h);
    for (int i = 0; i < 200000; ++i) {
        uint32_t b = lcg();
        float f;
        memcpy(&f, &b, sizeof f);
        if (isfinite(f)) (void)hqo_float_to_half(f);
    }
    /* the shrink around its limits */
    const double rs[] = {0.0, -0.0, 1e-300, -1e-300, 1e-12, 0.5, -3.0, 1e300};
    for (int i = 0; i < 8; ++i) (void)hqo_shrink(rs[i], 0.7f, 1.0f);
    printf("oracle driver: ok\n");
    return 0;
}
