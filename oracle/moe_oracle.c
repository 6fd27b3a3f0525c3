/*
 * moe_oracle.c -- plain, slow CPU oracle for one Beam-style Mixture-of-Experts
 * block forward pass.  TEST INFRASTRUCTURE ONLY: the product path never links,
 * loads or calls this file.  It shares no source with the HIP library.
 *
 * What it computes follows "Welcome Beam: a 501B open model you can own,
 * customize, and scale", section "Mixture of Experts" (the same text appears
 * in "Reflection Releases Beam: An Open 501B MoE Model with 1M Context",
 * section "Mixture of Experts"):
 *   - every expert gets a sigmoid score;
 *   - experts are split into G groups of E/G consecutive indices;
 *   - a group's rank is the sum of its two highest scores; the TG best groups
 *     are kept;
 *   - the k best experts among the kept groups are chosen;
 *   - the chosen scores are normalised to sum to one, the expert outputs are
 *     combined with those weights and the result is multiplied by a scale
 *     (2.5 for Beam);
 *   - every expert is a SwiGLU MLP: silu(x Wg^T) * (x Wu^T), then times Wd^T.
 * Section "Residual Stream" of the same page fixes FP32 for the router and for
 * the SwiGLU product.  Inputs are bf16 (widened exactly to fp32); every sum is
 * an fp32 sum taken in plain index order; the SwiGLU product is rounded to
 * bf16 (round-to-nearest-even) before the down projection; the expert output y
 * stays fp32.
 *
 * Readings where the page is silent: a router bias, if given, is added to the
 * logit before the sigmoid; ties go to the lower index, for groups and for
 * experts; a group of one expert ranks by that expert's score alone.
 *
 * Each output element is computed by one plain loop; OpenMP only spreads
 * independent tokens / pairs over host threads and never changes the order of
 * any sum.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG -1
#define ORACLE_ERR_NONFINITE -2

/* bf16 is the upper half of an IEEE binary32: widening is a 16-bit shift. */
static float bf16_bits_to_float(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round an fp32 value to the nearest bf16, ties to even (IEEE 754 default).
 * NaN is kept a quiet NaN.  Written from the definition: keep the upper 16
 * bits, add one unit in the last kept place when the dropped half is more than
 * half a unit, or exactly half and the kept part is odd. */
static uint16_t float_to_bf16_bits_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

static float sigmoidf_plain(float z) { return 1.0f / (1.0f + expf(-z)); }

/* ---- step 1: router scores -------------------------------------------------
 * scores[t,e] = sigmoid( sum_h x[t,h] * Wr[e,h]  + bias[e] ), fp32, h order. */
static void router_scores_one_token(int32_t H, int32_t E, const uint16_t* xrow,
                                    const uint16_t* w_router, const float* bias,
                                    float* s) {
    for (int32_t e = 0; e < E; ++e) {
        const uint16_t* wrow = w_router + (int64_t)e * H;
        float z = 0.0f;
        for (int32_t h = 0; h < H; ++h)
            z = z + bf16_bits_to_float(xrow[h]) * bf16_bits_to_float(wrow[h]);
        if (bias) z = z + bias[e];
        s[e] = sigmoidf_plain(z);
    }
}

/* ---- step 2: group score = sum of the group's two highest scores ---------- */
static float group_top2_sum(const float* s, int32_t first, int32_t size) {
    if (size == 1) return s[first];
    /* highest, lowest index on ties */
    int32_t a = first;
    for (int32_t e = first + 1; e < first + size; ++e)
        if (s[e] > s[a]) a = e;
    /* highest among the rest */
    int32_t b = -1;
    for (int32_t e = first; e < first + size; ++e) {
        if (e == a) continue;
        if (b < 0 || s[e] > s[b]) b = e;
    }
    return s[a] + s[b];
}

/* ---- steps 2-5 for one token: groups, kept groups, top-k, weights --------- */
static void select_one_token(int32_t E, int32_t G, int32_t TG, int32_t k, const float* s,
                             float* gscore, unsigned char* kept, unsigned char* taken,
                             int32_t* ids, float* weights) {
    const int32_t gs = E / G;
    for (int32_t g = 0; g < G; ++g) {
        gscore[g] = group_top2_sum(s, g * gs, gs);
        kept[g] = 0;
    }
    /* keep TG groups: repeatedly take the best not-yet-kept group (lower index
     * wins a tie because only a strictly greater score replaces the pick) */
    for (int32_t r = 0; r < TG; ++r) {
        int32_t best = -1;
        for (int32_t g = 0; g < G; ++g) {
            if (kept[g]) continue;
            if (best < 0 || gscore[g] > gscore[best]) best = g;
        }
        kept[best] = 1;
    }
    /* pick k experts among the kept groups, best first, lower index on ties */
    for (int32_t e = 0; e < E; ++e) taken[e] = 0;
    for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e) {
            if (!kept[e / gs] || taken[e]) continue;
            if (best < 0 || s[e] > s[best]) best = e;
        }
        taken[best] = 1;
        ids[j] = best;
    }
    /* normalise the chosen scores; the sum runs in selection order */
    float sum = 0.0f;
    for (int32_t j = 0; j < k; ++j) sum = sum + s[ids[j]];
    for (int32_t j = 0; j < k; ++j) weights[j] = s[ids[j]] / sum;
}

static int check_route_args(int64_t T, int32_t H, int32_t E, int32_t G, int32_t TG,
                            int32_t k) {
    if (T < 0 || H <= 0 || E <= 0 || G <= 0 || E % G != 0) return ORACLE_ERR_ARG;
    if (TG < 1 || TG > G) return ORACLE_ERR_ARG;
    if (k < 1 || k > TG * (E / G)) return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

/* Route T tokens.  x [T,H] bf16 bits, w_router [E,H] bf16 bits, bias [E] fp32
 * or NULL.  Writes topk_ids [T,k], topk_weights [T,k]; optional scores [T,E]
 * and group_scores [T,G] (NULL to skip).  Returns ORACLE_ERR_NONFINITE if any
 * score is not finite (the method is undefined there). */
int oracle_route(int64_t T, int32_t H, int32_t E, int32_t G, int32_t TG, int32_t k,
                 const uint16_t* x, const uint16_t* w_router, const float* bias,
                 int32_t* topk_ids, float* topk_weights, float* scores_out,
                 float* group_scores_out) {
    int rc = check_route_args(T, H, E, G, TG, k);
    if (rc) return rc;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t t = 0; t < T; ++t) {
        float* s = (float*)malloc(sizeof(float) * (size_t)E);
        float* gsc = (float*)malloc(sizeof(float) * (size_t)G);
        unsigned char* kept = (unsigned char*)malloc((size_t)G);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
        router_scores_one_token(H, E, x + t * H, w_router, bias, s);
        for (int32_t e = 0; e < E; ++e)
            if (!isfinite(s[e])) bad |= 1;
        select_one_token(E, G, TG, k, s, gsc, kept, taken, topk_ids + t * k,
                         topk_weights + t * k);
        if (scores_out) memcpy(scores_out + t * E, s, sizeof(float) * (size_t)E);
        if (group_scores_out) memcpy(group_scores_out + t * G, gsc, sizeof(float) * (size_t)G);
        free(s);
        free(gsc);
        free(kept);
        free(taken);
    }
    return bad ? ORACLE_ERR_NONFINITE : ORACLE_OK;
}

/* Selection only (steps 2-5), from given fp32 scores [T,E].  Lets tests pin the
 * selection on hand-built score tables. */
int oracle_select(int64_t T, int32_t E, int32_t G, int32_t TG, int32_t k, const float* scores,
                  int32_t* topk_ids, float* topk_weights) {
    int rc = check_route_args(T, 1, E, G, TG, k);
    if (rc) return rc;
    float* gsc = (float*)malloc(sizeof(float) * (size_t)G);
    unsigned char* kept = (unsigned char*)malloc((size_t)G);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    for (int64_t t = 0; t < T; ++t)
        select_one_token(E, G, TG, k, scores + t * E, gsc, kept, taken, topk_ids + t * k,
                         topk_weights + t * k);
    free(gsc);
    free(kept);
    free(taken);
    return ORACLE_OK;
}

/* ---- dispatch: stable counting sort of the T*k (token, slot) pairs ---------
 * Pair p = t*k + j goes to expert ids[p].  offsets[e] = number of pairs whose
 * expert is below e (offsets[E] = T*k); sorted_pairs lists the pair ids expert
 * by expert, each expert's pairs in increasing p; pair_rows[p] is the position
 * of p in sorted_pairs. */
int oracle_permute(int64_t T, int32_t k, int32_t E, const int32_t* ids, int32_t* offsets,
                   int32_t* sorted_pairs, int32_t* pair_rows) {
    if (T < 0 || k < 1 || E < 1) return ORACLE_ERR_ARG;
    const int64_t P = T * k;
    for (int32_t e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (ids[p] < 0 || ids[p] >= E) return ORACLE_ERR_ARG;
        offsets[ids[p] + 1] += 1;
    }
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    for (int32_t e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int64_t p = 0; p < P; ++p) {
        int32_t r = fill[ids[p]]++;
        sorted_pairs[r] = (int32_t)p;
        pair_rows[p] = r;
    }
    free(fill);
    return ORACLE_OK;
}

/* ---- one SwiGLU expert on one token ----------------------------------------
 * g[n] = sum_h x[h] Wg[n,h];  u[n] = sum_h x[h] Wu[n,h]   (fp32, h order)
 * a[n] = (g[n] * sigmoid(g[n])) * u[n]                   (fp32)
 * h[n] = bf16_rne(a[n])
 * y[m] = sum_n h[n] Wd[m,n]                              (fp32, n order)
 * Wg, Wu are [I,H]; Wd is [H,I]; all bf16 bits. */
static void swiglu_expert_one_token(int32_t H, int32_t I, const uint16_t* xrow,
                                    const uint16_t* wg, const uint16_t* wu,
                                    const uint16_t* wd, uint16_t* hbits, float* y) {
    for (int32_t n = 0; n < I; ++n) {
        const uint16_t* grow = wg + (int64_t)n * H;
        const uint16_t* urow = wu + (int64_t)n * H;
        float g = 0.0f, u = 0.0f;
        for (int32_t c = 0; c < H; ++c) {
            float xv = bf16_bits_to_float(xrow[c]);
            g = g + xv * bf16_bits_to_float(grow[c]);
            u = u + xv * bf16_bits_to_float(urow[c]);
        }
        float silu = g * sigmoidf_plain(g);
        float a = silu * u;
        hbits[n] = float_to_bf16_bits_rne(a);
    }
    for (int32_t m = 0; m < H; ++m) {
        const uint16_t* drow = wd + (int64_t)m * I;
        float acc = 0.0f;
        for (int32_t n = 0; n < I; ++n)
            acc = acc + bf16_bits_to_float(hbits[n]) * bf16_bits_to_float(drow[n]);
        y[m] = acc;
    }
}

/* Expert FFN for a list of (token, expert) pairs.  tok[q] indexes rows of x
 * [*,H]; exp[q] indexes the expert weight stacks wg/wu [*,I,H], wd [*,H,I].
 * Writes y [npairs,H] fp32 and, if h_out is not NULL, the bf16 SwiGLU product
 * h [npairs,I]. */
int oracle_ffn_pairs(int64_t npairs, int32_t H, int32_t I, const int32_t* tok,
                     const int32_t* exp, const uint16_t* x, const uint16_t* wg,
                     const uint16_t* wu, const uint16_t* wd, uint16_t* h_out, float* y) {
    if (npairs < 0 || H <= 0 || I <= 0) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < npairs; ++q) {
        const int64_t e = exp[q];
        uint16_t* hb = h_out ? h_out + q * I : (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
        swiglu_expert_one_token(H, I, x + (int64_t)tok[q] * H, wg + e * I * H, wu + e * I * H,
                                wd + e * H * I, hb, y + q * H);
        if (!h_out) free(hb);
    }
    return ORACLE_OK;
}

/* ---- FP8 expert weights ------------------------------------------------------
 * The pages give no FP8 scheme for the experts; the reading taken: each weight
 * matrix is stored as FP8 E4M3 codes (the OCP "e4m3fn" encoding: 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits, no infinities, 0x7f/0xff NaN)
 * with one fp32 scale per output channel (per row n of Wg/Wu, per row m of
 * Wd).  A channel's dot product is its scale times the dot product with the
 * decoded codes; activations and the SwiGLU product stay as in the bf16 path.
 *   g[n] = sg[n] * sum_h x[h] q_g[n,h]   (the sum in fp32, h order)
 *   u[n] = su[n] * sum_h x[h] q_u[n,h]
 *   h[n] = bf16_rne((g[n] * sigmoid(g[n])) * u[n])
 *   y[m] = sd[m] * sum_n h[n] q_d[m,n]  */
static float e4m3_to_float(uint8_t b) {
    const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
    float v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexpf((float)m, -9);            /* subnormal: m/8 * 2^-6 */
    else
        v = ldexpf((float)(8 + m), e - 10);  /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

static void swiglu_expert_one_token_fp8(int32_t H, int32_t I, const uint16_t* xrow,
                                        const uint8_t* qg, const float* sg, const uint8_t* qu,
                                        const float* su, const uint8_t* qd, const float* sd,
                                        uint16_t* hbits, float* y) {
    for (int32_t n = 0; n < I; ++n) {
        const uint8_t* grow = qg + (int64_t)n * H;
        const uint8_t* urow = qu + (int64_t)n * H;
        float g = 0.0f, u = 0.0f;
        for (int32_t c = 0; c < H; ++c) {
            float xv = bf16_bits_to_float(xrow[c]);
            g = g + xv * e4m3_to_float(grow[c]);
            u = u + xv * e4m3_to_float(urow[c]);
        }
        g = sg[n] * g;
        u = su[n] * u;
        float silu = g * sigmoidf_plain(g);
        hbits[n] = float_to_bf16_bits_rne(silu * u);
    }
    for (int32_t m = 0; m < H; ++m) {
        const uint8_t* drow = qd + (int64_t)m * I;
        float acc = 0.0f;
        for (int32_t n = 0; n < I; ++n)
            acc = acc + bf16_bits_to_float(hbits[n]) * e4m3_to_float(drow[n]);
        y[m] = sd[m] * acc;
    }
}

/* As oracle_ffn_pairs with FP8 weights: qg/qu [*,I,H] and qd [*,H,I] E4M3
 * codes, sg/su [*,I] and sd [*,H] fp32 per-channel scales. */
int oracle_ffn_pairs_fp8(int64_t npairs, int32_t H, int32_t I, const int32_t* tok,
                         const int32_t* exp, const uint16_t* x, const uint8_t* qg,
                         const float* sg, const uint8_t* qu, const float* su, const uint8_t* qd,
                         const float* sd, uint16_t* h_out, float* y) {
    if (npairs < 0 || H <= 0 || I <= 0) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < npairs; ++q) {
        const int64_t e = exp[q];
        uint16_t* hb = h_out ? h_out + q * I : (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
        swiglu_expert_one_token_fp8(H, I, x + (int64_t)tok[q] * H, qg + e * I * H, sg + e * I,
                                    qu + e * I * H, su + e * I, qd + e * H * I, sd + e * H, hb,
                                    y + q * H);
        if (!h_out) free(hb);
    }
    return ORACLE_OK;
}

/* Exposed for the test that pins the decoding against a library cast. */
void oracle_e4m3_decode(int64_t n, const uint8_t* src, float* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = e4m3_to_float(src[i]);
}

/* ---- recombination ----------------------------------------------------------
 * out[t,m] = scale * sum_j w[t,j] * y[t*k+j, m], the sum in j order, fp32.
 * y rows are in pair order (p = t*k+j). */
int oracle_combine(int64_t T, int32_t k, int32_t H, const float* y, const float* w,
                   float scale, float* out) {
    if (T < 0 || k < 1 || H <= 0) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t m = 0; m < H; ++m) {
            float acc = 0.0f;
            for (int32_t j = 0; j < k; ++j) acc = acc + w[t * k + j] * y[(t * k + j) * H + m];
            out[t * H + m] = scale * acc;
        }
    }
    return ORACLE_OK;
}

/* ---- sublayer epilogue: post-norm and the residual-stream update ----------
 * "Welcome Beam: a 501B open model you can own, customize, and scale", section
 * "Residual Stream": every sublayer output is normalised after the sublayer;
 * the embedding is step 1 of the stream and step s adds the (normalised)
 * sublayer output with weight 1/sqrt(s) while the stream keeps weight
 * sqrt((s-1)/s); the norms compute in FP32.  Readings: the norm is RMSNorm
 * (the only norm the page names) with a per-channel gain g and an eps added
 * to the mean square; s = 1 replaces the stream by the normalised output.
 *   n[m]   = (o[m] / sqrt(mean_m(o^2) + eps)) * g[m]
 *   res[m] = sqrt((s-1)/s) * res[m] + (1/sqrt(s)) * n[m]
 * All in fp32; the sum of squares runs in index order. */
int oracle_residual_norm(int64_t T, int32_t H, const float* o, const float* g, float eps,
                         int32_t step, float* res) {
    if (T < 0 || H <= 0 || step < 1 || !(eps > 0.0f)) return ORACLE_ERR_ARG;
    const float a = sqrtf((float)(step - 1) / (float)step);
    const float b = 1.0f / sqrtf((float)step);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float* ot = o + t * H;
        float ss = 0.0f;
        for (int32_t m = 0; m < H; ++m) ss = ss + ot[m] * ot[m];
        const float inv = 1.0f / sqrtf(ss / (float)H + eps);
        for (int32_t m = 0; m < H; ++m) {
            const float n = (ot[m] * inv) * g[m];
            res[t * H + m] = a * res[t * H + m] + b * n;
        }
    }
    return ORACLE_OK;
}

/* Exposed for tests that pin the rounding helper against a library cast. */
void oracle_f32_to_bf16_rne(int64_t n, const float* src, uint16_t* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = float_to_bf16_bits_rne(src[i]);
}

/* Number of threads the parallel loops above use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
