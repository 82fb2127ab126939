/*
 * oracle.c -- plain CPU oracle for gated GQA causal attention prefill.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header or table
 * with the HIP library; the two meet only at the seeded inputs.
 *
 * What it computes, per query row i (absolute position p = q_base + i) and
 * per query head h, following the rounding points that the QSA kernel page
 * ("feat(qwen4): add the QSA sparse-attention kernel and its golden",
 * sections "Semantics" and the final commit message) attributes to the
 * reference model:
 *
 *   1. q and the gate g are the two halves of head h's slice of the fused
 *      q|gate projection row ([Hq][2][D] per row).
 *   2. (1+w) RMSNorm, fp32 throughout, one cast to bf16 at the end.
 *   3. Partial RoPE on the first R of D dims, rotate-half pairs (j, j+R/2),
 *      cos/sin taken from the shared fp32 table and cast to bf16, each
 *      product and the sum rounded to bf16 (the rotation is bf16 arithmetic).
 *   4. Score = bf16(q . k) then times 1/sqrt(D) (exact for D = 256).
 *   5. fp32 softmax over the rounded scores of the visible keys; the
 *      normalised weights are rounded to bf16 before the context reduction.
 *   6. Context = bf16(sum_j w_j v_j), fp32 accumulation.
 *   7. Output = bf16(ctx * bf16(sigmoid(g))).
 *
 * Visibility: key j is visible to row i iff j <= p (causal pass; the
 * bidirectional pass drops this predicate, every key 0..T-1 is a candidate)
 * and, when a mask is given, mask[i][j] != 0 (non-zero = visible).  A row with
 * no visible key outputs 0.
 * KV head of query head h is h / (Hq / Hkv).
 *
 * Every sum runs in ascending index order in fp32.  Build with
 * -ffp-contract=off and without fast-math so the order and rounding are the
 * ones written here.  Products of two bf16 values are exact in fp32.
 *
 * ORACLE_MUTATION (compile-time, default 0) plants one deliberate mistake; the
 * CPU tests build the mutants to show that the oracle's pins catch each one.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTATION
#define ORACLE_MUTATION 0
#endif

typedef uint16_t bf16_t;

/* ---- bf16 <-> fp32, round to nearest even (IEEE 754 roundTiesToEven) ---- */

static float bf16_to_f32(bf16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static bf16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)          /* NaN stays NaN, made quiet */
        return (bf16_t)((u >> 16) | 0x0040u);
    /* Adding 0x7fff plus the kept lsb rounds to nearest with ties to even;
       a carry out of the mantissa bumps the exponent (up to infinity). */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

static float rb(float f) { return bf16_to_f32(f32_to_bf16(f)); }

/* ---- problem description (mirrors the inputs of one prefill call) ---- */

typedef struct {
    int32_t n_q_heads, n_kv_heads, head_dim, rotary_dim;
    float rms_eps;
    int32_t T;              /* keys 0..T-1                                  */
    int32_t q_base;         /* query rows are positions q_base..T-1         */
    const bf16_t *qg;       /* [T-q_base][Hq][2][D]                         */
    const bf16_t *k;        /* [T][Hkv][D] raw                              */
    const bf16_t *v;        /* [T][Hkv][D]                                  */
    const bf16_t *q_norm_w; /* [D], applied as (1+w)                        */
    const bf16_t *k_norm_w; /* [D]                                          */
    const float *cos_tab;   /* [n_pos][R/2]                                 */
    const float *sin_tab;   /* [n_pos][R/2]                                 */
    int32_t n_pos;
    const uint8_t *mask;    /* [T-q_base][T] or NULL                        */
    const bf16_t *kp;       /* prepared keys [Hkv][T][D] from oracle_prepare_keys */
    int32_t causal;         /* 1: causal pass; 0: bidirectional (q_base 0)   */
    int32_t score_f64;      /* 0: q . k summed in fp32, ascending; 1: summed in double, rounded once to fp32 */
} oracle_problem;

int oracle_abi(void) { return 3; }   /* 2: oracle_problem.causal; 3: .score_f64 */
int oracle_mutation(void) { return ORACLE_MUTATION; }

void oracle_bf16_round(const float *in, bf16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16(in[i]);
}

/*
 * (1+w) RMSNorm then partial RoPE of one head vector x[D] at table row
 * cos_row/sin_row (QSA kernel page, "Semantics": (1+w) RMSNorm at the model's
 * eps and 64-of-256 partial RoPE from the shared table; final commit message:
 * the normalised vector is rounded to bf16 a single time, the table's cos and
 * sin are rounded to bf16, and the rotation's products and sums are bf16).
 */
void oracle_norm_rope(const bf16_t *x, const bf16_t *w, const float *cos_row,
                      const float *sin_row, int32_t D, int32_t R, float eps, bf16_t *out)
{
    float ss = 0.0f;
    for (int32_t d = 0; d < D; ++d) {
        float xv = bf16_to_f32(x[d]);
        ss += xv * xv;
    }
#if ORACLE_MUTATION == 4
    float r = 1.0f / (sqrtf(ss / (float)D) + eps);        /* eps outside the root */
#else
    float r = 1.0f / sqrtf(ss / (float)D + eps);
#endif
    bf16_t *n = (bf16_t *)malloc(sizeof(bf16_t) * (size_t)D);
    for (int32_t d = 0; d < D; ++d) {
#if ORACLE_MUTATION == 5
        float scale = bf16_to_f32(w[d]);                  /* w instead of (1+w) */
#else
        float scale = 1.0f + bf16_to_f32(w[d]);
#endif
        n[d] = f32_to_bf16((bf16_to_f32(x[d]) * r) * scale);
    }
    const int32_t half = R / 2;
    for (int32_t d = 0; d < D; ++d)
        out[d] = n[d];
    for (int32_t j = 0; j < half; ++j) {
        float c = rb(cos_row[j]);
        float s = rb(sin_row[j]);
#if ORACLE_MUTATION == 3
        float a = bf16_to_f32(n[2 * j]), b = bf16_to_f32(n[2 * j + 1]);   /* interleaved pairs */
        out[2 * j] = f32_to_bf16(rb(a * c) + rb(-b * s));
        out[2 * j + 1] = f32_to_bf16(rb(b * c) + rb(a * s));
#else
        float a = bf16_to_f32(n[j]);
        float b = bf16_to_f32(n[j + half]);
        out[j] = f32_to_bf16(rb(a * c) + rb(-b * s));
#if ORACLE_MUTATION == 2
        out[j + half] = f32_to_bf16(rb(b * c) - rb(a * s));  /* wrong sign */
#else
        out[j + half] = f32_to_bf16(rb(b * c) + rb(a * s));
#endif
#endif
    }
    free(n);
}

/* Prepared keys kp[c][j][:] = norm_rope(k[j][c][:]) at position j. */
int oracle_prepare_keys(const oracle_problem *p, bf16_t *kp)
{
    const int32_t D = p->head_dim, R = p->rotary_dim, Hkv = p->n_kv_heads;
    if (p->n_pos < p->T)
        return -1;
    for (int32_t c = 0; c < Hkv; ++c)
        for (int32_t j = 0; j < p->T; ++j) {
#if ORACLE_MUTATION == 15
            const int32_t pos = 0;                        /* key position ignored */
#else
            const int32_t pos = j;
#endif
#if ORACLE_MUTATION == 16
            const int32_t src = 0;                        /* every KV head reads head 0's keys */
#else
            const int32_t src = c;
#endif
            oracle_norm_rope(p->k + ((size_t)j * Hkv + src) * D, p->k_norm_w,
                             p->cos_tab + (size_t)pos * (R / 2), p->sin_tab + (size_t)pos * (R / 2),
                             D, R, p->rms_eps, kp + ((size_t)c * p->T + j) * D);
        }
    return 0;
}

/* Prepared queries qp[i][h][:] = norm_rope(q part of qg[i][h]) at position q_base + i. */
int oracle_prepare_queries(const oracle_problem *p, bf16_t *qp)
{
    const int32_t D = p->head_dim, R = p->rotary_dim, Hq = p->n_q_heads;
    const int32_t rows = p->T - p->q_base;
    if (p->n_pos < p->T)
        return -1;
    for (int32_t i = 0; i < rows; ++i) {
#if ORACLE_MUTATION == 11
        const int32_t pos = i;                            /* position ignores q_base */
#else
        const int32_t pos = p->q_base + i;
#endif
        for (int32_t h = 0; h < Hq; ++h)
            oracle_norm_rope(p->qg + (((size_t)i * Hq + h) * 2 + 0) * D, p->q_norm_w,
                             p->cos_tab + (size_t)pos * (R / 2), p->sin_tab + (size_t)pos * (R / 2),
                             D, R, p->rms_eps, qp + ((size_t)i * Hq + h) * D);
    }
    return 0;
}

static int visible(const oracle_problem *p, int32_t i, int32_t j)
{
    const int32_t pos = p->q_base + i;
#if ORACLE_MUTATION == 14
    if (j > pos)                                          /* causal in the bidirectional pass */
        return 0;
#endif
#if ORACLE_MUTATION == 8
    if (p->causal && j >= pos)                            /* strict causality */
        return 0;
#else
    if (p->causal && j > pos)
        return 0;
#endif
    if (p->mask) {
#if ORACLE_MUTATION == 10
        return p->mask[(size_t)i * p->T + j] == 0;        /* inverted polarity */
#else
        return p->mask[(size_t)i * p->T + j] != 0;
#endif
    }
    return 1;
}

/*
 * Attention for the query rows listed in rows[0..n_rows) (indices into the
 * window, 0..T-q_base-1).  out[n][h*D + d] is the gated output of row rows[n].
 * Optional outputs (NULL to skip):
 *   ctx_out  [n_rows][Hq*D]      bf16 ungated context
 *   wsum_out [n_rows][Hq]        fp32 sum of the bf16 weights of the row-head
 *   wts_out  [n_rows][Hq][T]     fp32 value of each bf16 weight (0 when hidden)
 * p->kp must hold the prepared keys.  Returns 0, or -1 on bad arguments.
 */
int oracle_attention(const oracle_problem *p, const int32_t *rows, int32_t n_rows, bf16_t *out,
                     bf16_t *ctx_out, float *wsum_out, float *wts_out)
{
    const int32_t D = p->head_dim, R = p->rotary_dim, Hq = p->n_q_heads, Hkv = p->n_kv_heads;
    const int32_t G = Hq / Hkv, T = p->T, nrow_all = T - p->q_base;
    if (!p->kp || Hkv <= 0 || Hq % Hkv != 0 || p->n_pos < T)
        return -1;
    float *sc = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
    float *wt = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
    uint8_t *vis = (uint8_t *)malloc((size_t)(T > 0 ? T : 1));
    bf16_t *qr = (bf16_t *)malloc(sizeof(bf16_t) * (size_t)D);
    float *acc = (float *)malloc(sizeof(float) * (size_t)D);
    for (int32_t n = 0; n < n_rows; ++n) {
        const int32_t i = rows[n];
        if (i < 0 || i >= nrow_all) {
            free(sc); free(wt); free(vis); free(qr); free(acc);
            return -1;
        }
#if ORACLE_MUTATION == 11
        const int32_t pos = i;
#else
        const int32_t pos = p->q_base + i;
#endif
        for (int32_t h = 0; h < Hq; ++h) {
#if ORACLE_MUTATION == 7
            const int32_t c = h % Hkv;                    /* wrong GQA map */
#else
            const int32_t c = h / G;
#endif
            const bf16_t *q = p->qg + (((size_t)i * Hq + h) * 2 + 0) * D;
            const bf16_t *g = p->qg + (((size_t)i * Hq + h) * 2 + 1) * D;
            oracle_norm_rope(q, p->q_norm_w, p->cos_tab + (size_t)pos * (R / 2),
                             p->sin_tab + (size_t)pos * (R / 2), D, R, p->rms_eps, qr);
            /* Scores of visible keys: bf16(q . k), then the 1/sqrt(D) scale. */
            int any = 0;
            float m = -INFINITY;
            for (int32_t j = 0; j < T; ++j) {
                vis[j] = (uint8_t)visible(p, i, j);
                if (!vis[j])
                    continue;
                const bf16_t *kr = p->kp + ((size_t)c * T + j) * D;
                /* The pages fix the score as the bf16 rounding of the fp32 dot
                   product but not the order of its sum: by default it runs in
                   ascending dimension order in fp32; score_f64 sums in double
                   (each product of two bf16 values is exact) and rounds once. */
                float dot = 0.0f;
                if (p->score_f64) {
                    double acc = 0.0;
                    for (int32_t d = 0; d < D; ++d)
                        acc += (double)bf16_to_f32(qr[d]) * (double)bf16_to_f32(kr[d]);
                    dot = (float)acc;
                } else {
                    for (int32_t d = 0; d < D; ++d)
                        dot += bf16_to_f32(qr[d]) * bf16_to_f32(kr[d]);
                }
#if ORACLE_MUTATION == 6
                sc[j] = rb(dot);                          /* scale dropped */
#else
                sc[j] = rb(dot) * (1.0f / sqrtf((float)D));
#endif
                if (!any || sc[j] > m)
                    m = sc[j];
                any = 1;
            }
            float *o = acc;
            for (int32_t d = 0; d < D; ++d)
                o[d] = 0.0f;
            float wsum = 0.0f;
            if (any) {
                /* fp32 softmax over the rounded scores; weights rounded to bf16. */
                float l = 0.0f;
                for (int32_t j = 0; j < T; ++j) {
                    if (!vis[j])
                        continue;
                    wt[j] = (float)exp((double)(sc[j] - m));
                    l += wt[j];
                }
                for (int32_t j = 0; j < T; ++j) {
                    if (!vis[j])
                        continue;
                    wt[j] = rb(wt[j] / l);
                    wsum += wt[j];
                }
#if ORACLE_MUTATION == 12
                const int32_t jend = p->causal ? pos : T - 1;   /* drops the last visible key */
#else
                const int32_t jend = p->causal ? pos + 1 : T;
#endif
                for (int32_t j = 0; j < jend && j < T; ++j) {
                    if (!vis[j])
                        continue;
#if ORACLE_MUTATION == 13
                    const bf16_t *vr = p->k + ((size_t)j * Hkv + c) * D;   /* K in place of V */
#else
                    const bf16_t *vr = p->v + ((size_t)j * Hkv + c) * D;
#endif
                    for (int32_t d = 0; d < D; ++d)
                        o[d] += wt[j] * bf16_to_f32(vr[d]);
                }
            }
            for (int32_t d = 0; d < D; ++d) {
                float ctx = rb(o[d]);
                float gv = bf16_to_f32(g[d]);
#if ORACLE_MUTATION == 1
                float sg = 1.0f / (1.0f + (float)exp(-(double)gv));        /* sigmoid not rounded */
#else
                float sg = rb(1.0f / (1.0f + (float)exp(-(double)gv)));
#endif
                out[((size_t)n * Hq + h) * D + d] = any ? f32_to_bf16(ctx * sg) : 0;
                if (ctx_out)
                    ctx_out[((size_t)n * Hq + h) * D + d] = any ? f32_to_bf16(ctx) : 0;
            }
            if (wsum_out)
                wsum_out[(size_t)n * Hq + h] = wsum;
            if (wts_out) {
                float *wr = wts_out + ((size_t)n * Hq + h) * T;
                for (int32_t j = 0; j < T; ++j)
                    wr[j] = (any && vis[j]) ? wt[j] : 0.0f;
            }
        }
    }
    free(sc); free(wt); free(vis); free(qr); free(acc);
    return 0;
}
