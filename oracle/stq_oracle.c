/*
 * stq_oracle.c -- plain, slow, obviously-correct CPU oracle for the quantized
 * gated delta-rule decode step (STEPQuant-style recurrent-state quantization).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no header, helper, table or constant with the HIP
 * library; it carries its own reader and writer of the documented packed layout.
 *
 * Sources (the pages are the STEPQuant paper, "STEPQuant: When and Where Errors
 * Matter in Delta-Rule Recurrent State Quantization", arXiv 2609.38169):
 *   - gated delta rule and readout:      Sec. 2.1, Eq. (1) (update + y = S^T q)
 *   - symmetric uniform quantizer:       Sec. 2.2 (Q_{b,s}, q_b = 2^{b-1}-1)
 *   - dual-axis representation X = r c z: Sec. 4.3 ("Key-Row-Aware Dual-axis
 *                                         Fitting", representation and
 *                                         "Quantization" paragraph)
 *   - order of one decode step:          App. C.3, Table C2 (reconstruct ->
 *                                         update -> emit readout before
 *                                         requantization -> row factors -> pack)
 *
 * Readings taken where the pages leave a step open (each is also listed in the
 * design notes of the repository):
 *   R1  round() is round-half-to-even (rhe), written out from its definition.
 *   R2  the row factor is the absmax rule r_i = max_j |X_ij / c_j| / q_b, stored
 *       in fp32 and floored at 2^-126 (the paper only requires r_i > 0, Sec. 4.3).
 *   R3  the column factor c_j is fixed per head (set by offline calibration).
 *   R4  the gate is scalar: D_t = alpha * I (gated DeltaNet form of Eq. (1)).
 *   R5  value head h reads key head floor(h / (Hv/Hk)).
 *   R6  x_ij = X_ij / c_j is formed first (it feeds the row max), then x_ij / r_i.
 *   R7  codes are two's complement; 8-bit rows are int8, 4-bit rows are nibbles
 *       with the even column in the low nibble.
 *   R14 the refit variant keeps column factors per state and, after the row
 *       factors and codes of a step are taken against the current ones, refits
 *       them once with the codes held fixed (App. C.1 fixed-code update; Table
 *       C2 step 5) over all rows of the head, weights w2 = w^2; the new factor
 *       is rounded to fp32 and floored at 2^-126, a zero denominator keeps the
 *       old one.  The stored codes are those taken against the old factors.
 *   R15 row-impact weights: omega_i = sum over calibration samples of
 *       (alpha (q_i - beta k_i k.q))^2 (Sec. 4.1 with the scalar gate; with
 *       the diagonal gate, d_i in place of alpha, App. C.1), and
 *       w2_i = (omega_i / mean omega)^(1/4) (App. B.3: w ~ omega^(1/8)),
 *       floored at 2^-32; an all-zero head gets w2 = 1.
 *   R16 the diagonal gate (KDA form) is one fp32 value per (sequence, value
 *       head, logical key row); it scales row i of the previous state.
 *
 * Arithmetic: every intermediate is an IEEE double; the persisted quantities
 * (r, o) are rounded once to fp32.  Build with -ffp-contract=off so that the
 * expressions below are evaluated exactly as written.
 *
 * Packed layout (per head h of a slot; "physical" row p, logical row perm[h][p]):
 *   pool8  int8   [slot][Hv][n8][dv]         physical rows 0 .. n8-1   (8-bit)
 *   pool4  uint8  [slot][Hv][dk-n8][dv/2]    physical rows n8 .. dk-1  (4-bit)
 *   r      float  [slot][Hv][dk]             row factor, physical order
 *   c      float  [Hv][dv]                   column factor
 *   perm   int32  [Hv][dk]                   logical row of each physical row
 * The oracle's batched entry points take slot == batch index.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- basics -- */

/* Round half to even, from the definition: take the floor f of y; a fractional
 * part above one half rounds up, below one half rounds down, and exactly one
 * half goes to whichever of f, f+1 is even.  (Sec. 2.2 "round", reading R1.) */
double oracle_rhe(double y) {
    double f = floor(y);
    double frac = y - f; /* exact for |y| < 2^52 */
    if (frac > 0.5) return f + 1.0;
    if (frac < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* q_b = 2^(b-1) - 1 (Sec. 2.2). */
static int qmax_of_bits(int bits) { return (1 << (bits - 1)) - 1; }

/* Bit width of physical row p: the first n8 physical rows are 8-bit. */
static int row_bits(int p, int n8) { return p < n8 ? 8 : 4; }

/* Read the code of physical row p, column j of one head (reading R7). */
static int read_code(const int8_t *p8, const uint8_t *p4, int n8, int dv,
                     int p, int j) {
    if (p < n8) return (int)p8[(size_t)p * dv + j];
    uint8_t byte = p4[(size_t)(p - n8) * (dv / 2) + j / 2];
    int nib = (j % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return nib >= 8 ? nib - 16 : nib;
}

/* Write the code of physical row p, column j of one head (reading R7). */
static void write_code(int8_t *p8, uint8_t *p4, int n8, int dv, int p, int j,
                       int z) {
    if (p < n8) {
        p8[(size_t)p * dv + j] = (int8_t)z;
        return;
    }
    uint8_t *byte = &p4[(size_t)(p - n8) * (dv / 2) + j / 2];
    uint8_t nib = (uint8_t)(z & 0x0F);
    if (j % 2 == 0)
        *byte = (uint8_t)((*byte & 0xF0) | nib);
    else
        *byte = (uint8_t)((*byte & 0x0F) | (nib << 4));
}

/* ------------------------------------------------------- unit operations -- */

typedef struct {
    int hv, hk, dk, dv, n8;
} orc_shape;

static size_t unit8_bytes(const orc_shape *s) { return (size_t)s->n8 * s->dv; }
static size_t unit4_bytes(const orc_shape *s) {
    return (size_t)(s->dk - s->n8) * (s->dv / 2);
}

/* Reconstruct one head's state in logical row order:
 * S_ij = (r_p * c_j) * z_pj with i = perm[p]  (Sec. 4.3 representation;
 * Table C2 step 1). */
static void unit_dequant(const orc_shape *s, const int8_t *p8,
                         const uint8_t *p4, const float *r, const float *c,
                         const int32_t *perm, double *S) {
    for (int p = 0; p < s->dk; ++p) {
        int i = perm[p];
        for (int j = 0; j < s->dv; ++j) {
            double rc = (double)r[p] * (double)c[j];
            S[(size_t)i * s->dv + j] = rc * (double)read_code(p8, p4, s->n8, s->dv, p, j);
        }
    }
}

/* One gated delta-rule step with D_t = alpha*I, in place on a logical-order
 * double matrix S (dk x dv), and the readout taken from the updated state:
 *   u = S^T k;  S <- alpha*S + beta * k (v - alpha*u)^T;  o = S^T q
 * (Sec. 2.1 Eq. (1) with D_t = alpha I, reading R4; Table C2 steps 2-3). */
static void unit_delta_step(int dk, int dv, double *S, const double *q,
                            const double *k, const double *v, double alpha,
                            double beta, double *o) {
    double *u = (double *)calloc((size_t)dv, sizeof(double));
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * k[i];
        u[j] = acc;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) {
            double *x = &S[(size_t)i * dv + j];
            *x = alpha * (*x) + beta * k[i] * (v[j] - alpha * u[j]);
        }
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * q[i];
        o[j] = acc;
    }
    free(u);
}

/* The same step with a diagonal gate D_t = diag(d) over the key rows (Sec. 2.1
 * Eq. (1) with a per-channel gate, the KDA form named in Sec. 6.1 and App.
 * C.1), d in logical row order:
 *   u = (D S)^T k;  S <- D S + beta * k (v - u)^T;  o = S^T q            */
static void unit_delta_step_diag(int dk, int dv, double *S, const double *q,
                                 const double *k, const double *v,
                                 const double *d, double beta, double *o) {
    double *u = (double *)calloc((size_t)dv, sizeof(double));
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += d[i] * S[(size_t)i * dv + j] * k[i];
        u[j] = acc;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) {
            double *x = &S[(size_t)i * dv + j];
            *x = d[i] * (*x) + beta * k[i] * (v[j] - u[j]);
        }
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * q[i];
        o[j] = acc;
    }
    free(u);
}

/* Either gate: the scalar alpha of unit u, or the row gate gate[u][dk].
 * Also used by the ragged-format oracle (stq_alloc_oracle.c). */
void orc_unit_update(int dk, int dv, double *S, const double *q, const double *k,
                     const double *v, const float *alpha, const float *gate, long u,
                     double beta, double *o) {
    if (!gate) {
        unit_delta_step(dk, dv, S, q, k, v, (double)alpha[u], beta, o);
        return;
    }
    double *d = (double *)calloc((size_t)dk, sizeof(double));
    for (int i = 0; i < dk; ++i) d[i] = (double)gate[(size_t)u * dk + i];
    unit_delta_step_diag(dk, dv, S, q, k, v, d, beta, o);
    free(d);
}

/* Requantize a logical-order double matrix X into one head's packed rows
 * (Sec. 2.2 quantizer; Sec. 4.3 "Quantization"; Table C2 steps 4 and 6;
 * readings R2, R3, R6):
 *   x_ij = X_ij / c_j,  m_i = max_j |x_ij|,  r_i = max(fl32(m_i / q_b), 2^-126)
 *   z_ij = clip(rhe(x_ij / r_i), -q_b, q_b)                                 */
static void unit_requant(const orc_shape *s, const double *X, const float *c,
                         const int32_t *perm, int8_t *p8, uint8_t *p4,
                         float *r_out) {
    const double floor_r = ldexp(1.0, -126);
    for (int p = 0; p < s->dk; ++p) {
        int i = perm[p];
        int qb = qmax_of_bits(row_bits(p, s->n8));
        const double *row = &X[(size_t)i * s->dv];
        double m = 0.0;
        for (int j = 0; j < s->dv; ++j) {
            double x = row[j] / (double)c[j];
            if (fabs(x) > m) m = fabs(x);
        }
        double rr = (double)(float)(m / (double)qb);
        if (rr < floor_r) rr = floor_r;
        r_out[p] = (float)rr;
        for (int j = 0; j < s->dv; ++j) {
            double x = row[j] / (double)c[j];
            double z = oracle_rhe(x / rr);
            if (z > qb) z = qb;
            if (z < -qb) z = -qb;
            write_code(p8, p4, s->n8, s->dv, p, j, (int)z);
        }
    }
}

/* Online column refit of one head (App. C.1, the fixed-code update; Table C2
 * step 5; reading R14): with the codes z and row factors r just written for
 * the updated state X (logical order) and the squared row-impact weights w2
 * (logical order), every column factor becomes the weighted least-squares fit
 * of X by v = r z with the codes held fixed,
 *   c_j = sum_i w2_i v_ij X_ij / sum_i w2_i v_ij^2,   v_ij = r_i z_ij,
 * rounded to fp32 and floored at 2^-126; a zero denominator keeps the
 * previous c_j.  Sums run over physical rows in ascending order. */
static void unit_refit(const orc_shape *s, const double *X, const int32_t *perm,
                       const float *w2, const int8_t *p8, const uint8_t *p4,
                       const float *r, float *c) {
    const double floor_c = ldexp(1.0, -126);
    for (int j = 0; j < s->dv; ++j) {
        double num = 0.0, den = 0.0;
        for (int p = 0; p < s->dk; ++p) {
            int i = perm[p];
            double vij = (double)r[p] * (double)read_code(p8, p4, s->n8, s->dv, p, j);
            double wt = (double)w2[i];
            num += wt * vij * X[(size_t)i * s->dv + j];
            den += wt * vij * vij;
        }
        if (den > 0.0) {
            double cn = (double)(float)(num / den);
            if (cn < floor_c) cn = floor_c;
            c[j] = (float)cn;
        }
    }
}

/* ------------------------------------------------------------- threading -- */

typedef void (*unit_fn)(void *ctx, long unit);

typedef struct {
    unit_fn fn;
    void *ctx;
    long begin, end;
} span_t;

static void *span_run(void *arg) {
    span_t *sp = (span_t *)arg;
    for (long u = sp->begin; u < sp->end; ++u) sp->fn(sp->ctx, u);
    return NULL;
}

/* Run fn over units [0, n) on nthreads threads (static contiguous split).
 * Also used by the ragged-format oracle. */
void orc_for_units(long n, int nthreads, unit_fn fn, void *ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    span_t *sp = (span_t *)calloc((size_t)nthreads, sizeof(span_t));
    for (int t = 0; t < nthreads; ++t) {
        sp[t].fn = fn;
        sp[t].ctx = ctx;
        sp[t].begin = n * t / nthreads;
        sp[t].end = n * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, span_run, &sp[t]);
    span_run(&sp[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(sp);
}

/* ------------------------------------------------------ batched entries -- */

static int check_shape(const orc_shape *s) {
    if (s->hv <= 0 || s->hk <= 0 || s->dk <= 0 || s->dv <= 0) return -1;
    if (s->hv % s->hk != 0) return -1;
    if (s->dv % 2 != 0) return -1;
    if (s->n8 < 0 || s->n8 > s->dk) return -1;
    return 0;
}

typedef struct {
    orc_shape s;
    const int8_t *pool8;
    const uint8_t *pool4;
    const float *r, *c;
    const int32_t *perm;
    double *S;
} dequant_ctx;

static void dequant_unit(void *vctx, long u) {
    dequant_ctx *x = (dequant_ctx *)vctx;
    const orc_shape *s = &x->s;
    int h = (int)(u % s->hv);
    unit_dequant(s, x->pool8 + u * unit8_bytes(s), x->pool4 + u * unit4_bytes(s),
                 x->r + u * s->dk, x->c + (size_t)h * s->dv, x->perm + (size_t)h * s->dk,
                 x->S + (size_t)u * s->dk * s->dv);
}

/* Dequantize B slots x Hv heads into logical-order double states
 * S[B][Hv][dk][dv] (Sec. 4.3 representation). Returns 0 on success. */
int oracle_dequant(int B, int hv, int dk, int dv, int n8, const int8_t *pool8,
                   const uint8_t *pool4, const float *r, const float *c,
                   const int32_t *perm, double *S, int nthreads) {
    dequant_ctx x = {{hv, 1, dk, dv, n8}, pool8, pool4, r, c, perm, S};
    if (check_shape(&x.s)) return -1;
    orc_for_units((long)B * hv, nthreads, dequant_unit, &x);
    return 0;
}

typedef struct {
    orc_shape s;
    const float *S;
    const float *c;
    const int32_t *perm;
    int8_t *pool8;
    uint8_t *pool4;
    float *r;
} pack_ctx;

static void pack_unit(void *vctx, long u) {
    pack_ctx *x = (pack_ctx *)vctx;
    const orc_shape *s = &x->s;
    int h = (int)(u % s->hv);
    size_t n = (size_t)s->dk * s->dv;
    double *X = (double *)malloc(n * sizeof(double));
    for (size_t e = 0; e < n; ++e) X[e] = (double)x->S[(size_t)u * n + e];
    unit_requant(s, X, x->c + (size_t)h * s->dv, x->perm + (size_t)h * s->dk,
                 x->pool8 + u * unit8_bytes(s), x->pool4 + u * unit4_bytes(s),
                 x->r + u * s->dk);
    free(X);
}

/* Pack fp32 logical-order states S[B][Hv][dk][dv] into the packed layout:
 * the requantization half of a decode step applied to a given state (the
 * prefill-boundary pack; Table C2 steps 4 and 6). */
int oracle_pack(int B, int hv, int dk, int dv, int n8, const float *S,
                const float *c, const int32_t *perm, int8_t *pool8,
                uint8_t *pool4, float *r, int nthreads) {
    pack_ctx x = {{hv, 1, dk, dv, n8}, S, c, perm, pool8, pool4, r};
    if (check_shape(&x.s)) return -1;
    orc_for_units((long)B * hv, nthreads, pack_unit, &x);
    return 0;
}

typedef struct {
    orc_shape s;
    const int8_t *pool8;
    const uint8_t *pool4;
    const float *r, *c;
    const int32_t *perm;
    const float *q, *k, *v, *alpha, *beta;
    int8_t *pool8_out;
    uint8_t *pool4_out;
    float *r_out, *o;
    double *X_out;
    const float *gate; /* [B][Hv][dk] row gate, or NULL for the scalar alpha */
} step_ctx;

static void step_unit(void *vctx, long u) {
    step_ctx *x = (step_ctx *)vctx;
    const orc_shape *s = &x->s;
    long b = u / s->hv;
    int h = (int)(u % s->hv);
    int hk = h / (s->hv / s->hk); /* reading R5 */
    size_t n = (size_t)s->dk * s->dv;
    double *S = (double *)calloc(n, sizeof(double));
    double *q = (double *)calloc((size_t)s->dk, sizeof(double));
    double *k = (double *)calloc((size_t)s->dk, sizeof(double));
    double *v = (double *)calloc((size_t)s->dv, sizeof(double));
    double *o = (double *)calloc((size_t)s->dv, sizeof(double));
    const float *c = x->c + (size_t)h * s->dv;
    const int32_t *perm = x->perm + (size_t)h * s->dk;

    /* Table C2 step 1: reconstruct. */
    unit_dequant(s, x->pool8 + u * unit8_bytes(s), x->pool4 + u * unit4_bytes(s),
                 x->r + u * s->dk, c, perm, S);
    for (int i = 0; i < s->dk; ++i) {
        q[i] = (double)x->q[((size_t)b * s->hk + hk) * s->dk + i];
        k[i] = (double)x->k[((size_t)b * s->hk + hk) * s->dk + i];
    }
    for (int j = 0; j < s->dv; ++j) v[j] = (double)x->v[(size_t)u * s->dv + j];
    /* Table C2 steps 2-3: update, then emit the readout of the updated state
     * before it is requantized. */
    orc_unit_update(s->dk, s->dv, S, q, k, v, x->alpha, x->gate, u, (double)x->beta[u], o);
    for (int j = 0; j < s->dv; ++j) x->o[(size_t)u * s->dv + j] = (float)o[j];
    if (x->X_out) memcpy(x->X_out + (size_t)u * n, S, n * sizeof(double));
    /* Table C2 steps 4 and 6: row factors, codes, pack. */
    unit_requant(s, S, c, perm, x->pool8_out + u * unit8_bytes(s),
                 x->pool4_out + u * unit4_bytes(s), x->r_out + u * s->dk);
    free(S);
    free(q);
    free(k);
    free(v);
    free(o);
}

/* One quantized decode step for B slots x Hv value heads (Table C2).
 * q, k: [B][Hk][dk]; v: [B][Hv][dv]; alpha, beta: [B][Hv]; o: [B][Hv][dv].
 * The *_out arrays receive the requantized state.  X_out (optional, may be
 * NULL) receives the updated, not yet requantized state in logical order as
 * doubles [B][Hv][dk][dv]. */
int oracle_step(int B, int hv, int hk, int dk, int dv, int n8,
                const int8_t *pool8, const uint8_t *pool4, const float *r,
                const float *c, const int32_t *perm, const float *q,
                const float *k, const float *v, const float *alpha,
                const float *beta, int8_t *pool8_out, uint8_t *pool4_out,
                float *r_out, float *o, double *X_out, int nthreads) {
    step_ctx x = {{hv, hk, dk, dv, n8}, pool8, pool4, r, c, perm, q, k, v,
                  alpha, beta, pool8_out, pool4_out, r_out, o, X_out, NULL};
    if (check_shape(&x.s)) return -1;
    orc_for_units((long)B * hv, nthreads, step_unit, &x);
    return 0;
}

/* oracle_step with the row gate gate[B][Hv][dk] (logical rows) in place of
 * the scalar alpha (Eq. (1) with a diagonal D_t). */
int oracle_step_gated(int B, int hv, int hk, int dk, int dv, int n8,
                      const int8_t *pool8, const uint8_t *pool4, const float *r,
                      const float *c, const int32_t *perm, const float *q,
                      const float *k, const float *v, const float *gate,
                      const float *beta, int8_t *pool8_out, uint8_t *pool4_out,
                      float *r_out, float *o, double *X_out, int nthreads) {
    step_ctx x = {{hv, hk, dk, dv, n8}, pool8, pool4, r, c, perm, q, k, v,
                  NULL, beta, pool8_out, pool4_out, r_out, o, X_out, gate};
    if (check_shape(&x.s) || !gate) return -1;
    orc_for_units((long)B * hv, nthreads, step_unit, &x);
    return 0;
}

typedef struct {
    orc_shape s;
    double *S;
    const float *q, *k, *v, *alpha, *beta;
    double *o;
    const float *gate;
} fp_ctx;

static void fp_unit(void *vctx, long u) {
    fp_ctx *x = (fp_ctx *)vctx;
    const orc_shape *s = &x->s;
    long b = u / s->hv;
    int h = (int)(u % s->hv);
    int hk = h / (s->hv / s->hk);
    double *q = (double *)calloc((size_t)s->dk, sizeof(double));
    double *k = (double *)calloc((size_t)s->dk, sizeof(double));
    double *v = (double *)calloc((size_t)s->dv, sizeof(double));
    for (int i = 0; i < s->dk; ++i) {
        q[i] = (double)x->q[((size_t)b * s->hk + hk) * s->dk + i];
        k[i] = (double)x->k[((size_t)b * s->hk + hk) * s->dk + i];
    }
    for (int j = 0; j < s->dv; ++j) v[j] = (double)x->v[(size_t)u * s->dv + j];
    orc_unit_update(s->dk, s->dv, x->S + (size_t)u * s->dk * s->dv, q, k, v, x->alpha, x->gate,
                u, (double)x->beta[u], x->o + (size_t)u * s->dv);
    free(q);
    free(k);
    free(v);
}

/* One unquantized gated delta-rule step on double states S[B][Hv][dk][dv]
 * (in place), readout into o[B][Hv][dv] (Sec. 2.1 Eq. (1), D_t = alpha I).
 * This is the full-precision reference the quantized path drifts from. */
int oracle_fp_step(int B, int hv, int hk, int dk, int dv, double *S,
                   const float *q, const float *k, const float *v,
                   const float *alpha, const float *beta, double *o,
                   int nthreads) {
    fp_ctx x = {{hv, hk, dk, dv, 0}, S, q, k, v, alpha, beta, o, NULL};
    if (check_shape(&x.s)) return -1;
    orc_for_units((long)B * hv, nthreads, fp_unit, &x);
    return 0;
}

/* oracle_fp_step with the row gate gate[B][Hv][dk] (logical rows). */
int oracle_fp_step_gated(int B, int hv, int hk, int dk, int dv, double *S,
                         const float *q, const float *k, const float *v,
                         const float *gate, const float *beta, double *o,
                         int nthreads) {
    fp_ctx x = {{hv, hk, dk, dv, 0}, S, q, k, v, NULL, beta, o, gate};
    if (check_shape(&x.s) || !gate) return -1;
    orc_for_units((long)B * hv, nthreads, fp_unit, &x);
    return 0;
}

/* ---------------------------------------------- per-state column factors -- */
/* The refit variant keeps one column-factor vector per state, cs[B][Hv][dv],
 * instead of one per head (App. C.1: the shared scales are refit to each
 * updated state; reading R14). */

typedef struct {
    orc_shape s;
    const int8_t *pool8;
    const uint8_t *pool4;
    const float *r, *cs;
    const int32_t *perm;
    double *S;
} dequant_cs_ctx;

static void dequant_cs_unit(void *vctx, long u) {
    dequant_cs_ctx *x = (dequant_cs_ctx *)vctx;
    const orc_shape *s = &x->s;
    int h = (int)(u % s->hv);
    unit_dequant(s, x->pool8 + u * unit8_bytes(s), x->pool4 + u * unit4_bytes(s),
                 x->r + u * s->dk, x->cs + (size_t)u * s->dv, x->perm + (size_t)h * s->dk,
                 x->S + (size_t)u * s->dk * s->dv);
}

/* Dequantize states whose column factors are per state (cs[B][Hv][dv]). */
int oracle_dequant_cs(int B, int hv, int dk, int dv, int n8, const int8_t *pool8,
                      const uint8_t *pool4, const float *r, const float *cs,
                      const int32_t *perm, double *S, int nthreads) {
    dequant_cs_ctx x = {{hv, 1, dk, dv, n8}, pool8, pool4, r, cs, perm, S};
    if (check_shape(&x.s)) return -1;
    orc_for_units((long)B * hv, nthreads, dequant_cs_unit, &x);
    return 0;
}

typedef struct {
    orc_shape s;
    const float *S;
    const float *c0;
    const int32_t *perm;
    const float *w2;
    int8_t *pool8;
    uint8_t *pool4;
    float *r, *cs;
} pack_refit_ctx;

static void pack_refit_unit(void *vctx, long u) {
    pack_refit_ctx *x = (pack_refit_ctx *)vctx;
    const orc_shape *s = &x->s;
    int h = (int)(u % s->hv);
    size_t n = (size_t)s->dk * s->dv;
    double *X = (double *)malloc(n * sizeof(double));
    for (size_t e = 0; e < n; ++e) X[e] = (double)x->S[(size_t)u * n + e];
    float *c = x->cs + (size_t)u * s->dv;
    memcpy(c, x->c0 + (size_t)h * s->dv, (size_t)s->dv * sizeof(float));
    const int32_t *perm = x->perm + (size_t)h * s->dk;
    int8_t *p8 = x->pool8 + u * unit8_bytes(s);
    uint8_t *p4 = x->pool4 + u * unit4_bytes(s);
    float *r = x->r + u * s->dk;
    unit_requant(s, X, c, perm, p8, p4, r);
    unit_refit(s, X, perm, x->w2 + (size_t)h * s->dk, p8, p4, r, c);
    free(X);
}

/* Pack fp32 states with the refit: codes and row factors against the
 * calibrated column factors c0[Hv][dv], then each state's own column factors
 * refit to it (Table C2 steps 4-6 applied to a given state). */
int oracle_pack_refit(int B, int hv, int dk, int dv, int n8, const float *S,
                      const float *c0, const int32_t *perm, const float *w2,
                      int8_t *pool8, uint8_t *pool4, float *r, float *cs,
                      int nthreads) {
    pack_refit_ctx x = {{hv, 1, dk, dv, n8}, S, c0, perm, w2, pool8, pool4, r, cs};
    if (check_shape(&x.s)) return -1;
    orc_for_units((long)B * hv, nthreads, pack_refit_unit, &x);
    return 0;
}

typedef struct {
    orc_shape s;
    const int8_t *pool8;
    const uint8_t *pool4;
    const float *r, *cs;
    const int32_t *perm;
    const float *w2;
    const float *q, *k, *v, *alpha, *beta;
    int8_t *pool8_out;
    uint8_t *pool4_out;
    float *r_out, *cs_out, *o;
    double *X_out;
    const float *gate;
} step_refit_ctx;

static void step_refit_unit(void *vctx, long u) {
    step_refit_ctx *x = (step_refit_ctx *)vctx;
    const orc_shape *s = &x->s;
    long b = u / s->hv;
    int h = (int)(u % s->hv);
    int hk = h / (s->hv / s->hk); /* reading R5 */
    size_t n = (size_t)s->dk * s->dv;
    double *S = (double *)calloc(n, sizeof(double));
    double *q = (double *)calloc((size_t)s->dk, sizeof(double));
    double *k = (double *)calloc((size_t)s->dk, sizeof(double));
    double *v = (double *)calloc((size_t)s->dv, sizeof(double));
    double *o = (double *)calloc((size_t)s->dv, sizeof(double));
    const int32_t *perm = x->perm + (size_t)h * s->dk;
    float *c = x->cs_out + (size_t)u * s->dv;
    memcpy(c, x->cs + (size_t)u * s->dv, (size_t)s->dv * sizeof(float));

    /* Table C2 step 1: reconstruct with this state's own column factors. */
    unit_dequant(s, x->pool8 + u * unit8_bytes(s), x->pool4 + u * unit4_bytes(s),
                 x->r + u * s->dk, c, perm, S);
    for (int i = 0; i < s->dk; ++i) {
        q[i] = (double)x->q[((size_t)b * s->hk + hk) * s->dk + i];
        k[i] = (double)x->k[((size_t)b * s->hk + hk) * s->dk + i];
    }
    for (int j = 0; j < s->dv; ++j) v[j] = (double)x->v[(size_t)u * s->dv + j];
    /* Table C2 steps 2-3. */
    orc_unit_update(s->dk, s->dv, S, q, k, v, x->alpha, x->gate, u, (double)x->beta[u], o);
    for (int j = 0; j < s->dv; ++j) x->o[(size_t)u * s->dv + j] = (float)o[j];
    if (x->X_out) memcpy(x->X_out + (size_t)u * n, S, n * sizeof(double));
    /* Table C2 step 4: row factors and codes against the current column
     * factors; step 5: refit the column factors to the codes; step 6: store. */
    int8_t *p8 = x->pool8_out + u * unit8_bytes(s);
    uint8_t *p4 = x->pool4_out + u * unit4_bytes(s);
    float *r = x->r_out + u * s->dk;
    unit_requant(s, S, c, perm, p8, p4, r);
    unit_refit(s, S, perm, x->w2 + (size_t)h * s->dk, p8, p4, r, c);
    free(S);
    free(q);
    free(k);
    free(v);
    free(o);
}

/* One quantized decode step with per-state column factors and the online
 * column refit (Table C2 steps 1-6).  cs / cs_out: [B][Hv][dv]; w2:
 * [Hv][dk] squared row-impact weights in logical row order. */
int oracle_step_refit(int B, int hv, int hk, int dk, int dv, int n8,
                      const int8_t *pool8, const uint8_t *pool4, const float *r,
                      const float *cs, const int32_t *perm, const float *w2,
                      const float *q, const float *k, const float *v,
                      const float *alpha, const float *beta, int8_t *pool8_out,
                      uint8_t *pool4_out, float *r_out, float *cs_out, float *o,
                      double *X_out, int nthreads) {
    step_refit_ctx x = {{hv, hk, dk, dv, n8}, pool8, pool4, r, cs, perm, w2, q, k, v,
                        alpha, beta, pool8_out, pool4_out, r_out, cs_out, o, X_out, NULL};
    if (check_shape(&x.s)) return -1;
    orc_for_units((long)B * hv, nthreads, step_refit_unit, &x);
    return 0;
}

/* oracle_step_refit with the row gate gate[B][Hv][dk] (logical rows). */
int oracle_step_refit_gated(int B, int hv, int hk, int dk, int dv, int n8,
                            const int8_t *pool8, const uint8_t *pool4, const float *r,
                            const float *cs, const int32_t *perm, const float *w2,
                            const float *q, const float *k, const float *v,
                            const float *gate, const float *beta, int8_t *pool8_out,
                            uint8_t *pool4_out, float *r_out, float *cs_out, float *o,
                            double *X_out, int nthreads) {
    step_refit_ctx x = {{hv, hk, dk, dv, n8}, pool8, pool4, r, cs, perm, w2, q, k, v,
                        NULL, beta, pool8_out, pool4_out, r_out, cs_out, o, X_out, gate};
    if (check_shape(&x.s) || !gate) return -1;
    orc_for_units((long)B * hv, nthreads, step_refit_unit, &x);
    return 0;
}

/* Row impact (Sec. 4.1; App. C.1 with the scalar gate of reading R4): the
 * readout error caused by an error in key row i of the previous state is
 * carried by g_i = (A_t^T q_t)_i = alpha (q_i - beta k_i (k.q)), and
 * omega_i = E[g_i^2] over calibration samples.  omega[Hv][dk] (logical rows)
 * accumulates sum over the B samples of g_i^2 for every value head. */
static int impact_accumulate(int B, int hv, int hk, int dk, const float *q,
                             const float *k, const float *alpha, const float *gate,
                             const float *beta, double *omega) {
    if (hv <= 0 || hk <= 0 || hv % hk != 0 || dk <= 0) return -1;
    for (long b = 0; b < B; ++b)
        for (int h = 0; h < hv; ++h) {
            int g = h / (hv / hk);
            const float *qq = q + ((size_t)b * hk + g) * dk;
            const float *kk = k + ((size_t)b * hk + g) * dk;
            double kq = 0.0;
            for (int i = 0; i < dk; ++i) kq += (double)kk[i] * (double)qq[i];
            double be = (double)beta[(size_t)b * hv + h];
            for (int i = 0; i < dk; ++i) {
                double a = gate ? (double)gate[((size_t)b * hv + h) * dk + i]
                                : (double)alpha[(size_t)b * hv + h];
                double gi = a * ((double)qq[i] - be * (double)kk[i] * kq);
                omega[(size_t)h * dk + i] += gi * gi;
            }
        }
    return 0;
}

int oracle_impact_accumulate(int B, int hv, int hk, int dk, const float *q,
                             const float *k, const float *alpha,
                             const float *beta, double *omega) {
    return impact_accumulate(B, hv, hk, dk, q, k, alpha, NULL, beta, omega);
}

/* The same with the row gate (App. C.1: g_i = d_i (q_i - beta k_i k.q)),
 * gate[B][Hv][dk] in logical row order. */
int oracle_impact_accumulate_gated(int B, int hv, int hk, int dk, const float *q,
                                   const float *k, const float *gate,
                                   const float *beta, double *omega) {
    if (!gate) return -1;
    return impact_accumulate(B, hv, hk, dk, q, k, NULL, gate, beta, omega);
}

/* Squared row-impact weights from the accumulated omega (App. B.3: the row
 * factor scales as omega^(1/8), so its square as omega^(1/4); the per-head
 * normalisation cancels in the fit): w2_i = fl32((omega_i / mean omega)^(1/4))
 * floored at 2^-32; a head whose omega is all zero gets w2 = 1. */
int oracle_impact_weights(int hv, int dk, const double *omega, float *w2) {
    const double floor_w = ldexp(1.0, -32);
    for (int h = 0; h < hv; ++h) {
        double mean = 0.0;
        for (int i = 0; i < dk; ++i) mean += omega[(size_t)h * dk + i];
        mean /= (double)dk;
        for (int i = 0; i < dk; ++i) {
            double w = 1.0;
            if (mean > 0.0) {
                w = (double)(float)pow(omega[(size_t)h * dk + i] / mean, 0.25);
                if (w < floor_w) w = floor_w;
            }
            w2[(size_t)h * dk + i] = (float)w;
        }
    }
    return 0;
}

/* ------------------------------------------------------------ calibration -- */
/* Offline calibration for the fixed column factor and the 4/8-bit row split
 * (Sec. 3.2 and Sec. 4.4: precision map and scales are fixed offline across
 * requests; App. A.3: each batch element of a calibration step counts as one
 * sample).  The concrete rule is the reading taken for this path:
 *   c_j   = max over every recorded state and every row of |S_ij| (0 -> 1)
 *   score = sum over recorded states of sum_j S_ij^2   (per head, per row)
 *   the n8 highest-score rows become 8-bit, ties going to the lower row. */

/* colmax[h][j] = max(colmax[h][j], max over records and rows of |S|). */
int oracle_calib_cols(long n_rec, int hv, int dk, int dv, const double *S,
                      double *colmax) {
    for (long rec = 0; rec < n_rec; ++rec)
        for (int h = 0; h < hv; ++h)
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) {
                    double a = fabs(S[(((size_t)rec * hv + h) * dk + i) * dv + j]);
                    if (a > colmax[(size_t)h * dv + j]) colmax[(size_t)h * dv + j] = a;
                }
    return 0;
}

/* rowscore[h][i] += sum over records and columns of S_ij^2. */
int oracle_calib_rows(long n_rec, int hv, int dk, int dv, const double *S,
                      double *rowscore) {
    for (long rec = 0; rec < n_rec; ++rec)
        for (int h = 0; h < hv; ++h)
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) {
                    double x = S[(((size_t)rec * hv + h) * dk + i) * dv + j];
                    acc += x * x;
                }
                rowscore[(size_t)h * dk + i] += acc;
            }
    return 0;
}

/* c = colmax (a zero column gets 1); perm lists the n8 selected rows in
 * ascending order, then the remaining rows in ascending order.  Row i is
 * selected when fewer than n8 rows beat it, where row a beats row b if
 * score_a > score_b, or the scores are equal and a < b. */
int oracle_calib_finalize(int hv, int dk, int dv, int n8, const double *colmax,
                          const double *rowscore, float *c, int32_t *perm) {
    if (n8 < 0 || n8 > dk) return -1;
    int *sel = (int *)malloc((size_t)dk * sizeof(int));
    for (int h = 0; h < hv; ++h) {
        for (int j = 0; j < dv; ++j) {
            double m = colmax[(size_t)h * dv + j];
            c[(size_t)h * dv + j] = (m > 0.0) ? (float)m : 1.0f;
        }
        const double *sc = &rowscore[(size_t)h * dk];
        for (int i = 0; i < dk; ++i) {
            int beaten_by = 0;
            for (int a = 0; a < dk; ++a)
                if (sc[a] > sc[i] || (sc[a] == sc[i] && a < i)) ++beaten_by;
            sel[i] = beaten_by < n8;
        }
        int p = 0;
        for (int i = 0; i < dk; ++i)
            if (sel[i]) perm[(size_t)h * dk + p++] = i;
        for (int i = 0; i < dk; ++i)
            if (!sel[i]) perm[(size_t)h * dk + p++] = i;
    }
    free(sel);
    return 0;
}
