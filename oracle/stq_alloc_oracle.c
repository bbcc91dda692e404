/*
 * stq_alloc_oracle.c -- CPU oracle for the ragged row-class format (FP16
 * pivot rows and per-row bit widths from {2, 4, 6, 8}) and for the offline
 * lifetime-aware bit allocation that chooses them.
 *
 * TEST INFRASTRUCTURE ONLY, under the same rules as stq_oracle.c: nothing in
 * the product path links, loads or calls it; it shares nothing with the HIP
 * library and carries its own reader and writer of the documented layout.
 *
 * Sources (STEPQuant paper, "STEPQuant: When and Where Errors Matter in
 * Delta-Rule Recurrent State Quantization", arXiv 2609.38169):
 *   - FP16 pivots and the candidate widths {2,4,6,8} (4-bit budget) and
 *     {4,6,8} (6-bit budget):            App. C.2, Table C1
 *   - one decode step with pivots:        App. C.3, Table C2 (step 1 pivots
 *                                         reconstructed from FP16 values,
 *                                         step 5 column fit over non-pivot
 *                                         integer rows, step 6 pivots stored
 *                                         in FP16)
 *   - mean log retention and lifetime weight:
 *                                         App. A.3 "Mean log retention"
 *                                         (ell_u, L_u); Sec. 3.2
 *   - candidate distortion:               App. A.3 "KDA reconstruction
 *                                         distortion" (unweighted MSE of the
 *                                         candidate reconstruction)
 *   - pivot ranking:                      App. C.2 "KDA calibration"
 *                                         (lifetime-weighted reduction from
 *                                         integer to FP16 error)
 *   - allocation:                         App. C.2 "Allocation optimizers"
 *                                         (Lagrangian per unit with a shared
 *                                         multiplier, then a repair to meet
 *                                         the integer budget)
 *
 * Readings (listed with the others in the design notes):
 *   R17 per head, physical rows are sorted into classes k = 0..4 of widths
 *       16 (FP16 pivot), 8, 6, 4, 2 bits; counts[h][k] rows of class k; perm
 *       gives the logical row of each physical row.  A head's rows form one
 *       segment of the slot's byte pool: class 0 rows (2d bytes each), then
 *       class 1 (d), class 2 (3d/4), class 3 (d/2), class 4 (d/4); the
 *       segment is padded to a multiple of 16 bytes and the heads follow each
 *       other in order.  A slot occupies slot_bytes bytes of the pool.
 *   R18 a pivot row stores X in IEEE binary16, rounded to nearest even and
 *       saturated at +-65504; it has no row factor (r is written as 0) and no
 *       column factor, and it takes no part in the column refit.
 *   R19 integer rows use the quantizer of stq_oracle.c with q_b = 2^(b-1)-1
 *       (127, 31, 7, 1).  6-bit codes: two's complement in 6 bits; the low
 *       four bits of column j sit in nibble j of the row's first d/2 bytes
 *       (even column in the low nibble), the top two bits in the 2-bit field
 *       j of the next d/4 bytes.  2-bit codes (levels -1, 0, 1): two's
 *       complement in 2 bits, column j in bits 2(j%4)..2(j%4)+1 of byte j/4.
 *   R20 candidate distortion: d_u(b) = sum over records and columns of
 *       (S^(b) - S)^2 for row u, with S^(b) the row quantized at width b
 *       against the head's fixed column factors (b = 16: rounded to FP16).
 *       The 1/(|C| n_u) normalisation of the paper is left out: it is the
 *       same for every unit and does not change the assignment.
 *   R21 retention: ell_u = mean over calibration samples of log(retention);
 *       the scalar gate gives log(alpha) to every row of its head, the row
 *       gate log(d_i).  L_u = 1 + sum_{j=1}^{H-1} exp(2 j ell_u).
 *   R22 pivots: the P units of largest L_u (d_u(b_nom) - d_u(16)) over all
 *       heads (ties to the lower unit index u = h d + i), b_nom the nominal
 *       width.
 *   R23 assignment: every other unit starts at the smallest candidate.  Its
 *       candidates form points (b, L_u d_u(b)); only the lower convex hull
 *       counts, and only hull segments that lower the distortion.  Segments
 *       of all units are taken in order of decreasing distortion saved per
 *       bit (ties: lower unit, then lower width), each while the integer
 *       budget b_nom * (number of non-pivot units) still holds: up to the
 *       first segment that does not fit this is the Lagrangian solution of a
 *       shared multiplier; after it, a unit whose next segment does not fit
 *       keeps its width (the repair) and later segments that fit are taken.
 *       Physical order: pivots, then 8-, 6-, 4-, 2-bit rows, each class in
 *       ascending logical row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* from stq_oracle.c (same library) */
double oracle_rhe(double y);
typedef void (*unit_fn)(void *ctx, long unit);
void orc_for_units(long n, int nthreads, unit_fn fn, void *ctx);
void orc_unit_update(int dk, int dv, double *S, const double *q, const double *k,
                     const double *v, const float *alpha, const float *gate, long u,
                     double beta, double *o);

enum { NCLS = 5 };
static const int kBits[NCLS] = {16, 8, 6, 4, 2};

/* ---------------------------------------------------------------- binary16 -- */

/* IEEE binary16 from a double: round to nearest even, saturate at +-65504
 * (reading R18).  Written from the format's definition: 11 significant bits
 * for normal numbers, a fixed quantum of 2^-24 below 2^-14. */
uint16_t oracle_f16_from_double(double x) {
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isnan(x)) return 0x7E00u;
    if (a >= 65504.0) return (uint16_t)(sign | 0x7BFFu);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e); /* a = m 2^e, 0.5 <= m < 1 */
    int qe = e - 11;
    if (qe < -24) qe = -24;
    double n = oracle_rhe(ldexp(a, -qe)); /* integer count of quanta, exact scaling */
    double v = ldexp(n, qe);
    if (v >= 65504.0) return (uint16_t)(sign | 0x7BFFu);
    if (v < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)n); /* subnormal: n < 1024 */
    int e2;
    double m = frexp(v, &e2);             /* v = m 2^e2 */
    int E = e2 - 1 + 15;                  /* biased exponent */
    uint16_t mant = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)(E << 10) | mant);
}

double oracle_f16_to_double(uint16_t h) {
    int E = (h >> 10) & 0x1F, M = h & 0x3FF;
    double s = (h & 0x8000u) ? -1.0 : 1.0;
    if (E == 0) return s * ldexp((double)M, -24);
    if (E == 31) return M ? NAN : s * INFINITY;
    return s * ldexp(1024.0 + (double)M, E - 25);
}

/* ------------------------------------------------------------------ layout -- */

static int row_bytes(int k, int d) {
    switch (k) {
    case 0: return 2 * d;
    case 1: return d;
    case 2: return 3 * d / 4;
    case 3: return d / 2;
    default: return d / 4;
    }
}

typedef struct {
    int cls[128 * 4];     /* class of each physical row (d <= 512) */
    long row_off[128 * 4]; /* byte offset of each physical row in the segment */
    long seg;             /* segment bytes (padded to 16) */
} head_layout;

/* Class and offset of every physical row of one head (reading R17). */
static void layout_head(int d, const int32_t *cnt, head_layout *L) {
    long off = 0;
    int p = 0;
    for (int k = 0; k < NCLS; ++k)
        for (int n = 0; n < cnt[k]; ++n, ++p) {
            L->cls[p] = k;
            L->row_off[p] = off;
            off += row_bytes(k, d);
        }
    L->seg = (off + 15) / 16 * 16;
}

/* Byte offset of every head's segment within a slot; returns the bytes a
 * slot needs (sum of segments), or -1 for counts that do not sum to d. */
long oracle_alloc_layout(int hv, int d, const int32_t *counts, int64_t *head_off) {
    long off = 0;
    for (int h = 0; h < hv; ++h) {
        int sum = 0;
        for (int k = 0; k < NCLS; ++k) {
            if (counts[h * NCLS + k] < 0) return -1;
            sum += counts[h * NCLS + k];
        }
        if (sum != d) return -1;
        head_layout L;
        layout_head(d, counts + h * NCLS, &L);
        if (head_off) head_off[h] = off;
        off += L.seg;
    }
    return off;
}

/* Read the integer code of column j of an integer row (reading R19). */
static int read_int_code(const uint8_t *row, int k, int d, int j) {
    switch (k) {
    case 1: return (int)(int8_t)row[j];
    case 2: {
        int lo = (j % 2 == 0) ? (row[j / 2] & 0x0F) : (row[j / 2] >> 4);
        int hi = (row[d / 2 + j / 4] >> (2 * (j % 4))) & 0x3;
        int u = lo | (hi << 4);
        return u >= 32 ? u - 64 : u;
    }
    case 3: {
        int nib = (j % 2 == 0) ? (row[j / 2] & 0x0F) : (row[j / 2] >> 4);
        return nib >= 8 ? nib - 16 : nib;
    }
    default: {
        int u = (row[j / 4] >> (2 * (j % 4))) & 0x3;
        return u >= 2 ? u - 4 : u;
    }
    }
}

static void write_int_code(uint8_t *row, int k, int d, int j, int z) {
    switch (k) {
    case 1: row[j] = (uint8_t)(int8_t)z; return;
    case 2: {
        int u = z & 0x3F;
        uint8_t *b = &row[j / 2];
        if (j % 2 == 0) *b = (uint8_t)((*b & 0xF0) | (u & 0x0F));
        else *b = (uint8_t)((*b & 0x0F) | ((u & 0x0F) << 4));
        uint8_t *hb = &row[d / 2 + j / 4];
        int sh = 2 * (j % 4);
        *hb = (uint8_t)((*hb & ~(0x3 << sh)) | (((u >> 4) & 0x3) << sh));
        return;
    }
    case 3: {
        uint8_t *b = &row[j / 2];
        uint8_t nib = (uint8_t)(z & 0x0F);
        if (j % 2 == 0) *b = (uint8_t)((*b & 0xF0) | nib);
        else *b = (uint8_t)((*b & 0x0F) | (nib << 4));
        return;
    }
    default: {
        uint8_t *b = &row[j / 4];
        int sh = 2 * (j % 4);
        *b = (uint8_t)((*b & ~(0x3 << sh)) | ((z & 0x3) << sh));
        return;
    }
    }
}

static int qmax_of(int k) { return (1 << (kBits[k] - 1)) - 1; }

/* ------------------------------------------------------- unit operations -- */

/* S (logical order, doubles) of one head from its segment (reading R17, R18;
 * Table C2 step 1): integer rows r_p c_j z_pj, pivot rows their FP16 values. */
static void seg_dequant(int d, const head_layout *L, const uint8_t *seg, const float *r,
                        const float *c, const int32_t *perm, double *S) {
    for (int p = 0; p < d; ++p) {
        int i = perm[p];
        const uint8_t *row = seg + L->row_off[p];
        for (int j = 0; j < d; ++j) {
            double x;
            if (L->cls[p] == 0) {
                uint16_t h = (uint16_t)(row[2 * j] | (row[2 * j + 1] << 8));
                x = oracle_f16_to_double(h);
            } else {
                x = ((double)r[p] * (double)c[j]) * (double)read_int_code(row, L->cls[p], d, j);
            }
            S[(size_t)i * d + j] = x;
        }
    }
}

/* Requantize X (logical order) into one head's segment (Sec. 2.2; Sec. 4.3;
 * Table C2 steps 4 and 6; readings R2, R6, R18, R19). */
static void seg_requant(int d, const head_layout *L, const double *X, const float *c,
                        const int32_t *perm, uint8_t *seg, float *r_out) {
    const double floor_r = ldexp(1.0, -126);
    for (int p = 0; p < d; ++p) {
        int i = perm[p];
        const double *row = &X[(size_t)i * d];
        uint8_t *dst = seg + L->row_off[p];
        if (L->cls[p] == 0) {
            for (int j = 0; j < d; ++j) {
                uint16_t h = oracle_f16_from_double(row[j]);
                dst[2 * j] = (uint8_t)(h & 0xFF);
                dst[2 * j + 1] = (uint8_t)(h >> 8);
            }
            r_out[p] = 0.0f;
            continue;
        }
        int qb = qmax_of(L->cls[p]);
        double m = 0.0;
        for (int j = 0; j < d; ++j) {
            double x = row[j] / (double)c[j];
            if (fabs(x) > m) m = fabs(x);
        }
        double rr = (double)(float)(m / (double)qb);
        if (rr < floor_r) rr = floor_r;
        r_out[p] = (float)rr;
        for (int j = 0; j < d; ++j) {
            double z = oracle_rhe((row[j] / (double)c[j]) / rr);
            if (z > qb) z = qb;
            if (z < -qb) z = -qb;
            write_int_code(dst, L->cls[p], d, j, (int)z);
        }
    }
}

/* Column refit over the non-pivot integer rows (App. C.1 fixed-code update;
 * Table C2 step 5; readings R14, R18). */
static void seg_refit(int d, const head_layout *L, const double *X, const int32_t *perm,
                      const float *w2, const uint8_t *seg, const float *r, float *c) {
    const double floor_c = ldexp(1.0, -126);
    for (int j = 0; j < d; ++j) {
        double num = 0.0, den = 0.0;
        for (int p = 0; p < d; ++p) {
            if (L->cls[p] == 0) continue;
            int i = perm[p];
            double vij = (double)r[p] * (double)read_int_code(seg + L->row_off[p], L->cls[p], d, j);
            double wt = (double)w2[i];
            num += wt * vij * X[(size_t)i * d + j];
            den += wt * vij * vij;
        }
        if (den > 0.0) {
            double cn = (double)(float)(num / den);
            if (cn < floor_c) cn = floor_c;
            c[j] = (float)cn;
        }
    }
}

/* ------------------------------------------------------- batched entries -- */

typedef struct {
    int hv, hk, d;
    long slot_bytes;
    const int32_t *counts, *perm;
    const int64_t *head_off;
    const uint8_t *pool;
    const float *r, *c, *cs, *w2;
    const float *q, *k, *v, *alpha, *gate, *beta;
    const double *S_in;
    uint8_t *pool_out;
    float *r_out, *cs_out, *o;
    double *S_out, *X_out;
} alloc_ctx;

static int alloc_check(int hv, int hk, int d, long slot_bytes, const int32_t *counts,
                       int64_t *head_off) {
    if (hv <= 0 || hk <= 0 || hv % hk != 0) return -1;
    if (d != 16 && d != 32 && d != 64 && d != 128) return -1;
    long need = oracle_alloc_layout(hv, d, counts, head_off);
    if (need < 0 || need > slot_bytes) return -1;
    return 0;
}

/* column factors of unit u: the state's own (refit) or the head's */
static const float *unit_c(const alloc_ctx *x, long u) {
    int h = (int)(u % x->hv);
    return x->cs ? x->cs + (size_t)u * x->d : x->c + (size_t)h * x->d;
}

static void alloc_dequant_unit(void *vctx, long u) {
    alloc_ctx *x = (alloc_ctx *)vctx;
    long b = u / x->hv;
    int h = (int)(u % x->hv);
    head_layout L;
    layout_head(x->d, x->counts + h * NCLS, &L);
    seg_dequant(x->d, &L, x->pool + b * x->slot_bytes + x->head_off[h], x->r + u * x->d,
                unit_c(x, u), x->perm + (size_t)h * x->d, x->S_out + (size_t)u * x->d * x->d);
}

/* Reconstruct B slots (slot = batch index) into S [B][Hv][d][d] (logical
 * order).  cs (per state [B][Hv][d]) replaces c (per head) when not NULL. */
int oracle_alloc_dequant(int B, int hv, int d, long slot_bytes, const int32_t *counts,
                         const int32_t *perm, const uint8_t *pool, const float *r,
                         const float *c, const float *cs, double *S, int nthreads) {
    int64_t *ho = (int64_t *)calloc((size_t)hv, sizeof(int64_t));
    if (alloc_check(hv, 1, d, slot_bytes, counts, ho)) { free(ho); return -1; }
    alloc_ctx x;
    memset(&x, 0, sizeof x);
    x.hv = hv; x.hk = 1; x.d = d; x.slot_bytes = slot_bytes; x.counts = counts; x.perm = perm;
    x.head_off = ho; x.pool = pool; x.r = r; x.c = c; x.cs = cs; x.S_out = S;
    orc_for_units((long)B * hv, nthreads, alloc_dequant_unit, &x);
    free(ho);
    return 0;
}

static void alloc_pack_unit(void *vctx, long u) {
    alloc_ctx *x = (alloc_ctx *)vctx;
    long b = u / x->hv;
    int h = (int)(u % x->hv);
    int d = x->d;
    head_layout L;
    layout_head(d, x->counts + h * NCLS, &L);
    uint8_t *seg = x->pool_out + b * x->slot_bytes + x->head_off[h];
    const double *S = x->S_in + (size_t)u * d * d;
    float *r = x->r_out + u * d;
    const int32_t *perm = x->perm + (size_t)h * d;
    const float *c = x->c + (size_t)h * d;
    if (!x->cs_out) {
        seg_requant(d, &L, S, c, perm, seg, r);
        return;
    }
    /* refit variant: codes against the head's c, then this state's c fit */
    float *cs = x->cs_out + (size_t)u * d;
    memcpy(cs, c, (size_t)d * sizeof(float));
    seg_requant(d, &L, S, cs, perm, seg, r);
    seg_refit(d, &L, S, perm, x->w2 + (size_t)h * d, seg, r, cs);
}

/* Pack S [B][Hv][d][d] (logical order) into slots 0..B-1 of pool (reading
 * R17-R19).  With cs_out (refit format) the codes are taken against the
 * head's c and each state's column factors are then refit (weights w2). */
int oracle_alloc_pack(int B, int hv, int d, long slot_bytes, const int32_t *counts,
                      const int32_t *perm, const double *S, const float *c, const float *w2,
                      uint8_t *pool, float *r, float *cs_out, int nthreads) {
    int64_t *ho = (int64_t *)calloc((size_t)hv, sizeof(int64_t));
    if (alloc_check(hv, 1, d, slot_bytes, counts, ho)) { free(ho); return -1; }
    if (cs_out && !w2) { free(ho); return -1; }
    alloc_ctx x;
    memset(&x, 0, sizeof x);
    x.hv = hv; x.hk = 1; x.d = d; x.slot_bytes = slot_bytes; x.counts = counts; x.perm = perm;
    x.head_off = ho; x.S_in = S; x.c = c; x.w2 = w2; x.pool_out = pool; x.r_out = r;
    x.cs_out = cs_out;
    orc_for_units((long)B * hv, nthreads, alloc_pack_unit, &x);
    free(ho);
    return 0;
}

static void alloc_step_unit(void *vctx, long u) {
    alloc_ctx *x = (alloc_ctx *)vctx;
    int d = x->d;
    long b = u / x->hv;
    int h = (int)(u % x->hv);
    int hk = h / (x->hv / x->hk); /* reading R5 */
    size_t n = (size_t)d * d;
    double *S = (double *)calloc(n, sizeof(double));
    double *q = (double *)calloc((size_t)d, sizeof(double));
    double *k = (double *)calloc((size_t)d, sizeof(double));
    double *v = (double *)calloc((size_t)d, sizeof(double));
    double *o = (double *)calloc((size_t)d, sizeof(double));
    head_layout L;
    layout_head(d, x->counts + h * NCLS, &L);
    const int32_t *perm = x->perm + (size_t)h * d;
    const uint8_t *seg_in = x->pool + b * x->slot_bytes + x->head_off[h];
    uint8_t *seg_out = x->pool_out + b * x->slot_bytes + x->head_off[h];
    float *c;
    if (x->cs) {
        c = x->cs_out + (size_t)u * d;
        memcpy(c, x->cs + (size_t)u * d, (size_t)d * sizeof(float));
    } else {
        c = (float *)(x->c + (size_t)h * d); /* read only below */
    }
    /* Table C2 step 1: reconstruct (pivot rows from FP16). */
    seg_dequant(d, &L, seg_in, x->r + u * d, c, perm, S);
    for (int i = 0; i < d; ++i) {
        q[i] = (double)x->q[((size_t)b * x->hk + hk) * d + i];
        k[i] = (double)x->k[((size_t)b * x->hk + hk) * d + i];
    }
    for (int j = 0; j < d; ++j) v[j] = (double)x->v[(size_t)u * d + j];
    /* Table C2 steps 2-3: update with either gate, readout before requant. */
    orc_unit_update(d, d, S, q, k, v, x->alpha, x->gate, u, (double)x->beta[u], o);
    for (int j = 0; j < d; ++j) x->o[(size_t)u * d + j] = (float)o[j];
    if (x->X_out) memcpy(x->X_out + (size_t)u * n, S, n * sizeof(double));
    /* Table C2 steps 4-6: row factors and codes; refit over integer rows;
     * pivots stored in FP16. */
    memset(seg_out, 0, (size_t)L.seg);
    seg_requant(d, &L, S, c, perm, seg_out, x->r_out + u * d);
    if (x->cs) seg_refit(d, &L, S, perm, x->w2 + (size_t)h * d, seg_out, x->r_out + u * d, c);
    free(S);
    free(q);
    free(k);
    free(v);
    free(o);
}

/* One decode step on the ragged format for B slots x Hv value heads (Table
 * C2).  Exactly one of alpha [B][Hv] and gate [B][Hv][d] (logical rows) is
 * given.  Fixed column factors c [Hv][d], or per-state cs [B][Hv][d] with
 * the refit (then w2 [Hv][d] and cs_out are required).  X_out may be NULL. */
int oracle_alloc_step(int B, int hv, int hk, int d, long slot_bytes, const int32_t *counts,
                      const int32_t *perm, const uint8_t *pool, const float *r,
                      const float *c, const float *cs, const float *w2, const float *q,
                      const float *k, const float *v, const float *alpha, const float *gate,
                      const float *beta, uint8_t *pool_out, float *r_out, float *cs_out,
                      float *o, double *X_out, int nthreads) {
    int64_t *ho = (int64_t *)calloc((size_t)hv, sizeof(int64_t));
    if (alloc_check(hv, hk, d, slot_bytes, counts, ho)) { free(ho); return -1; }
    if ((alpha == NULL) == (gate == NULL)) { free(ho); return -1; }
    if (cs && (!w2 || !cs_out)) { free(ho); return -1; }
    if (!cs && !c) { free(ho); return -1; }
    alloc_ctx x;
    memset(&x, 0, sizeof x);
    x.hv = hv; x.hk = hk; x.d = d; x.slot_bytes = slot_bytes; x.counts = counts; x.perm = perm;
    x.head_off = ho; x.pool = pool; x.r = r; x.c = c; x.cs = cs; x.w2 = w2;
    x.q = q; x.k = k; x.v = v; x.alpha = alpha; x.gate = gate; x.beta = beta;
    x.pool_out = pool_out; x.r_out = r_out; x.cs_out = cs_out; x.o = o; x.X_out = X_out;
    orc_for_units((long)B * hv, nthreads, alloc_step_unit, &x);
    free(ho);
    return 0;
}

/* ---------------------------------------------------------- calibration -- */

/* Candidate distortions (App. A.3 KDA reconstruction distortion; reading
 * R20): dist[h][i][k] += sum over the n_rec records and columns j of
 * (S^(k)_ij - S_ij)^2, S^(k) row i of head h quantized at class k against
 * c[h] (k = 0: rounded to FP16).  S [n_rec][Hv][d][d] logical order. */
int oracle_alloc_distortion(long n_rec, int hv, int d, const double *S, const float *c,
                            double *dist) {
    const double floor_r = ldexp(1.0, -126);
    for (long s = 0; s < n_rec; ++s)
        for (int h = 0; h < hv; ++h)
            for (int i = 0; i < d; ++i) {
                const double *row = S + (((size_t)s * hv + h) * d + i) * d;
                const float *ch = c + (size_t)h * d;
                double *dd = dist + ((size_t)h * d + i) * NCLS;
                double e0 = 0.0;
                for (int j = 0; j < d; ++j) {
                    double y = oracle_f16_to_double(oracle_f16_from_double(row[j]));
                    e0 += (y - row[j]) * (y - row[j]);
                }
                dd[0] += e0;
                for (int k = 1; k < NCLS; ++k) {
                    int qb = qmax_of(k);
                    double m = 0.0;
                    for (int j = 0; j < d; ++j) {
                        double x = row[j] / (double)ch[j];
                        if (fabs(x) > m) m = fabs(x);
                    }
                    double rr = (double)(float)(m / (double)qb);
                    if (rr < floor_r) rr = floor_r;
                    double e = 0.0;
                    for (int j = 0; j < d; ++j) {
                        double z = oracle_rhe((row[j] / (double)ch[j]) / rr);
                        if (z > qb) z = qb;
                        if (z < -qb) z = -qb;
                        double y = (rr * (double)ch[j]) * z;
                        e += (y - row[j]) * (y - row[j]);
                    }
                    dd[k] += e;
                }
            }
    return 0;
}

/* Lifetime weights (App. A.3; reading R21): ell = logret / n, and
 * L = 1 + sum_{j=1}^{H-1} exp(2 j ell), per unit.  logret [Hv][d] holds the
 * sum of log retention over n samples. */
int oracle_alloc_lifetime(int hv, int d, const double *logret, double n, int horizon,
                          double *Lw) {
    if (n <= 0.0 || horizon < 1) return -1;
    for (int u = 0; u < hv * d; ++u) {
        double ell = logret[u] / n;
        double acc = 1.0;
        for (int j = 1; j < horizon; ++j) acc += exp(2.0 * (double)j * ell);
        Lw[u] = acc;
    }
    return 0;
}

typedef struct {
    double slope;
    int unit, from, to; /* hull indices into the unit's candidate list */
} seg_t;

static int seg_cmp(const void *a, const void *b) {
    const seg_t *x = (const seg_t *)a, *y = (const seg_t *)b;
    if (x->slope > y->slope) return -1;
    if (x->slope < y->slope) return 1;
    if (x->unit != y->unit) return x->unit < y->unit ? -1 : 1;
    return x->from < y->from ? -1 : (x->from > y->from ? 1 : 0);
}

typedef struct {
    double score;
    int unit;
} piv_t;

static int piv_cmp(const void *a, const void *b) {
    const piv_t *x = (const piv_t *)a, *y = (const piv_t *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return x->unit < y->unit ? -1 : (x->unit > y->unit ? 1 : 0);
}

/* Pivot selection and lifetime-aware assignment (App. C.2; readings R22,
 * R23).  dist [Hv][d][5], Lw [Hv][d]; cand_mask: bit k set when integer
 * class k (1..4 = 8, 6, 4, 2 bits) is a candidate; nominal: the nominal
 * width b_nom (a candidate); n_pivot: P.  Outputs bits [Hv][d] (16 for
 * pivots), counts [Hv][5] and perm [Hv][d].  Returns 0, or -1 on bad
 * arguments. */
int oracle_alloc_assign(int hv, int d, const double *dist, const double *Lw, int cand_mask,
                        int nominal, int n_pivot, int32_t *bits, int32_t *counts,
                        int32_t *perm) {
    int N = hv * d;
    int cand[NCLS], nc = 0, knom = -1;
    for (int k = NCLS - 1; k >= 1; --k) /* ascending width: 2, 4, 6, 8 */
        if (cand_mask & (1 << k)) {
            cand[nc++] = k;
            if (kBits[k] == nominal) knom = k;
        }
    if (nc == 0 || knom < 0 || n_pivot < 0 || n_pivot > N) return -1;
    int *is_piv = (int *)calloc((size_t)N, sizeof(int));
    /* pivots: largest lifetime-weighted reduction to FP16 error (R22) */
    piv_t *pv = (piv_t *)calloc((size_t)N, sizeof(piv_t));
    for (int u = 0; u < N; ++u) {
        pv[u].score = Lw[u] * (dist[(size_t)u * NCLS + knom] - dist[(size_t)u * NCLS + 0]);
        pv[u].unit = u;
    }
    qsort(pv, (size_t)N, sizeof(piv_t), piv_cmp);
    for (int n = 0; n < n_pivot; ++n) is_piv[pv[n].unit] = 1;
    free(pv);
    /* lower convex hull of (b, L d(b)) per unit, segments that save error (R23) */
    seg_t *segs = (seg_t *)calloc((size_t)N * NCLS, sizeof(seg_t));
    int *hull = (int *)calloc((size_t)N * NCLS, sizeof(int)); /* candidate indices */
    int *hlen = (int *)calloc((size_t)N, sizeof(int));
    int *level = (int *)calloc((size_t)N, sizeof(int)); /* index into the hull */
    int *frozen = (int *)calloc((size_t)N, sizeof(int));
    int nseg = 0;
    long n_int = 0;
    for (int u = 0; u < N; ++u) {
        if (is_piv[u]) continue;
        ++n_int;
        int *hu = hull + (size_t)u * NCLS;
        int m = 0;
        for (int a = 0; a < nc; ++a) {
            double bx = kBits[cand[a]], by = Lw[u] * dist[(size_t)u * NCLS + cand[a]];
            while (m >= 2) {
                double ox = kBits[cand[hu[m - 2]]], oy = Lw[u] * dist[(size_t)u * NCLS + cand[hu[m - 2]]];
                double ax = kBits[cand[hu[m - 1]]], ay = Lw[u] * dist[(size_t)u * NCLS + cand[hu[m - 1]]];
                double cross = (ax - ox) * (by - oy) - (ay - oy) * (bx - ox);
                if (cross <= 0.0) --m; /* middle point not strictly below: drop */
                else break;
            }
            hu[m++] = a;
        }
        /* keep the hull only while each step lowers the distortion */
        int keep = 1;
        while (keep < m) {
            double y0 = Lw[u] * dist[(size_t)u * NCLS + cand[hu[keep - 1]]];
            double y1 = Lw[u] * dist[(size_t)u * NCLS + cand[hu[keep]]];
            if (!(y1 < y0)) break;
            ++keep;
        }
        hlen[u] = keep;
        for (int s = 0; s + 1 < keep; ++s) {
            double y0 = Lw[u] * dist[(size_t)u * NCLS + cand[hu[s]]];
            double y1 = Lw[u] * dist[(size_t)u * NCLS + cand[hu[s + 1]]];
            double db = (double)(kBits[cand[hu[s + 1]]] - kBits[cand[hu[s]]]);
            segs[nseg].slope = (y0 - y1) / db;
            segs[nseg].unit = u;
            segs[nseg].from = s;
            segs[nseg].to = s + 1;
            ++nseg;
        }
    }
    long budget = (long)nominal * n_int;
    long used = (long)kBits[cand[0]] * n_int;
    if (used > budget) {
        free(is_piv); free(segs); free(hull); free(hlen); free(level); free(frozen);
        return -1;
    }
    qsort(segs, (size_t)nseg, sizeof(seg_t), seg_cmp);
    for (int s = 0; s < nseg; ++s) {
        int u = segs[s].unit;
        if (frozen[u] || level[u] != segs[s].from) continue;
        const int *hu = hull + (size_t)u * NCLS;
        long db = kBits[cand[hu[segs[s].to]]] - kBits[cand[hu[segs[s].from]]];
        if (used + db <= budget) {
            used += db;
            level[u] = segs[s].to;
        } else {
            frozen[u] = 1;
        }
    }
    /* bits, counts, perm */
    for (int h = 0; h < hv; ++h) {
        for (int k = 0; k < NCLS; ++k) counts[h * NCLS + k] = 0;
        for (int i = 0; i < d; ++i) {
            int u = h * d + i;
            int k = is_piv[u] ? 0 : cand[hull[(size_t)u * NCLS + level[u]]];
            bits[u] = kBits[k];
            counts[h * NCLS + k] += 1;
        }
        int p = 0;
        for (int k = 0; k < NCLS; ++k)
            for (int i = 0; i < d; ++i)
                if (bits[h * d + i] == kBits[k]) perm[h * d + p++] = i;
    }
    free(is_piv); free(segs); free(hull); free(hlen); free(level); free(frozen);
    return 0;
}
