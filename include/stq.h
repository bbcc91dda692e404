/*
 * stq.h -- C ABI of the quantized gated delta-rule decode library for AMD
 * MI355X (gfx950).
 *
 * What it computes (STEPQuant paper, "STEPQuant: When and Where Errors Matter in
 * Delta-Rule Recurrent State Quantization", arXiv 2609.38169):
 *   - the gated delta rule with a scalar gate, Sec. 2.1 Eq. (1) with D_t = a I:
 *       X = a S + b k (v - a S^T k)^T,      o = X^T q
 *   - over a recurrent state stored in the dual-axis form of Sec. 4.3,
 *       S_ij = r_i c_j z_ij,
 *     with per-key-row bit widths (4 or 8 bits, Sec. 3.2 mixed precision),
 *     a key-row factor r_i recomputed at every step and a value-column factor
 *     c_j fixed offline (Sec. 3.2 / Sec. 4.4: the precision map is calibrated
 *     offline and fixed across requests);
 *   - in the order of App. C.3 Table C2: reconstruct, update, emit the readout
 *     before requantization, derive row factors, pack and write back;
 *   - and the same step with a per-key-row (diagonal) gate, Eq. (1) with
 *     D_t = diag(d) (the KDA form, Sec. 6.1 and App. C.1):
 *       X = D S + b k (v - (D S)^T k)^T,    o = X^T q.
 * Quantizer (Sec. 2.2): z = clip(round(x / s), -q_b, q_b), q_b = 2^(b-1) - 1,
 * with round = round-half-to-even; row factor r_i = max(fl32(max_j |X_ij / c_j|
 * / q_b), 2^-126); the code of X_ij is taken against the stored r_i.
 *
 * Conventions
 *   - Every function is extern "C", returns stq_status and never throws.
 *   - All device memory is owned by the caller and passed as plain device
 *     pointers.  The library allocates nothing and keeps no global state, so it
 *     is re-entrant; the caller keeps every buffer alive until the work queued
 *     on the stream has finished.
 *   - Device work is queued on the caller's HIP stream (stq_stream_t is a
 *     hipStream_t; NULL means the default stream) with no implicit
 *     synchronisation.  Arguments are validated on the host before any launch;
 *     a rejected call queues nothing.
 *
 * Packed layout (slot s, value head h; physical row p holds logical key row
 * perm[h][p]; the first n8 physical rows are 8-bit, the rest 4-bit):
 *   pool8  int8   [n_slots][Hv][n8][dv]       two's-complement codes
 *   pool4  uint8  [n_slots][Hv][dk-n8][dv/2]  two's-complement nibbles; byte m
 *                                             holds column 2m in bits 0..3 and
 *                                             column 2m+1 in bits 4..7
 *   r      float  [n_slots][Hv][dk]           row factor, physical row order
 *   c      float  [Hv][dv]                    column factor (c_j > 0)
 *   perm   int32  [Hv][dk]                    logical row of physical row p
 * Vectors: q, k [B][Hk][dk]; v [B][Hv][dv]; alpha, beta [B][Hv] fp32;
 * o [B][Hv][dv] fp32.  Value head h reads key head h / (Hv / Hk).
 * States passed as fp32 matrices (pack input, dequant output, calibration
 * records) are [B or n_rec][Hv][dk][dv] in logical row order.
 */
#ifndef STQ_H
#define STQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *stq_stream_t; /* a hipStream_t; NULL = default stream */

typedef enum {
    STQ_OK = 0,
    STQ_E_ARG = 1,         /* null or misaligned pointer, bad flag or enum */
    STQ_E_SHAPE = 2,       /* inconsistent dimensions or batch size */
    STQ_E_UNSUPPORTED = 3, /* a d_k / d_v outside the compiled set */
    STQ_E_SPACE = 4,       /* caller buffer smaller than stq_state_bytes() */
    STQ_E_STATE = 5,       /* mixed state decoded before calibration */
    STQ_E_DEVICE = 6       /* a HIP launch or runtime call failed */
} stq_status;

typedef enum {
    STQ_FMT_MIXED48 = 0, /* 4/8-bit key rows, fp32 r, calibrated c and perm */
    STQ_FMT_INT8ROW = 1, /* uniform symmetric rowwise-absmax INT8: n8 = d_k,
                            c = 1, identity row order (Sec. 5.1 baseline) */
    STQ_FMT_FP32 = 2,    /* unquantized fp32 state (the FP32-state baseline) */
    STQ_FMT_REFIT = 3,   /* MIXED48 codes and row factors with column factors
                            kept per state and refit at every step (App. C.1,
                            Table C2 step 5); see "Online column refit" */
    STQ_FMT_ALLOC = 4,   /* ragged row classes per head: FP16 pivot rows and
                            8-, 6-, 4-, 2-bit rows chosen by the lifetime-aware
                            assignment (App. C.2, Table C2); fixed per-head c;
                            see "Ragged row classes" */
    STQ_FMT_ALLOC_REFIT = 5 /* ALLOC with per-state column factors refit over
                            the non-pivot integer rows (App. C.1, Table C2
                            step 5) */
} stq_format;

typedef enum { STQ_F32 = 0, STQ_BF16 = 1 } stq_dtype;
/* OR'd into the dtype argument of the decode steps: the readout o is written
 * in bf16 (rounded to nearest even from the fp32 readout; NaN for a skipped
 * slot) instead of fp32 -- the form the layer's next product consumes. */
#define STQ_OUT_BF16 0x100

/* Calibration flags (stq_calibrate), combinable. */
#define STQ_CAL_RESET 1u    /* zero the accumulated statistics first */
#define STQ_CAL_COLS 2u     /* fold records into the per-column absmax */
#define STQ_CAL_ROWS 4u     /* fold records into the per-row sum of squares */
#define STQ_CAL_FINALIZE 8u /* set c and perm from the statistics */
#define STQ_CAL_DIST 16u    /* ALLOC formats: fold records into the per-row
                               candidate distortions (against the current c) */

/* Geometry.  Supported: d_k == d_v in {16, 32, 64, 128}; 0 <= n8 <= d_k
 * (MIXED48; INT8ROW forces n8 = d_k); n_heads_v % n_heads_k == 0.
 * ALLOC formats: n8 = 0, nominal_bits in {2, 4, 6, 8} (the integer budget
 * per value), 0 <= n_pivot <= n_heads_v * d_k (FP16 pivot rows per slot);
 * every other format: nominal_bits = n_pivot = 0. */
typedef struct {
    int32_t n_slots;
    int32_t n_heads_v;
    int32_t n_heads_k;
    int32_t d_k;
    int32_t d_v;
    int32_t n8;  /* 8-bit rows per head (same for every head) */
    int32_t fmt; /* stq_format */
    int32_t nominal_bits;
    int32_t n_pivot;
} stq_desc;

/* A state carved out of one caller buffer by stq_alloc_state.  Plain device
 * pointers; fields that a format does not use are NULL. */
typedef struct {
    stq_desc desc;
    int8_t *pool8;
    uint8_t *pool4;
    float *r;
    float *c;
    int32_t *perm;
    float *colmax;      /* [Hv][dv]  calibration: column absmax */
    double *rowscore;   /* [Hv][dk]  calibration: row sum of squares */
    float *cal_colpart; /* [Hv][STQ_CAL_CHUNKS][dv] per-chunk partials */
    double *cal_rowpart;/* [Hv][STQ_CAL_CHUNKS][dk] per-chunk partials */
    float *s32;         /* [n_slots][Hv][dk][dv]  FP32 format only */
    float *cs;          /* [n_slots][Hv][dv]  REFIT: per-state column factors */
    float *w2;          /* [Hv][dk]  REFIT: squared row-impact weights,
                           logical rows (1 until calibrated) */
    double *impact;     /* [Hv][dk]  REFIT calibration: accumulated row impact */
    int32_t *layout;    /* [Hv][8]  ALLOC: class counts [0..4], segment offset
                           [5] and segment bytes [6] of each head; followed by
                           [Hv][64] words the library derives from them (the
                           d = 128 decode's per-slot row-chunk descriptors) */
    double *dist;       /* [Hv][dk][5]  ALLOC calibration: candidate distortions */
    double *logret;     /* [Hv][dk]  ALLOC calibration: summed log retention */
    double *nret;       /* [Hv]  ALLOC calibration: retention samples */
    int64_t slot_bytes; /* ALLOC: bytes of one slot of the byte pool */
    int32_t calibrated; /* host flag: c and perm hold a calibration */
    int32_t reserved;
} stq_state;

#define STQ_CAL_CHUNKS 64

/* Online column refit (format STQ_FMT_REFIT; the paper's online Key-Row-Aware
 * Dual-axis Fitting, Sec. 4.3 "Column factors", App. C.1 fixed-code update,
 * App. C.3 Table C2 step 5).  The state keeps its own column factors cs.  A
 * decode step reconstructs with them, takes row factors and codes against
 * them exactly as the MIXED48 step does, and then refits them once with the
 * new codes held fixed:
 *   c'_j = sum_i w2_i v_ij X_ij / sum_i w2_i v_ij^2,   v_ij = r'_i z'_ij,
 * rounded to fp32 and floored at 2^-126 (a zero denominator keeps c_j).  The
 * stored state is (z', r', c').  w2 are squared row-impact weights
 * (stq_calibrate_impact), 1 until calibrated.  Packing a state (prefill
 * boundary) starts from the calibrated per-head c and refits the same way. */

/* Ragged row classes (formats STQ_FMT_ALLOC and STQ_FMT_ALLOC_REFIT; the
 * paper's FP16 pivots and lifetime-aware bit allocation, App. C.2 Table C1,
 * App. C.3 Table C2, App. A.3).  Each head's physical rows are sorted into
 * classes k = 0..4: FP16 pivot rows, then 8-, 6-, 4- and 2-bit rows
 * (q_b = 127, 31, 7, 1), each class in ascending logical row; layout[h]
 * holds the five counts.  pool8 is a byte pool [n_slots][slot_bytes]; head
 * h's rows occupy bytes [layout[h][5], layout[h][5] + layout[h][6]) of a
 * slot: class 0 rows take 2 d bytes (binary16 values, little endian), class
 * 1 d bytes (int8), class 2 3d/4 bytes (the low four bits of column j in
 * nibble j of the first d/2 bytes, even column in the low nibble, the top
 * two bits in bits 2(j%4) of byte d/2 + j/4), class 3 d/2 bytes (nibbles),
 * class 4 d/4 bytes (column j in bits 2(j%4) of byte j/4); codes are two's
 * complement; segments are padded to 16 bytes.
 *   slot_bytes = round16(nominal_bits (Hv d - n_pivot) d / 8
 *                        + 2 d n_pivot + 16 Hv)
 * holds any assignment that keeps the integer budget.  Integer rows follow
 * the MIXED48 rules with their own q_b (r from the absmax, codes against
 * the stored r); a pivot row stores X rounded to nearest-even binary16,
 * saturated at +-65504, has r = 0 and no column factor, and does not enter
 * the column refit of ALLOC_REFIT.
 * Calibration: stq_calibrate with RESET, COLS over the records, FINALIZE
 * (sets c only), then DIST over records (the candidate distortions against
 * that c); stq_calibrate_retention over the gates of the calibration steps;
 * then stq_allocate chooses pivots and widths and writes layout and perm.
 * stq_set_alloc_layout installs a layout chosen elsewhere. */

/* Bytes of device memory a state with this geometry needs (host arithmetic
 * only, no device call); 0 if the descriptor is invalid or unsupported.  The
 * state is the representation of Sec. 4.3 (X = r_i c_j z_ij: low-bit codes
 * z, a factor per key row, a factor per value column) stored as the
 * slot-indexed packed pages of App. F.1, one page per request slot, sized
 * for the reserved slots of App. F.3: per (slot, head) the code rows of each
 * width plus the fp32 row factors; per head the calibration arrays. */
size_t stq_state_bytes(const stq_desc *desc);

/* Carve a state out of the caller's device buffer `dev` (256-byte aligned,
 * `bytes` >= stq_state_bytes) and queue its initialisation on `stream`: the
 * packed pages of App. F.1 (slot s of the pool is request slot s; slots are
 * initialised and reused by the caller) holding the Sec. 4.3 representation,
 * every page starting as the zero state:
 * codes 0, r = 2^-126 (the state S = 0), c = 1, cs = 1, w2 = 1,
 * perm = identity, fp32 state 0, statistics 0.  INT8ROW and FP32 states are
 * ready to decode at once; a MIXED48 or REFIT state must be calibrated
 * (stq_calibrate with STQ_CAL_FINALIZE, or stq_set_calibration) before
 * stq_decode_step accepts it.
 * Errors: STQ_E_ARG (null/misaligned), STQ_E_SHAPE / STQ_E_UNSUPPORTED (desc),
 * STQ_E_SPACE (short buffer), STQ_E_DEVICE (launch failed). */
stq_status stq_alloc_state(const stq_desc *desc, void *dev, size_t bytes,
                           stq_stream_t stream, stq_state *out);

/* Offline calibration of the fixed column factor and the 4/8-bit split of a
 * MIXED48 state (Sec. 3.2 and Sec. 4.4: calibrated offline, fixed across
 * requests; App. A.3: each batch element of a recorded step is one sample).
 * `records` are n_rec fp32 states [n_rec][Hv][dk][dv] in logical row order
 * (e.g. the states of an unquantized run at successive steps); n_rec may be 0
 * with only RESET and/or FINALIZE.  Rule:
 *   c_j    = max over all COLS records and rows of |S_ij| (a zero column -> 1)
 *   score_i= sum over all ROWS records of sum_j S_ij^2
 *   FINALIZE makes the n8 rows of highest score 8-bit (ties to the lower row),
 *   and sets perm to those rows ascending, then the others ascending.
 * FINALIZE rewrites c and perm, which invalidates packed contents: pack the
 * state again afterwards.  The statistics are reduced in a fixed order, so the
 * result does not depend on scheduling.
 * Errors: STQ_E_ARG (null state/records, unknown flags, format not MIXED48
 * or REFIT),
 * STQ_E_SHAPE (n_rec < 0), STQ_E_DEVICE. */
stq_status stq_calibrate(stq_state *st, const float *records, int64_t n_rec,
                         uint32_t flags, stq_stream_t stream);

/* stq_calibrate for callers that cannot allocate device memory (code under
 * graph capture, serving loops, harnesses that forbid allocation): the same
 * arguments, rules and results, with the per-chunk partial results held in a
 * fixed 6 MiB array of the library (one copy per GPU, kept until the process
 * ends) instead of the state's partial arrays.  Allocates nothing.  Limit:
 * n_heads_v * d_k <= 8192 head rows, else STQ_E_SPACE before anything is
 * queued.  The state must live on the current device.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other host threads) race and must be ordered by the caller.
 * Errors: as stq_calibrate, plus STQ_E_SPACE (too many head rows). */
stq_status stq_calibrate_static(stq_state *st, const float *records, int64_t n_rec,
                                uint32_t flags, stq_stream_t stream);

/* Row-impact calibration of a REFIT state (Sec. 4.1; App. C.1 with the
 * scalar gate; App. B.3 for the exponent): for B calibration samples of one
 * step (q, k [B][Hk][dk] fp32 or bf16 by `dtype`, alpha, beta [B][Hv] fp32),
 * accumulate impact[h][i] += sum_b (alpha (q_i - beta k_i (k.q)))^2 in
 * double, value head h reading key head h / (Hv / Hk).  Flags: STQ_CAL_RESET
 * zeroes the sums first; STQ_CAL_FINALIZE sets the weights
 *   w2[h][i] = fl32((impact_i / mean_i impact_i)^(1/4)), floored at 2^-32
 * (all-zero head: 1).  B may be 0 with only RESET and/or FINALIZE.  The
 * accumulation order is fixed, so results do not depend on scheduling.
 * Errors: STQ_E_ARG (format not REFIT, null or misaligned inputs, unknown
 * flags or dtype), STQ_E_SHAPE (B < 0), STQ_E_DEVICE. */
stq_status stq_calibrate_impact(stq_state *st, const void *q, const void *k,
                                int32_t dtype, const float *alpha, const float *beta,
                                int32_t B, uint32_t flags, stq_stream_t stream);

/* Row-impact calibration with a per-key-row gate (App. C.1: g_i = d_i (q_i -
 * beta k_i (k.q))): as stq_calibrate_impact with alpha replaced by
 * gate [B][Hv][dk] fp32 in logical key-row order,
 *   impact[h][i] += sum_b (gate[b][h][i] (q_i - beta k_i (k.q)))^2.
 * Errors: as stq_calibrate_impact; STQ_E_ARG for a null gate with B > 0. */
stq_status stq_calibrate_impact_gated(stq_state *st, const void *q, const void *k,
                                      int32_t dtype, const float *gate, const float *beta,
                                      int32_t B, uint32_t flags, stq_stream_t stream);

/* Mean log retention for the lifetime weights of the ALLOC formats (App. A.3):
 * logret[h][i] += sum_b log(retention), nret[h] += B, where the retention of
 * row i is alpha[b][h] (scalar gate, [B][Hv] fp32) or gate[b][h][i] (row gate,
 * [B][Hv][dk] fp32, logical rows); exactly one of alpha and gate is given when
 * B > 0.  STQ_CAL_RESET zeroes the sums first (the only flag).
 * Errors: STQ_E_ARG (format not ALLOC or ALLOC_REFIT, pointers, flags),
 * STQ_E_SHAPE (B < 0), STQ_E_DEVICE. */
stq_status stq_calibrate_retention(stq_state *st, const float *alpha, const float *gate,
                                   int32_t B, uint32_t flags, stq_stream_t stream);

/* Lifetime-aware assignment of an ALLOC state (App. C.2 "KDA calibration" and
 * "Allocation optimizers", Table C1; App. A.3 "Mean log retention"):
 *   L_u = sum_{j=0}^{horizon-1} exp(2 j ell_u), ell_u = logret_u / nret, the
 *   lifetime weight of row u;
 *   pivots: the desc.n_pivot rows of largest L_u (d_u(nominal) - d_u(FP16))
 *   over all heads (ties to the lower h * dk + i);
 *   every other row takes a width among the vertices of the lower convex hull
 *   of its points (b, L_u d_u(b)) that lower the objective.  For a shared
 *   multiplier lambda each row takes its minimiser of L_u d_u(b) + lambda b;
 *   lambda runs over the hull slopes (distortion saved per bit, ties: lower
 *   row, then lower width) down to the last at which the widths still sum to
 *   at most nominal_bits * (non-pivot rows).  The repair then takes the
 *   remaining hull steps in the same order wherever they still fit; a row
 *   whose next step does not fit keeps its width.
 * candidates: bit k set for class k (1: 8, 2: 6, 3: 4, 4: 2 bits); 0 picks
 * {8, 6, 4, 2} for nominal_bits <= 4 and {8, 6, 4} otherwise (Table C1).
 * Writes layout and perm and marks the state calibrated; c is left as set by
 * FINALIZE.  Synchronises the stream (reads the statistics to the host).
 * Errors: STQ_E_ARG (format, horizon < 1, bad candidates, nominal width not
 * a candidate, infeasible budget), STQ_E_STATE (no retention samples),
 * STQ_E_DEVICE. */
stq_status stq_allocate(stq_state *st, int32_t horizon, uint32_t candidates,
                        stq_stream_t stream);

/* The assignment of stq_allocate on statistics held in HOST memory (App. C.2
 * "KDA calibration" and "Allocation optimizers", Table C1; App. A.3 "Mean
 * log retention"): a planner can run it offline on saved statistics and
 * install the result with stq_set_alloc_layout.  Host code only: it touches
 * no device and needs no GPU.
 *   dist    [n_heads_v][d_k][5] fp64: candidate distortion of each logical
 *           row at class k (0: FP16 pivot, 1..4: 8, 6, 4, 2 bits), the sums
 *           of stq_calibrate's DIST pass;
 *   logret  [n_heads_v][d_k] fp64: sums of log retention over nret samples
 *           (stq_calibrate_retention), so ell_u = logret_u / nret;
 *   horizon, candidates, nominal_bits, n_pivot: as stq_allocate and the
 *           descriptor;
 *   counts  [n_heads_v][5] int32 and perm [n_heads_v][d_k] int32 (caller
 *           memory, overwritten): rows per class per head, and the logical
 *           row of each physical row (classes in order, each ascending).
 * The result depends on the arguments alone (all ties are broken by row and
 * width as stq_allocate states).
 * Errors: STQ_E_ARG (null pointers, n_heads_v or d_k < 1, horizon < 1,
 * nret <= 0 or NaN, bad candidates, nominal width not a candidate, n_pivot
 * outside [0, n_heads_v d_k], infeasible budget), STQ_E_SHAPE (more than
 * 2^24 rows). */
stq_status stq_assign_rows(int32_t n_heads_v, int32_t d_k, const double *dist,
                           const double *logret, double nret, int32_t horizon,
                           uint32_t candidates, int32_t nominal_bits, int32_t n_pivot,
                           int32_t *counts, int32_t *perm);

/* Install a ragged layout chosen elsewhere: counts [Hv][5] (HOST memory, each
 * head's counts >= 0 and summing to dk), c [Hv][dv] and perm [Hv][dk] (device
 * memory, as stq_set_calibration).  Marks the state calibrated and
 * invalidates packed contents.  Synchronises the stream.
 * Errors: STQ_E_ARG (format not ALLOC or ALLOC_REFIT, pointers, counts),
 * STQ_E_SPACE (the segments do not fit slot_bytes), STQ_E_DEVICE. */
stq_status stq_set_alloc_layout(stq_state *st, const int32_t *counts, const float *c,
                                const int32_t *perm, stq_stream_t stream);

/* Install a calibration computed elsewhere: copies c [Hv][dv] (each > 0) and
 * perm [Hv][dk] (a permutation of 0..dk-1 per head) from device memory and
 * marks the state calibrated.  Like FINALIZE it invalidates packed contents.
 * Errors: STQ_E_ARG (null, format not MIXED48 or REFIT), STQ_E_DEVICE. */
stq_status stq_set_calibration(stq_state *st, const float *c, const int32_t *perm,
                               stq_stream_t stream);

/* Pack fp32 states S [B][Hv][dk][dv] (logical order) into slots[b] (slots: a
 * device int32 array of B distinct slots, or NULL for slots 0..B-1): the
 * requantization half of a decode step applied to a given state: the pack at
 * the prefill boundary (App. F.1: prefill runs on unpacked states and packs
 * the boundary states; App. B.2: the uncompressed prefill state is packed
 * once, and decode then reads and rewrites the packed state), with the
 * quantizer of App. C.3 Table C2 steps 4 and 6.  FP32 format: copies S.  REFIT: codes and row
 * factors against the calibrated per-head c, then each state's column factors
 * refit (see "Online column refit").
 * Errors: STQ_E_ARG, STQ_E_SHAPE (B < 1 or B > n_slots), STQ_E_STATE
 * (MIXED48 not calibrated), STQ_E_DEVICE. */
stq_status stq_pack_state(const stq_state *st, const float *S, const int32_t *slots,
                          int32_t B, stq_stream_t stream);

/* One decode step for B sequences x Hv value heads, in place on slots[b]
 * (App. C.3 Table C2 steps 1-4 and 6-7, fused into a single read and a single
 * write of the packed state):
 *   S_hat = r c z;  u = S_hat^T k;  X = a S_hat + b k (v - a u)^T;  o = X^T q
 *   r'_i = max(fl32(max_j |X_ij / c_j| / q_b), 2^-126);
 *   z'_ij = clip(rhe(X_ij / c_j / r'_i), -q_b, q_b)
 * REFIT format: c is the state's own cs, refit after the codes are taken.
 * q, k, v are fp32 or bf16 (`dtype`); alpha and beta are fp32; o is fp32, or
 * bf16 with STQ_OUT_BF16 in `dtype`.
 * Preconditions: slots distinct within a call (not checked on the device;
 * with STQ_CHECK_SLOTS set in the environment the host copies the slot list,
 * synchronising the stream, and returns STQ_E_ARG for a repeated slot);
 * a slot outside [0, n_slots) is skipped and its o is filled with NaN.
 * Errors: STQ_E_ARG (null/misaligned pointer, bad dtype), STQ_E_SHAPE (B < 1
 * or B > n_slots), STQ_E_STATE (MIXED48 or REFIT not calibrated),
 * STQ_E_DEVICE. */
stq_status stq_decode_step(const stq_state *st, const int32_t *slots, int32_t B,
                           const void *q, const void *k, const void *v, int32_t dtype,
                           const float *alpha, const float *beta, void *o,
                           stq_stream_t stream);

/* The same decode step, reading slots[b] of `src` and writing the updated
 * packed codes and row factors (FP32 format: the updated state) into the same
 * slots of `dst`; `src` is left unchanged.  This is the double-buffered page
 * of App. C.3 Table C2 step 6 (the old representation stays valid until its
 * readers finish) and lets the write stream to other pages than the read.
 * dst must have the same descriptor as src.  The step reads c and perm from
 * src only, so the codes written to dst are relative to src's calibration:
 * give dst the same c and perm before reading it back or decoding from it.
 * REFIT: the refit column factors are written to dst's cs.
 * dst == src is the in-place step; pools that overlap partially are rejected.
 * Errors: as stq_decode_step; STQ_E_SHAPE if the descriptors differ,
 * STQ_E_ARG for partially overlapping pools. */
stq_status stq_decode_step_into(const stq_state *src, const stq_state *dst,
                                const int32_t *slots, int32_t B, const void *q,
                                const void *k, const void *v, int32_t dtype,
                                const float *alpha, const float *beta, void *o,
                                stq_stream_t stream);

/* The decode step with a per-key-row gate (Sec. 2.1 Eq. (1) with
 * D_t = diag(d), the KDA form of Sec. 6.1), reading slots[b] of `src` and
 * writing `dst` as stq_decode_step_into (dst == src: in place):
 *   S_hat = r c z;  u = (D S_hat)^T k;  X = D S_hat + b k (v - u)^T;  o = X^T q
 * then r', z' (and for REFIT the column refit) exactly as stq_decode_step.
 * gate is fp32 [B][Hv][dk]: gate[b][h][i] multiplies LOGICAL key row i of
 * value head h (the row the caller's q and k index, not the physical row).
 * A uniform gate d = a 1 gives the scalar-gate step.  Every format is
 * supported.
 * Errors: as stq_decode_step_into; STQ_E_ARG for a null or misaligned gate. */
stq_status stq_decode_step_gated(const stq_state *src, const stq_state *dst,
                                 const int32_t *slots, int32_t B, const void *q,
                                 const void *k, const void *v, int32_t dtype,
                                 const float *gate, const float *beta, void *o,
                                 stq_stream_t stream);

/* Reconstruct S_ij = r_i c_j z_ij (Sec. 4.3) of slots[b] into fp32
 * S_out [B][Hv][dk][dv] in logical row order (FP32 format: copies the state;
 * REFIT: c is the state's own cs).
 * Errors: STQ_E_ARG, STQ_E_SHAPE, STQ_E_DEVICE. */
stq_status stq_dequant_state(const stq_state *st, const int32_t *slots, int32_t B,
                             float *S_out, stq_stream_t stream);

/* Streaming copy of `bytes` (a multiple of 16, both pointers 16-byte aligned)
 * from src to dst with non-temporal loads and stores: the plain copy kernel
 * used to measure the practical HBM ceiling and to scale hardware byte
 * counters.
 * Errors: STQ_E_ARG, STQ_E_DEVICE. */
stq_status stq_stream_copy(const void *src, void *dst, size_t bytes, stq_stream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char *stq_status_str(int32_t status);

/* Library ABI version (bumped on any change to the declarations above):
 * 2 since the REFIT format and its state fields; 3 since the per-key-row
 * gate entry points; 4 since the ALLOC formats (descriptor and state fields,
 * retention and assignment entry points); 5 since STQ_OUT_BF16 (o is void *);
 * 6 since stq_calibrate_static; 7 since an ALLOC state's layout buffer also
 * holds the per-slot descriptors (its stq_state_bytes grows by 256 B a head). */
int32_t stq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STQ_H */
