/*
 * attn_oracle.c -- plain, slow, obviously-correct CPU oracle for exact
 * attention forward, in IEEE double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * GPU library.
 *
 * Inputs are 16-bit bit patterns (uint16): bf16, or IEEE binary16 (fp16)
 * through oracle_attn_rows_elem.  Each is widened exactly to double, so the
 * oracle works on the exact values the GPU receives.
 *
 * Layouts (all contiguous, row-major):
 *   q   [B, Hq,  Lq, dqk]      k [B, Hkv, Lk, dqk]      v [B, Hkv, Lk, dv]
 *   o   [n_rows, dv]  (double) lse [n_rows]  (double)
 * A "row" is one query vector, flat index r = (b*Hq + h)*Lq + i.
 *
 * Definitions followed (sources are the three pages on FlashAttention):
 *  - exact attention O = softmax(scale * Q K^T) V per head, softmax along keys:
 *    "Infra: Flash Attention", opening section (S = QK^T/sqrt d, P = softmax S,
 *    O = PV) and "Flash Attention 4 ..." (fangpin gpu-hpc-book ch. 13), section
 *    on the real bottleneck of attention.
 *  - safe softmax (subtract the row max): "Infra: Flash Attention", section on
 *    computing softmax in segments.
 *  - logsumexp L_i = m_i + log l_i = log sum_j e^{S_ij}: "Infra: Flash
 *    Attention", Algorithm 1 (output step) and the backward-recompute section.
 *  - causal mask aligned bottom-right (query i sees keys j <= i + Lk - Lq) and
 *    GQA head mapping (query head h reads K/V head h / (Hq/Hkv)): "Flash
 *    Attention 4 ..." ch. 13, section on causal attention and GQA.
 *  - a row with no valid key has no defined softmax; the pages leave its
 *    output to the operator.  Reading adopted: O = 0, lse = -inf.
 *
 * The online (tiled) variants in the second half follow the algorithms the
 * pages describe step by step; they exist to check that the tiled method
 * reaches the same result as the definition.  The key-segment form of the
 * definition and the merge of segment states check the split-key path.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of a bf16 bit pattern: bf16 is binary32 with the low 16
 * mantissa bits dropped, so shifting the pattern into the top half of a
 * 32-bit word gives the identical binary32 value. */
static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t word = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* Exact widening of an IEEE binary16 (fp16) bit pattern: 1 sign bit, 5
 * exponent bits (bias 15), 10 fraction bits.  Exponent 0 holds zero and the
 * subnormals f * 2^-24; exponent 31 holds infinities and NaNs; otherwise the
 * value is (1024 + f) * 2^(e - 25).  Every such value is a double. */
static double fp16_bits_to_double(uint16_t bits)
{
    int e = (bits >> 10) & 31;
    int f = bits & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (bits & 0x8000) ? -v : v;
}

/* Element types of the 16-bit inputs. */
enum { ELEM_BF16 = 0, ELEM_FP16 = 1 };

typedef struct {
    int64_t B, Hq, Hkv, Lq, Lk, dqk, dv;
    int causal;
    double scale;
    int elem; /* ELEM_BF16 or ELEM_FP16 */
} dims_t;

static double widen(const dims_t* d, uint16_t bits)
{
    return d->elem == ELEM_FP16 ? fp16_bits_to_double(bits) : bf16_bits_to_double(bits);
}

/* Test hook: the widening of one 16-bit pattern (elem 0 bf16, 1 fp16). */
double oracle_widen(uint16_t bits, int elem)
{
    dims_t d;
    memset(&d, 0, sizeof d);
    d.elem = elem;
    return widen(&d, bits);
}

static int check_dims(const dims_t* d)
{
    if (d->B < 1 || d->Hq < 1 || d->Hkv < 1 || d->Lq < 1 || d->Lk < 1 ||
        d->dqk < 1 || d->dv < 1)
        return 1;
    if (d->Hq % d->Hkv != 0)
        return 2;
    if (!(d->scale > 0.0) || !isfinite(d->scale))
        return 3;
    return 0;
}

/* Number of keys row i may attend: all Lk keys, or, with the bottom-right
 * causal mask, keys 0 .. i + Lk - Lq (clamped to [0, Lk]). */
static int64_t valid_keys(const dims_t* d, int64_t i)
{
    if (!d->causal)
        return d->Lk;
    int64_t last = i + d->Lk - d->Lq; /* last visible key index */
    if (last < 0)
        return 0;
    return last + 1 < d->Lk ? last + 1 : d->Lk;
}

typedef struct {
    const uint16_t* qrow; /* dqk */
    const uint16_t* kh;   /* [Lk, dqk] of the row's K/V head */
    const uint16_t* vh;   /* [Lk, dv] */
    int64_t i;            /* query position */
} row_ref_t;

static row_ref_t locate_row(const dims_t* d, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, int64_t r)
{
    row_ref_t rr;
    int64_t i = r % d->Lq;
    int64_t bh = r / d->Lq;
    int64_t h = bh % d->Hq;
    int64_t b = bh / d->Hq;
    int64_t group = d->Hq / d->Hkv;
    int64_t hk = h / group;
    rr.qrow = q + ((b * d->Hq + h) * d->Lq + i) * d->dqk;
    rr.kh = k + (b * d->Hkv + hk) * d->Lk * d->dqk;
    rr.vh = v + (b * d->Hkv + hk) * d->Lk * d->dv;
    rr.i = i;
    return rr;
}

/* ------------------------------------------------------------------------ */
/* 1. The definition, materialised: one full score row at a time.           */
/* ------------------------------------------------------------------------ */

/* Softmax attention of one query row over the visible keys j with
 * j0 <= j < j1 (the whole row when [j0, j1) = [0, Lk)). */
static void exact_row(const dims_t* d, row_ref_t rr, int64_t j0, int64_t j1, double* qd,
                      double* s, double* o_row, double* lse_out)
{
    int64_t n = valid_keys(d, rr.i);
    if (j1 > n)
        j1 = n;
    if (j0 < 0)
        j0 = 0;
    for (int64_t c = 0; c < d->dv; ++c)
        o_row[c] = 0.0;
    if (j1 <= j0) {
        *lse_out = -INFINITY;
        return;
    }
    for (int64_t c = 0; c < d->dqk; ++c)
        qd[c] = widen(d, rr.qrow[c]);

    /* S_i,j = scale * q_i . k_j for every key j in range */
    double m = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
        const uint16_t* kj = rr.kh + j * d->dqk;
        double dot = 0.0;
        for (int64_t c = 0; c < d->dqk; ++c)
            dot += qd[c] * widen(d, kj[c]);
        s[j] = d->scale * dot;
        if (s[j] > m)
            m = s[j];
    }
    /* P_i,j = e^{S_i,j - m} / l with l = sum_j e^{S_i,j - m} */
    double l = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* O_i = sum_j P_i,j V_j */
    for (int64_t j = j0; j < j1; ++j) {
        const uint16_t* vj = rr.vh + j * d->dv;
        double p = s[j] / l;
        for (int64_t c = 0; c < d->dv; ++c)
            o_row[c] += p * widen(d, vj[c]);
    }
    *lse_out = m + log(l);
}

/*
 * oracle_attn_rows_range: exact attention for a list of query rows (or all
 * rows when rows == NULL, in which case n_rows must equal B*Hq*Lq), with the
 * softmax taken over the visible keys in [k_begin, k_end) only.  That is the
 * partial state of one key segment: its normalised output and its
 * log-sum-exp, lse = -inf (and O = 0) where the segment holds no visible key.
 * ("Infra: Flash Attention", section on prefill versus decode: the key
 * sequence may be cut into segments computed separately and merged.)
 * Returns 0 on success, nonzero on bad arguments.
 */
int oracle_attn_rows_elem(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                          int64_t dqk, int64_t dv, int causal, double scale,
                          int64_t k_begin, int64_t k_end,
                          const int64_t* rows, int64_t n_rows,
                          double* o, double* lse, int n_threads, int elem)
{
    dims_t d = {B, Hq, Hkv, Lq, Lk, dqk, dv, causal, scale, elem};
    if (elem != ELEM_BF16 && elem != ELEM_FP16)
        return 8;
    int rc = check_dims(&d);
    if (rc)
        return rc;
    if (!q || !k || !v || !o || !lse)
        return 4;
    int64_t total = B * Hq * Lq;
    if (!rows && n_rows != total)
        return 5;
    if (rows)
        for (int64_t t = 0; t < n_rows; ++t)
            if (rows[t] < 0 || rows[t] >= total)
                return 6;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

    int failed = 0;
#pragma omp parallel
    {
        double* qd = (double*)malloc(sizeof(double) * (size_t)dqk);
        double* s = (double*)malloc(sizeof(double) * (size_t)Lk);
        int ok = qd && s;
        /* every thread reaches the worksharing loop, even after a failed
         * allocation, so the loop's barrier cannot deadlock */
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < n_rows; ++t) {
            if (!ok) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            int64_t r = rows ? rows[t] : t;
            row_ref_t rr = locate_row(&d, q, k, v, r);
            exact_row(&d, rr, k_begin, k_end, qd, s, o + t * dv, lse + t);
        }
        free(qd);
        free(s);
    }
    return failed ? 7 : 0;
}

/* oracle_attn_rows_range: oracle_attn_rows_elem on bf16 inputs. */
int oracle_attn_rows_range(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                           int64_t dqk, int64_t dv, int causal, double scale,
                           int64_t k_begin, int64_t k_end,
                           const int64_t* rows, int64_t n_rows,
                           double* o, double* lse, int n_threads)
{
    return oracle_attn_rows_elem(q, k, v, B, Hq, Hkv, Lq, Lk, dqk, dv, causal, scale, k_begin,
                                 k_end, rows, n_rows, o, lse, n_threads, ELEM_BF16);
}

/* oracle_attn_rows: the whole definition, every visible key of each row. */
int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                     int64_t dqk, int64_t dv, int causal, double scale,
                     const int64_t* rows, int64_t n_rows,
                     double* o, double* lse, int n_threads)
{
    return oracle_attn_rows_range(q, k, v, B, Hq, Hkv, Lq, Lk, dqk, dv, causal, scale, 0, Lk,
                                  rows, n_rows, o, lse, n_threads);
}

/*
 * oracle_merge_states: combine the partial states of n_parts key segments,
 * row by row, with the two-block merge rule of "Infra: Flash Attention"
 * (section on computing softmax in segments):
 *     m = max(m_A, m_B),  alpha = e^{m_A - m},  beta = e^{m_B - m},
 *     l = alpha l_A + beta l_B,  u = alpha u_A + beta u_B,  O = u / l.
 * A finished segment with normalised output O_g and log-sum-exp lse_g is the
 * state (m, l, u) = (lse_g, 1, O_g): with the reference at lse_g the
 * denominator sum_j e^{x_j - lse_g} is exactly 1.  The segments are folded
 * left to right into one state; a segment with lse = -inf holds no key and
 * is passed over.  The result is O = u / l and lse = m + ln l, or O = 0 and
 * lse = -inf when no segment holds a key.
 * Layouts: o_parts [n_parts, n_rows, dv], lse_parts [n_parts, n_rows],
 * o [n_rows, dv], lse [n_rows].
 */
int oracle_merge_states(const double* o_parts, const double* lse_parts, int64_t n_parts,
                        int64_t n_rows, int64_t dv, double* o, double* lse)
{
    if (!o_parts || !lse_parts || !o || !lse || n_parts < 1 || n_rows < 0 || dv < 1)
        return 1;
    for (int64_t r = 0; r < n_rows; ++r) {
        double m = -INFINITY, l = 0.0;
        double* u = o + r * dv;
        for (int64_t c = 0; c < dv; ++c)
            u[c] = 0.0;
        for (int64_t g = 0; g < n_parts; ++g) {
            double mb = lse_parts[g * n_rows + r];
            if (mb == -INFINITY)
                continue;
            const double* ob = o_parts + (g * n_rows + r) * dv;
            double mm = m > mb ? m : mb;
            double alpha = (m == -INFINITY) ? 0.0 : exp(m - mm);
            double beta = exp(mb - mm);
            l = alpha * l + beta * 1.0;
            for (int64_t c = 0; c < dv; ++c)
                u[c] = alpha * u[c] + beta * ob[c];
            m = mm;
        }
        if (m == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        for (int64_t c = 0; c < dv; ++c)
            u[c] /= l;
        lse[r] = m + log(l);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 1b. Variable-length batches: the definition inside each packed sequence.  */
/* ------------------------------------------------------------------------ */

/*
 * oracle_attn_varlen: exact attention over a batch of n_seq sequences of
 * different lengths packed along the token axis ("Flash Attention 4 ..."
 * review, method part on scheduling: variable-length batches, ordered by
 * work-tile execution time).  Sequence s owns query tokens
 * [cu_q[s], cu_q[s+1]) and key tokens [cu_k[s], cu_k[s+1]); a query sees only
 * the keys of its own sequence, with the causal mask aligned bottom-right
 * within the sequence (query i of Lq_s sees keys j <= i + Lk_s - Lq_s).
 * Layouts (contiguous, token-major):
 *   q [total_q, Hq, dqk]   k [total_k, Hkv, dqk]   v [total_k, Hkv, dv]
 *   row index r = h * total_q + t for query head h and token t (the layout
 *   of lse, [Hq, total_q]); o [n_rows, dv] and lse [n_rows] in double.
 * cu_q and cu_k hold n_seq + 1 non-decreasing offsets starting at 0.  A
 * sequence may be empty; a row whose sequence has no visible key gets O = 0
 * and lse = -inf.  rows == NULL means every row in order (n_rows must then
 * be Hq * total_q).  elem selects bf16 or fp16 inputs.
 */
int oracle_attn_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int64_t* cu_q, const int64_t* cu_k, int64_t n_seq,
                       int64_t Hq, int64_t Hkv, int64_t dqk, int64_t dv, int causal,
                       double scale, const int64_t* rows, int64_t n_rows,
                       double* o, double* lse, int n_threads, int elem)
{
    if (!q || !k || !v || !o || !lse || !cu_q || !cu_k)
        return 4;
    if (n_seq < 1 || Hq < 1 || Hkv < 1 || dqk < 1 || dv < 1 || Hq % Hkv != 0)
        return 1;
    if (!(scale > 0.0) || !isfinite(scale))
        return 3;
    if (elem != ELEM_BF16 && elem != ELEM_FP16)
        return 8;
    if (cu_q[0] != 0 || cu_k[0] != 0)
        return 9;
    for (int64_t s = 0; s < n_seq; ++s)
        if (cu_q[s + 1] < cu_q[s] || cu_k[s + 1] < cu_k[s])
            return 9;
    const int64_t total_q = cu_q[n_seq], total_k = cu_k[n_seq];
    const int64_t total = Hq * total_q;
    if (!rows && n_rows != total)
        return 5;
    if (rows)
        for (int64_t t = 0; t < n_rows; ++t)
            if (rows[t] < 0 || rows[t] >= total)
                return 6;
    int64_t max_lk = 1;
    for (int64_t s = 0; s < n_seq; ++s)
        if (cu_k[s + 1] - cu_k[s] > max_lk)
            max_lk = cu_k[s + 1] - cu_k[s];
    (void)total_k;
    dims_t d;
    memset(&d, 0, sizeof d);
    d.elem = elem;
    const int64_t group = Hq / Hkv;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

    int failed = 0;
#pragma omp parallel
    {
        double* qd = (double*)malloc(sizeof(double) * (size_t)dqk);
        double* s = (double*)malloc(sizeof(double) * (size_t)max_lk);
        int ok = qd && s;
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < n_rows; ++t) {
            if (!ok) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            const int64_t r = rows ? rows[t] : t;
            const int64_t h = r / total_q;
            const int64_t tok = r % total_q;
            const int64_t kvh = h / group;
            /* the sequence holding this token: cu_q[sq] <= tok < cu_q[sq + 1] */
            int64_t sq = 0;
            while (cu_q[sq + 1] <= tok)
                ++sq;
            const int64_t Lq = cu_q[sq + 1] - cu_q[sq];
            const int64_t Lk = cu_k[sq + 1] - cu_k[sq];
            const int64_t i = tok - cu_q[sq];
            /* visible keys of query i within its sequence */
            int64_t n = Lk;
            if (causal) {
                const int64_t last = i + Lk - Lq;
                n = last < 0 ? 0 : (last + 1 < Lk ? last + 1 : Lk);
            }
            double* o_row = o + t * dv;
            for (int64_t c = 0; c < dv; ++c)
                o_row[c] = 0.0;
            if (n == 0) {
                lse[t] = -INFINITY;
                continue;
            }
            const uint16_t* qrow = q + (tok * Hq + h) * dqk;
            for (int64_t c = 0; c < dqk; ++c)
                qd[c] = widen(&d, qrow[c]);
            /* S_j = scale * q . k_j over the sequence's visible keys */
            double m = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                const uint16_t* kj = k + ((cu_k[sq] + j) * Hkv + kvh) * dqk;
                double dot = 0.0;
                for (int64_t c = 0; c < dqk; ++c)
                    dot += qd[c] * widen(&d, kj[c]);
                s[j] = scale * dot;
                if (s[j] > m)
                    m = s[j];
            }
            /* P_j = e^{S_j - m} / l, O = sum_j P_j V_j, lse = m + ln l */
            double l = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const double e = exp(s[j] - m);
                s[j] = e;
                l += e;
            }
            for (int64_t j = 0; j < n; ++j) {
                const uint16_t* vj = v + ((cu_k[sq] + j) * Hkv + kvh) * dv;
                const double p = s[j] / l;
                for (int64_t c = 0; c < dv; ++c)
                    o_row[c] += p * widen(&d, vj[c]);
            }
            lse[t] = m + log(l);
        }
        free(qd);
        free(s);
    }
    return failed ? 7 : 0;
}

/* ------------------------------------------------------------------------ */
/* 2. The tiled method, block by block over K/V, for checking the algorithm. */
/* ------------------------------------------------------------------------ */
/*
 * mode 0 -- always rescale, natural exponent ("Infra: Flash Attention",
 *           Algorithm 1, FlashAttention-2 form):
 *             m' = max(m, rowmax S);  alpha = e^{m - m'};  W = e^{S - m'}
 *             l = alpha*l + rowsum W;  U = alpha*U + W V;  m = m'
 *           finally O = U / l and L = m + log l.  A row whose whole tile is
 *           masked skips the update (the pages' boundary conditions).
 * mode 1 -- conditional rescaling in base 2 ("Flash Attention 4 ..." ch. 13,
 *           section on online softmax and conditional rescaling):
 *           the reference r is kept in raw-score units (unscaled q.k);
 *           scale_log2 = log2(e) * scale;  the first block with a visible key
 *           adopts its own max with acc_scale = 1; afterwards
 *             cand = max(r, rowmax X);  delta = (r - cand) * scale_log2
 *             delta >= -tau : keep r, acc_scale = 1
 *             delta <  -tau : r = cand, acc_scale = 2^delta (a rescale event)
 *           l = acc_scale*l + sum 2^{(x - r)*scale_log2};  U likewise with V.
 *           Finally O = U / l and lse = scale*r + ln l (natural log; equal to
 *           the definition because u(r)/l(r) does not depend on r, "Infra:
 *           Flash Attention", section on why the exponent reference may lag).
 * mode 2 -- as mode 1, but the switch decision is shared by a group of
 *           `group` consecutive query rows of one head: if any row in the
 *           group needs a rescale, every row of the group moves its reference
 *           to its own candidate max (the FA4 review's wording that the whole
 *           warp rescales when any thread needs it).
 *
 * Inputs as for oracle_attn_rows; bn = keys per block.  rows lists query
 * rows (NULL = all).  Optional outputs: state[2*t] = final reference (mode 0:
 * m in scaled units; modes 1/2: r in raw units), state[2*t+1] = final l;
 * n_rescale (one counter for the whole call) counts rescale events.
 */

typedef struct {
    double ref;  /* running reference (-inf before the first visible key) */
    double l;    /* running denominator relative to ref */
    double* u;   /* running numerator, dv values */
    int64_t n;   /* visible keys of this row */
    int64_t i;   /* query position */
    int64_t events; /* blocks after the first at which the state was rescaled */
    row_ref_t rr;
    double* qd;
} online_state_t;

static void online_rows_group(const dims_t* d, int mode, int64_t bn, double tau,
                              online_state_t* st, int64_t g, double* x,
                              double* bmax, int* wants)
{
    const double scale_log2 = d->scale / M_LN2; /* = log2(e) * scale */
    int64_t nmax = 0;
    for (int64_t a = 0; a < g; ++a)
        if (st[a].n > nmax)
            nmax = st[a].n;

    for (int64_t j0 = 0; j0 < nmax; j0 += bn) {
        int64_t j1 = j0 + bn < d->Lk ? j0 + bn : d->Lk;
        int any_switch = 0;
        /* pass 1: raw scores x_ij of this block and the per-row decision */
        for (int64_t a = 0; a < g; ++a) {
            online_state_t* s = &st[a];
            bmax[a] = -INFINITY;
            wants[a] = 0;
            for (int64_t j = j0; j < j1; ++j) {
                double* xj = &x[a * bn + (j - j0)];
                if (j >= s->n) {
                    *xj = -INFINITY; /* masked (future key or past the end) */
                    continue;
                }
                const uint16_t* kj = s->rr.kh + j * d->dqk;
                double dot = 0.0;
                for (int64_t c = 0; c < d->dqk; ++c)
                    dot += s->qd[c] * widen(d, kj[c]);
                *xj = (mode == 0) ? d->scale * dot : dot;
                if (*xj > bmax[a])
                    bmax[a] = *xj;
            }
            if (mode != 0 && bmax[a] > -INFINITY && s->ref > -INFINITY) {
                double cand = bmax[a] > s->ref ? bmax[a] : s->ref;
                double delta = (s->ref - cand) * scale_log2;
                if (delta < -tau)
                    wants[a] = 1;
            }
            any_switch |= wants[a];
        }
        /* pass 2: update each row's state */
        for (int64_t a = 0; a < g; ++a) {
            online_state_t* s = &st[a];
            if (bmax[a] == -INFINITY)
                continue; /* the whole tile row is masked: skip the update */
            double acc_scale;
            double* xa = &x[a * bn];
            if (mode == 0) {
                double m_new = bmax[a] > s->ref ? bmax[a] : s->ref;
                acc_scale = exp(s->ref - m_new); /* e^{-inf} = 0 at the start */
                s->ref = m_new;
                s->l *= acc_scale;
                for (int64_t c = 0; c < d->dv; ++c)
                    s->u[c] *= acc_scale;
                for (int64_t j = j0; j < j1; ++j) {
                    double w = exp(xa[j - j0] - s->ref); /* e^{-inf} = 0 */
                    if (w == 0.0)
                        continue;
                    s->l += w;
                    const uint16_t* vj = s->rr.vh + j * d->dv;
                    for (int64_t c = 0; c < d->dv; ++c)
                        s->u[c] += w * widen(d, vj[c]);
                }
                continue;
            }
            if (s->ref == -INFINITY) {
                /* first block with a visible key: adopt its max */
                s->ref = bmax[a];
                acc_scale = 1.0;
            } else {
                double cand = bmax[a] > s->ref ? bmax[a] : s->ref;
                int do_switch = (mode == 1) ? wants[a] : any_switch;
                if (do_switch) {
                    acc_scale = exp2((s->ref - cand) * scale_log2);
                    s->ref = cand;
                    ++s->events;
                } else {
                    acc_scale = 1.0;
                }
            }
            s->l *= acc_scale;
            for (int64_t c = 0; c < d->dv; ++c)
                s->u[c] *= acc_scale;
            for (int64_t j = j0; j < j1; ++j) {
                double xv = xa[j - j0];
                if (xv == -INFINITY)
                    continue;
                double w = exp2((xv - s->ref) * scale_log2);
                s->l += w;
                const uint16_t* vj = s->rr.vh + j * d->dv;
                for (int64_t c = 0; c < d->dv; ++c)
                    s->u[c] += w * widen(d, vj[c]);
            }
        }
    }
}

int oracle_online_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                       int64_t dqk, int64_t dv, int causal, double scale,
                       int64_t bn, int mode, double tau, int64_t group,
                       const int64_t* rows, int64_t n_rows,
                       double* o, double* lse, double* state,
                       int64_t* n_rescale, int n_threads)
{
    dims_t d = {B, Hq, Hkv, Lq, Lk, dqk, dv, causal, scale, ELEM_BF16};
    int rc = check_dims(&d);
    if (rc)
        return rc;
    if (!q || !k || !v || !o || !lse)
        return 4;
    if (bn < 1 || mode < 0 || mode > 2 || !(tau >= 0.0) || (mode == 2 && group < 1))
        return 8;
    if (mode != 2)
        group = 1;
    int64_t total = B * Hq * Lq;
    if (!rows && n_rows != total)
        return 5;
    if (rows)
        for (int64_t t = 0; t < n_rows; ++t)
            if (rows[t] < 0 || rows[t] >= total)
                return 6;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

    int64_t events = 0;
    int failed = 0;
#pragma omp parallel reduction(+ : events)
    {
        online_state_t* st = (online_state_t*)calloc((size_t)group, sizeof *st);
        double* ubuf = (double*)malloc(sizeof(double) * (size_t)(group * dv));
        double* qbuf = (double*)malloc(sizeof(double) * (size_t)(group * dqk));
        double* x = (double*)malloc(sizeof(double) * (size_t)(group * bn));
        double* bmax = (double*)malloc(sizeof(double) * (size_t)group);
        int* wants = (int*)malloc(sizeof(int) * (size_t)group);
        int ok = st && ubuf && qbuf && x && bmax && wants;
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < n_rows; ++t) {
            if (!ok) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            {
                int64_t r = rows ? rows[t] : t;
                /* The group holding row r: rows of the same (b, h) whose
                 * positions share i / group.  Every member is computed so the
                 * shared decision is taken over the whole group. */
                int64_t i = r % Lq;
                int64_t first = r - (i % group);
                int64_t g = group;
                if ((i - i % group) + g > Lq)
                    g = Lq - (i - i % group);
                int64_t mine = r - first;
                for (int64_t a = 0; a < g; ++a) {
                    st[a].rr = locate_row(&d, q, k, v, first + a);
                    st[a].i = st[a].rr.i;
                    st[a].n = valid_keys(&d, st[a].i);
                    st[a].ref = -INFINITY;
                    st[a].l = 0.0;
                    st[a].events = 0;
                    st[a].u = ubuf + a * dv;
                    st[a].qd = qbuf + a * dqk;
                    for (int64_t c = 0; c < dv; ++c)
                        st[a].u[c] = 0.0;
                    for (int64_t c = 0; c < dqk; ++c)
                        st[a].qd[c] = widen(&d, st[a].rr.qrow[c]);
                }
                online_rows_group(&d, mode, bn, tau, st, g, x, bmax, wants);
                online_state_t* s = &st[mine];
                double* orow = o + t * dv;
                if (s->l > 0.0) {
                    for (int64_t c = 0; c < dv; ++c)
                        orow[c] = s->u[c] / s->l;
                    lse[t] = (mode == 0) ? s->ref + log(s->l)
                                         : scale * s->ref + log(s->l);
                } else {
                    for (int64_t c = 0; c < dv; ++c)
                        orow[c] = 0.0;
                    lse[t] = -INFINITY;
                }
                if (state) {
                    state[2 * t] = s->ref;
                    state[2 * t + 1] = s->l;
                }
                events += s->events; /* events of the requested row only */
            }
        }
        free(st);
        free(ubuf);
        free(qbuf);
        free(x);
        free(bmax);
        free(wants);
    }
    if (n_rescale)
        *n_rescale = events;
    return failed ? 7 : 0;
}

/* ------------------------------------------------------------------------ */
/* 3. The backward pass: gradients of the definition.                       */
/* ------------------------------------------------------------------------ */

/*
 * oracle_attn_bwd: dQ, dK, dV of L(Q, K, V) = <dO, O(Q, K, V)> for the
 * definition above, following the backward section of "Infra: Flash
 * Attention" (gradients by recomputation):
 *     P = softmax(scale * Q K^T)              (rows over the visible keys)
 *     dV = P^T dO,   dP = dO V^T,
 *     D_i = sum_j P_ij dP_ij                  (= dO_i . O_i),
 *     dS_ij = P_ij (dP_ij - D_i),
 *     dQ = scale * dS K,   dK = scale * dS^T Q.
 * With grouped-query attention a K/V head's dK and dV sum the contributions
 * of all query heads it serves.  A row with no visible key contributes
 * nothing.  Inputs are 16-bit bit patterns (elem as in
 * oracle_attn_rows_elem): q, k, v, dout contiguous [B, H, L, d]; outputs in
 * double: dq [B, Hq, Lq, dqk], dk [B, Hkv, Lk, dqk], dv [B, Hkv, Lk, dv], and
 * delta [B, Hq, Lq] (the D_i above).  Parallel over the query rows of one
 * K/V head at a time.
 */
int oracle_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const uint16_t* dout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                    int64_t Lk, int64_t dqk, int64_t dv, int causal, double scale, int elem,
                    double* dq, double* dk, double* dvo, double* delta, int n_threads)
{
    dims_t d = {B, Hq, Hkv, Lq, Lk, dqk, dv, causal, scale, elem};
    if (elem != ELEM_BF16 && elem != ELEM_FP16)
        return 8;
    int rc = check_dims(&d);
    if (rc)
        return rc;
    if (!q || !k || !v || !dout || !dq || !dk || !dvo || !delta)
        return 4;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
    const int nthr = omp_get_max_threads();
#else
    (void)n_threads;
    const int nthr = 1;
#endif
    const int64_t group = Hq / Hkv;
    int failed = 0;
    /* One K/V head at a time; its query rows (of every query head it serves)
     * are shared out over the threads, each summing its rows' dK and dV
     * contributions into a buffer of its own, added up afterwards. */
    double* part_k = (double*)malloc(sizeof(double) * (size_t)(nthr * Lk * dqk));
    double* part_v = (double*)malloc(sizeof(double) * (size_t)(nthr * Lk * dv));
    if (!part_k || !part_v) {
        free(part_k);
        free(part_v);
        return 7;
    }
    for (int64_t bk = 0; bk < B * Hkv && !failed; ++bk) {
        const int64_t b = bk / Hkv, hk = bk % Hkv;
        const uint16_t* kh = k + bk * Lk * dqk;
        const uint16_t* vh = v + bk * Lk * dv;
        for (int64_t t = 0; t < nthr * Lk * dqk; ++t)
            part_k[t] = 0.0;
        for (int64_t t = 0; t < nthr * Lk * dv; ++t)
            part_v[t] = 0.0;
#pragma omp parallel
        {
#ifdef _OPENMP
            const int tid = omp_get_thread_num();
#else
            const int tid = 0;
#endif
            double* dkh = part_k + (int64_t)tid * Lk * dqk;
            double* dvh = part_v + (int64_t)tid * Lk * dv;
            double* qd = (double*)malloc(sizeof(double) * (size_t)dqk);
            double* gd = (double*)malloc(sizeof(double) * (size_t)dv);
            double* p = (double*)malloc(sizeof(double) * (size_t)Lk);
            double* dp = (double*)malloc(sizeof(double) * (size_t)Lk);
            int ok = qd && gd && p && dp;
#pragma omp for schedule(static, 16)
            for (int64_t hi = 0; hi < group * Lq; ++hi) {
                if (!ok) {
#pragma omp atomic write
                    failed = 1;
                    continue;
                }
                const int64_t h = hk * group + hi / Lq, i = hi % Lq;
                const int64_t r = (b * Hq + h) * Lq + i;
                const uint16_t* qrow = q + r * dqk;
                const uint16_t* grow = dout + r * dv;
                double* dqrow = dq + r * dqk;
                for (int64_t c = 0; c < dqk; ++c)
                    dqrow[c] = 0.0;
                const int64_t n = valid_keys(&d, i);
                if (n == 0) {
                    delta[r] = 0.0;
                    continue;
                }
                for (int64_t c = 0; c < dqk; ++c)
                    qd[c] = widen(&d, qrow[c]);
                for (int64_t c = 0; c < dv; ++c)
                    gd[c] = widen(&d, grow[c]);
                /* P_i. over the visible keys (safe softmax) */
                double m = -INFINITY;
                for (int64_t j = 0; j < n; ++j) {
                    double dot = 0.0;
                    for (int64_t c = 0; c < dqk; ++c)
                        dot += qd[c] * widen(&d, kh[j * dqk + c]);
                    p[j] = scale * dot;
                    if (p[j] > m)
                        m = p[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j < n; ++j) {
                    p[j] = exp(p[j] - m);
                    l += p[j];
                }
                for (int64_t j = 0; j < n; ++j)
                    p[j] /= l;
                /* dP_ij = dO_i . V_j and D_i = sum_j P_ij dP_ij */
                double di = 0.0;
                for (int64_t j = 0; j < n; ++j) {
                    double dot = 0.0;
                    for (int64_t c = 0; c < dv; ++c)
                        dot += gd[c] * widen(&d, vh[j * dv + c]);
                    dp[j] = dot;
                    di += p[j] * dot;
                }
                delta[r] = di;
                for (int64_t j = 0; j < n; ++j) {
                    const double ds = p[j] * (dp[j] - di);
                    /* dV_j += P_ij dO_i;  dK_j += scale dS_ij Q_i;  dQ_i += scale dS_ij K_j */
                    for (int64_t c = 0; c < dv; ++c)
                        dvh[j * dv + c] += p[j] * gd[c];
                    for (int64_t c = 0; c < dqk; ++c) {
                        dkh[j * dqk + c] += scale * ds * qd[c];
                        dqrow[c] += scale * ds * widen(&d, kh[j * dqk + c]);
                    }
                }
            }
            free(qd);
            free(gd);
            free(p);
            free(dp);
        }
        /* the threads' partial sums, in thread order */
        double* dkh = dk + bk * Lk * dqk;
        double* dvh = dvo + bk * Lk * dv;
        for (int64_t t = 0; t < Lk * dqk; ++t) {
            double acc = 0.0;
            for (int th = 0; th < nthr; ++th)
                acc += part_k[(int64_t)th * Lk * dqk + t];
            dkh[t] = acc;
        }
        for (int64_t t = 0; t < Lk * dv; ++t) {
            double acc = 0.0;
            for (int th = 0; th < nthr; ++th)
                acc += part_v[(int64_t)th * Lk * dv + t];
            dvh[t] = acc;
        }
    }
    free(part_k);
    free(part_v);
    return failed ? 7 : 0;
}
