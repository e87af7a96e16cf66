/*
 * dsa_oracle.c -- plain CPU reference of the DSA layer step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is
 * checked against.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load it; the product library never calls it, and the two
 * share no source, header, table or helper.
 *
 * Arithmetic: IEEE double throughout.  A result that the method stores as
 * float (an index score) is rounded once, at the end.  Inputs arrive in their
 * storage format (f32, bf16 bits, OCP e4m3fn codes, or f64) and are decoded
 * here with decoders written from the format definitions.
 *
 * Sources (the pages this follows):
 *  - "Module glm5next_dsa_ref" (metrale docs): index_scores, visible,
 *    topk_pools, expand_selection, topk_to_mask, pool_states, kept_pools,
 *    mla_masked_attention, the INVALID sentinel and the invariants list.
 *  - "GLM-5.2: the DSA sparse attention moves onto the pure fak kernel":
 *    the section "The selection stays host-side BY DESIGN" (index score with
 *    per-head weights, relu and scale; selection in f64) and the table under
 *    "What changed" (per-head softmax(scale*q*k) and in-order sum of w*V,
 *    key width different from value width).
 *  - "Another DSA attempt" (ik_llama.cpp PR #2063), the squashed commit
 *    message of the batch-local indexer: relu(k.q), scaled per-head weights
 *    summed over heads, causal mask, top_k(min(top_k, n_tokens)).
 *
 * Parallelism: OpenMP over query rows only.  Each row is computed start to
 * finish by one thread in a fixed order, so results do not depend on the
 * thread count.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_INVALID (-1)

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_F64 = 3 };

/* ------------------------------------------------------------------------ */
/* Storage-format decoders (from the format definitions).                    */
/* ------------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits.  Exponent field 0 holds subnormals m * 2^-9.  There is no
 * infinity; S.1111.111 is NaN, so the largest finite magnitude is
 * 1.75 * 2^8 = 448. */
double orc_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

static double load(const void *p, int dtype, int64_t i)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_BF16: return orc_bf16_value(((const uint16_t *)p)[i]);
    case ORC_E4M3: return orc_e4m3_value(((const uint8_t *)p)[i]);
    default: return ((const double *)p)[i];
    }
}

/* ------------------------------------------------------------------------ */
/* Visibility ("visible": causal and not padding).                           */
/* ------------------------------------------------------------------------ */

/* A token key s is visible to the query at position qpos of a sequence with
 * `pad` left-padding tokens iff it is not padding and not in the future.  The
 * query's own position counts as visible. */
int orc_token_visible(int32_t pad, int32_t qpos, int64_t s)
{
    return s >= pad && s <= qpos;
}

/* Pool i (pooling starts at the first valid token) covers the tokens
 * pad + i*kpool .. pad + i*kpool + kpool - 1.  It is a candidate for the query
 * at qpos iff the query is not padding and every token of the pool is
 * visible to it, i.e. its last token is at or before qpos. */
int orc_pool_visible(int32_t pad, int32_t kpool, int32_t qpos, int64_t i)
{
    if (qpos < pad)
        return 0;
    return (int64_t)pad + (i + 1) * (int64_t)kpool - 1 <= (int64_t)qpos;
}

static int key_visible(int32_t pad, int32_t kpool, int32_t qpos, int64_t s)
{
    return kpool > 0 ? orc_pool_visible(pad, kpool, qpos, s)
                     : orc_token_visible(pad, qpos, s);
}

/* ------------------------------------------------------------------------ */
/* Index scores: score[q,s] = sum_h w[q,h] * relu(scale * q_h . k_s)        */
/* ------------------------------------------------------------------------ */

/* Rows are flat query ids r = b*Tq + t (all rows when `rows` is NULL).
 * q: [B,Tq,H,d]; k: [B,Tk,d] (one key head); k_scale: [B,Tk] multiplies the
 * decoded key (NULL = 1); w: [B,Tq,H] f32.  Invisible keys get -FLT_MAX.
 * A (optional) receives sum_h |w| |scale| sum_c |q_c k_c|, the magnitude that
 * bounds the rounding error of any evaluation order of the score.
 * Returns 0, or -1 if an input element is NaN. */
int orc_index_scores(int64_t B, int64_t Tq, int64_t Tk, int64_t H, int64_t d,
                     const void *q, int q_dtype, const void *k, int k_dtype,
                     const float *k_scale, const float *w, double scale,
                     const int32_t *q_pos, const int32_t *pad, int32_t kpool,
                     const int64_t *rows, int64_t n_rows, float *S, double *A)
{
    int bad = 0;
    (void)B;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t ri = 0; ri < n_rows; ++ri) {
        int64_t r = rows ? rows[ri] : ri;
        int64_t b = r / Tq;
        int32_t qp = q_pos[r];
        int32_t pd = pad[b];
        for (int64_t s = 0; s < Tk; ++s) {
            float *out = &S[ri * Tk + s];
            if (!key_visible(pd, kpool, qp, s)) {
                *out = -FLT_MAX;
                if (A)
                    A[ri * Tk + s] = 0.0;
                continue;
            }
            double ks = k_scale ? (double)k_scale[b * Tk + s] : 1.0;
            double total = 0.0, mag = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                double dot = 0.0, adot = 0.0;
                for (int64_t c = 0; c < d; ++c) {
                    double qv = load(q, q_dtype, (r * H + h) * d + c);
                    double kv = load(k, k_dtype, (b * Tk + s) * d + c) * ks;
                    dot += qv * kv;
                    adot += fabs(qv * kv);
                }
                double wh = (double)w[r * H + h];
                double logit = scale * dot;
                total += wh * (logit > 0.0 ? logit : 0.0);
                mag += fabs(wh) * fabs(scale) * adot;
            }
            if (isnan(total))
                bad = 1;
            *out = (float)total;
            if (A)
                A[ri * Tk + s] = mag;
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Top-k: higher score first, then smaller index.                            */
/* ------------------------------------------------------------------------ */

typedef struct {
    float score;
    int32_t idx;
} cand_t;

/* Total order of candidates: higher score first; equal scores (IEEE
 * equality, so +0 == -0) go to the smaller index. */
static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

/* Candidates of one row: the visible columns (token keys, or pools when
 * kpool > 0).  Returns the count, or -1 on a NaN score. */
static int64_t gather_candidates(const float *row, int64_t n_cols, int32_t pd,
                                 int32_t qp, int32_t kpool, cand_t *c)
{
    int64_t n = 0;
    for (int64_t s = 0; s < n_cols; ++s) {
        if (!key_visible(pd, kpool, qp, s))
            continue;
        if (isnan(row[s]))
            return -1;
        c[n].score = row[s];
        c[n].idx = (int32_t)s;
        ++n;
    }
    return n;
}

/* Attention-sink force-inclusion ("Another DSA attempt": the decode
 * indexer-K cache commit boosts the first key(s) so that the sink survives
 * top-k; the per-sequence sink commit adds the boost only to keys of the
 * query's own sequence; the serving-correctness commit anchors it on the
 * sequence's first PRESENT position).  The boost is an f32 addition of 1e20
 * to the score, as the pages' graph adds it before the top-k.  The sink keys
 * are the first n_sink candidates in column order -- the sequence's first
 * present positions that the query can see (the causal mask still applies
 * to them); for pooled keys, the first visible pools. */
static void add_sink_boost(cand_t *c, int64_t n, int32_t n_sink)
{
    for (int64_t j = 0; j < n && j < n_sink; ++j)
        c[j].score = c[j].score + 1e20f;
}

/* Per row: the min(k, #visible) visible columns in rank order, then INVALID
 * up to width k.  Row r's scores start at S + r*row_stride; its query
 * position and padding are row_qpos[r], row_pad[r].  n_sink > 0 boosts the
 * row's first n_sink visible columns (add_sink_boost) before ranking. */
int orc_topk(const float *S, int64_t n_rows, int64_t n_cols, int64_t row_stride,
             const int32_t *row_qpos, const int32_t *row_pad, int32_t kpool,
             int32_t k, int32_t n_sink, int32_t *out)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n_cols ? n_cols : 1));
        int64_t n = gather_candidates(S + r * row_stride, n_cols, row_pad[r],
                                      row_qpos[r], kpool, c);
        if (n < 0) {
            bad = 1;
            n = 0;
        }
        add_sink_boost(c, n, n_sink);
        qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
        for (int64_t i = 0; i < k; ++i)
            out[r * k + i] = i < n ? c[i].idx : ORC_INVALID;
        free(c);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Pool keys ("pool_states"): softmax over the slot axis, per channel.       */
/* ------------------------------------------------------------------------ */

/* k, gate: [B,L,d].  Pools start at the first valid token (pad[b]); pool i
 * holds tokens pad + i*kpool + j, j < kpool; a trailing partial pool is not a
 * pool, so n_pools[b] = floor((L - pad[b]) / kpool).  For each channel c,
 * pk = sum_j softmax_j(gate[t_j,c]) * k[t_j,c].  pk: [B, L/kpool, d] in f64;
 * rows i >= n_pools[b] are 0.  mag (optional, same shape) receives
 * sum_j softmax_j |k[t_j,c]|, which bounds the rounding error of any
 * evaluation of the weighted sum. */
int orc_pool_keys(int64_t B, int64_t L, int64_t d, int32_t kpool,
                  const void *k, int k_dtype, const void *gate, int g_dtype,
                  const int32_t *pad, double *pk, int32_t *n_pools, double *mag)
{
    int64_t np_max = L / kpool;
    for (int64_t b = 0; b < B; ++b) {
        int64_t valid = L - pad[b];
        int64_t np = valid > 0 ? valid / kpool : 0;
        n_pools[b] = (int32_t)np;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < np_max; ++i) {
            for (int64_t c = 0; c < d; ++c) {
                double *o = &pk[(b * np_max + i) * d + c];
                double *om = mag ? &mag[(b * np_max + i) * d + c] : NULL;
                if (i >= np) {
                    *o = 0.0;
                    if (om)
                        *om = 0.0;
                    continue;
                }
                int64_t t0 = pad[b] + i * kpool;
                double m = -INFINITY;
                for (int32_t j = 0; j < kpool; ++j) {
                    double g = load(gate, g_dtype, (b * L + t0 + j) * d + c);
                    if (g > m)
                        m = g;
                }
                double num = 0.0, den = 0.0, anum = 0.0;
                for (int32_t j = 0; j < kpool; ++j) {
                    double e = exp(load(gate, g_dtype, (b * L + t0 + j) * d + c) - m);
                    double kv = load(k, k_dtype, (b * L + t0 + j) * d + c);
                    num += e * kv;
                    anum += e * fabs(kv);
                    den += e;
                }
                *o = num / den;
                if (om)
                    *om = anum / den;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Pool select: topk_pools followed by expand_selection.                     */
/* ------------------------------------------------------------------------ */

/* Row r of S holds one query's scores over pools (row_stride apart).  The
 * candidates are the pools whose tokens are all visible (orc_pool_visible).
 * Up to select_k pools are taken in rank order (higher score, then smaller
 * pool id).  The token row lists each taken pool's kpool tokens ascending,
 * pools in rank order, then the visible tail -- the tokens after the last
 * complete visible pool up to and including the query -- ascending, then
 * INVALID up to out_width.  A padded query's row is all INVALID.
 * out_pools (optional) gets the pool ids, INVALID-padded to select_k.
 * Returns 0, -1 on NaN, -2 if a row would not fit in out_width. */
int orc_pool_select(const float *S, int64_t n_rows, int64_t n_cols,
                    int64_t row_stride, const int32_t *row_qpos,
                    const int32_t *row_pad, int32_t kpool, int32_t select_k,
                    int32_t out_width, int32_t *out_tok, int32_t *out_pools)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        int32_t pd = row_pad[r], qp = row_qpos[r];
        int32_t *tok = out_tok + r * out_width;
        for (int32_t i = 0; i < out_width; ++i)
            tok[i] = ORC_INVALID;
        if (out_pools)
            for (int32_t i = 0; i < select_k; ++i)
                out_pools[r * select_k + i] = ORC_INVALID;
        if (qp < pd)
            continue; /* padded query: stays all INVALID */
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n_cols ? n_cols : 1));
        int64_t n = gather_candidates(S + r * row_stride, n_cols, pd, qp, kpool, c);
        if (n < 0) {
            bad |= 1;
            n = 0;
        }
        qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
        int64_t take = n < select_k ? n : select_k;
        int64_t w = 0;
        for (int64_t i = 0; i < take; ++i) {
            if (out_pools)
                out_pools[r * select_k + i] = c[i].idx;
            for (int32_t j = 0; j < kpool; ++j) {
                if (w >= out_width) {
                    bad |= 2;
                    break;
                }
                tok[w++] = pd + c[i].idx * kpool + j;
            }
        }
        /* visible tail: n_full complete pools end before it */
        int64_t n_full = ((int64_t)qp - pd + 1) / kpool;
        for (int64_t t = pd + n_full * kpool; t <= qp; ++t) {
            if (w >= out_width) {
                bad |= 2;
                break;
            }
            tok[w++] = (int32_t)t;
        }
        free(c);
    }
    if (bad & 1)
        return -1;
    return (bad & 2) ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* topk_to_mask and sparse attention over the selected set.                  */
/* ------------------------------------------------------------------------ */

/* The selected set of one query: entries of its index row that are in
 * [0, Tk), not INVALID and (when pad/q_pos are given) visible; duplicates
 * collapse.  Written as a 0/1 mask over the Tk keys. */
void orc_topk_to_mask(const int32_t *idx_row, int64_t n_sel, int64_t Tk,
                      int has_vis, int32_t pd, int32_t qp, uint8_t *mask)
{
    memset(mask, 0, (size_t)Tk);
    for (int64_t i = 0; i < n_sel; ++i) {
        int64_t j = idx_row[i];
        if (j == ORC_INVALID || j < 0 || j >= Tk)
            continue;
        if (has_vis && !orc_token_visible(pd, qp, j))
            continue;
        mask[j] = 1;
    }
}

/* out[q,h,:] = sum_{j in J} softmax_j(scale * q_h . K_j) V_j over the selected
 * set J of the query, in ascending j.  lse = log sum_j exp(scale q_h.K_j).
 * An empty set gives out = 0, lse = -inf.
 * q: [B,Tq,H,kd].  Key row j of sequence b starts at K + (b*Tk + j)*k_row_stride
 * and holds kv_heads vectors of kd; head h reads kv head h / (H / kv_heads).
 * V likewise with vd and v_row_stride (V may alias K: absorbed MLA uses the
 * first vd columns of the latent row).  idx: [B,Tq,n_sel].  q_pos/pad may be
 * NULL (no visibility filter).  Rows as in orc_index_scores; out:
 * [n_rows,H,vd], lse: [n_rows,H] (optional). */
int orc_sparse_attend(int64_t B, int64_t Tq, int64_t Tk, int64_t H, int64_t kd,
                      int64_t vd, int64_t kv_heads, int64_t n_sel,
                      const void *q, int dtype, const void *K, int64_t k_row_stride,
                      const void *V, int64_t v_row_stride, const int32_t *idx,
                      const int32_t *q_pos, const int32_t *pad, double scale,
                      const int64_t *rows, int64_t n_rows, double *out, double *lse)
{
    (void)B;
    if (kv_heads <= 0 || H % kv_heads != 0)
        return -2;
    int64_t group = H / kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < n_rows; ++ri) {
        int64_t r = rows ? rows[ri] : ri;
        int64_t b = r / Tq;
        uint8_t *mask = (uint8_t *)malloc((size_t)(Tk ? Tk : 1));
        int64_t *J = (int64_t *)malloc(sizeof(int64_t) * (size_t)(Tk ? Tk : 1));
        double *logit = (double *)malloc(sizeof(double) * (size_t)(Tk ? Tk : 1));
        int has_vis = q_pos != NULL && pad != NULL;
        orc_topk_to_mask(idx + r * n_sel, n_sel, Tk, has_vis,
                         has_vis ? pad[b] : 0, has_vis ? q_pos[r] : 0, mask);
        int64_t nj = 0;
        for (int64_t j = 0; j < Tk; ++j)
            if (mask[j])
                J[nj++] = j;
        for (int64_t h = 0; h < H; ++h) {
            int64_t kvh = h / group;
            double *o = out + (ri * H + h) * vd;
            for (int64_t c = 0; c < vd; ++c)
                o[c] = 0.0;
            if (nj == 0) {
                if (lse)
                    lse[ri * H + h] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int64_t a = 0; a < nj; ++a) {
                int64_t krow = (b * Tk + J[a]) * k_row_stride + kvh * kd;
                double dot = 0.0;
                for (int64_t c = 0; c < kd; ++c)
                    dot += load(q, dtype, (r * H + h) * kd + c) * load(K, dtype, krow + c);
                logit[a] = scale * dot;
                if (logit[a] > m)
                    m = logit[a];
            }
            double den = 0.0;
            for (int64_t a = 0; a < nj; ++a) {
                double p = exp(logit[a] - m);
                int64_t vrow = (b * Tk + J[a]) * v_row_stride + kvh * vd;
                for (int64_t c = 0; c < vd; ++c)
                    o[c] += p * load(V, dtype, vrow + c);
                den += p;
            }
            for (int64_t c = 0; c < vd; ++c)
                o[c] /= den;
            if (lse)
                lse[ri * H + h] = m + log(den);
        }
        free(mask);
        free(J);
        free(logit);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Indexer-key cache write.                                                  */
/*                                                                           */
/* "Another DSA attempt" (ik_llama.cpp PR #2063), the commit message of the  */
/* decode indexer-K cache: the batch's indexer keys are Walsh-Hadamard       */
/* rotated -- orthonormal, so scores are unchanged -- and written into the   */
/* per-layer key cache at kv_head, from where scoring reads all past keys;   */
/* the queries get the same rotation.  The serving-correctness commit: the   */
/* rotation is the Sylvester construction, symmetric and orthonormal         */
/* (H*H = I).  The cache stores one fp8 e4m3 row with one f32 scale per key  */
/* (readings: scale = max|row| / 448, round to nearest even, saturating).    */
/* ------------------------------------------------------------------------ */

/* Entry (i, j) of the Sylvester Hadamard matrix of order 2^k: the sign
 * (-1)^(number of bit positions set in both i and j). */
static double sylvester_entry(int64_t i, int64_t j)
{
    return (__builtin_popcountll((unsigned long long)(i & j)) & 1) ? -1.0 : 1.0;
}

/* y[r][i] = (1/sqrt(d)) * sum_j H[i][j] x[r][j], the sum in f64 in column
 * order, then one multiplication by the f64 constant 1/sqrt(d).  y64 (may be
 * NULL) gets the f64 value, y32 (may be NULL) that value rounded once to f32.
 * d must be a power of two.  Returns -1 for a bad d. */
int orc_hadamard_rows(const void *x, int dtype, int64_t rows, int64_t d, double *y64, float *y32)
{
    if (d <= 0 || (d & (d - 1)) != 0)
        return -1;
    const double c = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < d; ++j)
                acc += sylvester_entry(i, j) * load(x, dtype, r * d + j);
            const double y = acc * c;
            if (y64)
                y64[r * d + i] = y;
            if (y32)
                y32[r * d + i] = (float)y;
        }
    }
    return 0;
}

/* OCP e4m3fn code of a finite f32: the representable value nearest to v,
 * ties to the code with an even last mantissa bit; magnitudes at or beyond
 * the largest finite value (448) give 448 (saturation).  The sign of v is
 * kept, so -0 and small negatives that round to zero give 0x80.  Found by
 * scanning the 127 non-negative finite codes, which are increasing in
 * value. */
uint8_t orc_e4m3_encode(float v)
{
    const int neg = signbit(v) ? 1 : 0;
    const double a = fabs((double)v);
    int best = 126;
    if (a < orc_e4m3_value(126)) {
        for (int c = 0; c < 126; ++c) {
            const double lo = orc_e4m3_value((uint8_t)c), hi = orc_e4m3_value((uint8_t)(c + 1));
            if (a >= lo && a <= hi) {
                const double dl = a - lo, dh = hi - a;
                if (dl < dh)
                    best = c;
                else if (dh < dl)
                    best = c + 1;
                else
                    best = (c & 1) ? c + 1 : c;
                break;
            }
        }
    }
    return (uint8_t)(best | (neg << 7));
}

/* One fp8 row per key: s = max_i |y_i| / 448 as an f32 division (1 when the
 * row is all zero), code_i = e4m3(y_i / s) with y_i / s an f32 division. */
void orc_quantize_e4m3_rows(const float *y, int64_t rows, int64_t d, uint8_t *codes,
                            float *scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float mx = 0.f;
        for (int64_t i = 0; i < d; ++i) {
            const float a = fabsf(y[r * d + i]);
            if (a > mx)
                mx = a;
        }
        volatile float s = mx / 448.0f;  /* one f32 division, not fused away */
        const float sc = mx > 0.f ? s : 1.0f;
        scales[r] = sc;
        for (int64_t i = 0; i < d; ++i) {
            volatile float q = y[r * d + i] / sc;
            codes[r * d + i] = orc_e4m3_encode(q);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* IndexShare ("Another DSA attempt": the IndexShare commit message and the  */
/* review comments around it).                                               */
/* ------------------------------------------------------------------------ */

/* GLM-5.2 marks some layers "full" (they compute their own indexer top-k)
 * and the rest "shared" (they reuse the selection of the most recent full
 * layer).  The rule the pages derive from the model config: layer il is
 * full iff il <= 1 or il % 4 == 2.  Returns the layer whose selection layer
 * il uses (il itself when full), or -1 for il < 0. */
int32_t orc_index_share_source(int32_t il)
{
    if (il < 0)
        return -1;
    for (int32_t l = il; l >= 0; --l)
        if (l <= 1 || l % 4 == 2)
            return l;
    return -1;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
