/*
 * oracle.c -- plain, slow fp64 reference of one sparse-KV decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes, step by step (the pages give no formulas, so each step is
 * the plainest reading of the passage cited next to it):
 *
 *  decode   bf16 is the upper half of an IEEE binary32; OCP fp8 e4m3fn has
 *           bias 7, subnormals 2^-6*m/8, no infinities, and S.1111.111 = NaN.
 *           An fp8 code is multiplied by its block's fp32 scale in fp64
 *           (exact: a 4-bit by 24-bit significand product fits in 53 bits).
 *  score    DualDecoder review, core claim and axiom ledger item 1: the
 *           retrieval index follows from the query and landmarks kept on the
 *           GPU, in the manner of QUEST and ShadowKV.  The landmark is the
 *           mean of a block's
 *           keys, so the score of block j for KV head g is the dot product of
 *           the query with it, summed over the query heads sharing g:
 *             s[b,t,g,j] = sum_{h in g} sum_i q[b,t,h,i] * lm[b,g,j,i].
 *           Candidates are the blocks holding a position before the recent
 *           window; other entries are -inf.  No 1/sqrt(d) (ranking only).
 *  select   PulseInfer section 2 (per-head sparse selection), DualDecoder
 *           ledger (a sparse KV budget in blocks): keep the k' = min(k_b,
 *           #candidates) blocks with the largest score, ties to the lowest
 *           block id; emit them in ascending block id, padded with -1.
 *  gather   PulseInfer section 2 (gather-scatter I/O engine) and DualDecoder
 *           Fig. 19 (contiguous block fetch plus a reorder): slot m of the
 *           staging buffer receives the bytes of the (pool block, head) chunk
 *           that the m-th selected logical block maps to.
 *  attend   Beyond abstract: dense attention over the recent window and
 *           per-head sparse attention over the selected blocks, fused by
 *           log-sum-exp.  Sparse set: positions of selected blocks below the
 *           window start; window set: the last W positions.  Logits
 *           z = q.k / sqrt(d); each part yields (m, l, o) with
 *           lse = m + ln l; the parts merge as
 *             o = sum_i e^{lse_i - M} o_i / sum_i e^{lse_i - M},
 *             lse = M + ln sum_i e^{lse_i - M}.
 *           An empty part has lse = -inf and weight 0.
 *           attend_tokens applies the same to every query token t (its own
 *           query and its own selection): the co-batched two-token attention
 *           of DualDecoder Fig. 18 computes exactly these values.
 *  overlap  DualDecoder core claim / Fig. 16: retrieval-index prediction
 *           accuracy = |I_real & I_spec| / |I_real| per (sequence, KV head).
 *
 * Parallelism: OpenMP over independent (sequence, KV head) pairs only; the
 * arithmetic inside a pair runs in the order written here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ------------------------------------------------------------------ decode */

double orc_bf16_value(uint16_t code) {
    uint32_t bits = ((uint32_t)code) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

double orc_e4m3fn_value(uint8_t code) {
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

static double load(const void *base, int dtype, int64_t idx) {
    switch (dtype) {
    case ORC_F32: return (double)((const float *)base)[idx];
    case ORC_BF16: return orc_bf16_value(((const uint16_t *)base)[idx]);
    case ORC_FP8: return orc_e4m3fn_value(((const uint8_t *)base)[idx]);
    }
    return NAN;
}

static int elem_size(int dtype) { return dtype == ORC_F32 ? 4 : dtype == ORC_BF16 ? 2 : 1; }

/* first element of the (pool block p, kv head g) chunk */
static int64_t chunk_offset(const orc_problem *pr, int64_t p, int g) {
    return p * pr->stride_block + (int64_t)g * pr->stride_head;
}

/* K or V element at sequence position pos of (b, g), dequantized */
static double kv_at(const orc_problem *pr, const void *pool, const float *scales,
                    const int32_t *block_table, int b, int g, int64_t pos, int i) {
    int j = (int)(pos / pr->blk);
    int r = (int)(pos % pr->blk);
    int64_t p = block_table[(int64_t)b * pr->max_blocks + j];
    double v = load(pool, pr->kv_dtype, chunk_offset(pr, p, g) + (int64_t)r * pr->d + i);
    if (pr->kv_dtype == ORC_FP8) v *= (double)scales[p * pr->Hkv + g];
    return v;
}

int orc_n_candidates(const orc_problem *pr, int L) {
    int ws = L - pr->window;
    if (ws < 0) ws = 0;
    return (ws + pr->blk - 1) / pr->blk;
}

/* ------------------------------------------------------------------- score */

void orc_scores(const orc_problem *pr, const void *q, const void *landmarks,
                const int32_t *seq_lens, double *scores) {
    const int G = pr->Hq / pr->Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < pr->B; ++b)
        for (int g = 0; g < pr->Hkv; ++g) {
            int nc = orc_n_candidates(pr, seq_lens[b]);
            for (int t = 0; t < pr->T; ++t) {
                double *row = scores + (((int64_t)b * pr->T + t) * pr->Hkv + g) * pr->max_blocks;
                for (int j = 0; j < pr->max_blocks; ++j) {
                    if (j >= nc) { row[j] = -INFINITY; continue; }
                    double s = 0.0;
                    for (int h = g * G; h < (g + 1) * G; ++h)
                        for (int i = 0; i < pr->d; ++i) {
                            double qv = load(q, pr->q_dtype, (((int64_t)b * pr->T + t) * pr->Hq + h) * pr->d + i);
                            double lv = load(landmarks, pr->lm_dtype,
                                             (((int64_t)b * pr->Hkv + g) * pr->max_blocks + j) * pr->d + i);
                            s += qv * lv;
                        }
                    row[j] = s;
                }
            }
        }
}

/* ------------------------------------------------------------------ select */

typedef struct { double s; int j; } scored;

static int by_score_then_id(const void *a, const void *b) {
    const scored *x = (const scored *)a, *y = (const scored *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int ascending_int(const void *a, const void *b) {
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

void orc_select(const orc_problem *pr, const double *scores, const int32_t *seq_lens,
                const int32_t *k_per_seq, int32_t *indices, int32_t *n_sel) {
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < pr->B; ++b)
        for (int g = 0; g < pr->Hkv; ++g) {
            int nc = orc_n_candidates(pr, seq_lens[b]);
            int k = k_per_seq[b] < nc ? k_per_seq[b] : nc;
            if (k < 0) k = 0;
            scored *cand = (scored *)malloc(sizeof(scored) * (nc > 0 ? nc : 1));
            int *chosen = (int *)malloc(sizeof(int) * (k > 0 ? k : 1));
            for (int t = 0; t < pr->T; ++t) {
                const double *row = scores + (((int64_t)b * pr->T + t) * pr->Hkv + g) * pr->max_blocks;
                for (int j = 0; j < nc; ++j) { cand[j].s = row[j]; cand[j].j = j; }
                qsort(cand, nc, sizeof(scored), by_score_then_id);
                for (int m = 0; m < k; ++m) chosen[m] = cand[m].j;
                qsort(chosen, k, sizeof(int), ascending_int);
                int32_t *out = indices + (((int64_t)b * pr->T + t) * pr->Hkv + g) * pr->k_max;
                for (int m = 0; m < pr->k_max; ++m) out[m] = m < k ? chosen[m] : -1;
                n_sel[((int64_t)b * pr->T + t) * pr->Hkv + g] = k;
            }
            free(cand);
            free(chosen);
        }
}

/* ----------------------------------------------------------------- overlap */

void orc_overlap(const orc_problem *pr, const int32_t *indices, const int32_t *n_sel, double *overlap) {
    for (int b = 0; b < pr->B; ++b)
        for (int g = 0; g < pr->Hkv; ++g) {
            const int32_t *i0 = indices + (((int64_t)b * pr->T + 0) * pr->Hkv + g) * pr->k_max;
            const int32_t *i1 = indices + (((int64_t)b * pr->T + 1) * pr->Hkv + g) * pr->k_max;
            int n0 = n_sel[((int64_t)b * pr->T + 0) * pr->Hkv + g];
            int n1 = n_sel[((int64_t)b * pr->T + 1) * pr->Hkv + g];
            int common = 0;
            for (int a = 0; a < n0; ++a)
                for (int c = 0; c < n1; ++c)
                    if (i0[a] == i1[c]) ++common;
            overlap[b * pr->Hkv + g] = n0 > 0 ? (double)common / (double)n0 : 1.0;
        }
}

/* ------------------------------------------------------------------ gather */

void orc_gather(const orc_problem *pr, const void *k_pool, const void *v_pool,
                const float *k_scales, const float *v_scales, const int32_t *block_table,
                const int32_t *indices, const int32_t *n_sel,
                void *k_stage, void *v_stage, float *k_stage_scales, float *v_stage_scales) {
    const int64_t chunk_elems = (int64_t)pr->blk * pr->d;
    const size_t chunk_bytes = (size_t)chunk_elems * elem_size(pr->kv_dtype);
    for (int b = 0; b < pr->B; ++b)
        for (int g = 0; g < pr->Hkv; ++g) {
            /* the real (first) query token's selection is gathered */
            const int32_t *idx = indices + (((int64_t)b * pr->T) * pr->Hkv + g) * pr->k_max;
            int n = n_sel[((int64_t)b * pr->T) * pr->Hkv + g];
            for (int m = 0; m < n; ++m) {
                int64_t p = block_table[(int64_t)b * pr->max_blocks + idx[m]];
                int64_t slot = ((int64_t)b * pr->Hkv + g) * pr->k_max + m;
                size_t es = (size_t)elem_size(pr->kv_dtype);
                memcpy((char *)k_stage + slot * chunk_bytes,
                       (const char *)k_pool + (size_t)chunk_offset(pr, p, g) * es, chunk_bytes);
                memcpy((char *)v_stage + slot * chunk_bytes,
                       (const char *)v_pool + (size_t)chunk_offset(pr, p, g) * es, chunk_bytes);
                if (pr->kv_dtype == ORC_FP8) {
                    k_stage_scales[slot] = k_scales[p * pr->Hkv + g];
                    v_stage_scales[slot] = v_scales[p * pr->Hkv + g];
                }
            }
        }
}

/* --------------------------------------------------------------- attention */

/*
 * Softmax partial of query head h of sequence b over an explicit list of
 * positions: m = max z, l = sum e^{z-m}, o = sum e^{z-m} v / l, lse = m + ln l.
 * An empty list gives lse = -inf and o = 0.
 */
static void partial_tok(const orc_problem *pr, const void *q, const void *k_pool, const void *v_pool,
                        const float *k_scales, const float *v_scales, const int32_t *block_table,
                        int b, int t, int h, const int64_t *pos, int n_pos, double *o, double *lse) {
    const int G = pr->Hq / pr->Hkv;
    const int g = h / G;
    const double inv_sqrt_d = 1.0 / sqrt((double)pr->d);
    for (int i = 0; i < pr->d; ++i) o[i] = 0.0;
    if (n_pos == 0) { *lse = -INFINITY; return; }
    double *z = (double *)malloc(sizeof(double) * n_pos);
    double m = -INFINITY;
    for (int n = 0; n < n_pos; ++n) {
        double dot = 0.0;
        for (int i = 0; i < pr->d; ++i) {
            double qv = load(q, pr->q_dtype, (((int64_t)b * pr->T + t) * pr->Hq + h) * pr->d + i);
            dot += qv * kv_at(pr, k_pool, k_scales, block_table, b, g, pos[n], i);
        }
        z[n] = dot * inv_sqrt_d;
        if (z[n] > m) m = z[n];
    }
    double l = 0.0;
    for (int n = 0; n < n_pos; ++n) {
        double w = exp(z[n] - m);
        l += w;
        for (int i = 0; i < pr->d; ++i)
            o[i] += w * kv_at(pr, v_pool, v_scales, block_table, b, g, pos[n], i);
    }
    for (int i = 0; i < pr->d; ++i) o[i] /= l;
    *lse = m + log(l);
    free(z);
}

void orc_partial(const orc_problem *pr, const void *q, const void *k_pool, const void *v_pool,
                 const float *k_scales, const float *v_scales, const int32_t *block_table,
                 int b, int h, const int64_t *pos, int n_pos, double *o, double *lse) {
    partial_tok(pr, q, k_pool, v_pool, k_scales, v_scales, block_table, b, 0, h, pos, n_pos, o, lse);
}

void orc_merge(int n_parts, int d, const double *o_parts, const double *lse_parts,
               double *o, double *lse) {
    double M = -INFINITY;
    for (int i = 0; i < n_parts; ++i)
        if (lse_parts[i] > M) M = lse_parts[i];
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (M == -INFINITY) { *lse = -INFINITY; return; }
    double den = 0.0;
    for (int i = 0; i < n_parts; ++i) {
        if (lse_parts[i] == -INFINITY) continue;
        double w = exp(lse_parts[i] - M);
        den += w;
        for (int c = 0; c < d; ++c) o[c] += w * o_parts[(int64_t)i * d + c];
    }
    for (int c = 0; c < d; ++c) o[c] /= den;
    *lse = M + log(den);
}

/* sparse positions: selected blocks' positions before the window start */
static int sparse_positions(const orc_problem *pr, int L, const int32_t *idx, int n, int64_t *pos) {
    int64_t ws = L - pr->window > 0 ? L - pr->window : 0;
    int cnt = 0;
    for (int m = 0; m < n; ++m)
        for (int r = 0; r < pr->blk; ++r) {
            int64_t p = (int64_t)idx[m] * pr->blk + r;
            if (p < ws) pos[cnt++] = p;
        }
    return cnt;
}

static int window_positions(const orc_problem *pr, int L, int64_t *pos) {
    int64_t ws = L - pr->window > 0 ? L - pr->window : 0;
    int cnt = 0;
    for (int64_t p = ws; p < L; ++p) pos[cnt++] = p;
    return cnt;
}

/* Attention of query token t of (b, g) over token t's own selection plus the
 * window: rows h of the group go to out_rows + (h - gG) * d, lse_rows[h - gG]
 * (and the two parts to part_o / part_lse when given). */
static void attend_pair(const orc_problem *pr, const void *q, const void *k_pool, const void *v_pool,
                        const float *k_scales, const float *v_scales, const int32_t *block_table,
                        const int32_t *seq_lens, const int32_t *indices, const int32_t *n_sel,
                        int b, int t, int g, double *out_rows, double *lse_rows, double *part_o,
                        double *part_lse) {
    const int G = pr->Hq / pr->Hkv;
    int L = seq_lens[b];
    const int32_t *idx = indices + (((int64_t)b * pr->T + t) * pr->Hkv + g) * pr->k_max;
    int n = n_sel[((int64_t)b * pr->T + t) * pr->Hkv + g];
    int64_t *sp = (int64_t *)malloc(sizeof(int64_t) * ((int64_t)n * pr->blk + 1));
    int64_t *wp = (int64_t *)malloc(sizeof(int64_t) * ((int64_t)pr->window + 1));
    int ns = sparse_positions(pr, L, idx, n, sp);
    int nw = window_positions(pr, L, wp);
    double *po = (double *)malloc(sizeof(double) * 2 * pr->d);
    double pl[2];
    for (int h = g * G; h < (g + 1) * G; ++h) {
        partial_tok(pr, q, k_pool, v_pool, k_scales, v_scales, block_table, b, t, h, sp, ns, po, &pl[0]);
        partial_tok(pr, q, k_pool, v_pool, k_scales, v_scales, block_table, b, t, h, wp, nw, po + pr->d, &pl[1]);
        const int r = h - g * G;
        if (part_o) {
            memcpy(part_o + (int64_t)r * 2 * pr->d, po, sizeof(double) * 2 * pr->d);
            part_lse[r * 2 + 0] = pl[0];
            part_lse[r * 2 + 1] = pl[1];
        }
        orc_merge(2, pr->d, po, pl, out_rows + (int64_t)r * pr->d, lse_rows + r);
    }
    free(po);
    free(sp);
    free(wp);
}

void orc_attend(const orc_problem *pr, const void *q, const void *k_pool, const void *v_pool,
                const float *k_scales, const float *v_scales, const int32_t *block_table,
                const int32_t *seq_lens, const int32_t *indices, const int32_t *n_sel,
                double *out, double *lse, double *part_o, double *part_lse) {
    const int G = pr->Hq / pr->Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < pr->B; ++b)
        for (int g = 0; g < pr->Hkv; ++g) {
            int64_t bh = (int64_t)b * pr->Hq + (int64_t)g * G;
            attend_pair(pr, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, indices, n_sel,
                        b, 0, g, out + bh * pr->d, lse + bh, part_o ? part_o + bh * 2 * pr->d : NULL,
                        part_lse ? part_lse + bh * 2 : NULL);
        }
}

/* DualDecoder Fig. 18 (the real and the speculative token attended together):
 * every query token t attends its own selection plus the window, exactly as
 * orc_attend does for token 0.  out [B][T][Hq][d], lse [B][T][Hq]. */
void orc_attend_tokens(const orc_problem *pr, const void *q, const void *k_pool, const void *v_pool,
                       const float *k_scales, const float *v_scales, const int32_t *block_table,
                       const int32_t *seq_lens, const int32_t *indices, const int32_t *n_sel,
                       double *out, double *lse) {
    const int G = pr->Hq / pr->Hkv;
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int b = 0; b < pr->B; ++b)
        for (int t = 0; t < pr->T; ++t)
            for (int g = 0; g < pr->Hkv; ++g) {
                int64_t row = ((int64_t)b * pr->T + t) * pr->Hq + (int64_t)g * G;
                attend_pair(pr, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, indices,
                            n_sel, b, t, g, out + row * pr->d, lse + row, NULL, NULL);
            }
}

/* dense attention over every position [0, L) (reference for k = all) */
void orc_dense(const orc_problem *pr, const void *q, const void *k_pool, const void *v_pool,
               const float *k_scales, const float *v_scales, const int32_t *block_table,
               const int32_t *seq_lens, double *out, double *lse) {
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < pr->B; ++b)
        for (int h = 0; h < pr->Hq; ++h) {
            int L = seq_lens[b];
            int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (L + 1));
            for (int p = 0; p < L; ++p) pos[p] = p;
            int64_t bh = (int64_t)b * pr->Hq + h;
            partial_tok(pr, q, k_pool, v_pool, k_scales, v_scales, block_table, b, 0, h, pos, L,
                        out + bh * pr->d, lse + bh);
            free(pos);
        }
}

/* ---------------------------------------------------------- decode step */

void orc_decode_step(const orc_problem *pr, const void *q, const void *landmarks,
                     const void *k_pool, const void *v_pool, const float *k_scales,
                     const float *v_scales, const int32_t *block_table, const int32_t *seq_lens,
                     const int32_t *k_per_seq, double *scores, int32_t *indices, int32_t *n_sel,
                     double *out, double *lse, double *overlap) {
    orc_scores(pr, q, landmarks, seq_lens, scores);
    orc_select(pr, scores, seq_lens, k_per_seq, indices, n_sel);
    orc_attend(pr, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, indices, n_sel,
               out, lse, NULL, NULL);
    if (pr->T == 2 && overlap) orc_overlap(pr, indices, n_sel, overlap);
}

int orc_max_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
