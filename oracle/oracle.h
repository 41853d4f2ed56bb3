/*
 * oracle.h -- fp64 CPU reference of the sparse-KV decode step.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline bench leg).
 * Independent of the HIP library: no shared header, type or constant.
 */
#ifndef SPARSEKV_ORACLE_H
#define SPARSEKV_ORACLE_H
#include <stdint.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };

typedef struct {
    int32_t B, T, Hq, Hkv, d, blk, max_blocks, n_pool_blocks;
    int64_t stride_block, stride_head; /* pool element strides of a (block, head) chunk */
    int32_t window, k_max;
    int32_t q_dtype, kv_dtype, lm_dtype;
} orc_problem;

double orc_bf16_value(uint16_t code);
double orc_e4m3fn_value(uint8_t code);
int orc_n_candidates(const orc_problem *pr, int L);

/* scores [B][T][Hkv][max_blocks] fp64; -inf for non-candidates */
void orc_scores(const orc_problem *pr, const void *q, const void *landmarks,
                const int32_t *seq_lens, double *scores);
/* indices [B][T][Hkv][k_max] ascending, -1 padded; n_sel [B][T][Hkv] */
void orc_select(const orc_problem *pr, const double *scores, const int32_t *seq_lens,
                const int32_t *k_per_seq, int32_t *indices, int32_t *n_sel);
/* overlap [B][Hkv] (T == 2) */
void orc_overlap(const orc_problem *pr, const int32_t *indices, const int32_t *n_sel, double *overlap);
/* stage [B][Hkv][k_max][blk][d]; stage scales [B][Hkv][k_max] */
void orc_gather(const orc_problem *pr, const void *k_pool, const void *v_pool,
                const float *k_scales, const float *v_scales, const int32_t *block_table,
                const int32_t *indices, const int32_t *n_sel,
                void *k_stage, void *v_stage, float *k_stage_scales, float *v_stage_scales);
void orc_partial(const orc_problem *pr, const void *q, const void *k_pool, const void *v_pool,
                 const float *k_scales, const float *v_scales, const int32_t *block_table,
                 int b, int h, const int64_t *pos, int n_pos, double *o, double *lse);
void orc_merge(int n_parts, int d, const double *o_parts, const double *lse_parts,
               double *o, double *lse);
/* out [B][Hq][d], lse [B][Hq]; part_o [B][Hq][2][d] and part_lse [B][Hq][2] may be NULL */
void orc_attend(const orc_problem *pr, const void *q, const void *k_pool, const void *v_pool,
                const float *k_scales, const float *v_scales, const int32_t *block_table,
                const int32_t *seq_lens, const int32_t *indices, const int32_t *n_sel,
                double *out, double *lse, double *part_o, double *part_lse);
/* every query token over its own selection: out [B][T][Hq][d], lse [B][T][Hq] */
void orc_attend_tokens(const orc_problem *pr, const void *q, const void *k_pool, const void *v_pool,
                       const float *k_scales, const float *v_scales, const int32_t *block_table,
                       const int32_t *seq_lens, const int32_t *indices, const int32_t *n_sel,
                       double *out, double *lse);
void orc_dense(const orc_problem *pr, const void *q, const void *k_pool, const void *v_pool,
               const float *k_scales, const float *v_scales, const int32_t *block_table,
               const int32_t *seq_lens, double *out, double *lse);
void orc_decode_step(const orc_problem *pr, const void *q, const void *landmarks,
                     const void *k_pool, const void *v_pool, const float *k_scales,
                     const float *v_scales, const int32_t *block_table, const int32_t *seq_lens,
                     const int32_t *k_per_seq, double *scores, int32_t *indices, int32_t *n_sel,
                     double *out, double *lse, double *overlap);
int orc_max_threads(void);
/* Threads the following calls use (OpenMP over independent (b, g) pairs). */
void orc_set_threads(int n);

#endif
