/*
 * sparsekv.h -- C ABI of the MI355X (gfx950) sparse-KV decode step.
 *
 * One decode step of one attention layer over a paged KV cache:
 *   score    every historical block's landmark against the query
 *            (DualDecoder review, core claim and axiom ledger item 1: the
 *            retrieval index follows from the query and landmarks resident on
 *            the GPU; the landmark is the mean of the block's keys);
 *   top-k    per KV head, keep the k highest-scoring blocks (PulseInfer
 *            article, section 2: per-head sparse selection; DualDecoder
 *            ledger: a sparse KV budget);
 *   gather   copy the selected (block, head) chunks into a dense staging
 *            buffer (PulseInfer article, section 2: an I/O engine that gathers
 *            the scattered selected entries and merges small transfers into
 *            large ones; DualDecoder Fig. 19: whole blocks fetched contiguously
 *            and reordered by GPU kernels; Fig. 11: two-layer ping-pong
 *            staging buffer);
 *   attend   split-K attention over the selected blocks plus dense attention
 *            over the recent window, the partial results fused by
 *            log-sum-exp (Beyond abstract).
 *
 * Notation: B batch, T query tokens per sequence (1, or 2 = real +
 * speculative), Hq query heads, Hkv KV heads, G = Hq/Hkv, d head dim, blk
 * block size in tokens, L_b length of sequence b, W window, ws_b =
 * max(0, L_b - W) window start.  Candidate blocks of sequence b are
 * j in [0, ceil(ws_b/blk)) (blocks holding a position before the window).
 *
 * Layouts (row-major, innermost last; "elements" are of the stated dtype):
 *   q          [B][T][Hq][d]            q_dtype
 *   landmarks  [B][Hkv][max_blocks][d]  landmark_dtype, logical block order
 *   K/V pool   chunk (p, g) = [blk][d] contiguous at element offset
 *              p*pool_stride_block + g*pool_stride_head  (kv_dtype)
 *   k/v scales [P][Hkv] fp32, fp8 pools only: value = code * scale
 *   block_table[B][max_blocks] int32 physical block of logical block j
 *   seq_lens   [B] int32,  k_per_seq [B] int32
 *   scores     [B][T][Hkv][max_blocks] fp32 (-inf for non-candidates)
 *   indices    [B][T][Hkv][k_max] int32, ascending block ids, -1 padded
 *   n_sel      [B][T][Hkv] int32 = min(k_b, #candidates)
 *   stage      [B][Hkv][k_max][blk][d] kv_dtype; stage scales [B][Hkv][k_max]
 *   window buf [B][Hkv][W][d] kv_dtype: row r holds position ws_b + r;
 *              fp8: per-row scales [B][Hkv][W] fp32 (row r's K and V scales,
 *              normally those of the pool block holding position ws_b + r)
 *   out        [B][Hq][d] fp32 (real token), lse [B][Hq] fp32 (natural log);
 *              co-batched attention: [B][T][Hq][d] and [B][T][Hq]
 *   overlap    [B][Hkv] fp32 = |I_real & I_spec| / |I_real| (T == 2)
 *
 * Ownership and execution: the caller owns every buffer (device memory, or
 * pinned host memory for a host pool).  The library allocates no memory (the
 * host-pool paths create HIP events to order their two streams); all work is
 * enqueued on the given HIP stream (NULL = default stream) and is
 * asynchronous, except where an entry point says it waits: the hybrid step
 * (its CPU part needs the selection) and the measurement aid
 * sparsekv_decode_step_launch_times.  Keep buffers alive until the work
 * completes.
 *
 * Errors: every argument is checked on the host before any launch; a bad
 * argument returns a non-zero status and launches nothing.  Unsupported
 * combinations return SKV_E_UNSUPPORTED (never a silent fallback).  A failed
 * launch returns SKV_E_HIP with the runtime's text in sparsekv_last_error().
 * Device-resident values (block ids, lengths, k) are not checked: an
 * out-of-range block id or a length above max_blocks*blk is undefined
 * behaviour.  No C++ exception crosses this interface.
 *
 * Supported: d in {64, 128}; blk in {16, 32, 64}; 1 <= G <= 8; T in {1, 2};
 * kv fp32 with q fp32, or kv bf16 / fp8 e4m3fn with q bf16; landmarks fp32 or
 * bf16; max_blocks <= 16384; k_max <= max_blocks.  The selection keeps a
 * pair's keys in one workgroup's 160 KiB of LDS, which bounds k_max further
 * (SKV_E_UNSUPPORTED before any launch beyond it):
 *   steps that select (decode_step when it takes two or three launches,
 *   decode_layers*, the hybrid step):
 *     4 * (T*d + T*C + 2*k_max + 512) + 4232 <= 163840 bytes,
 *     C = max_blocks - floor(W / blk) (the most candidates a sequence has);
 *     e.g. T = 2, d = 128, C = 16380: k_max <= 3187;  T = 1: k_max <= 11441;
 *   sparsekv_topk: 4 * (max_blocks + 2*k_max) + 4232 <= 163840 bytes,
 *     e.g. max_blocks = 16384: k_max <= 11759.
 * Alignment: q, landmarks, K/V pools, stages and window buffers are read with
 * 16-byte loads, so their addresses, pool_stride_block * element size and
 * pool_stride_head * element size must be multiples of 16 (SKV_E_SHAPE).
 */
#ifndef SPARSEKV_H
#define SPARSEKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SKV_OK = 0,
    SKV_E_NULL = 1,         /* a required pointer is NULL */
    SKV_E_SHAPE = 2,        /* a size is non-positive or inconsistent */
    SKV_E_DTYPE = 3,        /* unknown dtype code */
    SKV_E_UNSUPPORTED = 4,  /* valid but not implemented combination */
    SKV_E_WORKSPACE = 5,    /* workspace missing or too small */
    SKV_E_HIP = 6           /* the HIP runtime reported an error */
} skv_status;

typedef enum { SKV_F32 = 0, SKV_BF16 = 1, SKV_FP8_E4M3FN = 2 } skv_dtype;
typedef enum { SKV_POOL_DEVICE = 0, SKV_POOL_HOST = 1 } skv_pool_location;

/* One layer, one decode step. */
typedef struct {
    int32_t batch;               /* B >= 1 */
    int32_t n_q_tokens;          /* T: 1, or 2 (real, speculative) */
    int32_t n_q_heads;           /* Hq, a multiple of n_kv_heads */
    int32_t n_kv_heads;          /* Hkv */
    int32_t head_dim;            /* d */
    int32_t block_size;          /* blk */
    int32_t max_blocks_per_seq;  /* columns of block_table and landmarks */
    int32_t n_pool_blocks;       /* P */
    int64_t pool_stride_block;   /* elements between pool blocks p and p+1 */
    int64_t pool_stride_head;    /* elements between heads g and g+1 of a block */
    int32_t window;              /* W >= 0 */
    int32_t k_max;               /* >= every k_b; columns of indices */
    int32_t q_dtype, kv_dtype, landmark_dtype;  /* skv_dtype */
    int32_t pool_location;       /* skv_pool_location */
} skv_problem;

/* Where attention reads K/V from. */
typedef enum {
    SKV_SRC_PAGED = 0,   /* pool chunks through block_table (and indices for the sparse part) */
    SKV_SRC_STAGED = 1,  /* gathered stage buffers, slot m = m-th selected block */
    SKV_SRC_WINDOW = 2   /* window buffers [B][Hkv][W][d]; needs W % blk == 0 */
} skv_source_kind;

typedef struct {
    int32_t kind;                /* skv_source_kind */
    const void *k, *v;           /* pool, stage or window buffers */
    const float *k_scales, *v_scales;  /* fp8: pool [P][Hkv], stage [B][Hkv][k_max] or
                                          window buffer [B][Hkv][W] (one per row,
                                          16-byte aligned) */
    const int32_t *block_table;  /* PAGED only */
} skv_kv_source;

/* Per-layer inputs of a full decode step. */
typedef struct {
    const void *q, *landmarks;
    const void *k_pool, *v_pool;
    const float *k_scales, *v_scales;  /* fp8 only */
    const int32_t *block_table, *seq_lens, *k_per_seq;
    const void *window_k, *window_v;   /* host pools: HBM window buffers; else NULL */
    /* fp8 host pools with W > 0: the window buffers' per-row scales
       [B][Hkv][W] fp32 (16-byte aligned); else NULL.  fp8 device pools
       take no window buffers (SKV_E_UNSUPPORTED). */
    const float *window_k_scales, *window_v_scales;
} skv_step_inputs;

/* Per-layer outputs of a full decode step. */
typedef struct {
    int32_t *indices, *n_sel;
    float *out, *lse;            /* lse may be NULL */
    float *overlap;              /* T == 2 only; may be NULL */
} skv_step_outputs;

const char *sparsekv_status_string(int status);
/* Text of the last SKV_E_HIP / validation failure on the calling thread. */
const char *sparsekv_last_error(void);
/*
 * Every kernel takes its parameters by value, and each workgroup reads them
 * before its first memory access.  Run with the HIP runtime's kernel
 * arguments in device memory (HIP_FORCE_DEV_KERNARG=1 in the environment
 * before the runtime starts): kept in host memory they cost a host-link round
 * trip per launch, measured at 3.3 us (5%) on the 32k-context decode step.
 */

/* Library version as "major.minor.patch". */
const char *sparsekv_version(void);

/*
 * Measurement aid, not a step of the method: reads `bytes` of device memory
 * at `buffer` once with the same 16-byte non-temporal loads the step's
 * kernels use, four per thread in flight, so that the rate it reaches on a
 * buffer far larger than the caches is the streaming-read ceiling the step's
 * achieved bandwidth can be compared with.  `buffer` must be 16-byte aligned
 * and `bytes` a multiple of 16 (else SKV_E_SHAPE); a NULL `buffer` or `sink`
 * gives SKV_E_NULL, a launch failure SKV_E_HIP.  `sink` is a device buffer of
 * `sink_bytes` (at least 4, 4-aligned); it bounds the grid at one workgroup
 * per word (512 threads and 32 KiB per workgroup, at most 32768) and is
 * written only if a workgroup's folded data equals one fixed 32-bit value, so
 * its contents carry no meaning.  Asynchronous on `stream`; allocates nothing.
 */
skv_status sparsekv_stream_read(const void *buffer, size_t bytes, void *sink, size_t sink_bytes,
                                void *stream);

/*
 * Workspace: device scratch for split partials, score staging (or, for a
 * selection over split scoring rows, each chunk's own top-k candidates) and
 * arrival counters.  sparsekv_workspace_size() gives the bytes needed by
 * sparsekv_attend / sparsekv_decode_step / sparsekv_decode_layers for a
 * problem.  A new workspace must be cleared once with sparsekv_workspace_init
 * (a fill kernel, safe inside graph capture); every call returns its counters
 * to zero when it completes, so no further clearing is needed.  Calls that
 * share a workspace must not overlap in time.
 */
skv_status sparsekv_workspace_size(const skv_problem *pr, size_t *bytes);

/*
 * Kernel launches one sparsekv_decode_step enqueues for a problem (host-only,
 * no GPU work): 1 when the whole step runs as a single launch with one
 * workgroup per (sequence, KV head) -- device pool, head_dim 128, bf16
 * queries and landmarks, bf16 or fp8 K/V, blocks of 32 or 64 tokens, at
 * least 128 (sequence, KV head) pairs, and every wave of the pair's 8-wave
 * workgroup holding at most 64 32-token slices: ceil(w / (8 - T)) window
 * slices plus ceil(s / 8) selected ones, with w = (ceil(W / blk) + 1) * blk / 32
 * and s = k_max * blk / 32 (e.g. k_max <= 488 at blocks of 32 and W = 512);
 * 2 for the other device-pool problems (scoring, then attention); 3 for a
 * host pool (scoring with the selection, gather, attention).  *launches
 * receives the count.
 */
skv_status sparsekv_decode_step_launches(const skv_problem *pr, int32_t *launches);

/*
 * Name of the kernel that launch `launch` (0-based) of sparsekv_decode_step
 * runs for a problem (host-only, no GPU work), e.g. to match a profiler's
 * trace: "pair_step_kernel" (single launch); "score_kernel" then
 * "split_step_kernel" (few pairs with a two-level selection: the scoring
 * chunks publish their own top k', and every attention split makes the final
 * selection from them) or "attend_kernel" (the scoring launch selects);
 * host pools "score_kernel", "gather_kernel", "attend_kernel".  *name
 * receives a static string.  SKV_E_SHAPE for a launch outside
 * [0, sparsekv_decode_step_launches).
 */
skv_status sparsekv_decode_step_kernel(const skv_problem *pr, int32_t launch, const char **name);

/*
 * Per-launch device time of a device-pool decode step, a measurement aid:
 * enqueues one whole sparsekv_decode_step on `stream`, then each launch of the
 * step alone, n_steps times back to back (1 <= n_steps <= 4096) between two
 * events, and writes each launch's mean time in microseconds to
 * launch_us[0 .. sparsekv_decode_step_launches).  A launch reads what the
 * launches before it wrote and does not change it, so the repeats compute
 * the step's own values; a last whole step leaves the outputs as
 * sparsekv_decode_step would.  Waits for the stream; creates and destroys
 * its own events.  Host pools: SKV_E_UNSUPPORTED.
 */
skv_status sparsekv_decode_step_launch_times(const skv_problem *pr, const skv_step_inputs *in,
                                             const skv_step_outputs *out, void *workspace,
                                             size_t workspace_bytes, void *stream, int32_t n_steps,
                                             float *launch_us);
skv_status sparsekv_workspace_init(void *workspace, size_t bytes, void *stream);

/*
 * Landmark scoring (score step above).  For t < T, g < Hkv and candidate j:
 *   scores[b,t,g,j] = sum_{h = gG}^{gG+G-1} q[b,t,h,:] . landmarks[b,g,j,:]
 * accumulated in fp32 (no 1/sqrt(d): ranking only); -inf for j beyond the
 * candidates.  One landmark load serves every query token.
 */
skv_status sparsekv_score(const skv_problem *pr, const void *q, const void *landmarks,
                          const int32_t *seq_lens, float *scores, void *stream);

/*
 * Per-KV-head top-k (top-k step above): k'_b = min(k_per_seq[b], #candidates)
 * blocks with the largest score, ties to the lowest block id, written in
 * ascending id order and padded with -1; n_sel = k'_b.  With T == 2 and a
 * non-NULL overlap, also writes the index-overlap fraction of the two tokens
 * (DualDecoder review: retrieval-index prediction accuracy; 1.0 when k' = 0).
 */
skv_status sparsekv_topk(const skv_problem *pr, const float *scores, const int32_t *seq_lens,
                         const int32_t *k_per_seq, int32_t *indices, int32_t *n_sel,
                         float *overlap, void *stream);

/*
 * Gather (gather step above): for the real token's selection, copy each
 * selected (block, head) chunk of K and V -- and, for fp8, its two scales --
 * into staging slot m, byte for byte.  Slots >= n_sel are left untouched.
 * k_pool / v_pool may be pinned host memory (pool_location HOST): the copy
 * then reads it over the host link with 16-byte loads.
 */
skv_status sparsekv_gather(const skv_problem *pr, const void *k_pool, const void *v_pool,
                           const float *k_scales, const float *v_scales,
                           const int32_t *block_table, const int32_t *indices,
                           const int32_t *n_sel, void *k_stage, void *v_stage,
                           float *k_stage_scales, float *v_stage_scales, void *stream);

/*
 * Speculative prefetch correction (DualDecoder review, mechanism summary and
 * Fig. 19: blocks are fetched early by the index predicted from a speculative
 * token; once the real token's index is known the missing blocks are fetched
 * and a GPU kernel reorders the staged blocks into the real index's order).
 *
 * spec_k_stage / spec_v_stage (and, for fp8, spec_k_scales / spec_v_scales)
 * hold the gather of a speculative selection: slot m of row (b, g) holds
 * block spec_indices[b, spec_token, g, m].  This call writes into k_stage /
 * v_stage exactly the gather of the real selection -- byte for byte what
 * sparsekv_gather writes for it: a real block that the speculative row also
 * holds is copied from its speculative slot (device memory); the others, the
 * misses, are read from the pool (over the host link for a pinned pool).
 * Selections use the layouts sparsekv_topk writes ([B][T][Hkv][k_max] ids in
 * ascending order within n_sel, n_sel [B][T][Hkv]); spec_* and real_* may be
 * different arrays (the speculative one from an earlier step).  misses
 * [B][Hkv] (may be NULL) receives, per row, how many real blocks were not in
 * the speculative row.  The two stages must not overlap.  Slots >= n_sel of
 * the real row are left untouched.
 */
skv_status sparsekv_gather_correct(const skv_problem *pr, const void *k_pool, const void *v_pool,
                                   const float *k_scales, const float *v_scales,
                                   const int32_t *block_table, const int32_t *spec_indices,
                                   const int32_t *spec_n_sel, int32_t spec_token,
                                   const void *spec_k_stage, const void *spec_v_stage,
                                   const float *spec_k_scales, const float *spec_v_scales,
                                   const int32_t *real_indices, const int32_t *real_n_sel,
                                   int32_t real_token, void *k_stage, void *v_stage,
                                   float *k_stage_scales, float *v_stage_scales, int32_t *misses,
                                   void *stream);

/*
 * Attention (attend step above) for the real token (t = 0) of every query
 * head h of group g:
 *   sparse part: positions p = j*blk + r of the selected blocks j with p < ws_b
 *   window part: positions [ws_b, L_b)
 *   z_p = q_h . k_p / sqrt(d); each part is split over workgroups (split-K)
 *   and every split's (max, sum, unnormalised output) is fused by
 *   log-sum-exp into out (fp32) and lse = ln sum_p e^{z_p}.
 * Empty parts contribute nothing; with no position at all, out = 0 and
 * lse = -inf.  sparse->kind is PAGED (indices index the block table) or
 * STAGED; window->kind is PAGED or WINDOW (fp8: with per-row scales).
 */
skv_status sparsekv_attend(const skv_problem *pr, const void *q, const skv_kv_source *sparse,
                           const int32_t *indices, const int32_t *n_sel,
                           const skv_kv_source *window, const int32_t *seq_lens,
                           float *out, float *lse, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * Co-batched attention of both query tokens (DualDecoder review, Fig. 18:
 * the real and the speculative token attended in one launch instead of
 * two).  For t in {0, 1}, out[b,t,h,:] and lse[b,t,h] are exactly what
 * sparsekv_attend computes for token t alone -- token t's query over token
 * t's own selection (indices / n_sel rows of token t) plus the window
 * [ws_b, L_b) -- up to fp32 rounding order.  Each block of the union of the
 * two selections is read once per (sequence, KV head); a block that only one
 * token selected is masked for the other.  out is [B][T][Hq][d] fp32, lse
 * [B][T][Hq] (may be NULL).  T == 2 needs a device pool and a PAGED sparse
 * source (the union is read through the block table), and fp8 a PAGED
 * window source; SKV_E_UNSUPPORTED otherwise.  T == 1 is sparsekv_attend.  The workspace is the
 * one sparsekv_workspace_size gives for the problem.
 */
skv_status sparsekv_attend_cobatched(const skv_problem *pr, const void *q,
                                     const skv_kv_source *sparse, const int32_t *indices,
                                     const int32_t *n_sel, const skv_kv_source *window,
                                     const int32_t *seq_lens, float *out, float *lse,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Full decode step.  Device pool: scoring with in-kernel top-k, then
 * attention straight from the paged pool (the gather is fused into the
 * attention's loads; nothing is staged); with few (sequence, KV head) pairs
 * and a two-level selection, the final select runs in the attention launch
 * instead (sparsekv_decode_step_kernel).  Host pool: scoring and top-k on
 * `stream`, the gather from pinned host memory into k_stage/v_stage on
 * `copy_stream` (ordered by events), then attention of the staged blocks plus
 * the HBM window buffers on `stream`.  k_stage/v_stage ([B][Hkv][k_max][blk][d])
 * are required for host pools and ignored otherwise; copy_stream may be NULL
 * (then `stream` is used).
 */
skv_status sparsekv_decode_step(const skv_problem *pr, const skv_step_inputs *in,
                                const skv_step_outputs *out, void *k_stage, void *v_stage,
                                float *k_stage_scales, float *v_stage_scales,
                                void *workspace, size_t workspace_bytes,
                                void *stream, void *copy_stream);

/*
 * sparsekv_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid allocation).  Device pools only (SKV_E_UNSUPPORTED
 * for a host pool).  The workspace is a fixed array of 32 MiB inside the
 * library, one per GPU, held until the process ends; a problem whose
 * sparsekv_workspace_size exceeds it returns SKV_E_WORKSPACE before any GPU
 * work.  Every call on a GPU uses that GPU's one array: a fill kernel clears
 * its arrival counters first (no memset node, so the call can be captured),
 * and calls that overlap in time on one GPU -- on different streams, or from
 * different threads -- race on it and give undefined results.  The call
 * itself allocates nothing (its first call on a device looks up the array's
 * address there).  Results equal sparsekv_decode_step's bit for bit.
 */
skv_status sparsekv_decode_step_noalloc(const skv_problem *pr, const skv_step_inputs *in,
                                        const skv_step_outputs *out, void *stream);

/*
 * Host side of the hybrid step: the pool's host addresses and pinned host
 * buffers the caller owns (allocated with hipHostMalloc or equivalent, so the
 * GPU can read o and lse).  The call fills the buffers below.
 */
typedef struct {
    const void *k_pool, *v_pool;  /* host addresses of the pinned K/V pool (the memory whose
                                     device-visible addresses are in skv_step_inputs) */
    int32_t n_threads;            /* host threads for the sparse part; <= 0: all available */
    void *q;                      /* [B][T][Hq][d] q_dtype: copy of the queries */
    int32_t *seq_lens;            /* [B] */
    int32_t *block_table;         /* [B][max_blocks] */
    int32_t *indices;             /* [B][T][Hkv][k_max]: copy of the selection */
    int32_t *n_sel;               /* [B][T][Hkv] */
    float *k_scales, *v_scales;   /* [P][Hkv]: copies of the fp8 scales (fp8 only) */
    float *o;                     /* [B][Hq][d]: the sparse part's output */
    float *lse;                   /* [B][Hq]: its log-sum-exp (natural log) */
} skv_host_part;

/*
 * The host part of the hybrid step on its own (Beyond abstract: parallel
 * per-head sparse attention over the salient KV in CPU memory): for the
 * real token (t = 0) of every query head h of group g, attention over the
 * positions p = j*blk + r of the selected blocks j with p < ws_b, from
 * host->k_pool / v_pool (host addresses), with host->q, seq_lens,
 * block_table, indices, n_sel (and, for fp8, k_scales / v_scales) already
 * filled by the caller.  Writes host->o (normalised, fp32) and host->lse
 * (natural log; -inf and o = 0 when a head has no position).  Runs on the
 * calling thread's OpenMP team (host->n_threads); no GPU work, blocking.
 * Needs a host pool problem (pool_location HOST); layouts as above.
 */
skv_status sparsekv_host_attention(const skv_problem *pr, const skv_host_part *host);

/*
 * Hybrid CPU-GPU decode step (Beyond abstract: dense attention over the
 * recent KV in GPU memory, parallel per-head sparse attention over the
 * salient KV in CPU memory, the outputs fused by log-sum-exp, so that only
 * small results cross the host link).  Host pool only.
 *   GPU: scoring and top-k as in sparsekv_decode_step, then attention over
 *        the window buffers alone;
 *   CPU: on the calling thread's OpenMP team, the real token's attention over
 *        its selected blocks, read from the pinned pool in place (fp32
 *        arithmetic);
 *   GPU: the two parts fused by log-sum-exp into out->out / out->lse.
 * The results equal sparsekv_decode_step's up to fp32 rounding.  The call
 * blocks the calling thread until the selection has reached the host and
 * the sparse part is done (the window attention runs meanwhile); the fusion
 * is enqueued on `stream` and runs asynchronously.  fp8 window buffers
 * take their per-row scales from in->window_k_scales / window_v_scales.
 */
skv_status sparsekv_decode_step_hybrid(const skv_problem *pr, const skv_step_inputs *in,
                                       const skv_step_outputs *out, const skv_host_part *host,
                                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Host-pool layer pipeline with a two-slot (ping-pong) staging buffer
 * (DualDecoder Fig. 11 and the layer-aware schedule of its mechanism
 * summary).  Layer l's blocks are gathered into slot l % 2 on copy_stream as
 * soon as its indices exist and layer l-2's attention has released the slot;
 * attention of layer l runs on stream once its gather is done.  The staging
 * footprint is two slots for any number of layers.  in[l] / out[l] are the
 * per-layer inputs and outputs (n_layers >= 1); k_stage[2] / v_stage[2] are
 * the two slots.
 */
skv_status sparsekv_decode_layers(const skv_problem *pr, int32_t n_layers,
                                  const skv_step_inputs *in, const skv_step_outputs *out,
                                  void *const *k_stage, void *const *v_stage,
                                  float *const *k_stage_scales, float *const *v_stage_scales,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream, void *copy_stream);

/*
 * A layer's predicted selection for sparsekv_decode_layers_predicted: an
 * earlier selection in the layout sparsekv_topk writes ([B][T][Hkv][k_max]
 * ids ascending within n_sel, n_sel [B][T][Hkv]), of which row `token` is
 * the prediction -- for a two-token problem, the speculative token's row
 * (token 1) of the previous decode step's outputs for this layer.
 */
typedef struct {
    const int32_t *indices;
    const int32_t *n_sel;
    int32_t token;
    int32_t *misses;             /* [B][Hkv]: real blocks the prediction missed; may be NULL */
} skv_layer_prediction;

/*
 * Host-pool layer pipeline with prefetch by a predicted index (DualDecoder
 * review: mechanism summary -- blocks are prefetched by the index a
 * speculative token predicts, with a lead of two layers, and the blocks it
 * missed are fetched on demand; Fig. 19 -- predicted blocks fetched
 * contiguously, then reordered on the GPU into the real index's order;
 * Fig. 11 -- a two-slot ping-pong staging buffer).
 *   copy_stream: the predicted blocks of layer l (pred[l], a plain gather)
 *     go into prefetch slot l % 2 (pref_k / pref_v [2], and pref_k_scales /
 *     pref_v_scales [2] for fp8), as soon as layer l-2's correction has read
 *     that slot, so prefetches run up to two layers ahead of the compute;
 *   stream, per layer in order: scoring and top-k of layer l (its real
 *     selection, into out[l]); then, once layer l's prefetch is staged, the
 *     correction (sparsekv_gather_correct's kernel): blocks the prediction
 *     holds move from the prefetch slot into k_stage / v_stage in the real
 *     selection's order, the misses are read from the pinned pool; then the
 *     attention of the stage plus the HBM window buffers.
 * The misses are fetched on `stream`, directly before the attention that
 * needs them, so no background prefetch is queued ahead of them.  Each
 * layer's results equal sparsekv_decode_step's on in[l] (the stage holds the
 * real selection's gather byte for byte, whatever the prediction).  The
 * stage must not overlap a prefetch slot (SKV_E_SHAPE).  The copy stream
 * starts after the work already queued on `stream`; `stream` ends after
 * every layer's attention, which follows every prefetch.
 */
skv_status sparsekv_decode_layers_predicted(const skv_problem *pr, int32_t n_layers,
                                            const skv_step_inputs *in, const skv_step_outputs *out,
                                            const skv_layer_prediction *pred,
                                            void *const *pref_k, void *const *pref_v,
                                            float *const *pref_k_scales, float *const *pref_v_scales,
                                            void *k_stage, void *v_stage,
                                            float *k_stage_scales, float *v_stage_scales,
                                            void *workspace, size_t workspace_bytes,
                                            void *stream, void *copy_stream);

#ifdef __cplusplus
}
#endif
#endif /* SPARSEKV_H */
