// sparsekv.hip -- the C ABI declared in include/sparsekv.h: argument
// validation, launch planning, workspace carving, stream/event ordering.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <initializer_list>
#include <mutex>

#include "host_attn.h"
#include "skv_device.h"
#include "skv_internal.h"

namespace skv {

namespace {
thread_local char g_err[512] = "";
}  // namespace

skv_status fail(skv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

skv_status hip_fail(hipError_t e, const char* what) {
  return fail(SKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

namespace {

int elem_bytes(int dt) { return dt == SKV_F32 ? 4 : dt == SKV_BF16 ? 2 : 1; }

int kv_kind(int dt) { return dt == SKV_F32 ? KV_F32 : dt == SKV_BF16 ? KV_BF16 : KV_FP8; }

skv_status check_problem(const skv_problem* pr) {
  if (!pr) return fail(SKV_E_NULL, "problem is NULL");
  const skv_problem& p = *pr;
  if (p.batch < 1 || p.n_q_heads < 1 || p.n_kv_heads < 1 || p.head_dim < 1 || p.block_size < 1 ||
      p.max_blocks_per_seq < 1 || p.n_pool_blocks < 1 || p.window < 0 || p.k_max < 1)
    return fail(SKV_E_SHAPE, "non-positive size in problem");
  if (p.n_q_tokens != 1 && p.n_q_tokens != 2)
    return fail(SKV_E_SHAPE, "n_q_tokens must be 1 or 2 (got %d)", p.n_q_tokens);
  if (p.n_q_heads % p.n_kv_heads != 0)
    return fail(SKV_E_SHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d", p.n_q_heads,
                p.n_kv_heads);
  if (p.k_max > p.max_blocks_per_seq)
    return fail(SKV_E_SHAPE, "k_max %d exceeds max_blocks_per_seq %d", p.k_max, p.max_blocks_per_seq);
  if (p.pool_stride_block < 0 || p.pool_stride_head < 0)
    return fail(SKV_E_SHAPE, "negative pool stride");
  for (int dt : {p.q_dtype, p.kv_dtype, p.landmark_dtype})
    if (dt < SKV_F32 || dt > SKV_FP8_E4M3FN) return fail(SKV_E_DTYPE, "unknown dtype code %d", dt);
  if (p.pool_location != SKV_POOL_DEVICE && p.pool_location != SKV_POOL_HOST)
    return fail(SKV_E_SHAPE, "unknown pool_location %d", p.pool_location);
  // every (block, head) chunk is read with 16-byte loads
  const int64_t eb = elem_bytes(p.kv_dtype);
  if ((p.pool_stride_block * eb) % 16 != 0 || (p.pool_stride_head * eb) % 16 != 0)
    return fail(SKV_E_SHAPE, "pool strides (%lld, %lld elements) are not multiples of 16 bytes",
                (long long)p.pool_stride_block, (long long)p.pool_stride_head);
  const int G = p.n_q_heads / p.n_kv_heads;
  if (G > 8) return fail(SKV_E_UNSUPPORTED, "group size %d > 8", G);
  if (p.head_dim != 64 && p.head_dim != 128)
    return fail(SKV_E_UNSUPPORTED, "head_dim %d not in {64, 128}", p.head_dim);
  if (p.block_size != 16 && p.block_size != 32 && p.block_size != 64)
    return fail(SKV_E_UNSUPPORTED, "block_size %d not in {16, 32, 64}", p.block_size);
  if (p.max_blocks_per_seq > 16384)
    return fail(SKV_E_UNSUPPORTED, "max_blocks_per_seq %d > 16384", p.max_blocks_per_seq);
  if (p.q_dtype == SKV_FP8_E4M3FN || p.landmark_dtype == SKV_FP8_E4M3FN)
    return fail(SKV_E_UNSUPPORTED, "fp8 queries or landmarks");
  if (p.kv_dtype == SKV_F32 && p.q_dtype != SKV_F32)
    return fail(SKV_E_UNSUPPORTED, "fp32 K/V needs fp32 queries");
  if (p.kv_dtype != SKV_F32 && p.q_dtype != SKV_BF16)
    return fail(SKV_E_UNSUPPORTED, "bf16/fp8 K/V needs bf16 queries");
  return SKV_OK;
}

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Buffers read or written with 16-byte vector accesses (queries, landmarks,
// pools, stages, window buffers) must be 16-byte aligned; NULL passes (the
// NULL checks are separate).
skv_status check_align16(const char* where, std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs)
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0)
      return fail(SKV_E_SHAPE, "%s: buffer %p is not 16-byte aligned", where, x);
  return SKV_OK;
}

#ifndef SKV_ATTN_TARGET_WGS
#define SKV_ATTN_TARGET_WGS 256
#endif
constexpr int kAttnTargetWorkgroups = SKV_ATTN_TARGET_WGS;   // one 8-wave workgroup per CU
constexpr int kScoreSinglePairs = 128;       // from this many pairs on, one scoring workgroup per pair
constexpr int kScoreTargetWorkgroups = 256;
constexpr int kTwoLevelMinSaving = 2048;     // keys the chunks' own selections must save
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// single-launch step: used from this many (sequence, KV head) pairs on (one
// 8-wave workgroup per pair and compute unit), with at most this much LDS for
// the scoring region
constexpr int kStepMinPairs = 128;
constexpr size_t kStepMaxScoreLds = 48 * 1024;

}  // namespace

Plan make_plan(const skv_problem& p) {
  Plan pl{};
  const int G = p.n_q_heads / p.n_kv_heads;
  const int blk = p.block_size, D = p.head_dim;
  pl.max_cand = p.max_blocks_per_seq - p.window / blk;
  if (pl.max_cand < 0) pl.max_cand = 0;
  const int pairs = p.batch * p.n_kv_heads;
  // scoring: with many (sequence, KV head) pairs one workgroup scores all of a
  // pair's candidates into LDS and selects in place; with few pairs the rows
  // are split over about kScoreTargetWorkgroups workgroups
  const int lm_es = p.landmark_dtype == SKV_F32 ? 4 : 2;
  const int rps = 8 * (64 / (D * lm_es / 16));   // rows per 512-thread step
  if (pairs >= kScoreSinglePairs || pl.max_cand <= rps) {
    pl.rows_per_chunk = round_up(pl.max_cand > 0 ? pl.max_cand : 1, rps);
  } else {
    const int per_pair = (kScoreTargetWorkgroups + pairs - 1) / pairs;
    pl.rows_per_chunk = round_up((pl.max_cand + per_pair - 1) / per_pair, rps);
  }
  pl.score_chunks = pl.max_cand > 0 ? (pl.max_cand + pl.rows_per_chunk - 1) / pl.rows_per_chunk : 1;
  // Selecting within each chunk first costs a second select (measured about
  // 3.3 us fixed plus 2 us per 1000 keys per token) and a hand-off of about
  // 1.5 us; it pays when it leaves the last chunk at least 2048 fewer keys.
  pl.score_two_level = pl.score_chunks > 1 &&
                       pl.max_cand - pl.rows_per_chunk - pl.score_chunks * std::min(p.k_max, pl.rows_per_chunk) >=
                           kTwoLevelMinSaving;
  // attention: items (32-token slices) of the sparse + window list per split,
  // aiming at about three resident workgroups per compute unit
  const int sub = blk / attn_item_tokens(kv_kind(p.kv_dtype), blk, p.head_dim);
  const int nwb = p.window == 0 ? 0 : (p.window + blk - 1) / blk + 1;
  const int total_items = (p.k_max + nwb) * sub;
  int ips = (int)(((int64_t)pairs * total_items + kAttnTargetWorkgroups - 1) / kAttnTargetWorkgroups);
  if (ips < 16) ips = 16;
  if (ips > 128) ips = 128;
  pl.items_per_split = ips;
  pl.n_splits = (total_items + ips - 1) / ips;
  const int total = pl.n_splits;
  // co-batched attention of two tokens: the list holds up to 2 k_max union
  // blocks; a split covers at most kCobatchMaxSplitBlocks - 2 blocks' items
  size_t part_rows = (size_t)total * G;
  if (p.n_q_tokens == 2) {
    const int cob_items = (2 * p.k_max + nwb) * sub;
    int ips2 = (int)(((int64_t)pairs * cob_items + kAttnTargetWorkgroups - 1) / kAttnTargetWorkgroups);
    ips2 = std::max(16, std::min(ips2, (kCobatchMaxSplitBlocks - 2) * sub));
    pl.cob_items_per_split = ips2;
    pl.cob_n_splits = (cob_items + ips2 - 1) / ips2;
    part_rows = std::max(part_rows, (size_t)pl.cob_n_splits * 2 * G);
  }

  // single-launch step
  pl.fused_step = 0;
#ifndef SKV_NO_STEP_KERNEL
  // the window slices go to the waves that do not select, the selected ones to all
  if (step_kernel_available(p) && pairs >= kStepMinPairs &&
      wave_items_fit(nwb * sub, kStepWaves - p.n_q_tokens, p.k_max * sub, kStepWaves)) {
    pl.step_lds = score_lds_bytes(p.n_q_tokens, D, pl.max_cand > 0 ? pl.max_cand : 1, p.k_max, true, true);
    pl.fused_step = pl.step_lds <= kStepMaxScoreLds &&
                    step_static_lds_bytes(p) + pl.step_lds <= kLdsPerCu;
  }
#endif
  pl.select_lds = score_lds_bytes(p.n_q_tokens, D, pl.max_cand > 0 ? pl.max_cand : 1, p.k_max, true) +
                  select_static_lds_bytes();
  pl.select_fits = pl.select_lds <= kLdsPerWorkgroup;
  // split step: with a two-level selection on a device pool, the final select
  // moves into the attention launch (every split makes it from the chunks'
  // candidates) instead of running in the scoring launch's last chunk
  pl.split_step = 0;
#ifndef SKV_NO_SPLIT_STEP
  if (!pl.fused_step && pl.score_two_level && pl.select_fits) {
    pl.cand_cols = pl.score_chunks * std::min(p.k_max, pl.rows_per_chunk);
    const size_t chunk_lds = score_lds_bytes(p.n_q_tokens, D, pl.max_cand, p.k_max, true, true) +
                             select_static_lds_bytes();
    pl.split_step = chunk_lds <= kLdsPerWorkgroup && split_step_fits(p, pl.n_splits, pl.cand_cols, &pl.split_lds);
  }
#endif
  size_t off = 0;
  pl.off_score_counters = off;
  off = align256(off + (size_t)pairs * 4);
  pl.off_attn_counters = off;
  off = align256(off + (size_t)pairs * 4);
  pl.off_scores = off;
  // stand-alone scores, or a fused selection's per-chunk (key, id) candidates
  const size_t score_words = (size_t)(pl.max_cand > 0 ? pl.max_cand : 1);
  const size_t cand_words = !pl.score_two_level ? 0
                            : pl.split_step ? (size_t)3 * pl.cand_cols
                                            : (size_t)pl.score_chunks * 2 * p.k_max;
  off = align256(off + (size_t)pairs * p.n_q_tokens * std::max(score_words, cand_words) * 4);
  pl.off_partials = off;
  off = align256(off + (size_t)pairs * part_rows * (D + 2) * 4);
  pl.off_phys = off;
  off = align256(off + (size_t)pairs * p.n_q_tokens * p.k_max * 4);
  pl.off_hybrid = off;
  off = align256(off + (size_t)p.batch * p.n_q_heads * (D + 1) * 4);
  pl.total_bytes = off;
  return pl;
}

namespace {

ScoreParams score_params(const skv_problem& p, const void* q, const void* lm, const int32_t* seq_lens) {
  ScoreParams s{};
  s.q = q;
  s.landmarks = lm;
  s.seq_lens = seq_lens;
  s.B = p.batch;
  s.T = p.n_q_tokens;
  s.Hq = p.n_q_heads;
  s.Hkv = p.n_kv_heads;
  s.G = p.n_q_heads / p.n_kv_heads;
  s.D = p.head_dim;
  s.blk = p.block_size;
  s.max_blocks = p.max_blocks_per_seq;
  s.window = p.window;
  s.q_f32 = p.q_dtype == SKV_F32;
  s.lm_f32 = p.landmark_dtype == SKV_F32;
  s.k_max = p.k_max;
  return s;
}

AttnParams attn_params(const skv_problem& p, const Plan& pl, const void* q, const int32_t* seq_lens,
                       float* out, float* lse, char* ws) {
  AttnParams a{};
  a.kv = kv_kind(p.kv_dtype);
  a.q = q;
  a.B = p.batch;
  a.T = p.n_q_tokens;
  a.Hq = p.n_q_heads;
  a.Hkv = p.n_kv_heads;
  a.G = p.n_q_heads / p.n_kv_heads;
  a.D = p.head_dim;
  a.blk = p.block_size;
  a.window = p.window;
  a.max_blocks = p.max_blocks_per_seq;
  a.k_max = p.k_max;
  a.qk_scale = kLog2e / std::sqrt((float)p.head_dim);
  a.stride_block = p.pool_stride_block;
  a.stride_head = p.pool_stride_head;
  a.seq_lens = seq_lens;
  a.n_splits = pl.n_splits;
  a.items_per_split = pl.items_per_split;
  a.partials = Handoff<float>(reinterpret_cast<float*>(ws + pl.off_partials));
  a.counters = reinterpret_cast<unsigned*>(ws + pl.off_attn_counters);
  a.out = out;
  a.lse = lse;
  return a;
}

skv_status set_source(const skv_problem& p, AttnParams& a, const skv_kv_source* src, bool sparse) {
  if (!src) return fail(SKV_E_NULL, "%s source is NULL", sparse ? "sparse" : "window");
  if (!src->k || !src->v) return fail(SKV_E_NULL, "%s source K/V is NULL", sparse ? "sparse" : "window");
  SKV_TRY(check_align16(sparse ? "sparse source" : "window source", {src->k, src->v}));
  const bool fp8 = p.kv_dtype == SKV_FP8_E4M3FN;
  if (fp8 && (!src->k_scales || !src->v_scales))
    return fail(SKV_E_NULL, "fp8 %s source needs scales", sparse ? "sparse" : "window");
  // fp8 window buffers: one scale per row, read four rows at a time
  if (fp8 && !sparse && src->kind == SKV_SRC_WINDOW)
    SKV_TRY(check_align16("window scales", {src->k_scales, src->v_scales}));
  if (sparse) {
    if (src->kind != SKV_SRC_PAGED && src->kind != SKV_SRC_STAGED)
      return fail(SKV_E_UNSUPPORTED, "sparse source kind %d", src->kind);
    if (src->kind == SKV_SRC_PAGED && !src->block_table)
      return fail(SKV_E_NULL, "paged sparse source needs a block table");
    a.sparse_kind = src->kind;
    a.sk = src->k;
    a.sv = src->v;
    a.sks = fp8 ? src->k_scales : nullptr;
    a.svs = fp8 ? src->v_scales : nullptr;
    a.block_table = src->block_table;
  } else {
    if (src->kind != SKV_SRC_PAGED && src->kind != SKV_SRC_WINDOW)
      return fail(SKV_E_UNSUPPORTED, "window source kind %d", src->kind);
    if (src->kind == SKV_SRC_PAGED && !src->block_table)
      return fail(SKV_E_NULL, "paged window source needs a block table");
    if (src->kind == SKV_SRC_WINDOW) {
      if (p.window % p.block_size != 0)
        return fail(SKV_E_SHAPE, "window buffer needs window %% block_size == 0");
    }
    a.window_kind = src->kind;
    a.wk = src->k;
    a.wv = src->v;
    a.wks = fp8 ? src->k_scales : nullptr;
    a.wvs = fp8 ? src->v_scales : nullptr;
    a.window_table = src->block_table;
  }
  return SKV_OK;
}

skv_status check_ws(const Plan& pl, void* ws, size_t bytes) {
  if (!ws) return fail(SKV_E_WORKSPACE, "workspace is NULL");
  if (bytes < pl.total_bytes)
    return fail(SKV_E_WORKSPACE, "workspace %zu bytes < %zu needed", bytes, pl.total_bytes);
  return SKV_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Scoring with the in-kernel selection (first half of a decode step).  With
// cand_only (split step) the chunks publish their candidates and stop.
skv_status enqueue_score_select(const skv_problem& p, const Plan& pl, const skv_step_inputs& in,
                                const skv_step_outputs& out, char* ws, hipStream_t s, bool cand_only = false) {
  ScoreParams sp = score_params(p, in.q, in.landmarks, in.seq_lens);
  sp.scores = reinterpret_cast<float*>(ws + pl.off_scores);
  sp.score_cols = pl.max_cand > 0 ? pl.max_cand : 1;
  sp.rows_per_chunk = pl.rows_per_chunk;
  sp.fused_select = 1;
  sp.single_chunk = pl.score_chunks == 1;
  sp.two_level = pl.score_two_level;
  sp.cand_only = cand_only;
  sp.cand_cols = pl.cand_cols;
  sp.cand = Handoff<int32_t>(reinterpret_cast<int32_t*>(ws + pl.off_scores));
  sp.cand_stride = cand_only ? 3 * pl.cand_cols : pl.score_chunks * 2 * p.k_max;
  sp.cand_ids_lds = score_lds_bytes(sp.T, sp.D, sp.score_cols, sp.k_max, true, false, true) + kScoreStaticLds <=
                    kLdsPerWorkgroup;
  sp.block_table = in.block_table;
  sp.phys = reinterpret_cast<int32_t*>(ws + pl.off_phys);
  sp.k_per_seq = in.k_per_seq;
  sp.indices = out.indices;
  sp.n_sel = out.n_sel;
  sp.overlap = p.n_q_tokens == 2 ? out.overlap : nullptr;
  sp.counters = reinterpret_cast<unsigned*>(ws + pl.off_score_counters);
  SKV_TRY_HIP(launch_score(sp, pl.score_chunks, s), "score/top-k launch");
  return SKV_OK;
}

skv_status check_step_io(const skv_problem& p, const skv_step_inputs* in, const skv_step_outputs* out) {
  if (!in || !out) return fail(SKV_E_NULL, "inputs/outputs NULL");
  if (!in->q || !in->landmarks || !in->block_table || !in->seq_lens || !in->k_per_seq)
    return fail(SKV_E_NULL, "a required input pointer is NULL");
  if (!out->indices || !out->n_sel || !out->out)
    return fail(SKV_E_NULL, "a required output pointer is NULL");
  if (p.pool_location == SKV_POOL_DEVICE && (!in->k_pool || !in->v_pool))
    return fail(SKV_E_NULL, "K/V pool is NULL");
  if (p.pool_location == SKV_POOL_HOST && (!in->k_pool || !in->v_pool))
    return fail(SKV_E_NULL, "host K/V pool is NULL");
  if (p.pool_location == SKV_POOL_HOST && p.window > 0 && (!in->window_k || !in->window_v))
    return fail(SKV_E_NULL, "host pools need HBM window buffers");
  if (p.kv_dtype == SKV_FP8_E4M3FN && (!in->k_scales || !in->v_scales))
    return fail(SKV_E_NULL, "fp8 pools need scales");
  if (p.kv_dtype == SKV_FP8_E4M3FN && p.window > 0 && in->window_k) {
    // the device pool's fused step reads the window from the pool itself
    if (p.pool_location == SKV_POOL_DEVICE)
      return fail(SKV_E_UNSUPPORTED, "fp8 window buffers serve host pools only");
    if (!in->window_k_scales || !in->window_v_scales)
      return fail(SKV_E_NULL, "fp8 window buffers need per-row scales");
  }
  SKV_TRY(check_align16("decode step", {in->q, in->landmarks, in->k_pool, in->v_pool, in->window_k,
                                        in->window_v, in->window_k_scales, in->window_v_scales}));
  return SKV_OK;
}

// The scoring launch with the fused selection holds the keys of every
// candidate of a pair (both tokens), the selected ids and the selection's
// histograms in one workgroup's LDS.
skv_status check_select_lds(const skv_problem& p, const Plan& pl) {
  if (!pl.select_fits)
    return fail(SKV_E_UNSUPPORTED,
                "selection needs %zu bytes of LDS (> %zu): %d token(s) x %d candidates with k_max %d",
                pl.select_lds, kLdsPerWorkgroup, p.n_q_tokens, pl.max_cand, p.k_max);
  return SKV_OK;
}

// Attention of a device-pool step's second launch, straight from the pool
// through the selection's physical blocks; checked, not enqueued.
skv_status prepare_attend_paged(const skv_problem& p, const Plan& pl, const skv_step_inputs& in,
                                const skv_step_outputs& out, char* ws, AttnParams* a) {
  *a = attn_params(p, pl, in.q, in.seq_lens, out.out, out.lse, ws);
  skv_kv_source sparse{SKV_SRC_PAGED, in.k_pool, in.v_pool, in.k_scales, in.v_scales, in.block_table};
  skv_kv_source win = in.window_k
      ? skv_kv_source{SKV_SRC_WINDOW, in.window_k, in.window_v, nullptr, nullptr, nullptr}
      : sparse;
  SKV_TRY(set_source(p, *a, &sparse, true));
  SKV_TRY(set_source(p, *a, &win, false));
  a->indices = out.indices;
  a->n_sel = out.n_sel;
  a->phys = reinterpret_cast<const int32_t*>(ws + pl.off_phys);
  return SKV_OK;
}

// Compute units of the current device, queried once per device.
skv_status compute_units(int* cus) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  SKV_TRY_HIP(hipGetDevice(&dev), "device query");
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return SKV_OK;
    }
  }
  int c = 0;
  SKV_TRY_HIP(hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev), "device query");
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return SKV_OK;
}

// The whole device-pool step as one launch (step.hip).
skv_status enqueue_step(const skv_problem& p, const Plan& pl, const skv_step_inputs& in,
                        const skv_step_outputs& out, char* ws, hipStream_t s, size_t clear_bytes) {
  ScoreParams sp = score_params(p, in.q, in.landmarks, in.seq_lens);
  sp.scores = reinterpret_cast<float*>(ws + pl.off_scores);
  sp.score_cols = pl.max_cand > 0 ? pl.max_cand : 1;
  sp.rows_per_chunk = sp.score_cols;   // one chunk: the scores stay in LDS
  sp.fused_select = 1;
  sp.single_chunk = 1;
  sp.k_per_seq = in.k_per_seq;
  sp.indices = out.indices;
  sp.n_sel = out.n_sel;
  sp.overlap = p.n_q_tokens == 2 ? out.overlap : nullptr;
  sp.counters = reinterpret_cast<unsigned*>(ws + pl.off_score_counters);
  AttnParams a = attn_params(p, pl, in.q, in.seq_lens, out.out, out.lse, ws);
  skv_kv_source sparse{SKV_SRC_PAGED, in.k_pool, in.v_pool, in.k_scales, in.v_scales, in.block_table};
  skv_kv_source win = in.window_k
      ? skv_kv_source{SKV_SRC_WINDOW, in.window_k, in.window_v, nullptr, nullptr, nullptr}
      : sparse;
  SKV_TRY(set_source(p, a, &sparse, true));
  SKV_TRY(set_source(p, a, &win, false));
  a.indices = out.indices;
  a.n_sel = out.n_sel;
  a.n_splits = 1;
  int cus = 0;
  SKV_TRY(compute_units(&cus));
  a.longest_first = p.batch * p.n_kv_heads > cus;
  if (clear_bytes) SKV_TRY_HIP(launch_fill_zero(ws, clear_bytes, s), "workspace clear");
  SKV_TRY_HIP(launch_step(sp, a, pl.step_lds, s), "decode step launch");
  return SKV_OK;
}

// Gather of token 0's selection (the fields of a speculative correction stay null).
GatherParams gather_params(const skv_problem& p, const void* k_pool, const void* v_pool,
                           const float* k_scales, const float* v_scales, const int32_t* block_table,
                           const int32_t* indices, const int32_t* n_sel, void* k_stage, void* v_stage,
                           float* k_stage_scales, float* v_stage_scales) {
  GatherParams gp{};
  gp.k_pool = k_pool;
  gp.v_pool = v_pool;
  gp.k_scales = k_scales;
  gp.v_scales = v_scales;
  gp.block_table = block_table;
  gp.indices = indices;
  gp.n_sel = n_sel;
  gp.k_stage = k_stage;
  gp.v_stage = v_stage;
  gp.k_stage_scales = k_stage_scales;
  gp.v_stage_scales = v_stage_scales;
  gp.B = p.batch;
  gp.T = p.n_q_tokens;
  gp.Hkv = p.n_kv_heads;
  gp.max_blocks = p.max_blocks_per_seq;
  gp.k_max = p.k_max;
  gp.stride_block = p.pool_stride_block;
  gp.stride_head = p.pool_stride_head;
  gp.elem_bytes = elem_bytes(p.kv_dtype);
  gp.chunk_bytes = (int64_t)p.block_size * p.head_dim * gp.elem_bytes;
  gp.has_scales = p.kv_dtype == SKV_FP8_E4M3FN;
  return gp;
}

// A host-pool layer's gather (pinned pool -> stage slot) and attention (stage
// plus HBM window buffers), with every argument checked; nothing is enqueued.
struct HostLayer {
  GatherParams gp;
  AttnParams a;
};

skv_status prepare_host_layer(const skv_problem& p, const Plan& pl, const skv_step_inputs& in,
                              const skv_step_outputs& out, void* k_stage, void* v_stage,
                              float* k_stage_scales, float* v_stage_scales, char* ws, HostLayer* hl) {
  if (!k_stage || !v_stage) return fail(SKV_E_NULL, "host pools need staging buffers");
  if (p.kv_dtype == SKV_FP8_E4M3FN && (!k_stage_scales || !v_stage_scales))
    return fail(SKV_E_NULL, "fp8 staging needs scale buffers");
  SKV_TRY(check_align16("staging", {k_stage, v_stage}));
  hl->gp = gather_params(p, in.k_pool, in.v_pool, in.k_scales, in.v_scales, in.block_table, out.indices,
                         out.n_sel, k_stage, v_stage, k_stage_scales, v_stage_scales);
  hl->a = attn_params(p, pl, in.q, in.seq_lens, out.out, out.lse, ws);
  skv_kv_source sparse{SKV_SRC_STAGED, k_stage, v_stage, k_stage_scales, v_stage_scales, nullptr};
  SKV_TRY(set_source(p, hl->a, &sparse, true));
  if (p.window > 0) {
    skv_kv_source win{SKV_SRC_WINDOW, in.window_k, in.window_v, in.window_k_scales, in.window_v_scales, nullptr};
    SKV_TRY(set_source(p, hl->a, &win, false));
  } else {
    hl->a.window_kind = SKV_SRC_WINDOW;  // no window splits are launched
  }
  hl->a.indices = out.indices;
  hl->a.n_sel = out.n_sel;
  return SKV_OK;
}

// Gather on the copy stream once the layer's indices exist (ev_sel, recorded
// by the caller after the selection) and, if given, once slot_free has
// fired; attention on the compute stream once the gather is done.
skv_status enqueue_host_layer(const HostLayer& hl, hipStream_t s, hipStream_t cs, hipEvent_t ev_sel,
                              hipEvent_t ev_gather, hipEvent_t slot_free) {
  SKV_TRY_HIP(hipStreamWaitEvent(cs, ev_sel, 0), "stream wait");
  if (slot_free) SKV_TRY_HIP(hipStreamWaitEvent(cs, slot_free, 0), "stream wait");
  SKV_TRY_HIP(launch_gather(hl.gp, cs), "gather launch");
  SKV_TRY_HIP(hipEventRecord(ev_gather, cs), "event record");
  SKV_TRY_HIP(hipStreamWaitEvent(s, ev_gather, 0), "stream wait");
  SKV_TRY_HIP(launch_attend(hl.a, s), "attention launch");
  return SKV_OK;
}

struct EventSet {
  hipEvent_t e[64] = {};
  int n = 0;
  ~EventSet() {
    for (int i = 0; i < n; ++i) (void)hipEventDestroy(e[i]);
  }
  hipError_t make(int count, bool timing = false) {
    for (; n < count; ++n) {
      hipError_t r = hipEventCreateWithFlags(&e[n], timing ? hipEventDefault : hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
};

}  // namespace

skv_status check_device_step(const skv_problem* pr, const skv_step_inputs* in, const skv_step_outputs* out,
                             Plan* pl) {
  SKV_TRY(check_problem(pr));
  const skv_problem& p = *pr;
  if (p.pool_location != SKV_POOL_DEVICE) return fail(SKV_E_UNSUPPORTED, "device pools only");
  SKV_TRY(check_step_io(p, in, out));
  *pl = make_plan(p);
  if (!pl->fused_step) SKV_TRY(check_select_lds(p, *pl));
  return SKV_OK;
}

skv_status enqueue_device_step(const skv_problem& p, const Plan& pl, const skv_step_inputs& in,
                               const skv_step_outputs& out, char* ws, hipStream_t s, size_t clear_bytes,
                               int only) {
  if (pl.fused_step) return enqueue_step(p, pl, in, out, ws, s, clear_bytes);
  AttnParams a;
  SKV_TRY(prepare_attend_paged(p, pl, in, out, ws, &a));
  if (clear_bytes) SKV_TRY_HIP(launch_fill_zero(ws, clear_bytes, s), "workspace clear");
  if (only != 1) SKV_TRY(enqueue_score_select(p, pl, in, out, ws, s, pl.split_step != 0));
  if (only == 0) return SKV_OK;
  if (!pl.split_step) {
    SKV_TRY_HIP(launch_attend(a, s), "attention launch");
    return SKV_OK;
  }
  // split step: the final selection and the attention in one launch
  ScoreParams sp = score_params(p, in.q, in.landmarks, in.seq_lens);
  sp.score_cols = pl.cand_cols;
  sp.rows_per_chunk = pl.rows_per_chunk;
  sp.cand = Handoff<int32_t>(reinterpret_cast<int32_t*>(ws + pl.off_scores));
  sp.cand_cols = pl.cand_cols;
  sp.cand_stride = 3 * pl.cand_cols;
  sp.k_per_seq = in.k_per_seq;
  sp.indices = out.indices;
  sp.n_sel = out.n_sel;
  sp.overlap = p.n_q_tokens == 2 ? out.overlap : nullptr;
  SKV_TRY_HIP(launch_split_step(sp, a, pl.split_lds, s), "selection + attention launch");
  return SKV_OK;
}

}  // namespace skv

using namespace skv;

extern "C" {

const char* sparsekv_status_string(int status) {
  switch (status) {
    case SKV_OK: return "ok";
    case SKV_E_NULL: return "null pointer";
    case SKV_E_SHAPE: return "bad shape";
    case SKV_E_DTYPE: return "bad dtype";
    case SKV_E_UNSUPPORTED: return "unsupported combination";
    case SKV_E_WORKSPACE: return "workspace missing or too small";
    case SKV_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* sparsekv_last_error(void) { return g_err; }

const char* sparsekv_version(void) { return "0.1.0"; }

skv_status sparsekv_workspace_size(const skv_problem* pr, size_t* bytes) {
  SKV_TRY(check_problem(pr));
  if (!bytes) return fail(SKV_E_NULL, "bytes is NULL");
  *bytes = make_plan(*pr).total_bytes;
  return SKV_OK;
}

skv_status sparsekv_decode_step_launches(const skv_problem* pr, int32_t* launches) {
  SKV_TRY(check_problem(pr));
  if (!launches) return fail(SKV_E_NULL, "launches is NULL");
  if (pr->pool_location == SKV_POOL_HOST) *launches = 3;
  else *launches = make_plan(*pr).fused_step ? 1 : 2;
  return SKV_OK;
}

skv_status sparsekv_decode_step_kernel(const skv_problem* pr, int32_t launch, const char** name) {
  SKV_TRY(check_problem(pr));
  if (!name) return fail(SKV_E_NULL, "name is NULL");
  static const char* const kHost[] = {"score_kernel", "gather_kernel", "attend_kernel"};
  static const char* const kFused[] = {"pair_step_kernel"};
  static const char* const kSplit[] = {"score_kernel", "split_step_kernel"};
  static const char* const kTwo[] = {"score_kernel", "attend_kernel"};
  const char* const* names;
  int n;
  if (pr->pool_location == SKV_POOL_HOST) {
    names = kHost;
    n = 3;
  } else {
    const Plan pl = make_plan(*pr);
    names = pl.fused_step ? kFused : pl.split_step ? kSplit : kTwo;
    n = pl.fused_step ? 1 : 2;
  }
  if (launch < 0 || launch >= n) return fail(SKV_E_SHAPE, "launch %d outside [0, %d)", (int)launch, n);
  *name = names[launch];
  return SKV_OK;
}

skv_status sparsekv_decode_step_launch_times(const skv_problem* pr, const skv_step_inputs* in,
                                             const skv_step_outputs* out, void* workspace,
                                             size_t workspace_bytes, void* stream, int32_t n_steps,
                                             float* launch_us) {
  Plan pl;
  SKV_TRY(check_device_step(pr, in, out, &pl));
  SKV_TRY(check_ws(pl, workspace, workspace_bytes));
  if (!launch_us) return fail(SKV_E_NULL, "launch_us is NULL");
  if (n_steps < 1 || n_steps > 4096) return fail(SKV_E_SHAPE, "n_steps %d outside [1, 4096]", (int)n_steps);
  const int nl = pl.fused_step ? 1 : 2;
  hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  EventSet ev;
  SKV_TRY_HIP(ev.make(2, true), "event create");
  // one whole step, so every launch finds its inputs; then each launch alone,
  // n_steps times back to back (a launch does not change what it reads)
  SKV_TRY(enqueue_device_step(*pr, pl, *in, *out, ws, s, 0));
  for (int l = 0; l < nl; ++l) {
    SKV_TRY_HIP(hipEventRecord(ev.e[0], s), "event record");
    for (int i = 0; i < n_steps; ++i) SKV_TRY(enqueue_device_step(*pr, pl, *in, *out, ws, s, 0, nl == 1 ? -1 : l));
    SKV_TRY_HIP(hipEventRecord(ev.e[1], s), "event record");
    SKV_TRY_HIP(hipEventSynchronize(ev.e[1]), "event synchronize");
    float ms = 0.f;
    SKV_TRY_HIP(hipEventElapsedTime(&ms, ev.e[0], ev.e[1]), "event time");
    launch_us[l] = ms * 1e3f / (float)n_steps;
  }
  // the outputs end as a whole step leaves them
  if (nl > 1) SKV_TRY(enqueue_device_step(*pr, pl, *in, *out, ws, s, 0));
  SKV_TRY_HIP(hipStreamSynchronize(s), "stream synchronize");
  return SKV_OK;
}

skv_status sparsekv_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace) return fail(SKV_E_NULL, "workspace is NULL");
  SKV_TRY_HIP(launch_fill_zero(workspace, bytes, as_stream(stream)), "workspace fill");
  return SKV_OK;
}

skv_status sparsekv_stream_read(const void* buffer, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
  if (!buffer || !sink) return fail(SKV_E_NULL, "stream_read: NULL argument");
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buffer) % 16 != 0)
    return fail(SKV_E_SHAPE, "stream_read: buffer and size must be multiples of 16 bytes");
  if (sink_bytes < 4 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return fail(SKV_E_SHAPE, "stream_read: the sink needs at least one aligned 32-bit word");
  const size_t words = sink_bytes / 4;
  SKV_TRY_HIP(launch_stream_read(buffer, bytes, static_cast<uint32_t*>(sink),
                                 (int)(words < (1u << 20) ? words : (1u << 20)), as_stream(stream)),
              "stream read launch");
  return SKV_OK;
}

skv_status sparsekv_score(const skv_problem* pr, const void* q, const void* landmarks,
                          const int32_t* seq_lens, float* scores, void* stream) {
  SKV_TRY(check_problem(pr));
  if (!q || !landmarks || !seq_lens || !scores) return fail(SKV_E_NULL, "score: NULL argument");
  SKV_TRY(check_align16("score", {q, landmarks}));
  const skv_problem& p = *pr;
  ScoreParams sp = score_params(p, q, landmarks, seq_lens);
  sp.scores = scores;
  sp.score_cols = p.max_blocks_per_seq;
  const int lm_es = p.landmark_dtype == SKV_F32 ? 4 : 2;
  const int rps = 8 * (64 / (p.head_dim * lm_es / 16));
#ifndef SKV_SCORE_STEPS
#define SKV_SCORE_STEPS 16
#endif
  sp.rows_per_chunk = rps * SKV_SCORE_STEPS;
  sp.fused_select = 0;
  const int chunks = (p.max_blocks_per_seq + sp.rows_per_chunk - 1) / sp.rows_per_chunk;
  SKV_TRY_HIP(launch_score(sp, chunks, as_stream(stream)), "score launch");
  return SKV_OK;
}

skv_status sparsekv_topk(const skv_problem* pr, const float* scores, const int32_t* seq_lens,
                         const int32_t* k_per_seq, int32_t* indices, int32_t* n_sel, float* overlap,
                         void* stream) {
  SKV_TRY(check_problem(pr));
  const skv_problem& p = *pr;
  // one workgroup holds a row's keys and the selected ids in LDS
  const size_t lds = topk_lds_bytes(p.max_blocks_per_seq) + (size_t)2 * p.k_max * 4 + select_static_lds_bytes();
  if (lds > kLdsPerWorkgroup)
    return fail(SKV_E_UNSUPPORTED, "topk needs %zu bytes of LDS (> %zu): max_blocks %d, k_max %d", lds,
                kLdsPerWorkgroup, p.max_blocks_per_seq, p.k_max);
  if (!scores || !seq_lens || !k_per_seq || !indices || !n_sel)
    return fail(SKV_E_NULL, "topk: NULL argument");
  TopkParams tp{};
  tp.scores = scores;
  tp.seq_lens = seq_lens;
  tp.k_per_seq = k_per_seq;
  tp.indices = indices;
  tp.n_sel = n_sel;
  tp.overlap = p.n_q_tokens == 2 ? overlap : nullptr;
  tp.B = p.batch;
  tp.T = p.n_q_tokens;
  tp.Hkv = p.n_kv_heads;
  tp.blk = p.block_size;
  tp.max_blocks = p.max_blocks_per_seq;
  tp.window = p.window;
  tp.k_max = p.k_max;
  SKV_TRY_HIP(launch_topk(tp, as_stream(stream)), "top-k launch");
  return SKV_OK;
}

skv_status sparsekv_gather(const skv_problem* pr, const void* k_pool, const void* v_pool,
                           const float* k_scales, const float* v_scales, const int32_t* block_table,
                           const int32_t* indices, const int32_t* n_sel, void* k_stage, void* v_stage,
                           float* k_stage_scales, float* v_stage_scales, void* stream) {
  SKV_TRY(check_problem(pr));
  const skv_problem& p = *pr;
  if (!k_pool || !v_pool || !block_table || !indices || !n_sel || !k_stage || !v_stage)
    return fail(SKV_E_NULL, "gather: NULL argument");
  const bool fp8 = p.kv_dtype == SKV_FP8_E4M3FN;
  if (fp8 && (!k_scales || !v_scales || !k_stage_scales || !v_stage_scales))
    return fail(SKV_E_NULL, "gather: fp8 needs pool and stage scales");
  SKV_TRY(check_align16("gather", {k_pool, v_pool, k_stage, v_stage}));
  GatherParams gp = gather_params(p, k_pool, v_pool, k_scales, v_scales, block_table, indices, n_sel,
                                  k_stage, v_stage, k_stage_scales, v_stage_scales);
  SKV_TRY_HIP(launch_gather(gp, as_stream(stream)), "gather launch");
  return SKV_OK;
}

skv_status sparsekv_gather_correct(const skv_problem* pr, const void* k_pool, const void* v_pool,
                                   const float* k_scales, const float* v_scales,
                                   const int32_t* block_table, const int32_t* spec_indices,
                                   const int32_t* spec_n_sel, int32_t spec_token,
                                   const void* spec_k_stage, const void* spec_v_stage,
                                   const float* spec_k_scales, const float* spec_v_scales,
                                   const int32_t* real_indices, const int32_t* real_n_sel,
                                   int32_t real_token, void* k_stage, void* v_stage,
                                   float* k_stage_scales, float* v_stage_scales, int32_t* misses,
                                   void* stream) {
  SKV_TRY(check_problem(pr));
  const skv_problem& p = *pr;
  if (!k_pool || !v_pool || !block_table || !spec_indices || !spec_n_sel || !spec_k_stage ||
      !spec_v_stage || !real_indices || !real_n_sel || !k_stage || !v_stage)
    return fail(SKV_E_NULL, "gather_correct: NULL argument");
  if (spec_token < 0 || spec_token >= p.n_q_tokens || real_token < 0 || real_token >= p.n_q_tokens)
    return fail(SKV_E_SHAPE, "gather_correct: tokens %d, %d not in [0, %d)", spec_token, real_token,
                p.n_q_tokens);
  const bool fp8 = p.kv_dtype == SKV_FP8_E4M3FN;
  if (fp8 && (!k_scales || !v_scales || !k_stage_scales || !v_stage_scales || !spec_k_scales ||
              !spec_v_scales))
    return fail(SKV_E_NULL, "gather_correct: fp8 needs pool and stage scales");
  SKV_TRY(check_align16("gather_correct", {k_pool, v_pool, spec_k_stage, spec_v_stage, k_stage, v_stage}));
  const size_t stage_bytes = (size_t)p.batch * p.n_kv_heads * p.k_max * p.block_size * p.head_dim *
                             elem_bytes(p.kv_dtype);
  auto overlaps = [&](const void* a, const void* b) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + stage_bytes && y < x + stage_bytes;
  };
  if (overlaps(k_stage, spec_k_stage) || overlaps(v_stage, spec_v_stage))
    return fail(SKV_E_SHAPE, "gather_correct: the speculative and the output stages overlap");
  GatherParams gp = gather_params(p, k_pool, v_pool, k_scales, v_scales, block_table, real_indices,
                                  real_n_sel, k_stage, v_stage, k_stage_scales, v_stage_scales);
  gp.token = real_token;
  gp.spec_indices = spec_indices;
  gp.spec_n_sel = spec_n_sel;
  gp.spec_token = spec_token;
  gp.spec_k_stage = spec_k_stage;
  gp.spec_v_stage = spec_v_stage;
  gp.spec_k_scales = spec_k_scales;
  gp.spec_v_scales = spec_v_scales;
  gp.misses = misses;
  SKV_TRY_HIP(launch_gather(gp, as_stream(stream)), "gather_correct launch");
  return SKV_OK;
}

skv_status sparsekv_attend(const skv_problem* pr, const void* q, const skv_kv_source* sparse,
                           const int32_t* indices, const int32_t* n_sel, const skv_kv_source* window,
                           const int32_t* seq_lens, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  SKV_TRY(check_problem(pr));
  const skv_problem& p = *pr;
  if (!q || !indices || !n_sel || !seq_lens || !out) return fail(SKV_E_NULL, "attend: NULL argument");
  SKV_TRY(check_align16("attend", {q}));
  const Plan pl = make_plan(p);
  SKV_TRY(check_ws(pl, workspace, workspace_bytes));
  char* ws = static_cast<char*>(workspace);
  AttnParams a = attn_params(p, pl, q, seq_lens, out, lse, ws);
  SKV_TRY(set_source(p, a, sparse, true));
  if (p.window > 0) SKV_TRY(set_source(p, a, window, false));
  else a.window_kind = SKV_SRC_WINDOW;
  a.indices = indices;
  a.n_sel = n_sel;
  SKV_TRY_HIP(launch_attend(a, as_stream(stream)), "attention launch");
  return SKV_OK;
}

skv_status sparsekv_attend_cobatched(const skv_problem* pr, const void* q, const skv_kv_source* sparse,
                                     const int32_t* indices, const int32_t* n_sel,
                                     const skv_kv_source* window, const int32_t* seq_lens, float* out,
                                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  SKV_TRY(check_problem(pr));
  const skv_problem& p = *pr;
  // one token: the output layouts coincide with sparsekv_attend's
  if (p.n_q_tokens == 1)
    return sparsekv_attend(pr, q, sparse, indices, n_sel, window, seq_lens, out, lse, workspace,
                           workspace_bytes, stream);
  if (!q || !indices || !n_sel || !seq_lens || !out) return fail(SKV_E_NULL, "attend_cobatched: NULL argument");
  SKV_TRY(check_align16("attend_cobatched", {q}));
  if (!sparse) return fail(SKV_E_NULL, "sparse source is NULL");
  if (sparse->kind != SKV_SRC_PAGED)
    return fail(SKV_E_UNSUPPORTED, "attend_cobatched reads the union of the selections from a paged source");
  if (p.pool_location != SKV_POOL_DEVICE)
    return fail(SKV_E_UNSUPPORTED, "attend_cobatched needs a device pool");
  if (p.kv_dtype == SKV_FP8_E4M3FN && p.window > 0 && window && window->kind == SKV_SRC_WINDOW)
    return fail(SKV_E_UNSUPPORTED, "attend_cobatched: fp8 window buffers");
  const Plan pl = make_plan(p);
  SKV_TRY(check_ws(pl, workspace, workspace_bytes));
  char* ws = static_cast<char*>(workspace);
  AttnParams a = attn_params(p, pl, q, seq_lens, out, lse, ws);
  a.n_splits = pl.cob_n_splits;
  a.items_per_split = pl.cob_items_per_split;
  SKV_TRY(set_source(p, a, sparse, true));
  if (p.window > 0) SKV_TRY(set_source(p, a, window, false));
  else a.window_kind = SKV_SRC_WINDOW;
  a.indices = indices;
  a.n_sel = n_sel;
  SKV_TRY_HIP(launch_attend_cobatched(a, as_stream(stream)), "co-batched attention launch");
  return SKV_OK;
}

skv_status sparsekv_decode_step(const skv_problem* pr, const skv_step_inputs* in,
                                const skv_step_outputs* out, void* k_stage, void* v_stage,
                                float* k_stage_scales, float* v_stage_scales, void* workspace,
                                size_t workspace_bytes, void* stream, void* copy_stream) {
  SKV_TRY(check_problem(pr));
  const skv_problem& p = *pr;
  SKV_TRY(check_step_io(p, in, out));
  const Plan pl = make_plan(p);
  if (p.pool_location == SKV_POOL_HOST || !pl.fused_step) SKV_TRY(check_select_lds(p, pl));
  SKV_TRY(check_ws(pl, workspace, workspace_bytes));
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = as_stream(stream);
  if (p.pool_location == SKV_POOL_DEVICE) return enqueue_device_step(p, pl, *in, *out, ws, s, 0);
  HostLayer hl;
  SKV_TRY(prepare_host_layer(p, pl, *in, *out, k_stage, v_stage, k_stage_scales, v_stage_scales, ws, &hl));
  hipStream_t cs = copy_stream ? as_stream(copy_stream) : s;
  EventSet ev;
  SKV_TRY_HIP(ev.make(2), "event create");
  SKV_TRY(enqueue_score_select(p, pl, *in, *out, ws, s));
  SKV_TRY_HIP(hipEventRecord(ev.e[0], s), "event record");
  return enqueue_host_layer(hl, s, cs, ev.e[0], ev.e[1], nullptr);
}

namespace {
HostAttnArgs host_args(const skv_problem& p, const skv_host_part& host) {
  HostAttnArgs h{};
  h.B = p.batch;
  h.T = p.n_q_tokens;
  h.Hq = p.n_q_heads;
  h.Hkv = p.n_kv_heads;
  h.D = p.head_dim;
  h.blk = p.block_size;
  h.window = p.window;
  h.max_blocks = p.max_blocks_per_seq;
  h.k_max = p.k_max;
  h.kv_dtype = p.kv_dtype;
  h.stride_block = p.pool_stride_block;
  h.stride_head = p.pool_stride_head;
  h.q = host.q;
  h.seq_lens = host.seq_lens;
  h.block_table = host.block_table;
  h.indices = host.indices;
  h.n_sel = host.n_sel;
  h.k_pool = host.k_pool;
  h.v_pool = host.v_pool;
  h.k_scales = host.k_scales;
  h.v_scales = host.v_scales;
  h.o = host.o;
  h.lse = host.lse;
  h.n_threads = host.n_threads;
  return h;
}

skv_status check_host_part(const skv_problem& p, const skv_host_part* host) {
  if (p.pool_location != SKV_POOL_HOST) return fail(SKV_E_UNSUPPORTED, "host attention: host pools only");
  if (!host || !host->k_pool || !host->v_pool || !host->q || !host->seq_lens || !host->block_table ||
      !host->indices || !host->n_sel || !host->o || !host->lse)
    return fail(SKV_E_NULL, "host attention: NULL host buffer");
  if (p.kv_dtype == SKV_FP8_E4M3FN && (!host->k_scales || !host->v_scales))
    return fail(SKV_E_NULL, "host attention: fp8 needs host scales");
  return SKV_OK;
}
}  // namespace

skv_status sparsekv_host_attention(const skv_problem* pr, const skv_host_part* host) {
  SKV_TRY(check_problem(pr));
  SKV_TRY(check_host_part(*pr, host));
  host_sparse_attention(host_args(*pr, *host));
  return SKV_OK;
}

skv_status sparsekv_decode_step_hybrid(const skv_problem* pr, const skv_step_inputs* in,
                                       const skv_step_outputs* out, const skv_host_part* host,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  SKV_TRY(check_problem(pr));
  const skv_problem& p = *pr;
  if (p.pool_location != SKV_POOL_HOST) return fail(SKV_E_UNSUPPORTED, "hybrid step: host pools only");
  SKV_TRY(check_step_io(p, in, out));
  SKV_TRY(check_host_part(p, host));
  const bool fp8 = p.kv_dtype == SKV_FP8_E4M3FN;
  if (p.window > 0 && p.window % p.block_size != 0)
    return fail(SKV_E_SHAPE, "hybrid step: window buffers need window %% block_size == 0");
  const Plan pl = make_plan(p);
  SKV_TRY(check_select_lds(p, pl));
  SKV_TRY(check_ws(pl, workspace, workspace_bytes));
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = as_stream(stream);
  const int D = p.head_dim;

  // ---- checks and lookups before any GPU work: the window attention's
  // arguments and the device addresses of the host part's pinned outputs
  float* o_win = reinterpret_cast<float*>(ws + pl.off_hybrid);
  float* lse_win = o_win + (size_t)p.batch * p.n_q_heads * D;
  AttnParams a{};
  if (p.window > 0) {
    a = attn_params(p, pl, in->q, in->seq_lens, o_win, lse_win, ws);
    skv_kv_source win{SKV_SRC_WINDOW, in->window_k, in->window_v, in->window_k_scales, in->window_v_scales,
                      nullptr};
    SKV_TRY(set_source(p, a, &win, false));
    // no sparse item is attended; waves without an item read row 0 of the
    // window buffers (and, fp8, the first of their scales)
    skv_kv_source none{SKV_SRC_STAGED, in->window_k, in->window_v, in->window_k_scales, in->window_v_scales,
                       nullptr};
    SKV_TRY(set_source(p, a, &none, true));
    a.indices = out->indices;
    a.n_sel = out->n_sel;
    a.window_only = 1;
  }
  float* o_host = nullptr;
  float* lse_host = nullptr;
  SKV_TRY_HIP(hipHostGetDevicePointer(reinterpret_cast<void**>(&o_host), host->o, 0), "host output address");
  SKV_TRY_HIP(hipHostGetDevicePointer(reinterpret_cast<void**>(&lse_host), host->lse, 0), "host lse address");
  EventSet ev;
  SKV_TRY_HIP(ev.make(1), "event create");

  // ---- GPU: scoring and selection, then the inputs of the sparse part to the host
  SKV_TRY(enqueue_score_select(p, pl, *in, *out, ws, s));
  const size_t qbytes = (size_t)p.batch * p.n_q_tokens * p.n_q_heads * D * elem_bytes(p.q_dtype);
  const size_t sel = (size_t)p.batch * p.n_q_tokens * p.n_kv_heads;
  auto d2h = [&](void* dst, const void* src, size_t bytes) {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, s);
  };
  SKV_TRY_HIP(d2h(host->q, in->q, qbytes), "query copy");
  SKV_TRY_HIP(d2h(host->seq_lens, in->seq_lens, (size_t)p.batch * 4), "length copy");
  SKV_TRY_HIP(d2h(host->block_table, in->block_table, (size_t)p.batch * p.max_blocks_per_seq * 4), "table copy");
  SKV_TRY_HIP(d2h(host->indices, out->indices, sel * p.k_max * 4), "selection copy");
  SKV_TRY_HIP(d2h(host->n_sel, out->n_sel, sel * 4), "selection copy");
  if (fp8) {
    SKV_TRY_HIP(d2h(host->k_scales, in->k_scales, (size_t)p.n_pool_blocks * p.n_kv_heads * 4), "scale copy");
    SKV_TRY_HIP(d2h(host->v_scales, in->v_scales, (size_t)p.n_pool_blocks * p.n_kv_heads * 4), "scale copy");
  }
  SKV_TRY_HIP(hipEventRecord(ev.e[0], s), "event record");

  // ---- GPU: attention over the window alone, while the host works
  if (p.window > 0) SKV_TRY_HIP(launch_attend(a, s), "window attention launch");

  // ---- host: the sparse part, once the selection has arrived
  SKV_TRY_HIP(hipEventSynchronize(ev.e[0]), "selection wait");
  host_sparse_attention(host_args(p, *host));

  // ---- GPU: fuse the two parts
  SKV_TRY_HIP(launch_lse_merge(p.window > 0 ? o_win : nullptr, p.window > 0 ? lse_win : nullptr, o_host, lse_host,
                               out->out, out->lse, p.batch * p.n_q_heads, D, s),
              "fusion launch");
  return SKV_OK;
}

namespace {
constexpr int kMaxLayers = 16;

skv_status check_layers(const skv_problem& p, int32_t n_layers, const skv_step_inputs* in,
                        const skv_step_outputs* out, const char* where) {
  if (p.pool_location != SKV_POOL_HOST) return fail(SKV_E_UNSUPPORTED, "%s pipelines host pools only", where);
  if (n_layers < 1 || n_layers > kMaxLayers)
    return fail(SKV_E_SHAPE, "%s: n_layers %d not in [1, %d]", where, n_layers, kMaxLayers);
  if (!in || !out) return fail(SKV_E_NULL, "%s: NULL argument", where);
  for (int l = 0; l < n_layers; ++l) SKV_TRY(check_step_io(p, &in[l], &out[l]));
  return SKV_OK;
}

skv_status check_slots(const skv_problem& p, int32_t n_layers, void* const* k, void* const* v,
                       float* const* ks, float* const* vs, const char* what) {
  if (!k || !v) return fail(SKV_E_NULL, "%s: NULL slot array", what);
  for (int slot = 0; slot < 2 && slot < n_layers; ++slot) {
    if (!k[slot] || !v[slot]) return fail(SKV_E_NULL, "%s slot %d is NULL", what, slot);
    if (p.kv_dtype == SKV_FP8_E4M3FN && (!ks || !vs || !ks[slot] || !vs[slot]))
      return fail(SKV_E_NULL, "fp8 %s slot %d needs scales", what, slot);
    SKV_TRY(check_align16(what, {k[slot], v[slot]}));
  }
  return SKV_OK;
}
}  // namespace

skv_status sparsekv_decode_layers(const skv_problem* pr, int32_t n_layers, const skv_step_inputs* in,
                                  const skv_step_outputs* out, void* const* k_stage,
                                  void* const* v_stage, float* const* k_stage_scales,
                                  float* const* v_stage_scales, void* workspace,
                                  size_t workspace_bytes, void* stream, void* copy_stream) {
  SKV_TRY(check_problem(pr));
  const skv_problem& p = *pr;
  SKV_TRY(check_layers(p, n_layers, in, out, "decode_layers"));
  SKV_TRY(check_slots(p, n_layers, k_stage, v_stage, k_stage_scales, v_stage_scales, "staging"));
  const Plan pl = make_plan(p);
  SKV_TRY(check_select_lds(p, pl));
  SKV_TRY(check_ws(pl, workspace, workspace_bytes));
  char* ws = static_cast<char*>(workspace);
  HostLayer layers[kMaxLayers];
  for (int l = 0; l < n_layers; ++l) {
    const int slot = l & 1;
    SKV_TRY(prepare_host_layer(p, pl, in[l], out[l], k_stage[slot], v_stage[slot],
                               k_stage_scales ? k_stage_scales[slot] : nullptr,
                               v_stage_scales ? v_stage_scales[slot] : nullptr, ws, &layers[l]));
  }
  hipStream_t s = as_stream(stream);
  hipStream_t cs = copy_stream ? as_stream(copy_stream) : s;
  EventSet ev;
  SKV_TRY_HIP(ev.make(3 * n_layers), "event create");
  hipEvent_t* ev_sel = ev.e;
  hipEvent_t* ev_gather = ev.e + n_layers;
  hipEvent_t* ev_attn = ev.e + 2 * n_layers;
  // Selection of every layer first (the per-layer queries are given up front),
  // so the copy stream can run ahead; slot l % 2 is reused once layer l-2's
  // attention is done.
  for (int l = 0; l < n_layers; ++l) {
    SKV_TRY(enqueue_score_select(p, pl, in[l], out[l], ws, s));
    SKV_TRY_HIP(hipEventRecord(ev_sel[l], s), "event record");
  }
  for (int l = 0; l < n_layers; ++l) {
    SKV_TRY(enqueue_host_layer(layers[l], s, cs, ev_sel[l], ev_gather[l], l >= 2 ? ev_attn[l - 2] : nullptr));
    SKV_TRY_HIP(hipEventRecord(ev_attn[l], s), "event record");
  }
  // the caller's stream ends after every layer's attention; join the copy stream too
  if (cs != s) SKV_TRY_HIP(hipStreamWaitEvent(s, ev_gather[n_layers - 1], 0), "stream wait");
  return SKV_OK;
}

skv_status sparsekv_decode_layers_predicted(const skv_problem* pr, int32_t n_layers,
                                            const skv_step_inputs* in, const skv_step_outputs* out,
                                            const skv_layer_prediction* pred, void* const* pref_k,
                                            void* const* pref_v, float* const* pref_k_scales,
                                            float* const* pref_v_scales, void* k_stage, void* v_stage,
                                            float* k_stage_scales, float* v_stage_scales, void* workspace,
                                            size_t workspace_bytes, void* stream, void* copy_stream) {
  SKV_TRY(check_problem(pr));
  const skv_problem& p = *pr;
  SKV_TRY(check_layers(p, n_layers, in, out, "decode_layers_predicted"));
  if (!pred) return fail(SKV_E_NULL, "decode_layers_predicted: NULL prediction array");
  for (int l = 0; l < n_layers; ++l) {
    if (!pred[l].indices || !pred[l].n_sel) return fail(SKV_E_NULL, "prediction of layer %d is NULL", l);
    if (pred[l].token < 0 || pred[l].token >= p.n_q_tokens)
      return fail(SKV_E_SHAPE, "prediction of layer %d: token %d not in [0, %d)", l, pred[l].token,
                  p.n_q_tokens);
  }
  SKV_TRY(check_slots(p, n_layers, pref_k, pref_v, pref_k_scales, pref_v_scales, "prefetch"));
  const Plan pl = make_plan(p);
  SKV_TRY(check_select_lds(p, pl));
  SKV_TRY(check_ws(pl, workspace, workspace_bytes));
  char* ws = static_cast<char*>(workspace);
  // the real stage must not overlap a prefetch slot: a hit reads a prefetch
  // slot while other workgroups write the real stage
  const size_t stage_bytes = (size_t)p.batch * p.n_kv_heads * p.k_max * p.block_size * p.head_dim *
                             elem_bytes(p.kv_dtype);
  auto overlaps = [&](const void* a, const void* b) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + stage_bytes && y < x + stage_bytes;
  };
  for (int slot = 0; slot < 2 && slot < n_layers; ++slot)
    if (overlaps(k_stage, pref_k[slot]) || overlaps(v_stage, pref_v[slot]) || overlaps(k_stage, pref_v[slot]) ||
        overlaps(v_stage, pref_k[slot]))
      return fail(SKV_E_SHAPE, "decode_layers_predicted: the stage overlaps prefetch slot %d", slot);
  // per layer: the prefetch gather (prediction -> slot l % 2), the correction
  // (slot -> stage, misses from the pool) and the attention of the stage
  GatherParams prefetch[kMaxLayers];
  HostLayer layers[kMaxLayers];
  for (int l = 0; l < n_layers; ++l) {
    const int slot = l & 1;
    float* pks = pref_k_scales ? pref_k_scales[slot] : nullptr;
    float* pvs = pref_v_scales ? pref_v_scales[slot] : nullptr;
    prefetch[l] = gather_params(p, in[l].k_pool, in[l].v_pool, in[l].k_scales, in[l].v_scales,
                                in[l].block_table, pred[l].indices, pred[l].n_sel, pref_k[slot], pref_v[slot],
                                pks, pvs);
    prefetch[l].token = pred[l].token;
    SKV_TRY(prepare_host_layer(p, pl, in[l], out[l], k_stage, v_stage, k_stage_scales, v_stage_scales, ws,
                               &layers[l]));
    GatherParams& gp = layers[l].gp;
    gp.spec_indices = pred[l].indices;
    gp.spec_n_sel = pred[l].n_sel;
    gp.spec_token = pred[l].token;
    gp.spec_k_stage = pref_k[slot];
    gp.spec_v_stage = pref_v[slot];
    gp.spec_k_scales = pks;
    gp.spec_v_scales = pvs;
    gp.misses = pred[l].misses;
  }
  hipStream_t s = as_stream(stream);
  hipStream_t cs = copy_stream ? as_stream(copy_stream) : s;
  EventSet ev;
  SKV_TRY_HIP(ev.make(2 * n_layers + 1), "event create");
  hipEvent_t* ev_pref = ev.e;
  hipEvent_t* ev_corr = ev.e + n_layers;
  hipEvent_t ev_start = ev.e[2 * n_layers];
  // the copy stream starts after the work the caller queued on `stream`
  // (which may still be writing the predictions)
  SKV_TRY_HIP(hipEventRecord(ev_start, s), "event record");
  SKV_TRY_HIP(hipStreamWaitEvent(cs, ev_start, 0), "stream wait");
  // copy stream: every layer's predicted blocks, two layers ahead at most
  // (slot l % 2 is free once layer l-2's correction has read it)
  auto enqueue_prefetch = [&](int l) -> skv_status {
    if (l >= 2) SKV_TRY_HIP(hipStreamWaitEvent(cs, ev_corr[l - 2], 0), "stream wait");
    SKV_TRY_HIP(launch_gather(prefetch[l], cs), "prefetch launch");
    SKV_TRY_HIP(hipEventRecord(ev_pref[l], cs), "event record");
    return SKV_OK;
  };
  for (int l = 0; l < n_layers && l < 2; ++l) SKV_TRY(enqueue_prefetch(l));
  // compute stream, per layer in order: selection, then (once the layer's
  // prefetch is staged) the correction that fetches only the misses, then
  // the attention of the corrected stage
  for (int l = 0; l < n_layers; ++l) {
    SKV_TRY(enqueue_score_select(p, pl, in[l], out[l], ws, s));
    SKV_TRY_HIP(hipStreamWaitEvent(s, ev_pref[l], 0), "stream wait");
    SKV_TRY_HIP(launch_gather(layers[l].gp, s), "correction launch");
    SKV_TRY_HIP(hipEventRecord(ev_corr[l], s), "event record");
    SKV_TRY_HIP(launch_attend(layers[l].a, s), "attention launch");
    if (l + 2 < n_layers) SKV_TRY(enqueue_prefetch(l + 2));
  }
  return SKV_OK;
}

}  // extern "C"
