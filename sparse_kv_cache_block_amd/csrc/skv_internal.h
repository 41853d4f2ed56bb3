// skv_internal.h -- parameter blocks and launchers shared between the C ABI
// (sparsekv.hip) and the kernel translation units.  Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sparsekv.h"

namespace skv {

// ------------------------------------------------------------------ errors
// Set the calling thread's error text (sparsekv_last_error) and return st.
skv_status fail(skv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// SKV_E_HIP with the runtime's text for e.
skv_status hip_fail(hipError_t e, const char* what);

#define SKV_TRY_HIP(expr, what)                          \
  do {                                                   \
    hipError_t e_ = (expr);                              \
    if (e_ != hipSuccess) return ::skv::hip_fail(e_, what); \
  } while (0)

#define SKV_TRY(expr)                  \
  do {                                 \
    skv_status s_ = (expr);            \
    if (s_ != SKV_OK) return s_;       \
  } while (0)

// A buffer that the workgroups of one launch hand to each other (split
// partials, the chunks' candidates).  The XCDs' L2 caches are not coherent
// with each other, and the hand-off avoids fences (see publish_f32 in
// skv_device.h), so every value in such a buffer must be written with an
// agent-scope atomic store and read with an agent-scope atomic load.  The
// class offers only those two accesses: a plain load or store into the buffer
// does not compile.
template <class T>
class Handoff {
 public:
  Handoff() = default;
  __host__ __device__ explicit Handoff(T* p) : p_(p) {}
  __host__ __device__ Handoff operator+(int64_t i) const { return Handoff(p_ + i); }
  __device__ void put(int64_t i, T v) const {
    __hip_atomic_store(p_ + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ T get(int64_t i) const { return __hip_atomic_load(p_ + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

 private:
  T* p_ = nullptr;
};

// ------------------------------------------------------------ scoring / top-k
struct ScoreParams {
  const void* q;            // [B][T][Hq][d]
  const void* landmarks;    // [B][Hkv][max_blocks][d]
  const int32_t* seq_lens;
  float* scores;            // [B][T][Hkv][score_cols]
  int score_cols;           // max_blocks (standalone) or max candidates (fused)
  int B, T, Hq, Hkv, G, D, blk, max_blocks, window;
  int q_f32, lm_f32;        // 1 when q / landmarks are fp32, else bf16
  int rows_per_chunk;
  int fused_select;         // 1: the top-k runs in the scoring launch
  int single_chunk;         // fused: one workgroup per (b, g) scores into LDS and selects
  // fused selection outputs
  const int32_t* k_per_seq;
  int32_t* indices;         // [B][T][Hkv][k_max]
  int32_t* n_sel;           // [B][T][Hkv]
  float* overlap;           // [B][Hkv] or null
  int k_max;
  unsigned* counters;       // [B][Hkv], zero between calls
  const int32_t* block_table;  // when set, the selection also writes
  int32_t* phys;               // phys[b][t][g][m] = block_table[b][indices[b][t][g][m]]
  // fused, several chunks, two_level: each chunk's own top-k as (key, id)
  // rows, [B][T][Hkv][chunks][2][k_max] (cand_stride = chunks * 2 * k_max);
  // otherwise the chunks publish every score to `scores`
  int two_level;
  Handoff<int32_t> cand;
  int cand_stride;
  int cand_ids_lds;         // 1: the last chunk stages the candidates' ids in LDS (when they fit)
  // 1: the chunks publish their candidates and stop there; the attention
  // launch makes the final selection (split step).  Rows [B][T][Hkv][3]
  // [cand_cols] (cand_stride = 3 * cand_cols) of keys, ids and physical blocks
  // (token 0's only), dense in chunk order: chunk c's m-th candidate sits at
  // c * min(k', rows per chunk) + m, k' the pair's selection size.
  int cand_only;
  int cand_cols;
};

struct TopkParams {
  const float* scores;      // [B][T][Hkv][max_blocks]
  const int32_t* seq_lens;
  const int32_t* k_per_seq;
  int32_t* indices;
  int32_t* n_sel;
  float* overlap;
  int B, T, Hkv, blk, max_blocks, window, k_max;
};

// ------------------------------------------------------------------ attention
struct AttnParams {
  int kv;                   // KvKind of K/V
  const void* q;            // [B][T][Hq][d]; token 0 attended (both when co-batched)
  int B, T, Hq, Hkv, G, D, blk, window, max_blocks, k_max;
  float qk_scale;           // log2(e) / sqrt(d)
  // sparse part
  int sparse_kind;          // SKV_SRC_PAGED or SKV_SRC_STAGED
  const void* sk;
  const void* sv;
  const float* sks;
  const float* svs;
  const int32_t* block_table;
  int64_t stride_block, stride_head;  // pool element strides
  const int32_t* indices;   // [B][T][Hkv][k_max] (token 0 rows used)
  const int32_t* phys;      // same layout: physical block of each index, or null
  const int32_t* n_sel;     // [B][T][Hkv]
  // window part
  int window_kind;          // SKV_SRC_PAGED or SKV_SRC_WINDOW
  const void* wk;
  const void* wv;
  const float* wks;
  const float* wvs;
  const int32_t* window_table;  // block table for a PAGED window
  const int32_t* seq_lens;
  // split-K layout: workgroup s of (b, g) owns items [s*n, (s+1)*n) of the
  // concatenated list (sparse slices, then window slices), n = ceil(items of
  // (b, g) / n_splits) <= items_per_split
  int n_splits, items_per_split;
  Handoff<float> partials;  // [B][Hkv][n_splits][tokens * G][d + 2]
  unsigned* counters;       // [B][Hkv]
  float* out;               // [B][Hq][d]; co-batched [B][2][Hq][d]
  float* lse;               // [B][Hq] or null; co-batched [B][2][Hq]
  int longest_first;        // single-launch step: workgroup row r takes the sequence of
                            // length rank r (descending), so long pairs start first
  int window_only;          // hybrid step: the sparse part is left to the host
};

// --------------------------------------------------------------------- gather
struct GatherParams {
  const void* k_pool;
  const void* v_pool;
  const float* k_scales;
  const float* v_scales;
  const int32_t* block_table;
  const int32_t* indices;
  const int32_t* n_sel;
  void* k_stage;
  void* v_stage;
  float* k_stage_scales;
  float* v_stage_scales;
  int B, T, Hkv, max_blocks, k_max;
  int64_t stride_block, stride_head;  // elements
  int64_t chunk_bytes;      // blk * d * element size
  int elem_bytes;
  int has_scales;
  int token;                // the selection gathered: token `token` of indices / n_sel
  // speculative correction (null spec_indices: a plain gather)
  const int32_t* spec_indices;
  const int32_t* spec_n_sel;
  int spec_token;
  const void* spec_k_stage;
  const void* spec_v_stage;
  const float* spec_k_scales;
  const float* spec_v_scales;
  int32_t* misses;          // [B][Hkv] or null
};

// Launch shapes decided on the host; the workspace layout depends on them.
struct Plan {
  int max_cand;             // upper bound of candidates per sequence
  int rows_per_chunk, score_chunks;
  int score_two_level;      // several chunks: select per chunk, then over the chunks' candidates
  int items_per_split, n_splits;   // attention split-K
  int cob_items_per_split, cob_n_splits;   // co-batched two-token attention (T = 2)
  // single-launch step: one workgroup per (sequence, KV head) scores,
  // selects and attends (fused_step = 1 when the shape has that kernel and
  // there are enough pairs to fill the chip)
  int fused_step;
  size_t step_lds;          // dynamic LDS bytes of the step kernel (scoring region)
  // split step (device pools, few pairs, two-level selection): the scoring
  // launch publishes the chunks' candidates and the attention launch selects
  int split_step;
  int cand_cols;            // split step: chunk candidates per token (chunks x min(k_max, rows))
  size_t split_lds;         // its dynamic LDS bytes
  // scoring with the fused selection (two-launch, host-pool, hybrid and layer
  // steps): static plus dynamic LDS of its workgroups, and whether that fits
  size_t select_lds;
  int select_fits;
  size_t off_score_counters, off_attn_counters, off_scores, off_partials, off_phys;
  size_t off_hybrid;        // hybrid step: the window part's o [B][Hq][d] and lse [B][Hq]
  size_t total_bytes;
};

Plan make_plan(const skv_problem& pr);

// Host-side checks of a device-pool decode step (problem, step pointers, the
// selection's LDS); fills *pl.  Issues no HIP call.
skv_status check_device_step(const skv_problem* pr, const skv_step_inputs* in, const skv_step_outputs* out,
                             Plan* pl);
// Enqueue a checked device-pool decode step on workspace ws (pl.total_bytes).
// With clear_bytes > 0, a fill kernel first zeroes ws[0, clear_bytes); every
// remaining argument check runs before it.  only >= 0 (two-launch plans):
// enqueue launch `only` alone.
skv_status enqueue_device_step(const skv_problem& p, const Plan& pl, const skv_step_inputs& in,
                               const skv_step_outputs& out, char* ws, hipStream_t s, size_t clear_bytes,
                               int only = -1);

hipError_t launch_score(const ScoreParams& p, int chunks, hipStream_t s);
hipError_t launch_topk(const TopkParams& p, hipStream_t s);
hipError_t launch_attend(const AttnParams& p, hipStream_t s);
// Co-batched attention of both query tokens (T = 2, paged sparse source).
hipError_t launch_attend_cobatched(const AttnParams& p, hipStream_t s);
// Union blocks one co-batched split can cover: its items per split stay at
// most (this - 1) * items per block.
constexpr int kCobatchMaxSplitBlocks = 130;
hipError_t launch_step(const ScoreParams& s, const AttnParams& a, size_t lds, hipStream_t st);
// Whether a step kernel is built for this shape (device pool, d = 128, bf16
// queries and landmarks, bf16 or fp8 K/V, blocks of 32 or 64 tokens).
bool step_kernel_available(const skv_problem& p);
// Static LDS bytes of the step kernel for the problem's K/V type and block size.
size_t step_static_lds_bytes(const skv_problem& p);
// Waves of a single-launch step workgroup, and the items (32-token slices)
// it can hold: each wave keeps one item descriptor per lane.
#ifndef SKV_PAIR_WAVES
#define SKV_PAIR_WAVES 8
#endif
constexpr int kStepWaves = SKV_PAIR_WAVES;
constexpr int kStepMaxItems = kStepWaves * 64;
// Whether an nw-wave attention workgroup can hold its items as attend_items
// deals them: up to n_early early items over early_waves waves and up to
// n_late late items over all nw waves, one descriptor per lane, so at most 64
// items per wave.
constexpr bool wave_items_fit(int n_early, int early_waves, int n_late, int nw) {
  return (n_early + early_waves - 1) / early_waves + (n_late + nw - 1) / nw <= 64;
}
// Split step (few pairs): the scoring launch's chunks publish their own
// candidates, and the second launch (grid n_splits x Hkv x B, 8 waves) makes
// the final selection in every split and attends the split's share.
hipError_t launch_split_step(const ScoreParams& s, const AttnParams& a, size_t lds, hipStream_t st);
// Whether the split step is built for this shape and fits one workgroup's
// LDS with n_splits splits and cand_cols chunk candidates per token; sets
// *lds to its dynamic LDS bytes.
bool split_step_fits(const skv_problem& p, int n_splits, int cand_cols, size_t* lds);
// The split step's key region (words): T rows of cand_cols keys, and at
// least the overlap's bitmap of max_blocks bits.
__host__ __device__ inline int split_step_key_words(int T, int cand_cols, int max_blocks) {
  const int k = T * cand_cols, bits = (max_blocks + 31) / 32;
  return k > bits ? k : bits;
}
__host__ __device__ inline size_t split_step_lds_bytes(int T, int cand_cols, int k_max, int max_blocks) {
  return (size_t)4 * (split_step_key_words(T, cand_cols, max_blocks) + (size_t)T * cand_cols + cand_cols +
                      2 * (size_t)k_max + 2 * 256);
}
// LDS of one compute unit on gfx950, the most one workgroup may use.
constexpr size_t kLdsPerCu = 160 * 1024;
hipError_t launch_gather(const GatherParams& p, hipStream_t s);
// out = log-sum-exp fusion of (o_a, lse_a) (may be null: no part) and (o_b, lse_b), per row of D.
hipError_t launch_lse_merge(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                            float* out, float* lse, int rows, int D, hipStream_t s);
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);
// Streaming read of `bytes` (a multiple of 16) with one 512-thread workgroup
// per 32 KiB, at most 32768 and at most sink_words workgroups;
// sink[workgroup] is written only in the improbable case noted at the kernel.
hipError_t launch_stream_read(const void* ptr, size_t bytes, uint32_t* sink, int sink_words, hipStream_t s);

// LDS bytes of a scoring workgroup: qbar [T][d] floats, keys [T][score_cols]
// (fused selection only), the selected ids [2][k_max], two 256-bin top-byte
// key histograms and, for the single-launch step, the physical blocks of
// the candidates [score_cols].
// Layout: group-summed queries [T][D] fp32, keys [T][score_cols], selected
// ids [2][k_max], top-byte histograms [2][256]; then the step kernel's
// block-table row [score_cols] (table) or, for a fused selection over several
// chunks, the candidates' ids [T][score_cols] (cand_ids).
__host__ __device__ inline size_t score_lds_bytes(int T, int D, int score_cols, int k_max, bool fused,
                                                  bool table = false, bool cand_ids = false) {
  size_t b = (size_t)T * D * 4;
  if (fused) b += (size_t)T * score_cols * 4 + (size_t)2 * k_max * 4 + (size_t)2 * 256 * 4;
  if (table) b += (size_t)score_cols * 4;
  if (cand_ids) b += (size_t)T * score_cols * 4;
  return b;
}

// LDS of one workgroup (bytes), and an allowance for the score kernel's
// static LDS (selection state) next to its dynamic region.
constexpr size_t kLdsPerWorkgroup = 160 * 1024;
constexpr size_t kScoreStaticLds = 8 * 1024;

// LDS bytes the score kernel needs for a fused selection over max_cand keys.
size_t topk_lds_bytes(int max_cand);
// Static LDS of the 512-thread scoring / selection kernels (selection state
// and a flag), next to their dynamic region.
size_t select_static_lds_bytes();

}  // namespace skv
