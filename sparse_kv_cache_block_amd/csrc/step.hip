// step.hip -- the whole decode step of one (sequence, KV head) in one
// workgroup, for gfx950: landmark scoring into LDS, the per-head top-k, and
// the attention over the recent window and the selected blocks, fused by
// log-sum-exp, in a single launch with one workgroup of kStepWaves (8)
// waves per pair.
//
// The window part does not depend on the selection (Beyond abstract: the
// recent window is attended densely, the older entries sparsely per head).
// Once the scores are in LDS, wave t alone runs the radix select of query
// token t (no workgroup barrier) while the other waves attend the window
// slices, whose loads they issued as soon as their scoring was done.  Wave 0
// then raises an LDS flag; a wave that reaches its first selected block
// waits for that flag.  The window descriptors, the attention's query
// operand and the block-table row of the candidates are loaded before the
// scoring, so the selected blocks' physical ids come from LDS.
//
// The selection stays in LDS until the attention is done (global stores
// issued during the select would queue behind the window loads), and the
// selected ids, counts and the dual-query overlap are written at the end.
//
// The arithmetic of every phase is that of the stand-alone kernels
// (select_dev.h, attend_dev.h).  One workgroup owns a pair, so there is a
// single split and the output is written without a merge.
#include "attend_dev.h"
#include "select_dev.h"

namespace skv {

constexpr int kPairWaves = kStepWaves;
constexpr int kPairThreads = kPairWaves * kWave;
#ifndef SKV_PAIR_SCORE_UR
#define SKV_PAIR_SCORE_UR 4
#endif
constexpr int kTableRegs = 2;   // block-table entries per thread held through the scoring
// Selected blocks go to the waves in turn, so a pair's result is the same on
// every run.  Handing them out from an LDS counter instead (kLateShared)
// measured 0.5 us faster at llama32k but makes the fp32 sums depend on timing.
#ifndef SKV_STEP_LATE
#define SKV_STEP_LATE kLateStrided
#endif

// The sequence whose length has rank r in descending order (ties to the lower
// index).  Every wave computes it (scalar broadcasts of 64 lengths at a time),
// so no barrier is needed.
__device__ __forceinline__ int sequence_of_rank(const int32_t* seq_lens, int B, int r) {
  const int lane = lane_id();
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int i = c0 + lane;
    const int Li = i < B ? seq_lens[i] : -1;
    int rank = 0;
    for (int j0 = 0; j0 < B; j0 += kWave) {
      const int Lj_lane = j0 + lane < B ? seq_lens[j0 + lane] : -1;
      const int nj = min(kWave, B - j0);
      for (int t = 0; t < nj; ++t) {
        const int Lj = __builtin_amdgcn_readlane(Lj_lane, t);
        rank += (Lj > Li || (Lj == Li && j0 + t < i)) ? 1 : 0;
      }
    }
    const uint64_t hit = __ballot(i < B && rank == r);
    if (hit) return c0 + (int)__builtin_ctzll(hit);
  }
  return r;
}

template <int KV, int BLK>
__global__ __launch_bounds__(kPairThreads) void pair_step_kernel(ScoreParams s, AttnParams a) {
  constexpr int D = 128;
  using C = AttnCfg<KV, D, BLK>;
  __shared__ __attribute__((aligned(16))) char smem[attn_lds_bytes<KV, D, BLK>(kPairWaves)];
  extern __shared__ __attribute__((aligned(16))) uint32_t score_smem[];
  __shared__ TopkShared<kPairThreads> sh;
  __shared__ int s_flag;
  __shared__ int s_sel_ready;
  __shared__ int s_late_next;

  // Workgroups start in linear order and go to the XCDs in turn.  With more
  // pairs than compute units the grid is (KV head, rank): rows take the
  // sequences longest first, so the short pairs fill in at the end.  Otherwise
  // it is (sequence, KV head), so each XCD serves every KV head of a share of
  // the sequences rather than one KV head of every sequence (measured 0.4 us
  // faster at 256 pairs).
  const int g = a.longest_first ? (int)blockIdx.x : (int)blockIdx.y;
  const int b = a.longest_first ? sequence_of_rank(a.seq_lens, a.B, blockIdx.y) : (int)blockIdx.x;
  const int L = a.seq_lens[b];
  const int k = s.k_per_seq[b];
  // the query and the first landmark rows are requested before anything
  // waits for the sequence's length
  __builtin_amdgcn_sched_barrier(0);
  ScoreHead<SKV_PAIR_SCORE_UR> head;
  score_head<D, false, false, kPairThreads, SKV_PAIR_SCORE_UR>(s, 0, g, b, head);
  __builtin_amdgcn_sched_barrier(0);
  const int ws = L - a.window > 0 ? L - a.window : 0;
  const int nc = n_candidates(L, a.window, a.blk);
  // the selection returns clamp(min(k, candidates), 0, k_max) blocks
  int nsel = min(k, nc);
  nsel = max(0, min(nsel, a.k_max));
  const int nwin_items = window_blocks(a, L, ws) * C::SUB;
  const int count = nwin_items + nsel * C::SUB;
  const int T = s.T;
  const int w = wave_id(), lane = lane_id();
  // dynamic LDS: group-summed queries, keys [T][score_cols], selected ids
  // [2][k_max], top-byte key histograms [2][256], the candidates' physical
  // blocks [score_cols]
  uint32_t* keys = score_smem + T * D;
  int32_t* lds_idx = reinterpret_cast<int32_t*>(keys + T * s.score_cols);
  const uint32_t* hist0 = reinterpret_cast<const uint32_t*>(lds_idx + 2 * s.k_max);
  int32_t* lds_table = lds_idx + 2 * s.k_max + 2 * 256;
  if (threadIdx.x == 0) {
    s_sel_ready = 0;
    s_late_next = 0;
  }
  // the candidates' row of the block table: loaded into registers before the
  // scoring's loads, stored to LDS after them (no wait in between)
  const int32_t* table_row = a.block_table + (int64_t)b * a.max_blocks;
  int32_t trow[kTableRegs];
#pragma unroll
  for (int i = 0; i < kTableRegs; ++i) {
    const int j = (int)threadIdx.x + kPairThreads * i;
    trow[i] = table_row[j < nc ? j : 0];
  }

  attend_items<KV, D, BLK, kPairWaves, 1, false, SKV_STEP_LATE>(
      a, smem, b, g, 0, count, nwin_items, T,
      // window slices, early: taken by the waves that do not select
      [&](int item) { return describe_window<KV, D, BLK>(a, b, g, item / C::SUB, item % C::SUB, ws); },
      // selected blocks, late: ids from the selection, physical blocks from
      // the table row, both in LDS
      [&](int item) {
        const int it = item - nwin_items;
        const int m = it / C::SUB;
        const int j = lds_idx[m];
        return describe_paged<KV, D, BLK>(j, lds_table[j], it % C::SUB);
      },
      [&] {
        while (__hip_atomic_load(&s_sel_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
          __builtin_amdgcn_s_sleep(1);
      },
      [&](auto&& issue_first) {
        (void)score_rows<D, false, false, kPairThreads, SKV_PAIR_SCORE_UR, true>(s, 0, g, b, score_smem, &head);
#pragma unroll
        for (int i = 0; i < kTableRegs; ++i) {
          const int j = (int)threadIdx.x + kPairThreads * i;
          if (j < nc) lds_table[j] = trow[i];
        }
        for (int j = (int)threadIdx.x + kPairThreads * kTableRegs; j < nc; j += kPairThreads)
          lds_table[j] = table_row[j];
        lds_barrier();   // every wave's keys, key histograms and table entries are in LDS
        issue_first();   // the window slices' waves issue their first slice
      },
      [&] {
        // wave t selects token t's blocks alone while the other waves attend
        // the window; wave 0 then releases the waves waiting for its ids
        if (w < T) {
          (void)wave_select(keys + w * s.score_cols, nc, k, s.k_max, lds_idx + w * s.k_max, sh.hist[w],
                            hist0 + w * 256);
          if (w == 0 && lane == 0) __hip_atomic_store(&s_sel_ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      },
      &s_late_next);
  attend_finish<KV, D, BLK, kPairWaves>(a, smem, b, g, 0, 1, &s_flag);

  // ---- the selection's outputs: ids (-1 past the count), counts, overlap
  // (every wave has passed the combine barriers, so both tokens' ids are in LDS)
  const float overlap = T == 2 ? list_overlap<kPairThreads>(lds_idx, nsel, lds_idx + s.k_max, nsel, nc, keys, sh) : 1.0f;
  for (int i = threadIdx.x; i < T * s.k_max; i += kPairThreads) {
    const int t = i / s.k_max, m = i % s.k_max;
    s.indices[(((int64_t)b * T + t) * s.Hkv + g) * s.k_max + m] = lds_idx[i];
  }
  if (threadIdx.x < T) s.n_sel[((int64_t)b * T + threadIdx.x) * s.Hkv + g] = nsel;
  if (T == 2 && s.overlap && threadIdx.x == 0) s.overlap[b * s.Hkv + g] = overlap;
}

static_assert(kStepMaxItems == kPairWaves * kWave, "one item descriptor per lane");

bool step_kernel_available(const skv_problem& p) {
  return p.pool_location == SKV_POOL_DEVICE && p.head_dim == 128 && p.q_dtype == SKV_BF16 &&
         p.landmark_dtype == SKV_BF16 && (p.kv_dtype == SKV_BF16 || p.kv_dtype == SKV_FP8_E4M3FN) &&
         (p.block_size == 32 || p.block_size == 64);
}

size_t step_static_lds_bytes(const skv_problem& p) {
  const bool fp8 = p.kv_dtype == SKV_FP8_E4M3FN;
  const size_t attn = fp8 ? (p.block_size == 32 ? attn_lds_bytes<KV_FP8, 128, 32>(kPairWaves)
                                                : attn_lds_bytes<KV_FP8, 128, 64>(kPairWaves))
                          : (p.block_size == 32 ? attn_lds_bytes<KV_BF16, 128, 32>(kPairWaves)
                                                : attn_lds_bytes<KV_BF16, 128, 64>(kPairWaves));
  return attn + sizeof(TopkShared<kPairThreads>) + 16;
}

hipError_t launch_step(const ScoreParams& s, const AttnParams& a, size_t lds, hipStream_t st) {
  const dim3 grid = a.longest_first ? dim3(a.Hkv, a.B) : dim3(a.B, a.Hkv);
  const dim3 block(kPairThreads);
  if (a.kv == KV_FP8) {
    if (a.blk == 32) hipLaunchKernelGGL((pair_step_kernel<KV_FP8, 32>), grid, block, lds, st, s, a);
    else hipLaunchKernelGGL((pair_step_kernel<KV_FP8, 64>), grid, block, lds, st, s, a);
  } else {
    if (a.blk == 32) hipLaunchKernelGGL((pair_step_kernel<KV_BF16, 32>), grid, block, lds, st, s, a);
    else hipLaunchKernelGGL((pair_step_kernel<KV_BF16, 64>), grid, block, lds, st, s, a);
  }
  return hipGetLastError();
}

}  // namespace skv
