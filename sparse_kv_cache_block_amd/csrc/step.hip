// step.hip -- the whole decode step of one (sequence, KV head) in one
// workgroup, for gfx950: landmark scoring into LDS, the per-head top-k, and
// the attention over the recent window and the selected blocks, fused by
// log-sum-exp, in a single launch with one 8-wave workgroup per pair.
//
// The window part does not depend on the selection (Beyond abstract: the
// recent window is attended densely, the older entries sparsely per head), so
// the workgroup's item list puts the window slices first and each wave issues
// the loads of its first window slice as soon as its scoring is done: the
// radix select runs in LDS while those loads are in flight, and its barriers
// wait for LDS traffic only.  The window descriptors and the attention's query
// operand are loaded before the scoring; the sparse descriptors (block ids from
// the selection in LDS, physical ids from the block table) after it, while the
// waves work through their window slices.
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

constexpr int kPairWaves = 8;
constexpr int kPairThreads = kPairWaves * kWave;
#ifndef SKV_PAIR_SCORE_UR
#define SKV_PAIR_SCORE_UR 4
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

  // workgroups start in row order: with more pairs than compute units, rows
  // take the sequences longest first so the short pairs fill in at the end
  const int g = blockIdx.x;
  const int b = a.longest_first ? sequence_of_rank(a.seq_lens, a.B, blockIdx.y) : (int)blockIdx.y;
  const int L = a.seq_lens[b];
  const int ws = L - a.window > 0 ? L - a.window : 0;
  const int nc = n_candidates(L, a.window, a.blk);
  const int k = s.k_per_seq[b];
  // the selection returns clamp(min(k, candidates), 0, k_max) blocks
  int nsel = min(k, nc);
  nsel = max(0, min(nsel, a.k_max));
  const int nwin_items = window_blocks(a, L, ws) * C::SUB;
  const int count = nwin_items + nsel * C::SUB;
  uint32_t* keys = score_smem + s.T * D;
  int32_t* lds_idx = reinterpret_cast<int32_t*>(keys + s.T * s.score_cols);
  float overlap = 1.0f;

  attend_items<KV, D, BLK, kPairWaves>(
      a, smem, b, g, 0, count,
      // window slices first (clamped for lanes past them) ...
      [&](int item) {
        if (nwin_items == 0) return ItemDesc{0, 0, 0};
        const int it = min(item, nwin_items - 1);
        return describe_window<KV, D, BLK>(a, b, g, it / C::SUB, it % C::SUB, ws);
      },
      // ... then the selected blocks, described once the selection is in LDS
      [&](int item) {
        if (nsel == 0) return ItemDesc{0, 0, 0};
        const int it = max(item - nwin_items, 0);
        const int m = min(it / C::SUB, nsel - 1);
        return describe_sparse<KV, D, BLK>(a, b, g, m, lds_idx[m], -1, it % C::SUB);
      },
      [&](int item) { return item < nwin_items; },
      [&](auto&& issue_first) {
        (void)score_rows<D, false, false, kPairThreads, SKV_PAIR_SCORE_UR, true>(s, 0, g, b, score_smem);
        issue_first();
      },
      [&] {
        // the selection stays in LDS here: global stores would queue behind
        // the window loads just issued
        lds_barrier();
        overlap = select_rows<kPairThreads, false>(nullptr, 0, false, keys, s.score_cols, nc, s.T, k, s.k_max,
                                                   nullptr, 0, nullptr, 0, nullptr, lds_idx, sh,
                                                   reinterpret_cast<const uint32_t*>(lds_idx + 2 * s.k_max));
      });
  attend_finish<KV, D, BLK, kPairWaves>(a, smem, b, g, 0, 1, &s_flag, nullptr);

  // ---- the selection's outputs: ids (-1 past the count), counts, overlap
  const int T = s.T;
  for (int i = threadIdx.x; i < T * s.k_max; i += kPairThreads) {
    const int t = i / s.k_max, m = i % s.k_max;
    s.indices[(((int64_t)b * T + t) * s.Hkv + g) * s.k_max + m] = lds_idx[i];
  }
  if (threadIdx.x < T) s.n_sel[((int64_t)b * T + threadIdx.x) * s.Hkv + g] = nsel;
  if (T == 2 && s.overlap && threadIdx.x == 0) s.overlap[b * s.Hkv + g] = overlap;
}

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
  const dim3 grid(a.Hkv, a.B);
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
