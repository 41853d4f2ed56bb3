// split_step.hip -- the second launch of the decode step when there are too
// few (sequence, KV head) pairs to give each its own compute unit, for gfx950.
//
// The first launch scores each pair's landmarks in chunks over about 256
// workgroups; each chunk keeps its own top k' and publishes it as (key, id,
// physical block) rows, then exits (the kernel boundary is the hand-off).
// Here a pair has n_splits workgroups, and each of them
//   1. loads the pair's chunk candidates into LDS and makes the pair's final
//      selection over them: wave 0 alone finds where the selection cuts (the
//      radix passes of the single-launch step's select), then all waves emit
//      the chosen positions in ascending order, each a contiguous run placed
//      by two block scans.  Under the selection's total order -- score
//      descending, id ascending -- the pair's top k' lies among its chunks'
//      top k', so this is the selection over all candidates.  The loads of
//      this split's share of the recent window are in flight meanwhile; that
//      part needs no index (Beyond abstract: the window is attended densely,
//      the older entries sparsely per head);
//   2. attends its equal share of the selected blocks, whose ids and physical
//      blocks are in LDS, so no descriptor waits on a global load;
//   3. publishes its partial, and the last split of the pair to arrive merges
//      all of them by log-sum-exp.
// Every split computes the same selection; split 0 also selects the second
// query token's blocks (wave 1 finds its cut, half the waves emit each
// token's positions), and its waves 0 and 1 write the ids, counts and the two
// tokens' overlap (DualDecoder core claim: the speculative token's index is
// the prediction of the next step's) before they attend.  The arithmetic is that of the
// stand-alone kernels (select_dev.h, attend_dev.h).
#include "attend_dev.h"
#include "select_dev.h"

namespace skv {

constexpr int kSplitWaves = 8;
constexpr int kSplitThreads = kSplitWaves * kWave;
constexpr int kSplitCandRegs = 4;   // candidates per thread whose loads are issued before the window's

template <int KV, int BLK>
__global__ __launch_bounds__(kSplitThreads) void split_step_kernel(ScoreParams s, AttnParams a) {
  constexpr int D = 128;
  using C = AttnCfg<KV, D, BLK>;
  __shared__ __attribute__((aligned(16))) char smem[attn_lds_bytes<KV, D, BLK>(kSplitWaves)];
  extern __shared__ __attribute__((aligned(16))) uint32_t sel_smem[];
  __shared__ TopkShared<kSplitThreads> sh;
  __shared__ int s_flag;

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = a.seq_lens[b];
  const int k = s.k_per_seq[b];
  const int T = s.T;
  const bool writer = split == 0;                  // also selects token 1 and writes the selection
  const int TS = writer ? T : 1;                   // tokens this workgroup selects
  const int SC = s.score_cols;
  const Handoff<int32_t> cand = s.cand + ((int64_t)b * T * s.Hkv + g) * s.cand_stride;
  const int64_t cand_t = (int64_t)s.Hkv * s.cand_stride;
  const int w = wave_id(), lane = lane_id();
  const int ws = L - a.window > 0 ? L - a.window : 0;
  const int nc = n_candidates(L, a.window, a.blk);
  const int R = s.rows_per_chunk;
  const int nchunks = max(1, (nc + R - 1) / R);
  // the selection returns clamp(min(k, candidates), 0, k_max) blocks; a chunk
  // published min(that, its rows) candidates
  int kk = min(k, nc);
  kk = max(0, min(kk, s.k_max));
  const int m_full = min(kk, R);
  const int m_last = min(kk, nc - (nchunks - 1) * R);
  const int M = (nchunks - 1) * m_full + m_last;   // candidates per token, chunk after chunk

  // dynamic LDS (split_step_lds_bytes): keys [T][score_cols] (later the
  // overlap's bitmap), ids [T][score_cols], token 0's physical blocks
  // [score_cols], the selected positions [2][k_max], top-byte key histograms
  // [2][256]; score_cols holds every chunk's candidates of one token
  uint32_t* keys = sel_smem;
  int32_t* ids = reinterpret_cast<int32_t*>(keys + split_step_key_words(T, SC, s.max_blocks));
  int32_t* phys = ids + T * SC;
  int32_t* lds_idx = phys + SC;
  uint32_t* hist0 = reinterpret_cast<uint32_t*>(lds_idx + 2 * s.k_max);
  for (int i = threadIdx.x; i < 2 * 256; i += kSplitThreads) hist0[i] = 0u;

  // this split's equal shares of the window slices and of the selected slices
  const int nwin = window_blocks(a, L, ws) * C::SUB;
  const int nsp = kk * C::SUB;
  const int wpi = (nwin + a.n_splits - 1) / a.n_splits;
  const int spi = (nsp + a.n_splits - 1) / a.n_splits;
  const int win0 = split * wpi, my_win = max(0, min(wpi, nwin - win0));
  const int sp0 = split * spi, my_sp = max(0, min(spi, nsp - sp0));

  const int k_max = s.k_max;
  auto stash = [&](int t, int j, int32_t key, int32_t id, int32_t ph) {
    keys[t * SC + j] = (uint32_t)key;
    ids[t * SC + j] = id;
    if (t == 0) phys[j] = ph;
    atomicAdd(&hist0[t * 256 + ((uint32_t)key >> 24)], 1u);
  };
  // The selection's outputs, written by the selecting waves of split 0 as
  // soon as their lists exist: token t's ids in ascending order (-1 past the
  // count) and its count; after both lists, the overlap.
  int32_t* idx_out = s.indices + ((int64_t)b * T * s.Hkv + g) * k_max;
  auto write_ids = [&](int t) {
    for (int m = lane; m < k_max; m += kWave) {
      const int pos = lds_idx[t * k_max + m];
      idx_out[(int64_t)t * s.Hkv * k_max + m] = pos >= 0 ? ids[t * SC + pos] : -1;
    }
    if (lane == 0) s.n_sel[((int64_t)b * T + t) * s.Hkv + g] = kk;
  };

  attend_items<KV, D, BLK, kSplitWaves, 1, false, kLateStrided>(
      a, smem, b, g, 0, my_win + my_sp, my_win, TS,
      // window slices, early: taken by the waves that do not find a cut
      [&](int item) {
        const int it = win0 + item;
        return describe_window<KV, D, BLK>(a, b, g, it / C::SUB, it % C::SUB, ws);
      },
      // selected slices, late: positions from the selection, ids and physical
      // blocks from the candidates, all in LDS
      [&](int item) {
        const int it = sp0 + item - my_win;
        const int pos = lds_idx[it / C::SUB];
        return describe_paged<KV, D, BLK>(ids[pos], phys[pos], it % C::SUB);
      },
      [] {},   // the selection is in LDS before any wave takes an item (post)
      [&](auto&& issue_first) {
        // The candidates are stashed before the window slices' loads are
        // issued: their addresses need neither the sequence's length nor its
        // k (slots past the pair's count are read and dropped), and the
        // selection waits for them, not for the slices.
        int32_t kv[kSplitCandRegs], iv[kSplitCandRegs], pv[kSplitCandRegs];
#pragma unroll
        for (int u = 0; u < kSplitCandRegs; ++u) {
          const int i = (int)threadIdx.x + kSplitThreads * u;
          const int t = i / SC, j = i - t * SC;
          const Handoff<int32_t> cr = t < TS ? cand + t * cand_t + j : cand;
          kv[u] = cr.get(0);
          iv[u] = cr.get(SC);
          pv[u] = cr.get(2 * SC);
        }
        lds_barrier();   // the histograms are clear
#pragma unroll
        for (int u = 0; u < kSplitCandRegs; ++u) {
          const int i = (int)threadIdx.x + kSplitThreads * u;
          const int t = i / SC, j = i - t * SC;
          if (t < TS && j < M) stash(t, j, kv[u], iv[u], pv[u]);
        }
        for (int i = (int)threadIdx.x + kSplitThreads * kSplitCandRegs; i < TS * SC; i += kSplitThreads) {
          const int t = i / SC, j = i - t * SC;
          if (j >= M) continue;
          const Handoff<int32_t> cr = cand + t * cand_t + j;
          stash(t, j, cr.get(0), cr.get(SC), t == 0 ? cr.get(2 * SC) : 0);
        }
        issue_first();
        lds_barrier();   // every candidate and the key histograms are in LDS
      },
      [&] {
        // wave t finds where token t's selection cuts, alone (radix passes),
        // while the window slices' loads are in flight; then every wave
        // emits its run of the chosen positions
        if (w < TS) {
          const SelectCut cut = wave_threshold(keys + w * SC, M, k, k_max, sh.hist[w], hist0 + w * 256);
          if (lane == 0) sh.cut[w] = cut;
        }
        lds_barrier();   // the cuts are in LDS
        if (TS == 2)
          block_emit<kSplitThreads, 2>(keys, SC, M, sh.cut, k_max, lds_idx, sh.scan_w[0], sh.scan_w[1]);
        else
          block_emit<kSplitThreads, 1>(keys, SC, M, sh.cut, k_max, lds_idx, sh.scan_w[0], sh.scan_w[1]);
        lds_barrier();   // every token's chosen positions are in LDS
        if (!writer || w >= TS) return;
        write_ids(w);
        if (w != 1) return;
        // wave 1 (T = 2): |I_0 & I_1| / |I_0|, through a bitmap of token 1's
        // ids in the key region (the selection is done with the keys)
        uint32_t* bits = keys;
        const int words = (nc + 31) / 32;
        for (int i = lane; i < words; i += kWave) bits[i] = 0u;
        wave_lds_sync();
        for (int m = lane; m < kk; m += kWave) {
          const uint32_t x = (uint32_t)ids[SC + lds_idx[k_max + m]];
          atomicOr(&bits[x >> 5], 1u << (x & 31u));
        }
        wave_lds_sync();
        uint32_t hits = 0;
        for (int m0 = 0; m0 < kk; m0 += kWave) {
          bool hit = false;
          if (m0 + lane < kk) {
            const uint32_t x = (uint32_t)ids[lds_idx[m0 + lane]];
            hit = (bits[x >> 5] >> (x & 31u)) & 1u;
          }
          hits += (uint32_t)__builtin_popcountll(__ballot(hit));
        }
        if (s.overlap && lane == 0) s.overlap[b * s.Hkv + g] = kk > 0 ? (float)hits / (float)kk : 1.0f;
      });
  attend_finish<KV, D, BLK, kSplitWaves>(a, smem, b, g, split, a.n_splits, &s_flag);
}

bool split_step_fits(const skv_problem& p, int n_splits, int cand_cols, size_t* lds) {
  if (!step_kernel_available(p)) return false;
  const int blk = p.block_size;
  const int sub = blk / attn_item_tokens(p.kv_dtype == SKV_FP8_E4M3FN ? KV_FP8 : KV_BF16, blk, p.head_dim);
  const int nwb = p.window == 0 ? 0 : (p.window + blk - 1) / blk + 1;
  // a split's window slices go to the waves that do not find a cut (8 - T in
  // split 0), its selected slices to all of its waves
  const int win_per_split = (nwb * sub + n_splits - 1) / n_splits;
  const int sel_per_split = (p.k_max * sub + n_splits - 1) / n_splits;
  if (!wave_items_fit(win_per_split, kSplitWaves - p.n_q_tokens, sel_per_split, kSplitWaves)) return false;
  *lds = split_step_lds_bytes(p.n_q_tokens, cand_cols, p.k_max, p.max_blocks_per_seq);
  const size_t stat = (p.kv_dtype == SKV_FP8_E4M3FN
                           ? (blk == 32 ? attn_lds_bytes<KV_FP8, 128, 32>(kSplitWaves)
                                        : attn_lds_bytes<KV_FP8, 128, 64>(kSplitWaves))
                           : (blk == 32 ? attn_lds_bytes<KV_BF16, 128, 32>(kSplitWaves)
                                        : attn_lds_bytes<KV_BF16, 128, 64>(kSplitWaves))) +
                      sizeof(TopkShared<kSplitThreads>) + 16;
  return stat + *lds <= kLdsPerCu;
}

hipError_t launch_split_step(const ScoreParams& s, const AttnParams& a, size_t lds, hipStream_t st) {
  const dim3 grid(a.n_splits, a.Hkv, a.B);
  const dim3 block(kSplitThreads);
  if (a.kv == KV_FP8) {
    if (a.blk == 32) hipLaunchKernelGGL((split_step_kernel<KV_FP8, 32>), grid, block, lds, st, s, a);
    else hipLaunchKernelGGL((split_step_kernel<KV_FP8, 64>), grid, block, lds, st, s, a);
  } else {
    if (a.blk == 32) hipLaunchKernelGGL((split_step_kernel<KV_BF16, 32>), grid, block, lds, st, s, a);
    else hipLaunchKernelGGL((split_step_kernel<KV_BF16, 64>), grid, block, lds, st, s, a);
  }
  return hipGetLastError();
}

}  // namespace skv
