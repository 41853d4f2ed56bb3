// attend.hip -- stand-alone split-K decode attention kernels for gfx950:
// grid (split, KV head, sequence), 8-wave workgroups, each owning one equal
// range of the concatenated sparse + window item list of its (sequence, KV
// head).  One kernel attends the real token; the co-batched one attends both
// query tokens over the union of their selections.  The attention arithmetic
// lives in attend_dev.h.
#include "attend_dev.h"
#include "select_dev.h"

namespace skv {

constexpr int kAttnWaves = 8;                 // waves per attention workgroup
constexpr int kAttnThreads = kAttnWaves * kWave;

// WROW: fp8 window buffers with one scale per row (host pools).
template <int KV, int D, int BLK, bool WROW = false>
__global__ __launch_bounds__(kAttnThreads) void attend_kernel(AttnParams p) {
  using C = AttnCfg<KV, D, BLK>;
  __shared__ __attribute__((aligned(16))) char smem[attn_lds_bytes<KV, D, BLK>(kAttnWaves)];
  __shared__ int s_last;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = p.seq_lens[b];
  const int ws = L - p.window > 0 ? L - p.window : 0;
  const int nsel = p.window_only ? 0 : p.n_sel[(int64_t)b * p.T * p.Hkv + g];
  const int total = (nsel + window_blocks(p, L, ws)) * C::SUB;
  // the pair's items in equal contiguous ranges (at most items_per_split each)
  const int ips = (total + p.n_splits - 1) / p.n_splits;
  const int first = split * ips;
  const int count = max(0, min(ips, total - first));
  attend_items<KV, D, BLK, kAttnWaves, 1, true, kLateStrided, WROW>(
      p, smem, b, g, first, count, count, 0,
      [&](int item) { return describe<KV, D, BLK>(p, b, g, item, nsel, ws); },
      [](int) { return ItemDesc{0, 0, 0}; }, [] {}, [](auto&& issue_first) { issue_first(); }, [] {});
  attend_finish<KV, D, BLK, kAttnWaves>(p, smem, b, g, split, p.n_splits, &s_last);
}

// First index of the ascending a[0..n) holding a value >= x.
__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Union of two ascending selections s0[0..n0) and s1[0..n1).  A block x has
// rank #{s0 < x} + #{s1 < x} - #{blocks of both < x} in the ascending union.
// Once the union's size nu is known, r0 = first_rank(nu) names the first rank
// this workgroup needs; the blocks with rank in [r0, r0 + nr) go to
// tab[rank - r0] as (block id, tokens that did not select it: bit 0 token 0,
// bit 1 token 1).  When both rows fit in `stage` (stage_ints ints of LDS, free
// during the call) they are copied there first, so the binary searches run in
// LDS rather than as chains of dependent global loads.  Every thread of the
// workgroup calls it; returns nu.
template <int NT, class FirstRankFn>
__device__ int selection_union(const int32_t* s0, int n0, const int32_t* s1, int n1, FirstRankFn first_rank,
                               int nr, int2* tab, uint32_t* scan_w, int32_t* stage, int stage_ints) {
  auto ranks = [&](const int32_t* a0, const int32_t* a1) {
    int call = 0;
    // blocks of both selections: token 0's blocks found in token 1's row
    uint32_t both = 0;
    for (int c0 = 0; c0 < n0; c0 += NT) {
      const int i = c0 + (int)threadIdx.x;
      bool dup = false;
      if (i < n0) {
        const int c = lower_bound_i32(a1, n1, a0[i]);
        dup = c < n1 && a1[c] == a0[i];
      }
      uint32_t tot;
      (void)block_exclusive_scan<NT>(dup ? 1u : 0u, scan_w + (call++ & 1) * (NT / kWave), tot);
      both += tot;
    }
    const int nu = n0 + n1 - (int)both;
    const int r0 = first_rank(nu);
    for (int side = 0; side < 2; ++side) {
      const int32_t* x = side ? a1 : a0;
      const int32_t* y = side ? a0 : a1;
      const int nx = side ? n1 : n0, ny = side ? n0 : n1;
      uint32_t before = 0;  // blocks of both among the earlier chunks of x
      for (int c0 = 0; c0 < nx; c0 += NT) {
        const int i = c0 + (int)threadIdx.x;
        int v = 0, c = 0;
        bool dup = false;
        if (i < nx) {
          v = x[i];
          c = lower_bound_i32(y, ny, v);
          dup = c < ny && y[c] == v;
        }
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan<NT>(dup ? 1u : 0u, scan_w + (call++ & 1) * (NT / kWave), tot);
        // a block of both selections is placed once, from token 0's side
        if (i < nx && !(side == 1 && dup)) {
          const int rank = i + c - (int)(before + ex);
          if (rank >= r0 && rank < r0 + nr) tab[rank - r0] = make_int2(v, side == 0 ? (dup ? 0 : 2) : 1);
        }
        before += tot;
      }
    }
    __syncthreads();
    return nu;
  };
  if (n0 + n1 <= stage_ints) {
    for (int i = threadIdx.x; i < n0 + n1; i += NT) stage[i] = i < n0 ? s0[i] : s1[i - n0];
    __syncthreads();
    return ranks(stage, stage + n0);
  }
  return ranks(s0, s1);
}

// Co-batched attention of the two query tokens of (b, g): items are the
// union blocks (split into slices) followed by the window blocks, dealt to
// the pair's n_splits workgroups in equal contiguous ranges once the union's
// size is known; each workgroup rebuilds the part of the union its range
// covers.
template <int KV, int D, int BLK>
__global__ __launch_bounds__(kAttnThreads) void attend_cobatched_kernel(AttnParams p) {
  using C = AttnCfg<KV, D, BLK>;
  __shared__ __attribute__((aligned(16))) char smem[attn_lds_bytes<KV, D, BLK>(kAttnWaves)];
  __shared__ int2 tab[kCobatchMaxSplitBlocks];
  __shared__ uint32_t scan_w[2][kAttnWaves];
  __shared__ int s_last;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = p.seq_lens[b];
  const int ws = L - p.window > 0 ? L - p.window : 0;
  const int nwin = window_blocks(p, L, ws);
  const int64_t row0 = ((int64_t)b * 2) * p.Hkv + g, row1 = row0 + p.Hkv;
  int first = 0, count = 0;
  const int nu = selection_union<kAttnThreads>(
      p.indices + row0 * p.k_max, p.n_sel[row0], p.indices + row1 * p.k_max, p.n_sel[row1],
      [&](int n_union) {
        // equal ranges; at most items_per_split (the plan's bound for a union of
        // every selected block), which the union table is sized for
        const int total = (n_union + nwin) * C::SUB;
        const int ips = (total + p.n_splits - 1) / p.n_splits;
        first = split * ips;
        count = max(0, min(ips, total - first));
        return first / C::SUB;
      },
      kCobatchMaxSplitBlocks, tab, &scan_w[0][0], reinterpret_cast<int32_t*>(smem), (int)(sizeof(smem) / 4));
  const int r0 = first / C::SUB;
  attend_items<KV, D, BLK, kAttnWaves, 2>(
      p, smem, b, g, first, count, count, 0,
      [&](int item) {
        const int bi = item / C::SUB, sub = item % C::SUB;
        if (bi < nu) {
          const int2 e = tab[bi - r0];
          ItemDesc d = describe_sparse<KV, D, BLK>(p, b, g, 0, e.x, -1, sub);
          d.sub |= e.y << 8;
          return d;
        }
        return describe_window<KV, D, BLK>(p, b, g, bi - nu, sub, ws);
      },
      [](int) { return ItemDesc{0, 0, 0}; }, [] {}, [](auto&& issue_first) { issue_first(); }, [] {});
  attend_finish<KV, D, BLK, kAttnWaves, 2>(p, smem, b, g, split, p.n_splits, &s_last);
}

template <int KV, int D>
static hipError_t launch_blk(const AttnParams& p, dim3 grid, hipStream_t s, bool cob) {
  // fp8 window buffers carry one scale per row
  const bool wrow = KV == KV_FP8 && p.window > 0 && p.window_kind == SKV_SRC_WINDOW;
  switch (p.blk) {
#define SKV_ATTEND_CASE(BLK)                                                                          \
  case BLK:                                                                                           \
    if (cob) hipLaunchKernelGGL((attend_cobatched_kernel<KV, D, BLK>), grid, dim3(kAttnThreads), 0, s, p); \
    else if (wrow) hipLaunchKernelGGL((attend_kernel<KV, D, BLK, KV == KV_FP8>), grid, dim3(kAttnThreads), 0, s, p); \
    else hipLaunchKernelGGL((attend_kernel<KV, D, BLK>), grid, dim3(kAttnThreads), 0, s, p);           \
    break;
    SKV_ATTEND_CASE(16)
    SKV_ATTEND_CASE(32)
    SKV_ATTEND_CASE(64)
#undef SKV_ATTEND_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KV>
static hipError_t launch_d(const AttnParams& p, dim3 grid, hipStream_t s, bool cob) {
  return p.D == 128 ? launch_blk<KV, 128>(p, grid, s, cob) : launch_blk<KV, 64>(p, grid, s, cob);
}

static hipError_t launch_kind(const AttnParams& p, hipStream_t s, bool cob) {
  const dim3 grid(p.n_splits, p.Hkv, p.B);
  switch (p.kv) {
    case KV_F32: return launch_d<KV_F32>(p, grid, s, cob);
    case KV_BF16: return launch_d<KV_BF16>(p, grid, s, cob);
    case KV_FP8: return launch_d<KV_FP8>(p, grid, s, cob);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attend(const AttnParams& p, hipStream_t s) { return launch_kind(p, s, false); }

hipError_t launch_attend_cobatched(const AttnParams& p, hipStream_t s) { return launch_kind(p, s, true); }

}  // namespace skv
