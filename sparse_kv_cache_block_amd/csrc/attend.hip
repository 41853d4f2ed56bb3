// attend.hip -- stand-alone split-K decode attention kernel for gfx950:
// grid (split, KV head, sequence), 8-wave workgroups, each owning one range of
// the concatenated sparse + window item list of its (sequence, KV head).  The
// attention arithmetic lives in attend_dev.h.
#include "attend_dev.h"

namespace skv {

constexpr int kAttnWaves = 8;                 // waves per attention workgroup
constexpr int kAttnThreads = kAttnWaves * kWave;

template <int KV, int D, int BLK>
__global__ __launch_bounds__(kAttnThreads) void attend_kernel(AttnParams p) {
  using C = AttnCfg<KV, D, BLK>;
  __shared__ __attribute__((aligned(16))) char smem[attn_lds_bytes<KV, D, BLK>(kAttnWaves)];
  __shared__ int s_last;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = p.seq_lens[b];
  const int ws = L - p.window > 0 ? L - p.window : 0;
  const int nsel = p.n_sel[(int64_t)b * p.T * p.Hkv + g];
  const int total = (nsel + window_blocks(p, L, ws)) * C::SUB;
  const int first = split * p.items_per_split;
  const int count = max(0, min(p.items_per_split, total - first));
  attend_items<KV, D, BLK, kAttnWaves>(
      p, smem, b, g, first, count, [&](int item) { return describe<KV, D, BLK>(p, b, g, item, nsel, ws); },
      [](int) { return ItemDesc{0, 0, 0}; }, [](int) { return true; },
      [](auto&& issue_first) { issue_first(); }, [] {});
  attend_finish<KV, D, BLK, kAttnWaves>(p, smem, b, g, split, p.n_splits, &s_last, nullptr);
}

template <int KV, int D>
static hipError_t launch_blk(const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (p.blk) {
    case 16: hipLaunchKernelGGL((attend_kernel<KV, D, 16>), grid, dim3(kAttnThreads), 0, s, p); break;
    case 32: hipLaunchKernelGGL((attend_kernel<KV, D, 32>), grid, dim3(kAttnThreads), 0, s, p); break;
    case 64: hipLaunchKernelGGL((attend_kernel<KV, D, 64>), grid, dim3(kAttnThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KV>
static hipError_t launch_d(const AttnParams& p, dim3 grid, hipStream_t s) {
  return p.D == 128 ? launch_blk<KV, 128>(p, grid, s) : launch_blk<KV, 64>(p, grid, s);
}

hipError_t launch_attend(const AttnParams& p, hipStream_t s) {
  const dim3 grid(p.n_splits, p.Hkv, p.B);
  switch (p.kv) {
    case KV_F32: return launch_d<KV_F32>(p, grid, s);
    case KV_BF16: return launch_d<KV_BF16>(p, grid, s);
    case KV_FP8: return launch_d<KV_FP8>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace skv
