// score_topk.hip -- stand-alone landmark scoring and per-KV-head top-k
// selection kernels for gfx950 (512-thread workgroups).  The scoring and
// selection arithmetic lives in select_dev.h; this file holds the kernels of
// the separate entry points and of the two-launch decode step.
//
// In the fused decode step the scoring grid is split over workgroups per
// (sequence, KV head); the last workgroup to finish (device-scope atomic
// counter, reset by that workgroup) runs the selection over the fp32 scores
// its siblings published to the workspace with device-scope stores.
#include "select_dev.h"

namespace skv {

constexpr int kSelThreads = 512;             // threads of the scoring / selection workgroups
#ifndef SKV_SCORE_UR
#define SKV_SCORE_UR 4
#endif

// Grid (chunk, g, b); see score_task for the modes.
template <int D, bool LM_F32, bool Q_F32>
__global__ __launch_bounds__(kSelThreads) void score_kernel(ScoreParams p) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  __shared__ TopkShared<kSelThreads> sh;
  __shared__ int s_flag;
  (void)score_task<D, LM_F32, Q_F32, kSelThreads, SKV_SCORE_UR, false>(p, blockIdx.x, blockIdx.y, blockIdx.z,
                                                                       smem, sh, &s_flag);
}

// Stand-alone selection over a caller's score array: one workgroup per (g, b).
__global__ __launch_bounds__(kSelThreads) void topk_kernel(TopkParams p) {
  const int g = blockIdx.x, b = blockIdx.y;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  __shared__ TopkShared<kSelThreads> sh;
  const int nc = n_candidates(p.seq_lens[b], p.window, p.blk);
  uint32_t* keys = smem;
  int32_t* lds_idx = reinterpret_cast<int32_t*>(keys + p.max_blocks);
  const int64_t t_stride = (int64_t)p.Hkv * p.max_blocks;
  (void)select_rows<kSelThreads, false>(p.scores + ((int64_t)b * p.T * p.Hkv + g) * p.max_blocks, t_stride, false, keys, 0, nc,
              p.T, p.k_per_seq[b], p.k_max, p.indices + ((int64_t)b * p.T * p.Hkv + g) * p.k_max,
              (int64_t)p.Hkv * p.k_max, p.n_sel + (int64_t)b * p.T * p.Hkv + g, p.Hkv,
              p.overlap ? p.overlap + b * p.Hkv + g : nullptr, lds_idx, sh);
}

// ------------------------------------------------------------ launchers

size_t topk_lds_bytes(int max_cand) { return (size_t)max_cand * 4; }

size_t select_static_lds_bytes() { return sizeof(TopkShared<kSelThreads>) + sizeof(int); }

hipError_t launch_score(const ScoreParams& p, int chunks, hipStream_t s) {
  const dim3 grid(chunks, p.Hkv, p.B);
  const size_t lds = score_lds_bytes(p.T, p.D, p.score_cols, p.k_max, p.fused_select != 0, p.cand_only != 0,
                                     p.fused_select && p.two_level && p.cand_ids_lds && !p.cand_only);
#define SKV_SCORE_LAUNCH(D_, LMF, QF) \
  hipLaunchKernelGGL((score_kernel<D_, LMF, QF>), grid, dim3(kSelThreads), lds, s, p)
  const int sel = (p.D == 128 ? 4 : 0) + (p.lm_f32 ? 2 : 0) + (p.q_f32 ? 1 : 0);
  switch (sel) {
    case 0: SKV_SCORE_LAUNCH(64, false, false); break;
    case 1: SKV_SCORE_LAUNCH(64, false, true); break;
    case 2: SKV_SCORE_LAUNCH(64, true, false); break;
    case 3: SKV_SCORE_LAUNCH(64, true, true); break;
    case 4: SKV_SCORE_LAUNCH(128, false, false); break;
    case 5: SKV_SCORE_LAUNCH(128, false, true); break;
    case 6: SKV_SCORE_LAUNCH(128, true, false); break;
    default: SKV_SCORE_LAUNCH(128, true, true); break;
  }
#undef SKV_SCORE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
  const size_t lds = topk_lds_bytes(p.max_blocks) + (size_t)2 * p.k_max * 4;
  hipLaunchKernelGGL(topk_kernel, dim3(p.Hkv, p.B), dim3(kSelThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace skv
