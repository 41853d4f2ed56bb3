// hybrid.hip -- GPU side of the hybrid decode step (Beyond abstract: dense
// attention over the recent KV on the GPU, per-head sparse attention over the
// salient KV in CPU memory, the two outputs fused by log-sum-exp).  The
// window part runs as window-only attention (attend.hip); this kernel fuses
// it with the sparse part the host computed into pinned memory.
#include "skv_device.h"
#include "skv_internal.h"

namespace skv {

// One workgroup per (sequence, query head): out = sum_i e^(lse_i - M) o_i /
// sum_i e^(lse_i - M), lse = M + ln sum_i e^(lse_i - M) over the two parts;
// a part with lse = -inf has weight 0 (both empty: out = 0, lse = -inf).
__global__ __launch_bounds__(128) void lse_merge_kernel(const float* o_a, const float* lse_a, const float* o_b,
                                                        const float* lse_b, float* out, float* lse, int D) {
  const int64_t bh = blockIdx.x;
  const float la = lse_a ? lse_a[bh] : -INFINITY;
  const float lb = lse_b[bh];
  const float M = fmaxf(la, lb);
  const float wa = la == -INFINITY ? 0.f : expf(la - M);
  const float wb = lb == -INFINITY ? 0.f : expf(lb - M);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float v = 0.f;
    if (M != -INFINITY) {
      const float oa = wa > 0.f ? o_a[bh * D + d] : 0.f;
      const float ob = wb > 0.f ? o_b[bh * D + d] : 0.f;
      v = (wa * oa + wb * ob) / (wa + wb);
    }
    out[bh * D + d] = v;
  }
  if (threadIdx.x == 0 && lse) lse[bh] = M == -INFINITY ? -INFINITY : M + logf(wa + wb);
}

hipError_t launch_lse_merge(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                            float* out, float* lse, int rows, int D, hipStream_t s) {
  hipLaunchKernelGGL(lse_merge_kernel, dim3(rows), dim3(128), 0, s, o_a, lse_a, o_b, lse_b, out, lse, D);
  return hipGetLastError();
}

}  // namespace skv
