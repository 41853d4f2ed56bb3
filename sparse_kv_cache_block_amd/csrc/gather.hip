// gather.hip -- gather of the selected (block, head) chunks into a dense
// staging buffer, and the workspace fill kernel, for gfx950.
//
// PulseInfer (article, section 2) pairs sparse selection with a
// gather-scatter I/O engine that merges many small, scattered transfers into
// few large ones; DualDecoder (Fig. 19) fetches whole blocks contiguously and
// lets GPU kernels reorder them.  Here one workgroup moves one selected chunk
// of K and one of V (blk*d elements each, contiguous in the pool) with
// 16-byte loads, several in flight per lane, into slot m of the staging
// buffer, so every request is a whole-chunk sequential read.  The source may
// be device memory or pinned host memory read over the host link; in the
// host-major pool layout neighbouring selected blocks of a head are adjacent,
// so runs of them form one sequential stream.
#include "skv_device.h"
#include "skv_internal.h"

namespace skv {

__global__ __launch_bounds__(kThreads) void gather_kernel(GatherParams p) {
  const int m = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t row = (int64_t)b * p.T * p.Hkv + g;  // token 0 selection
  if (m >= p.n_sel[row]) return;
  const int j = p.indices[row * p.k_max + m];
  const int64_t phys = p.block_table[(int64_t)b * p.max_blocks + j];
  const int64_t src_off = (phys * p.stride_block + (int64_t)g * p.stride_head) * p.elem_bytes;
  const int64_t slot = ((int64_t)b * p.Hkv + g) * p.k_max + m;
  const int64_t dst_off = slot * p.chunk_bytes;
  const int nvec = (int)(p.chunk_bytes / 16);
  constexpr int UR = 4;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const uint4* src = reinterpret_cast<const uint4*>(
        static_cast<const char*>(which ? p.v_pool : p.k_pool) + src_off);
    uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(which ? p.v_stage : p.k_stage) + dst_off);
    for (int base = threadIdx.x; base < nvec; base += UR * kThreads) {
      uint4 v[UR];
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const int i = base + u * kThreads;
        if (i < nvec) v[u] = src[i];
      }
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const int i = base + u * kThreads;
        if (i < nvec) dst[i] = v[u];
      }
    }
  }
  if (p.has_scales && threadIdx.x == 0) {
    p.k_stage_scales[slot] = p.k_scales[phys * p.Hkv + g];
    p.v_stage_scales[slot] = p.v_scales[phys * p.Hkv + g];
  }
}

__global__ void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
  hipLaunchKernelGGL(gather_kernel, dim3(p.k_max, p.Hkv, p.B), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<uint4*>(ptr), n16);
  return hipGetLastError();
}

}  // namespace skv
