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
//
// The same kernel corrects a speculative prefetch (DualDecoder, mechanism
// summary and Fig. 19): blocks staged for a speculative selection are moved
// into the real selection's slots on the GPU, and only the misses are read
// from the pool.
#include "skv_device.h"
#include "skv_internal.h"

namespace skv {

// First position of `id` in the ascending ids[0..n), or -1.
__device__ __forceinline__ int find_sorted(const int32_t* ids, int n, int id) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ids[mid] < id) lo = mid + 1; else hi = mid;
  }
  return lo < n && ids[lo] == id ? lo : -1;
}

// Grid (slot m, KV head g, sequence b).  With a speculative selection, the
// chunk comes from the speculative stage when the speculative row holds the
// block (the reorder), else from the pool (a miss); the slot-0 workgroup of
// each row also counts the row's misses.
__global__ __launch_bounds__(kThreads) void gather_kernel(GatherParams p) {
  const int m = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t row = ((int64_t)b * p.T + p.token) * p.Hkv + g;
  const int n_real = p.n_sel[row];
  const int32_t* real_ids = p.indices + row * p.k_max;
  const int64_t srow = ((int64_t)b * p.T + p.spec_token) * p.Hkv + g;
  const int n_spec = p.spec_indices ? min(p.spec_n_sel[srow], p.k_max) : 0;
  const int32_t* spec_ids = p.spec_indices ? p.spec_indices + srow * p.k_max : nullptr;

  if (m == 0 && p.misses) {
    __shared__ int s_miss;
    if (threadIdx.x == 0) s_miss = 0;
    __syncthreads();
    int local = 0;
    for (int i = threadIdx.x; i < n_real; i += kThreads)
      local += (spec_ids ? find_sorted(spec_ids, n_spec, real_ids[i]) : -1) < 0;
    if (local) atomicAdd(&s_miss, local);
    __syncthreads();
    if (threadIdx.x == 0) p.misses[(int64_t)b * p.Hkv + g] = s_miss;
  }
  if (m >= n_real) return;

  const int j = real_ids[m];
  const int ms = spec_ids ? find_sorted(spec_ids, n_spec, j) : -1;
  const int64_t slot = ((int64_t)b * p.Hkv + g) * p.k_max + m;
  const int64_t dst_off = slot * p.chunk_bytes;
  const char* ksrc;
  const char* vsrc;
  int64_t phys = 0, sslot = 0;
  if (ms >= 0) {   // reorder: from the speculative slot
    sslot = ((int64_t)b * p.Hkv + g) * p.k_max + ms;
    ksrc = static_cast<const char*>(p.spec_k_stage) + sslot * p.chunk_bytes;
    vsrc = static_cast<const char*>(p.spec_v_stage) + sslot * p.chunk_bytes;
  } else {         // from the pool
    phys = p.block_table[(int64_t)b * p.max_blocks + j];
    const int64_t src_off = (phys * p.stride_block + (int64_t)g * p.stride_head) * p.elem_bytes;
    ksrc = static_cast<const char*>(p.k_pool) + src_off;
    vsrc = static_cast<const char*>(p.v_pool) + src_off;
  }
  const int nvec = (int)(p.chunk_bytes / 16);
  constexpr int UR = 4;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const uint4* src = reinterpret_cast<const uint4*>(which ? vsrc : ksrc);
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
    p.k_stage_scales[slot] = ms >= 0 ? p.spec_k_scales[sslot] : p.k_scales[phys * p.Hkv + g];
    p.v_stage_scales[slot] = ms >= 0 ? p.spec_v_scales[sslot] : p.v_scales[phys * p.Hkv + g];
  }
}

__global__ void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// A plain streaming read of n16 16-byte words with the non-temporal loads
// the step's kernels use, four per thread in flight.  The words are folded
// into one value that is stored only if it equals a constant no input is
// expected to give, so the loads stay live and nothing is written in practice.
__global__ __launch_bounds__(512) void stream_read_kernel(const uint4* p, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = load_stream16(p + i), b = load_stream16(p + i + stride);
    const uint4 c = load_stream16(p + i + 2 * stride), d = load_stream16(p + i + 3 * stride);
    acc += (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) + (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const uint4 a = load_stream16(p + i);
    acc += a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x5eed1e55u) sink[blockIdx.x] = acc;
}

// 512-thread workgroups, one per 32 KiB up to 32768 of them: the fastest of
// a sweep over 256/512/1024 threads, 1024-131072 workgroups and 4/8/16 loads
// in flight (7.0-7.1 TB/s over 2 GiB, against 6.5 for 256-thread workgroups).
constexpr int kReadThreads = 512;
constexpr size_t kReadMaxWorkgroups = 32768;

hipError_t launch_stream_read(const void* ptr, size_t bytes, uint32_t* sink, int sink_words, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 4 * kReadThreads - 1) / (4 * kReadThreads);
  if (blocks > kReadMaxWorkgroups) blocks = kReadMaxWorkgroups;
  if (blocks > (size_t)sink_words) blocks = (size_t)sink_words;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, s,
                     static_cast<const uint4*>(ptr), n16, sink);
  return hipGetLastError();
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
