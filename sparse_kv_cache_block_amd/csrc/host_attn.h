// host_attn.h -- the CPU side of the hybrid decode step: per-head sparse
// attention over the selected blocks of a KV pool in host memory.  Plain C++
// (no HIP types), so the CPU translation unit builds with the host compiler.
#pragma once

#include <stdint.h>

namespace skv {

struct HostAttnArgs {
  int B, T, Hq, Hkv, D, blk, window, max_blocks, k_max;
  int kv_dtype;                       // skv_dtype of K/V; queries are fp32 for fp32 K/V, else bf16
  int64_t stride_block, stride_head;  // pool element strides
  const void* q;                      // [B][T][Hq][D]; token 0 attended
  const int32_t* seq_lens;            // [B]
  const int32_t* block_table;         // [B][max_blocks]
  const int32_t* indices;             // [B][T][Hkv][k_max], token 0 rows used
  const int32_t* n_sel;               // [B][T][Hkv]
  const void* k_pool;                 // host addresses
  const void* v_pool;
  const float* k_scales;              // [P][Hkv], fp8 only
  const float* v_scales;
  float* o;                           // [B][Hq][D]: normalised output of the sparse part
  float* lse;                         // [B][Hq]: its log-sum-exp (natural log), -inf when empty
  int n_threads;                      // <= 0: every available thread
};

// Attention of the real token of every query head over the positions
// p = j * blk + r of its KV head's selected blocks j with p < max(0, L - W),
// in fp32, one task per (sequence, KV head).
void host_sparse_attention(const HostAttnArgs& a);

}  // namespace skv
