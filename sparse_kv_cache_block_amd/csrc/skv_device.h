// skv_device.h -- device helpers shared by the gfx950 kernels of the
// sparse-KV decode step (bf16 / fp8 e4m3fn decoding, MFMA wrappers,
// cross-lane reductions).  Internal to the HIP library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

constexpr int kWave = 64;
constexpr int kWaves = 4;               // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

// Tokens per attention item (one slice of a block): 32, or the whole block
// when it is shorter; 16 for fp32 K/V with d = 128, whose 32-token item
// (32 KB of K and V in registers) would not fit a wave's registers.  (64-token
// fp8 items, the same 16 KB of K and V as a bf16 item, measured slower on the
// 262k dual-query workload: its waves hold two or three items each and are
// latency bound, so the item size is kept.)
__host__ __device__ constexpr int attn_item_tokens(int kv, int blk, int d) {
  return blk < 16 ? blk : (kv == KV_F32 && d == 128) ? 16 : (blk < 32 ? blk : 32);
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// Two OCP e4m3fn codes (bytes 0,1 of w when !HI, bytes 2,3 when HI) -> fp32.
// gfx950's conversion instruction decodes the OCP encoding exactly.
template <bool HI>
__device__ __forceinline__ float2 fp8x2_to_f32(uint32_t w) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
  return make_float2(v[0], v[1]);
}

// Four e4m3fn codes -> four bf16 packed in two words, by gfx950's scaled
// conversion with scale 1 (one instruction per two codes).  Exact: an e4m3fn
// value has a 4-bit significand and an exponent well inside bf16's range.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

// Sixteen e4m3fn codes -> sixteen bf16.
__device__ __forceinline__ void fp8x16_to_bf16x16(uint4 c, uint4& lo, uint4& hi) {
  uint2 a = fp8x4_to_bf16x4(c.x), b = fp8x4_to_bf16x4(c.y);
  uint2 d = fp8x4_to_bf16x4(c.z), e = fp8x4_to_bf16x4(c.w);
  lo = make_uint4(a.x, a.y, b.x, b.y);
  hi = make_uint4(d.x, d.y, e.x, e.y);
}

// Order-preserving map of an fp32 score to an unsigned key (larger score ->
// larger key).  -0 is folded onto +0 so that equal scores give equal keys;
// NaN maps to the smallest key.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) return 0u;
  if (s == 0.0f) s = 0.0f;
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16-byte load of streamed, read-once data (K/V chunks, landmarks) with the
// non-temporal hint, so it does not displace reused lines in the caches
// (plain loads measured 65.6 -> 73.6 us on the 32k step).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- lanes

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

// Data-parallel-primitive (DPP) lane moves inside a 16-lane row: plain VALU
// operands, no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of N lanes (N in {4, 8, 16, 32, 64}); every lane of
// a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float a) {
  a += dpp_f<kDppQuadXor1>(a);
  a += dpp_f<kDppQuadXor2>(a);
  if constexpr (N >= 8) a += dpp_f<kDppRowHalfMirror>(a);
  if constexpr (N >= 16) a += dpp_f<kDppRowMirror>(a);
  if constexpr (N >= 32) a += __shfl_xor(a, 16, kWave);
  if constexpr (N >= 64) a += __shfl_xor(a, 32, kWave);
  return a;
}
__device__ __forceinline__ float shfl_f(float v, int src) { return __shfl(v, src, kWave); }

// Compiler and LDS ordering point between one wave's LDS writes and its own
// later reads (LDS operations of a wave complete in order).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS traffic,
// not for its global loads, so loads issued before it stay in flight.
// The scheduling barrier keeps the compiler from hoisting work that consumes
// those loads above it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------- cross-workgroup hand-off
// Split results travel between workgroups of one launch through device-scope
// (agent) atomic stores and loads, which the memory system keeps coherent
// across the XCDs' separate L2 caches.  A producer waits for its own stores to
// complete (vmcnt), the workgroup barrier makes that true for every thread,
// and only then does one thread bump the arrival counter; the last arriver
// reads the others' values with device-scope loads.  This avoids an
// agent-scope fence per workgroup, which on this chip writes back and
// invalidates the whole L2 of the XCD.
//
// The rule this relies on: every value a last arriver reads from another
// workgroup must have been written with an agent-scope atomic store
// (publish_f32, put_i32<true> / put_f32<true>), and read with fetch_f32 /
// fetch_i32.  The counter increment is relaxed, so it orders nothing by
// itself: a plain store into the split partials or the candidate rows may
// still sit in the producer's XCD-private L2 when the last arriver (on
// another XCD) reads, and would be seen stale.  The s_waitcnt below only makes
// the atomic stores complete at device scope before the increment.  The split
// partials and the chunks' candidates are held as Handoff buffers
// (skv_internal.h), which allow no other access.
__device__ __forceinline__ void publish_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch_f32(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t fetch_i32(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_own_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Called by every thread after its publish_f32 stores; returns true in the
// workgroup that arrives last among `expected`, after resetting the counter.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected, int* flag) {
  wait_own_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == expected - 1;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

}  // namespace skv
