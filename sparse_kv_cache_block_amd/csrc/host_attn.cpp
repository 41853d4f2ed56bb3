// host_attn.cpp -- the CPU side of the hybrid decode step (Beyond abstract:
// dense attention over the recent KV on the GPU, per-head sparse attention
// over the salient KV in CPU memory, the two fused by log-sum-exp).
//
// One task per (sequence, KV head), spread over OpenMP threads.  A task
// serves the G query heads of its group from each selected block: logits of
// every row of the block, an online softmax update per head, then the V rows
// accumulated into the G outputs.
// The row loops use AVX2 + FMA (x86-64-v3) with the G heads register-blocked.
#include "host_attn.h"

#include <immintrin.h>
#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>

#include "../../include/sparsekv.h"

namespace skv {
namespace {

constexpr int kMaxBlk = 64;

inline float bf16_to_f32(uint16_t h) {
  const uint32_t bits = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &bits, sizeof f);
  return f;
}

// OCP fp8 e4m3fn: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
// is subnormal (2^-6 * m/8); S.1111.111 is NaN; no infinities.
struct E4m3Table {
  float v[256];
  E4m3Table() {
    for (int c = 0; c < 256; ++c) {
      const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
      float x;
      if (e == 15 && m == 7) x = std::numeric_limits<float>::quiet_NaN();
      else if (e == 0) x = std::ldexp((float)m / 8.0f, -6);
      else x = std::ldexp(1.0f + (float)m / 8.0f, e - 7);
      v[c] = s ? -x : x;
    }
  }
};
const E4m3Table kE4m3;   // built when the library loads

// 8 consecutive elements of a K/V row as fp32 (fp8: times `scale`).
inline __m256 load8(const void* base, int kv_dtype, int64_t elem_off, __m256 scale) {
  if (kv_dtype == SKV_BF16) {
    const __m128i h = _mm_loadu_si128(reinterpret_cast<const __m128i*>(static_cast<const uint16_t*>(base) + elem_off));
    return _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
  }
  if (kv_dtype == SKV_FP8_E4M3FN) {
    const int64_t c8 = *reinterpret_cast<const int64_t*>(static_cast<const uint8_t*>(base) + elem_off);
    const __m256i idx = _mm256_cvtepu8_epi32(_mm_cvtsi64_si128(c8));
    return _mm256_mul_ps(_mm256_i32gather_ps(kE4m3.v, idx, 4), scale);
  }
  return _mm256_loadu_ps(static_cast<const float*>(base) + elem_off);
}

inline float hsum(__m256 v) {
  const __m128 s = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  const __m128 t = _mm_add_ps(s, _mm_movehl_ps(s, s));
  return _mm_cvtss_f32(_mm_add_ss(t, _mm_shuffle_ps(t, t, 1)));
}

// One (sequence, KV head): the G heads of the group over the group's
// selected blocks.  Per block: logits of every row for all G heads (each K
// row read once into G accumulators), an online softmax update per head,
// then P V with the G outputs of an 8-column slice held in registers while
// the block's V rows stream past.
template <int D, int G>
void pair_task(const HostAttnArgs& a, int b, int g) {
  constexpr int C8 = D / 8;
  const int L = a.seq_lens[b];
  const int64_t ws = std::max(0, L - a.window);
  const int64_t sel_row = ((int64_t)b * a.T * a.Hkv + g);
  const int32_t* idx = a.indices + sel_row * a.k_max;
  const int n = a.n_sel[sel_row];
  const float qk_scale = 1.0f / std::sqrt((float)D);
  const float ninf = -std::numeric_limits<float>::infinity();

  alignas(32) float qf[G][D];
  for (int h = 0; h < G; ++h) {
    const int64_t qrow = (((int64_t)b * a.T) * a.Hq + (int64_t)g * G + h) * D;
    for (int i = 0; i < D; ++i)
      qf[h][i] = (a.kv_dtype == SKV_F32 ? static_cast<const float*>(a.q)[qrow + i]
                                        : bf16_to_f32(static_cast<const uint16_t*>(a.q)[qrow + i])) * qk_scale;
  }
  alignas(32) float acc[G][D];
  float m_run[G], l_run[G];
  for (int h = 0; h < G; ++h) {
    m_run[h] = ninf;
    l_run[h] = 0.f;
    std::fill(acc[h], acc[h] + D, 0.f);
  }
  alignas(32) float pr[G][kMaxBlk];

  for (int m = 0; m < n; ++m) {
    const int64_t j = idx[m];
    const int64_t p0 = j * a.blk;
    const int rows = (int)std::min<int64_t>(a.blk, ws - p0);
    if (rows <= 0) continue;
    const int64_t phys = a.block_table[(int64_t)b * a.max_blocks + j];
    const int64_t off = phys * a.stride_block + (int64_t)g * a.stride_head;
    const bool fp8 = a.kv_dtype == SKV_FP8_E4M3FN;
    const __m256 ks = _mm256_set1_ps(fp8 ? a.k_scales[phys * a.Hkv + g] : 1.f);
    const __m256 vs = _mm256_set1_ps(fp8 ? a.v_scales[phys * a.Hkv + g] : 1.f);
    if (m + 1 < n) {   // the next block's first lines while this one is processed
      const int64_t jn = idx[m + 1];
      const int64_t pn = a.block_table[(int64_t)b * a.max_blocks + jn];
      const int64_t on = (pn * a.stride_block + (int64_t)g * a.stride_head) * (a.kv_dtype == SKV_F32 ? 4 : a.kv_dtype == SKV_BF16 ? 2 : 1);
      __builtin_prefetch(static_cast<const char*>(a.k_pool) + on);
      __builtin_prefetch(static_cast<const char*>(a.v_pool) + on);
    }
    // logits
    for (int r = 0; r < rows; ++r) {
      __m256 s[G];
      for (int h = 0; h < G; ++h) s[h] = _mm256_setzero_ps();
      for (int c = 0; c < C8; ++c) {
        const __m256 kv = load8(a.k_pool, a.kv_dtype, off + (int64_t)r * D + 8 * c, ks);
        for (int h = 0; h < G; ++h) s[h] = _mm256_fmadd_ps(_mm256_load_ps(&qf[h][8 * c]), kv, s[h]);
      }
      for (int h = 0; h < G; ++h) pr[h][r] = hsum(s[h]);
    }
    // online softmax update per head
    for (int h = 0; h < G; ++h) {
      float bm = pr[h][0];
      for (int r = 1; r < rows; ++r) bm = std::max(bm, pr[h][r]);
      const float m_new = std::max(m_run[h], bm);
      const float c = m_run[h] == ninf ? 0.f : std::exp(m_run[h] - m_new);
      float psum = 0.f;
      for (int r = 0; r < rows; ++r) {
        pr[h][r] = std::exp(pr[h][r] - m_new);
        psum += pr[h][r];
      }
      l_run[h] = l_run[h] * c + psum;
      m_run[h] = m_new;
      if (c != 1.f) {
        const __m256 cv = _mm256_set1_ps(c);
        for (int i = 0; i < D; i += 8) _mm256_store_ps(&acc[h][i], _mm256_mul_ps(_mm256_load_ps(&acc[h][i]), cv));
      }
    }
    // P V, one 8-column slice of the G outputs at a time
    for (int c = 0; c < C8; ++c) {
      __m256 o[G];
      for (int h = 0; h < G; ++h) o[h] = _mm256_load_ps(&acc[h][8 * c]);
      for (int r = 0; r < rows; ++r) {
        const __m256 vv = load8(a.v_pool, a.kv_dtype, off + (int64_t)r * D + 8 * c, vs);
        for (int h = 0; h < G; ++h) o[h] = _mm256_fmadd_ps(_mm256_broadcast_ss(&pr[h][r]), vv, o[h]);
      }
      for (int h = 0; h < G; ++h) _mm256_store_ps(&acc[h][8 * c], o[h]);
    }
  }
  for (int h = 0; h < G; ++h) {
    const int64_t bh = (int64_t)b * a.Hq + (int64_t)g * G + h;
    float* o = a.o + bh * D;
    if (l_run[h] > 0.f) {
      const float inv = 1.f / l_run[h];
      for (int i = 0; i < D; ++i) o[i] = acc[h][i] * inv;
      a.lse[bh] = m_run[h] + std::log(l_run[h]);
    } else {
      std::fill(o, o + D, 0.f);
      a.lse[bh] = ninf;
    }
  }
}

template <int D>
void pair_task_d(const HostAttnArgs& a, int b, int g) {
  switch (a.Hq / a.Hkv) {
    case 1: pair_task<D, 1>(a, b, g); break;
    case 2: pair_task<D, 2>(a, b, g); break;
    case 3: pair_task<D, 3>(a, b, g); break;
    case 4: pair_task<D, 4>(a, b, g); break;
    case 5: pair_task<D, 5>(a, b, g); break;
    case 6: pair_task<D, 6>(a, b, g); break;
    case 7: pair_task<D, 7>(a, b, g); break;
    default: pair_task<D, 8>(a, b, g); break;
  }
}

}  // namespace

void host_sparse_attention(const HostAttnArgs& a) {
  const int tasks = a.B * a.Hkv;
  const int nt = a.n_threads > 0 ? a.n_threads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int t = 0; t < tasks; ++t) {
    const int b = t / a.Hkv, g = t % a.Hkv;
    if (a.D == 128) pair_task_d<128>(a, b, g);
    else pair_task_d<64>(a, b, g);
  }
}

}  // namespace skv
