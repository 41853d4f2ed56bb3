// attend.hip -- split-K decode attention over the selected blocks plus the
// recent window, fused by log-sum-exp, for gfx950.
//
// Method (Beyond abstract: dense attention over the recent window and per-head
// sparse attention over salient KV, combined by a log-sum-exp scheme): every
// workgroup owns one split of one (sequence, KV head) -- a run of selected
// blocks or of window blocks -- and each of its four waves streams whole
// (block, head) chunks.  A wave computes, for the G query heads of the group,
//   S^T = K Q^T   with v_mfma_f32_16x16x32_bf16 (16 tokens x 16 columns),
// where the 16 columns hold the G heads twice (or once for fp32 K/V), so the
// C layout leaves lane (column n, row group j) with the logits of tokens
// 4j..4j+3 -- exactly the A-operand layout the P V product needs.  Columns
// G..2G-1 carry the low part of a hi/lo bf16 split of P, so
//   O = P_hi V + P_lo V
// keeps P to about 2^-17 relative accuracy with one MFMA per 32 tokens.  V is
// staged through LDS to read it token-major for the B operand; fp8 e4m3fn
// blocks are decoded to bf16 on the way (exact), their K scale multiplies the
// logits and their V scale multiplies P.  Online softmax runs in the log2
// domain in fp32.  The four waves' partials are combined in LDS, each
// workgroup writes (max, sum, unnormalised O) per head, and the last
// workgroup of the (sequence, KV head) -- device-scope atomic counter --
// merges all splits into the fp32 output and lse.
#include "skv_device.h"
#include "skv_internal.h"

namespace skv {

template <int KV, int D, int BLK>
struct AttnCfg {
  static constexpr int NT = BLK / 16;                     // QK tiles per block
  static constexpr int DT = D / 16;                       // PV output tiles
  static constexpr int ES = KV == KV_F32 ? 4 : (KV == KV_BF16 ? 2 : 1);
  static constexpr int KS = KV == KV_F32 ? D / 4 : D / 32;  // QK k-steps
  static constexpr int NPAIR = (NT + 1) / 2;              // PV k-steps of 32 tokens
  static constexpr int VE = KV == KV_F32 ? 4 : 2;         // LDS element bytes
  static constexpr int VROW = D * VE + 16;                // padded LDS row bytes
  static constexpr int VTILE = BLK * VROW;
  static constexpr int COMB = 16 * D * 4 + 2 * 16 * 4;    // O rows + m + l
  static constexpr int PER_WAVE = VTILE > COMB ? VTILE : COMB;
  static constexpr int CHUNK = BLK * D * ES;              // bytes of one (block, head) chunk
  static constexpr int NV = CHUNK / (kWave * 16);         // 16-byte V loads per lane
};

struct BlockRef {
  const char* k;
  const char* v;
  float ks, vs;   // fp8 scales
  int pos0;       // sequence position of the chunk's row 0
};

// Locate item `i` of this workgroup's split.
template <int ES, int BLK>
__device__ __forceinline__ BlockRef locate(const AttnParams& p, bool sparse, int b, int g, int i,
                                           int ws) {
  BlockRef r;
  r.ks = 1.f;
  r.vs = 1.f;
  if (sparse) {
    const int64_t row = ((int64_t)b * p.T * p.Hkv + g) * p.k_max;  // token 0
    const int j = p.indices[row + i];
    r.pos0 = j * BLK;
    if (p.sparse_kind == SKV_SRC_PAGED) {
      const int64_t phys = p.block_table[(int64_t)b * p.max_blocks + j];
      const int64_t off = phys * p.stride_block + (int64_t)g * p.stride_head;
      r.k = static_cast<const char*>(p.sk) + off * ES;
      r.v = static_cast<const char*>(p.sv) + off * ES;
      if (p.sks) {
        r.ks = p.sks[phys * p.Hkv + g];
        r.vs = p.svs[phys * p.Hkv + g];
      }
    } else {
      const int64_t slot = ((int64_t)b * p.Hkv + g) * p.k_max + i;
      r.k = static_cast<const char*>(p.sk) + slot * (int64_t)BLK * p.D * ES;
      r.v = static_cast<const char*>(p.sv) + slot * (int64_t)BLK * p.D * ES;
      if (p.sks) {
        r.ks = p.sks[slot];
        r.vs = p.svs[slot];
      }
    }
  } else if (p.window_kind == SKV_SRC_PAGED) {
    const int j = ws / BLK + i;
    r.pos0 = j * BLK;
    const int64_t phys = p.window_table[(int64_t)b * p.max_blocks + j];
    const int64_t off = phys * p.stride_block + (int64_t)g * p.stride_head;
    r.k = static_cast<const char*>(p.wk) + off * ES;
    r.v = static_cast<const char*>(p.wv) + off * ES;
    if (p.wks) {
      r.ks = p.wks[phys * p.Hkv + g];
      r.vs = p.wvs[phys * p.Hkv + g];
    }
  } else {
    r.pos0 = ws + i * BLK;
    const int64_t off = (((int64_t)b * p.Hkv + g) * p.window + (int64_t)i * BLK) * p.D;
    r.k = static_cast<const char*>(p.wk) + off * ES;
    r.v = static_cast<const char*>(p.wv) + off * ES;
  }
  return r;
}

template <int KV, int D, int BLK>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttnParams p) {
  using C = AttnCfg<KV, D, BLK>;
  __shared__ __attribute__((aligned(16))) char smem[kWaves * C::PER_WAVE];
  __shared__ int s_last;

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = lane_id(), w = wave_id();
  const int n = lane & 15;   // C/B column, A row
  const int kg = lane >> 4;  // row group / k group
  const int G = p.G;
  const int L = p.seq_lens[b];
  const int ws = L - p.window > 0 ? L - p.window : 0;
  const int total_splits = p.n_sparse_splits + p.n_window_splits;

  // ---- this workgroup's items
  const bool sparse = split < p.n_sparse_splits;
  int first, count, lo, hi;
  if (sparse) {
    const int nsel = p.n_sel[(int64_t)b * p.T * p.Hkv + g];
    first = split * p.bps;
    count = min(p.bps, nsel - first);
    lo = 0;
    hi = ws;
  } else {
    const int s2 = split - p.n_sparse_splits;
    int nwin = 0;
    if (ws < L) {
      if (p.window_kind == SKV_SRC_PAGED) nwin = (L - 1) / BLK - ws / BLK + 1;
      else nwin = (L - ws + BLK - 1) / BLK;
    }
    first = s2 * p.bpw;
    count = min(p.bpw, nwin - first);
    lo = ws;
    hi = L;
  }
  if (count < 0) count = 0;

  // ---- query operand: column n holds head n (and head n-G for the low half)
  const int ncols = KV == KV_F32 ? G : 2 * G;
  const int hq = n < G ? n : (n < ncols ? n - G : -1);
  uint4 qop[KV == KV_F32 ? 1 : C::KS];
  float qopf[KV == KV_F32 ? C::KS : 1];
  {
    const int64_t qrow = (((int64_t)b * p.T) * p.Hq + (int64_t)g * G + (hq < 0 ? 0 : hq)) * D;
    if constexpr (KV == KV_F32) {
      const float* qp = static_cast<const float*>(p.q) + qrow + (D / 4) * kg;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) qopf[s] = hq < 0 ? 0.f : qp[s];
    } else {
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + qrow + (D / 4) * kg;
#pragma unroll
      for (int s = 0; s < C::KS; ++s)
        qop[s] = hq < 0 ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4*>(qp + 8 * s);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  char* vt = smem + w * C::PER_WAVE;

  for (int it = w; it < count; it += kWaves) {
    const BlockRef br = locate<C::ES, BLK>(p, sparse, b, g, first + it, ws);

    // ---- K rows of this lane: row (16*tile + n), elements [(D/4)kg, (D/4)(kg+1))
    f32x4_t st[C::NT];
#pragma unroll
    for (int tile = 0; tile < C::NT; ++tile) {
      const char* krow = br.k + (int64_t)(16 * tile + n) * D * C::ES + (D / 4) * kg * C::ES;
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (KV == KV_BF16) {
#pragma unroll
        for (int s = 0; s < C::KS; ++s)
          acc = mfma_bf16(*reinterpret_cast<const uint4*>(krow + 16 * s), qop[s], acc);
      } else if constexpr (KV == KV_FP8) {
#pragma unroll
        for (int s2 = 0; s2 < C::KS / 2; ++s2) {
          uint4 lo16, hi16;
          fp8x16_to_bf16x16(*reinterpret_cast<const uint4*>(krow + 16 * s2), lo16, hi16);
          acc = mfma_bf16(lo16, qop[2 * s2], acc);
          acc = mfma_bf16(hi16, qop[2 * s2 + 1], acc);
        }
      } else {
#pragma unroll
        for (int s4 = 0; s4 < C::KS / 4; ++s4) {
          const float4 kk = *reinterpret_cast<const float4*>(krow + 16 * s4);
          acc = mfma_f32(kk.x, qopf[4 * s4 + 0], acc);
          acc = mfma_f32(kk.y, qopf[4 * s4 + 1], acc);
          acc = mfma_f32(kk.z, qopf[4 * s4 + 2], acc);
          acc = mfma_f32(kk.w, qopf[4 * s4 + 3], acc);
        }
      }
      st[tile] = acc;
    }

    // ---- V chunk -> LDS (token-major, padded rows); rows outside [lo, hi) are zeroed
    const bool partial = br.pos0 < lo || br.pos0 + BLK > hi;
#pragma unroll
    for (int i = 0; i < C::NV; ++i) {
      const int off = 16 * (lane + kWave * i);
      const int row = off / (D * C::ES);
      const int col = off % (D * C::ES);
      const uint4 raw = *reinterpret_cast<const uint4*>(br.v + off);
      const bool ok = !partial || (br.pos0 + row >= lo && br.pos0 + row < hi);
      if constexpr (KV == KV_FP8) {
        uint4 a, c;
        fp8x16_to_bf16x16(raw, a, c);
        if (!ok) a = c = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(vt + row * C::VROW + 2 * col) = a;
        *reinterpret_cast<uint4*>(vt + row * C::VROW + 2 * col + 16) = c;
      } else {
        *reinterpret_cast<uint4*>(vt + row * C::VROW + col) = ok ? raw : make_uint4(0, 0, 0, 0);
      }
    }

    // ---- online softmax (log2 domain)
    const float sc = p.qk_scale * br.ks;
    float bm = -INFINITY;
#pragma unroll
    for (int tile = 0; tile < C::NT; ++tile)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = br.pos0 + 16 * tile + 4 * kg + r;
        float z = st[tile][r] * sc;
        z = (pos >= lo && pos < hi) ? z : -INFINITY;
        st[tile][r] = z;
        bm = fmaxf(bm, z);
      }
    bm = fmaxf(bm, shfl_xor_f(bm, 16));
    bm = fmaxf(bm, shfl_xor_f(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int tile = 0; tile < C::NT; ++tile)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = none ? 0.f : exp2f(st[tile][r] - m_new);
        st[tile][r] = pv;
        psum += pv;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    if (__ballot(n < ncols && alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * kg + i;
        const int head = row < ncols ? row % G : 0;
        const float a = shfl_f(alpha, head);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) o[dt][i] *= a;
      }
    }

    wave_lds_sync();

    // ---- O += P V
    if constexpr (KV == KV_F32) {
#pragma unroll
      for (int tile = 0; tile < C::NT; ++tile)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = n < G ? st[tile][r] : 0.f;
          const char* vrow = vt + (16 * tile + 4 * kg + r) * C::VROW + 4 * n;
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
            o[dt] = mfma_f32(a, *reinterpret_cast<const float*>(vrow + 64 * dt), o[dt]);
        }
    } else {
#pragma unroll
      for (int u = 0; u < C::NPAIR; ++u) {
        uint32_t pw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          uint32_t bits[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int e = 2 * e2 + h2;
            const int tile = 2 * u + e / 4;
            float pv = tile < C::NT ? st[tile < C::NT ? tile : 0][e % 4] : 0.f;
            if constexpr (KV == KV_FP8) pv *= br.vs;
            const uint32_t hb = f32_to_bf16_rne(pv);
            uint32_t x = 0;
            if (n < G) x = hb;
            else if (n < ncols) x = f32_to_bf16_rne(pv - __uint_as_float(hb << 16));
            bits[h2] = x;
          }
          pw[e2] = pack_bf16(bits[0], bits[1]);
        }
        const uint4 aop = make_uint4(pw[0], pw[1], pw[2], pw[3]);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          uint32_t vw[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t hv[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const int e = 2 * e2 + h2;
              const int tile = 2 * u + e / 4;
              const int tok = 16 * tile + 4 * kg + (e % 4);
              hv[h2] = tile < C::NT
                           ? *reinterpret_cast<const uint16_t*>(vt + tok * C::VROW + 2 * (16 * dt + n))
                           : 0u;
            }
            vw[e2] = pack_bf16(hv[0], hv[1]);
          }
          o[dt] = mfma_bf16(aop, make_uint4(vw[0], vw[1], vw[2], vw[3]), o[dt]);
        }
      }
    }
    wave_lds_sync();
  }

  // ---- combine the four waves in LDS
  float lsum = l_run;
  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);
  __syncthreads();
  {
    float* comb = reinterpret_cast<float*>(smem + w * C::PER_WAVE);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) comb[(4 * kg + i) * D + 16 * dt + n] = o[dt][i];
    if (kg == 0) {
      comb[16 * D + n] = m_run;
      comb[16 * D + 16 + n] = lsum;
    }
  }
  __syncthreads();
  float* part = p.partials + (((int64_t)b * p.Hkv + g) * total_splits + split) * G * (D + 2);
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww)
      M = fmaxf(M, reinterpret_cast<const float*>(smem + ww * C::PER_WAVE)[16 * D + h]);
    float O = 0.f, Ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float* comb = reinterpret_cast<const float*>(smem + ww * C::PER_WAVE);
        const float mw = comb[16 * D + h];
        if (mw == -INFINITY) continue;
        const float f = exp2f(mw - M);
        float ov = comb[h * D + d];
        if constexpr (KV != KV_F32) ov += comb[(G + h) * D + d];
        O += f * ov;
        Ls += f * comb[16 * D + 16 + h];
      }
    }
    part[h * (D + 2) + 2 + d] = O;
    if (d == 0) {
      part[h * (D + 2)] = M;
      part[h * (D + 2) + 1] = Ls;
    }
  }

  // ---- the last split of (b, g) merges every split
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = p.counters + b * p.Hkv + g;
    const unsigned old = atomicAdd(cnt, 1u);
    s_last = old == (unsigned)(total_splits - 1);
    if (s_last) *cnt = 0u;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* pb = p.partials + ((int64_t)b * p.Hkv + g) * total_splits * G * (D + 2);
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
    for (int s = 0; s < total_splits; ++s) M = fmaxf(M, pb[((int64_t)s * G + h) * (D + 2)]);
    float O = 0.f, Ls = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < total_splits; ++s) {
        const float* ps = pb + ((int64_t)s * G + h) * (D + 2);
        if (ps[0] == -INFINITY) continue;
        const float f = exp2f(ps[0] - M);
        O += f * ps[2 + d];
        Ls += f * ps[1];
      }
    }
    const int64_t bh = (int64_t)b * p.Hq + (int64_t)g * G + h;
    p.out[bh * D + d] = M == -INFINITY ? 0.f : O / Ls;
    if (d == 0 && p.lse) p.lse[bh] = M == -INFINITY ? -INFINITY : (M + log2f(Ls)) * kLn2;
  }
}

template <int KV, int D>
static hipError_t launch_blk(const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (p.blk) {
    case 16: hipLaunchKernelGGL((attend_kernel<KV, D, 16>), grid, dim3(kThreads), 0, s, p); break;
    case 32: hipLaunchKernelGGL((attend_kernel<KV, D, 32>), grid, dim3(kThreads), 0, s, p); break;
    case 64: hipLaunchKernelGGL((attend_kernel<KV, D, 64>), grid, dim3(kThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KV>
static hipError_t launch_d(const AttnParams& p, dim3 grid, hipStream_t s) {
  return p.D == 128 ? launch_blk<KV, 128>(p, grid, s) : launch_blk<KV, 64>(p, grid, s);
}

hipError_t launch_attend(const AttnParams& p, hipStream_t s) {
  const dim3 grid(p.n_sparse_splits + p.n_window_splits, p.Hkv, p.B);
  switch (p.kv) {
    case KV_F32: return launch_d<KV_F32>(p, grid, s);
    case KV_BF16: return launch_d<KV_BF16>(p, grid, s);
    case KV_FP8: return launch_d<KV_FP8>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace skv
