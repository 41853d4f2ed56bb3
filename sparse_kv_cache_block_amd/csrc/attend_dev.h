// attend_dev.h -- device code of split-K decode attention over the selected
// blocks plus the recent window, fused by log-sum-exp, for gfx950; shared by
// the stand-alone attention kernel and the single-launch decode step.
//
// Method (Beyond abstract: the recent window is attended densely on the GPU,
// the important older entries sparsely per head, and the two results are
// merged through their log-sum-exp).  For one (sequence, KV head) the work is
// a list of items -- 32-token slices of the selected blocks (positions before
// the window start), then slices of the window blocks (positions in the
// window) -- and each workgroup owns one contiguous range of that list
// (split-K).  Sparse and window items keep separate position masks, so the
// sparse and window parts stay disjoint and every partial is an exact softmax
// partial of its own position set; merging all of them by log-sum-exp is the
// sparse/window fusion itself.
//
// Per item a wave computes, for the G query heads of the group,
//   S^T = K Q^T    with v_mfma_f32_16x16x32_bf16 (16 tokens x 16 columns);
// the 16 columns hold the G heads twice (once for fp32), so the C layout
// leaves lane (column n, row group j) with the logits of tokens 4j..4j+3 --
// exactly the A-operand layout of the P V product.  Columns G..2G-1 carry the
// low half of a hi/lo bf16 split of P, so O = P_hi V + P_lo V keeps P to about
// 2^-17 relative accuracy with one MFMA per 32 tokens.  K rows are read with
// 16-byte loads straight into the MFMA layout (one 64-byte run of a row per
// instruction); V goes through LDS and comes back token-major with
// ds_read_b64_tr_b16.  fp8 e4m3fn data are decoded to bf16 exactly; the K
// scale multiplies the logits and the V scale multiplies P.  The next item's
// K/V loads are issued before the current item's softmax and P V, so each
// wave keeps one item in flight while it computes.  Online softmax runs in
// the log2 domain in fp32.
//
// Co-batched attention of two query tokens (DualDecoder review, Fig. 18: the
// real and the speculative token attended in one launch): the 16 columns hold
// the 2G (token, head) pairs, the low half of P takes a second MFMA, and the
// sparse items are the union of the two tokens' selections; an item that one
// token did not select is masked in that token's columns, so each token's
// result is its own attention over its own selection plus the window.  The waves' partials are combined in LDS; each
// workgroup publishes (max, sum, unnormalised O) per head, and the last
// workgroup of the (sequence, KV head) merges all of them into the fp32
// output and lse.
#pragma once

#include <type_traits>

#include "skv_device.h"
#include "skv_internal.h"

namespace skv {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <int KV, int D, int BLK>
struct AttnCfg {
  static constexpr int ES = KV == KV_F32 ? 4 : (KV == KV_BF16 ? 2 : 1);
  static constexpr int TB = attn_item_tokens(KV, BLK, D);  // tokens per item
  static constexpr int SUB = BLK / TB;                   // items per block
  static constexpr int NT = TB / 16;                     // QK tiles per item
  static constexpr int DT = D / 16;                      // PV output tiles
  static constexpr int GRAN = D * ES / 64;               // 16-byte K granules per lane per row
  static constexpr int KS = KV == KV_F32 ? D / 4 : D / 32;  // QK k-steps
  static constexpr int VE = KV == KV_F32 ? 4 : 2;        // LDS element bytes
  static constexpr int VROW = D * VE + 16;               // padded LDS row bytes
  static constexpr int VTILE = TB * VROW;
  static constexpr int COMB = 16 * D * 4 + 2 * 16 * 4;   // combine region: O rows + m + l
  static constexpr int PER_WAVE = VTILE > COMB ? VTILE : COMB;
  static constexpr int ITEM_BYTES = TB * D * ES;         // bytes of one item's K (or V)
  static constexpr int NV = ITEM_BYTES / (kWave * 16);   // 16-byte V loads per lane
};

// Descriptor of one item, held by one lane of the wave that processes it.
// It keeps the block's row in its source as loaded (no arithmetic on it), so
// building a descriptor never waits for a table lookup; the element offset
// and the fp8 scales are formed when the item's loads are issued.
struct ItemDesc {
  int row;        // physical block (paged source), staging slot, or first token row (window buffer)
  int pos0;       // sequence position of the item's row 0; bit 31 marks a window item
  int sub;        // slice of the block (bits 0-7); bits 8-9: query tokens that skip the item
};

// Slice `sub` of block j of a paged source whose physical block is known.
template <int KV, int D, int BLK>
__device__ __forceinline__ ItemDesc describe_paged(int j, int phys, int sub) {
  using C = AttnCfg<KV, D, BLK>;
  return ItemDesc{phys, j * BLK + sub * C::TB, sub};
}

// Slice `sub` of the m-th selected block of (b, g), block id j.  A paged
// source reads physical block `phys` (negative: look it up in the block
// table); a staged source reads slot m of the (b, g) staging row.
template <int KV, int D, int BLK>
__device__ __forceinline__ ItemDesc describe_sparse(const AttnParams& p, int b, int g, int m, int j,
                                                    int64_t phys, int sub) {
  using C = AttnCfg<KV, D, BLK>;
  ItemDesc d;
  d.sub = sub;
  d.pos0 = j * BLK + sub * C::TB;
  if (p.sparse_kind == SKV_SRC_PAGED)
    d.row = phys >= 0 ? (int)phys : p.block_table[(int64_t)b * p.max_blocks + j];
  else
    d.row = (b * p.Hkv + g) * p.k_max + m;
  return d;
}

// Slice `sub` of the c-th block of (b, g)'s recent window (window start ws).
template <int KV, int D, int BLK>
__device__ __forceinline__ ItemDesc describe_window(const AttnParams& p, int b, int g, int c, int sub, int ws) {
  using C = AttnCfg<KV, D, BLK>;
  ItemDesc d;
  d.sub = sub;
  if (p.window_kind == SKV_SRC_PAGED) {
    const int j = ws / BLK + c;
    d.pos0 = j * BLK + sub * C::TB;
    d.row = p.window_table[(int64_t)b * p.max_blocks + j];
  } else {
    d.pos0 = ws + c * BLK + sub * C::TB;
    d.row = (b * p.Hkv + g) * p.window + c * BLK;
  }
  d.pos0 |= (int)0x80000000;
  return d;
}

// Item `item` of (b, g)'s list: slices of the nsel selected blocks (ids and,
// when given, physical ids from the selection's output rows), then slices of
// the window blocks.
template <int KV, int D, int BLK>
__device__ __forceinline__ ItemDesc describe(const AttnParams& p, int b, int g, int item, int nsel, int ws) {
  using C = AttnCfg<KV, D, BLK>;
  const int blk_item = item / C::SUB, sub = item % C::SUB;
  if (blk_item < nsel) {
    const int64_t row = ((int64_t)b * p.T * p.Hkv + g) * p.k_max + blk_item;
    // physical ids emitted by the selection save the dependent table lookup
    return describe_sparse<KV, D, BLK>(p, b, g, blk_item, p.indices[row], p.phys ? p.phys[row] : -1, sub);
  }
  return describe_window<KV, D, BLK>(p, b, g, blk_item - nsel, sub, ws);
}

// LDS bytes of an NW-wave attention workgroup (per-wave V tiles / combine rows).
template <int KV, int D, int BLK>
constexpr int attn_lds_bytes(int nw) { return nw * AttnCfg<KV, D, BLK>::PER_WAVE; }

// Window blocks of a sequence of length L (window start ws).
__device__ __forceinline__ int window_blocks(const AttnParams& p, int L, int ws) {
  if (ws >= L || p.window <= 0) return 0;
  if (p.window_kind == SKV_SRC_PAGED) return (L - 1) / p.blk - ws / p.blk + 1;
  return (L - ws + p.blk - 1) / p.blk;
}

// One NW-wave workgroup's attention of (b, g) over items [first, first+count)
// of its list.  The first n_early items are early: described by desc_early
// before the hooks and taken in turn by waves early_wave0 .. NW-1.  The rest
// are late, shared out by LATE: kLateStrided, in turn over all NW waves;
// kLateShared, one at a time to whichever wave needs one next, from the LDS
// counter *late_next (which starts at 0; the split then depends on timing,
// so fp32 sums vary in their last bits from run to run).  Late items are
// described by desc_late, in a wave only once late_ready() has returned in
// it (late_ready waits until late descriptors can be formed).  A wave works through its early items, then its late ones;
// lane j of the wave holds the descriptor of the wave's j-th item, so a wave
// takes at most 64 statically assigned items.  The descriptor functions are
// called for the lanes past a wave's items with its last item of that kind,
// and never for an item outside the list.  pre(issue_first) runs once the
// query loads are issued and must call issue_first() exactly once, which
// issues the loads of the wave's first item if that item is early.  With
// PAD_FIRST a wave without one issues the same loads from row 0 of its
// source, so every path has the same count of loads in flight; without it
// such a wave issues nothing and reaches post() at once.  post() runs after
// pre (both hooks run in every thread).  WROW (fp8 only): the window source
// is a window buffer whose every row has its own K and V scale (p.wks / p.wvs
// [B][Hkv][W], row r of the pair at (b * Hkv + g) * W + r); each token's
// logit and probability then take its row's scales.  Leaves each wave's
// unnormalised O rows, running max and sum in its LDS combine region.
constexpr int kLateStrided = 0, kLateShared = 1;

template <int KV, int D, int BLK, int NW, int NTOK = 1, bool PAD_FIRST = true, int LATE = kLateStrided,
          bool WROW = false, class EarlyDescFn, class LateDescFn, class LateReadyFn, class PreFn, class PostFn>
__device__ __forceinline__ void attend_items(const AttnParams& p, char* smem, int b, int g, int first,
                                             int count, int n_early, int early_wave0, EarlyDescFn desc_early,
                                             LateDescFn desc_late, LateReadyFn late_ready, PreFn pre,
                                             PostFn post, int* late_next = nullptr) {
  using C = AttnCfg<KV, D, BLK>;
  const int lane = lane_id(), w = wave_id();
  const int n = lane & 15;   // C/B column, A row
  const int kg = lane >> 4;  // row group / k group
  const int G = p.G;
  const int L = p.seq_lens[b];
  const int ws = L - p.window > 0 ? L - p.window : 0;

  // ---- query operand.  One token: column n holds head n, and for bf16/fp8
  // head n-G again in columns G..2G-1, which carry the low half of P.  Two
  // tokens (co-batched): column n holds token n/G, head n%G, and the low half
  // of P takes a second MFMA.
  constexpr bool LO_PACKED = NTOK == 1 && KV != KV_F32;
  const int nq = NTOK * G;                    // query columns
  const int ncols = LO_PACKED ? 2 * G : nq;   // columns holding a query
  const int qc = n < nq ? n : (n < ncols ? n - G : -1);
  const int tq = qc < 0 ? 0 : qc / G;         // this column's token
  const int hq = qc < 0 ? -1 : qc % G;
  uint4 qop[KV == KV_F32 ? 1 : C::KS];
  float qopf[KV == KV_F32 ? C::KS : 1];
  {
    const int64_t qrow = (((int64_t)b * p.T + tq) * p.Hq + (int64_t)g * G + (hq < 0 ? 0 : hq)) * D;
    if constexpr (KV == KV_F32) {
      // k-step s of group kg is element 16(s/4) + 4kg + s%4 of the row
      const float* qp = static_cast<const float*>(p.q) + qrow;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) qopf[s] = hq < 0 ? 0.f : qp[16 * (s / 4) + 4 * kg + (s % 4)];
    } else {
      // bf16: k-step s of group kg is elements 32s + 8kg .. +7;
      // fp8: k-step s is elements 64(s/2) + 16kg + 8(s%2) .. +7
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + qrow;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const int off = KV == KV_BF16 ? 32 * s + 8 * kg : 64 * (s / 2) + 16 * kg + 8 * (s % 2);
        qop[s] = hq < 0 ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4*>(qp + off);
      }
    }
  }

  // this wave's items: early ones strided over waves early_wave0 .. NW-1,
  // then its late ones
  constexpr bool DYN_LATE = LATE == kLateShared;
  const int ew = NW - early_wave0, we = w - early_wave0;
  const int n_late = count - n_early;
  const int my_early = (we >= 0 && n_early > we) ? (n_early - we + ew - 1) / ew : 0;
  const int my_late = DYN_LATE ? 0 : (n_late > w ? (n_late - w + NW - 1) / NW : 0);
  int my_items = my_early + my_late;   // with kLateShared it grows as late items are taken
  // lane j describes this wave's item j; early and late descriptors stay in
  // separate registers, so reading an early item never waits for the loads
  // behind a late one
  ItemDesc d_early{0, 0, 0}, d_late{0, 0, 0};
  if (my_early > 0) d_early = desc_early(first + we + ew * min(lane, my_early - 1));
  auto describe_late = [&] {
    late_ready();
    d_late = desc_late(first + n_early + w + NW * min(max(lane - my_early, 0), my_late - 1));
  };

  const char* kbase_s = static_cast<const char*>(p.sk);
  const char* vbase_s = static_cast<const char*>(p.sv);
  const char* kbase_w = static_cast<const char*>(p.wk);
  const char* vbase_w = static_cast<const char*>(p.wv);

  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  char* vt = smem + w * C::PER_WAVE;
  uint4 kr[C::NT][C::GRAN];
  uint4 vr[C::NV];
  int pos0 = 0, skip = 0;
  float ksc = 1.f, vsc = 1.f;
  // WROW: the K and V scales of the tokens this lane's logits belong to
  // (token 16 * tile + 4 * kg + r of the slice is element r of tile)
  constexpr int NWS = WROW ? C::NT : 1;
  f32x4_t ksw[NWS], vsw[NWS];
#pragma unroll
  for (int t = 0; t < NWS; ++t) ksw[t] = vsw[t] = f32x4_t{1.f, 1.f, 1.f, 1.f};

  // Issue the loads of the slice `sub` of `row` (pos0 already set).
  auto issue = [&](int row, int sub) {
    skip = sub >> 8;
    sub &= 0xff;
    // element offset of the slice, and its fp8 scales, from the source kind
    const bool win = pos0 < 0;
    const int kind = win ? p.window_kind : p.sparse_kind;
    int64_t off;
    if (kind == SKV_SRC_PAGED) off = (int64_t)row * p.stride_block + (int64_t)g * p.stride_head;
    else if (kind == SKV_SRC_STAGED) off = (int64_t)row * BLK * D;
    else off = (int64_t)row * D;
    off += (int64_t)sub * C::TB * D;
    if constexpr (KV == KV_FP8) {
      // paged: per (block, head) scales; staged: per slot; window buffer: per row (WROW)
      if (kind != SKV_SRC_WINDOW) {
        const int64_t si = kind == SKV_SRC_PAGED ? (int64_t)row * p.Hkv + g : row;
        ksc = (win ? p.wks : p.sks)[si];
        vsc = (win ? p.wvs : p.svs)[si];
      } else if constexpr (WROW) {
        const int64_t r0 = (int64_t)row + sub * C::TB;   // the slice's first row of the window buffer
#pragma unroll
        for (int tile = 0; tile < NWS; ++tile) {
          ksw[tile] = *reinterpret_cast<const f32x4_t*>(p.wks + r0 + 16 * tile + 4 * kg);
          vsw[tile] = *reinterpret_cast<const f32x4_t*>(p.wvs + r0 + 16 * tile + 4 * kg);
        }
      }
    }
    const char* kb = (win ? kbase_w : kbase_s) + off * C::ES;
    const char* vb = (win ? vbase_w : vbase_s) + off * C::ES;
#pragma unroll
    for (int tile = 0; tile < C::NT; ++tile) {
      const char* krow = kb + (16 * tile + n) * (D * C::ES) + 16 * kg;
#pragma unroll
      for (int q = 0; q < C::GRAN; ++q) kr[tile][q] = load_stream16(krow + 64 * q);
    }
#pragma unroll
    for (int i = 0; i < C::NV; ++i) vr[i] = load_stream16(vb + 16 * (lane + kWave * i));
  };
  // Issue the loads of the wave's item j (descriptor broadcast from lane j;
  // scalar selects between the early and late descriptors).
  auto load_item = [&](int j) {
    const bool e = j < my_early;
    const int re = __builtin_amdgcn_readlane(d_early.row, j), rl = __builtin_amdgcn_readlane(d_late.row, j);
    const int pe = __builtin_amdgcn_readlane(d_early.pos0, j), pl = __builtin_amdgcn_readlane(d_late.pos0, j);
    const int se = __builtin_amdgcn_readlane(d_early.sub, j), sl = __builtin_amdgcn_readlane(d_late.sub, j);
    pos0 = e ? pe : pl;
    issue(e ? re : rl, e ? se : sl);
  };

  const bool first_early = my_early > 0;
  pre([&] {
    const int r0 = __builtin_amdgcn_readlane(d_early.row, 0);
    const int s0 = __builtin_amdgcn_readlane(d_early.sub, 0);
    const int p0 = __builtin_amdgcn_readlane(d_early.pos0, 0);
    if (PAD_FIRST || first_early) {
      pos0 = first_early ? p0 : 0;
      issue(first_early ? r0 : 0, first_early ? s0 : 0);
    }
  });
  // DYN_LATE: take the next late item and issue its loads; false when none is left
  bool late_open = false;
  auto take_late = [&]() -> bool {
    if (!late_open) {
      late_ready();
      late_open = true;
    }
    int v = 0;
    if (lane == 0) v = atomicAdd(late_next, 1);
    v = __builtin_amdgcn_readfirstlane(v);
    if (v >= n_late) return false;
    const ItemDesc d = desc_late(first + n_early + v);
    pos0 = __builtin_amdgcn_readfirstlane(d.pos0);
    issue(__builtin_amdgcn_readfirstlane(d.row), __builtin_amdgcn_readfirstlane(d.sub));
    return true;
  };
  post();
  if constexpr (DYN_LATE) {
    if (!first_early && take_late()) my_items = 1;
  } else if (!first_early && my_late > 0) {
    describe_late();
    load_item(0);
  }

  for (int j = 0; j < my_items; ++j) {
    const bool win = pos0 < 0;
    const int p0 = pos0 & 0x7fffffff;
    const int lo = win ? ws : 0;
    const int hi = win ? L : ws;
    const float ks_cur = ksc, vs_cur = vsc;
    // per-row scales of a window-buffer slice (WROW), else the item's scales
    const bool rows_scaled = WROW && win;
    f32x4_t ksw_cur[NWS], vsw_cur[NWS];
#pragma unroll
    for (int t = 0; t < NWS; ++t) {
      ksw_cur[t] = ksw[t];
      vsw_cur[t] = vsw[t];
    }
    // a co-batched item that one token did not select is masked in that token's columns
    const bool col_ok = NTOK == 1 || !((skip >> tq) & 1);

    // ---- S^T = K Q^T
    f32x4_t st[C::NT];
#pragma unroll
    for (int tile = 0; tile < C::NT; ++tile) {
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (KV == KV_BF16) {
#pragma unroll
        for (int q = 0; q < C::GRAN; ++q) acc = mfma_bf16(kr[tile][q], qop[q], acc);
      } else if constexpr (KV == KV_FP8) {
#pragma unroll
        for (int q = 0; q < C::GRAN; ++q) {
          uint4 lo16, hi16;
          fp8x16_to_bf16x16(kr[tile][q], lo16, hi16);
          acc = mfma_bf16(lo16, qop[2 * q], acc);
          acc = mfma_bf16(hi16, qop[2 * q + 1], acc);
        }
      } else {
#pragma unroll
        for (int q = 0; q < C::GRAN; ++q) {
          acc = mfma_f32(__uint_as_float(kr[tile][q].x), qopf[4 * q + 0], acc);
          acc = mfma_f32(__uint_as_float(kr[tile][q].y), qopf[4 * q + 1], acc);
          acc = mfma_f32(__uint_as_float(kr[tile][q].z), qopf[4 * q + 2], acc);
          acc = mfma_f32(__uint_as_float(kr[tile][q].w), qopf[4 * q + 3], acc);
        }
      }
      st[tile] = acc;
    }

    // ---- V -> LDS (token-major rows; rows outside [lo, hi) become zero)
    const bool partial = p0 < lo || p0 + C::TB > hi;
#pragma unroll
    for (int i = 0; i < C::NV; ++i) {
      const int off = 16 * (lane + kWave * i);
      const int row = off / (D * C::ES);
      const int col = off % (D * C::ES);
      const bool ok = !partial || (p0 + row >= lo && p0 + row < hi);
      if constexpr (KV == KV_FP8) {
        uint4 a, c;
        fp8x16_to_bf16x16(vr[i], a, c);
        if (!ok) a = c = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(vt + row * C::VROW + 2 * col) = a;
        *reinterpret_cast<uint4*>(vt + row * C::VROW + 2 * col + 16) = c;
      } else {
        uint4 val = vr[i];
        if (partial && !ok) val = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(vt + row * C::VROW + col) = val;
      }
    }

    // ---- prefetch the next item while this one finishes
    if constexpr (DYN_LATE) {
      if (j + 1 < my_early) load_item(j + 1);
      else if (take_late()) ++my_items;
    } else if (j + 1 < my_items) {
      if (j + 1 == my_early) describe_late();
      load_item(j + 1);
    }

    // ---- online softmax (log2 domain)
    const float sc = p.qk_scale * ks_cur;
    float bm = -INFINITY;
#pragma unroll
    for (int tile = 0; tile < C::NT; ++tile)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = p0 + 16 * tile + 4 * kg + r;
        const bool in_range = pos >= lo && pos < hi && col_ok;
        float z = st[tile][r] * (rows_scaled ? p.qk_scale * ksw_cur[tile < NWS ? tile : 0][r] : sc);
        z = in_range ? z : -INFINITY;
        // a window-buffer row outside the window may hold any scale
        if constexpr (WROW) vsw_cur[tile < NWS ? tile : 0][r] = in_range ? vsw_cur[tile < NWS ? tile : 0][r] : 0.f;
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
        const int col = row < ncols ? (row < nq ? row : row - G) : 0;
        const float a = shfl_f(alpha, col);
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
          const float a = n < nq ? st[tile][r] : 0.f;
          const char* vrow = vt + (16 * tile + 4 * kg + r) * C::VROW + 4 * n;
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
            o[dt] = mfma_f32(a, *reinterpret_cast<const float*>(vrow + 64 * dt), o[dt]);
        }
    } else {
      // one MFMA per 32-token half of the item (two tiles)
      constexpr int NH = (C::NT + 1) / 2;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        // P operand: element e of lane (n, kg) is token 4kg + e%4 of tile 2hh + e/4
        uint32_t pw[4], plo[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          constexpr int NT = C::NT;
          const int t0 = 2 * hh + (2 * e2) / 4;
          const int tc = t0 < NT ? t0 : NT - 1;
          f32x2_t pv = {t0 < NT ? st[tc][(2 * e2) % 4] : 0.f, t0 < NT ? st[tc][(2 * e2 + 1) % 4] : 0.f};
          if constexpr (KV == KV_FP8) {
            if (rows_scaled) {
              const int tw = tc < NWS ? tc : 0;
              pv.x *= vsw_cur[tw][(2 * e2) % 4];
              pv.y *= vsw_cur[tw][(2 * e2 + 1) % 4];
            } else {
              pv *= vs_cur;
            }
          }
          const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(pv, bf16x2_t));
          const f32x2_t rest = {pv.x - bf16_lo(hw), pv.y - bf16_hi(hw)};
          const uint32_t lw = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, bf16x2_t));
          pw[e2] = n < nq ? hw : (n < ncols ? lw : 0u);
          plo[e2] = n < nq ? lw : 0u;
        }
        const uint4 aop = make_uint4(pw[0], pw[1], pw[2], pw[3]);
        const uint4 aop_lo = make_uint4(plo[0], plo[1], plo[2], plo[3]);
        // B operand: lane r of row group kg reads row 32hh + 4kg + r/4 (and +16),
        // columns 16dt + 4(r%4) .. +3; the transposing read hands lane n column
        // 16dt + n of those four rows, i.e. tokens 4kg .. 4kg+3 of each tile.
        const char* tbase = vt + (32 * hh + 4 * kg + (n >> 2)) * C::VROW + 8 * (n & 3);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(tbase + 32 * dt));
          i16x4_t hi4 = i16x4_t{0, 0, 0, 0};
          if (C::NT > 2 * hh + 1)
            hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t*)(tbase + 16 * C::VROW + 32 * dt));
          const uint2 l2 = __builtin_bit_cast(uint2, lo4);
          const uint2 h2 = __builtin_bit_cast(uint2, hi4);
          const uint4 bop = make_uint4(l2.x, l2.y, h2.x, h2.y);
          o[dt] = mfma_bf16(aop, bop, o[dt]);
          if constexpr (!LO_PACKED) o[dt] = mfma_bf16(aop_lo, bop, o[dt]);
        }
      }
    }
    wave_lds_sync();
  }

  // ---- combine the waves in LDS
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
}

// Combine the NW waves' regions into the workgroup's partial for split
// `split` of n_splits; a single split writes the output directly, otherwise
// the last split of (b, g) to arrive merges all of them.
// With NTOK query tokens the rows are (token, head) pairs and the output row
// of token t, head h is (b, t, gG + h) of out [B][NTOK][Hq][d].
template <int KV, int D, int BLK, int NW, int NTOK = 1>
__device__ __forceinline__ void attend_finish(const AttnParams& p, char* smem, int b, int g, int split,
                                              int n_splits, int* s_last) {
  using C = AttnCfg<KV, D, BLK>;
  constexpr int NTH = NW * kWave;
  constexpr bool LO_PACKED = NTOK == 1 && KV != KV_F32;
  const int G = p.G;
  const int NQ = NTOK * G;
  const int64_t pair = (int64_t)b * p.Hkv + g;
  auto out_row = [&](int c) { return ((int64_t)b * NTOK + c / G) * p.Hq + (int64_t)g * G + c % G; };
  const Handoff<float> part = p.partials + (pair * n_splits + split) * NQ * (D + 2);
  for (int idx = threadIdx.x; idx < NQ * D; idx += NTH) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww)
      M = fmaxf(M, reinterpret_cast<const float*>(smem + ww * C::PER_WAVE)[16 * D + h]);
    float O = 0.f, Ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float* comb = reinterpret_cast<const float*>(smem + ww * C::PER_WAVE);
        const float mw = comb[16 * D + h];
        if (mw == -INFINITY) continue;
        const float f = exp2f(mw - M);
        float ov = comb[h * D + d];
        if constexpr (LO_PACKED) ov += comb[(G + h) * D + d];
        O += f * ov;
        Ls += f * comb[16 * D + 16 + h];
      }
    }
    if (n_splits == 1) {
      // a single split is the whole attention of (b, g): write the result directly
      const int64_t bh = out_row(h);
      p.out[bh * D + d] = M == -INFINITY ? 0.f : O / Ls;
      if (d == 0 && p.lse) p.lse[bh] = M == -INFINITY ? -INFINITY : (M + log2f(Ls)) * kLn2;
      continue;
    }
    part.put(h * (D + 2) + 2 + d, O);
    if (d == 0) {
      part.put(h * (D + 2), M);
      part.put(h * (D + 2) + 1, Ls);
    }
  }
  if (n_splits == 1) return;

  // ---- the last split of (b, g) merges every split
  if (!arrive_last(p.counters + pair, (unsigned)n_splits, s_last)) return;
  // each thread merges its outputs over the splits online, reading 8 splits'
  // (max, sum, output) per round of loads: one round for up to 8 splits, and
  // no LDS whatever the split count
  const Handoff<float> pb = p.partials + pair * n_splits * NQ * (D + 2);
  // OU outputs per thread per round, so their loads are in flight together
  // (two where the outputs outnumber the threads)
  auto merge = [&](auto ou) {
    constexpr int OU = decltype(ou)::value;
    for (int idx0 = threadIdx.x; idx0 < NQ * D; idx0 += OU * NTH) {
      float M[OU], Ls[OU], acc[OU];
#pragma unroll
      for (int o = 0; o < OU; ++o) {
        M[o] = -INFINITY;
        Ls[o] = acc[o] = 0.f;
      }
      constexpr int SB = 8;
      for (int s0 = 0; s0 < n_splits; s0 += SB) {
        float mv[OU][SB], lv[OU][SB], ov[OU][SB];
#pragma unroll
        for (int o = 0; o < OU; ++o) {
          const int idx = idx0 + o * NTH;
          const int ic = idx < NQ * D ? idx : idx0;
          const int h = ic / D, d = ic % D;
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            const bool in = s0 + u < n_splits;
            const Handoff<float> ps = pb + ((int64_t)(in ? s0 + u : s0) * NQ + h) * (D + 2);
            mv[o][u] = ps.get(0);
            lv[o][u] = ps.get(1);
            ov[o][u] = ps.get(2 + d);
            if (!in) mv[o][u] = -INFINITY;
          }
        }
#pragma unroll
        for (int o = 0; o < OU; ++o) {
          float Mc = M[o];
#pragma unroll
          for (int u = 0; u < SB; ++u) Mc = fmaxf(Mc, mv[o][u]);
          if (Mc == -INFINITY) continue;
          const float r = M[o] == -INFINITY ? 0.f : exp2f(M[o] - Mc);
          Ls[o] *= r;
          acc[o] *= r;
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            if (mv[o][u] == -INFINITY) continue;
            const float f = exp2f(mv[o][u] - Mc);
            Ls[o] += f * lv[o][u];
            acc[o] += f * ov[o][u];
          }
          M[o] = Mc;
        }
      }
#pragma unroll
      for (int o = 0; o < OU; ++o) {
        const int idx = idx0 + o * NTH;
        if (idx >= NQ * D) continue;
        const int h = idx / D, d = idx % D;
        const int64_t bh = out_row(h);
        p.out[bh * D + d] = M[o] == -INFINITY ? 0.f : acc[o] / Ls[o];
        if (d == 0 && p.lse) p.lse[bh] = M[o] == -INFINITY ? -INFINITY : (M[o] + log2f(Ls[o])) * kLn2;
      }
    }
  };
  if (NQ * D > NTH) merge(std::integral_constant<int, 2>{});
  else merge(std::integral_constant<int, 1>{});
}

}  // namespace skv
