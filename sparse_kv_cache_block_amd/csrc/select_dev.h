// select_dev.h -- device code of landmark scoring and per-KV-head top-k
// block selection, shared by the stand-alone kernels and the single-launch
// decode step.
//
// Scoring (DualDecoder review, core claim and axiom ledger item 1: the
// retrieval index follows from the query and the landmarks resident on the
// GPU): score(b,t,g,j) = qbar(b,t,g) . landmark(b,g,j), where qbar is the sum
// of the G query heads of KV head g.  Summing the heads first turns the
// group's G dot products into one, so scoring is a streaming gemv over the
// landmarks: each landmark row is read once with 16-byte loads (16 lanes per
// 256-byte bf16 row) and serves both query tokens of a dual-query step.
//
// Selection (PulseInfer article, section 2: per-head sparse selection;
// DualDecoder ledger: a budget of k blocks): an LDS radix select on
// order-preserving 32-bit keys (four 8-bit passes) finds the k-th largest key;
// blocks above it are kept, blocks equal to it are kept in ascending id order
// until k are chosen (ties to the lowest id), and the chosen ids are written
// in ascending order after one block-wide scan.  When a pair's scoring rows
// are split over several workgroups, each may first keep its own top k (a
// block of the pair's top k is always among its chunk's top k under the same
// order) and the last to finish selects among those candidates
// (select_scored).
//
// NT is the workgroup size.  PUB selects device-scope atomic stores for the
// selection results, for readers in other workgroups of the same launch.
// Workgroup barriers here hand off LDS only (lds_barrier), so global loads a
// caller issued before a selection stay in flight through it.
#pragma once

#include "skv_device.h"
#include "skv_internal.h"

namespace skv {

// Inclusive prefix sum across the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum over the NT threads of a workgroup (one barrier; the
// caller alternates `lds_w` between two buffers on consecutive calls).
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds_w, uint32_t& total) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id(), w = wave_id();
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == kWave - 1) lds_w[w] = x;
  lds_barrier();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t t = lds_w[i];
    base += (i < w) ? t : 0u;
    tot += t;
  }
  total = tot;
  return base + x - v;
}

// Where a selection of k' = clamp(min(k, n), 0, k_max) of n keys cuts: every
// key above thresh is chosen, and the first take_eq keys equal to it in
// position order (take_all: every key).
struct SelectCut {
  uint32_t thresh, take_eq;
  int kk;
  int take_all;
};

template <int NT>
struct TopkShared {
  uint32_t hist[2][256];
  union {
    uint32_t hist1[2][256];   // the second token's, when two tokens select side by side (block_select_two)
    SelectCut cut[2];         // the cuts wave_threshold hands to block_emit (never beside block_select_two)
  };
  uint32_t scan_w[2][NT / kWave];
  uint32_t ov_w[NT / kWave];          // list_overlap's per-wave hit counts
  uint32_t digit, above, exact;
  uint32_t digit2[2], above2[2], exact2[2];
};

template <bool PUB>
__device__ __forceinline__ void put_i32(int32_t* p, int32_t v) {
  if constexpr (PUB) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool PUB>
__device__ __forceinline__ void put_f32(float* p, float v) {
  if constexpr (PUB) publish_f32(p, v);
  else *p = v;
}

// Select the k largest of keys[0..n) (ties to the lowest index).  Writes the
// chosen indices in ascending order to lds_out[0..k') and -1 to
// lds_out[k'..k_max), and the same to out unless it is null.  Returns
// k' = clamp(min(k, n), 0, k_max).  hist0, when given, is the histogram of the
// keys' top bytes (built while the keys were written); it replaces the first
// pass's counting.
//
// Radix select on 8-bit digits, most significant first: each pass builds the
// histogram of the digit among the keys that match the known prefix, one wave
// finds the digit holding the k'-th largest key, and after four passes that
// key T is known exactly.  Keys above T are all kept; keys equal to T are kept
// in ascending index order until k' are chosen.  A pass whose boundary digit
// holds exactly the keys still needed ends the search early: the selection is
// then every key at or above that prefix.
template <int NT, bool PUB>
__device__ __forceinline__ int block_select(const uint32_t* keys, int n, int k, int k_max, int32_t* out,
                                            int32_t* lds_out, TopkShared<NT>& sh,
                                            const uint32_t* hist0 = nullptr) {
  static_assert(NT >= 256, "the histogram is cleared by the first 256 threads");
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  int kk = k < n ? k : n;
  if (kk > k_max) kk = k_max;  // the output row holds k_max entries
  if (kk < 0) kk = 0;
  const bool take_all = kk >= n;
  uint32_t thresh = 0, take_eq = 0;
  if (!take_all && kk > 0) {
    uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)kk;
    bool at_or_above = false;
    if (!hist0) {
      if (tid < 256) sh.hist[0][tid] = 0;
      lds_barrier();
    }
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t* hist = sh.hist[pass & 1];
      if (pass == 0 && hist0) {
        hist = hist0;
      } else {
        for (int j = tid; j < n; j += NT) {
          const uint32_t key = keys[j];
          if ((key & pmask) == prefix) atomicAdd(&sh.hist[pass & 1][(key >> shift) & 255u], 1u);
        }
        lds_barrier();
      }
      if (w == 0) {
        // lane l owns digits 255-4l .. 252-4l (descending)
        uint32_t c[4], lsum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c[i] = hist[255 - 4 * lane - i];
          lsum += c[i];
        }
        uint32_t above = wave_inclusive_scan(lsum) - lsum;  // keys in higher digits
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (above < remaining && above + c[i] >= remaining) {
            sh.digit = 255u - 4 * lane - i;
            sh.above = above;
            sh.exact = above + c[i] == remaining;
          }
          above += c[i];
        }
      } else if (w == 1) {
        // meanwhile wave 1 clears the other histogram for the next pass
        for (int t = lane; t < 256; t += kWave) sh.hist[(pass + 1) & 1][t] = 0;
      }
      lds_barrier();
      prefix |= sh.digit << shift;
      pmask |= 255u << shift;
      remaining -= sh.above;
      if (sh.exact && prefix != 0u) {   // the whole boundary bin is taken
        at_or_above = true;
        break;
      }
    }
    thresh = at_or_above ? prefix - 1u : prefix;
    take_eq = at_or_above ? 0u : remaining;
  }
  // Emit in ascending index order: thread tid owns indices [j0, j1).
  const int per = (n + NT - 1) / NT;
  const int j0 = tid * per;
  const int j1 = min(n, j0 + per);
  uint32_t gt = 0, eq = 0;
  if (!take_all && kk > 0)
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = keys[j];
      gt += key > thresh;
      eq += key == thresh;
    }
  uint32_t tot;
  const uint32_t ex = block_exclusive_scan<NT>((gt << 16) | eq, sh.scan_w[0], tot);
  if (take_all) {
    for (int j = j0; j < j1; ++j) {
      if (out) put_i32<PUB>(out + j, j);
      lds_out[j] = j;
    }
  } else if (kk > 0) {
    const uint32_t gt_before = ex >> 16, eq_before = ex & 0xffffu;
    int pos = (int)(gt_before + min(eq_before, take_eq));
    uint32_t eq_seen = eq_before;
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = keys[j];
      bool keep = key > thresh;
      if (key == thresh) {
        keep = eq_seen < take_eq;
        ++eq_seen;
      }
      if (keep) {
        if (out) put_i32<PUB>(out + pos, j);
        lds_out[pos] = j;
        ++pos;
      }
    }
  }
  const int nsel = take_all ? n : kk;
  for (int m = nsel + tid; m < k_max; m += NT) {
    if (out) put_i32<PUB>(out + m, -1);
    lds_out[m] = -1;
  }
  lds_barrier();  // scan buffer and lds_out are reused by the caller
  return nsel;
}

// The selections of two query tokens made side by side: threads [0, NT/2)
// count and emit token 0's keys (keys[0..n)), threads [NT/2, NT) token 1's
// (keys[key_stride..]); the two share every barrier, and each half's result
// is exactly block_select's for its token.  Token t's ids go to
// lds_out + t * k_max and, unless out is null, out + t * out_t_stride.
// Returns k' (the same for both tokens).
template <int NT, bool PUB>
__device__ __forceinline__ int block_select_two(const uint32_t* keys, int key_stride, int n, int k, int k_max,
                                                int32_t* out, int64_t out_t_stride, int32_t* lds_out,
                                                TopkShared<NT>& sh) {
  constexpr int NH = NT / 2, NWH = NH / kWave;
  static_assert(NH >= 256 && NWH >= 2, "a half clears 256 bins and has two waves");
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int half = tid / NH, htid = tid % NH, hw = w % NWH;
  const uint32_t* kt = keys + half * key_stride;
  uint32_t(*hist)[256] = half ? sh.hist1 : sh.hist;
  int kk = k < n ? k : n;
  if (kk > k_max) kk = k_max;
  if (kk < 0) kk = 0;
  const bool take_all = kk >= n;
  uint32_t thresh = 0, take_eq = 0;
  if (!take_all && kk > 0) {
    // both tokens' state in every thread, so the pass loop stays uniform
    uint32_t prefix[2] = {0, 0}, pmask[2] = {0, 0}, remaining[2] = {(uint32_t)kk, (uint32_t)kk};
    bool done[2] = {false, false};
    if (htid < 256) hist[0][htid] = 0;
    lds_barrier();
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (!done[half])
        for (int j = htid; j < n; j += NH) {
          const uint32_t key = kt[j];
          if ((key & pmask[half]) == prefix[half]) atomicAdd(&hist[pass & 1][(key >> shift) & 255u], 1u);
        }
      lds_barrier();
      if (hw == 0) {
        if (!done[half]) {
          uint32_t c[4], lsum = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            c[i] = hist[pass & 1][255 - 4 * lane - i];
            lsum += c[i];
          }
          uint32_t above = wave_inclusive_scan(lsum) - lsum;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (above < remaining[half] && above + c[i] >= remaining[half]) {
              sh.digit2[half] = 255u - 4 * lane - i;
              sh.above2[half] = above;
              sh.exact2[half] = above + c[i] == remaining[half];
            }
            above += c[i];
          }
        }
      } else if (hw == 1) {
        for (int t = lane; t < 256; t += kWave) hist[(pass + 1) & 1][t] = 0;
      }
      lds_barrier();
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (done[t]) continue;
        prefix[t] |= sh.digit2[t] << shift;
        pmask[t] |= 255u << shift;
        remaining[t] -= sh.above2[t];
        if (sh.exact2[t] && prefix[t] != 0u) {   // the whole boundary bin is taken
          done[t] = true;
          prefix[t] -= 1u;                     // then every key at or above the old prefix is kept
          remaining[t] = 0;
        }
      }
      if (done[0] && done[1]) break;
    }
    thresh = prefix[half];
    take_eq = remaining[half];
  }
  // emit each token in ascending index order: thread htid of a half owns
  // indices [j0, j1) of its token
  const int per = (n + NH - 1) / NH;
  const int j0 = htid * per;
  const int j1 = min(n, j0 + per);
  uint32_t gt = 0, eq = 0;
  if (!take_all && kk > 0)
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = kt[j];
      gt += key > thresh;
      eq += key == thresh;
    }
  // exclusive scan within the half: wave scans, then the half's earlier waves
  const uint32_t v = (gt << 16) | eq;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == kWave - 1) sh.scan_w[0][w] = x;
  lds_barrier();
  uint32_t ex = x - v;
  for (int i = half * NWH; i < w; ++i) ex += sh.scan_w[0][i];
  int32_t* lo = lds_out + half * k_max;
  int32_t* go = out ? out + half * out_t_stride : nullptr;
  if (take_all) {
    for (int j = j0; j < j1; ++j) {
      if (go) put_i32<PUB>(go + j, j);
      lo[j] = j;
    }
  } else if (kk > 0) {
    const uint32_t gt_before = ex >> 16, eq_before = ex & 0xffffu;
    int pos = (int)(gt_before + min(eq_before, take_eq));
    uint32_t eq_seen = eq_before;
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = kt[j];
      bool keep = key > thresh;
      if (key == thresh) {
        keep = eq_seen < take_eq;
        ++eq_seen;
      }
      if (keep) {
        if (go) put_i32<PUB>(go + pos, j);
        lo[pos] = j;
        ++pos;
      }
    }
  }
  const int nsel = take_all ? n : kk;
  for (int m = nsel + htid; m < k_max; m += NH) {
    if (go) put_i32<PUB>(go + m, -1);
    lo[m] = -1;
  }
  lds_barrier();
  return nsel;
}

// The cut of a selection found by one wave alone (radix passes of 8 bits,
// with no workgroup barrier, so the workgroup's other waves can do other
// work meanwhile).  hist is the wave's own 256-bin LDS histogram; keys and
// hist0 as in block_select.  Keys are read 8 per lane before they are used,
// so a pass waits for LDS about once per 512 keys.  The passes stop as soon as
// the boundary digit's bin is taken whole.
__device__ __forceinline__ SelectCut wave_threshold(const uint32_t* keys, int n, int k, int k_max, uint32_t* hist,
                                                    const uint32_t* hist0 = nullptr) {
  constexpr int U = 8;  // keys per lane per round of LDS reads
  const int lane = lane_id();
  int kk = k < n ? k : n;
  if (kk > k_max) kk = k_max;
  if (kk < 0) kk = 0;
  const bool take_all = kk >= n;
  uint32_t thresh = 0, take_eq = 0;
  if (!take_all && kk > 0) {
    uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)kk;
    bool at_or_above = false;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t* h = hist;
      if (pass == 0 && hist0) {
        h = hist0;
      } else {
        for (int t = lane; t < 256; t += kWave) hist[t] = 0;
        wave_lds_sync();
        for (int j0 = 0; j0 < n; j0 += U * kWave) {
          uint32_t kv[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int j = j0 + u * kWave + lane;
            kv[u] = keys[j < n ? j : 0];
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int j = j0 + u * kWave + lane;
            if (j < n && (kv[u] & pmask) == prefix) atomicAdd(&hist[(kv[u] >> shift) & 255u], 1u);
          }
        }
        wave_lds_sync();
      }
      // lane l owns digits 255-4l .. 252-4l (descending); exactly one lane
      // holds the digit of the k'-th largest matching key
      uint32_t c[4], lsum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = h[255 - 4 * lane - i];
        lsum += c[i];
      }
      uint32_t above = wave_inclusive_scan(lsum) - lsum;
      int my_digit = -1;
      uint32_t my_above = 0, my_exact = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above < remaining && above + c[i] >= remaining) {
          my_digit = 255 - 4 * lane - i;
          my_above = above;
          my_exact = above + c[i] == remaining;
        }
        above += c[i];
      }
      const uint64_t hit = __ballot(my_digit >= 0);
      const int src = hit ? (int)__builtin_ctzll(hit) : 0;
      const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane(my_digit, src);
      prefix |= digit << shift;
      pmask |= 255u << shift;
      remaining -= (uint32_t)__builtin_amdgcn_readlane((int)my_above, src);
      if (__builtin_amdgcn_readlane((int)my_exact, src) && prefix != 0u) {   // the whole boundary bin is taken
        at_or_above = true;
        break;
      }
    }
    thresh = at_or_above ? prefix - 1u : prefix;
    take_eq = at_or_above ? 0u : remaining;
  }
  return SelectCut{thresh, take_eq, kk, take_all ? 1 : 0};
}

// The same selection as block_select made by one wave alone: wave_threshold,
// then the chosen indices emitted in ascending order 64 at a time with
// ballots.  Returns k'.
__device__ __forceinline__ int wave_select(const uint32_t* keys, int n, int k, int k_max, int32_t* lds_out,
                                           uint32_t* hist, const uint32_t* hist0 = nullptr) {
  constexpr int U = 8;
  const int lane = lane_id();
  const uint64_t below = (1ull << lane) - 1ull;  // lanes under this one
  const SelectCut cut = wave_threshold(keys, n, k, k_max, hist, hist0);
  const int kk = cut.kk;
  const bool take_all = cut.take_all != 0;
  const uint32_t thresh = cut.thresh, take_eq = cut.take_eq;
  // emit in ascending index order, 64 keys per ballot: keys above the
  // threshold, and the first take_eq keys equal to it
  if (take_all) {
    for (int j = lane; j < n; j += kWave) lds_out[j] = j;
  } else if (kk > 0) {
    int base = 0;
    uint32_t eq_seen = 0;
    for (int j0 = 0; j0 < n; j0 += U * kWave) {
      uint32_t kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * kWave + lane;
        kv[u] = keys[j < n ? j : 0];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * kWave + lane;
        const bool eq = j < n && kv[u] == thresh;
        const uint64_t meq = __ballot(eq);
        const bool keep = (j < n && kv[u] > thresh) ||
                          (eq && eq_seen + (uint32_t)__builtin_popcountll(meq & below) < take_eq);
        const uint64_t mk = __ballot(keep);
        if (keep) lds_out[base + __builtin_popcountll(mk & below)] = j;
        base += __builtin_popcountll(mk);
        eq_seen += (uint32_t)__builtin_popcountll(meq);
      }
    }
  }
  const int nsel = take_all ? n : kk;
  for (int m = nsel + lane; m < k_max; m += kWave) lds_out[m] = -1;
  wave_lds_sync();
  return nsel;
}

// Exclusive prefix sums over NSEG equal segments of a workgroup's NT threads
// (each segment whole waves; one barrier; the caller alternates `lds_w`
// between two buffers on consecutive calls).
template <int NT, int NSEG>
__device__ __forceinline__ uint32_t segment_exclusive_scan(uint32_t v, uint32_t* lds_w) {
  constexpr int NW = NT / kWave, WPS = NW / NSEG;
  static_assert(NW % NSEG == 0, "segments of whole waves");
  const int lane = lane_id(), w = wave_id();
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == kWave - 1) lds_w[w] = x;
  lds_barrier();
  const int w0 = (w / WPS) * WPS;
  uint32_t base = 0;
#pragma unroll
  for (int i = 0; i < WPS; ++i) base += (w0 + i < w) ? lds_w[w0 + i] : 0u;
  return base + x - v;
}

// The indices the cuts of NTOK tokens choose, emitted in ascending order by
// all NT threads together, NT / NTOK per token: a token's thread i owns the
// contiguous positions [i * r, (i + 1) * r), r = ceil(n / (NT / NTOK)); one
// scan counts the keys equal to the threshold before each thread's run, a
// second the chosen ones.  Token t's keys are at keys + t * key_stride; it
// writes out[t * k_max + 0 .. k') and -1 up to k_max; the caller's barrier
// publishes them.  scan_a and scan_b are two NT / 64-word LDS buffers.
template <int NT, int NTOK>
__device__ __forceinline__ void block_emit(const uint32_t* keys, int key_stride, int n, const SelectCut* cuts,
                                           int k_max, int32_t* out, uint32_t* scan_a, uint32_t* scan_b) {
  constexpr int NH = NT / NTOK;
  const int t = (int)threadIdx.x / NH, i = (int)threadIdx.x % NH;
  const SelectCut cut = cuts[t];
  const uint32_t* kt = keys + t * key_stride;
  int32_t* ot = out + t * k_max;
  const int r = (n + NH - 1) / NH;
  const int j0 = i * r, j1 = min(n, j0 + r);
  const bool cutting = !cut.take_all && cut.kk > 0;
  uint32_t gt = 0, eq = 0;
  if (cutting) {
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = kt[j];
      gt += key > cut.thresh ? 1u : 0u;
      eq += key == cut.thresh ? 1u : 0u;
    }
  }
  // every thread takes part in both scans, whatever its token's cut
  uint32_t eq_before = segment_exclusive_scan<NT, NTOK>(eq, scan_a);
  const uint32_t eq_kept = eq_before >= cut.take_eq ? 0u : min(eq, cut.take_eq - eq_before);
  uint32_t slot = segment_exclusive_scan<NT, NTOK>(gt + eq_kept, scan_b);
  if (cut.take_all) {
    for (int j = j0; j < j1; ++j) ot[j] = j;
  } else if (cutting) {
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = kt[j];
      const bool is_eq = key == cut.thresh;
      if (key > cut.thresh || (is_eq && eq_before < cut.take_eq)) ot[slot++] = j;
      eq_before += is_eq ? 1u : 0u;
    }
  }
  for (int m = cut.kk + i; m < k_max; m += NH) ot[m] = -1;
}

// |a & b| / |a| for two lists of distinct ids in [0, n_ids) in LDS (1 when a
// is empty).  b's ids are marked in an LDS bitmap (`bits`, ceil(n_ids / 32)
// words of scratch), a's ids test it, and the hits are summed with ballots:
// three LDS round trips, no search and no shared counter.
template <int NT>
__device__ __forceinline__ float list_overlap(const int32_t* a, int na, const int32_t* b, int nb, int n_ids,
                                              uint32_t* bits, TopkShared<NT>& sh) {
  constexpr int NW = NT / kWave;
  const int words = (n_ids + 31) / 32;
  for (int i = threadIdx.x; i < words; i += NT) bits[i] = 0u;
  lds_barrier();
  for (int i = threadIdx.x; i < nb; i += NT) {
    const uint32_t x = (uint32_t)b[i];
    atomicOr(&bits[x >> 5], 1u << (x & 31u));
  }
  lds_barrier();
  uint32_t hits = 0;
  for (int i0 = 0; i0 < na; i0 += NT) {
    const int i = i0 + (int)threadIdx.x;
    bool hit = false;
    if (i < na) {
      const uint32_t x = (uint32_t)a[i];
      hit = (bits[x >> 5] >> (x & 31u)) & 1u;
    }
    hits += (uint32_t)__builtin_popcountll(__ballot(hit));
  }
  if (lane_id() == 0) sh.ov_w[wave_id()] = hits;
  lds_barrier();
  uint32_t common = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) common += sh.ov_w[w];
  return na > 0 ? (float)common / (float)na : 1.0f;
}

__device__ __forceinline__ int n_candidates(int L, int window, int blk) {
  const int ws = L - window > 0 ? L - window : 0;
  return (ws + blk - 1) / blk;
}

// Keys of every token's row (T <= 2; token t's at row + t * t_stride) from a
// score array in global memory into LDS (token t's at keys + t * key_stride),
// both rows in the same round of loads.
template <int NT>
__device__ __forceinline__ void load_keys(const float* row, int64_t t_stride, int T, int nc, bool coherent,
                                          uint32_t* keys, int key_stride) {
  constexpr int KB = 8;  // loads in flight per thread and row
  for (int j0 = threadIdx.x; j0 < nc; j0 += KB * NT) {
    float v0[KB], v1[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = j0 + u * NT;
      v0[u] = j < nc ? (coherent ? fetch_f32(row + j) : row[j]) : 0.f;
      v1[u] = (T == 2 && j < nc) ? (coherent ? fetch_f32(row + t_stride + j) : row[t_stride + j]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = j0 + u * NT;
      if (j < nc) {
        keys[j] = score_key(v0[u]);
        if (T == 2) keys[key_stride + j] = score_key(v1[u]);
      }
    }
  }
}

// Selection for one (b, g) and every query token.  Token t's keys are at
// keys + t * key_stride (already there when `scores` is null, else loaded
// from scores + t * t_stride).  Token t's ids go to lds_idx + t * k_max and,
// unless the pointers are null, to the global index and count rows.  Returns
// the overlap of the two tokens' lists (1 with one token), also written to
// overlap_out unless it is null.  hist0, when given, holds each token's
// top-byte key histogram (256 counts per token).
template <int NT, bool PUB>
__device__ __forceinline__ float select_rows(const float* scores, int64_t t_stride, bool coherent,
                                            uint32_t* keys, int key_stride, int nc, int T, int k,
                                            int k_max, int32_t* indices, int64_t idx_t_stride,
                                            int32_t* n_sel, int64_t nsel_t_stride, float* overlap_out,
                                            int32_t* lds_idx, TopkShared<NT>& sh,
                                            const uint32_t* hist0 = nullptr) {
  int ns0 = 0, ns1 = 0;
  // with a row of keys per token, both are loaded and selected side by side;
  // with one shared row (key_stride 0) the tokens go one after the other
  const bool side_by_side = T == 2 && key_stride != 0 && !hist0;
  if (scores && key_stride != 0) {
    load_keys<NT>(scores, t_stride, T, nc, coherent, keys, key_stride);
    lds_barrier();
  }
  if (side_by_side) {
    // the two tokens' selections side by side, one per half of the workgroup
    const int ns = block_select_two<NT, PUB>(keys, key_stride, nc, k, k_max, indices, idx_t_stride, lds_idx, sh);
    if (n_sel && threadIdx.x < 2) put_i32<PUB>(n_sel + threadIdx.x * nsel_t_stride, ns);
    lds_barrier();
    const float ov = list_overlap<NT>(lds_idx, ns, lds_idx + k_max, ns, nc, keys, sh);
    if (overlap_out && threadIdx.x == 0) put_f32<PUB>(overlap_out, ov);
    return ov;
  }
  for (int t = 0; t < T; ++t) {
    uint32_t* kt = keys + t * key_stride;
    if (scores && key_stride == 0) {
      load_keys<NT>(scores + t * t_stride, 0, 1, nc, coherent, kt, 0);
      lds_barrier();
    }
    const int ns = block_select<NT, PUB>(kt, nc, k, k_max, indices ? indices + t * idx_t_stride : nullptr,
                                         lds_idx + t * k_max, sh, hist0 ? hist0 + t * 256 : nullptr);
    if (t == 0) ns0 = ns; else ns1 = ns;
    if (n_sel && threadIdx.x == 0) put_i32<PUB>(n_sel + t * nsel_t_stride, ns);
    lds_barrier();
  }
  float ov = 1.0f;
  if (T == 2) {
    ov = list_overlap<NT>(lds_idx, ns0, lds_idx + k_max, ns1, nc, keys, sh);
    if (overlap_out && threadIdx.x == 0) put_f32<PUB>(overlap_out, ov);
  }
  return ov;
}

// The selection of every token (T <= 2) over keys already in LDS (token t's
// at keys + t * key_stride): positions, ascending, to lds_idx + t * k_max
// (-1 past k'), nothing to global memory.  Returns k'.
template <int NT>
__device__ __forceinline__ int select_lds(const uint32_t* keys, int key_stride, int n, int T, int k, int k_max,
                                          int32_t* lds_idx, TopkShared<NT>& sh) {
  if (T == 2) return block_select_two<NT, false>(keys, key_stride, n, k, k_max, nullptr, 0, lds_idx, sh);
  return block_select<NT, false>(keys, n, k, k_max, nullptr, lds_idx, sh);
}

// Physical block of every selected index (row b of the block table).
template <int NT, bool PUB>
__device__ __forceinline__ void write_phys(const int32_t* lds_idx, int T, int k_max,
                                           const int32_t* table_row, int32_t* phys,
                                           int64_t t_stride) {
  lds_barrier();
  for (int i = threadIdx.x; i < T * k_max; i += NT) {
    const int t = i / k_max, m = i % k_max;
    const int j = lds_idx[i];
    put_i32<PUB>(phys + t * t_stride + m, j >= 0 ? table_row[j] : -1);
  }
}

// The first loads of a scoring workgroup: the G query rows of each token
// (summed into the group query by score_rows) and the first batch of
// landmark rows of chunk c.  The batch's rows are clamped to the pair's
// max_blocks rows, not to its candidates, so its addresses do not wait for
// the sequence's length; rows past the candidates stay inside the landmark
// array and are ignored by score_rows.
template <int UR>
struct ScoreHead {
  uint32_t qraw[8];
  uint4 va[UR];
};

template <int D, bool LM_F32, bool Q_F32, int NT, int UR>
__device__ __forceinline__ void score_head(const ScoreParams& p, int c, int g, int b, ScoreHead<UR>& h) {
  constexpr int NW = NT / kWave;
  constexpr int ES = LM_F32 ? 4 : 2;
  constexpr int LPR = D * ES / 16;
  constexpr int RPW = kWave / LPR;
  constexpr int RPS = RPW * NW;
  const int lane = lane_id(), w = wave_id();
  const int sub = lane % LPR, rw = lane / LPR;
  const int qi = threadIdx.x;
  const bool q_owner = qi < p.T * D;
  {
    const int t = q_owner ? qi / D : 0, d = q_owner ? qi % D : 0;
    const int64_t base = ((int64_t)(b * p.T + t) * p.Hq + (int64_t)g * p.G) * D + d;
    if constexpr (Q_F32) {
      const uint32_t* qp = static_cast<const uint32_t*>(p.q) + base;
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) h.qraw[hh] = qp[(int64_t)min(hh, p.G - 1) * D];
    } else {
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + base;
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) h.qraw[hh] = qp[(int64_t)min(hh, p.G - 1) * D];
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // q loads issue first: waiting on them leaves the batch in flight
  const char* lm = static_cast<const char*>(p.landmarks) +
                   ((int64_t)(b * p.Hkv + g) * p.max_blocks) * D * ES + sub * 16;
  const int row_begin = c * p.rows_per_chunk;
  const int last_row = max(0, min(p.max_blocks, row_begin + p.rows_per_chunk) - 1);
#pragma unroll
  for (int u = 0; u < UR; ++u) {
    const int r = min(row_begin + u * RPS + w * RPW + rw, last_row);
    h.va[u] = load_stream16(lm + (int64_t)r * D * ES);
  }
}

// Landmark scoring of (b, g) rows of chunk c.  Modes: stand-alone scoring
// (scores to global, -inf past the candidates); fused with one chunk per
// (b, g) (scores go straight to the LDS keys for the selection); fused with
// several chunks (scores are published to the workspace for the chunk that
// selects).  Returns false when a fused chunk has no rows.  `smem` holds
// score_lds_bytes().
// LDS_KEYS: the keys go to LDS with each token's top-byte histogram (the
// single-launch step, and the split step's scoring chunks).  head: the query
// and first-batch loads score_head issued for the same (c, g, b), or null
// (then they are issued here).
template <int D, bool LM_F32, bool Q_F32, int NT, int UR, bool LDS_KEYS = false>
__device__ __forceinline__ bool score_rows(const ScoreParams& p, int c, int g, int b, uint32_t* smem,
                                           const ScoreHead<UR>* head = nullptr) {
  constexpr int NW = NT / kWave;
  constexpr int ES = LM_F32 ? 4 : 2;
  constexpr int LPR = D * ES / 16;      // lanes per landmark row
  constexpr int EPL = 16 / ES;          // landmark elements per lane
  constexpr int RPW = kWave / LPR;      // rows per wave per step
  constexpr int RPS = RPW * NW;         // rows per workgroup per step
  static_assert(2 * D <= NT, "the group-summed query needs T * D threads");

  const int T = p.T;
  const int L = p.seq_lens[b];
  const int nc = n_candidates(L, p.window, p.blk);
  const int R = p.rows_per_chunk;
  int row_begin, row_end, nchunks = 1;
  if (LDS_KEYS || p.fused_select) {
    nchunks = max(1, (nc + R - 1) / R);
    if (c >= nchunks) return false;
    row_begin = c * R;
    row_end = min(nc, row_begin + R);
  } else {
    row_begin = c * R;
    row_end = min(p.max_blocks, row_begin + R);
  }
  // fused: the keys stay in LDS when this workgroup selects over them
  const bool in_lds = LDS_KEYS || (p.fused_select && (p.single_chunk || p.two_level));

  float* qbar = reinterpret_cast<float*>(smem);  // [T][D]
  uint32_t* keys = smem + T * D;                 // [T][score_cols]
  // LDS_KEYS: top-byte histogram of each token's keys, after the selected ids
  uint32_t* hist0 = keys + T * p.score_cols + 2 * p.k_max;   // [2][256]

  const int lane = lane_id(), w = wave_id();
  const int sub = lane % LPR, rw = lane / LPR;
  const char* lm = static_cast<const char*>(p.landmarks) +
                   ((int64_t)(b * p.Hkv + g) * p.max_blocks) * D * ES + sub * 16;
  const int steps = (row_end - row_begin + RPS - 1) / RPS;

  // Rows past the range are loaded from the last valid row (and ignored), so
  // the loads carry no branches and all of a batch is in flight together.
  const int last_row = max(row_begin, min(row_end, nc) - 1);
  // Two batches alternate (software pipelining): the next batch's loads are
  // issued before the current one is consumed, so each wave streams while it
  // computes.
  uint4 va[UR], vb[UR];
  auto load_batch = [&](uint4 (&v)[UR], int s0) {
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int r = min(row_begin + (s0 + u) * RPS + w * RPW + rw, last_row);
      v[u] = load_stream16(lm + (int64_t)r * D * ES);
    }
  };
  const bool any_rows = row_end > row_begin && nc > 0;

  // group-summed query: its G loads per element are issued first (they are
  // few), then the first landmark batch, so waiting for the query leaves the
  // landmark loads in flight
  const int qi = threadIdx.x;
  const bool q_owner = qi < T * D;
  uint32_t qraw[8];
  if (head) {
#pragma unroll
    for (int h = 0; h < 8; ++h) qraw[h] = head->qraw[h];
#pragma unroll
    for (int u = 0; u < UR; ++u) va[u] = head->va[u];
  } else {
    ScoreHead<UR> own;
    score_head<D, LM_F32, Q_F32, NT, UR>(p, c, g, b, own);   // always in bounds; ignored without rows
#pragma unroll
    for (int h = 0; h < 8; ++h) qraw[h] = own.qraw[h];
#pragma unroll
    for (int u = 0; u < UR; ++u) va[u] = own.va[u];
  }
  if (q_owner) {
    float sum = 0.f;
#pragma unroll
    for (int h = 0; h < 8; ++h)
      sum += h < p.G ? (Q_F32 ? __uint_as_float(qraw[h]) : __uint_as_float(qraw[h] << 16)) : 0.f;
    qbar[qi] = sum;
  }
  if constexpr (LDS_KEYS) {
    for (int i = threadIdx.x; i < 2 * 256; i += NT) hist0[i] = 0u;
  }
  lds_barrier();
  float qr[2][EPL];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qr[t][e] = (t < T) ? qbar[t * D + sub * EPL + e] : 0.f;

  float* sc = p.scores + ((int64_t)b * T * p.Hkv + g) * p.score_cols;
  const int64_t t_stride = (int64_t)p.Hkv * p.score_cols;

  auto consume = [&](const uint4 (&v)[UR], int s0) {
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int r = row_begin + (s0 + u) * RPS + w * RPW + rw;
      float x[EPL];
      if constexpr (LM_F32) {
        x[0] = __uint_as_float(v[u].x); x[1] = __uint_as_float(v[u].y);
        x[2] = __uint_as_float(v[u].z); x[3] = __uint_as_float(v[u].w);
      } else {
        x[0] = bf16_lo(v[u].x); x[1] = bf16_hi(v[u].x); x[2] = bf16_lo(v[u].y); x[3] = bf16_hi(v[u].y);
        x[4] = bf16_lo(v[u].z); x[5] = bf16_hi(v[u].z); x[6] = bf16_lo(v[u].w); x[7] = bf16_hi(v[u].w);
      }
      float acc[2] = {0.f, 0.f};
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[0] = fmaf(qr[0][e], x[e], acc[0]);
      acc[0] = group_sum<LPR>(acc[0]);
      if (T == 2) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[1] = fmaf(qr[1][e], x[e], acc[1]);
        acc[1] = group_sum<LPR>(acc[1]);
      }
      if (sub == 0 && s0 + u < steps && r < row_end) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (t >= T) break;
          float val = acc[t];
          if (val == 0.0f) val = 0.0f;  // one zero
          if (in_lds) {
            const uint32_t key = score_key(val);
            keys[t * p.score_cols + r] = key;
            if constexpr (LDS_KEYS) atomicAdd(&hist0[t * 256 + (key >> 24)], 1u);
          } else {
            val = (r < nc) ? val : -INFINITY;
            if (p.fused_select) publish_f32(sc + t * t_stride + r, val);
            else sc[t * t_stride + r] = val;
          }
        }
      }
    }
  };
  // Exactly the batches that hold rows are loaded, each issued one batch
  // ahead: the main loop runs while two more batches follow, and the tail
  // (one or two batches) is straight-line code, so every wait before a
  // consume() leaves the next batch in flight and nothing is outstanding at
  // the end.
  const int nb = any_rows ? (steps + UR - 1) / UR : 0;
  int bi = 0;
  for (; bi + 2 < nb; bi += 2) {
    load_batch(vb, (bi + 1) * UR);
    consume(va, bi * UR);
    load_batch(va, (bi + 2) * UR);
    consume(vb, (bi + 1) * UR);
  }
  if (nb - bi == 2) {
    load_batch(vb, (bi + 1) * UR);
    consume(va, bi * UR);
    consume(vb, (bi + 1) * UR);
  } else if (nb - bi == 1) {
    consume(va, bi * UR);
  }

  return true;
}

// The selection of a fused scoring launch, after score_rows of chunk c:
// single chunk -- the keys are in LDS; several chunks -- the last chunk of
// (b, g) to arrive reads the published scores.  Returns true in the
// workgroup that selected.
// nc: the candidates of sequence b, k: its k (both as read by the caller).
// SINGLE: compiled for the single-chunk mode only.
template <int NT, bool PUB, bool SINGLE = false>
__device__ __forceinline__ bool select_scored(const ScoreParams& p, int c, int g, int b, int nc, int k,
                                              uint32_t* smem, TopkShared<NT>& sh, int* s_flag) {
  const int T = p.T;
  const int R = p.rows_per_chunk;
  const int nchunks = max(1, (nc + R - 1) / R);
  uint32_t* keys = smem + T * p.D;
  int32_t* lds_idx = reinterpret_cast<int32_t*>(keys + T * p.score_cols);
  int32_t* idx_out = p.indices + ((int64_t)b * T * p.Hkv + g) * p.k_max;
  int32_t* nsel_out = p.n_sel + (int64_t)b * T * p.Hkv + g;
  float* ov_out = p.overlap ? p.overlap + b * p.Hkv + g : nullptr;
  const bool single = SINGLE || p.single_chunk;
  if (single || !p.two_level) {
    // one chunk: the keys are in LDS; several: the last chunk of (b, g) to
    // arrive reads every published score
    if (single) {
      lds_barrier();
    } else if (!arrive_last(p.counters + b * p.Hkv + g, (unsigned)nchunks, s_flag)) {
      return false;
    }
    const float* sc = single ? nullptr : p.scores + ((int64_t)b * T * p.Hkv + g) * p.score_cols;
    (void)select_rows<NT, PUB>(sc, (int64_t)p.Hkv * p.score_cols, true, keys, p.score_cols, nc, T, k, p.k_max,
                               idx_out, (int64_t)p.Hkv * p.k_max, nsel_out, p.Hkv, ov_out, lds_idx, sh);
  } else {
    // ---- several chunks.  Level 1: the chunk keeps its own top-k' and
    // publishes it as (key, id).  Under the selection's total order (key
    // descending, id ascending) a block among the pair's top k' is among its
    // chunk's top k', so these candidates hold the whole selection.
    const int k_max = p.k_max;
    const int row_begin = c * R;
    const int rows = min(nc, row_begin + R) - row_begin;
    const Handoff<int32_t> cand = p.cand + ((int64_t)b * T * p.Hkv + g) * p.cand_stride;
    const int64_t cand_t = (int64_t)p.Hkv * p.cand_stride;
    lds_barrier();   // the chunk's keys are in LDS
    const int ns1 = select_lds<NT>(keys + row_begin, p.score_cols, rows, T, k, k_max, lds_idx, sh);
    for (int i = threadIdx.x; i < T * ns1; i += NT) {
      const int t = i / ns1, m = i - t * ns1;
      const int pos = lds_idx[t * k_max + m];
      const Handoff<int32_t> ct = cand + t * cand_t + (int64_t)c * 2 * k_max;
      ct.put(m, (int32_t)keys[t * p.score_cols + row_begin + pos]);
      ct.put(k_max + m, row_begin + pos);
    }
    if (!arrive_last(p.counters + b * p.Hkv + g, (unsigned)nchunks, s_flag)) return false;
    // Level 2, in the last chunk to arrive: every chunk's candidates in chunk
    // order, so position order is id order and ties still go to the lowest id.
    int kk = k < k_max ? k : k_max;
    if (kk < 0) kk = 0;
    const int m_full = min(kk, R);                        // candidates of a full chunk
    const int m_last = min(kk, nc - (nchunks - 1) * R);   // of the last chunk
    const int M = (nchunks - 1) * m_full + m_last;
    // Candidate j of a token is slot j - cc * m_full of chunk cc.
    int32_t* ids = reinterpret_cast<int32_t*>(lds_idx + 2 * k_max + 2 * 256);   // [T][score_cols]
    const bool ids_lds = p.cand_ids_lds != 0;
    constexpr int KB = 4;   // candidates per thread whose loads are in flight together
    for (int i0 = threadIdx.x; i0 < T * M; i0 += KB * NT) {
      int32_t kv[KB], iv[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int i = i0 + u * NT;
        const int t = i / M, j = i - t * M;
        const int cc = min(j / max(m_full, 1), nchunks - 1);
        const Handoff<int32_t> ct = cand + t * cand_t + (int64_t)cc * 2 * k_max + (j - cc * m_full);
        kv[u] = i < T * M ? ct.get(0) : 0;
        iv[u] = (ids_lds && i < T * M) ? ct.get(k_max) : 0;
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int i = i0 + u * NT;
        if (i < T * M) {
          const int t = i / M, j = i - t * M;
          keys[t * p.score_cols + j] = (uint32_t)kv[u];
          if (ids_lds) ids[t * p.score_cols + j] = iv[u];
        }
      }
    }
    lds_barrier();
    const int ns = select_lds<NT>(keys, p.score_cols, M, T, k, k_max, lds_idx, sh);
    for (int i = threadIdx.x; i < T * k_max; i += NT) {
      const int t = i / k_max, m = i - t * k_max;
      const int pos = lds_idx[i];
      int32_t id = -1;
      if (pos >= 0) {
        if (ids_lds) {
          id = ids[t * p.score_cols + pos];
        } else {   // the ids did not fit in LDS: read the selected ones back
          const int cc = min(pos / max(m_full, 1), nchunks - 1);
          id = cand.get(t * cand_t + (int64_t)cc * 2 * k_max + k_max + (pos - cc * m_full));
        }
      }
      lds_idx[i] = id;
      put_i32<PUB>(idx_out + t * (int64_t)p.Hkv * k_max + m, id);
    }
    if (threadIdx.x < T) put_i32<PUB>(nsel_out + threadIdx.x * p.Hkv, ns);
    lds_barrier();
    if (T == 2) {
      const float ov = list_overlap<NT>(lds_idx, ns, lds_idx + k_max, ns, nc, keys, sh);
      if (ov_out && threadIdx.x == 0) put_f32<PUB>(ov_out, ov);
    }
  }
  if (p.phys)   // the attention reads the real token's physical blocks only
    write_phys<NT, PUB>(lds_idx, 1, p.k_max, p.block_table + (int64_t)b * p.max_blocks,
                        p.phys + ((int64_t)b * T * p.Hkv + g) * p.k_max, (int64_t)p.Hkv * p.k_max);
  return true;
}

// Scoring of chunk c of (b, g), then (fused) the selection; see score_rows
// and select_scored.
// Split step, scoring launch (cand_only): chunk c of (b, g) scores its rows
// into LDS, counting each token's top-byte key histogram as it goes; wave t
// then finds where token t's top k' of the chunk cuts, all waves emit the
// chosen positions, and the chunk publishes (key, id, physical block) of
// its candidates in dense rows: chunk c's m-th candidate at c * min(k', R) + m,
// since every earlier chunk is full.  The chunk's rows of the block table are
// loaded before the scoring (up to kChunkTableRegs per thread, the rest after
// it) and staged in LDS for the physical blocks.
constexpr int kChunkTableRegs = 2;

template <int D, bool LM_F32, bool Q_F32, int NT, int UR>
__device__ __forceinline__ void chunk_candidates(const ScoreParams& p, int c, int g, int b, uint32_t* smem,
                                                 TopkShared<NT>& sh) {
  const int T = p.T, R = p.rows_per_chunk, k_max = p.k_max;
  const int nc = n_candidates(p.seq_lens[b], p.window, p.blk);
  const int k = p.k_per_seq[b];
  const int row_begin = c * R;
  const int rows = min(nc, row_begin + R) - row_begin;
  const int32_t* table_row = p.block_table + (int64_t)b * p.max_blocks + row_begin;
  int32_t trow[kChunkTableRegs];
#pragma unroll
  for (int i = 0; i < kChunkTableRegs; ++i) {
    const int j = (int)threadIdx.x + NT * i;
    trow[i] = j < rows ? table_row[j] : 0;
  }
  if (!score_rows<D, LM_F32, Q_F32, NT, UR, true>(p, c, g, b, smem)) return;
  uint32_t* keys = smem + T * p.D;
  int32_t* lds_idx = reinterpret_cast<int32_t*>(keys + T * p.score_cols);
  const uint32_t* hist0 = reinterpret_cast<const uint32_t*>(lds_idx + 2 * k_max);
  int32_t* tab = lds_idx + 2 * k_max + 2 * 256;
#pragma unroll
  for (int i = 0; i < kChunkTableRegs; ++i) {
    const int j = (int)threadIdx.x + NT * i;
    if (j < rows) tab[j] = trow[i];
  }
  for (int j = (int)threadIdx.x + NT * kChunkTableRegs; j < rows; j += NT) tab[j] = table_row[j];
  lds_barrier();   // the chunk's keys, their histograms and its table entries are in LDS
  // wave t finds where token t's selection cuts, then every wave emits its
  // run of the chosen positions
  const int w = wave_id();
  if (w < T) {
    const SelectCut cut = wave_threshold(keys + w * p.score_cols + row_begin, rows, k, k_max, sh.hist[w],
                                         hist0 + w * 256);
    if (lane_id() == 0) sh.cut[w] = cut;
  }
  lds_barrier();
  if (T == 2)
    block_emit<NT, 2>(keys + row_begin, p.score_cols, rows, sh.cut, k_max, lds_idx, sh.scan_w[0], sh.scan_w[1]);
  else
    block_emit<NT, 1>(keys + row_begin, p.score_cols, rows, sh.cut, k_max, lds_idx, sh.scan_w[0], sh.scan_w[1]);
  lds_barrier();   // both tokens' chunk selections are in LDS
  // the chunk keeps clamp(min(k, rows), 0, k_max) candidates; the pair's k'
  // is clamp(min(k, nc), 0, k_max)
  int ns1 = min(k, rows), kk = min(k, nc);
  ns1 = max(0, min(ns1, k_max));
  kk = max(0, min(kk, k_max));
  const int at = c * min(kk, R);
  const Handoff<int32_t> cand = p.cand + ((int64_t)b * T * p.Hkv + g) * p.cand_stride;
  const int64_t cand_t = (int64_t)p.Hkv * p.cand_stride;
  for (int i = threadIdx.x; i < T * ns1; i += NT) {
    const int t = i / ns1, m = i - t * ns1;
    const int pos = lds_idx[t * k_max + m];
    const Handoff<int32_t> ct = cand + t * cand_t + at + m;
    ct.put(0, (int32_t)keys[t * p.score_cols + row_begin + pos]);
    ct.put(p.cand_cols, row_begin + pos);
    if (t == 0) ct.put(2 * p.cand_cols, tab[pos]);
  }
}

template <int D, bool LM_F32, bool Q_F32, int NT, int UR, bool PUB>
__device__ __forceinline__ bool score_task(const ScoreParams& p, int c, int g, int b, uint32_t* smem,
                                           TopkShared<NT>& sh, int* s_flag) {
  if (p.cand_only) {
    chunk_candidates<D, LM_F32, Q_F32, NT, UR>(p, c, g, b, smem, sh);
    return false;
  }
  if (!score_rows<D, LM_F32, Q_F32, NT, UR>(p, c, g, b, smem)) return false;
  if (!p.fused_select) return false;
  return select_scored<NT, PUB>(p, c, g, b, n_candidates(p.seq_lens[b], p.window, p.blk), p.k_per_seq[b],
                                smem, sh, s_flag);
}

}  // namespace skv
