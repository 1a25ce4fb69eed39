// Top-K select and kept-index emission (gfx950).
//
// Kept set S = top-K(document scores) ∪ (every non-document token)
// ("TokenGate 与 T2Quant ... 精读", sections 3.1 and 4.1).  Order among document
// tokens: higher score, then lower index.
//
// Prompts of up to 16K tokens: one launch, one 1024-thread workgroup per
// prompt, keys in registers for all passes (thread t owns R = 16 consecutive
// tokens).  At that size the cost is latency, so launches, global atomics and
// fences are avoided.  Longer prompts use the multi-workgroup path below.
//
// Scores become order-preserving 32-bit keys (score_key); the K-th largest
// document key T is found exactly by a three-digit MSB radix select
// (11 + 11 + 10 bits) with LDS histograms (integer atomics: exact); when a
// pass's chosen bin holds exactly the keys still needed, every key of that bin
// is kept and the later passes are skipped (the same set).  Then
// every token is classified in index order: non-document or key > T is kept,
// key == T is kept while fewer than need = K_eff - #{key > T} ties have been
// kept before it.  A block-wide exclusive scan gives every kept token its
// output row, so the output is ascending and identical on every run.
#include <type_traits>

#include "common.h"

namespace tg {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kSub = 4;  // LDS sub-histograms (by wave) to spread atomic contention

struct SelSmem {
  uint32_t hist[kSub][kBins];
  uint32_t wave_tot[2][kWaves];
  uint32_t found_digit;
  uint32_t found_rem;
  uint32_t found_cnt;  // keys in the found bin
};

// Inclusive scan of two counters across the workgroup; returns the exclusive
// prefixes, and the block totals through tot0 / tot1.
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb, uint32_t& tot0,
                                            uint32_t& tot1, SelSmem& sm) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t xa = wave_incl_scan(a), xb = wave_incl_scan(b);
  if (lane == 63) {
    sm.wave_tot[0][wave] = xa;
    sm.wave_tot[1][wave] = xb;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t va = sm.wave_tot[0][w], vb = sm.wave_tot[1][w];
    if (w < wave) {
      pa += va;
      pb += vb;
    }
    ta += va;
    tb += vb;
  }
  __syncthreads();  // wave_tot is reused by the next scan
  ea = pa + xa - a;
  eb = pb + xb - b;
  tot0 = ta;
  tot1 = tb;
}

// Finds the bin (counted from the top) that holds the rem-th largest key.
// Every thread owns BINS/1024 consecutive bins, highest first.
template <uint32_t BINS>
__device__ __forceinline__ void find_digit(SelSmem& sm, uint32_t rem) {
  constexpr uint32_t bins = BINS;
  const int tid = threadIdx.x;
  constexpr uint32_t per = bins / kThreads;  // 2 or 1
  uint32_t c[2] = {0u, 0u};
  uint32_t sum = 0u;
#pragma unroll
  for (uint32_t j = 0; j < per; ++j) {
    const uint32_t b = bins - 1u - (tid * per + j);
    uint32_t v = 0u;
#pragma unroll
    for (int s = 0; s < kSub; ++s) v += sm.hist[s][b];
    c[j] = v;
    sum += v;
  }
  uint32_t before, unused, t0, t1;
  block_scan2(sum, 0u, before, unused, t0, t1, sm);
  if (before < rem && rem <= before + sum) {
    uint32_t acc = before;
#pragma unroll
    for (uint32_t j = 0; j < per; ++j) {
      if (acc + c[j] >= rem) {
        sm.found_digit = bins - 1u - (tid * per + j);
        sm.found_rem = rem - acc;
        sm.found_cnt = c[j];
        break;
      }
      acc += c[j];
    }
  }
  __syncthreads();
}

// This thread's R tokens of the prompt as keys, and which of them are document tokens.
template <int R>
__device__ __forceinline__ void load_keys(const float* __restrict__ seg_scores, const tg_segment& seg,
                                          uint32_t (&key)[R], uint32_t& docmask) {
  const int t0 = (int)threadIdx.x * R;
  docmask = 0u;
  float v[R];
  const bool full = t0 + R <= seg.seg_len;
  if (full && ((reinterpret_cast<uintptr_t>(seg_scores + t0) & 15u) == 0)) {
#pragma unroll
    for (int i = 0; i < R; i += 4) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(seg_scores + t0 + i);
      v[i] = q[0];
      v[i + 1] = q[1];
      v[i + 2] = q[2];
      v[i + 3] = q[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) v[i] = (t0 + i < seg.seg_len) ? seg_scores[t0 + i] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int t = t0 + i;
    key[i] = score_key(v[i]);
    if (t >= seg.doc_begin && t < seg.doc_end) docmask |= 1u << i;
  }
}

template <int R>
__global__ __launch_bounds__(kThreads) void select_topk_kernel(const float* __restrict__ scores,
                                                               SegTable segs,
                                                               int32_t* __restrict__ kept_idx) {
  __shared__ SelSmem sm;
  // launched only when every prompt has at most kThreads R tokens (the table entry is clamped to that
  // maximum), so the whole prompt sits in registers: thread t owns tokens R t .. R t + R - 1
  const tg_segment seg = segs.at_uniform(blockIdx.x);
  if (seg.seg_len <= 0) return;
  const int tid = threadIdx.x;
  const int sub = (tid >> 6) & (kSub - 1);
  const float* ss = scores + seg.seg_start;
  const int n_doc = seg.doc_end - seg.doc_begin;

  uint32_t key[R];
  uint32_t docmask = 0u;
  load_keys<R>(ss, seg, key, docmask);

  uint32_t thresh, need;
  if (seg.k_eff <= 0) {
    thresh = 0xffffffffu;  // no key reaches it: no document kept
    need = 0u;
  } else if (seg.k_eff >= n_doc) {
    thresh = 0u;  // every document kept, NaNs (key 0) included
    need = 0xffffffffu;
  } else {
    uint32_t prefix = 0u;
    uint32_t rem = (uint32_t)seg.k_eff;
    // one radix pass with its digit position as constants; true when the search has ended
    auto pass = [&](auto p_) -> bool {
      constexpr int P = decltype(p_)::value;
      constexpr int shift = P == 0 ? 21 : (P == 1 ? 10 : 0);
      constexpr uint32_t bins = P == 2 ? 1024u : 2048u;
      constexpr uint32_t mask = P == 0 ? 0u : (P == 1 ? 0xffe00000u : 0xfffffc00u);
#pragma unroll
      for (int s = 0; s < kSub; ++s)
#pragma unroll
        for (int i = tid; i < (int)bins; i += kThreads) sm.hist[s][i] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < R; ++i) {
        if (((docmask >> i) & 1u) && (key[i] & mask) == prefix)
          atomicAdd(&sm.hist[sub][(key[i] >> shift) & (bins - 1u)], 1u);
      }
      __syncthreads();
      find_digit<bins>(sm, rem);
      prefix |= sm.found_digit << shift;
      rem = sm.found_rem;
      const bool whole_bin = sm.found_cnt == rem && prefix != 0u;
      __syncthreads();
      if (whole_bin) {
        // every key of the found bin is kept: the same set as the exact
        // threshold (its smallest key) with all its ties, so stop here
        prefix -= 1u;
        rem = 0u;
      }
      return whole_bin;
    };
    if (!pass(std::integral_constant<int, 0>()) && !pass(std::integral_constant<int, 1>()))
      pass(std::integral_constant<int, 2>());
    thresh = prefix;
    need = rem;
  }

  // Emission in index order.
  int32_t* out = kept_idx + seg.kept_start;
  const int t0 = tid * R;
  uint32_t fd = 0u, ft = 0u;  // bit i: token t0 + i kept for sure / tie at T
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int t = t0 + i;
    if (t < seg.seg_len) {
      if (!((docmask >> i) & 1u) || key[i] > thresh)
        fd |= 1u << i;
      else if (key[i] == thresh)
        ft |= 1u << i;
    }
  }
  uint32_t ed, et, td, tt;
  block_scan2((uint32_t)__builtin_popcount(fd), (uint32_t)__builtin_popcount(ft), ed, et, td, tt, sm);
  // Ties before this thread: et; it keeps its first need - et ties (none once the quota is used up).  Kept
  // tokens then land in index order from row ed + min(et, need) on, so the j-th kept token of the thread goes
  // to that row + j: one store per kept token, the loop running over the set bits of the thread's kept mask
  // only.
  uint32_t quota = need > et ? need - et : 0u;
  uint32_t kept = fd;
  for (uint32_t m = ft; m != 0u && quota != 0u; m &= m - 1u, --quota) kept |= m & (0u - m);
  uint32_t pos = ed + (et < need ? et : need);
  for (uint32_t m = kept; m != 0u; m &= m - 1u, ++pos)
    if (pos < (uint32_t)seg.kept_len) out[pos] = seg.seg_start + t0 + __builtin_ctz(m);
}


// ---------------------------------------------------------------------------
// Long prompts (more than 16K tokens): the same algorithm spread over many
// workgroups.  Every prompt is cut into 512-token slices, one 256-thread
// workgroup each (so a 131072-token prompt fills the GPU's 256 CUs).  A radix pass accumulates each slice's LDS histogram into a
// global one with integer atomics (exact, so the result does not depend on
// the order); the next pass's workgroups all re-derive the chosen digit from
// it with the same integer scan, so they agree without exchanging anything.
// A pass whose chosen bin holds exactly the keys still needed ends the search
// early, as in the one-workgroup kernel (the later histogram launches exit at
// once).  After the passes a count kernel records, per slice, how many tokens are
// kept for sure and how many tie the threshold; the emission kernel turns
// the counts of the earlier slices into its output offset and the tie quota
// left for it, then writes its kept indices in index order.
// Workspace: hist [3][n_seg][2048] u32 | state [n_seg][8] u32 | cnt [n_seg][n_slices][2] u32.  state holds, per
// prompt, the search after pass 0 and after pass 1 (prefix, keys still needed, and whether the chosen bin is
// kept whole, which ends the search: then prefix and needed are already the threshold and tie quota), written
// by the first workgroup of the launch that derives it, and the final threshold and tie quota, written by the
// count kernel; each later launch reads them instead of re-deriving the earlier digits from the histograms.

// Slice sizes: 512 tokens while the launch would otherwise have few workgroups (256 for one
// 131072-token prompt), 4096 for large batches, where more slices only add global atomics.
constexpr int kSliceSmall = 512, kSliceLarge = 4096;
constexpr int kMT = 256;
constexpr int kState = 8;            // state words per prompt

struct MultiSmem {
  uint32_t hist[kBins];
  uint32_t wtot[2][4];
  uint32_t digit, rem, cnt;
};

// exclusive prefixes of two counters over the 256 threads; block totals out
__device__ __forceinline__ void scan256(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb, uint32_t& ta,
                                        uint32_t& tb, MultiSmem& sm) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t xa = wave_incl_scan(a), xb = wave_incl_scan(b);
  if (lane == 63) {
    sm.wtot[0][wave] = xa;
    sm.wtot[1][wave] = xb;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  ta = tb = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t va = sm.wtot[0][w], vb = sm.wtot[1][w];
    if (w < wave) {
      pa += va;
      pb += vb;
    }
    ta += va;
    tb += vb;
  }
  __syncthreads();
  ea = pa + xa - a;
  eb = pb + xb - b;
}

// Digit (counted from the top) of the global histogram h that holds the
// rem-th largest key, the rank left inside it, and the bin's key count.
__device__ void multi_find(const uint32_t* __restrict__ h, uint32_t bins, uint32_t& rem, uint32_t& digit,
                           uint32_t& count, MultiSmem& sm) {
  const int tid = threadIdx.x;
  const uint32_t per = bins / kMT;  // 8 or 4 bins per thread, highest first
  uint32_t c[8];
  uint32_t sum = 0u;
  for (uint32_t j = 0; j < per; ++j) {
    c[j] = h[bins - 1u - (tid * per + j)];
    sum += c[j];
  }
  uint32_t before, u0, t0, t1;
  scan256(sum, 0u, before, u0, t0, t1, sm);
  if (before < rem && rem <= before + sum) {
    uint32_t acc = before;
    for (uint32_t j = 0; j < per; ++j) {
      if (acc + c[j] >= rem) {
        sm.digit = bins - 1u - (tid * per + j);
        sm.rem = rem - acc;
        sm.cnt = c[j];
        break;
      }
      acc += c[j];
    }
  }
  __syncthreads();
  digit = sm.digit;
  rem = sm.rem;
  count = sm.cnt;
  __syncthreads();
}

__device__ __forceinline__ void pass_shape(int pass, int& shift, uint32_t& bins, uint32_t& mask) {
  shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
  bins = pass == 2 ? 1024u : 2048u;
  mask = pass == 0 ? 0u : (pass == 1 ? 0xffe00000u : 0xfffffc00u);
}

__global__ __launch_bounds__(256) void select_zero_kernel(uint32_t* __restrict__ w, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) w[i] = 0u;
}

template <int PASS, int SLICE>
__global__ __launch_bounds__(kMT) void select_hist_kernel(const float* __restrict__ scores,
                                                          SegTable segs, int n_seg,
                                                          uint32_t* __restrict__ ws) {
  __shared__ MultiSmem sm;
  const tg_segment seg = segs.at_uniform(blockIdx.y);
  const int n_doc = seg.doc_end - seg.doc_begin;
  if (seg.k_eff <= 0 || seg.k_eff >= n_doc) return;  // no selection to make
  const int t0 = blockIdx.x * SLICE;
  if (t0 >= seg.seg_len) return;
  const int tid = threadIdx.x;
  uint32_t* hs = ws + (int64_t)blockIdx.y * kBins;  // + p * n_seg * kBins for pass p
  uint32_t* state = ws + (int64_t)3 * n_seg * kBins + (int64_t)blockIdx.y * kState;
  uint32_t prefix = 0u, rem = (uint32_t)seg.k_eff;
  if (PASS == 2) {  // the search after pass 0, from the previous launch
    if (state[2] != 0u) return;  // ended at pass 0 (uniform)
    prefix = state[0];
    rem = state[1];
  }
  if (PASS >= 1) {  // digit of pass PASS - 1, from its completed histogram
    constexpr int p = PASS - 1;
    int shift;
    uint32_t bins, mask, digit, count;
    pass_shape(p, shift, bins, mask);
    multi_find(hs + (int64_t)p * n_seg * kBins, bins, rem, digit, count, sm);
    prefix |= digit << shift;
    const bool whole = count == rem && prefix != 0u;  // that bin is kept whole: no later pass needed
    if (blockIdx.x == 0 && tid == 0) {
      state[3 * p] = whole ? prefix - 1u : prefix;
      state[3 * p + 1] = whole ? 0u : rem;
      state[3 * p + 2] = whole ? 1u : 0u;
    }
    if (whole) return;  // uniform
  }
  int shift;
  uint32_t bins, mask;
  pass_shape(PASS, shift, bins, mask);
  for (int i = tid; i < kBins; i += kMT) sm.hist[i] = 0u;
  __syncthreads();
  const float* ss = scores + seg.seg_start;
#pragma unroll
  for (int i = 0; i < SLICE / kMT; ++i) {
    const int t = t0 + i * kMT + tid;  // coalesced
    if (t < seg.seg_len && t >= seg.doc_begin && t < seg.doc_end) {
      const uint32_t key = score_key(ss[t]);
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & (bins - 1u)], 1u);
    }
  }
  __syncthreads();
  uint32_t* hg = hs + (int64_t)PASS * n_seg * kBins;
  for (int b = tid; b < (int)bins; b += kMT) {
    const uint32_t v = sm.hist[b];
    if (v != 0u) atomicAdd(&hg[b], v);
  }
}

// Threshold key T and tie quota `need` of a prompt (as in the one-workgroup kernel).
__device__ void multi_threshold(const tg_segment& seg, int n_seg, const uint32_t* __restrict__ ws, MultiSmem& sm,
                                uint32_t& thresh, uint32_t& need) {
  const int n_doc = seg.doc_end - seg.doc_begin;
  if (seg.k_eff <= 0) {
    thresh = 0xffffffffu;
    need = 0u;
  } else if (seg.k_eff >= n_doc) {
    thresh = 0u;
    need = 0xffffffffu;
  } else {
    const uint32_t* state = ws + (int64_t)3 * n_seg * kBins + (int64_t)blockIdx.y * kState;
    if (state[2] != 0u) {  // ended at pass 0
      thresh = state[0];
      need = state[1];
    } else if (state[5] != 0u) {  // ended at pass 1
      thresh = state[3];
      need = state[4];
    } else {  // the last digit, from pass 2's histogram
      uint32_t prefix = state[3], rem = state[4];
      int shift;
      uint32_t bins, mask, digit, count;
      pass_shape(2, shift, bins, mask);
      multi_find(ws + (int64_t)blockIdx.y * kBins + (int64_t)2 * n_seg * kBins, bins, rem, digit, count, sm);
      prefix |= digit << shift;
      if (count == rem && prefix != 0u) {  // the found bin is kept whole: the same set with all its ties
        prefix -= 1u;
        rem = 0u;
      }
      thresh = prefix;
      need = rem;
    }
  }
}

// Per slice: tokens kept for sure (non-document or key > T) and ties at T.
template <int SLICE>
__global__ __launch_bounds__(kMT) void select_count_kernel(const float* __restrict__ scores,
                                                           SegTable segs, int n_seg,
                                                           int n_slices, uint32_t* __restrict__ ws) {
  __shared__ MultiSmem sm;
  const tg_segment seg = segs.at_uniform(blockIdx.y);
  const int t0 = blockIdx.x * SLICE;
  if (t0 >= seg.seg_len) return;
  uint32_t thresh, need;
  multi_threshold(seg, n_seg, ws, sm, thresh, need);
  if (blockIdx.x == 0 && threadIdx.x == 0) {  // every prompt with tokens has slice 0
    uint32_t* state = ws + (int64_t)3 * n_seg * kBins + (int64_t)blockIdx.y * kState;
    state[6] = thresh;
    state[7] = need;
  }
  const float* ss = scores + seg.seg_start;
  uint32_t nd = 0u, nt = 0u;
#pragma unroll
  for (int i = 0; i < SLICE / kMT; ++i) {
    const int t = t0 + i * kMT + (int)threadIdx.x;
    if (t < seg.seg_len) {
      if (t < seg.doc_begin || t >= seg.doc_end) {
        ++nd;
      } else {
        const uint32_t key = score_key(ss[t]);
        nd += key > thresh;
        nt += key == thresh;
      }
    }
  }
  uint32_t e0, e1, td, tt;
  scan256(nd, nt, e0, e1, td, tt, sm);
  if (threadIdx.x == 0) {
    uint32_t* cnt = ws + (int64_t)3 * n_seg * kBins + (int64_t)n_seg * kState + ((int64_t)blockIdx.y * n_slices + blockIdx.x) * 2;
    cnt[0] = td;
    cnt[1] = tt;
  }
}

template <int SLICE>
__global__ __launch_bounds__(kMT) void select_emit_kernel(const float* __restrict__ scores,
                                                          SegTable segs, int n_seg,
                                                          int n_slices, const uint32_t* __restrict__ ws,
                                                          int32_t* __restrict__ kept_idx) {
  __shared__ MultiSmem sm;
  const tg_segment seg = segs.at_uniform(blockIdx.y);
  const int s0 = blockIdx.x * SLICE;
  if (s0 >= seg.seg_len) return;
  // the threshold and tie quota the count kernel derived (it ran before this launch, on the same stream)
  const uint32_t* state = ws + (int64_t)3 * n_seg * kBins + (int64_t)blockIdx.y * kState;
  const uint32_t thresh = state[6], need = state[7];
  // offsets from the earlier slices of this prompt
  const uint32_t* cnt = ws + (int64_t)3 * n_seg * kBins + (int64_t)n_seg * kState + (int64_t)blockIdx.y * n_slices * 2;
  uint32_t bd = 0u, bt = 0u;
  {
    const int j = threadIdx.x;  // one earlier slice per thread (n_slices <= 256 per 1M tokens; looped beyond)
    uint32_t d = 0u, t = 0u;
    for (int jj = j; jj < (int)blockIdx.x; jj += kMT) {
      d += cnt[2 * jj];
      t += cnt[2 * jj + 1];
    }
    uint32_t e0, e1;
    scan256(d, t, e0, e1, bd, bt, sm);
  }
  // thread-contiguous ownership for the index-ordered emission
  const float* ss = scores + seg.seg_start;
  const int t0 = s0 + (int)threadIdx.x * (SLICE / kMT);
  uint32_t fd = 0u, ft = 0u;
#pragma unroll
  for (int i = 0; i < SLICE / kMT; ++i) {
    const int t = t0 + i;
    if (t < seg.seg_len && t < s0 + SLICE) {
      if (t < seg.doc_begin || t >= seg.doc_end) {
        fd |= 1u << i;
      } else {
        const uint32_t key = score_key(ss[t]);
        if (key > thresh)
          fd |= 1u << i;
        else if (key == thresh)
          ft |= 1u << i;
      }
    }
  }
  uint32_t ed, et, td, tt;
  scan256((uint32_t)__builtin_popcount(fd), (uint32_t)__builtin_popcount(ft), ed, et, td, tt, sm);
  // as in select_topk_kernel: the thread keeps its first need - t_before ties, and its kept tokens land in
  // index order from row def_before + min(t_before, need) on
  const uint32_t t_before = bt + et;
  uint32_t quota = need > t_before ? need - t_before : 0u;
  uint32_t kept = fd;
  for (uint32_t m = ft; m != 0u && quota != 0u; m &= m - 1u, --quota) kept |= m & (0u - m);
  uint32_t pos = bd + ed + (t_before < need ? t_before : need);
  int32_t* out = kept_idx + seg.kept_start;
  for (uint32_t m = kept; m != 0u; m &= m - 1u, ++pos)
    if (pos < (uint32_t)seg.kept_len) out[pos] = seg.seg_start + t0 + __builtin_ctz(m);
}

}  // namespace

// One workgroup per prompt up to 16K tokens (keys resident in registers);
// past that the six-launch multi-workgroup path is faster (measured: 17.2 vs
// 18.2 us at 24576 tokens, 17.2 vs 20.9 at 32768; 12.2 vs 17.1 at 16384).
static bool use_multi(const tg_plan_info& info) { return info.max_seg_len > kThreads * 16; }

static int slice_of(const tg_plan_info& info) {
  const int64_t large = (int64_t)info.n_seg * ((info.max_seg_len + kSliceLarge - 1) / kSliceLarge);
  return large >= 256 ? kSliceLarge : kSliceSmall;
}
static int n_slices(const tg_plan_info& info) {
  const int s = slice_of(info);
  return (int)((info.max_seg_len + s - 1) / s);
}

size_t select_workspace_bytes(const tg_plan_info& info) {
  if (!use_multi(info)) return 0;  // the one-workgroup kernel keeps its state on chip
  const size_t words = (size_t)3 * info.n_seg * kBins + (size_t)info.n_seg * kState + (size_t)info.n_seg * n_slices(info) * 2;
  return (words * 4 + 255) / 256 * 256;
}

hipError_t launch_select_topk(const float* scores, const tg_segment* segs_in, const tg_plan_info& info,
                              int32_t* kept_idx, void* workspace, hipStream_t stream) {
  const SegTable segs = seg_table(segs_in, info);
  if (info.max_seg_len <= 0) return hipSuccess;
  if (!use_multi(info)) {
    hipLaunchKernelGGL(select_topk_kernel<16>, dim3(info.n_seg), dim3(kThreads), 0, stream, scores, segs, kept_idx);
    return hipGetLastError();
  }
  uint32_t* ws = static_cast<uint32_t*>(workspace);
  const int ns = n_slices(info);
  const int n_seg = (int)info.n_seg;
  const int64_t hist_words = (int64_t)3 * n_seg * kBins;
  hipLaunchKernelGGL(select_zero_kernel, dim3((unsigned)((hist_words + 255) / 256 < 1024 ? (hist_words + 255) / 256 : 1024)),
                     dim3(256), 0, stream, ws, hist_words);
  const dim3 grid(ns, n_seg);
#define TG_SELECT_MULTI(S)                                                                                      \
  hipLaunchKernelGGL((select_hist_kernel<0, S>), grid, dim3(kMT), 0, stream, scores, segs, n_seg, ws);         \
  hipLaunchKernelGGL((select_hist_kernel<1, S>), grid, dim3(kMT), 0, stream, scores, segs, n_seg, ws);         \
  hipLaunchKernelGGL((select_hist_kernel<2, S>), grid, dim3(kMT), 0, stream, scores, segs, n_seg, ws);         \
  hipLaunchKernelGGL((select_count_kernel<S>), grid, dim3(kMT), 0, stream, scores, segs, n_seg, ns, ws);       \
  hipLaunchKernelGGL((select_emit_kernel<S>), grid, dim3(kMT), 0, stream, scores, segs, n_seg, ns, ws, kept_idx)
  if (slice_of(info) == kSliceSmall) {
    TG_SELECT_MULTI(kSliceSmall);
  } else {
    TG_SELECT_MULTI(kSliceLarge);
  }
#undef TG_SELECT_MULTI
  return hipGetLastError();
}

}  // namespace tg
