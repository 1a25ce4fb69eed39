// Top-K select and kept-index emission (gfx950).
//
// Kept set S = top-K(document scores) ∪ (every non-document token)
// ("TokenGate 与 T2Quant ... 精读", sections 3.1 and 4.1).  Order among document
// tokens: higher score, then lower index.
//
// One launch, one 1024-thread workgroup per prompt.  At batch 1 the scores
// are 64-512 KiB: the cost is latency, not bandwidth, so everything a
// multi-block design would spend on launches, global atomics and fences is
// avoided.  Thread t owns R consecutive tokens of every 1024 R-token chunk;
// when the prompt fits one chunk the keys stay in registers for all passes.
//
// Scores become order-preserving 32-bit keys (score_key); the K-th largest
// document key T is found exactly by a three-digit MSB radix select
// (11 + 11 + 10 bits) with LDS histograms (integer atomics: exact).  Then
// every token is classified in index order: non-document or key > T is kept,
// key == T is kept while fewer than need = K_eff - #{key > T} ties have been
// kept before it.  A block-wide exclusive scan gives every kept token its
// output row, so the output is ascending and identical on every run.
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
};

// Inclusive scan of two counters across the workgroup; returns the exclusive
// prefixes, and the block totals through tot0 / tot1.
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb, uint32_t& tot0,
                                            uint32_t& tot1, SelSmem& sm) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t xa = a, xb = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t ya = __shfl_up(xa, o);
    const uint32_t yb = __shfl_up(xb, o);
    if (lane >= o) {
      xa += ya;
      xb += yb;
    }
  }
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
// Every thread owns bins/1024 consecutive bins, highest first.
__device__ __forceinline__ void find_digit(SelSmem& sm, uint32_t bins, uint32_t rem) {
  const int tid = threadIdx.x;
  const uint32_t per = bins / kThreads;  // 2 or 1
  uint32_t c[2] = {0u, 0u};
  uint32_t sum = 0u;
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
    for (uint32_t j = 0; j < per; ++j) {
      if (acc + c[j] >= rem) {
        sm.found_digit = bins - 1u - (tid * per + j);
        sm.found_rem = rem - acc;
        break;
      }
      acc += c[j];
    }
  }
  __syncthreads();
}

template <int R>
__device__ __forceinline__ void load_chunk(const float* __restrict__ seg_scores, const tg_segment& seg, int base,
                                           uint32_t (&key)[R], uint32_t& docmask) {
  const int t0 = base + (int)threadIdx.x * R;
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
                                                               const tg_segment* __restrict__ segs,
                                                               int32_t* __restrict__ kept_idx) {
  __shared__ SelSmem sm;
  constexpr int kChunk = kThreads * R;
  const tg_segment seg = segs[blockIdx.x];
  if (seg.seg_len <= 0) return;
  const int tid = threadIdx.x;
  const int sub = (tid >> 6) & (kSub - 1);
  const float* ss = scores + seg.seg_start;
  const int n_doc = seg.doc_end - seg.doc_begin;
  const int n_chunks = (seg.seg_len + kChunk - 1) / kChunk;
  const bool resident = n_chunks == 1;

  uint32_t key[R];
  uint32_t docmask = 0u;
  if (resident) load_chunk<R>(ss, seg, 0, key, docmask);

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
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t bins = pass == 2 ? 1024u : 2048u;
      const uint32_t mask = pass == 0 ? 0u : (pass == 1 ? 0xffe00000u : 0xfffffc00u);
      for (int i = tid; i < kSub * kBins; i += kThreads) (&sm.hist[0][0])[i] = 0u;
      __syncthreads();
#pragma unroll 1
      for (int c = 0; c < n_chunks; ++c) {
        if (!resident) load_chunk<R>(ss, seg, c * kChunk, key, docmask);
#pragma unroll
        for (int i = 0; i < R; ++i) {
          if (((docmask >> i) & 1u) && (key[i] & mask) == prefix)
            atomicAdd(&sm.hist[sub][(key[i] >> shift) & (bins - 1u)], 1u);
        }
      }
      __syncthreads();
      find_digit(sm, bins, rem);
      prefix |= sm.found_digit << shift;
      rem = sm.found_rem;
      __syncthreads();
    }
    thresh = prefix;
    need = rem;
  }

  // Emission in index order.
  int32_t* out = kept_idx + seg.kept_start;
  uint32_t def_base = 0u, tie_base = 0u;
#pragma unroll 1
  for (int c = 0; c < n_chunks; ++c) {
    if (!resident) load_chunk<R>(ss, seg, c * kChunk, key, docmask);
    const int t0 = c * kChunk + tid * R;
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
    uint32_t rdf = def_base + ed;
    uint32_t rtie = tie_base + et;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const bool d = (fd >> i) & 1u;
      const bool tt_ = (ft >> i) & 1u;
      const uint32_t taken = rtie < need ? rtie : need;
      if (d || (tt_ && rtie < need)) {
        const uint32_t pos = rdf + taken;
        if (pos < (uint32_t)seg.kept_len) out[pos] = seg.seg_start + t0 + i;
      }
      rdf += d;
      rtie += tt_;
    }
    def_base += td;
    tie_base += tt;
  }
}

}  // namespace

size_t select_workspace_bytes(const tg_plan_info& info) {
  (void)info;
  return 0;
}

hipError_t launch_select_topk(const float* scores, const tg_segment* segs, const tg_plan_info& info,
                              int32_t* kept_idx, void* workspace, hipStream_t stream) {
  (void)workspace;
  if (info.max_seg_len <= 0) return hipSuccess;
  dim3 grid(info.n_seg);
  if (info.max_seg_len <= kThreads * 16)
    hipLaunchKernelGGL(select_topk_kernel<16>, grid, dim3(kThreads), 0, stream, scores, segs, kept_idx);
  else
    hipLaunchKernelGGL(select_topk_kernel<32>, grid, dim3(kThreads), 0, stream, scores, segs, kept_idx);
  return hipGetLastError();
}

}  // namespace tg
