// Token-gated causal GQA attention over the kept rows, prefill (gfx950).
//
// "TokenGate 与 T2Quant ... 精读", section 4.1, component two: the kept token's
// gate score enters the attention logits as a bias, with a per-(layer, head)
// gain and a temperature:
//   z_rt = tau_h (q_r . k_t) / sqrt(D) + g_h s_t,   t <= r (kept rows, original order)
//
// Flash-style, one pass over the keys with an online softmax in the exp2
// domain.  A workgroup owns one key/value head and a 128/G-row query tile of
// all G query heads sharing it, so every K/V tile staged in LDS serves G
// heads.  Its 8 waves form two groups of 4 (one wave of each group per SIMD);
// each wave owns 32 query rows of one head, group 0 takes the even 64-key
// tiles and group 1 the odd ones, and the two are merged at the end.
//
// Ping-pong schedule.  Each wave alternates an MFMA phase (PV of its previous
// tile, then QK of its next tile) and a softmax phase (VALU), and the two
// groups are half a step apart, separated by workgroup barriers: while one
// wave of a SIMD issues MFMAs the other runs its exp2s, so the matrix cores
// and the VALU work at the same time.  All 512 threads stage the next K tile
// (threads 0-255, with the scores) and the V tile due next (threads 256-511):
// by direct-to-LDS loads into three LDS stages (the kernel at the end of this
// file), or, for gathered rows of prompts past 8192 kept rows, through
// registers, loaded during one half-step and written to LDS at the end of the
// next.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16).  Scores are computed transposed,
// S^T = K . Q^T, so a lane owns one query column (l % 32) and 16 key rows per
// 32-key half: the softmax row max/sum is a register loop plus one swap with
// the other half-wave.  The output is accumulated transposed too,
// O^T += V^T . P^T, which lets P^T be fed from the score registers without
// any data movement (the key order inside each 16-key MFMA step is permuted
// identically on both operands) and keeps the per-query rescale lane-local.
// The register-staged kernel stores V transposed in LDS and K row-major, both
// with padded rows, so the 16- and 8-byte LDS reads are bank-conflict free;
// the direct-to-LDS kernel keeps both row-major and reads V^T with transposing
// LDS reads.
//
// Logit arithmetic.  With c_h = |tau_h| log2(e) / sqrt(D) (floored at 1e-30;
// a negative temperature flips the sign of Q, which is exact) the score
// accumulators start from the key's bias divided by c_h, so the MFMA returns
// a_rt = q.k + g_h log2(e) s_t / c_h and the exp2-domain logit is c_h a_rt:
// the softmax needs one FMA and one exp2 per element.  The row sum is taken
// over the bf16-rounded probabilities (the values the PV product uses).
// Tiles are launched longest-first (the last query tile of a prompt first).
//
// Per-query temperature (same section, second refinement): the temperature of
// kept row r can instead be softplus(sigma_h) log(m_r) / log(max(2, p_r)),
// with m_r = r + 1 its rank among the prompt's kept rows and p_r = 1 + its
// original position.  The lane owning row r then has its own c_r, the staged
// bias is g_h log2(e) s_t, and the accumulator seed is that times 1 / c_r.
#include <algorithm>
#include <atomic>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <tuple>
#include <type_traits>
#include <vector>

#include "common.h"

namespace tg {
namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 512;  // two groups of 4 waves
constexpr int kMaxGatherRows = 16384;  // kept rows per prompt the gathering variant supports (indices in LDS)
constexpr int kDmaGatherRows = 8192;   // up to this many, gathering reads use direct-to-LDS staging
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct alignas(16) AttnSmem {
  static constexpr int kLd = D + 8;    // K row stride (bf16)
  static constexpr int vLd = kBN + 4;  // V^T row stride (bf16)
  uint16_t k[2][kBN * kLd];            // two stages (tile parity)
  uint16_t vt[2][D * vLd];
  float s[2][4][kBN];                  // [stage][head of the KV group][key]: bias / c_h
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// Threads 0-255 stage K tiles (and the scores), threads 256-511 V tiles.
template <int D>
struct Stager {
  static constexpr int kTpr = D / 8;          // K: threads per row (16 bytes each)
  static constexpr int kRpi = 256 / kTpr;     // K: rows per load instruction
  static constexpr int kKLoads = kBN / kRpi;  // = D / 32
  int k_row, k_col;  // K: first row and column of this thread
  int v_dc, v_kq;    // V: unit of 8 dims (v_dc) x 4 keys (v_kq)
  bool v_on;
  __device__ explicit Stager(int t) {  // t = thread index within its half
    k_row = t / kTpr;
    k_col = (t % kTpr) * 8;
    v_dc = (t & 1) + 2 * ((t >> 4) % (D / 16));
    v_kq = ((t >> 1) & 7) + 8 * (t / D);
    v_on = t < 2 * D;
  }
  __device__ __forceinline__ uint32_t k_off(uint32_t row_bytes) const {
    return (uint32_t)k_row * row_bytes + (uint32_t)k_col * 2u;
  }
  __device__ __forceinline__ uint32_t v_off(uint32_t row_bytes) const {
    return (uint32_t)(4 * v_kq) * row_bytes + (uint32_t)v_dc * 16u;
  }
};

// Gathered rows: kept row r of the prompt is source row sidx[r]; rows at or
// past `nvalid` get an offset past every buffer range, so they read as zeros.
constexpr uint32_t kPastRange = 0xfffffff0u;

// Kernel variants: compacted rows (per-head temperature), gather on load, and
// compacted rows with the per-query temperature.
enum AttnMode { kCompacted = 0, kGather = 1, kQueryTau = 2 };

template <int D, bool GATHER>
__device__ __forceinline__ void load_k(const Stager<D>& st, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rs,
                                       uint32_t koff, uint32_t row_bytes, int kv0, int t, u32x4 (&r)[4], float& sr,
                                       const int32_t* sidx, int nvalid) {
  if (!GATHER) {
#pragma unroll
    for (int j = 0; j < Stager<D>::kKLoads; ++j)
      r[j] = buf_load16(rk, koff, (uint32_t)(kv0 + Stager<D>::kRpi * j) * row_bytes);
    if (t < kBN) sr = buf_load4f(rs, (uint32_t)t * 4u, (uint32_t)kv0 * 4u);
  } else {
#pragma unroll
    for (int j = 0; j < Stager<D>::kKLoads; ++j) {
      const int row = kv0 + st.k_row + Stager<D>::kRpi * j;
      const uint32_t off = row < nvalid ? (uint32_t)sidx[row] * row_bytes + (uint32_t)st.k_col * 2u : kPastRange;
      r[j] = buf_load16(rk, off, 0u);
    }
    if (t < kBN) {
      const int row = kv0 + t;
      sr = buf_load4f(rs, row < nvalid ? (uint32_t)sidx[row] * 4u : kPastRange, 0u);
    }
  }
}

template <int D, int G>
__device__ __forceinline__ void store_k(const Stager<D>& st, AttnSmem<D>& sm, int buf, int t, const u32x4 (&r)[4],
                                        float sr, const float (&ratio)[G]) {
#pragma unroll
  for (int j = 0; j < Stager<D>::kKLoads; ++j)
    *reinterpret_cast<u32x4*>(&sm.k[buf][(st.k_row + Stager<D>::kRpi * j) * AttnSmem<D>::kLd + st.k_col]) = r[j];
  if (t < kBN) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) sm.s[buf][hh][t] = ratio[hh] * sr;
  }
}

template <int D, bool GATHER>
__device__ __forceinline__ void load_v(const Stager<D>& st, __amdgpu_buffer_rsrc_t rv, uint32_t voff,
                                       uint32_t row_bytes, int kv0, u32x4 (&r)[4], const int32_t* sidx, int nvalid) {
  if (st.v_on) {
    if (!GATHER) {
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = buf_load16(rv, voff, (uint32_t)(kv0 + i) * row_bytes);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = kv0 + 4 * st.v_kq + i;
        const uint32_t off = row < nvalid ? (uint32_t)sidx[row] * row_bytes + (uint32_t)st.v_dc * 16u : kPastRange;
        r[i] = buf_load16(rv, off, 0u);
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void store_v(const Stager<D>& st, AttnSmem<D>& sm, int buf, const u32x4 (&r)[4]) {
  if (st.v_on) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // dim e of the 4 keys: low or high bf16 of word e / 2 of each key row, packed pairwise
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const int w = e >> 1;
      const u32x2 pk = u32x2{__builtin_amdgcn_perm(r[1][w], r[0][w], sel),
                             __builtin_amdgcn_perm(r[3][w], r[2][w], sel)};
      *reinterpret_cast<u32x2*>(&sm.vt[buf][(st.v_dc * 8 + e) * AttnSmem<D>::vLd + 4 * st.v_kq]) = pk;
    }
  }
}

// Softmax phase of one 64-key tile starting at key kv0: causal mask on the
// diagonal tiles, running max with the lazy rescale, exp2 of the logits, row
// sums over the bf16-rounded probabilities, and the P^T operands of the 4 PV
// steps.
template <int D>
__device__ __forceinline__ void softmax_tile(int kv0, int qrow, int qw0, int n, int g, float cs, f32x16 (&sa)[2],
                                             float& m_run, float& l_run, f32x16 (&o)[D / 32], u32x4 (&pf)[4]) {
  if (kv0 + kBN - 1 > qw0 || kv0 + kBN > n) {
    // the lane's last visible key (tile-local), less its 4 g row offset, so that
    // every comparison below is against a constant
    const int lim = min(qrow, n - 1) - kv0 - 4 * g;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (hf * 32 + 8 * (i / 4) + (i % 4) > lim) sa[hf][i] = -__builtin_inff();
  }
  float m0 = -__builtin_inff(), m1 = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    m0 = __builtin_fmaxf(m0, __builtin_fmaxf(sa[0][i], sa[0][i + 1]));
    m1 = __builtin_fmaxf(m1, __builtin_fmaxf(sa[1][i], sa[1][i + 1]));
  }
  const float x = cs * xor32_max(__builtin_fmaxf(m0, m1));
  // Lazy rescale: the reference point m_run only moves when some row's
  // max exceeds it by more than 2^8 (or on the first visible tile);
  // softmax does not depend on the reference point, and
  // exp2(x - m_run) <= 2^8 stays well inside fp32 and bf16 range.
  if (__ballot(x > m_run + 8.0f) != 0) {
    asm volatile("; rare rescale");  // keeps this a branch rather than a select on every tile
    const float m_new = __builtin_fmaxf(m_run, x);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
    m_run = m_new;
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[hf][8 * sub + 2 * j], cs, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[hf][8 * sub + 2 * j + 1], cs, -m_run));
        // (bit-cast a scalar: a bit-cast of the vector element w[j] reads element 0 with this compiler)
        const uint32_t pk = pack_bf16(p0, p1);
        w[j] = pk;
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), ones, l_run, false);
      }
      pf[2 * hf + sub] = w;
    }
}

// Merges the two wave groups, normalises, and stores the bf16 output rows
// (and the natural-log log-sum-exp when lse is given).  Both groups put their
// (m, l) and the half of O^T the other group finishes into LDS at xo (8 waves
// x kMergeRec<D> floats); group 0 then finishes dims [0, D/2) and group 1 dims
// [D/2, D), so each wave moves and stores half the output.
template <int D>
constexpr int kMergeRec = D * 16 + 64;  // floats per wave: half of O^T (D/2 x 32), m, l

// The half of O^T the partner group finishes, and this wave's (m, l), into LDS.
template <int D, bool G0>
__device__ __forceinline__ void merge_publish(float* xo, int wave, int lane, int g, int l32, const f32x16 (&o)[D / 32],
                                              float m_run, float l_half) {
  constexpr int kHalf = D / 64;         // 32-dim tiles per group
  constexpr int give = G0 ? kHalf : 0;  // first tile of the half the partner finishes
  float* mine = xo + ((G0 ? 0 : 4) + wave) * kMergeRec<D>;
#pragma unroll
  for (int t = 0; t < kHalf; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) mine[(t * 16 + i) * 64 + lane] = o[give + t][i];
  if (g == 0) {
    mine[D * 16 + l32] = m_run;
    mine[D * 16 + 32 + l32] = l_half;
  }
}

// Merges this group's half of the dims with the partner's partial state and stores it.
template <int D, bool G0>
__device__ __forceinline__ void merge_finish(const float* xo, int wave, int lane, int g, int l32,
                                             const f32x16 (&o)[D / 32], float m_run, float l_half, int qrow, int n,
                                             const tg_segment& seg, int64_t q_stride, int h, int hq,
                                             float* __restrict__ lse, uint16_t* __restrict__ out) {
  constexpr int kHalf = D / 64;
  constexpr int keep = G0 ? 0 : kHalf;  // first tile of the half this group finishes
  const float* theirs = xo + ((G0 ? 4 : 0) + wave) * kMergeRec<D>;
  const float mo = theirs[D * 16 + l32];
  const float lo = theirs[D * 16 + 32 + l32];
  // group 0's and group 1's partial states, the same in both groups
  const float m0 = G0 ? m_run : mo, m1 = G0 ? mo : m_run;
  const float l0 = G0 ? l_half : lo, l1 = G0 ? lo : l_half;
  const float m = __builtin_fmaxf(m0, m1);
  const float a0 = m0 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m0 - m);
  const float a1 = m1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
  const float l_all = __builtin_fmaf(l0, a0, l1 * a1);
  const float inv = 1.0f / l_all;
  // natural-log log-sum-exp of the row's logits (kept for the backward pass)
  if (G0 && lse != nullptr && qrow < n && g == 0)
    lse[((int64_t)seg.kept_start + qrow) * hq + h] = (m + __log2f(l_all)) * 0.6931471805599453f;
  if (qrow < n) {
    uint16_t* orow = out + ((int64_t)seg.kept_start + qrow) * q_stride + (int64_t)h * D;
#pragma unroll
    for (int t = 0; t < kHalf; ++t) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q4 + e;
          const float own = o[keep + t][i];
          const float other = theirs[(t * 16 + i) * 64 + lane];
          r[e] = (G0 ? __builtin_fmaf(own, a0, other * a1) : __builtin_fmaf(other, a0, own * a1)) * inv;
        }
        *reinterpret_cast<u32x2*>(orow + 32 * (keep + t) + 8 * q4 + 4 * g) = u32x2{pack_bf16(r[0], r[1]),
                                                                                   pack_bf16(r[2], r[3])};
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void merge_and_store(float* xo, int grp, int wave, int lane, int g, int l32,
                                                const f32x16 (&o)[D / 32], float m_run, float l_run, int qrow, int n,
                                                const tg_segment& seg, int64_t q_stride, int h, int hq,
                                                float* __restrict__ lse, uint16_t* __restrict__ out) {
  const float l_half = xor32_sum(l_run);  // both half-waves: same bits
  if (grp == 0)  // uniform per wave
    merge_publish<D, true>(xo, wave, lane, g, l32, o, m_run, l_half);
  else
    merge_publish<D, false>(xo, wave, lane, g, l32, o, m_run, l_half);
  __syncthreads();
  if (grp == 0)
    merge_finish<D, true>(xo, wave, lane, g, l32, o, m_run, l_half, qrow, n, seg, q_stride, h, hq, lse, out);
  else
    merge_finish<D, false>(xo, wave, lane, g, l32, o, m_run, l_half, qrow, n, seg, q_stride, h, hq, lse, out);
}

// Epilogue of a split query tile.  The groups merge as in merge_and_store
// (unnormalised, in group 0), then the workgroup counts itself in at
// flags[0].  The first half to arrive publishes (O^T, m, l) of its rows to
// `mine` (4 waves x (D x 32 + 64) floats, in the register layout), then sets
// flags[1]; the second waits for flags[1] (the first is already past its count
// and waits on nothing, so the wait ends; it is also bounded), reads the
// record from `other`, merges, normalises, stores, and resets both flags for
// the next launch.  The merge is symmetric (both products rounded before the
// sum), so the result does not depend on the arrival order.
//
// Ordering (AMDGPU memory model, agent scope, gfx950: one L2 per XCD, not
// coherent with the others).  Every record and flag access is an agent-scope
// atomic with relaxed order, which the compiler emits with the sc1 bit: the
// access bypasses the XCD's L2 and goes to memory, where all XCDs see it.  The
// publisher waits (vmcnt 0) until its record stores are acknowledged before it
// stores the flag, so the record is in memory before the flag is; the consumer
// issues its record loads only after its flag load has returned the raised
// flag (the loop exit depends on it), and those loads also bypass L2, so they
// cannot return older data.  That is the release / acquire pair the exchange
// needs without the L2 write-back and invalidation that agent-scope fences
// (release / acquire orderings) imply on this chip, which would also evict the
// K/V tiles of every other workgroup of the XCD (measured: twice as slow).
//
// A workspace left inconsistent is detected instead of merged: an arrival
// count of 2 or more means the counters were not zero when this launch
// started (a previous wait ran out, or the workspace was not zero-filled);
// then, and when this call's own wait runs out, the tile's rows (and
// log-sum-exp) are written as NaN, a bit is set in the status word at the
// start of the workspace, and the counters are left as they are (every later
// call sees the same state until the caller zero-fills the workspace).
constexpr int kSplitMaxSpins = 1 << 22;  // 134 ns per poll on MI355X (L2-bypassing load + s_sleep 1): ~0.56 s
constexpr int kSplitStatusPoisoned = 1, kSplitStatusExpired = 2;

template <int D>
__device__ __forceinline__ void merge_split(float* xo, int grp, int wave, int lane, int g, int l32,
                                            f32x16 (&o)[D / 32], float m_run, float l_run, int qrow, int n,
                                            const tg_segment& seg, int64_t q_stride, int h, int hq,
                                            float* __restrict__ lse, uint16_t* __restrict__ out, float* mine_rec,
                                            float* other_rec, int* flags, int* status) {
  constexpr int kRec = D * 32 + 64;
  float* mine = xo + wave * kRec;
  int* arrival = reinterpret_cast<int*>(xo + 4 * kRec);
  const float l_half = xor32_sum(l_run);  // both half-waves: same bits
  if (grp == 1) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mine[(dt * 16 + i) * 64 + lane] = o[dt][i];
    if (g == 0) {
      mine[D * 32 + l32] = m_run;
      mine[D * 32 + 32 + l32] = l_half;
    }
  }
  __syncthreads();
  float m = m_run, l = l_half;
  if (grp == 0) {
    const float m1 = mine[D * 32 + l32];
    const float l1 = mine[D * 32 + 32 + l32];
    m = __builtin_fmaxf(m_run, m1);
    const float a0 = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
    l = l_half * a0 + l1 * a1;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = o[dt][i] * a0 + mine[(dt * 16 + i) * 64 + lane] * a1;
  }
  if (threadIdx.x == 0) arrival[0] = atomicAdd(&flags[0], 1);
  __syncthreads();
  const int arrived = arrival[0];
  if (arrived == 0) {  // uniform: first half in publishes its record
    if (grp == 0) {
      float* rec = mine_rec + wave * kRec;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          __hip_atomic_store(&rec[(dt * 16 + i) * 64 + lane], o[dt][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (g == 0) {
        __hip_atomic_store(&rec[D * 32 + l32], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&rec[D * 32 + 32 + l32], l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      wait_vm<0>();  // the record writes have completed before the flag below
    }
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(&flags[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // arrival count 2 or more: the counters were already set when this launch began (poisoned workspace)
  if (arrived == 1 && threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(&flags[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0 && ++spins < kSplitMaxSpins)
      __builtin_amdgcn_s_sleep(1);
    arrival[1] = spins >= kSplitMaxSpins ? kSplitStatusExpired : 0;
  }
  __syncthreads();
  // A poisoned workspace or an expired wait: the record may be stale, so these rows are written as NaN
  // rather than as a plausible wrong merge, the status word records why, and the counters stay as they are.
  const int bad = arrived == 1 ? arrival[1] : kSplitStatusPoisoned;
  const bool expired = bad != 0;
  if (expired && threadIdx.x == 0) atomicOr(status, bad);
  if (grp == 0) {
    // both products rounded before the sum (no fused multiply-add), so the two arrival orders give the same bits
#pragma clang fp contract(off)
    const float* rec = other_rec + wave * kRec;
    float ob[D / 32][16];  // the whole record is requested before any of it is used
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        ob[dt][i] = __hip_atomic_load(&rec[(dt * 16 + i) * 64 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float mb = __hip_atomic_load(&rec[D * 32 + l32], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float lb = __hip_atomic_load(&rec[D * 32 + 32 + l32], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float mm = __builtin_fmaxf(m, mb);
    const float aa = m == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m - mm);
    const float ab = mb == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mb - mm);
    const float l_all = l * aa + lb * ab;
    const float inv = 1.0f / l_all;
    // NaN is chosen on the stored bits: this file is built without NaN semantics for float arithmetic
    if (lse != nullptr && qrow < n && g == 0)
      reinterpret_cast<uint32_t*>(lse)[((int64_t)seg.kept_start + qrow) * hq + h] =
          expired ? 0x7fc00000u : __builtin_bit_cast(uint32_t, (mm + __log2f(l_all)) * 0.6931471805599453f);
    if (qrow < n) {
      uint16_t* orow = out + ((int64_t)seg.kept_start + qrow) * q_stride + (int64_t)h * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * q4 + e;
            r[e] = (o[dt][i] * aa + ob[dt][i] * ab) * inv;
          }
          *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * q4 + 4 * g) =
              expired ? u32x2{0x7fc07fc0u, 0x7fc07fc0u} : u32x2{pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3])};
        }
      }
    }
  }
  if (threadIdx.x == 0 && !expired) {
    __hip_atomic_store(&flags[0], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&flags[1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Register-staged kernel, launched for gathering reads of prompts with more
// than 8192 kept rows (their indices take up to 64 KiB of LDS, which leaves no
// room for three direct-to-LDS stages).
// kGather: q, k, v and key_score hold every token (n_src rows); kept row r of
// a prompt is read from source row kept_idx[kept_start + r] (gather on load,
// no compacted copies).  The output is always compacted.
// kQueryTau: tau holds sigma_h and qpos the original positions of the kept rows.
template <int D, int G, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gated_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ tau, const float* __restrict__ gain,
    SegTable segs, int hq, int hkv, const int32_t* __restrict__ kept_idx, int64_t n_src,
    const int32_t* __restrict__ qpos, float* __restrict__ lse, uint16_t* __restrict__ out) {
  constexpr bool GATHER = MODE == kGather;
  constexpr bool QTAU = MODE == kQueryTau;
  constexpr int kBM = 128 / G;  // query rows per workgroup
  constexpr int kWavesPerHead = 4 / G;
  __shared__ AttnSmem<D> sm;
  static_assert(8 * kMergeRec<D> * 4 <= (int)sizeof(AttnSmem<D>), "group merge fits in LDS");
  __shared__ int32_t sidx[GATHER ? kMaxGatherRows : 1];  // source rows of the kept rows [0, q_end)

  const tg_segment seg = segs.at_uniform(blockIdx.z);
  const int n = seg.kept_len;
  const int q0 = (gridDim.y - 1 - blockIdx.y) * kBM;
  if (q0 >= n) return;  // uniform
  const int q_end = min(q0 + kBM, n);  // keys needed: t < q_end
  if (GATHER) {
    for (int i = threadIdx.x; i < q_end; i += kThreads) sidx[i] = kept_idx[seg.kept_start + i];
    __syncthreads();
  }

  const int tid = threadIdx.x;
  const int grp = tid >> 8;      // 0: even key tiles, 1: odd key tiles
  const int gtid = tid & 255;    // thread index inside the group (and inside its staging half)
  const int lane = tid & 63;
  const int wave = gtid >> 6;    // wave inside the group
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int c = blockIdx.x;
  const int hl = wave / kWavesPerHead;  // this wave's head inside the KV group
  const int h = c * G + hl;
  const int qw0 = q0 + (wave % kWavesPerHead) * 32;  // first query row of this wave
  const int qrow = qw0 + l32;                         // the query column this lane owns

  const int64_t q_stride = (int64_t)hq * D;
  const int64_t kv_stride = (int64_t)hkv * D;
  const int64_t row0 = GATHER ? 0 : seg.kept_start;                  // first row of the K/V/score buffers
  const uint32_t nrows = GATHER ? (uint32_t)n_src : (uint32_t)n;     // rows the buffers cover
  const uint16_t* kb = k + row0 * kv_stride + (int64_t)c * D;
  const uint16_t* vb = v + row0 * kv_stride + (int64_t)c * D;
  const bool use_bias = key_score != nullptr && gain != nullptr;
  const uint32_t row_bytes = (uint32_t)kv_stride * 2u;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, nrows * row_bytes - (uint32_t)c * D * 2u);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, nrows * row_bytes - (uint32_t)c * D * 2u);
  // no bias: an empty range makes every score load return 0
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(use_bias ? key_score + row0 : key_score, use_bias ? nrows * 4u : 0u);
  const Stager<D> stg(gtid);
  const bool stage_k = grp == 0;  // threads 0-255 stage K, 256-511 V
  const uint32_t koff = stg.k_off(row_bytes), voff = stg.v_off(row_bytes);

  // logit scale c_h of this wave's head, and g_h log2(e) / c_h of every head of the group (for the staged bias)
  const float base = kLog2e / __builtin_sqrtf((float)D);
  float ratio[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float th = tau != nullptr ? tau[c * G + hh] : 1.0f;
    ratio[hh] = !use_bias ? 0.0f
                : QTAU    ? gain[c * G + hh] * kLog2e
                          : gain[c * G + hh] * kLog2e / __builtin_fmaxf(__builtin_fabsf(th) * base, 1e-30f);
  }
  float th = tau != nullptr ? tau[h] : 1.0f;
  if (QTAU) {
    // tau_r = softplus(sigma_h) log(r + 1) / log(max(2, p_r + 1)) for this lane's row r (>= 0)
    const int r = qrow < n ? qrow : n - 1;
    const float sp = th > 20.0f ? th : log1pf(expf(th));
    const float pr = (float)max(2, qpos[seg.kept_start + r] + 1);
    th = sp * (logf((float)(r + 1)) / logf(pr));
  }
  const float cs = __builtin_fmaxf(__builtin_fabsf(th) * base, 1e-30f);
  const float inv_cs = QTAU ? 1.0f / cs : 1.0f;

  // Q^T operand: lane holds q[qrow][16 ks + 8 g .. + 7]
  u32x4 qf[D / 16];
  {
    const int r = qrow < n ? qrow : n - 1;
    int64_t qsrc = (int64_t)seg.kept_start + r;
    if (GATHER) {
      qsrc = sidx[r];
      if (qsrc < 0 || qsrc >= n_src) qsrc = 0;  // a bad index never reads outside q
    }
    const u32x4* src = reinterpret_cast<const u32x4*>(q + qsrc * q_stride + (int64_t)h * D + 8 * g);
    const uint32_t flip = th < 0.0f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = src[2 * ks] ^ flip;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(qf[ks]));  // keep Q resident, never re-read
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  f32x16 sa[2];  // S^T accumulators of the two 32-key halves
  u32x4 pf[4];   // P^T operands of the 4 PV steps (16 keys each)

  const int ntiles = (q_end + kBN - 1) / kBN;
  const int wlast = qw0 + 31;  // this wave's last query row

  // Staging registers, two sets (set = tile parity): a tile's global loads are
  // issued at the start of one half-step and stored to LDS at the end of the
  // next, so they have two half-steps to land.
  u32x4 sreg[2][4];
  float sr[2] = {0.0f, 0.0f};
  if (stage_k) {
    if (ntiles > 0) {
      load_k<D, GATHER>(stg, rk, rs, koff, row_bytes, 0, gtid, sreg[0], sr[0], sidx, q_end);
      store_k<D, G>(stg, sm, 0, gtid, sreg[0], sr[0], ratio);
    }
    if (ntiles > 1) load_k<D, GATHER>(stg, rk, rs, koff, row_bytes, kBN, gtid, sreg[1], sr[1], sidx, q_end);
  }
  __syncthreads();

  // One half-step; P = hs & 1 (compile time, so the register sets are static).
  auto half_step = [&](int hs, auto p_) {
    constexpr int P = decltype(p_)::value;
    // loads: K tile hs + 2 (threads 0-255) and V tile hs (threads 256-511) into set P
    if (stage_k) {
      if (hs + 2 < ntiles)
        load_k<D, GATHER>(stg, rk, rs, koff, row_bytes, (hs + 2) * kBN, gtid, sreg[P], sr[P], sidx, q_end);
    } else {
      if (hs < ntiles) load_v<D, GATHER>(stg, rv, voff, row_bytes, hs * kBN, sreg[P], sidx, q_end);
    }

    if (P == grp) {
      // MFMA phase: PV of tile hs - 2, then QK of tile hs
      const int jp = hs - 2;
      if (jp >= 0 && jp * kBN <= wlast) {
        const uint16_t* vt = sm.vt[jp & 1];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const uint16_t* vrow = vt + (dt * 32 + l32) * AttnSmem<D>::vLd + 16 * s4 + 4 * g;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
            o[dt] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[s4], o[dt]);
          }
        }
        // keep 4 V fragment reads in flight ahead of the MFMAs (left alone, the
        // compiler waits for each read right before its MFMA)
        sched_reads_ahead<4 * (D / 32), 4 * (D / 32), 8>();
      }
      const int jq = hs;
      if (jq < ntiles && jq * kBN <= wlast) {
        const float* bias = sm.s[jq & 1][hl];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 bv = *reinterpret_cast<const f32x4*>(&bias[hf * 32 + 8 * q4 + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sa[hf][4 * q4 + e] = QTAU ? bv[e] * inv_cs : bv[e];
          }
        const uint16_t* krow0 = &sm.k[jq & 1][l32 * AttnSmem<D>::kLd + 8 * g];
        const uint16_t* krow1 = krow0 + 32 * AttnSmem<D>::kLd;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(krow0 + 16 * ks);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(krow1 + 16 * ks);
          sa[0] = mfma32(a0, qf[ks], sa[0]);
          sa[1] = mfma32(a1, qf[ks], sa[1]);
        }
        sched_reads_ahead<D / 8, 8 + D / 8, 8 + 8>();  // the 8 bias reads and 8 K fragments ahead
      }
    } else {
      // softmax phase of tile hs - 1
      const int js = hs - 1;
      if (js >= 0 && js < ntiles && js * kBN <= wlast)
        softmax_tile<D>(js * kBN, qrow, qw0, n, g, cs, sa, m_run, l_run, o, pf);
    }

    // stores last: K tile hs + 1 and V tile hs - 1 from set P ^ 1 (loaded one
    // half-step ago, so each global load has two half-steps to land) into the
    // buffers nobody reads during this half-step
    if (stage_k) {
      if (hs + 1 < ntiles) store_k<D, G>(stg, sm, P ^ 1, gtid, sreg[P ^ 1], sr[P ^ 1], ratio);
    } else {
      if (hs >= 1 && hs - 1 < ntiles) store_v<D>(stg, sm, P ^ 1, sreg[P ^ 1]);
    }
    __syncthreads();
  };
  for (int hs = 0; hs < ntiles + 2; hs += 2) {
    half_step(hs, std::integral_constant<int, 0>());
    if (hs + 1 < ntiles + 2) half_step(hs + 1, std::integral_constant<int, 1>());
  }

  // Merge the two groups through LDS (each finishes half of the head dims).
  merge_and_store<D>(reinterpret_cast<float*>(&sm), grp, wave, lane, g, l32, o, m_run, l_run, qrow, n, seg, q_stride, h,
                     hq, lse, out);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS staging (compacted rows with a per-head or per-query
// temperature, and gathered rows for prompts of up to 8192 kept rows, whose
// source-row indices are kept in LDS: each DMA lane then reads its 16 bytes
// from the kept row's source row).
//
// The same schedule, but K, V and the key scores go from global memory straight
// into LDS (buffer loads with the LDS destination), so no staging registers and
// no LDS store instructions.  Three LDS stages per operand.  In half-step hs
// the group in its softmax phase issues the DMAs of V tile hs and of K tile
// hs + 2 (with its scores) at the start, each into a stage nobody reads during
// hs; the MFMA-phase group issues none, so the issue of the DMAs (which can
// stall while the memory pipeline takes them) overlaps exp2 and VALU work
// instead of delaying matrix work (2-4 % faster than V waves issuing V at the
// start of every half-step and K waves K at its end).  A group waits (vmcnt 0)
// for the DMAs it issued one half-step before at the end of its MFMA phase,
// so every tile has about two half-steps to land.  The barriers are plain
// s_barrier with explicit waits: a workgroup fence would also wait for the
// DMAs just issued.
//
// Both tiles are row-major with their 16-byte chunks swizzled per row, for
// the 256-byte (64-bank) LDS cycle of gfx950.  K: chunk c of row r sits at
// c ^ (r & 15) (D = 128) or c ^ ((r >> 1) & 7) (D = 64), so the 16 rows a
// cycle of QK fragment reads touches land on 16 distinct chunk slots.  V:
// chunk c of row r sits at c ^ 4 (r & 3) (D = 128) or c ^ 4 ((r >> 1) & 1)
// (D = 64); the PV operand V^T is read with ds_read_b64_tr_b16, where 16 lanes
// fetch a 4-key x 16-dim block and each lane receives the 4 keys of one dim,
// and the 4 rows x 64 bytes of a cycle land on distinct banks.  Out-of-range
// rows read as zeros (the buffer range check also covers the DMA).

template <int D>
struct alignas(16) DmaSmem {
  uint16_t k[3][kBN * D];
  uint16_t v[3][kBN * D];
  float s[3][kBN];  // raw key scores
};

template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

template <int D, int G, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gated_attention_dma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ tau, const float* __restrict__ gain,
    SegTable segs, int hq, int hkv, const int32_t* __restrict__ kept_idx, int64_t n_src,
    const int32_t* __restrict__ qpos, float* __restrict__ lse, uint16_t* __restrict__ out, int split_t, int ns_max,
    int* __restrict__ split_status, int* __restrict__ split_cnt, float* __restrict__ split_part) {
  constexpr bool GATHER = MODE == kGather;
  constexpr bool QTAU = MODE == kQueryTau;
  constexpr int kBM = 128 / G;
  constexpr int kWavesPerHead = 4 / G;
  constexpr int NC = D / 8;   // 16-byte chunks per row
  constexpr int NJ = NC / 4;  // DMA instructions per staging wave per tile (64 NC chunks over 4 waves)
  __shared__ DmaSmem<D> sm;
  static_assert(8 * kMergeRec<D> * 4 <= (int)sizeof(DmaSmem<D>), "group merge fits in LDS");
  __shared__ int32_t sidx[GATHER ? kDmaGatherRows : 1];  // source rows of the kept rows [0, q_end)

  const tg_segment seg = segs.at_uniform(blockIdx.z);
  const int n = seg.kept_len;
  // Work item: query tile qi (kBM rows) and key tiles [t0, t1) of it.  With split_t > 0 every query tile with
  // more than split_t key tiles is split in two items, an owner (key tiles [0, split_t)) and a helper (the rest);
  // each publishes its partial result and the second to finish merges both.  blockIdx.y runs over the owners,
  // then the helpers, then the whole tiles, each longest first.
  const int nq = (n + kBM - 1) / kBM;
  const int qs = (split_t > 0 && n > kBN * split_t) ? min(nq, (kBN * split_t) / kBM) : nq;  // first split tile
  const int ns = nq - qs;
  const int y = blockIdx.y;
  int qi, role;  // role 0: whole tile, 1: owner, 2: helper
  if (y < ns) {
    qi = nq - 1 - y;
    role = 1;
  } else if (y < 2 * ns) {
    qi = nq - 1 - (y - ns);
    role = 2;
  } else if (y < 2 * ns + qs) {
    qi = qs - 1 - (y - 2 * ns);
    role = 0;
  } else {
    return;  // uniform: past this prompt's items
  }
  const int q0 = qi * kBM;
  const int q_end = min(q0 + kBM, n);
  const int t0 = role == 2 ? split_t : 0;
  const int t1 = role == 1 ? split_t : (q_end + kBN - 1) / kBN;
  if (GATHER) {
    for (int i = threadIdx.x; i < q_end; i += kThreads) sidx[i] = kept_idx[seg.kept_start + i];
    __syncthreads();
  }

  const int tid = threadIdx.x;
  const int grp = tid >> 8;
  const int gtid = tid & 255;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(gtid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int c = blockIdx.x;
  const int hl = wave / kWavesPerHead;
  const int h = c * G + hl;
  const int qw0 = q0 + (wave % kWavesPerHead) * 32;
  const int qrow = qw0 + l32;

  const int64_t q_stride = (int64_t)hq * D;
  const int64_t kv_stride = (int64_t)hkv * D;
  const int64_t row0 = GATHER ? 0 : seg.kept_start;               // first row of the K/V/score buffers
  const uint32_t nrows = GATHER ? (uint32_t)n_src : (uint32_t)n;  // rows the buffers cover
  const uint16_t* kb = k + row0 * kv_stride + (int64_t)c * D;
  const uint16_t* vb = v + row0 * kv_stride + (int64_t)c * D;
  const bool use_bias = key_score != nullptr && gain != nullptr;
  const uint32_t row_bytes = (uint32_t)kv_stride * 2u;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, nrows * row_bytes - (uint32_t)c * D * 2u);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, nrows * row_bytes - (uint32_t)c * D * 2u);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(use_bias ? key_score + row0 : key_score, use_bias ? nrows * 4u : 0u);
  const bool stage_k = grp == 0;  // threads 0-255 stage the first two K tiles

  // DMA source offsets inside a tile: chunk slot (j 4 + wave) 64 + lane holds row drow[j], chunk dcolk[j] (K)
  // or dcolv[j] (V); every wave stages both tensors
  int drow[NJ];
  uint32_t dcolk[NJ], dcolv[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int p = (j * 4 + wave) * 64 + lane;
    const int r = p / NC;
    drow[j] = r;
    dcolk[j] = (uint32_t)((p % NC) ^ kswz<D>(r)) * 16u;
    dcolv[j] = (uint32_t)((p % NC) ^ vswz<D>(r)) * 16u;
  }
  // byte offset of a tile row in the K/V buffers (gathered: its source row; rows at or past q_end read as zeros)
  auto row_off = [&](int row) -> uint32_t {
    if (!GATHER) return (uint32_t)row * row_bytes;
    return row < q_end ? (uint32_t)sidx[row] * row_bytes : kPastRange;
  };
  auto dma_k = [&](int lt, int buf) {  // lt: tile index inside the item
    const int tile = t0 + lt;
    if (!GATHER) {
      const uint32_t soff = (uint32_t)(tile * kBN) * row_bytes;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        dma16(rk, &sm.k[buf][(j * 4 + wave) * 64 * 8], (uint32_t)drow[j] * row_bytes + dcolk[j], soff);
      if (lane < 16) dma4(rs, &sm.s[buf][16 * wave], (uint32_t)(16 * wave + lane) * 4u, (uint32_t)(tile * kBN) * 4u);
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t ro = row_off(tile * kBN + drow[j]);
        dma16(rk, &sm.k[buf][(j * 4 + wave) * 64 * 8], ro == kPastRange ? ro : ro + dcolk[j], 0u);
      }
      if (lane < 16) {
        const int row = tile * kBN + 16 * wave + lane;
        dma4(rs, &sm.s[buf][16 * wave], row < q_end ? (uint32_t)sidx[row] * 4u : kPastRange, 0u);
      }
    }
  };
  auto dma_v = [&](int lt, int buf) {
    const int tile = t0 + lt;
    if (!GATHER) {
      const uint32_t soff = (uint32_t)(tile * kBN) * row_bytes;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        dma16(rv, &sm.v[buf][(j * 4 + wave) * 64 * 8], (uint32_t)drow[j] * row_bytes + dcolv[j], soff);
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t ro = row_off(tile * kBN + drow[j]);
        dma16(rv, &sm.v[buf][(j * 4 + wave) * 64 * 8], ro == kPastRange ? ro : ro + dcolv[j], 0u);
      }
    }
  };

  const float base = kLog2e / __builtin_sqrtf((float)D);
  float th = tau != nullptr ? tau[h] : 1.0f;
  const float rat = !use_bias ? 0.0f
                    : QTAU    ? gain[h] * kLog2e
                              : gain[h] * kLog2e / __builtin_fmaxf(__builtin_fabsf(th) * base, 1e-30f);
  if (QTAU) {
    const int r = qrow < n ? qrow : n - 1;
    const float sp = th > 20.0f ? th : log1pf(expf(th));
    const float pr = (float)max(2, qpos[seg.kept_start + r] + 1);
    th = sp * (logf((float)(r + 1)) / logf(pr));
  }
  const float cs = __builtin_fmaxf(__builtin_fabsf(th) * base, 1e-30f);
  const float inv_cs = QTAU ? 1.0f / cs : 1.0f;

  const int ntiles = t1 - t0;  // key tiles of the item; local tile j is key tile t0 + j
  const int wlast = qw0 + 31;

  u32x4 qf[D / 16];
  {
    const int r = qrow < n ? qrow : n - 1;
    int64_t qsrc = (int64_t)seg.kept_start + r;
    if (GATHER) {
      qsrc = sidx[r];
      if (qsrc < 0 || qsrc >= n_src) qsrc = 0;  // a bad index never reads outside q
    }
    const u32x4* src = reinterpret_cast<const u32x4*>(q + qsrc * q_stride + (int64_t)h * D + 8 * g);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = src[2 * ks];
  }
  if (stage_k) {
    dma_k(0, 0);
    if (ntiles > 1) dma_k(1, 1);
  }
  {
    const uint32_t flip = th < 0.0f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] ^= flip;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  // LDS element offsets of this lane's fragment reads inside a tile.
  // K (QK A operand): row l32 (+32 for the second half), chunk 2 ks + g.
  uint32_t kaddr[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) kaddr[ks] = (uint32_t)(l32 * D + (((2 * ks + g) ^ kswz<D>(l32)) * 8));
  // V (PV A operand, transposing read): 16-lane group qg = lane / 16 covers dims 32 dt + 16 (qg % 2) + 0..15
  // and keys 4 (qg / 2) + 0..3 of a 16-key step; source lane s points at row 4 g + s / 4, dims + 4 (s % 4).
  uint32_t vaddr[D / 32];
  {
    const int s = lane & 15, qg = lane >> 4;
    const int r = 4 * g + (s >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int cc = 4 * dt + 2 * (qg & 1) + ((s & 3) >> 1);
      vaddr[dt] = (uint32_t)(r * D + ((cc ^ vswz<D>(r)) * 8) + 4 * (s & 1));
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  f32x16 sa[2];
  u32x4 pf[4];

  if (stage_k && ntiles > 1)
    wait_vm<NJ + 1>();  // K tile 0 landed; tile 1 may still be in flight
  else
    wait_vm<0>();
  lds_barrier();

  int b_cur = 0;  // hs % 3
  auto half_step = [&](int hs, auto p_) {
    constexpr int P = decltype(p_)::value;
    const int b1 = b_cur == 2 ? 0 : b_cur + 1;  // (hs + 1) % 3 == (hs - 2) % 3
    const int b2 = b1 == 2 ? 0 : b1 + 1;        // (hs + 2) % 3
    const bool my_dma = P != grp;  // the group in its softmax phase stages this half-step's tiles
    if (my_dma) {
      if (hs < ntiles) dma_v(hs, b_cur);        // V tile hs
      if (hs + 2 < ntiles) dma_k(hs + 2, b2);   // K tile hs + 2 and its scores
    }

    if (P == grp) {
      const int jp = hs - 2;
      if (jp >= 0 && (t0 + jp) * kBN <= wlast) {
        const uint16_t* vt = sm.v[b1];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            typedef short short4v __attribute__((ext_vector_type(4)));
            const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(vt + vaddr[dt] + 16 * s4 * D));
            const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(vt + vaddr[dt] + (16 * s4 + 8) * D));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            o[dt] = mfma32(u32x4{l2[0], l2[1], h2[0], h2[1]}, pf[s4], o[dt]);
          }
        }
        sched_two_reads_ahead<4 * (D / 32), 8>();
      }
      const int jq = hs;
      if (jq < ntiles && (t0 + jq) * kBN <= wlast) {
        const float* bias = sm.s[b_cur];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 bv = *reinterpret_cast<const f32x4*>(&bias[hf * 32 + 8 * q4 + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sa[hf][4 * q4 + e] = QTAU ? (bv[e] * rat) * inv_cs : bv[e] * rat;
          }
        const uint16_t* kt = sm.k[b_cur];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(kt + kaddr[ks]);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(kt + kaddr[ks] + 32 * D);
          sa[0] = mfma32(a0, qf[ks], sa[0]);
          sa[1] = mfma32(a1, qf[ks], sa[1]);
        }
        sched_reads_ahead<D / 8, 8 + D / 8, 8 + 8>();
      }
    } else {
      // softmax phase of tile hs - 1
      const int js = hs - 1;
      if (js >= 0 && js < ntiles && (t0 + js) * kBN <= wlast)
        softmax_tile<D>((t0 + js) * kBN, qrow, qw0, n, g, cs, sa, m_run, l_run, o, pf);
    }

    // the MFMA-phase group staged K tile hs + 1 and V tile hs - 1 one half-step ago: they must have landed;
    // the softmax group's fresh DMAs may stay in flight
    if (!my_dma) wait_vm<0>();
    lds_barrier();
    b_cur = b1;
  };
  for (int hs = 0; hs < ntiles + 2; hs += 2) {
    half_step(hs, std::integral_constant<int, 0>());
    if (hs + 1 < ntiles + 2) half_step(hs + 1, std::integral_constant<int, 1>());
  }

  // Merge the two groups through LDS (each finishes half of the head dims; split tiles also merge across items).
  if (role == 0) {
    merge_and_store<D>(reinterpret_cast<float*>(&sm), grp, wave, lane, g, l32, o, m_run, l_run, qrow, n, seg, q_stride,
                       h, hq, lse, out);
  } else {
    const int slot = (blockIdx.z * hkv + c) * ns_max + (nq - 1 - qi);
    constexpr int kPart = 4 * (D * 32 + 64);  // floats per half: 4 waves x (O^T, m, l)
    merge_split<D>(reinterpret_cast<float*>(&sm), grp, wave, lane, g, l32, o, m_run, l_run, qrow, n, seg, q_stride, h,
                   hq, lse, out, split_part + ((int64_t)slot * 2 + (role - 1)) * kPart,
                   split_part + ((int64_t)slot * 2 + (2 - role)) * kPart, split_cnt + 2 * slot, split_status);
  }
}

// Splitting the long query tiles of one prompt.  Items are scheduled in
// blockIdx order on the CUs that serve a KV head (blockIdx.x is the head, so a
// head's workgroups share an XCD); an item of k 64-key tiles costs about
// k + 2 half-steps plus kItemFixed for its prologue and output (measured on
// MI355X at head_dim 128: ~1.04 us per half-step, ~5 us fixed), and a split
// half kItemMerge more (fitted to measured split times at 500-3000 kept
// rows).  The split point T (owner: key tiles [0, T), helper: the rest)
// minimises the modelled makespan of list scheduling in the kernel's item
// order; splitting is used only for a single prompt whose modelled time drops
// below kSplitGain of the unsplit one.
constexpr double kItemFixed = 4.8, kItemMerge = 3.5, kSplitGain = 0.93;

int device_cu_count() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n > 0) return n;
  int dev = 0;
  n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  cached.store(n, std::memory_order_relaxed);
  return n;
}

double list_makespan(const std::vector<double>& items, int ncu) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < ncu; ++i) free_at.push(0.0);
  double end = 0.0;
  for (double c : items) {
    const double t = free_at.top() + c;
    free_at.pop();
    free_at.push(t);
    end = std::max(end, t);
  }
  return end;
}

struct SplitPlan {
  int t = 0;       // split point in 64-key tiles; 0: no split
  int ns_max = 0;  // split query tiles of the longest prompt
};

SplitPlan choose_split(const tg_plan_info& info, int G, int hkv) {
  SplitPlan sp;
  const int n = (int)info.max_kept_len;
  if (info.n_seg != 1 || n <= 0 || hkv <= 0) return sp;
  const int kBM = 128 / G;
  const int nq = (n + kBM - 1) / kBM;
  const int per_head = std::max(1, device_cu_count() / hkv);
  if (nq > 2 * per_head || nq > 128) return sp;  // enough whole tiles to balance the CUs (the model's search
                                                 // is quadratic in nq: bounded here)
  static std::mutex mu;
  static std::map<std::tuple<int, int, int>, SplitPlan> cache;
  const auto key = std::make_tuple(n, G, per_head);
  {
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  auto nk = [&](int qi) { return (std::min((qi + 1) * kBM, n) + kBN - 1) / kBN; };
  std::vector<double> items;
  auto model = [&](int T) {
    items.clear();
    for (int qi = nq - 1; qi >= 0; --qi)
      if (T > 0 && nk(qi) > T) items.push_back(kItemFixed + kItemMerge + T + 2);
    for (int qi = nq - 1; qi >= 0; --qi)
      if (T > 0 && nk(qi) > T) items.push_back(kItemFixed + kItemMerge + (nk(qi) - T) + 2);
    for (int qi = nq - 1; qi >= 0; --qi)
      if (T == 0 || nk(qi) <= T) items.push_back(kItemFixed + nk(qi) + 2);
    return list_makespan(items, per_head);
  };
  const double whole = model(0);
  double best = whole;
  int best_t = 0;
  for (int T = 1; T < nk(nq - 1); ++T) {
    const double ms = model(T);
    if (ms < best) {
      best = ms;
      best_t = T;
    }
  }
  if (best_t > 0 && best < kSplitGain * whole) {
    sp.t = best_t;
    sp.ns_max = nq - std::min(nq, (kBN * best_t) / kBM);
  }
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = sp;
  return sp;
}

// workspace: a 256-byte header (the int status word first), int flags
// [n_seg x hkv x ns_max][2] (arrivals, record ready) padded to 256 bytes, then
// the fp32 records [slot][half][4 waves][D x 32 + 64]
constexpr size_t kSplitHeader = 256;
size_t split_flag_bytes(size_t slots) { return (slots * 8 + 255) / 256 * 256; }
size_t split_bytes(const SplitPlan& sp, const tg_plan_info& info, int hkv, int D) {
  if (sp.t == 0) return 0;
  const size_t slots = (size_t)info.n_seg * hkv * sp.ns_max;
  return kSplitHeader + split_flag_bytes(slots) + slots * 2 * 4 * ((size_t)D * 32 + 64) * 4;
}

template <int D, int G>
hipError_t launch_dg(const void* q, const void* k, const void* v, const float* ks, const float* tau,
                     const float* gain, const tg_segment* segs_in, const tg_plan_info& info, int hq, int hkv,
                     const int32_t* kept_idx, int64_t n_src, const int32_t* qpos, float* lse, void* out,
                     hipStream_t stream, void* split_ws) {
  const SegTable segs = seg_table(segs_in, info);
  constexpr int kBM = 128 / G;
  int ntiles = (info.max_kept_len + kBM - 1) / kBM;
  if (ntiles == 0) return hipSuccess;
  SplitPlan sp;
  if (split_ws != nullptr && !(kept_idx != nullptr && info.max_kept_len > kDmaGatherRows)) sp = choose_split(info, G, hkv);
  int* split_status = nullptr;
  int* split_cnt = nullptr;
  float* split_part = nullptr;
  if (sp.t > 0) {
    const size_t slots = (size_t)info.n_seg * hkv * sp.ns_max;
    split_status = reinterpret_cast<int*>(split_ws);
    split_cnt = reinterpret_cast<int*>(reinterpret_cast<char*>(split_ws) + kSplitHeader);
    split_part = reinterpret_cast<float*>(reinterpret_cast<char*>(split_ws) + kSplitHeader + split_flag_bytes(slots));
    ntiles += sp.ns_max;
  }
  dim3 grid(hkv, ntiles, info.n_seg);
  auto* qb = reinterpret_cast<const uint16_t*>(q);
  auto* kb = reinterpret_cast<const uint16_t*>(k);
  auto* vb = reinterpret_cast<const uint16_t*>(v);
  auto* ob = reinterpret_cast<uint16_t*>(out);
  if (kept_idx != nullptr && info.max_kept_len <= kDmaGatherRows)
    hipLaunchKernelGGL((gated_attention_dma_kernel<D, G, kGather>), grid, dim3(kThreads), 0, stream, qb, kb, vb, ks,
                       tau, gain, segs, hq, hkv, kept_idx, n_src, nullptr, lse, ob, sp.t, sp.ns_max, split_status, split_cnt,
                       split_part);
  else if (kept_idx != nullptr)
    hipLaunchKernelGGL((gated_attention_kernel<D, G, kGather>), grid, dim3(kThreads), 0, stream, qb, kb, vb, ks, tau,
                       gain, segs, hq, hkv, kept_idx, n_src, nullptr, lse, ob);
  else if (qpos != nullptr)
    hipLaunchKernelGGL((gated_attention_dma_kernel<D, G, kQueryTau>), grid, dim3(kThreads), 0, stream, qb, kb, vb, ks,
                       tau, gain, segs, hq, hkv, nullptr, (int64_t)0, qpos, lse, ob, sp.t, sp.ns_max, split_status, split_cnt,
                       split_part);
  else
    hipLaunchKernelGGL((gated_attention_dma_kernel<D, G, kCompacted>), grid, dim3(kThreads), 0, stream, qb, kb, vb,
                       ks, tau, gain, segs, hq, hkv, nullptr, (int64_t)0, nullptr, lse, ob, sp.t, sp.ns_max, split_status, split_cnt,
                       split_part);
  return hipGetLastError();
}

}  // namespace

size_t attention_prefill_workspace_bytes(const tg_plan_info& info, int hq, int hkv, int head_dim) {
  if (hkv <= 0 || hq % hkv != 0) return 0;
  const int G = hq / hkv;
  if (!(G == 1 || G == 2 || G == 4)) return 0;
  return split_bytes(choose_split(info, G, hkv), info, hkv, head_dim);
}

hipError_t launch_gated_attention(const void* q, const void* k, const void* v, const float* key_score,
                                  const float* tau, const float* gain, const tg_segment* segs,
                                  const tg_plan_info& info, int hq, int hkv, int head_dim, const int32_t* kept_idx,
                                  int64_t n_src, const int32_t* qpos, float* lse, void* out, hipStream_t stream,
                                  void* split_ws) {
  const int G = hq / hkv;
#define TG_ATTN_CASE(DD, GG) \
  if (head_dim == DD && G == GG) \
    return launch_dg<DD, GG>(q, k, v, key_score, tau, gain, segs, info, hq, hkv, kept_idx, n_src, qpos, lse, out, \
                             stream, split_ws);
  TG_ATTN_CASE(128, 1)
  TG_ATTN_CASE(128, 2)
  TG_ATTN_CASE(128, 4)
  TG_ATTN_CASE(64, 1)
  TG_ATTN_CASE(64, 2)
  TG_ATTN_CASE(64, 4)
#undef TG_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace tg
