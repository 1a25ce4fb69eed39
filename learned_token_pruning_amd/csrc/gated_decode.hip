// Token-gated attention, one decode step over a pruned KV cache (gfx950).
//
// "TokenGate 与 T2Quant ... 精读", section 4.1: pruned tokens leave no KV entry,
// the tokens being generated are not prunable (score 0), and at decode time
// the gate term is an additive attention mask.  For sequence b, query head h
// (key/value head c = h / G) and cache rows j < len_b:
//   z_j = tau_h (q_h . k_j) / sqrt(D) + g_h s_j,   out[b, h] = sum_j softmax_j(z) v_j
//
// The step reads every cached K/V row once and does G multiply-adds per
// element read, so it is bound by HBM, not by the matrix cores: plain fp32
// VALU arithmetic, laid out for coalesced row reads.  Split-KV in two kernels:
//
// decode_partial: one workgroup per (KV head, 256-row chunk, sequence); the
// KV head is the fastest grid index, so the workgroups dispatched together
// read the neighbouring head slices of the same cache rows.  The
// D/8 lanes of a row read it as D/8 contiguous 16-byte pieces (a wave reads
// 64/(D/8) whole rows per instruction), so every K and V load of the chunk is
// issued up front.  q . k is a lane-local 8-term dot product per head plus a
// butterfly over the row's lanes; each wave then runs the softmax over its 64
// rows in the exp2 domain (max, exp2, sum) and accumulates P V with the same
// row layout, and the four waves are merged through LDS into one partial
// (max, sum, unnormalised output) per head and chunk.
//
// decode_combine: one workgroup per (query head, sequence) merges the chunk
// partials in chunk order and writes the bf16 output (0 for an empty cache).
#include "common.h"

namespace tg {
namespace {

constexpr int kChunk = 256;        // cache rows per workgroup
constexpr int kDecThreads = 256;   // 4 waves x 64 rows
constexpr float kLog2eD = 1.4426950408889634f;

template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const float* __restrict__ key_score, const float* __restrict__ tau, int tau_per_query,
    const float* __restrict__ gain, const int32_t* __restrict__ lens, int64_t cap, int hq, int hkv, int n_chunks,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int LPK = D / 8;       // lanes per cache row (16 bytes each)
  constexpr int KPI = 64 / LPK;    // rows per wave instruction
  constexpr int NIT = 64 / KPI;    // instructions per wave (64 rows)
  __shared__ float sp[G][kChunk];  // exp2-domain logits, then probabilities
  __shared__ float wml[4][G][2];   // per-wave max and sum
  __shared__ float wo[4][G][D];    // per-wave unnormalised outputs

  const int b = blockIdx.z, c = blockIdx.x, ch = blockIdx.y;
  const int len = min(max(lens[b], 0), (int)min(cap, (int64_t)0x7fffffff));
  const int k0 = ch * kChunk;
  if (k0 >= len) return;  // uniform: nothing of this sequence in the chunk
  const int kn = min(kChunk, len - k0);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane % LPK;  // 16-byte piece of the row: dims 8 sub .. 8 sub + 7
  const int ks = lane / LPK;   // row slot inside one instruction
  const uint32_t row_bytes = (uint32_t)hkv * D * 2u;
  const uint16_t* kb = kc + (((int64_t)b * cap + k0) * hkv + c) * D;
  const uint16_t* vb = vc + (((int64_t)b * cap + k0) * hkv + c) * D;
  // rows past the sequence read as zeros (range ends with row kn - 1)
  const uint32_t range = (uint32_t)(kn - 1) * row_bytes + (uint32_t)D * 2u;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, range);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, range);

  // every K and V piece of the wave's 64 rows is requested first
  u32x4 kr[NIT], vr[NIT];
  const uint32_t voff = (uint32_t)(64 * wave + ks) * row_bytes + (uint32_t)sub * 16u;
#pragma unroll
  for (int it = 0; it < NIT; ++it) kr[it] = buf_load16(rk, voff + (uint32_t)(it * KPI) * row_bytes, 0u);
#pragma unroll
  for (int it = 0; it < NIT; ++it) vr[it] = buf_load16(rv, voff + (uint32_t)(it * KPI) * row_bytes, 0u);

  // q of the G heads, pre-scaled by the exp2-domain logit scale tau log2(e) / sqrt(D)
  const float base = kLog2eD / __builtin_sqrtf((float)D);
  float qf[G][8];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const int h = c * G + gg;
    const float th = tau == nullptr ? 1.0f : tau[tau_per_query ? (int64_t)b * hq + h : h];
    const u32x4 w = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * hq + h) * D + 8 * sub);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[gg][2 * e] = bf16_lo(w[e]) * (th * base);
      qf[gg][2 * e + 1] = bf16_hi(w[e]) * (th * base);
    }
  }
  const bool use_bias = key_score != nullptr && gain != nullptr;

  // logits of the wave's rows (lanes with sub == 0 publish them)
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int jl = 64 * wave + it * KPI + ks;  // row inside the chunk
    float sb = 0.0f;
    if (use_bias && sub == 0 && jl < kn) sb = key_score[(int64_t)b * cap + k0 + jl] * kLog2eD;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a = __builtin_fmaf(qf[gg][2 * e], bf16_lo(kr[it][e]), a);
        a = __builtin_fmaf(qf[gg][2 * e + 1], bf16_hi(kr[it][e]), a);
      }
      a = group_sum<LPK>(a);
      if (sub == 0) sp[gg][jl] = jl < kn ? (use_bias ? __builtin_fmaf(gain[c * G + gg], sb, a) : a) : -__builtin_inff();
    }
  }
  __syncthreads();

  // softmax over the wave's 64 rows: lane j owns row 64 wave + j
  float mw[G], lw[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float z = sp[gg][64 * wave + lane];
    const float m = wave_max(z);
    // a wave whose rows are all past the sequence keeps max -inf and weight 0
    const float p = m == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(z - m);
    const float l = wave_sum(p);
    mw[gg] = m;
    lw[gg] = l;
    sp[gg][64 * wave + lane] = p;
  }
  __syncthreads();

  // P V over the wave's rows, in the load layout; then sum the KPI row slots
  float o[G][8];
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[gg][e] = 0.0f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int jl = 64 * wave + it * KPI + ks;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float p = sp[gg][jl];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[gg][2 * e] = __builtin_fmaf(p, bf16_lo(vr[it][e]), o[gg][2 * e]);
        o[gg][2 * e + 1] = __builtin_fmaf(p, bf16_hi(vr[it][e]), o[gg][2 * e + 1]);
      }
    }
  }
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      o[gg][e] = stride_sum<LPK>(o[gg][e]);
  if (ks == 0) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
#pragma unroll
      for (int e = 0; e < 8; ++e) wo[wave][gg][8 * sub + e] = o[gg][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      wml[wave][gg][0] = mw[gg];
      wml[wave][gg][1] = lw[gg];
    }
  }
  __syncthreads();

  // merge the four waves (fixed order) into the chunk's partial
  const int64_t slot = ((int64_t)b * hkv + c) * n_chunks + ch;  // [b][c][chunk]
  for (int i = tid; i < G * D; i += kDecThreads) {
    const int gg = i / D, d = i % D;
    float m = wml[0][gg][0];
#pragma unroll
    for (int w = 1; w < 4; ++w) m = __builtin_fmaxf(m, wml[w][gg][0]);
    float acc = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mwv = wml[w][gg][0];
      const float a = mwv == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mwv - m);
      acc = __builtin_fmaf(a, wo[w][gg][d], acc);
      l = __builtin_fmaf(a, wml[w][gg][1], l);
    }
    part_o[(slot * G + gg) * D + d] = acc;
    if (d == 0) {
      part_ml[(slot * G + gg) * 2] = m;
      part_ml[(slot * G + gg) * 2 + 1] = l;
    }
  }
}

// One workgroup of D threads per (query head, sequence).  The chunk maxima
// and sums are read in parallel (thread i takes chunks i, i + D, ...), the
// maximum and the chunk weights go through LDS, then every thread sums its
// output dimension over the chunks in chunk order (four loads in flight).
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const int32_t* __restrict__ lens, int64_t cap, int hq,
                                                           int hkv, int n_chunks, const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           uint16_t* __restrict__ out) {
  constexpr int kW = D / 64;
  __shared__ float wred[kW];
  __shared__ float wts[D];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x, lane = d & 63, wv = d >> 6;
  const int G = hq / hkv, c = h / G, gg = h % G;
  const int len = min(max(lens[b], 0), (int)min(cap, (int64_t)0x7fffffff));
  const int nc = (len + kChunk - 1) / kChunk;
  const int64_t slot0 = ((int64_t)b * hkv + c) * n_chunks;
  float m = -__builtin_inff();
  for (int i = d; i < nc; i += D) m = __builtin_fmaxf(m, part_ml[((slot0 + i) * G + gg) * 2]);
  m = wave_max(m);
  if (lane == 0) wred[wv] = m;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kW; ++w) m = __builtin_fmaxf(m, wred[w]);
  float acc = 0.0f, l = 0.0f;
  for (int i0 = 0; i0 < nc; i0 += D) {
    const int cnt = min(D, nc - i0);
    __syncthreads();  // the previous group's weights are consumed
    if (d < cnt) wts[d] = __builtin_amdgcn_exp2f(part_ml[((slot0 + i0 + d) * G + gg) * 2] - m);
    __syncthreads();
    int i = 0;
    for (; i + 4 <= cnt; i += 4) {
      float o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = part_o[((slot0 + i0 + i + u) * G + gg) * D + d];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc = __builtin_fmaf(wts[i + u], o[u], acc);
        l = __builtin_fmaf(wts[i + u], part_ml[((slot0 + i0 + i + u) * G + gg) * 2 + 1], l);
      }
    }
    for (; i < cnt; ++i) {
      acc = __builtin_fmaf(wts[i], part_o[((slot0 + i0 + i) * G + gg) * D + d], acc);
      l = __builtin_fmaf(wts[i], part_ml[((slot0 + i0 + i) * G + gg) * 2 + 1], l);
    }
  }
  const float r = nc == 0 ? 0.0f : acc / l;
  out[((int64_t)b * hq + h) * D + d] = (uint16_t)f32_to_bf16(r);
}

template <int D, int G>
hipError_t launch_decode_dg(const void* q, const void* kc, const void* vc, const float* ks, const float* tau,
                            int tau_per_query, const float* gain, const int32_t* lens, int batch, int64_t cap,
                            int hq, int hkv, void* out, void* workspace, hipStream_t stream) {
  const int n_chunks = (int)((cap + kChunk - 1) / kChunk);
  float* part_o = reinterpret_cast<float*>(workspace);
  float* part_ml = part_o + (int64_t)batch * hq * n_chunks * D;
  if (n_chunks > 0) {  // an empty cache only needs the combine step (zero outputs)
    hipLaunchKernelGGL((decode_partial_kernel<D, G>), dim3(hkv, n_chunks, batch), dim3(kDecThreads), 0, stream,
                       reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(kc),
                       reinterpret_cast<const uint16_t*>(vc), ks, tau, tau_per_query, gain, lens, cap, hq, hkv,
                       n_chunks, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(hq, batch), dim3(D), 0, stream, lens, cap, hq, hkv, n_chunks,
                     part_o, part_ml, reinterpret_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int batch, int hq, int head_dim, int64_t cap) {
  const int64_t n_chunks = (cap + kChunk - 1) / kChunk;
  return (size_t)((int64_t)batch * hq * (n_chunks > 0 ? n_chunks : 1) * (head_dim + 2) * 4);
}

hipError_t launch_gated_decode(const void* q, const void* kc, const void* vc, const float* key_score,
                               const float* tau, int tau_per_query, const float* gain, const int32_t* lens,
                               int batch, int64_t cap, int hq, int hkv, int head_dim, void* out, void* workspace,
                               hipStream_t stream) {
  const int G = hq / hkv;
#define TG_DEC_CASE(DD, GG) \
  if (head_dim == DD && G == GG) \
    return launch_decode_dg<DD, GG>(q, kc, vc, key_score, tau, tau_per_query, gain, lens, batch, cap, hq, hkv, out, \
                                    workspace, stream);
  TG_DEC_CASE(128, 1)
  TG_DEC_CASE(128, 2)
  TG_DEC_CASE(128, 4)
  TG_DEC_CASE(64, 1)
  TG_DEC_CASE(64, 2)
  TG_DEC_CASE(64, 4)
#undef TG_DEC_CASE
  return hipErrorInvalidValue;
}

}  // namespace tg
