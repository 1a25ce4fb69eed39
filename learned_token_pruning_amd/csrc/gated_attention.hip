// Token-gated causal GQA attention over the kept rows, prefill (gfx950).
//
// "TokenGate 与 T2Quant ... 精读", section 4.1, component two: the kept token's
// gate score enters the attention logits as a bias, with a per-(layer, head)
// gain and a temperature:
//   z_rt = tau_h (q_r . k_t) / sqrt(D) + g_h s_t,   t <= r (kept rows, original order)
//
// Flash-style, one pass over the keys with an online softmax in the exp2
// domain.  A workgroup (4 waves) owns one key/value head and a 128/G-row
// query tile of all G query heads sharing it, so every K/V tile staged in LDS
// serves G heads.  Each wave owns 32 query rows of one head.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16).  Scores are computed transposed,
// S^T = K . Q^T, so a lane owns one query column (l % 32) and 16 key rows per
// 32-key half: the softmax row max/sum is a register loop plus one swap with
// the other half-wave.  The output is accumulated transposed too,
// O^T += V^T . P^T, which lets P^T be fed from the score registers without
// any data movement (the key order inside each 16-key MFMA step is permuted
// identically on both operands) and keeps the per-query rescale lane-local.
// V is therefore staged transposed in LDS; K row-major.  Both use padded rows
// so that the 16- and 8-byte LDS reads are bank-conflict free.
//
// The gate bias g_h s_t is fused into the same FMA that applies the
// temperature: x = S * (tau_h log2(e) / sqrt(D)) + (g_h log2(e)) s_t.
// Tiles are launched longest-first (the last query tile of a prompt first).
#include "common.h"

namespace tg {
namespace {

constexpr int kBN = 64;  // keys per tile
constexpr int kThreads = 512;  // two groups of 4 waves
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct AttnSmem {
  static constexpr int kLd = D + 8;        // K row stride (bf16)
  static constexpr int vLd = kBN + 4;      // V^T row stride (bf16)
  uint16_t k[1][kBN * kLd];
  uint16_t vt[1][D * vLd];
  float s[4][kBN];  // gate bias of every key, pre-multiplied by g_h log2(e), one row per query head of the group
};

// Per-thread constant parts of the K/V/score tile loads (byte offsets).
template <int D>
struct TileAddr {
  uint32_t k_off;  // K: D/8 threads per row, 16 bytes each, rows tid / (D/8) + j 256/(D/8)
  uint32_t v_off;  // V: 4 consecutive rows x 8 dims (see store_kv_tile)
  uint32_t s_off;  // score: one key per thread (tid < 64)
  __device__ TileAddr(int tid, uint32_t row_bytes) {
    k_off = (uint32_t)(tid / (D / 8)) * row_bytes + (uint32_t)(tid % (D / 8)) * 16u;
    const int dc = (tid & 1) + 2 * ((tid >> 4) % (D / 16));
    const int kq = ((tid >> 1) & 7) + 8 * (tid / D);
    v_off = (uint32_t)(4 * kq) * row_bytes + (uint32_t)dc * 16u;
    s_off = (uint32_t)tid * 4u;
  }
};

// Buffer loads of one 64-key tile; keys past the prompt read as zeros.
template <int D>
__device__ __forceinline__ void load_kv_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                             __amdgpu_buffer_rsrc_t rs, const TileAddr<D>& ad, uint32_t row_bytes,
                                             int kv0, int tid, u32x4 (&kr)[D / 32], u32x4 (&vr)[4], float& sr) {
  constexpr int kRpi = 256 / (D / 8);  // K rows per load instruction
#pragma unroll
  for (int j = 0; j < D / 32; ++j) kr[j] = buf_load16(rk, ad.k_off, (uint32_t)(kv0 + kRpi * j) * row_bytes);
  if (tid < 2 * D) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = buf_load16(rv, ad.v_off, (uint32_t)(kv0 + i) * row_bytes);
  }
  if (tid < kBN) sr = buf_load4f(rs, ad.s_off, (uint32_t)kv0 * 4u);
}

template <int D, int G>
__device__ __forceinline__ void store_kv_tile(AttnSmem<D>& sm, int buf, int tid, const u32x4 (&kr)[D / 32],
                                              const u32x4 (&vr)[4], float sr, const float (&bscale)[G]) {
  {
    constexpr int kTpr = D / 8;
    constexpr int kRpi = 256 / kTpr;
    const int c = (tid % kTpr) * 8;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
      *reinterpret_cast<u32x4*>(&sm.k[buf][(tid / kTpr + kRpi * j) * AttnSmem<D>::kLd + c]) = kr[j];
  }
  if (tid < 2 * D) {
    const int dc = (tid & 1) + 2 * ((tid >> 4) % (D / 16));
    const int kq = ((tid >> 1) & 7) + 8 * (tid / D);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // dim e of the 4 rows: low or high bf16 of word e / 2 of each row, packed pairwise
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const int w = e >> 1;
      const u32x2 pk = u32x2{__builtin_amdgcn_perm(vr[1][w], vr[0][w], sel),
                             __builtin_amdgcn_perm(vr[3][w], vr[2][w], sel)};
      *reinterpret_cast<u32x2*>(&sm.vt[buf][(dc * 8 + e) * AttnSmem<D>::vLd + 4 * kq]) = pk;
    }
  }
  if (tid < kBN) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) sm.s[hh][tid] = bscale[hh] * sr;
  }
}

// One key tile for one wave: S^T = K . Q^T, masked exp2-domain online softmax
// with the gate bias, O^T += V^T . P^T.  `lim` (MASK only): the lane's last
// visible key, tile-local (keys after it are causally masked or past the end).
template <int D, bool MASK>
__device__ __forceinline__ void attend_tile(const AttnSmem<D>& s_, int hl, const u32x4 (&qf)[D / 16],
                                            f32x16 (&o)[D / 32], float& m_run, float& l_run, float qk_scale, int lim,
                                            int g, int l32) {
  // S^T for the two 32-key halves; the two accumulation chains are interleaved
  f32x16 st[2] = {f32x16{}, f32x16{}};
  const uint16_t* krow0 = &s_.k[0][l32 * AttnSmem<D>::kLd + 8 * g];
  const uint16_t* krow1 = krow0 + 32 * AttnSmem<D>::kLd;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(krow0 + 16 * ks);
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(krow1 + 16 * ks);
    st[0] = mfma32(a0, qf[ks], st[0]);
    st[1] = mfma32(a1, qf[ks], st[1]);
  }
  // logits in the exp2 domain, tile max
  float tmax = -__builtin_inff();
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int kl = hf * 32 + 8 * q4 + 4 * g;  // first of 4 consecutive keys (tile-local)
      const f32x4 sv = *reinterpret_cast<const f32x4*>(&s_.s[hl][kl]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float xv = __builtin_fmaf(st[hf][4 * q4 + e], qk_scale, sv[e]);
        if (MASK && kl + e > lim) xv = -__builtin_inff();
        st[hf][4 * q4 + e] = xv;
        tmax = __builtin_fmaxf(tmax, xv);
      }
    }
  }
  tmax = xor32_max(tmax);
  // Lazy rescale: the reference point m_run only moves when some row's max
  // exceeds it by more than 2^8 (or on the first visible tile); softmax does
  // not depend on the reference point, and exp2(x - m_run) <= 2^8 stays well
  // inside fp32 and bf16 range.
  if (__ballot(tmax > m_run + 8.0f) != 0) {
    asm volatile("; rare rescale");  // keeps this a branch rather than a select on every tile
    const float m_new = __builtin_fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
    m_run = m_new;
  }
  float psum = 0.0f;
  u32x4 pf[4];  // P^T operands of the 4 PV steps (16 keys each)
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const float p0 = __builtin_amdgcn_exp2f(st[hf][8 * sub + 2 * j] - m_run);
        const float p1 = __builtin_amdgcn_exp2f(st[hf][8 * sub + 2 * j + 1] - m_run);
        psum += p0 + p1;
        w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{p0, p1}), bf16x2));
      }
      pf[2 * hf + sub] = w;
    }
  }
  l_run += psum;
  // O^T += V^T . P^T
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const uint16_t* vrow = &s_.vt[0][(dt * 32 + l32) * AttnSmem<D>::vLd + 16 * s4 + 4 * g];
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
      o[dt] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[s4], o[dt]);
    }
  }
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void gated_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ tau, const float* __restrict__ gain,
    const tg_segment* __restrict__ segs, int hq, int hkv, uint16_t* __restrict__ out) {
  constexpr int kBM = 128 / G;  // query rows per workgroup
  constexpr int kWavesPerHead = 4 / G;
  // smem[stage][group]: the two wave groups work on alternate key tiles
  __shared__ AttnSmem<D> sm[2][2];

  const tg_segment seg = segs[blockIdx.z];
  const int n = seg.kept_len;
  const int q0 = (gridDim.y - 1 - blockIdx.y) * kBM;
  if (q0 >= n) return;  // uniform

  const int tid = threadIdx.x;
  const int grp = tid >> 8;      // 0: even key tiles, 1: odd key tiles
  const int gtid = tid & 255;    // thread index inside the group
  const int lane = tid & 63;
  const int wave = gtid >> 6;    // wave inside the group
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int c = blockIdx.x;
  const int h = c * G + wave / kWavesPerHead;
  const int qw0 = q0 + (wave % kWavesPerHead) * 32;  // first query row of this wave
  const int qrow = qw0 + l32;                         // the query column this lane owns

  const int64_t q_stride = (int64_t)hq * D;
  const int64_t kv_stride = (int64_t)hkv * D;
  const uint16_t* qb = q + (int64_t)seg.kept_start * q_stride + (int64_t)h * D;
  const uint16_t* kb = k + (int64_t)seg.kept_start * kv_stride + (int64_t)c * D;
  const uint16_t* vb = v + (int64_t)seg.kept_start * kv_stride + (int64_t)c * D;
  const bool use_bias = key_score != nullptr && gain != nullptr;
  const uint32_t row_bytes = (uint32_t)kv_stride * 2u;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)n * row_bytes - (uint32_t)c * D * 2u);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)n * row_bytes - (uint32_t)c * D * 2u);
  // no bias: an empty range makes every score load return 0
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(use_bias ? key_score + seg.kept_start : key_score,
                                              use_bias ? (uint32_t)n * 4u : 0u);
  const TileAddr<D> ad(gtid, row_bytes);

  const float th = tau != nullptr ? tau[h] : 1.0f;
  const float qk_scale = th * kLog2e * (1.0f / __builtin_sqrtf((float)D));
  float bscale[G];  // g_h log2(e) of every query head of the group (0 without a bias)
#pragma unroll
  for (int hh = 0; hh < G; ++hh) bscale[hh] = use_bias ? gain[c * G + hh] * kLog2e : 0.0f;
  const int hl = wave / kWavesPerHead;  // this wave's head inside the group

  // Q^T operand: lane holds q[qrow][16 ks + 8 g .. + 7]
  u32x4 qf[D / 16];
  {
    const int r = qrow < n ? qrow : n - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(qb + (int64_t)r * q_stride + 8 * g);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = src[2 * ks];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(qf[ks]));  // keep Q resident, never re-read
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  const int q_end = min(q0 + kBM, n);  // keys needed: t < q_end
  const int ntiles = (q_end + kBN - 1) / kBN;
  const int npairs = (ntiles + 1) / 2;

  u32x4 kr[D / 32];
  u32x4 vr[4];
  float sr = 0.0f;
  // pair 0: group 0 stages tile 0, group 1 tile 1 (if any)
  if (grp < ntiles) {
    load_kv_tile<D>(rk, rv, rs, ad, row_bytes, grp * kBN, gtid, kr, vr, sr);
    store_kv_tile<D, G>(sm[0][grp], 0, gtid, kr, vr, sr, bscale);
  }
  __syncthreads();

  for (int ip = 0; ip < npairs; ++ip) {
    const int buf = ip & 1;
    const int jt = 2 * ip + grp;  // this group's key tile
    const int kv0 = jt * kBN;
    const int jn = jt + 2;        // this group's next key tile
    const bool more = jn < ntiles;
    if (more) load_kv_tile<D>(rk, rv, rs, ad, row_bytes, jn * kBN, gtid, kr, vr, sr);

    if (jt < ntiles && kv0 <= qw0 + 31) {  // some key of this tile is visible to some row of this wave
      const AttnSmem<D>& s_ = sm[buf][grp];
      if ((kv0 + kBN - 1 > qw0) || (kv0 + kBN > n))
        attend_tile<D, true>(s_, hl, qf, o, m_run, l_run, qk_scale, min(qrow, n - 1) - kv0, g, l32);
      else
        attend_tile<D, false>(s_, hl, qf, o, m_run, l_run, qk_scale, 0, g, l32);
    }

    if (more) store_kv_tile<D, G>(sm[buf ^ 1][grp], 0, gtid, kr, vr, sr, bscale);
    __syncthreads();
  }

  // Merge the two groups: group 1 hands (m, l, O^T) to group 0 through LDS.
  float* xo = reinterpret_cast<float*>(&sm[0][0]);  // 4 waves x (D x 32 + 64) floats, fits in the K/V buffers
  float* mine = xo + wave * (D * 32 + 64);
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
  if (grp == 0) {
    const float m1 = mine[D * 32 + l32];
    const float l1 = mine[D * 32 + 32 + l32];
    const float m = __builtin_fmaxf(m_run, m1);
    const float a0 = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
    const float inv = 1.0f / (l_half * a0 + l1 * a1);
    if (qrow < n) {
      uint16_t* orow = out + ((int64_t)seg.kept_start + qrow) * q_stride + (int64_t)h * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          typedef float f32x2 __attribute__((ext_vector_type(2)));
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * q4 + e;
            r[e] = (o[dt][i] * a0 + mine[(dt * 16 + i) * 64 + lane] * a1) * inv;
          }
          const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r[0], r[1]}), bf16x2));
          const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r[2], r[3]}), bf16x2));
          *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * q4 + 4 * g) = u32x2{w0, w1};
        }
      }
    }
  }
}

template <int D, int G>
hipError_t launch_dg(const void* q, const void* k, const void* v, const float* ks, const float* tau,
                     const float* gain, const tg_segment* segs, const tg_plan_info& info, int hq, int hkv, void* out,
                     hipStream_t stream) {
  constexpr int kBM = 128 / G;
  const int ntiles = (info.max_kept_len + kBM - 1) / kBM;
  if (ntiles == 0) return hipSuccess;
  dim3 grid(hkv, ntiles, info.n_seg);
  hipLaunchKernelGGL((gated_attention_kernel<D, G>), grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k),
                     reinterpret_cast<const uint16_t*>(v), ks, tau, gain, segs, hq, hkv,
                     reinterpret_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_attention(const void* q, const void* k, const void* v, const float* key_score,
                                  const float* tau, const float* gain, const tg_segment* segs,
                                  const tg_plan_info& info, int hq, int hkv, int head_dim, void* out,
                                  hipStream_t stream) {
  const int G = hq / hkv;
#define TG_ATTN_CASE(DD, GG) \
  if (head_dim == DD && G == GG) \
    return launch_dg<DD, GG>(q, k, v, key_score, tau, gain, segs, info, hq, hkv, out, stream);
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
