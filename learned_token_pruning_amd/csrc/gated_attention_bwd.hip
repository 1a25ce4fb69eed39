// Backward pass of token-gated causal GQA attention (gfx950).
//
// "TokenGate 与 T2Quant ... 精读", section 4.1, engineering notes: the biased
// attention kernel is also run backwards, and the gradient of the per-key bias
// flows back into the gate's scorer.  With z = tau_h q.k / sqrt(D) + g_h s_t,
// P = softmax(z) (causal, over the kept rows of a prompt) and upstream dO:
//   dV = P^T dO,  dZ = P o (dO V^T - rowsum(dO o O)),
//   dQ = tau_h/sqrt(D) dZ K,  dK = tau_h/sqrt(D) dZ^T Q,
//   ds_t = sum_h g_h sum_r dZ_rt,  dg_h = sum dZ_rt s_t,  dtau_h = sum dZ_rt q_r.k_t / sqrt(D).
// P is recomputed from the log-sum-exp the forward saved (flash-style: no
// M x M matrix is stored), in the exp2 domain.
//
// Kernels:
//  bwd_rowdot   Dt[r, h] = dO[r, h] . O[r, h]  (fp32; one row piece per lane group)
//  bwd_dkdv     one workgroup per (KV head, 128-key block, prompt), wave w owning
//               32 keys.  S = Q K^T is computed with the keys on the MFMA
//               columns, so a lane owns one key and its registers hold 16 query
//               rows: P and dZ are then, without any data movement, the B
//               operand of dV^T += dO^T P and dK^T += Q^T dZ (the query order
//               inside each 16-row MFMA step is permuted identically on both
//               operands).  Q and dO blocks of 32 rows are staged in LDS both
//               row-major (A operands of S and dP = dO V^T) and transposed.  The
//               lane-local key sums give ds, dg and dtau partials.
//  bwd_dq       the forward's transposed layout (a lane owns one query):
//               S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dZ^T, with K, V and K^T
//               tiles of 64 keys staged in LDS.
//  bwd_reduce   sums the per-KV-head ds partials and the per-workgroup dg /
//               dtau partials in a fixed order (deterministic results).
// bf16 MFMA operands (P and the scaled dZ are rounded to bf16 for the
// products), fp32 accumulation and fp32 gradient outputs.
#include <type_traits>

#include "common.h"

namespace tg {
namespace {

constexpr float kL2e = 1.4426950408889634f;
constexpr int kBwdThreads = 256;
constexpr int kKeyBlock = 128;  // keys per bwd_dkdv workgroup (4 waves x 32)
constexpr int kTile = 64;       // keys per bwd_dq tile

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// Row r (0-based) of register i of a 32x32 MFMA result for half-wave g.
__device__ __forceinline__ int c_row(int i, int g) { return 8 * (i / 4) + 4 * g + (i % 4); }

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_rowdot_kernel(const uint16_t* __restrict__ dout,
                                                                 const uint16_t* __restrict__ out, int64_t n_rows,
                                                                 float* __restrict__ dt) {
  constexpr int LPK = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * (kBwdThreads / LPK) + threadIdx.x / LPK;  // (row, head)
  const int sub = threadIdx.x % LPK;
  float a = 0.0f;
  if (idx < n_rows) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(dout + idx * D + 8 * sub);
    const u32x4 y = *reinterpret_cast<const u32x4*>(out + idx * D + 8 * sub);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a = __builtin_fmaf(bf16_lo(x[e]), bf16_lo(y[e]), a);
      a = __builtin_fmaf(bf16_hi(x[e]), bf16_hi(y[e]), a);
    }
  }
  a = group_sum<LPK>(a);
  if (idx < n_rows && sub == 0) dt[idx] = a;
}

// Staging of a block of 32 rows x D of one head: units of 4 rows x 8 dims,
// written row-major (stride D + 8) and transposed (stride 36: dim-major, rows
// contiguous).  Rows at or past `nvalid` are staged as zeros.
template <int D>
struct RowBlock {
  static constexpr int kLd = D + 8;
  static constexpr int tLd = 32 + 4;
  static constexpr int kUnits = 8 * (D / 8);
};

template <int D>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ src, int64_t row_stride, int r0, int nvalid,
                                          int u, u32x4 (&r)[4]) {
  const int rq = u % 8, dc = u / 8;  // rows 4 rq .. 4 rq + 3, dims 8 dc .. 8 dc + 7
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + 4 * rq + i;
    r[i] = row < nvalid ? *reinterpret_cast<const u32x4*>(src + (int64_t)row * row_stride + 8 * dc) : u32x4{0, 0, 0, 0};
  }
}

template <int D>
__device__ __forceinline__ void store_rows(int u, const u32x4 (&r)[4], uint16_t* rm, uint16_t* tr) {
  const int rq = u % 8, dc = u / 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&rm[(4 * rq + i) * RowBlock<D>::kLd + 8 * dc]) = r[i];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    const int w = e >> 1;
    const u32x2 pk = u32x2{__builtin_amdgcn_perm(r[1][w], r[0][w], sel), __builtin_amdgcn_perm(r[3][w], r[2][w], sel)};
    *reinterpret_cast<u32x2*>(&tr[(8 * dc + e) * RowBlock<D>::tLd + 4 * rq]) = pk;
  }
}

// 512 threads: two streams of 4 waves (waves w and w + 4 share a SIMD), wave
// w & 3 owning keys kb0 + 32 (w & 3) .. + 31 in both streams.  Stream s takes
// the (head, query block) items s, s + 2, s + 4, ... of the chunk with LDS
// staging of its own; the K/V rows of the workgroup are shared.  The streams'
// dK, dV and ds are summed in a fixed order at the end.
constexpr int kDkdvThreads = 512;

template <int D, int G>
__global__ __launch_bounds__(kDkdvThreads) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ tau, const float* __restrict__ gain,
    SegTable segs, int hq, int hkv, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dt, int n_chunks, int qc, float* __restrict__ dk_part,
    float* __restrict__ dv_part, float* __restrict__ ds_part, int64_t total_kept, float* __restrict__ part_g,
    float* __restrict__ part_t) {
  using RB = RowBlock<D>;
  struct alignas(16) Stage {
    uint16_t qs[32 * RB::kLd], qt[D * RB::tLd], os[32 * RB::kLd], ot[D * RB::tLd];
    float lse2[32], dts[32];
  };
  struct alignas(16) Smem {
    uint16_t kvk[kKeyBlock * RB::kLd], kvv[kKeyBlock * RB::kLd];
    Stage st[2];
  };
  __shared__ Smem sm;
  __shared__ float red[8][G][2];

  const tg_segment seg = segs.at_uniform(blockIdx.z);
  const int n = seg.kept_len;
  // blockIdx.y = key block x query chunk: the chunk covers query blocks
  // [kb0 / 32 + ci qc, + qc) of the prompt (possibly none: then zero partials)
  const int ci = blockIdx.y % n_chunks;
  const int kb0 = (blockIdx.y / n_chunks) * kKeyBlock;
  if (kb0 >= n) return;  // uniform
  const int c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int strm = wave >> 2, kslot = wave & 3;
  const int t = tid & 255;  // thread index inside the stream
  const int g = lane >> 5, l32 = lane & 31;
  const int kw0 = kb0 + 32 * kslot;  // first key of this wave
  const int kj = kw0 + l32;          // the key this lane owns
  const bool key_ok = kj < n;
  const int64_t base = seg.kept_start;
  const int64_t q_stride = (int64_t)hq * D, kv_stride = (int64_t)hkv * D;
  Stage& my = sm.st[strm];

  // the workgroup's K and V rows, staged once (row-major; B operands of S and
  // dP read the lane's key row at k = 16 ks + 8 g .. + 7)
  for (int u = tid; u < kKeyBlock * (D / 8); u += kDkdvThreads) {
    const int r = u / (D / 8), col = 8 * (u % (D / 8));
    const int key = kb0 + r;
    const int64_t off = (base + key) * kv_stride + (int64_t)c * D + col;
    *reinterpret_cast<u32x4*>(&sm.kvk[r * RB::kLd + col]) =
        key < n ? *reinterpret_cast<const u32x4*>(k + off) : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(&sm.kvv[r * RB::kLd + col]) =
        key < n ? *reinterpret_cast<const u32x4*>(v + off) : u32x4{0, 0, 0, 0};
  }
  const uint16_t* krow_l = &sm.kvk[(32 * kslot + l32) * RB::kLd + 8 * g];
  const uint16_t* vrow_l = &sm.kvv[(32 * kslot + l32) * RB::kLd + 8 * g];
  const bool use_bias = key_score != nullptr && gain != nullptr;
  const float s_key = use_bias && key_ok ? key_score[base + kj] : 0.0f;

  f32x16 dkt[D / 32], dvt[D / 32];
#pragma unroll
  for (int dtile = 0; dtile < D / 32; ++dtile) {
    dkt[dtile] = f32x16{};
    dvt[dtile] = f32x16{};
  }
  float ds_acc = 0.0f;
  float dg_acc[G], dtau_acc[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) dg_acc[gg] = dtau_acc[gg] = 0.0f;
  const float inv_sqrt_d = 1.0f / __builtin_sqrtf((float)D);

  // items (head, query block) of the chunk: it -> head it / nqb, block qb_begin + it % nqb
  const int qb_begin = kb0 / 32 + ci * qc;
  const int nqb = max(0, min(qb_begin + qc, (n + 31) / 32) - qb_begin);
  const int total = G * nqb;
  const int iters = (total + 1) / 2;
  u32x4 sreg[4];
  float slse = 0.0f, sdt = 0.0f;
  auto load_item = [&](int it) {  // it < total
    const int h = c * G + it / nqb, q0 = 32 * (qb_begin + it % nqb);
    if (t < RB::kUnits)
      load_rows<D>(q + base * q_stride + (int64_t)h * D, q_stride, q0, n, t, sreg);
    else if (t < 2 * RB::kUnits)
      load_rows<D>(dout + base * q_stride + (int64_t)h * D, q_stride, q0, n, t - RB::kUnits, sreg);
    if (t < 32) {
      const int row = q0 + t;
      slse = row < n ? lse[(base + row) * hq + h] * kL2e : __builtin_inff();
      sdt = row < n ? dt[(base + row) * hq + h] : 0.0f;
    }
  };
  if (strm < total) load_item(strm);
  for (int j = 0; j < iters; ++j) {
    const int it = 2 * j + strm;  // this stream's item (none when it >= total)
    const bool have = it < total;
    __syncthreads();  // the previous items' LDS reads are done
    if (have) {
      if (t < RB::kUnits)
        store_rows<D>(t, sreg, my.qs, my.qt);
      else if (t < 2 * RB::kUnits)
        store_rows<D>(t - RB::kUnits, sreg, my.os, my.ot);
      if (t < 32) {
        my.lse2[t] = slse;
        my.dts[t] = sdt;
      }
      if (it + 2 < total) load_item(it + 2);
    }
    __syncthreads();
    const int gg = have ? it / nqb : 0, q0 = have ? 32 * (qb_begin + it % nqb) : 0;
    if (!have || kw0 > q0 + 31) continue;  // no item, or every key after every query (uniform per wave)

    const int h = c * G + gg;
    const float th = tau != nullptr ? tau[h] : 1.0f;
    const float scale2 = th * kL2e * inv_sqrt_d;  // exp2-domain logit per unit q.k
    const float dscale = th * inv_sqrt_d;         // dZ -> dQ, dK factor
    const float gh = use_bias ? gain[h] : 0.0f;
    const float bias2 = gh * kL2e * s_key;        // exp2-domain bias of the lane's key

    f32x16 sacc = f32x16{}, dpacc = f32x16{};
    const uint16_t* qrow = &my.qs[l32 * RB::kLd + 8 * g];
    const uint16_t* orow = &my.os[l32 * RB::kLd + 8 * g];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      sacc = mfma32(*reinterpret_cast<const u32x4*>(qrow + 16 * ks), *reinterpret_cast<const u32x4*>(krow_l + 16 * ks),
                    sacc);
      dpacc = mfma32(*reinterpret_cast<const u32x4*>(orow + 16 * ks),
                     *reinterpret_cast<const u32x4*>(vrow_l + 16 * ks), dpacc);
    }
    // register i holds query row q0 + c_row(i, g), key kj
    float pz[16], dz[16];
    float dg_i = 0.0f, dtau_i = 0.0f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&my.lse2[8 * q4 + 4 * g]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&my.dts[8 * q4 + 4 * g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q4 + e;
        const int row = q0 + c_row(i, g);
        const bool ok = key_ok && kj <= row && row < n;
        const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(scale2, sacc[i], bias2) - l4[e]) : 0.0f;
        const float z = p * (dpacc[i] - d4[e]);
        pz[i] = p;
        dz[i] = z;
        ds_acc = __builtin_fmaf(gh, z, ds_acc);
        dg_i = __builtin_fmaf(z, s_key, dg_i);
        dtau_i = __builtin_fmaf(z, sacc[i] * inv_sqrt_d, dtau_i);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (hh == gg) {
        dg_acc[hh] += dg_i;
        dtau_acc[hh] += dtau_i;
      }
    }
    // B operands of the two 16-query MFMA steps: register 8 st + e
    u32x4 pb[2], zb[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i = 8 * st + 2 * jj;
        const uint32_t pp = pack2(pz[i], pz[i + 1]);
        const uint32_t zz = pack2(dz[i] * dscale, dz[i + 1] * dscale);
        pb[st][jj] = pp;
        zb[st][jj] = zz;
      }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int dtile = 0; dtile < D / 32; ++dtile) {
        const uint16_t* ro = &my.ot[(dtile * 32 + l32) * RB::tLd + 16 * st + 4 * g];
        const uint16_t* rq = &my.qt[(dtile * 32 + l32) * RB::tLd + 16 * st + 4 * g];
        const u32x2 olo = *reinterpret_cast<const u32x2*>(ro), ohi = *reinterpret_cast<const u32x2*>(ro + 8);
        const u32x2 qlo = *reinterpret_cast<const u32x2*>(rq), qhi = *reinterpret_cast<const u32x2*>(rq + 8);
        dvt[dtile] = mfma32(u32x4{olo[0], olo[1], ohi[0], ohi[1]}, pb[st], dvt[dtile]);
        dkt[dtile] = mfma32(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, zb[st], dkt[dtile]);
      }
    }
  }
  // per-head dg / dtau of the wave
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float a = wave_sum(dg_acc[gg]), b = wave_sum(dtau_acc[gg]);
    if (lane == 0) {
      red[wave][gg][0] = a;
      red[wave][gg][1] = b;
    }
  }
  // stream 1 hands its dK, dV and ds to stream 0 through LDS (the staging
  // buffers are free now), which adds them in a fixed order
  __syncthreads();
  constexpr int kRec = D * 32 * 2 + 64;  // floats per wave: dK^T, dV^T, ds
  float* xo = reinterpret_cast<float*>(&sm);
  static_assert(4 * kRec * 4 <= sizeof(Smem), "stream exchange fits in LDS");
  float* rec = xo + kslot * kRec;
  if (strm == 1) {
#pragma unroll
    for (int dtile = 0; dtile < D / 32; ++dtile)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        rec[((2 * dtile) * 16 + i) * 64 + lane] = dkt[dtile][i];
        rec[((2 * dtile + 1) * 16 + i) * 64 + lane] = dvt[dtile][i];
      }
    rec[D * 32 * 2 + lane] = ds_acc;
  }
  __syncthreads();
  if (strm == 0) {
#pragma unroll
    for (int dtile = 0; dtile < D / 32; ++dtile)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dkt[dtile][i] += rec[((2 * dtile) * 16 + i) * 64 + lane];
        dvt[dtile][i] += rec[((2 * dtile + 1) * 16 + i) * 64 + lane];
      }
    ds_acc += rec[D * 32 * 2 + lane];
    // dK, dV of the lane's key: register i of tile t holds dim 32 t + c_row(i, g)
    if (key_ok) {
      const int64_t prow = ((int64_t)ci * total_kept + base + kj) * kv_stride + (int64_t)c * D;
      float* dkr = dk_part + prow;
      float* dvr = dv_part + prow;
#pragma unroll
      for (int dtile = 0; dtile < D / 32; ++dtile)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * dtile + 8 * q4 + 4 * g;
          *reinterpret_cast<f32x4*>(dkr + d0) =
              f32x4{dkt[dtile][4 * q4], dkt[dtile][4 * q4 + 1], dkt[dtile][4 * q4 + 2], dkt[dtile][4 * q4 + 3]};
          *reinterpret_cast<f32x4*>(dvr + d0) =
              f32x4{dvt[dtile][4 * q4], dvt[dtile][4 * q4 + 1], dvt[dtile][4 * q4 + 2], dvt[dtile][4 * q4 + 3]};
        }
    }
    const float ds_key = xor32_sum(ds_acc);  // the two half-waves hold different query rows
    if (key_ok && g == 0) ds_part[((int64_t)ci * hkv + c) * total_kept + base + kj] = ds_key;
  }
  if (tid < G) {
    const int64_t slot = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
    float sg = 0.0f, st = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      sg += red[w][tid][0];
      st += red[w][tid][1];
    }
    part_g[slot * hq + c * G + tid] = sg;
    part_t[slot * hq + c * G + tid] = st;
  }
}

// dK, dV (head dim 128) with direct-to-LDS staging and the forward's ping-pong
// schedule.  Same work split as bwd_dkdv_kernel: a workgroup owns one KV head,
// 128 keys (wave w & 3 owns 32 of them in both groups) and a chunk of the
// prompt's 32-row query blocks; its two groups of four waves take alternate
// (head, query block) items.  In its MFMA phase a wave runs dV^T += dO^T P and
// dK^T += Q^T dZ for its previous item, then S = Q K^T and dP = dO V^T for its
// next one; in its other phase it forms P and dZ of the item in between.  The
// workgroup's K and V rows are staged once; each item's Q and dO rows, lse and
// row terms come in by DMA into five stages (an item's rows are read for S
// and dP at its half-step and, transposed, for dK and dV two half-steps
// later).  Q and dO chunks are swizzled as in bwd_dq_dma_kernel's K, K and V
// rows as c ^ (r & 15).  The arithmetic, and its order, is that of
// bwd_dkdv_kernel, so the results are the same bits.
//
// rt_swz: chunk swizzle of a row-major tile that is read both by rows and by
// transposing reads: chunk c of row r sits at c ^ rt_swz(r), which puts the 16
// rows of a row-read cycle on 16 distinct chunks and the 4 rows of a
// transposing read on 4 distinct 64-byte groups.
__device__ __forceinline__ int rt_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

constexpr int kDkStages = 5;

struct alignas(16) DkdvSmem {
  uint16_t kv[2][kKeyBlock * 128];   // K, V rows of the workgroup
  uint16_t qs[kDkStages][32 * 128];  // Q rows of an item
  uint16_t os[kDkStages][32 * 128];  // dO rows of an item
  float lse[kDkStages][32];          // natural-log lse of the item's rows
  float dts[kDkStages][32];          // row terms dO . O
};

template <int G>
__global__ __launch_bounds__(kDkdvThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_dma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ tau, const float* __restrict__ gain,
    SegTable segs, int hq, int hkv, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dt, int n_chunks, int qc, float* __restrict__ dk_part,
    float* __restrict__ dv_part, float* __restrict__ ds_part, int64_t total_kept, float* __restrict__ part_g,
    float* __restrict__ part_t) {
  constexpr int D = 128;
  __shared__ DkdvSmem sm;
  __shared__ float red[8][G][2];

  const tg_segment seg = segs.at_uniform(blockIdx.z);
  const int n = seg.kept_len;
  const int ci = blockIdx.y % n_chunks;
  const int kb0 = (blockIdx.y / n_chunks) * kKeyBlock;
  if (kb0 >= n) return;  // uniform
  const int c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int grp = tid >> 8;
  const int wave = __builtin_amdgcn_readfirstlane((tid & 255) >> 6);  // wave inside its group = key slot
  const int g = lane >> 5, l32 = lane & 31;
  const int kw0 = kb0 + 32 * wave;  // first key of this wave
  const int kj = kw0 + l32;         // the key this lane owns
  const bool key_ok = kj < n;
  const int64_t base = seg.kept_start;
  const int64_t q_stride = (int64_t)hq * D, kv_stride = (int64_t)hkv * D;
  const uint32_t q_row_bytes = (uint32_t)q_stride * 2u, kv_row_bytes = (uint32_t)kv_stride * 2u;
  const bool use_bias = key_score != nullptr && gain != nullptr;
  // threads 0-255 stage Q and lse, 256-511 dO and the row terms (a wave-uniform value: the DMA operands are scalar)
  const bool stage_q = __builtin_amdgcn_readfirstlane(tid >> 8) == 0;

  // buffers: the workgroup's K / V rows of head c; the prompt's Q / dO rows and lse / row terms
  const uint32_t kv_rows = (uint32_t)(n - kb0);
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(k + (base + kb0) * kv_stride + (int64_t)c * D, kv_rows * kv_row_bytes - (uint32_t)c * D * 2u);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(v + (base + kb0) * kv_stride + (int64_t)c * D, kv_rows * kv_row_bytes - (uint32_t)c * D * 2u);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(stage_q ? q + base * q_stride : dout + base * q_stride,
                                              (uint32_t)n * q_row_bytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(stage_q ? lse + base * hq : dt + base * hq, (uint32_t)n * (uint32_t)hq * 4u);

  // K and V rows: 128 rows x 16 chunks each, 4 chunks per thread and tensor
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = (j * 8 + wave8) * 64 + lane;
    const int r = p / 16, cc = p % 16;
    const uint32_t off = (uint32_t)r * kv_row_bytes + (uint32_t)(cc ^ (r & 15)) * 16u;
    dma16(rk, &sm.kv[0][(j * 8 + wave8) * 64 * 8], off, 0u);
    dma16(rv, &sm.kv[1][(j * 8 + wave8) * 64 * 8], off, 0u);
  }

  // items (head, query block) of the chunk: it -> head it / nqb, block qb_begin + it % nqb
  const int qb_begin = kb0 / 32 + ci * qc;
  const int nqb = max(0, min(qb_begin + qc, (n + 31) / 32) - qb_begin);
  const int total = G * nqb;
  // Q (or dO) rows of item it into stage buf: 32 rows x 16 chunks, 2 chunks per staging lane; lse (or row terms)
  // of its 32 rows from lanes 0-7 of each staging wave
  uint32_t doff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = (j * 4 + wave) * 64 + lane;
    const int r = p / 16;
    doff[j] = (uint32_t)r * q_row_bytes + (uint32_t)((p % 16) ^ rt_swz(r)) * 16u;
  }
  auto stage_item = [&](int it, int buf) {
    const int h = c * G + it / nqb, q0 = 32 * (qb_begin + it % nqb);
    uint16_t* dst = stage_q ? sm.qs[buf] : sm.os[buf];
    const uint32_t soff = (uint32_t)q0 * q_row_bytes + (uint32_t)h * D * 2u;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(rq, &dst[(j * 4 + wave) * 64 * 8], doff[j], soff);
    float* ldst = stage_q ? sm.lse[buf] : sm.dts[buf];
    if (lane < 8)
      dma4(rl, &ldst[8 * wave], (uint32_t)(8 * wave + lane) * (uint32_t)hq * 4u, ((uint32_t)q0 * hq + h) * 4u);
  };
  if (total > 0) stage_item(0, 0);
  if (total > 1) stage_item(1, 1);

  // LDS element offsets of this lane's fragment reads.
  // K / V rows (B operands of S and dP): key row 32 wave + l32, chunk 2 ks + g.
  uint32_t kaddr[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int r = 32 * wave + l32;
    kaddr[ks] = (uint32_t)(r * D + (((2 * ks + g) ^ (r & 15)) * 8));
  }
  // Q / dO rows (A operands of S and dP): row l32, chunk 2 ks + g.
  uint32_t raddr[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) raddr[ks] = (uint32_t)(l32 * D + (((2 * ks + g) ^ rt_swz(l32)) * 8));
  // Q^T / dO^T (A operands of dK and dV, transposing reads): as bwd_dq_dma_kernel's K^T, rows of a 16-query step.
  uint32_t taddr[2][D / 32];
  {
    const int s2 = lane & 15, qg = lane >> 4;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 8 * hi + 4 * g + (s2 >> 2);
#pragma unroll
      for (int dtile = 0; dtile < D / 32; ++dtile) {
        const int cc = 4 * dtile + 2 * (qg & 1) + ((s2 & 3) >> 1);
        taddr[hi][dtile] = (uint32_t)(r * D + ((cc ^ rt_swz(r)) * 8) + 4 * (s2 & 1));
      }
    }
  }

  const float s_key = use_bias && key_ok ? key_score[base + kj] : 0.0f;
  f32x16 dkt[D / 32], dvt[D / 32];
#pragma unroll
  for (int dtile = 0; dtile < D / 32; ++dtile) {
    dkt[dtile] = f32x16{};
    dvt[dtile] = f32x16{};
  }
  float ds_acc = 0.0f;
  float dg_acc[G], dtau_acc[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) dg_acc[gg] = dtau_acc[gg] = 0.0f;
  const float inv_sqrt_d = 1.0f / __builtin_sqrtf((float)D);
  f32x16 sacc, dpacc;
  u32x4 pb[2], zb[2];

  if (total > 1)
    wait_vm<3>();  // K, V and item 0 landed; item 1 may be in flight
  else
    wait_vm<0>();
  lds_barrier();

  auto item_q0 = [&](int it) { return 32 * (qb_begin + it % nqb); };
  auto half_step = [&](int hs, auto p_) {
    constexpr int P = decltype(p_)::value;
    const bool dma_now = hs + 2 < total;
    if (dma_now && !stage_q) stage_item(hs + 2, (hs + 2) % kDkStages);  // dO of item hs + 2 at the start
    if (P == grp) {
      const int jp = hs - 2;  // dV, dK of item jp
      if (jp >= 0 && kw0 <= item_q0(jp) + 31) {
        const int b = jp % kDkStages;
        const uint16_t* ot = sm.os[b];
        const uint16_t* qt = sm.qs[b];
        typedef short short4v __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int dtile = 0; dtile < D / 32; ++dtile) {
            const short4v olo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(ot + taddr[0][dtile] + 16 * st * D));
            const short4v ohi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(ot + taddr[1][dtile] + 16 * st * D));
            const short4v qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(qt + taddr[0][dtile] + 16 * st * D));
            const short4v qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(qt + taddr[1][dtile] + 16 * st * D));
            const u32x2 o2l = __builtin_bit_cast(u32x2, olo), o2h = __builtin_bit_cast(u32x2, ohi);
            const u32x2 q2l = __builtin_bit_cast(u32x2, qlo), q2h = __builtin_bit_cast(u32x2, qhi);
            dvt[dtile] = mfma32(u32x4{o2l[0], o2l[1], o2h[0], o2h[1]}, pb[st], dvt[dtile]);
            dkt[dtile] = mfma32(u32x4{q2l[0], q2l[1], q2h[0], q2h[1]}, zb[st], dkt[dtile]);
          }
        }
        sched_two_reads_ahead<2 * 2 * (D / 32), 8>();
      }
      const int jq = hs;  // S, dP of item jq
      if (jq < total && kw0 <= item_q0(jq) + 31) {
        const int b = jq % kDkStages;
        const uint16_t* qr = sm.qs[b];
        const uint16_t* orr = sm.os[b];
        const uint16_t* kt = sm.kv[0];
        const uint16_t* vt = sm.kv[1];
        sacc = f32x16{};
        dpacc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          sacc = mfma32(*reinterpret_cast<const u32x4*>(qr + raddr[ks]), *reinterpret_cast<const u32x4*>(kt + kaddr[ks]),
                        sacc);
          dpacc = mfma32(*reinterpret_cast<const u32x4*>(orr + raddr[ks]),
                         *reinterpret_cast<const u32x4*>(vt + kaddr[ks]), dpacc);
        }
        sched_two_reads_ahead<2 * (D / 16), 8>();
      }
    } else {
      const int js = hs - 1;  // P and dZ of item js
      if (js >= 0 && js < total && kw0 <= item_q0(js) + 31) {
        const int b = js % kDkStages;
        const int gg = js / nqb, q0 = item_q0(js);
        const int h = c * G + gg;
        const float th = tau != nullptr ? tau[h] : 1.0f;
        const float scale2 = th * kL2e * inv_sqrt_d;  // exp2-domain logit per unit q.k
        const float dscale = th * inv_sqrt_d;         // dZ -> dQ, dK factor
        const float gh = use_bias ? gain[h] : 0.0f;
        const float bias2 = gh * kL2e * s_key;        // exp2-domain bias of the lane's key
        // register i holds query row q0 + c_row(i, g), key kj
        float pz[16], dz[16];
        float dg_i = 0.0f, dtau_i = 0.0f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 l4r = *reinterpret_cast<const f32x4*>(&sm.lse[b][8 * q4 + 4 * g]);
          const f32x4 d4r = *reinterpret_cast<const f32x4*>(&sm.dts[b][8 * q4 + 4 * g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * q4 + e;
            const int row = q0 + c_row(i, g);
            const bool ok = key_ok && kj <= row && row < n;
            const float l4 = row < n ? l4r[e] * kL2e : __builtin_inff();
            const float d4 = row < n ? d4r[e] : 0.0f;
            const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(scale2, sacc[i], bias2) - l4) : 0.0f;
            const float z = p * (dpacc[i] - d4);
            pz[i] = p;
            dz[i] = z;
            ds_acc = __builtin_fmaf(gh, z, ds_acc);
            dg_i = __builtin_fmaf(z, s_key, dg_i);
            dtau_i = __builtin_fmaf(z, sacc[i] * inv_sqrt_d, dtau_i);
          }
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          if (hh == gg) {
            dg_acc[hh] += dg_i;
            dtau_acc[hh] += dtau_i;
          }
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int i = 8 * st + 2 * jj;
            pb[st][jj] = pack2(pz[i], pz[i + 1]);
            zb[st][jj] = pack2(dz[i] * dscale, dz[i + 1] * dscale);
          }
      }
    }
    if (dma_now && stage_q) stage_item(hs + 2, (hs + 2) % kDkStages);  // Q of item hs + 2 at the end
    // item hs + 1 (issued one half-step ago) must have landed; this half-step's DMAs may stay in flight
    if (dma_now)
      wait_vm<3>();
    else
      wait_vm<0>();
    lds_barrier();
  };
  for (int hs = 0; hs < total + 2; hs += 2) {
    half_step(hs, std::integral_constant<int, 0>());
    if (hs + 1 < total + 2) half_step(hs + 1, std::integral_constant<int, 1>());
  }

  // per-head dg / dtau of the wave
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float a = wave_sum(dg_acc[gg]), b = wave_sum(dtau_acc[gg]);
    if (lane == 0) {
      red[wave8][gg][0] = a;
      red[wave8][gg][1] = b;
    }
  }
  // group 1 hands its dK, dV and ds to group 0 through LDS (the stages are free now: the last half-step ended
  // with a barrier), which adds them in a fixed order
  constexpr int kRec = D * 32 * 2 + 64;  // floats per wave: dK^T, dV^T, ds
  float* xo = reinterpret_cast<float*>(&sm);
  static_assert(4 * kRec * 4 <= sizeof(DkdvSmem), "group exchange fits in LDS");
  float* rec = xo + wave * kRec;
  if (grp == 1) {
#pragma unroll
    for (int dtile = 0; dtile < D / 32; ++dtile)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        rec[((2 * dtile) * 16 + i) * 64 + lane] = dkt[dtile][i];
        rec[((2 * dtile + 1) * 16 + i) * 64 + lane] = dvt[dtile][i];
      }
    rec[D * 32 * 2 + lane] = ds_acc;
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int dtile = 0; dtile < D / 32; ++dtile)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dkt[dtile][i] += rec[((2 * dtile) * 16 + i) * 64 + lane];
        dvt[dtile][i] += rec[((2 * dtile + 1) * 16 + i) * 64 + lane];
      }
    ds_acc += rec[D * 32 * 2 + lane];
    // dK, dV of the lane's key: register i of tile t holds dim 32 t + c_row(i, g)
    if (key_ok) {
      const int64_t prow = ((int64_t)ci * total_kept + base + kj) * kv_stride + (int64_t)c * D;
      float* dkr = dk_part + prow;
      float* dvr = dv_part + prow;
#pragma unroll
      for (int dtile = 0; dtile < D / 32; ++dtile)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * dtile + 8 * q4 + 4 * g;
          *reinterpret_cast<f32x4*>(dkr + d0) =
              f32x4{dkt[dtile][4 * q4], dkt[dtile][4 * q4 + 1], dkt[dtile][4 * q4 + 2], dkt[dtile][4 * q4 + 3]};
          *reinterpret_cast<f32x4*>(dvr + d0) =
              f32x4{dvt[dtile][4 * q4], dvt[dtile][4 * q4 + 1], dvt[dtile][4 * q4 + 2], dvt[dtile][4 * q4 + 3]};
        }
    }
    const float ds_key = xor32_sum(ds_acc);  // the two half-waves hold different query rows
    if (key_ok && g == 0) ds_part[((int64_t)ci * hkv + c) * total_kept + base + kj] = ds_key;
  }
  if (tid < G) {
    const int64_t slot = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
    float sg = 0.0f, st = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      sg += red[w][tid][0];
      st += red[w][tid][1];
    }
    part_g[slot * hq + c * G + tid] = sg;
    part_t[slot * hq + c * G + tid] = st;
  }
}

template <int D>
struct KeyTile {
  static constexpr int kLd = D + 8;       // K, V row-major
  static constexpr int tLd = kTile + 4;   // K^T
};

template <int D, int G>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ tau, const float* __restrict__ gain,
    SegTable segs, int hq, int hkv, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dt, float* __restrict__ dq) {
  using KT = KeyTile<D>;
  constexpr int kBM = 128 / G;
  constexpr int kWavesPerHead = 4 / G;
  __shared__ __attribute__((aligned(16))) uint16_t ks_[kTile * KT::kLd], vs[kTile * KT::kLd], kt[D * KT::tLd];
  __shared__ float sc[kTile];

  const tg_segment seg = segs.at_uniform(blockIdx.z);
  const int n = seg.kept_len;
  const int q0 = (gridDim.y - 1 - blockIdx.y) * kBM;
  if (q0 >= n) return;
  const int q_end = min(q0 + kBM, n);
  const int c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int hl = wave / kWavesPerHead, h = c * G + hl;
  const int qw0 = q0 + (wave % kWavesPerHead) * 32;
  const int qrow = qw0 + l32;
  const bool row_ok = qrow < n;
  const int64_t base = seg.kept_start;
  const int64_t q_stride = (int64_t)hq * D, kv_stride = (int64_t)hkv * D;

  u32x4 qf[D / 16], of[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int64_t off = (base + qrow) * q_stride + (int64_t)h * D + 16 * ks + 8 * g;
    qf[ks] = row_ok ? *reinterpret_cast<const u32x4*>(q + off) : u32x4{0, 0, 0, 0};
    of[ks] = row_ok ? *reinterpret_cast<const u32x4*>(dout + off) : u32x4{0, 0, 0, 0};
  }
  const float th = tau != nullptr ? tau[h] : 1.0f;
  const float inv_sqrt_d = 1.0f / __builtin_sqrtf((float)D);
  const float scale2 = th * kL2e * inv_sqrt_d, dscale = th * inv_sqrt_d;
  const bool use_bias = key_score != nullptr && gain != nullptr;
  const float gb2 = use_bias ? gain[h] * kL2e : 0.0f;
  const float lse_row = row_ok ? lse[(base + qrow) * hq + h] * kL2e : __builtin_inff();
  const float dt_row = row_ok ? dt[(base + qrow) * hq + h] : 0.0f;

  f32x16 dqt[D / 32];
#pragma unroll
  for (int dtile = 0; dtile < D / 32; ++dtile) dqt[dtile] = f32x16{};
  const int wlast = qw0 + 31;
  const int ntiles = (q_end + kTile - 1) / kTile;

  // K / V units of 4 keys x 8 dims: the next tile's are loaded into registers
  // while the current tile computes
  constexpr int kUnitsK = (kTile / 4) * (D / 8);  // <= kBwdThreads
  u32x4 kr[4], vr[4];
  float scr = 0.0f;
  auto load_tile = [&](int jt) {
    const int kv0 = jt * kTile;
    if (tid < kUnitsK) {
      const int kq = tid % (kTile / 4), dc = tid / (kTile / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kv0 + 4 * kq + i;
        const int64_t off = (base + key) * kv_stride + (int64_t)c * D + 8 * dc;
        kr[i] = key < n ? *reinterpret_cast<const u32x4*>(k + off) : u32x4{0, 0, 0, 0};
        vr[i] = key < n ? *reinterpret_cast<const u32x4*>(v + off) : u32x4{0, 0, 0, 0};
      }
    }
    if (tid < kTile) scr = use_bias && kv0 + tid < n ? key_score[base + kv0 + tid] : 0.0f;
  };
  load_tile(0);
  for (int jt = 0; jt < ntiles; ++jt) {
    const int kv0 = jt * kTile;
    __syncthreads();  // the previous tile's LDS reads are done
    if (tid < kUnitsK) {  // K row-major and transposed, V row-major
      const int kq = tid % (kTile / 4), dc = tid / (kTile / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<u32x4*>(&ks_[(4 * kq + i) * KT::kLd + 8 * dc]) = kr[i];
        *reinterpret_cast<u32x4*>(&vs[(4 * kq + i) * KT::kLd + 8 * dc]) = vr[i];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const int w = e >> 1;
        const u32x2 pk = u32x2{__builtin_amdgcn_perm(kr[1][w], kr[0][w], sel),
                               __builtin_amdgcn_perm(kr[3][w], kr[2][w], sel)};
        *reinterpret_cast<u32x2*>(&kt[(8 * dc + e) * KT::tLd + 4 * kq]) = pk;
      }
    }
    if (tid < kTile) sc[tid] = scr;
    if (jt + 1 < ntiles) load_tile(jt + 1);
    __syncthreads();
    if (kv0 > wlast) continue;  // uniform per wave

    u32x4 zb[4];  // scaled dZ^T, B operands of the 4 16-key MFMA steps
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
      const uint16_t* krow = &ks_[(hf * 32 + l32) * KT::kLd + 8 * g];
      const uint16_t* vrow = &vs[(hf * 32 + l32) * KT::kLd + 8 * g];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        sacc = mfma32(*reinterpret_cast<const u32x4*>(krow + 16 * ks), qf[ks], sacc);
        dpacc = mfma32(*reinterpret_cast<const u32x4*>(vrow + 16 * ks), of[ks], dpacc);
      }
      // register i holds key kv0 + 32 hf + c_row(i, g), query qrow
      float z[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(&sc[hf * 32 + 8 * q4 + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q4 + e;
          const int key = kv0 + hf * 32 + c_row(i, g);
          const bool ok = row_ok && key <= qrow && key < n;
          const float p =
              ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(scale2, sacc[i], gb2 * s4[e]) - lse_row) : 0.0f;
          z[i] = p * (dpacc[i] - dt_row) * dscale;
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t zz = pack2(z[8 * st + 2 * j], z[8 * st + 2 * j + 1]);
          zb[2 * hf + st][j] = zz;
        }
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int dtile = 0; dtile < D / 32; ++dtile) {
        const uint16_t* kr = &kt[(dtile * 32 + l32) * KT::tLd + 16 * s4 + 4 * g];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(kr), hi = *reinterpret_cast<const u32x2*>(kr + 8);
        dqt[dtile] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, zb[s4], dqt[dtile]);
      }
  }
  if (row_ok) {
    float* dqr = dq + (base + qrow) * q_stride + (int64_t)h * D;
#pragma unroll
    for (int dtile = 0; dtile < D / 32; ++dtile)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(dqr + 32 * dtile + 8 * q4 + 4 * g) =
            f32x4{dqt[dtile][4 * q4], dqt[dtile][4 * q4 + 1], dqt[dtile][4 * q4 + 2], dqt[dtile][4 * q4 + 3]};
  }
}

// dQ with direct-to-LDS staging and the forward's ping-pong schedule (D = 128).
// A workgroup owns one KV head and a 128/G-row query tile of its G heads; its
// 8 waves form two groups of 4 (one wave of each per SIMD), group 0 taking the
// even 64-key tiles and group 1 the odd ones.  In its MFMA phase a wave runs
// dQ^T += K^T dZ^T for its previous tile and S^T = K Q^T, dP^T = V dO^T for its
// next one; in its other phase it turns S^T and dP^T into dZ^T (P from the
// saved log-sum-exp, so no running maximum).  K and V come in by DMA: a K tile
// is read twice (for S at its own half-step, for dQ two half-steps later), so K
// has five LDS stages and V three.  K^T is read from the row-major K tile with
// transposing LDS reads; K and V chunks are swizzled so that both read patterns
// are conflict free (chunk c of row r at c ^ (((r & 3) << 2) | ((r >> 2) & 3)):
// the 16 rows of a row-read cycle hit 16 distinct chunks, the 4 rows of a
// transposing read 4 distinct 64-byte groups).  The two groups' dQ^T are added
// through LDS at the end.
constexpr int kDqThreads = 512;
constexpr int kDqK = 5;  // K stages
constexpr int kDqV = 3;  // V stages

struct alignas(16) DqSmem {
  uint16_t k[kDqK][kTile * 128];
  uint16_t v[kDqV][kTile * 128];
  float s[kDqK][kTile];  // key scores, with their K tile
};


template <int G>
__global__ __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_dma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ tau, const float* __restrict__ gain,
    SegTable segs, int hq, int hkv, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dt, float* __restrict__ dq) {
  constexpr int D = 128;
  constexpr int kBM = 128 / G;
  constexpr int kWavesPerHead = 4 / G;
  constexpr int NC = D / 8;   // 16-byte chunks per row
  constexpr int NJ = NC / 4;  // DMA instructions per staging wave per tile
  __shared__ DqSmem sm;

  const tg_segment seg = segs.at_uniform(blockIdx.z);
  const int n = seg.kept_len;
  const int q0 = (gridDim.y - 1 - blockIdx.y) * kBM;
  if (q0 >= n) return;  // uniform
  const int q_end = min(q0 + kBM, n);
  const int tid = threadIdx.x;
  const int grp = tid >> 8;
  const int gtid = tid & 255;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(gtid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int c = blockIdx.x;
  const int hl = wave / kWavesPerHead, h = c * G + hl;
  const int qw0 = q0 + (wave % kWavesPerHead) * 32;
  const int qrow = qw0 + l32;
  const bool row_ok = qrow < n;
  const int64_t base = seg.kept_start;
  const int64_t q_stride = (int64_t)hq * D, kv_stride = (int64_t)hkv * D;
  const uint32_t row_bytes = (uint32_t)kv_stride * 2u;
  const uint32_t nrows = (uint32_t)n;
  const bool use_bias = key_score != nullptr && gain != nullptr;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + base * kv_stride + (int64_t)c * D, nrows * row_bytes - (uint32_t)c * D * 2u);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + base * kv_stride + (int64_t)c * D, nrows * row_bytes - (uint32_t)c * D * 2u);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(use_bias ? key_score + base : key_score, use_bias ? nrows * 4u : 0u);
  const bool stage_k = grp == 0;  // threads 0-255 stage K and the scores, 256-511 V

  // DMA source offsets inside a tile: chunk slot (j 4 + wave) 64 + lane
  uint32_t doff[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int p = (j * 4 + wave) * 64 + lane;
    const int r = p / NC;
    doff[j] = (uint32_t)r * row_bytes + (uint32_t)((p % NC) ^ rt_swz(r)) * 16u;
  }
  auto dma_k = [&](int tile, int buf) {
    const uint32_t soff = (uint32_t)(tile * kTile) * row_bytes;
#pragma unroll
    for (int j = 0; j < NJ; ++j) dma16(rk, &sm.k[buf][(j * 4 + wave) * 64 * 8], doff[j], soff);
    if (lane < 16) dma4(rs, &sm.s[buf][16 * wave], (uint32_t)(16 * wave + lane) * 4u, (uint32_t)(tile * kTile) * 4u);
  };
  auto dma_v = [&](int tile, int buf) {
    const uint32_t soff = (uint32_t)(tile * kTile) * row_bytes;
#pragma unroll
    for (int j = 0; j < NJ; ++j) dma16(rv, &sm.v[buf][(j * 4 + wave) * 64 * 8], doff[j], soff);
  };

  const float th = tau != nullptr ? tau[h] : 1.0f;
  const float inv_sqrt_d = 1.0f / __builtin_sqrtf((float)D);
  const float scale2 = th * kL2e * inv_sqrt_d, dscale = th * inv_sqrt_d;
  const float gb2 = use_bias ? gain[h] * kL2e : 0.0f;
  const float lse_row = row_ok ? lse[(base + qrow) * hq + h] * kL2e : __builtin_inff();
  const float dt_row = row_ok ? dt[(base + qrow) * hq + h] : 0.0f;
  const int ntiles = (q_end + kTile - 1) / kTile;
  const int wlast = qw0 + 31;

  if (stage_k) {
    dma_k(0, 0);
    if (ntiles > 1) dma_k(1, 1);
  } else {
    dma_v(0, 0);
    if (ntiles > 1) dma_v(1, 1);
  }
  // Q^T and dO^T operands: lane holds row qrow, dims 16 ks + 8 g .. + 7
  u32x4 qf[D / 16], of[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int64_t off = (base + qrow) * q_stride + (int64_t)h * D + 16 * ks + 8 * g;
    qf[ks] = row_ok ? *reinterpret_cast<const u32x4*>(q + off) : u32x4{0, 0, 0, 0};
    of[ks] = row_ok ? *reinterpret_cast<const u32x4*>(dout + off) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    asm volatile("" : "+v"(qf[ks]));  // keep them resident, never re-read
    asm volatile("" : "+v"(of[ks]));
  }

  // LDS element offsets of this lane's fragment reads inside a tile.
  // K and V rows (A operands of S^T and dP^T): row l32 (+32 for the second half), chunk 2 ks + g.
  uint32_t raddr[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) raddr[ks] = (uint32_t)(l32 * D + (((2 * ks + g) ^ rt_swz(l32)) * 8));
  // K^T (A operand of dQ^T, transposing read): 16-lane group qg covers dims 32 dt + 16 (qg % 2) + 0..15 and
  // keys 4 g + 0..3 (+8 for the upper half of a 16-key step); source lane s points at row 4 g + s / 4 (+8).
  uint32_t taddr[2][D / 32];
  {
    const int s = lane & 15, qg = lane >> 4;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 8 * hi + 4 * g + (s >> 2);
#pragma unroll
      for (int dtile = 0; dtile < D / 32; ++dtile) {
        const int cc = 4 * dtile + 2 * (qg & 1) + ((s & 3) >> 1);
        taddr[hi][dtile] = (uint32_t)(r * D + ((cc ^ rt_swz(r)) * 8) + 4 * (s & 1));
      }
    }
  }

  f32x16 dqt[D / 32];
#pragma unroll
  for (int dtile = 0; dtile < D / 32; ++dtile) dqt[dtile] = f32x16{};
  f32x16 sa[2], dpa[2];
  u32x4 zb[4];  // scaled dZ^T, B operands of the 4 16-key steps of the dQ product

  if (stage_k) {
    if (ntiles > 1)
      wait_vm<NJ + 1>();
    else
      wait_vm<0>();
  } else {
    if (ntiles > 1)
      wait_vm<NJ>();
    else
      wait_vm<0>();
  }
  lds_barrier();

  int kc = 0, vc = 0;  // hs % kDqK, hs % kDqV
  auto half_step = [&](int hs, auto p_) {
    constexpr int P = decltype(p_)::value;
    const int k_m2 = kc >= 2 ? kc - 2 : kc + kDqK - 2;  // stage of K tile hs - 2
    const int k_m1 = kc >= 1 ? kc - 1 : kc + kDqK - 1;  // stage of K tile hs - 1
    const int k_p2 = kc + 2 < kDqK ? kc + 2 : kc + 2 - kDqK;
    const int v_p2 = vc + 2 < kDqV ? vc + 2 : vc + 2 - kDqV;
    const bool dma_now = hs + 2 < ntiles;
    if (dma_now && !stage_k) dma_v(hs + 2, v_p2);  // V tile hs + 2 at the start

    if (P == grp) {
      const int jp = hs - 2;
      if (jp >= 0 && jp * kTile <= wlast) {
        const uint16_t* kt = sm.k[k_m2];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
          for (int dtile = 0; dtile < D / 32; ++dtile) {
            typedef short short4v __attribute__((ext_vector_type(4)));
            const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(kt + taddr[0][dtile] + 16 * s4 * D));
            const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(kt + taddr[1][dtile] + 16 * s4 * D));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            dqt[dtile] = mfma32(u32x4{l2[0], l2[1], h2[0], h2[1]}, zb[s4], dqt[dtile]);
          }
        }
        sched_two_reads_ahead<4 * (D / 32), 8>();
      }
      if (hs < ntiles && hs * kTile <= wlast) {
        const uint16_t* kt = sm.k[kc];
        const uint16_t* vt = sm.v[vc];
        sa[0] = sa[1] = dpa[0] = dpa[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(kt + raddr[ks]);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(kt + raddr[ks] + 32 * D);
          const u32x4 b0 = *reinterpret_cast<const u32x4*>(vt + raddr[ks]);
          const u32x4 b1 = *reinterpret_cast<const u32x4*>(vt + raddr[ks] + 32 * D);
          sa[0] = mfma32(a0, qf[ks], sa[0]);
          sa[1] = mfma32(a1, qf[ks], sa[1]);
          dpa[0] = mfma32(b0, of[ks], dpa[0]);
          dpa[1] = mfma32(b1, of[ks], dpa[1]);
        }
        sched_reads_ahead<4 * (D / 16), 4 * (D / 16), 16>();
      }
    } else {
      // dZ^T of tile hs - 1 from this wave's S^T and dP^T
      const int js = hs - 1;
      if (js >= 0 && js < ntiles && js * kTile <= wlast) {
        const int kv0 = js * kTile;
        const float* scs = sm.s[k_m1];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float z[16];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 s4v = *reinterpret_cast<const f32x4*>(&scs[hf * 32 + 8 * q4 + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * q4 + e;
              const int key = kv0 + hf * 32 + c_row(i, g);
              const bool ok = row_ok && key <= qrow && key < n;
              const float p =
                  ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(scale2, sa[hf][i], gb2 * s4v[e]) - lse_row) : 0.0f;
              z[i] = p * (dpa[hf][i] - dt_row) * dscale;
            }
          }
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int j = 0; j < 4; ++j) zb[2 * hf + st][j] = pack2(z[8 * st + 2 * j], z[8 * st + 2 * j + 1]);
        }
      }
    }

    if (dma_now && stage_k) {
      // K tile hs + 2 at the end; its stage last held tile hs - 3, whose last read (dQ) was at hs - 1
      dma_k(hs + 2, k_p2);
    }
    // K and V tiles hs + 1 (issued one half-step ago) must have landed; this half-step's DMAs may stay in flight
    if (dma_now) {
      if (stage_k)
        wait_vm<NJ + 1>();
      else
        wait_vm<NJ>();
    } else {
      wait_vm<0>();
    }
    lds_barrier();
    kc = kc + 1 < kDqK ? kc + 1 : 0;
    vc = vc + 1 < kDqV ? vc + 1 : 0;
  };
  for (int hs = 0; hs < ntiles + 2; hs += 2) {
    half_step(hs, std::integral_constant<int, 0>());
    if (hs + 1 < ntiles + 2) half_step(hs + 1, std::integral_constant<int, 1>());
  }

  // dQ = group 0's dQ^T + group 1's: group 1 hands its fragments over through LDS
  float* mine = reinterpret_cast<float*>(&sm) + wave * (D * 32);
  if (grp == 1) {
#pragma unroll
    for (int dtile = 0; dtile < D / 32; ++dtile)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(&mine[((dtile * 4 + q4) * 64 + lane) * 4]) =
            f32x4{dqt[dtile][4 * q4], dqt[dtile][4 * q4 + 1], dqt[dtile][4 * q4 + 2], dqt[dtile][4 * q4 + 3]};
  }
  __syncthreads();
  if (grp == 0 && row_ok) {
    float* dqr = dq + (base + qrow) * q_stride + (int64_t)h * D;
#pragma unroll
    for (int dtile = 0; dtile < D / 32; ++dtile)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(&mine[((dtile * 4 + q4) * 64 + lane) * 4]);
        *reinterpret_cast<f32x4*>(dqr + 32 * dtile + 8 * q4 + 4 * g) =
            f32x4{dqt[dtile][4 * q4] + o1[0], dqt[dtile][4 * q4 + 1] + o1[1], dqt[dtile][4 * q4 + 2] + o1[2],
                  dqt[dtile][4 * q4 + 3] + o1[3]};
      }
  }
}

// dk, dv: sum of the chunk partials; ds[t] = sum over chunks and KV heads
// (fixed order, so results are deterministic)
__global__ __launch_bounds__(kBwdThreads) void bwd_reduce_rows_kernel(int n_chunks, int hkv, int64_t total_kept,
                                                                      int64_t kv_elems, const float* __restrict__ dk_part,
                                                                      const float* __restrict__ dv_part,
                                                                      const float* __restrict__ ds_part,
                                                                      float* __restrict__ dk, float* __restrict__ dv,
                                                                      float* __restrict__ ds) {
  const int64_t i = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;  // 4-float group of dk / dv, or a ds row
  const int64_t n4 = kv_elems / 4;
  if (i < n4) {
    f32x4 a = *reinterpret_cast<const f32x4*>(dk_part + 4 * i);
    f32x4 b = *reinterpret_cast<const f32x4*>(dv_part + 4 * i);
    for (int c = 1; c < n_chunks; ++c) {
      a += *reinterpret_cast<const f32x4*>(dk_part + c * kv_elems + 4 * i);
      b += *reinterpret_cast<const f32x4*>(dv_part + c * kv_elems + 4 * i);
    }
    *reinterpret_cast<f32x4*>(dk + 4 * i) = a;
    *reinterpret_cast<f32x4*>(dv + 4 * i) = b;
  } else if (ds != nullptr && i - n4 < total_kept) {
    const int64_t t = i - n4;
    float a = 0.0f;
    for (int c = 0; c < n_chunks; ++c)
      for (int h = 0; h < hkv; ++h) a += ds_part[((int64_t)c * hkv + h) * total_kept + t];
    ds[t] = a;
  }
}

// dgain / dtau = sum over the workgroup slots that ran, one block per head
__global__ __launch_bounds__(kBwdThreads) void bwd_reduce_params_kernel(SegTable segs, int n_seg,
                                                                        int slots_per_seg, int n_chunks, int hq,
                                                                        const float* __restrict__ part_g,
                                                                        const float* __restrict__ part_t,
                                                                        float* __restrict__ dgain,
                                                                        float* __restrict__ dtau) {
  __shared__ float red[2][kBwdThreads];
  const int tid = threadIdx.x, h = blockIdx.x;
  float sg = 0.0f, st = 0.0f;
  const int64_t n_slots = (int64_t)n_seg * slots_per_seg;
  for (int64_t s = tid; s < n_slots; s += kBwdThreads) {
    const int seg_i = (int)(s / slots_per_seg), y = (int)(s % slots_per_seg);
    if ((y / n_chunks) * kKeyBlock < segs.at(seg_i).kept_len) {
      sg += part_g[s * hq + h];
      st += part_t[s * hq + h];
    }
  }
  red[0][tid] = sg;
  red[1][tid] = st;
  __syncthreads();
  for (int w = kBwdThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      red[0][tid] += red[0][tid + w];
      red[1][tid] += red[1][tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (dgain != nullptr) dgain[h] = red[0][0];
    if (dtau != nullptr) dtau[h] = red[1][0];
  }
}

// Work split of bwd_dkdv: 128-key blocks x query chunks of qc 32-row blocks.
// Up to four chunks per key block (then the longest workgroup walks a quarter
// of the prompt), but only as many as needed for about two workgroups per CU:
// every chunk costs a pass over fp32 dK / dV partials.
struct BwdGeom {
  int key_blocks, qc, n_chunks;
  int64_t n_slots;
};
BwdGeom bwd_geom(const tg_plan_info& info, int hkv) {
  BwdGeom g;
  const int max_len = (int)info.max_kept_len;
  g.key_blocks = max(1, (max_len + kKeyBlock - 1) / kKeyBlock);
  const int max_qb = max(1, (max_len + 31) / 32);
  const int64_t wgs = (int64_t)hkv * g.key_blocks * info.n_seg;
  const int want = (int)min((int64_t)4, max((int64_t)1, (512 + wgs - 1) / wgs));
  g.qc = max(8, (max_qb + want - 1) / want);
  g.n_chunks = (max_qb + g.qc - 1) / g.qc;
  g.n_slots = (int64_t)info.n_seg * g.key_blocks * g.n_chunks;
  return g;
}

struct BwdWs {
  float* dt;
  float* ds_part;
  float* dk_part;
  float* dv_part;
  float* part_g;
  float* part_t;
};

int64_t round64(int64_t x) { return (x + 63) / 64 * 64; }

int64_t bwd_ws_floats(const tg_plan_info& info, int hq, int hkv, int head_dim) {
  const BwdGeom g = bwd_geom(info, hkv);
  const int64_t kv = info.total_kept * hkv * head_dim;
  return round64(info.total_kept * hq) + round64((int64_t)g.n_chunks * hkv * info.total_kept) +
         2 * round64(g.n_chunks * kv) + 2 * g.n_slots * hq;
}

BwdWs carve(void* ws, const tg_plan_info& info, int hq, int hkv, int head_dim) {
  const BwdGeom g = bwd_geom(info, hkv);
  const int64_t kv = info.total_kept * hkv * head_dim;
  BwdWs w;
  w.dt = reinterpret_cast<float*>(ws);
  w.ds_part = w.dt + round64(info.total_kept * hq);
  w.dk_part = w.ds_part + round64((int64_t)g.n_chunks * hkv * info.total_kept);
  w.dv_part = w.dk_part + round64(g.n_chunks * kv);
  w.part_g = w.dv_part + round64(g.n_chunks * kv);
  w.part_t = w.part_g + g.n_slots * hq;
  return w;
}

template <int D, int G>
hipError_t launch_bwd_dg(const void* q, const void* k, const void* v, const float* ks, const float* tau,
                         const float* gain, const tg_segment* segs_in, const tg_plan_info& info, int hq, int hkv,
                         const void* out, const void* dout, const float* lse, float* dq, float* dk, float* dv,
                         float* ds, float* dgain, float* dtau, void* workspace, hipStream_t stream) {
  const SegTable segs = seg_table(segs_in, info);
  const BwdWs w = carve(workspace, info, hq, hkv, D);
  const BwdGeom geo = bwd_geom(info, hkv);
  auto* qb = reinterpret_cast<const uint16_t*>(q);
  auto* kb = reinterpret_cast<const uint16_t*>(k);
  auto* vb = reinterpret_cast<const uint16_t*>(v);
  auto* ob = reinterpret_cast<const uint16_t*>(out);
  auto* dob = reinterpret_cast<const uint16_t*>(dout);
  if (info.total_kept > 0) {  // with no kept rows only the parameter reduction runs (zero dgain / dtau)
    const int64_t rows = info.total_kept * hq;
    const int per_block = kBwdThreads / (D / 8);
    hipLaunchKernelGGL((bwd_rowdot_kernel<D>), dim3((unsigned)((rows + per_block - 1) / per_block)),
                       dim3(kBwdThreads), 0, stream, dob, ob, rows, w.dt);
    // the DMA kernels address a prompt's rows with 32-bit buffer ranges (Q / dO: hq heads per row)
    const bool kv_fits = (int64_t)info.max_kept_len * hkv * D * 2 < 0xffffff00LL;
    const bool q_fits = (int64_t)info.max_kept_len * hq * D * 4 < 0xffffff00LL;
    if (D == 128 && kv_fits && q_fits)
      hipLaunchKernelGGL((bwd_dkdv_dma_kernel<G>), dim3(hkv, geo.key_blocks * geo.n_chunks, info.n_seg),
                         dim3(kDkdvThreads), 0, stream, qb, kb, vb, ks, tau, gain, segs, hq, hkv, dob, lse, w.dt,
                         geo.n_chunks, geo.qc, w.dk_part, w.dv_part, w.ds_part, info.total_kept, w.part_g, w.part_t);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, G>), dim3(hkv, geo.key_blocks * geo.n_chunks, info.n_seg),
                         dim3(kDkdvThreads), 0, stream, qb, kb, vb, ks, tau, gain, segs, hq, hkv, dob, lse, w.dt,
                         geo.n_chunks, geo.qc, w.dk_part, w.dv_part, w.ds_part, info.total_kept, w.part_g, w.part_t);
    constexpr int kBM = 128 / G;
    const int q_tiles = (int)((info.max_kept_len + kBM - 1) / kBM);
    // the DMA kernel addresses a prompt's K / V rows with 32-bit buffer ranges
    const bool dq_dma = D == 128 && kv_fits;
    if (dq_dma)
      hipLaunchKernelGGL((bwd_dq_dma_kernel<G>), dim3(hkv, q_tiles, info.n_seg), dim3(kDqThreads), 0, stream, qb, kb,
                         vb, ks, tau, gain, segs, hq, hkv, dob, lse, w.dt, dq);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, G>), dim3(hkv, q_tiles, info.n_seg), dim3(kBwdThreads), 0, stream, qb,
                         kb, vb, ks, tau, gain, segs, hq, hkv, dob, lse, w.dt, dq);
    const int64_t kv_elems = info.total_kept * hkv * D;
    const int64_t items = kv_elems / 4 + info.total_kept;
    hipLaunchKernelGGL(bwd_reduce_rows_kernel, dim3((unsigned)((items + kBwdThreads - 1) / kBwdThreads)),
                       dim3(kBwdThreads), 0, stream, geo.n_chunks, hkv, info.total_kept, kv_elems, w.dk_part,
                       w.dv_part, w.ds_part, dk, dv, ds);
  }
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3(hq), dim3(kBwdThreads), 0, stream, segs, info.n_seg,
                     geo.key_blocks * geo.n_chunks, geo.n_chunks, hq, w.part_g, w.part_t, dgain, dtau);
  return hipGetLastError();
}

}  // namespace

size_t attention_backward_workspace_bytes(const tg_plan_info& info, int hq, int hkv, int head_dim) {
  return (size_t)(bwd_ws_floats(info, hq, hkv, head_dim) * 4);
}

hipError_t launch_gated_attention_backward(const void* q, const void* k, const void* v, const float* key_score,
                                           const float* tau, const float* gain, const tg_segment* segs,
                                           const tg_plan_info& info, int hq, int hkv, int head_dim, const void* out,
                                           const void* dout, const float* lse, float* dq, float* dk, float* dv,
                                           float* ds, float* dgain, float* dtau, void* workspace,
                                           hipStream_t stream) {
  const int G = hq / hkv;
#define TG_BWD_CASE(DD, GG) \
  if (head_dim == DD && G == GG) \
    return launch_bwd_dg<DD, GG>(q, k, v, key_score, tau, gain, segs, info, hq, hkv, out, dout, lse, dq, dk, dv, ds, \
                                 dgain, dtau, workspace, stream);
  TG_BWD_CASE(128, 1)
  TG_BWD_CASE(128, 2)
  TG_BWD_CASE(128, 4)
  TG_BWD_CASE(64, 1)
  TG_BWD_CASE(64, 2)
  TG_BWD_CASE(64, 4)
#undef TG_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace tg
