// Dense decoder-layer support kernels (gfx950): bf16 GEMM with fused
// epilogues, RMSNorm and rotary embedding.  They run the layers below and
// above the gate of a Qwen3-1.7B-shaped stack (RMSNorm -> QKV -> RoPE ->
// attention -> O + residual -> RMSNorm -> SwiGLU MLP + residual); the gate,
// selector, compaction and token-gated attention are the other kernels of
// this library ("TokenGate 与 T2Quant ... 精读", section 4.1: the layers above
// the gate run on the kept tokens only).
//
// GEMM: Y[m][n] = sum_k X[m][k] W[n][k] (X activations, W weights, both
// k-contiguous), fp32 accumulation on v_mfma_f32_32x32x16_bf16.  The product
// is computed transposed (W rows on the MFMA rows), so each lane owns one
// activation row and 16 output columns per 32x32 tile: four runs of four
// consecutive columns (8-byte stores), and with W's gate/up rows interleaved
// in groups of 8 the SwiGLU pair of an output column sits in the same lane.
// gemm_kernel: workgroup tile 128 (n) x 256 (m), 4 waves of 64 x 128, k step
// 64, both operands double-buffered in LDS (padded rows: conflict-free 16-byte
// reads), the next k block prefetched into registers while the current one is
// multiplied.  gemm_dma_kernel (n a multiple of 256) is described at its
// definition.
#include "common.h"

namespace tg {
namespace {

constexpr int kGT = 256;       // threads
constexpr int kBN = 128;       // weight rows (output columns) per workgroup
constexpr int kBM = 256;       // activation rows per workgroup
constexpr int kBK = 64;        // k per stage
constexpr int kLd = kBK + 8;   // LDS row stride (bf16)
constexpr int kWN = 64;        // per-wave tile: 64 output columns
constexpr int kWM = 128;       //                x 128 activation rows
constexpr int kTN = kWN / 32;  // 2 MFMA tiles along n
constexpr int kTM = kWM / 32;  // 4 MFMA tiles along m
// loads of one stage: (128 + 256) rows x 128 bytes = 3072 16-byte units, 12 per thread
constexpr int kLoadsW = kBN * kBK / 8 / kGT;  // 4
constexpr int kLoadsX = kBM * kBK / 8 / kGT;  // 8

enum Epi { kEpiStore = 0, kEpiResidual = 1, kEpiSwiGLU = 2 };

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __builtin_amdgcn_exp2f(-v * 1.4426950408889634f)); }

template <int EPI>
__global__ __launch_bounds__(kGT) void gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                   const uint16_t* __restrict__ w, int64_t ldw, int64_t m, int n, int k,
                                                   const uint16_t* __restrict__ res, int64_t ldr,
                                                   uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][kBN * kLd];
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kBM * kLd];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = blockIdx.x * kBN;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int wn = (wave & 1) * kWN;  // wave's column offset inside the tile
  const int wm = (wave >> 1) * kWM;  // wave's row offset inside the tile

  // per-thread load slots: unit u = i * 256 + tid -> row u / 8, 16-byte column (u % 8) * 8
  const uint16_t* wsrc[kLoadsW];
  const uint16_t* xsrc[kLoadsX];
#pragma unroll
  for (int i = 0; i < kLoadsW; ++i) {
    const int u = i * kGT + tid;
    wsrc[i] = w + (int64_t)(n0 + u / 8) * ldw + (u % 8) * 8;
  }
#pragma unroll
  for (int i = 0; i < kLoadsX; ++i) {
    const int u = i * kGT + tid;
    int64_t r = m0 + u / 8;
    if (r >= m) r = m - 1;  // rows past the end re-read the last row; their results are not stored
    xsrc[i] = x + r * ldx + (u % 8) * 8;
  }
  auto load_stage = [&](int kk, u32x4 (&rw)[kLoadsW], u32x4 (&rx)[kLoadsX]) {
#pragma unroll
    for (int i = 0; i < kLoadsW; ++i) rw[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + kk);
#pragma unroll
    for (int i = 0; i < kLoadsX; ++i) rx[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + kk);
  };
  auto store_stage = [&](int buf, const u32x4 (&rw)[kLoadsW], const u32x4 (&rx)[kLoadsX]) {
#pragma unroll
    for (int i = 0; i < kLoadsW; ++i) {
      const int u = i * kGT + tid;
      *reinterpret_cast<u32x4*>(&ws[buf][(u / 8) * kLd + (u % 8) * 8]) = rw[i];
    }
#pragma unroll
    for (int i = 0; i < kLoadsX; ++i) {
      const int u = i * kGT + tid;
      *reinterpret_cast<u32x4*>(&xs[buf][(u / 8) * kLd + (u % 8) * 8]) = rx[i];
    }
  };

  f32x16 acc[kTN][kTM];
#pragma unroll
  for (int a = 0; a < kTN; ++a)
#pragma unroll
    for (int b = 0; b < kTM; ++b) acc[a][b] = f32x16{};

  u32x4 rw[kLoadsW], rx[kLoadsX];
  load_stage(0, rw, rx);
  store_stage(0, rw, rx);
  __syncthreads();
  const int nk = k / kBK;
  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < nk;
    if (more) load_stage((kb + 1) * kBK, rw, rx);
    const uint16_t* wb = ws[buf];
    const uint16_t* xb = xs[buf];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      u32x4 fa[kTN], fb[kTM];
#pragma unroll
      for (int a = 0; a < kTN; ++a)
        fa[a] = *reinterpret_cast<const u32x4*>(wb + (wn + 32 * a + l32) * kLd + 16 * ks + 8 * g);
#pragma unroll
      for (int b = 0; b < kTM; ++b)
        fb[b] = *reinterpret_cast<const u32x4*>(xb + (wm + 32 * b + l32) * kLd + 16 * ks + 8 * g);
#pragma unroll
      for (int a = 0; a < kTN; ++a)
#pragma unroll
        for (int b = 0; b < kTM; ++b) acc[a][b] = mfma32(fa[a], fb[b], acc[a][b]);
      __builtin_amdgcn_sched_group_barrier(0x100, kTN + kTM, 0);  // the step's LDS reads first
      __builtin_amdgcn_sched_group_barrier(0x008, kTN * kTM, 0);  // then its MFMAs
    }
    if (more) store_stage(buf ^ 1, rw, rx);
    __syncthreads();
  }

  // Epilogue.  acc[a][b] register i: output column n0 + wn + 32 a + 8 (i / 4) + 4 g + (i % 4),
  // activation row m0 + wm + 32 b + l32.
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int b = 0; b < kTM; ++b) {
    const int64_t row = m0 + wm + 32 * b + l32;
    if (row >= m) continue;
#pragma unroll
    for (int a = 0; a < kTN; ++a) {
      if (EPI == kEpiSwiGLU) {
        // weight rows come in groups of 8: gate j .. j+7 then up j .. j+7, so registers i and i + 4
        // (i % 8 < 4) hold gate and up of the same intermediate column
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c0 = (n0 + wn + 32 * a) / 2 + 8 * q + 4 * g;  // intermediate column of register 8 q
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = silu(acc[a][b][8 * q + e]) * acc[a][b][8 * q + 4 + e];
          const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r[0], r[1]}), bf16x2));
          const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r[2], r[3]}), bf16x2));
          *reinterpret_cast<u32x2*>(y + row * ldy + c0) = u32x2{w0, w1};
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn + 32 * a + 8 * q + 4 * g;
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = acc[a][b][4 * q + e];
          if (EPI == kEpiResidual) {
            const u32x2 rv = *reinterpret_cast<const u32x2*>(res + row * ldr + col);
            r[0] += bf16_lo(rv[0]);
            r[1] += bf16_hi(rv[0]);
            r[2] += bf16_lo(rv[1]);
            r[3] += bf16_hi(rv[1]);
          }
          const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r[0], r[1]}), bf16x2));
          const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r[2], r[3]}), bf16x2));
          *reinterpret_cast<u32x2*>(y + row * ldy + col) = u32x2{w0, w1};
        }
      }
    }
  }
}

// Large-tile GEMM for n % 256 == 0 (the stack's projections): the same product, orientation and epilogues as
// gemm_kernel, on a 256 (n) x 256 (m) workgroup tile with 8 waves (two per SIMD, so one wave's LDS reads and
// waits overlap the other's MFMAs), each wave 128 output columns x 64 activation rows (4 x 2 MFMA tiles: six
// fragment reads feed eight MFMAs).  Both operand tiles go from global memory straight into LDS with buffer
// loads that have an LDS destination (no staging registers, no LDS store instructions; the buffer range check
// zero-fills rows past m), two 64 KiB stages: the loads of k block kb + 1 are issued before block kb is
// multiplied and waited for after it.  Tiles are stored as 128-byte rows of eight 16-byte chunks, chunk c of
// row r at c ^ ((r >> 1) & 7), so each 16-lane group of a fragment read covers 16 distinct chunk slots of the
// 256-byte LDS cycle (conflict free).
constexpr int kDT = 512;   // threads
constexpr int kDN = 256;   // output columns (weight rows) per workgroup
constexpr int kDK = 64;    // k per stage
constexpr int kDWN = 128;  // per-wave tile: 128 output columns x 64 activation rows
constexpr int kDTN = kDWN / 32;

constexpr int kDM = 256;   // activation rows per workgroup
constexpr int kDWM = 64;
constexpr int kDTM = kDWM / 32;

struct GemmDmaSmem {
  uint16_t w[2][kDN * kDK];
  uint16_t x[2][kDM * kDK];
};

__device__ __forceinline__ int dchunk(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int EPI>
__global__ __launch_bounds__(kDT) void gemm_dma_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                       const uint16_t* __restrict__ w, int64_t ldw, int64_t m, int n,
                                                       int k, const uint16_t* __restrict__ res, int64_t ldr,
                                                       uint16_t* __restrict__ y, int64_t ldy) {
  constexpr int kJ = 8;  // wave loads per wave per stage (32 for the W tile, 32 for the X tile)
  __shared__ GemmDmaSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = blockIdx.x * kDN;
  const int64_t m0 = (int64_t)blockIdx.y * kDM;
  const int wn = (wave & 1) * kDWN;
  const int wm = (wave >> 1) * kDWM;

  // Buffer ranges: this tile's weight rows (n is a multiple of 256) and activation rows (rows past m read 0).
  const int64_t m_rows = m - m0 < kDM ? m - m0 : kDM;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (int64_t)n0 * ldw, (uint32_t)(kDN * ldw * 2));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + m0 * ldx, (uint32_t)(m_rows * ldx * 2));
  // DMA slots: a stage is 2048 16-byte slots of W then 2048 of X, 64 wave loads of 64 slots; wave w issues
  // loads j * 8 + w.  Slot s of a tile holds row s / 8, physical chunk s % 8 = lane % 8, i.e. logical
  // chunk dchunk(row, lane % 8).
  uint32_t voff[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int t = j * 8 + wave;  // 0..31: W tile, 32..: X tile
    const int s = (t & 31) * 64 + lane;
    const int row = s >> 3;
    const int64_t ld = t < 32 ? ldw : ldx;
    voff[j] = (uint32_t)(row * ld * 2 + dchunk(row, lane & 7) * 16);
  }
  auto issue = [&](int kb, int buf) {
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int t = j * 8 + wave;
      uint16_t* dst = t < 32 ? &sm.w[buf][t * 512] : &sm.x[buf][(t - 32) * 512];
      dma16(t < 32 ? rw : rx, dst, voff[j], (uint32_t)(kb * kDK * 2));
    }
  };

  f32x16 acc[kDTN][kDTM];
#pragma unroll
  for (int a = 0; a < kDTN; ++a)
#pragma unroll
    for (int b = 0; b < kDTM; ++b) acc[a][b] = f32x16{};

  // fragment addresses (bf16 elements) of this lane's rows, chunk 2 ks + g applied per step
  int ra[kDTN], rb[kDTM];
#pragma unroll
  for (int a = 0; a < kDTN; ++a) ra[a] = wn + 32 * a + l32;
#pragma unroll
  for (int b = 0; b < kDTM; ++b) rb[b] = wm + 32 * b + l32;

  const int nk = k / kDK;
  issue(0, 0);
  wait_vm<0>();
  lds_barrier();
  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nk) issue(kb + 1, buf ^ 1);
    const uint16_t* wb = sm.w[buf];
    const uint16_t* xb = sm.x[buf];
    // fragments of k step ks + 1 are read while the MFMAs of step ks run
    u32x4 fa[2][kDTN], fb[2][kDTM];
    auto read = [&](int ks, int set) {
#pragma unroll
      for (int a = 0; a < kDTN; ++a)
        fa[set][a] = *reinterpret_cast<const u32x4*>(wb + ra[a] * kDK + dchunk(ra[a], 2 * ks + g) * 8);
#pragma unroll
      for (int b = 0; b < kDTM; ++b)
        fb[set][b] = *reinterpret_cast<const u32x4*>(xb + rb[b] * kDK + dchunk(rb[b], 2 * ks + g) * 8);
    };
    read(0, 0);
#pragma unroll
    for (int ks = 0; ks < kDK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < kDK / 16) read(ks + 1, cur ^ 1);
#pragma unroll
      for (int a = 0; a < kDTN; ++a)
#pragma unroll
        for (int b = 0; b < kDTM; ++b) acc[a][b] = mfma32(fa[cur][a], fb[cur][b], acc[a][b]);
      if (ks + 1 < kDK / 16) {
#pragma unroll
        for (int i = 0; i < kDTN + kDTM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kDTN * kDTM - (kDTN + kDTM), 0);
      }
    }
    wait_vm<0>();   // this wave's loads of block kb + 1 have landed
    lds_barrier();  // every wave's have, and every wave is done reading block kb
  }

  // Epilogue, as gemm_kernel's: acc[a][b] register i holds output column n0 + wn + 32 a + 8 (i / 4) + 4 g + (i % 4)
  // of activation row m0 + wm + 32 b + l32.
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int b = 0; b < kDTM; ++b) {
    const int64_t row = m0 + wm + 32 * b + l32;
    if (row >= m) continue;
#pragma unroll
    for (int a = 0; a < kDTN; ++a) {
      if (EPI == kEpiSwiGLU) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c0 = (n0 + wn + 32 * a) / 2 + 8 * q + 4 * g;
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = silu(acc[a][b][8 * q + e]) * acc[a][b][8 * q + 4 + e];
          const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r[0], r[1]}), bf16x2));
          const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r[2], r[3]}), bf16x2));
          *reinterpret_cast<u32x2*>(y + row * ldy + c0) = u32x2{w0, w1};
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn + 32 * a + 8 * q + 4 * g;
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = acc[a][b][4 * q + e];
          if (EPI == kEpiResidual) {
            const u32x2 rv = *reinterpret_cast<const u32x2*>(res + row * ldr + col);
            r[0] += bf16_lo(rv[0]);
            r[1] += bf16_hi(rv[0]);
            r[2] += bf16_lo(rv[1]);
            r[3] += bf16_hi(rv[1]);
          }
          const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r[0], r[1]}), bf16x2));
          const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r[2], r[3]}), bf16x2));
          *reinterpret_cast<u32x2*>(y + row * ldy + col) = u32x2{w0, w1};
        }
      }
    }
  }
}

// RMSNorm of bf16 rows: y = x / sqrt(mean(x^2) + eps) * weight, fp32 math, one wave per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, int64_t ldx, int64_t m, int d,
                                                      const uint16_t* __restrict__ weight, float eps,
                                                      uint16_t* __restrict__ y, int64_t ldy) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* xr = x + row * ldx;
  float ss = 0.0f;
  for (int c = lane * 8; c < d; c += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(v[j]), b = bf16_hi(v[j]);
      ss += a * a + b * b;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float inv = 1.0f / __builtin_sqrtf(ss / (float)d + eps);
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  for (int c = lane * 8; c < d; c += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
    const u32x4 wv = *reinterpret_cast<const u32x4*>(weight + c);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                               (f32x2{bf16_lo(v[j]) * inv * bf16_lo(wv[j]),
                                                      bf16_hi(v[j]) * inv * bf16_hi(wv[j])}),
                                               bf16x2));
    *reinterpret_cast<u32x4*>(y + row * ldy + c) = o;
  }
}

// RoPE (rotate-half) of Q and K and the Q/K/V split: the fused projection
// output [m, (hq + 2 hkv) D] is written to separate token-major Q, K, V
// arrays.  Position p of row r is positions[r]; pair i (i < D/2) of every Q
// and K head turns by p * theta^(-2 i / D), the angle and its sin / cos taken
// in fp64 (at positions up to 2^17 an fp32 angle, or an fp32 log2 theta,
// carries errors of 1e-3 .. 1e-2 rad) and rounded to fp32 once per row: one
// wave per row computes the row's D/2 angles into LDS, then rotates all
// hq + hkv heads with them and copies V.
__global__ __launch_bounds__(256) void rope_split_kernel(const uint16_t* __restrict__ qkv, int64_t ldqkv, int64_t m,
                                                         int hq, int hkv, int dh, const int32_t* __restrict__ positions,
                                                         double log2_theta, uint16_t* __restrict__ q,
                                                         uint16_t* __restrict__ k, uint16_t* __restrict__ v) {
  __shared__ float tab[4][2][128];  // per wave: cos, sin of the row's angles (dh <= 256)
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  const bool on = row < m;
  const int half = dh / 2;
  if (on) {
    const double p = (double)positions[row];
    for (int i = lane; i < half; i += 64) {
      const double ang = p * exp2(-log2_theta * (2.0 * (double)i / (double)dh));
      double sd, cd;
      sincos(ang, &sd, &cd);
      tab[wave][0][i] = (float)cd;
      tab[wave][1][i] = (float)sd;
    }
  }
  __syncthreads();
  if (!on) return;
  const uint16_t* src = qkv + row * ldqkv;
  for (int h = 0; h < hq + hkv; ++h) {
    const uint16_t* sh = src + (int64_t)h * dh;
    uint16_t* dst = h < hq ? q + (row * hq + h) * dh : k + (row * hkv + (h - hq)) * dh;
    for (int i = lane; i < half; i += 64) {
      const float c = tab[wave][0][i], s = tab[wave][1][i];
      const float x1 = bf16_lo((uint32_t)sh[i]), x2 = bf16_lo((uint32_t)sh[i + half]);
      dst[i] = (uint16_t)f32_to_bf16(x1 * c - x2 * s);
      dst[i + half] = (uint16_t)f32_to_bf16(x2 * c + x1 * s);
    }
  }
  const uint16_t* sv = src + (int64_t)(hq + hkv) * dh;
  uint16_t* dv = v + row * hkv * dh;
  for (int e = lane; e < hkv * dh; e += 64) dv[e] = sv[e];
}

}  // namespace

hipError_t launch_gemm(int epi, const void* x, int64_t ldx, const void* w, int64_t ldw, int64_t m, int n, int k,
                       const void* res, int64_t ldr, void* y, int64_t ldy, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
  const uint16_t* wp = reinterpret_cast<const uint16_t*>(w);
  const uint16_t* rp = reinterpret_cast<const uint16_t*>(res);
  uint16_t* yp = reinterpret_cast<uint16_t*>(y);
  // the large-tile kernel: whole 256-column tiles, and 32-bit buffer ranges and offsets for a 256-row tile
  if (n % kDN == 0 && (int64_t)kDN * ldw * 2 < 0x7fffffffLL && (int64_t)kDM * ldx * 2 < 0x7fffffffLL) {
    dim3 grid2(n / kDN, (unsigned)((m + kDM - 1) / kDM));
    if (epi == kEpiStore)
      hipLaunchKernelGGL(gemm_dma_kernel<kEpiStore>, grid2, dim3(kDT), 0, stream, xp, ldx, wp, ldw, m, n, k, rp, ldr,
                         yp, ldy);
    else if (epi == kEpiResidual)
      hipLaunchKernelGGL(gemm_dma_kernel<kEpiResidual>, grid2, dim3(kDT), 0, stream, xp, ldx, wp, ldw, m, n, k, rp,
                         ldr, yp, ldy);
    else
      hipLaunchKernelGGL(gemm_dma_kernel<kEpiSwiGLU>, grid2, dim3(kDT), 0, stream, xp, ldx, wp, ldw, m, n, k, rp,
                         ldr, yp, ldy);
    return hipGetLastError();
  }
  dim3 grid(n / kBN, (unsigned)((m + kBM - 1) / kBM));
  if (epi == kEpiStore)
    hipLaunchKernelGGL(gemm_kernel<kEpiStore>, grid, dim3(kGT), 0, stream, xp, ldx, wp, ldw, m, n, k, rp, ldr, yp, ldy);
  else if (epi == kEpiResidual)
    hipLaunchKernelGGL(gemm_kernel<kEpiResidual>, grid, dim3(kGT), 0, stream, xp, ldx, wp, ldw, m, n, k, rp, ldr, yp,
                       ldy);
  else
    hipLaunchKernelGGL(gemm_kernel<kEpiSwiGLU>, grid, dim3(kGT), 0, stream, xp, ldx, wp, ldw, m, n, k, rp, ldr, yp,
                       ldy);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const void* x, int64_t ldx, int64_t m, int d, const void* weight, float eps, void* y,
                          int64_t ldy, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)((m + 3) / 4)), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), ldx, m, d, reinterpret_cast<const uint16_t*>(weight), eps,
                     reinterpret_cast<uint16_t*>(y), ldy);
  return hipGetLastError();
}

hipError_t launch_rope_split(const void* qkv, int64_t ldqkv, int64_t m, int hq, int hkv, int dh,
                             const int32_t* positions, float theta, void* q, void* k, void* v, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_split_kernel, dim3((unsigned)((m + 3) / 4)), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(qkv), ldqkv, m, hq, hkv, dh, positions, log2((double)theta),
                     reinterpret_cast<uint16_t*>(q), reinterpret_cast<uint16_t*>(k), reinterpret_cast<uint16_t*>(v));
  return hipGetLastError();
}

}  // namespace tg
