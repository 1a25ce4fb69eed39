// Gate score kernels (gfx950).
//
// TokenGate's gate ("TokenGate 与 T2Quant ... 精读", section 4.1, component one):
// a small MLP reads the hidden row of every prunable token and outputs one
// scalar; the scalars are RMS-normalised along the prompt's document and the
// non-prunable tokens get a fixed 0.
//
// Kernel 1 (gate_mlp): one workgroup owns 64 document rows and all h hidden
// units.  U^T = W1 . X^T runs on v_mfma_f32_32x32x16_bf16 with W1 as the A
// operand (read straight from global memory: every wave owns a disjoint
// 64-unit slice of W1, so there is nothing to share) and the X tile as the B
// operand (staged through LDS, double-buffered, shared by the 4 waves).
// Putting W1 on the rows of the product leaves each lane with one token
// column, so the epilogue (bias, erf-GELU, w2 dot) reduces over hidden units
// inside the lane's registers, then across the two half-waves and the four
// waves in a fixed order.  Hidden activations stay fp32; nothing is rounded
// to bf16 after the first layer.  The raw score r_j goes to `scores`, the
// tile's sum of squares (fp64) to the workspace.
//
// Kernel 2 (gate_normalize): every block re-reduces its prompt's tile sums
// in the same fixed order (so all blocks agree bit for bit), then rescales
// its tokens and writes 0 for non-document tokens.
#include "common.h"

namespace tg {
namespace {

constexpr int kRows = 64;      // document rows per workgroup
constexpr int kKB = 64;        // d per pipeline stage
constexpr int kThreads = 256;  // 4 waves
constexpr int kXLd = kKB + 8;  // LDS row stride in bf16 (144 B: conflict-free 16-byte reads)

// GELU(u) = u Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), with erf from Abramowitz &
// Stegun, Handbook of Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7):
//   erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),  t = 1 / (1 + p z),  z >= 0.
// With q = erfc(|z|) from that formula, 1 + erf(z) is 2 - q for z >= 0 and q otherwise.
__device__ __forceinline__ float gelu_erf(float u) {
  const float z = fabsf(u) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.0f));
  float p = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  p = __builtin_fmaf(p, t, 1.421413741f);
  p = __builtin_fmaf(p, t, -0.284496736f);
  p = __builtin_fmaf(p, t, 0.254829592f);
  p *= t;
  const float q = p * __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);
  return 0.5f * u * (u >= 0.0f ? 2.0f - q : q);
}

// Loads this thread's share of an X stage (64 rows x 64 k): 8 threads per
// 128-byte row, rows tid / 8 and 32 + tid / 8, 16 bytes at column (tid % 8) * 8.
// Rows past the tile's last document row re-read that row (their results are
// discarded), so the load is unconditional.
__device__ __forceinline__ void load_x_stage(const uint16_t* __restrict__ x, int64_t ld_x, int64_t row0, int nrows,
                                             int k0, int tid, u32x4 (&p)[2]) {
  const int c = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = min((tid >> 3) + 32 * i, nrows - 1);
    p[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (row0 + r) * ld_x + k0 + c));
  }
}

__device__ __forceinline__ void store_x_stage(uint16_t* lds, int tid, const u32x4 (&p)[2]) {
  const int c = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(lds + ((tid >> 3) + 32 * i) * kXLd + c) = p[i];
}

// W1 in MFMA-fragment order (built by pack_w1_kernel in the workspace): for
// k block kb, 32-unit tile ut and MFMA step j, 64 lanes x 16 bytes are
// contiguous, lane l holding W1[32 ut + l % 32][64 kb + 32 (l / 32) + 8 j .. + 7].
// Every wave load is then one contiguous KiB.  MFMA step j of a k block
// consumes k = 32 g + 8 j .. + 7 on both operands (a permutation of the block's
// k order, applied identically to X).
__device__ __forceinline__ void load_w_frag(const u32x4* __restrict__ w1p, int n_ut, int ut, int kb, int lane,
                                            u32x4 (&w)[4]) {
  const u32x4* src = w1p + ((int64_t)(kb * n_ut + ut) * 4) * 64 + lane;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = src[j * 64];
}

__global__ __launch_bounds__(256) void pack_w1_kernel(const uint16_t* __restrict__ w1, int d, int h,
                                                      u32x4* __restrict__ w1p) {
  // one thread per packed 16-byte chunk: chunk = ((kb * n_ut + ut) * 4 + j) * 64 + lane
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)d * h / 8;
  if (i >= total) return;
  const int lane = (int)(i & 63);
  const int j = (int)((i >> 6) & 3);
  const int64_t rest = i >> 8;
  const int n_ut = h / 32;
  const int ut = (int)(rest % n_ut);
  const int kb = (int)(rest / n_ut);
  const int unit = 32 * ut + (lane & 31);
  const int k = 64 * kb + 32 * (lane >> 5) + 8 * j;
  w1p[i] = *reinterpret_cast<const u32x4*>(w1 + (int64_t)unit * d + k);
}

// NCT: 32-unit column tiles per wave (1 or 2).  S: k blocks in flight (W1 and
// X are prefetched S - 1 blocks ahead in registers); d / 64 is a multiple of S,
// so the pipelined loop has no guards and the compiler can count the loads
// still in flight exactly.
template <int NCT, int S>
__global__ __launch_bounds__(kThreads) void gate_mlp_kernel(const uint16_t* __restrict__ x, int64_t ld_x, int d,
                                                            const u32x4* __restrict__ w1p,
                                                            const float* __restrict__ b1,
                                                            const float* __restrict__ w2, float b2, int h,
                                                            const tg_segment* __restrict__ segs, int max_tiles,
                                                            float* __restrict__ scores,
                                                            double* __restrict__ tile_sumsq) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kRows * kXLd];
  __shared__ float red[4][kRows];
  __shared__ double red2[kRows];

  const tg_segment seg = segs[blockIdx.y];
  const int n_doc = seg.doc_end - seg.doc_begin;
  const int tile = blockIdx.x;
  if (tile * kRows >= n_doc) return;  // uniform across the workgroup
  const int64_t row0 = (int64_t)seg.seg_start + seg.doc_begin + (int64_t)tile * kRows;
  const int nrows = min(kRows, n_doc - tile * kRows);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int unit_base = wave * 32 * NCT;
  const bool active = unit_base < h;  // waves past h compute on a valid slice and drop the result
  const int ut0 = active ? unit_base / 32 : 0;
  const int n_ut = h / 32;

  f32x16 acc[NCT][2];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) acc[ct][rt] = f32x16{};

  const int nkb = d / kKB;
  u32x4 wr[S][NCT][4];  // W1 ring (registers)
  u32x4 xr[S][2];       // X ring (registers; written to LDS one block ahead of use)

  // prologue: blocks 0 .. S-2 in flight, block 0 in LDS
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    load_x_stage(x, ld_x, row0, nrows, s * kKB, tid, xr[s]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) load_w_frag(w1p, n_ut, ut0 + ct, s, lane, wr[s][ct]);
  }
  if (S == 1) {
    load_x_stage(x, ld_x, row0, nrows, 0, tid, xr[0]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) load_w_frag(w1p, n_ut, ut0 + ct, 0, lane, wr[0][ct]);
  }
  store_x_stage(xs[0], tid, xr[0]);
  __syncthreads();

  for (int kb0 = 0; kb0 < nkb; kb0 += S) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int kb = kb0 + s;
      // block kb + S - 1 starts loading now (clamped: the tail re-reads the last block)
      const int kn = min(kb + S - 1, nkb - 1);
      if (S > 1) {
        load_x_stage(x, ld_x, row0, nrows, kn * kKB, tid, xr[(s + S - 1) % S]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) load_w_frag(w1p, n_ut, ut0 + ct, kn, lane, wr[(s + S - 1) % S][ct]);
      }
      const uint16_t* xb = xs[kb & 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 xf[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          xf[rt] = *reinterpret_cast<const u32x4*>(xb + (rt * 32 + l32) * kXLd + 32 * g + 8 * j);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) acc[ct][rt] = mfma32(wr[s][ct][j], xf[rt], acc[ct][rt]);
      }
      if (S == 1) {  // no ring: load the next block now
        const int k1 = min(kb + 1, nkb - 1);
        load_x_stage(x, ld_x, row0, nrows, k1 * kKB, tid, xr[0]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) load_w_frag(w1p, n_ut, ut0 + ct, k1, lane, wr[0][ct]);
        store_x_stage(xs[(kb + 1) & 1], tid, xr[0]);
      } else {
        store_x_stage(xs[(kb + 1) & 1], tid, xr[(s + 1) % S]);
      }
      __syncthreads();
    }
  }

  // Epilogue: lane holds U^T[unit][row] for unit = unit_base + 32 ct + 8 (i/4) + 4 g + (i%4), row = 32 rt + l32.
  float part[2] = {0.f, 0.f};
  if (active) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int u0 = unit_base + 32 * ct + 8 * q4 + 4 * g;
        const f32x4 w2v = *reinterpret_cast<const f32x4*>(w2 + u0);
        f32x4 b1v = f32x4{0.f, 0.f, 0.f, 0.f};
        if (b1 != nullptr) b1v = *reinterpret_cast<const f32x4*>(b1 + u0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) part[rt] += gelu_erf(acc[ct][rt][4 * q4 + e] + b1v[e]) * w2v[e];
        }
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const float both = xor32_sum(part[rt]);  // both half-waves hold the same bits
    if (g == 0) red[wave][rt * 32 + l32] = both;
  }
  __syncthreads();
  if (tid < kRows) {
    const float r = ((red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid])) + b2;
    double sq = 0.0;
    if (tid < nrows) {
      scores[row0 + tid] = r;
      sq = (double)r * (double)r;
    }
    red2[tid] = sq;
  }
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int i = 0; i < kRows; ++i) s += red2[i];
    tile_sumsq[(int64_t)blockIdx.y * max_tiles + tile] = s;
  }
}

constexpr int kNormThreads = 256;
constexpr int kNormTokens = 1024;  // tokens per block

__global__ __launch_bounds__(kNormThreads) void gate_normalize_kernel(const tg_segment* __restrict__ segs,
                                                                     int max_tiles,
                                                                     const double* __restrict__ tile_sumsq,
                                                                     float rms_eps, float* __restrict__ scores) {
  __shared__ double red[kNormThreads];
  const tg_segment seg = segs[blockIdx.y];
  const int t0 = blockIdx.x * kNormTokens;
  if (t0 >= seg.seg_len) return;
  const int n_doc = seg.doc_end - seg.doc_begin;
  const int tid = threadIdx.x;
  float rho = 1.0f;
  const bool norm = rms_eps >= 0.0f && n_doc > 0;
  if (norm) {
    const int ntiles = (n_doc + kRows - 1) / kRows;
    const double* ts = tile_sumsq + (int64_t)blockIdx.y * max_tiles;
    double s = 0.0;
    for (int i = tid; i < ntiles; i += kNormThreads) s += ts[i];
    red[tid] = s;
    __syncthreads();
#pragma unroll
    for (int w = kNormThreads / 2; w > 0; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    const double ms = red[0] / (double)n_doc;
    rho = (float)sqrt(ms + (double)rms_eps);
  }
  for (int i = tid; i < kNormTokens; i += kNormThreads) {
    const int t = t0 + i;
    if (t >= seg.seg_len) break;
    const int64_t gi = (int64_t)seg.seg_start + t;
    float v = 0.0f;
    if (t >= seg.doc_begin && t < seg.doc_end) {
      v = scores[gi];
      if (norm) v = v / rho;
    }
    scores[gi] = v;
  }
}

}  // namespace

static size_t sumsq_bytes(const tg_plan_info& info) {
  const int64_t max_tiles = (info.max_doc_len + kRows - 1) / kRows;
  const int64_t n = (int64_t)info.n_seg * (max_tiles > 0 ? max_tiles : 1);
  return (size_t)(((n * (int64_t)sizeof(double)) + 255) / 256 * 256);
}

size_t gate_workspace_bytes(const tg_plan_info& info, int d, int h) {
  return sumsq_bytes(info) + (size_t)d * (size_t)h * 2;  // tile sums + W1 in fragment order
}

hipError_t launch_gate_score(const void* x, int64_t ld_x, int d, const void* w1, const float* b1, const float* w2,
                             float b2, int h, const tg_segment* segs, const tg_plan_info& info, float rms_eps,
                             float* scores, void* workspace, hipStream_t stream) {
  int max_tiles = (info.max_doc_len + kRows - 1) / kRows;
  if (max_tiles < 1) max_tiles = 1;
  double* ts = reinterpret_cast<double*>(workspace);
  u32x4* w1p = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(workspace) + sumsq_bytes(info));
  if (info.max_doc_len > 0) {
    const int64_t chunks = (int64_t)d * h / 8;
    hipLaunchKernelGGL(pack_w1_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint16_t*>(w1), d, h, w1p);
    dim3 grid(max_tiles, info.n_seg);
    const int nkb = d / kKB;
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
    const u32x4* wp = w1p;
#define TG_GATE_LAUNCH(NCT, S)                                                                                 \
  hipLaunchKernelGGL((gate_mlp_kernel<NCT, S>), grid, dim3(kThreads), 0, stream, xp, ld_x, d, wp, b1, w2, b2, h, \
                     segs, max_tiles, scores, ts)
    if (h <= 128) {
      if (nkb % 4 == 0) TG_GATE_LAUNCH(1, 4); else if (nkb % 2 == 0) TG_GATE_LAUNCH(1, 2); else TG_GATE_LAUNCH(1, 1);
    } else {
      if (nkb % 4 == 0) TG_GATE_LAUNCH(2, 4); else if (nkb % 2 == 0) TG_GATE_LAUNCH(2, 2); else TG_GATE_LAUNCH(2, 1);
    }
#undef TG_GATE_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (info.max_seg_len > 0) {
    dim3 grid((info.max_seg_len + kNormTokens - 1) / kNormTokens, info.n_seg);
    hipLaunchKernelGGL(gate_normalize_kernel, grid, dim3(kNormThreads), 0, stream, segs, max_tiles, ts, rms_eps,
                       scores);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace tg
