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

__device__ __forceinline__ float gelu_erf(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }

// Loads this thread's share of an X stage: row = tid / 4, 16 bf16 at column (tid % 4) * 16.
__device__ __forceinline__ void load_x_stage(const uint16_t* __restrict__ x, int64_t ld_x, int64_t row0, int nrows,
                                             int k0, int tid, u32x4& p0, u32x4& p1) {
  const int r = tid >> 2;
  const int c = (tid & 3) * 16;
  if (r < nrows) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (row0 + r) * ld_x + k0 + c);
    p0 = __builtin_nontemporal_load(src);
    p1 = __builtin_nontemporal_load(src + 1);
  } else {
    p0 = u32x4{0u, 0u, 0u, 0u};
    p1 = p0;
  }
}

__device__ __forceinline__ void store_x_stage(uint16_t* lds, int tid, const u32x4& p0, const u32x4& p1) {
  const int r = tid >> 2;
  const int c = (tid & 3) * 16;
  u32x4* dst = reinterpret_cast<u32x4*>(lds + r * kXLd + c);
  dst[0] = p0;
  dst[1] = p1;
}

// W1 fragment of one 32-unit column tile for one 64-wide k block: lane holds
// 32 consecutive k (64 bytes) of hidden unit `unit`: k0 + 32 g .. k0 + 32 g + 31.
// MFMA step j consumes k0 + 32 g + 8 j .. + 7, so A and B use the same
// (permuted) k order inside the block.
__device__ __forceinline__ void load_w_frag(const uint16_t* __restrict__ w1, int d, int unit, int k0, int g,
                                            u32x4 (&w)[4]) {
  const u32x4* src = reinterpret_cast<const u32x4*>(w1 + (int64_t)unit * d + k0 + 32 * g);
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = src[j];
}

template <int NCT>  // 32-unit column tiles per wave (1 or 2)
__global__ __launch_bounds__(kThreads) void gate_mlp_kernel(const uint16_t* __restrict__ x, int64_t ld_x, int d,
                                                            const uint16_t* __restrict__ w1,
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
  const bool active = unit_base < h;  // waves beyond h only help stage X

  f32x16 acc[NCT][2];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) acc[ct][rt] = f32x16{};

  const uint16_t* w1u = reinterpret_cast<const uint16_t*>(w1);
  const int nkb = d / kKB;

  u32x4 xp0, xp1;
  load_x_stage(x, ld_x, row0, nrows, 0, tid, xp0, xp1);
  store_x_stage(xs[0], tid, xp0, xp1);
  u32x4 wc[NCT][4];
  if (active) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) load_w_frag(w1u, d, unit_base + 32 * ct + l32, 0, g, wc[ct]);
  }
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < nkb;
    u32x4 wn[NCT][4];
    if (more) {
      load_x_stage(x, ld_x, row0, nrows, (kb + 1) * kKB, tid, xp0, xp1);
      if (active) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) load_w_frag(w1u, d, unit_base + 32 * ct + l32, (kb + 1) * kKB, g, wn[ct]);
      }
    }
    if (active) {
      const uint16_t* xb = xs[buf];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 xf[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          xf[rt] = *reinterpret_cast<const u32x4*>(xb + (rt * 32 + l32) * kXLd + 32 * g + 8 * j);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) acc[ct][rt] = mfma32(wc[ct][j], xf[rt], acc[ct][rt]);
      }
    }
    if (more) {
      store_x_stage(xs[buf ^ 1], tid, xp0, xp1);
      if (active) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int j = 0; j < 4; ++j) wc[ct][j] = wn[ct][j];
      }
    }
    __syncthreads();
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
    const float other = __shfl_xor(part[rt], 32);
    const float both = part[rt] + other;  // commutative: both half-waves hold the same bits
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

size_t gate_workspace_bytes(const tg_plan_info& info) {
  const int64_t max_tiles = (info.max_doc_len + kRows - 1) / kRows;
  const int64_t n = (int64_t)info.n_seg * (max_tiles > 0 ? max_tiles : 1);
  return (size_t)(((n * (int64_t)sizeof(double)) + 255) / 256 * 256);
}

hipError_t launch_gate_score(const void* x, int64_t ld_x, int d, const void* w1, const float* b1, const float* w2,
                             float b2, int h, const tg_segment* segs, const tg_plan_info& info, float rms_eps,
                             float* scores, void* workspace, hipStream_t stream) {
  int max_tiles = (info.max_doc_len + kRows - 1) / kRows;
  if (max_tiles < 1) max_tiles = 1;
  double* ts = reinterpret_cast<double*>(workspace);
  if (info.max_doc_len > 0) {
    dim3 grid(max_tiles, info.n_seg);
    if (h <= 128) {
      hipLaunchKernelGGL(gate_mlp_kernel<1>, grid, dim3(kThreads), 0, stream,
                         reinterpret_cast<const uint16_t*>(x), ld_x, d, reinterpret_cast<const uint16_t*>(w1), b1,
                         w2, b2, h, segs, max_tiles, scores, ts);
    } else {
      hipLaunchKernelGGL(gate_mlp_kernel<2>, grid, dim3(kThreads), 0, stream,
                         reinterpret_cast<const uint16_t*>(x), ld_x, d, reinterpret_cast<const uint16_t*>(w1), b1,
                         w2, b2, h, segs, max_tiles, scores, ts);
    }
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
