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
#include <atomic>
#include <mutex>

#include "common.h"

namespace tg {
namespace {

constexpr int kRows = 64;      // smallest tile height (document rows per workgroup)
constexpr int kThreads = 256;  // 4 waves

// GELU(u) = u Phi(u) = max(u, 0) - |u| erfc(|u| / sqrt 2) / 2, with erfc from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (|error| <= 1.5e-7):
//   erfc(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),  t = 1 / (1 + p z),  z >= 0.
// The halving is folded into the a_i (exactly: a power of two), 1 / sqrt 2
// into p, and exp(-z^2) is exp2(-u^2 log2(e) / 2): 13 vector operations and
// two transcendentals per unit.
__device__ __forceinline__ float gelu_erf(float u) {
  const float au = fabsf(u);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f * 0.70710678118654752f, au, 1.0f));
  float p = __builtin_fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
  p = __builtin_fmaf(p, t, 0.5f * 1.421413741f);
  p = __builtin_fmaf(p, t, 0.5f * -0.284496736f);
  p = __builtin_fmaf(p, t, 0.5f * 0.254829592f);
  p *= t;
  const float e = __builtin_amdgcn_exp2f(u * u * -0.72134752044448170f);
  return __builtin_fmaf(-au, p * e, fmaxf(u, 0.0f));
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

// One workgroup per (k block kb, 32-unit tile ut): the 32 x 64 block of W1 is
// read row by row (8 lanes x 16 bytes per 128-byte row slice), staged in LDS
// and written out in fragment order as 4 contiguous KiB.
__global__ __launch_bounds__(256) void pack_w1_kernel(const uint16_t* __restrict__ w1, int d, int h,
                                                      u32x4* __restrict__ w1p) {
  __shared__ u32x4 blk[32][8 + 1];  // [unit][16-byte k chunk], padded
  const int n_ut = h / 32;
  const int ut = blockIdx.x % n_ut;
  const int kb = blockIdx.x / n_ut;
  const int tid = threadIdx.x;
  {
    const int u = tid >> 3, c = tid & 7;  // unit row, 16-byte chunk of its 64 k values
    blk[u][c] = *reinterpret_cast<const u32x4*>(w1 + (int64_t)(32 * ut + u) * d + 64 * kb + 8 * c);
  }
  __syncthreads();
  // fragment chunk i = j * 64 + lane holds W1[32 ut + lane % 32][64 kb + 32 (lane / 32) + 8 j .. + 7]
  const int lane = tid & 63, j = tid >> 6;
  w1p[((int64_t)(kb * n_ut + ut) * 4 + j) * 64 + lane] = blk[lane & 31][4 * (lane >> 5) + j];
}

// NCT: 32-unit column tiles per wave (1 or 2).  RT: 32-row tiles per workgroup
// (BM = 32 RT document rows); every wave covers all BM rows for its units, so
// a W1 fragment feeds RT MFMAs.  XB: 64-wide k blocks per X stage.
//
// X goes through LDS in stages of BM rows x 64 XB columns.  Each wave load
// reads a contiguous 16 x (64 XB / 8)-byte slice of one row (1 KiB at XB = 8):
// long row bursts instead of 128-byte pieces scattered over thousands of rows
// is what lets the HBM stream reach bandwidth.  The next stage is loaded into
// registers in two halves during the current one (issued at blocks 0 and
// XB/2, written to the other LDS buffer half a stage later), so there is one
// barrier per stage.  W1 fragments come straight from the fragment-packed copy
// through a register ring S blocks deep.  d is a multiple of 64 XB.
template <int NCT, int S, int RT, int XB>
__global__ __launch_bounds__(kThreads) void gate_mlp_kernel(const uint16_t* __restrict__ x, int64_t ld_x, int d,
                                                            const u32x4* __restrict__ w1p,
                                                            const float* __restrict__ b1,
                                                            const float* __restrict__ w2, float b2, int h,
                                                            SegTable segs, int max_tiles,
                                                            float* __restrict__ scores,
                                                            double* __restrict__ tile_sumsq) {
  constexpr int BM = 32 * RT;
  constexpr int KX = 64 * XB;               // k per X stage
  constexpr int LD = KX + 8;                // LDS row stride (bf16): 16-byte pad keeps fragment reads conflict free
  constexpr int UPR = KX / 8;               // 16-byte units per row slice
  constexpr int HALF = BM * UPR / 2 / kThreads;  // 16-byte loads per thread per half stage
  static_assert((XB % 2 == 0 || XB == 1) && XB % S == 0, "stage shape");
  static_assert(HALF >= 1 && (BM * UPR / 2) % kThreads == 0, "stage split");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * LD];
  __shared__ float red[4][BM];
  __shared__ __attribute__((aligned(16))) float w2s[4 * 32 * NCT], b1s[4 * 32 * NCT];  // read in the epilogue
  __shared__ double red2[BM];

  const tg_segment seg = segs.at_uniform(blockIdx.y);
  const int n_doc = seg.doc_end - seg.doc_begin;
  const int tile = blockIdx.x;
  if (tile * BM >= n_doc) return;  // uniform across the workgroup
  const int64_t row0 = (int64_t)seg.seg_start + seg.doc_begin + (int64_t)tile * BM;
  const int nrows = min(BM, n_doc - tile * BM);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int unit_base = wave * 32 * NCT;
  const bool active = unit_base < h;  // waves past h compute on a valid slice and drop the result
  const int ut0 = active ? unit_base / 32 : 0;
  const int n_ut = h / 32;

  // X half-stage h (0: rows [0, BM/2), 1: rows [BM/2, BM)): unit u = i kThreads + tid of the half
  auto x_src = [&](int hf, int i, int k0) -> const u32x4* {
    const int u = i * kThreads + tid;
    const int r = min(hf * (BM / 2) + u / UPR, nrows - 1);  // rows past the tile re-read its last row
    return reinterpret_cast<const u32x4*>(x + (row0 + r) * ld_x + k0 + (u % UPR) * 8);
  };
  auto x_dst = [&](uint16_t* buf, int hf, int i) -> u32x4* {
    const int u = i * kThreads + tid;
    return reinterpret_cast<u32x4*>(buf + (hf * (BM / 2) + u / UPR) * LD + (u % UPR) * 8);
  };

  f32x16 acc[NCT][RT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[ct][rt] = f32x16{};

  const int nkb = d / 64;
  const int nst = nkb / XB;
  u32x4 wr[S][NCT][4];  // W1 ring
  u32x4 xr[HALF];       // X half stage in flight

  // prologue: X stage 0 into LDS, W1 blocks 0 .. S-2 in flight, w2 and b1 into LDS
  for (int u = threadIdx.x; u < 4 * 32 * NCT; u += blockDim.x) {
    w2s[u] = u < h ? w2[u] : 0.0f;
    b1s[u] = u < h && b1 != nullptr ? b1[u] : 0.0f;
  }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int i = 0; i < HALF; ++i) xr[i] = __builtin_nontemporal_load(x_src(hf, i, 0));
#pragma unroll
    for (int i = 0; i < HALF; ++i) *x_dst(xs[0], hf, i) = xr[i];
  }
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) load_w_frag(w1p, n_ut, ut0 + ct, s, lane, wr[s][ct]);
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const uint16_t* xb = xs[st & 1];
    uint16_t* xn = xs[(st + 1) & 1];
    const bool next = st + 1 < nst;
    const int kx_next = (st + 1) * KX;
    // X fragments of the current block and the next one: block c + 1's LDS reads
    // go out during block c's MFMAs (within a stage; the next stage's buffer is
    // complete only after the stage barrier)
    u32x4 xfb[2][4][RT];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        xfb[0][j][rt] = *reinterpret_cast<const u32x4*>(xb + (rt * 32 + l32) * LD + 32 * g + 8 * j);
#pragma unroll
    for (int c = 0; c < XB; ++c) {
      const int kb = st * XB + c;
      if (next && c == 0) {
#pragma unroll
        for (int i = 0; i < HALF; ++i) xr[i] = __builtin_nontemporal_load(x_src(0, i, kx_next));
      }
      if (next && c == XB / 2) {
#pragma unroll
        for (int i = 0; i < HALF; ++i) *x_dst(xn, 0, i) = xr[i];
#pragma unroll
        for (int i = 0; i < HALF; ++i) xr[i] = __builtin_nontemporal_load(x_src(1, i, kx_next));
      }
      {  // W1 block kb + S - 1 starts loading now (clamped: the tail re-reads the last block)
        const int kn = min(kb + S - 1, nkb - 1);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) load_w_frag(w1p, n_ut, ut0 + ct, kn, lane, wr[(c + S - 1) % S][ct]);
      }
      if (c + 1 < XB) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            xfb[(c + 1) & 1][j][rt] =
                *reinterpret_cast<const u32x4*>(xb + (rt * 32 + l32) * LD + 64 * (c + 1) + 32 * g + 8 * j);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) acc[ct][rt] = mfma32(wr[c % S][ct][j], xfb[c & 1][j][rt], acc[ct][rt]);
      if (c + 1 < XB) {  // the next block's reads spread over this block's MFMAs
#pragma unroll
        for (int i = 0; i < 4 * RT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, NCT, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }
    if (next) {
#pragma unroll
      for (int i = 0; i < HALF; ++i) *x_dst(xn, 1, i) = xr[i];
    }
    __syncthreads();
  }

  // Epilogue: lane holds U^T[unit][row] for unit = unit_base + 32 ct + 8 (i/4) + 4 g + (i%4), row = 32 rt + l32.
  float part[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) part[rt] = 0.f;
  if (active) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int u0 = unit_base + 32 * ct + 8 * q4 + 4 * g;
        const f32x4 w2v = *reinterpret_cast<const f32x4*>(&w2s[u0]);
        const f32x4 b1v = *reinterpret_cast<const f32x4*>(&b1s[u0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) part[rt] += gelu_erf(acc[ct][rt][4 * q4 + e] + b1v[e]) * w2v[e];
        }
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float both = xor32_sum(part[rt]);  // both half-waves hold the same bits
    if (g == 0) red[wave][rt * 32 + l32] = both;
  }
  __syncthreads();
  for (int i = tid; i < BM; i += kThreads) {
    const float r = ((red[0][i] + red[1][i]) + (red[2][i] + red[3][i])) + b2;
    double sq = 0.0;
    if (i < nrows) {
      scores[row0 + i] = r;
      sq = (double)r * (double)r;
    }
    red2[i] = sq;
  }
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int i = 0; i < BM; ++i) s += red2[i];
    tile_sumsq[(int64_t)blockIdx.y * max_tiles + tile] = s;
  }
}

constexpr int kNormThreads = 256;  // one token per thread

// Per-prompt RMS of the document scores from the per-tile sums of squares,
// then every token's score divided by it (0 outside the document span).  The
// fp64 sum has a fixed order: thread i sums tiles i, i + 256, ..., then the
// 256 partial sums are added pairwise, halving the count each step (the last
// six steps inside one wave by lane shifts).  Each thread's score load is
// issued before the reduction, so its latency overlaps it.
__global__ __launch_bounds__(kNormThreads) void gate_normalize_kernel(SegTable segs,
                                                                     int max_tiles, int rows_per_tile,
                                                                     const double* __restrict__ tile_sumsq,
                                                                     float rms_eps, float* __restrict__ scores) {
  __shared__ double red128[128];
  __shared__ double red64[64];
  __shared__ float rho_s;
  const tg_segment seg = segs.at_uniform(blockIdx.y);
  const int t0 = blockIdx.x * kNormThreads;
  if (t0 >= seg.seg_len) return;  // uniform
  const int n_doc = seg.doc_end - seg.doc_begin;
  const int tid = threadIdx.x;
  const int t = t0 + tid;
  const int64_t gi = (int64_t)seg.seg_start + t;
  const bool mine = t < seg.seg_len;
  const bool doc = mine && t >= seg.doc_begin && t < seg.doc_end;
  const float v = doc ? scores[gi] : 0.0f;
  float rho = 1.0f;
  const bool norm = rms_eps >= 0.0f && n_doc > 0;
  if (norm) {
    const int ntiles = (n_doc + rows_per_tile - 1) / rows_per_tile;
    const double* ts = tile_sumsq + (int64_t)blockIdx.y * max_tiles;
    double s = 0.0;
    for (int i = tid; i < ntiles; i += kNormThreads) s += ts[i];
    if (tid >= 128) red128[tid - 128] = s;
    __syncthreads();
    if (tid < 128) {
      s += red128[tid];
      if (tid >= 64) red64[tid - 64] = s;
    }
    __syncthreads();
    if (tid < 64) {
      s += red64[tid];
#pragma unroll
      for (int w = 32; w > 0; w >>= 1) s += __shfl_down(s, w);
      if (tid == 0) rho_s = (float)sqrt(s / (double)n_doc + (double)rms_eps);
    }
    __syncthreads();
    rho = rho_s;
  }
  if (mine) scores[gi] = norm ? v / rho : v;
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

template <int NCT, int RT, int XB, int S>
static void launch_mlp(dim3 grid, hipStream_t stream, const uint16_t* xp, int64_t ld_x, int d, const u32x4* wp,
                       const float* b1, const float* w2, float b2, int h, SegTable segs, int max_tiles,
                       float* scores, double* ts) {
  hipLaunchKernelGGL((gate_mlp_kernel<NCT, S, RT, XB>), grid, dim3(kThreads), 0, stream, xp, ld_x, d, wp, b1, w2, b2,
                     h, segs, max_tiles, scores, ts);
}

template <int NCT>
static void launch_mlp_d(dim3 grid, hipStream_t stream, const uint16_t* xp, int64_t ld_x, int d, const u32x4* wp,
                         const float* b1, const float* w2, float b2, int h, SegTable segs, int max_tiles,
                         float* scores, double* ts) {
  // X stage of 256 columns (512-byte row bursts) when d allows; measured best among 128-1024-byte bursts
  if (d % 256 == 0)
    launch_mlp<NCT, 2, 4, 4>(grid, stream, xp, ld_x, d, wp, b1, w2, b2, h, segs, max_tiles, scores, ts);
  else if (d % 128 == 0)
    launch_mlp<NCT, 2, 2, 2>(grid, stream, xp, ld_x, d, wp, b1, w2, b2, h, segs, max_tiles, scores, ts);
  else
    launch_mlp<NCT, 2, 1, 1>(grid, stream, xp, ld_x, d, wp, b1, w2, b2, h, segs, max_tiles, scores, ts);
}

hipError_t launch_gate_pack_w1(const void* w1, int d, int h, void* w1_packed, hipStream_t stream) {
  hipLaunchKernelGGL(pack_w1_kernel, dim3((unsigned)((d / 64) * (h / 32))), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(w1), d, h, reinterpret_cast<u32x4*>(w1_packed));
  return hipGetLastError();
}

// Scratch of the entry point that allocates nothing (tg_gate_score_prepacked_noalloc): the per-tile sums of
// squares live in this fixed array, one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in): the device address of each GPU's copy is looked
// up once, with that GPU current, and kept.
constexpr size_t kGateScratchBytes = (size_t)512 << 10;
static __device__ __align__(256) double scratch[kGateScratchBytes / sizeof(double)];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

size_t gate_scratch_bytes() { return kGateScratchBytes; }
size_t gate_sumsq_bytes(const tg_plan_info& info) { return sumsq_bytes(info); }

hipError_t gate_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy (the device is current)
      if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_gate_score(const void* x, int64_t ld_x, int d, const void* w1, bool w1_prepacked, const float* b1,
                             const float* w2, float b2, int h, const tg_segment* segs_in, const tg_plan_info& info,
                             float rms_eps, float* scores, void* workspace, hipStream_t stream) {
  const SegTable segs = seg_table(segs_in, info);
  int max_tiles = (info.max_doc_len + kRows - 1) / kRows;  // at the smallest tile height: an upper bound
  if (max_tiles < 1) max_tiles = 1;
  double* ts = reinterpret_cast<double*>(workspace);
  const u32x4* w1p = w1_prepacked
                         ? reinterpret_cast<const u32x4*>(w1)
                         : reinterpret_cast<const u32x4*>(reinterpret_cast<char*>(workspace) + sumsq_bytes(info));
  if (info.max_doc_len > 0) {
    if (!w1_prepacked) {
      const hipError_t e = launch_gate_pack_w1(w1, d, h, const_cast<u32x4*>(w1p), stream);
      if (e != hipSuccess) return e;
    }
    dim3 grid(max_tiles, info.n_seg);
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
    if (h <= 128)
      launch_mlp_d<1>(grid, stream, xp, ld_x, d, w1p, b1, w2, b2, h, segs, max_tiles, scores, ts);
    else
      launch_mlp_d<2>(grid, stream, xp, ld_x, d, w1p, b1, w2, b2, h, segs, max_tiles, scores, ts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (info.max_seg_len > 0) {
    dim3 grid((info.max_seg_len + kNormThreads - 1) / kNormThreads, info.n_seg);
    hipLaunchKernelGGL(gate_normalize_kernel, grid, dim3(kNormThreads), 0, stream, segs, max_tiles, kRows, ts, rms_eps,
                       scores);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace tg
