// Top-K select and kept-index emission (gfx950).
//
// Kept set S = top-K(document scores) ∪ (every non-document token)
// ("TokenGate 与 T2Quant ... 精读", sections 3.1 and 4.1).  Order among document
// tokens: higher score, then lower index.
//
// Scores become order-preserving 32-bit keys (score_key), so the K-th largest
// document key T is found exactly with a three-digit MSB radix select
// (11 + 11 + 10 bits).  Each pass is one launch over all prompts: every block
// histograms its 4096 keys in LDS and adds the non-empty bins to the prompt's
// global histogram with integer atomics (exact, so order does not matter);
// the last block to arrive (atomic ticket) scans the histogram from the top
// and fixes the next digit of T.  After the passes, n_gt = #{key > T} and
// need = K_eff - n_gt ties at T are kept, lowest indices first.  Emission is
// an index-ordered scan (block counts, then per-block offsets), so the output
// is ascending and identical on every run.
#include "common.h"

namespace tg {
namespace {

constexpr int kSelThreads = 256;
constexpr int kKeysPerThread = 16;
constexpr int kChunk = kSelThreads * kKeysPerThread;  // keys per block
constexpr int kBins = 2048;

struct SelState {
  uint32_t hist[3][kBins];
  uint32_t ticket[3];
  uint32_t prefix;     // digits of T fixed so far
  uint32_t remaining;  // keys still to take inside the current prefix bin
  uint32_t resolved;   // 1: T and need are final (set by init for K_eff in {0, n_doc})
  uint32_t thresh;     // T
  uint32_t need;       // ties at T to keep
  uint32_t pad[56];    // keep the struct a multiple of 256 bytes
};
static_assert(sizeof(SelState) % 256 == 0, "SelState alignment");

struct Counts {
  uint32_t def;  // kept for sure (non-document, or document key > T)
  uint32_t tie;  // document key == T
};

__device__ __forceinline__ int pass_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t pass_bins(int p) { return p == 2 ? 1024u : 2048u; }
__device__ __forceinline__ uint32_t prefix_mask(int p) {
  return p == 0 ? 0u : (p == 1 ? 0xffe00000u : 0xfffffc00u);
}

__global__ __launch_bounds__(kSelThreads) void sel_init_kernel(const tg_segment* __restrict__ segs,
                                                               SelState* __restrict__ st) {
  const tg_segment seg = segs[blockIdx.x];
  SelState* s = st + blockIdx.x;
  uint32_t* w = reinterpret_cast<uint32_t*>(s);
  for (int i = threadIdx.x; i < (int)(sizeof(SelState) / 4); i += kSelThreads) w[i] = 0u;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int n_doc = seg.doc_end - seg.doc_begin;
    if (seg.k_eff <= 0) {  // keep no document: nothing compares above this key
      s->resolved = 1u;
      s->thresh = 0xffffffffu;
      s->need = 0u;
    } else if (seg.k_eff >= n_doc) {  // keep every document, NaNs included
      s->resolved = 1u;
      s->thresh = 0u;
      s->need = 0xffffffffu;
    } else {
      s->remaining = (uint32_t)seg.k_eff;
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void sel_pass_kernel(const float* __restrict__ scores,
                                                               const tg_segment* __restrict__ segs,
                                                               SelState* __restrict__ st, int pass) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scan[kSelThreads];
  __shared__ int is_last;
  const tg_segment seg = segs[blockIdx.y];
  SelState* s = st + blockIdx.y;
  if (s->resolved) return;
  const int n_doc = seg.doc_end - seg.doc_begin;
  const int nblk = (n_doc + kChunk - 1) / kChunk;
  if ((int)blockIdx.x >= nblk) return;
  const int tid = threadIdx.x;
  const uint32_t bins = pass_bins(pass);
  const int shift = pass_shift(pass);
  const uint32_t mask = prefix_mask(pass);
  const uint32_t prefix = s->prefix;

  for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0u;
  __syncthreads();
  const float* base = scores + seg.seg_start + seg.doc_begin;
  const int k0 = blockIdx.x * kChunk;
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    const int t = k0 + i * kSelThreads + tid;
    if (t < n_doc) {
      const uint32_t key = score_key(base[t]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (bins - 1u)], 1u);
    }
  }
  __syncthreads();
  for (uint32_t b = tid; b < bins; b += kSelThreads) {
    const uint32_t c = hist[b];
    if (c) atomicAdd(&s->hist[pass][b], c);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = (atomicAdd(&s->ticket[pass], 1u) == (uint32_t)(nblk - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // Last block: counts per bin from the top; find the bin holding the remaining-th key.
  const uint32_t per = bins / kSelThreads;  // 8 or 4 bins per thread, thread 0 owns the top bins
  uint32_t local[8];
  uint32_t sum = 0u;
  for (uint32_t j = 0; j < per; ++j) {
    const uint32_t b = bins - 1u - (tid * per + j);
    local[j] = __hip_atomic_load(&s->hist[pass][b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sum += local[j];
  }
  scan[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {  // inclusive scan, top bins first
    const uint32_t v = tid >= off ? scan[tid - off] : 0u;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const uint32_t remaining = s->remaining;
  const uint32_t before = scan[tid] - sum;
  if (before < remaining && remaining <= scan[tid]) {
    uint32_t acc = before;
    for (uint32_t j = 0; j < per; ++j) {
      if (acc + local[j] >= remaining) {
        const uint32_t b = bins - 1u - (tid * per + j);
        const uint32_t new_prefix = prefix | (b << shift);
        const uint32_t new_rem = remaining - acc;
        s->prefix = new_prefix;
        s->remaining = new_rem;
        if (pass == 2) {
          s->thresh = new_prefix;
          s->need = new_rem;
          s->resolved = 1u;
        }
        break;
      }
      acc += local[j];
    }
  }
}

constexpr int kEmitThreads = 256;
constexpr int kEmitPerThread = 16;
constexpr int kEmitChunk = kEmitThreads * kEmitPerThread;

__device__ __forceinline__ void classify(const float* __restrict__ scores, const tg_segment& seg, int t,
                                         uint32_t thresh, uint32_t& def, uint32_t& tie) {
  def = 0u;
  tie = 0u;
  if (t >= seg.seg_len) return;
  if (t < seg.doc_begin || t >= seg.doc_end) {
    def = 1u;
    return;
  }
  const uint32_t key = score_key(scores[seg.seg_start + t]);
  if (key > thresh)
    def = 1u;
  else if (key == thresh)
    tie = 1u;
}

__global__ __launch_bounds__(kEmitThreads) void sel_count_kernel(const float* __restrict__ scores,
                                                                 const tg_segment* __restrict__ segs,
                                                                 const SelState* __restrict__ st,
                                                                 Counts* __restrict__ counts, int max_eblk) {
  __shared__ uint32_t rd[kEmitThreads], rt[kEmitThreads];
  const tg_segment seg = segs[blockIdx.y];
  const int t0 = blockIdx.x * kEmitChunk;
  if (t0 >= seg.seg_len) return;
  const uint32_t thresh = st[blockIdx.y].thresh;
  const int tid = threadIdx.x;
  uint32_t d = 0u, tt = 0u;
  for (int i = 0; i < kEmitPerThread; ++i) {
    uint32_t a, b;
    classify(scores, seg, t0 + i * kEmitThreads + tid, thresh, a, b);
    d += a;
    tt += b;
  }
  rd[tid] = d;
  rt[tid] = tt;
  __syncthreads();
  for (int w = kEmitThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      rd[tid] += rd[tid + w];
      rt[tid] += rt[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) counts[(int64_t)blockIdx.y * max_eblk + blockIdx.x] = Counts{rd[0], rt[0]};
}

__global__ __launch_bounds__(kEmitThreads) void sel_write_kernel(const float* __restrict__ scores,
                                                                 const tg_segment* __restrict__ segs,
                                                                 const SelState* __restrict__ st,
                                                                 const Counts* __restrict__ counts, int max_eblk,
                                                                 int32_t* __restrict__ kept_idx) {
  __shared__ uint32_t sd[kEmitThreads], stt[kEmitThreads];
  __shared__ uint32_t base_def, base_tie;
  const tg_segment seg = segs[blockIdx.y];
  const int t0 = blockIdx.x * kEmitChunk;
  if (t0 >= seg.seg_len) return;
  const uint32_t thresh = st[blockIdx.y].thresh;
  const uint32_t need = st[blockIdx.y].need;
  const int tid = threadIdx.x;

  // counts of the blocks before this one
  uint32_t pd = 0u, pt = 0u;
  const Counts* cs = counts + (int64_t)blockIdx.y * max_eblk;
  for (int b = tid; b < (int)blockIdx.x; b += kEmitThreads) {
    pd += cs[b].def;
    pt += cs[b].tie;
  }
  sd[tid] = pd;
  stt[tid] = pt;
  __syncthreads();
  for (int w = kEmitThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      sd[tid] += sd[tid + w];
      stt[tid] += stt[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    base_def = sd[0];
    base_tie = stt[0];
  }
  __syncthreads();

  // this thread owns 16 consecutive tokens
  const int tb = t0 + tid * kEmitPerThread;
  uint32_t fd[kEmitPerThread], ft[kEmitPerThread];
  uint32_t cd = 0u, ct = 0u;
#pragma unroll
  for (int i = 0; i < kEmitPerThread; ++i) {
    classify(scores, seg, tb + i, thresh, fd[i], ft[i]);
    cd += fd[i];
    ct += ft[i];
  }
  sd[tid] = cd;
  stt[tid] = ct;
  __syncthreads();
  for (int off = 1; off < kEmitThreads; off <<= 1) {  // inclusive scan over threads
    const uint32_t vd = tid >= off ? sd[tid - off] : 0u;
    const uint32_t vt = tid >= off ? stt[tid - off] : 0u;
    __syncthreads();
    sd[tid] += vd;
    stt[tid] += vt;
    __syncthreads();
  }
  uint32_t rdf = base_def + sd[tid] - cd;  // definite keeps before this thread's first token
  uint32_t rtie = base_tie + stt[tid] - ct;
  int32_t* out = kept_idx + seg.kept_start;
#pragma unroll
  for (int i = 0; i < kEmitPerThread; ++i) {
    const uint32_t taken = rtie < need ? rtie : need;
    const bool keep = fd[i] || (ft[i] && rtie < need);
    if (keep && rdf + taken < (uint32_t)seg.kept_len) out[rdf + taken] = seg.seg_start + tb + i;
    rdf += fd[i];
    rtie += ft[i];
  }
}

int max_emit_blocks(const tg_plan_info& info) {
  const int b = (info.max_seg_len + kEmitChunk - 1) / kEmitChunk;
  return b > 0 ? b : 1;
}

}  // namespace

size_t select_workspace_bytes(const tg_plan_info& info) {
  const size_t st = sizeof(SelState) * (size_t)info.n_seg;
  const size_t cn = sizeof(Counts) * (size_t)info.n_seg * (size_t)max_emit_blocks(info);
  return st + (cn + 255) / 256 * 256;
}

hipError_t launch_select_topk(const float* scores, const tg_segment* segs, const tg_plan_info& info,
                              int32_t* kept_idx, void* workspace, hipStream_t stream) {
  SelState* st = reinterpret_cast<SelState*>(workspace);
  Counts* counts = reinterpret_cast<Counts*>(reinterpret_cast<char*>(workspace) + sizeof(SelState) * info.n_seg);
  const int max_eblk = max_emit_blocks(info);
  hipLaunchKernelGGL(sel_init_kernel, dim3(info.n_seg), dim3(kSelThreads), 0, stream, segs, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (info.max_doc_len > 0) {
    const int nblk = (info.max_doc_len + kChunk - 1) / kChunk;
    for (int p = 0; p < 3; ++p) {
      hipLaunchKernelGGL(sel_pass_kernel, dim3(nblk, info.n_seg), dim3(kSelThreads), 0, stream, scores, segs, st,
                         p);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (info.max_seg_len > 0) {
    dim3 grid(max_eblk, info.n_seg);
    hipLaunchKernelGGL(sel_count_kernel, grid, dim3(kEmitThreads), 0, stream, scores, segs, st, counts, max_eblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sel_write_kernel, grid, dim3(kEmitThreads), 0, stream, scores, segs, st, counts, max_eblk,
                       kept_idx);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace tg
