// Row gather of the kept rows (gfx950).
//
// Pruned tokens never reach the layers above the gate and get no KV entries
// there ("TokenGate 与 T2Quant ... 精读", section 4.1), so the kept rows of the
// hidden states, Q, K, V and the scores are copied, in original order, into
// dense arrays.  One launch moves every tensor: the grid is split between the
// tensors in proportion to their bytes, every thread moves 4 units (16, 4 or
// 1 bytes) and issues all its loads before its stores.  Pure data movement,
// bound by HBM bandwidth.
#include "common.h"

namespace tg {
namespace {

constexpr int kThreads = 256;
constexpr int kUnitsPerThread = 4;
constexpr int kUnitsPerBlock = kThreads * kUnitsPerThread;

struct CompactArgs {
  CompactDesc d;
  int64_t blk_start[TG_COMPACT_MAX_TENSORS + 1];
  int32_t unit_bytes[TG_COMPACT_MAX_TENSORS];
  int32_t upr_log2[TG_COMPACT_MAX_TENSORS];  // units per row, log2, or -1 when not a power of two
  int64_t upr[TG_COMPACT_MAX_TENSORS];
};

template <typename U>
__device__ __forceinline__ void copy_units(const int32_t* __restrict__ kept_idx, int64_t n_kept, int64_t n_src,
                                           const char* src,
                                           char* dst, int64_t src_stride, int64_t dst_stride, int64_t upr,
                                           int upr_log2, int64_t u0) {
  const int64_t total = n_kept * upr;
  U v[kUnitsPerThread];
  int64_t doff[kUnitsPerThread];
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i) {
    const int64_t u = u0 + (int64_t)i * kThreads;
    doff[i] = -1;
    if (u < total) {
      int64_t row, col;
      if (upr_log2 >= 0) {
        row = u >> upr_log2;
        col = u & (upr - 1);
      } else {
        row = u / upr;
        col = u - row * upr;
      }
      const int64_t srow = kept_idx[row];
      if (srow >= 0 && srow < n_src) {  // an index outside the source is skipped, never read
        v[i] = *reinterpret_cast<const U*>(src + srow * src_stride + col * (int64_t)sizeof(U));
        doff[i] = row * dst_stride + col * (int64_t)sizeof(U);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i)
    if (doff[i] >= 0) *reinterpret_cast<U*>(dst + doff[i]) = v[i];
}

__global__ __launch_bounds__(kThreads) void compact_kernel(const int32_t* __restrict__ kept_idx, int64_t n_kept,
                                                           int64_t n_src, CompactArgs a) {
  const int64_t b = blockIdx.x;
  int t = 0;
  while (t + 1 < a.d.n && b >= a.blk_start[t + 1]) ++t;
  const int64_t u0 = (b - a.blk_start[t]) * kUnitsPerBlock + threadIdx.x;
  switch (a.unit_bytes[t]) {
    case 16:
      copy_units<u32x4>(kept_idx, n_kept, n_src, a.d.src[t], a.d.dst[t], a.d.src_stride[t], a.d.dst_stride[t], a.upr[t],
                        a.upr_log2[t], u0);
      break;
    case 4:
      copy_units<uint32_t>(kept_idx, n_kept, n_src, a.d.src[t], a.d.dst[t], a.d.src_stride[t], a.d.dst_stride[t],
                           a.upr[t], a.upr_log2[t], u0);
      break;
    default:
      copy_units<uint8_t>(kept_idx, n_kept, n_src, a.d.src[t], a.d.dst[t], a.d.src_stride[t], a.d.dst_stride[t], a.upr[t],
                          a.upr_log2[t], u0);
      break;
  }
}

int unit_for(const char* s, const char* d, int64_t rb, int64_t ss, int64_t ds) {
  const uint64_t all = (uint64_t)(uintptr_t)s | (uint64_t)(uintptr_t)d | (uint64_t)rb | (uint64_t)ss | (uint64_t)ds;
  if ((all & 15u) == 0) return 16;
  if ((all & 3u) == 0) return 4;
  return 1;
}

}  // namespace

hipError_t launch_compact(const int32_t* kept_idx, int64_t n_kept, int64_t n_src, const CompactDesc& desc,
                          hipStream_t stream) {
  if (n_kept == 0) return hipSuccess;
  CompactArgs a{};
  a.d = desc;
  int64_t blocks = 0;
  for (int t = 0; t < desc.n; ++t) {
    const int ub = unit_for(desc.src[t], desc.dst[t], desc.row_bytes[t], desc.src_stride[t], desc.dst_stride[t]);
    a.unit_bytes[t] = ub;
    const int64_t upr = desc.row_bytes[t] / ub;
    a.upr[t] = upr;
    a.upr_log2[t] = -1;
    if (upr > 0 && (upr & (upr - 1)) == 0) {
      int l = 0;
      while ((int64_t(1) << l) < upr) ++l;
      a.upr_log2[t] = l;
    }
    a.blk_start[t] = blocks;
    blocks += (n_kept * upr + kUnitsPerBlock - 1) / kUnitsPerBlock;
  }
  a.blk_start[desc.n] = blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, kept_idx, n_kept, n_src, a);
  return hipGetLastError();
}

}  // namespace tg
