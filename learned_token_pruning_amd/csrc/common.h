// Internal helpers shared by the gfx950 kernels of libtokengate (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tokengate.h"

namespace tg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// 32x32x16 bf16 MFMA, fp32 accumulate (CDNA4).  Operand layout, lane l, g = l / 32:
//   A[m][k]: lane holds m = l % 32, k = 8 g .. 8 g + 7
//   B[k][n]: lane holds n = l % 32, k = 8 g .. 8 g + 7
//   C[m][n]: register i holds m = 8 (i / 4) + 4 g + (i % 4), n = l % 32
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Raw buffer resource (gfx9 family): base address, byte range, no stride.
// Loads past the range return zeros, which handles ragged tiles without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ float buf_load4f(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

// Combine every lane with lane ^ 32 (v_permlane32_swap, no LDS round trip).
// The swap returns the two halves in both orders, so max / sum of the pair is
// the same expression, with the same rounding, in both half-waves.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane reductions on DPP row operations and the gfx950 row swaps (no LDS
// round trip).  Every step combines a lane with its partner in an order-free
// way (a + b and b + a, max), so all lanes of a group end with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xb1, kQuadXor2 = 0x4e, kRowHalfMirror = 0x141, kRowMirror = 0x140, kRowRor8 = 0x128;

__device__ __forceinline__ float swap16_sum(float x) {  // x + x of lane ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum over aligned groups of N lanes (N = 8 or 16)
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  if (N == 16) x += dpp<kRowMirror>(x);
  return x;
}
__device__ __forceinline__ float wave_sum(float x) { return xor32_sum(swap16_sum(group_sum<16>(x))); }
__device__ __forceinline__ float wave_max(float x) {
  x = __builtin_fmaxf(x, dpp<kQuadXor1>(x));
  x = __builtin_fmaxf(x, dpp<kQuadXor2>(x));
  x = __builtin_fmaxf(x, dpp<kRowHalfMirror>(x));
  x = __builtin_fmaxf(x, dpp<kRowMirror>(x));
  return xor32_max(swap16_max(x));
}
// sum over the lanes sharing lane % N (N = 8 or 16)
template <int N>
__device__ __forceinline__ float stride_sum(float x) {
  if (N == 8) x += dpp<kRowRor8>(x);
  return xor32_sum(swap16_sum(x));
}

// Inclusive prefix sum over the 64 lanes of a wave on DPP: Hillis-Steele
// shifts inside each 16-lane row (shifted-in lanes read 0), then row 15's and
// row 31's totals broadcast into the later rows.  Compiles to six v_add_u32_dpp.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_shift_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xf, true);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_shift_u32<0x111, 0xf>(x);  // row_shr:1
  x += dpp_shift_u32<0x112, 0xf>(x);  // row_shr:2
  x += dpp_shift_u32<0x114, 0xf>(x);  // row_shr:4
  x += dpp_shift_u32<0x118, 0xf>(x);  // row_shr:8
  x += dpp_shift_u32<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_shift_u32<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (inputs here are finite or inf; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Order-preserving key of an fp32 score: larger score -> larger key; -0.0 and
// +0.0 share a key; NaN maps to 0, below every number (-inf -> 0x007fffff).
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Direct-to-LDS staging and LDS-read scheduling helpers shared by the attention kernels.
#define TG_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// One DMA instruction: every active lane copies 16 (or 4) bytes from the buffer
// at voff + soff into LDS at lds_dst + 16 (or 4) x lane.  Issued in asm so the
// compiler does not order later LDS reads after it; every consumer waits with
// an explicit vmcnt (the instruction has no destination registers).
// A device segment table together with the totals of its plan, which the host validated and sized every
// grid and buffer from.  Kernels read entries only through at(), which clamps each field into those totals:
// 0 <= seg_start <= n_tokens, seg_len <= min(max_seg_len, n_tokens - seg_start),
// 0 <= doc_begin <= doc_end <= seg_len with doc_end - doc_begin <= max_doc_len, 0 <= k_eff <= that length,
// 0 <= kept_start <= total_kept, kept_len <= min(max_kept_len, total_kept - kept_start).
// A table that agrees with its info passes unchanged; one that does not yields wrong values, never an access
// outside the arrays.
struct SegTable {
  const tg_segment* p;
  int32_t n_tokens, total_kept, max_seg_len, max_doc_len, max_kept_len;

  static __host__ __device__ __forceinline__ int32_t clampi(int64_t x, int32_t lo, int32_t hi) {
    return x < lo ? lo : (x > hi ? hi : (int32_t)x);
  }
  // the clamped copy of entry r (host-callable, so the rule can be checked without a device)
  static __host__ __device__ __forceinline__ tg_segment clamp(const tg_segment& r, int32_t n_tokens,
                                                              int32_t total_kept, int32_t max_seg_len,
                                                              int32_t max_doc_len, int32_t max_kept_len) {
    tg_segment s;
    s.seg_start = clampi(r.seg_start, 0, n_tokens);
    s.seg_len = clampi(r.seg_len, 0, n_tokens - s.seg_start < max_seg_len ? n_tokens - s.seg_start : max_seg_len);
    s.doc_begin = clampi(r.doc_begin, 0, s.seg_len);
    const int32_t room = s.seg_len - s.doc_begin;
    s.doc_end = s.doc_begin + clampi((int64_t)r.doc_end - s.doc_begin, 0, room < max_doc_len ? room : max_doc_len);
    s.k_eff = clampi(r.k_eff, 0, s.doc_end - s.doc_begin);
    s.kept_start = clampi(r.kept_start, 0, total_kept);
    const int32_t left = total_kept - s.kept_start;
    s.kept_len = clampi(r.kept_len, 0, left < max_kept_len ? left : max_kept_len);
    s.reserved = 0;
    return s;
  }
  __device__ __forceinline__ tg_segment at(int i) const {
    return clamp(p[i], n_tokens, total_kept, max_seg_len, max_doc_len, max_kept_len);
  }
  // at(i) for an index that is the same in every lane (a workgroup's own prompt): the fields stay in
  // scalar registers, as buffer descriptors and LDS DMA addresses built from them need.
  __device__ __forceinline__ tg_segment at_uniform(int i) const {
    tg_segment s = at(i);
    s.seg_start = __builtin_amdgcn_readfirstlane(s.seg_start);
    s.seg_len = __builtin_amdgcn_readfirstlane(s.seg_len);
    s.doc_begin = __builtin_amdgcn_readfirstlane(s.doc_begin);
    s.doc_end = __builtin_amdgcn_readfirstlane(s.doc_end);
    s.k_eff = __builtin_amdgcn_readfirstlane(s.k_eff);
    s.kept_start = __builtin_amdgcn_readfirstlane(s.kept_start);
    s.kept_len = __builtin_amdgcn_readfirstlane(s.kept_len);
    return s;
  }
};

// info has passed the host checks (n_tokens < 2^31, total_kept <= n_tokens, maxima >= 0).
inline SegTable seg_table(const tg_segment* p, const tg_plan_info& info) {
  return SegTable{p, (int32_t)info.n_tokens, (int32_t)info.total_kept, info.max_seg_len, info.max_doc_len,
                  info.max_kept_len};
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void* lds_dst, uint32_t voff, uint32_t soff) {
  const uint32_t m0v = (uint32_t)(uintptr_t)TG_LDS(lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0v), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, const void* lds_dst, uint32_t voff, uint32_t soff) {
  const uint32_t m0v = (uint32_t)(uintptr_t)TG_LDS(lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(m0v), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


// Instruction order for a block of MFMAS matrix ops fed by READS LDS reads:
// AHEAD reads first, then alternating MFMA / read, then the remaining MFMAs.
// Left alone, the compiler waits for each read right before its MFMA.
template <int MFMAS, int READS, int AHEAD>
__device__ __forceinline__ void sched_reads_ahead() {
  static_assert(READS >= AHEAD && MFMAS >= READS - AHEAD, "pattern");
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
#pragma unroll
  for (int i = 0; i < READS - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < MFMAS - (READS - AHEAD); ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}


// Instruction order for MFMAS matrix ops fed by two LDS reads each: AHEAD
// reads first, then MFMA / read / read, then the remaining MFMAs.
template <int MFMAS, int AHEAD>
__device__ __forceinline__ void sched_two_reads_ahead() {
  constexpr int READS = 2 * MFMAS;
  constexpr int PAIRS = (READS - AHEAD) / 2;
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int i = 0; i < PAIRS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
#pragma unroll
  for (int i = 0; i < MFMAS - PAIRS; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

}  // namespace tg

// Launchers (one per kernel family), defined in the kernel sources.  They
// only launch; arguments are validated by the ABI layer.
namespace tg {
// w1_prepacked: w1 is already in fragment order (launch_gate_pack_w1), not [h, d].
hipError_t launch_gate_score(const void* x, int64_t ld_x, int d, const void* w1, bool w1_prepacked, const float* b1,
                             const float* w2, float b2, int h, const tg_segment* segs, const tg_plan_info& info,
                             float rms_eps, float* scores, void* workspace, hipStream_t stream);
hipError_t launch_gate_pack_w1(const void* w1, int d, int h, void* w1_packed, hipStream_t stream);
size_t gate_workspace_bytes(const tg_plan_info& info, int d, int h);
// The prepacked gate's scratch (per-tile sums of squares): bytes needed for a plan, the fixed capacity of the
// library's own array, and the device address of the current GPU's copy of that array.
size_t gate_sumsq_bytes(const tg_plan_info& info);
size_t gate_scratch_bytes();
hipError_t gate_scratch(void** ptr);

hipError_t launch_select_topk(const float* scores, const tg_segment* segs, const tg_plan_info& info,
                              int32_t* kept_idx, void* workspace, hipStream_t stream);
size_t select_workspace_bytes(const tg_plan_info& info);

struct CompactDesc {
  int n;
  const char* src[TG_COMPACT_MAX_TENSORS];
  char* dst[TG_COMPACT_MAX_TENSORS];
  int64_t row_bytes[TG_COMPACT_MAX_TENSORS];
  int64_t src_stride[TG_COMPACT_MAX_TENSORS];
  int64_t dst_stride[TG_COMPACT_MAX_TENSORS];
};
hipError_t launch_compact(const int32_t* kept_idx, int64_t n_kept, int64_t n_src, const CompactDesc& desc,
                          hipStream_t stream);

// kept_idx == nullptr: q, k, v, key_score are the compacted kept rows.  Otherwise
// they hold n_src rows and kept row r of a prompt is row kept_idx[kept_start + r].
// split_ws: nullptr, or a zero-initialised workspace of attention_prefill_workspace_bytes
// (the counters are left at zero): long query tiles of a prompt too short to fill the
// GPU are then split over two workgroups.
hipError_t launch_gated_attention(const void* q, const void* k, const void* v, const float* key_score,
                                  const float* tau, const float* gain, const tg_segment* segs,
                                  const tg_plan_info& info, int hq, int hkv, int head_dim, const int32_t* kept_idx,
                                  int64_t n_src, const int32_t* qpos, float* lse, void* out, hipStream_t stream,
                                  void* split_ws = nullptr);
// Bytes of split_ws for these shapes on the current device; 0 when no query tile is split.
size_t attention_prefill_workspace_bytes(const tg_plan_info& info, int hq, int hkv, int head_dim);
constexpr int64_t kAttnMaxGatherRows = 16384;

// Backward of the compacted-row attention; lse from the forward (natural log).
size_t attention_backward_workspace_bytes(const tg_plan_info& info, int hq, int hkv, int head_dim);
hipError_t launch_gated_attention_backward(const void* q, const void* k, const void* v, const float* key_score,
                                           const float* tau, const float* gain, const tg_segment* segs,
                                           const tg_plan_info& info, int hq, int hkv, int head_dim, const void* out,
                                           const void* dout, const float* lse, float* dq, float* dk, float* dv,
                                           float* ds, float* dgain, float* dtau, void* workspace,
                                           hipStream_t stream);

// One decode step over per-sequence KV caches [batch, cap, hkv, head_dim];
// the workspace holds the split-KV partials.
size_t decode_workspace_bytes(int batch, int hq, int head_dim, int64_t cap);
hipError_t launch_gated_decode(const void* q, const void* kc, const void* vc, const float* key_score,
                               const float* tau, int tau_per_query, const float* gain, const int32_t* lens,
                               int batch, int64_t cap, int hq, int hkv, int head_dim, void* out, void* workspace,
                               hipStream_t stream);

hipError_t launch_gemm(int epi, const void* x, int64_t ldx, const void* w, int64_t ldw, int64_t m, int n, int k,
                       const void* res, int64_t ldr, void* y, int64_t ldy, hipStream_t stream);
hipError_t launch_rmsnorm(const void* x, int64_t ldx, int64_t m, int d, const void* weight, float eps, void* y,
                          int64_t ldy, hipStream_t stream);
hipError_t launch_rope_split(const void* qkv, int64_t ldqkv, int64_t m, int hq, int hkv, int dh,
                             const int32_t* positions, float theta, void* q, void* k, void* v, hipStream_t stream);
}  // namespace tg
