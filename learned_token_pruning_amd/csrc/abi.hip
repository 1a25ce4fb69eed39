// C ABI of libtokengate: argument validation, device checks and dispatch to
// the kernel launchers.  Nothing here allocates device memory or synchronises.
#include <atomic>
#include <cstring>

#include "common.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return TG_ERR_NO_DEVICE;
  }
  if (dev < kMaxDevices) {
    const int s = g_arch_state[dev].load(std::memory_order_relaxed);
    if (s == 1) return TG_OK;
    if (s == -1) return TG_ERR_NO_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return TG_ERR_NO_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_state[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  return ok ? TG_OK : TG_ERR_NO_DEVICE;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? TG_OK : TG_ERR_HIP; }

int check_info(const tg_segment* segs, const tg_plan_info* info) {
  if (segs == nullptr || info == nullptr) return TG_ERR_INVALID_ARG;
  if (info->n_seg < 1 || info->n_tokens < 0 || info->total_kept < 0 || info->max_seg_len < 0 ||
      info->max_doc_len < 0 || info->max_kept_len < 0)
    return TG_ERR_INVALID_ARG;
  if (info->max_doc_len > info->max_seg_len || info->max_kept_len > info->max_seg_len ||
      info->n_tokens > 0x7fffffffLL || info->total_kept > info->n_tokens)
    return TG_ERR_INVALID_ARG;
  if (!aligned(segs, 4)) return TG_ERR_INVALID_ARG;
  return TG_OK;
}

}  // namespace

extern "C" {

const char* tg_status_string(int status) {
  switch (status) {
    case TG_OK: return "ok";
    case TG_ERR_INVALID_ARG: return "invalid argument";
    case TG_ERR_UNSUPPORTED: return "unsupported shape or layout";
    case TG_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TG_ERR_NO_DEVICE: return "no gfx950 HIP device";
    case TG_ERR_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

int tg_abi_version(void) { return TG_ABI_VERSION; }

int64_t tg_kept_count(int64_t n_doc, int64_t n_other, int64_t k) {
  if (n_doc < 0 || n_other < 0 || k < 0) return -1;
  return (k < n_doc ? k : n_doc) + n_other;
}

int tg_plan_segments(int n_seg, const int32_t* seg_start, const int32_t* doc_begin, const int32_t* doc_end,
                     const int32_t* k_budget, tg_segment* table, tg_plan_info* info) {
  if (n_seg < 1 || !seg_start || !doc_begin || !doc_end || !k_budget || !table || !info) return TG_ERR_INVALID_ARG;
  if (seg_start[0] != 0) return TG_ERR_INVALID_ARG;
  int64_t kept = 0;
  int32_t max_seg = 0, max_doc = 0, max_kept = 0;
  for (int i = 0; i < n_seg; ++i) {
    const int64_t a = seg_start[i], b = seg_start[i + 1];
    if (b < a) return TG_ERR_INVALID_ARG;
    const int64_t len = b - a;
    const int64_t db = doc_begin[i], de = doc_end[i];
    if (db < 0 || de < db || de > len) return TG_ERR_INVALID_ARG;
    if (k_budget[i] < 0) return TG_ERR_INVALID_ARG;
    const int64_t n_doc = de - db;
    const int64_t keff = k_budget[i] < n_doc ? k_budget[i] : n_doc;
    const int64_t klen = keff + (len - n_doc);
    tg_segment s;
    s.seg_start = (int32_t)a;
    s.seg_len = (int32_t)len;
    s.doc_begin = (int32_t)db;
    s.doc_end = (int32_t)de;
    s.k_eff = (int32_t)keff;
    s.kept_start = (int32_t)kept;
    s.kept_len = (int32_t)klen;
    s.reserved = 0;
    table[i] = s;
    kept += klen;
    if (len > max_seg) max_seg = (int32_t)len;
    if (n_doc > max_doc) max_doc = (int32_t)n_doc;
    if (klen > max_kept) max_kept = (int32_t)klen;
  }
  info->n_tokens = seg_start[n_seg];
  info->total_kept = kept;
  info->n_seg = n_seg;
  info->max_seg_len = max_seg;
  info->max_doc_len = max_doc;
  info->max_kept_len = max_kept;
  return TG_OK;
}

size_t tg_gate_workspace_bytes(const tg_plan_info* info, int d, int h) {
  if (info == nullptr || info->n_seg < 1 || d <= 0 || h <= 0) return 0;
  return tg::gate_workspace_bytes(*info, d, h);
}

int tg_gate_score(const void* x, int64_t ld_x, int d, const void* w1, const float* b1, const float* w2, float b2,
                  int h, const tg_segment* segs, const tg_plan_info* info, float rms_eps, float* scores,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_info(segs, info);
  if (st != TG_OK) return st;
  if (!x || !w1 || !w2 || !scores || d <= 0 || h <= 0 || ld_x < d) return TG_ERR_INVALID_ARG;
  if (rms_eps != rms_eps) return TG_ERR_INVALID_ARG;  // NaN
  if (d % 64 != 0 || d > 65536 || h % 64 != 0 || h > 256 || ld_x % 8 != 0) return TG_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || (b1 && !aligned(b1, 16)) || !aligned(scores, 4))
    return TG_ERR_UNSUPPORTED;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < tg::gate_workspace_bytes(*info, d, h))
    return TG_ERR_WORKSPACE;
  st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_gate_score(x, ld_x, d, w1, false, b1, w2, b2, h, segs, *info, rms_eps, scores,
                                          workspace, reinterpret_cast<hipStream_t>(stream)));
}

size_t tg_gate_packed_w1_bytes(int d, int h) {
  if (d <= 0 || h <= 0) return 0;
  return (size_t)d * (size_t)h * 2;
}

int tg_gate_pack_w1(const void* w1, int d, int h, void* w1_packed, void* stream) {
  if (!w1 || !w1_packed || d <= 0 || h <= 0) return TG_ERR_INVALID_ARG;
  if (d % 64 != 0 || d > 65536 || h % 64 != 0 || h > 256) return TG_ERR_UNSUPPORTED;
  if (!aligned(w1, 16) || !aligned(w1_packed, 16)) return TG_ERR_UNSUPPORTED;
  const int st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_gate_pack_w1(w1, d, h, w1_packed, reinterpret_cast<hipStream_t>(stream)));
}

int tg_gate_score_prepacked(const void* x, int64_t ld_x, int d, const void* w1_packed, const float* b1,
                            const float* w2, float b2, int h, const tg_segment* segs, const tg_plan_info* info,
                            float rms_eps, float* scores, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_info(segs, info);
  if (st != TG_OK) return st;
  if (!x || !w1_packed || !w2 || !scores || d <= 0 || h <= 0 || ld_x < d) return TG_ERR_INVALID_ARG;
  if (rms_eps != rms_eps) return TG_ERR_INVALID_ARG;  // NaN
  if (d % 64 != 0 || d > 65536 || h % 64 != 0 || h > 256 || ld_x % 8 != 0) return TG_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w1_packed, 16) || !aligned(w2, 16) || (b1 && !aligned(b1, 16)) ||
      !aligned(scores, 4))
    return TG_ERR_UNSUPPORTED;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < tg::gate_workspace_bytes(*info, d, h))
    return TG_ERR_WORKSPACE;
  st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_gate_score(x, ld_x, d, w1_packed, true, b1, w2, b2, h, segs, *info, rms_eps, scores,
                                          workspace, reinterpret_cast<hipStream_t>(stream)));
}

int tg_gate_score_prepacked_noalloc(const void* x, int64_t ld_x, int d, const void* w1_packed, const float* b1,
                                    const float* w2, float b2, int h, const tg_segment* segs,
                                    const tg_plan_info* info, float rms_eps, float* scores, void* stream) {
  int st = check_info(segs, info);
  if (st != TG_OK) return st;
  if (!x || !w1_packed || !w2 || !scores || d <= 0 || h <= 0 || ld_x < d) return TG_ERR_INVALID_ARG;
  if (rms_eps != rms_eps) return TG_ERR_INVALID_ARG;  // NaN
  if (d % 64 != 0 || d > 65536 || h % 64 != 0 || h > 256 || ld_x % 8 != 0) return TG_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w1_packed, 16) || !aligned(w2, 16) || (b1 && !aligned(b1, 16)) ||
      !aligned(scores, 4))
    return TG_ERR_UNSUPPORTED;
  if (tg::gate_sumsq_bytes(*info) > tg::gate_scratch_bytes()) return TG_ERR_WORKSPACE;
  st = check_device();
  if (st != TG_OK) return st;
  void* scratch = nullptr;
  if (tg::gate_scratch(&scratch) != hipSuccess) {
    (void)hipGetLastError();
    return TG_ERR_HIP;
  }
  return hip_status(tg::launch_gate_score(x, ld_x, d, w1_packed, true, b1, w2, b2, h, segs, *info, rms_eps, scores,
                                          scratch, reinterpret_cast<hipStream_t>(stream)));
}

size_t tg_gate_noalloc_max_tiles(void) { return tg::gate_scratch_bytes() / sizeof(double); }

size_t tg_select_workspace_bytes(const tg_plan_info* info) {
  if (info == nullptr || info->n_seg < 1) return 0;
  return tg::select_workspace_bytes(*info);
}

int tg_select_topk(const float* scores, const tg_segment* segs, const tg_plan_info* info, int32_t* kept_idx,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_info(segs, info);
  if (st != TG_OK) return st;
  if (!scores || (!kept_idx && info->total_kept > 0)) return TG_ERR_INVALID_ARG;
  if (!aligned(scores, 4) || (kept_idx && !aligned(kept_idx, 4))) return TG_ERR_INVALID_ARG;
  const size_t ws_need = tg::select_workspace_bytes(*info);
  if (ws_need > 0 && (!workspace || !aligned(workspace, 256) || workspace_bytes < ws_need)) return TG_ERR_WORKSPACE;
  st = check_device();
  if (st != TG_OK) return st;
  return hip_status(
      tg::launch_select_topk(scores, segs, *info, kept_idx, workspace, reinterpret_cast<hipStream_t>(stream)));
}

int tg_compact_kept(const int32_t* kept_idx, int64_t n_kept, int64_t n_src_rows, int n_tensors, const void* const* src,
                    void* const* dst, const int64_t* row_bytes, const int64_t* src_stride,
                    const int64_t* dst_stride, void* stream) {
  if (n_kept < 0 || n_src_rows < 0 || n_tensors < 1 || n_tensors > TG_COMPACT_MAX_TENSORS) return TG_ERR_INVALID_ARG;
  if (!src || !dst || !row_bytes || !src_stride || !dst_stride) return TG_ERR_INVALID_ARG;
  if (n_kept > 0 && (!kept_idx || !aligned(kept_idx, 4))) return TG_ERR_INVALID_ARG;
  tg::CompactDesc desc{};
  desc.n = n_tensors;
  for (int t = 0; t < n_tensors; ++t) {
    if (row_bytes[t] < 0 || src_stride[t] < 0 || dst_stride[t] < row_bytes[t]) return TG_ERR_INVALID_ARG;
    if (row_bytes[t] > 0 && n_kept > 0) {
      if (!src[t] || !dst[t]) return TG_ERR_INVALID_ARG;
      if (src[t] == dst[t]) return TG_ERR_INVALID_ARG;  // an in-place gather would race
    }
    desc.src[t] = static_cast<const char*>(src[t]);
    desc.dst[t] = static_cast<char*>(dst[t]);
    desc.row_bytes[t] = row_bytes[t];
    desc.src_stride[t] = src_stride[t];
    desc.dst_stride[t] = dst_stride[t];
  }
  if (n_kept == 0) return TG_OK;
  int st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_compact(kept_idx, n_kept, n_src_rows, desc, reinterpret_cast<hipStream_t>(stream)));
}

namespace {
// Shapes every attention kernel supports.  `buffer_ranges`: the kernel
// addresses one prompt's K/V rows through buffer descriptors, whose byte
// ranges are 32-bit.
int check_attention_shapes(const tg_segment* segs, const tg_plan_info* info, int hq, int hkv, int head_dim,
                           bool buffer_ranges) {
  int st = check_info(segs, info);
  if (st != TG_OK) return st;
  if (hq <= 0 || hkv <= 0 || head_dim <= 0) return TG_ERR_INVALID_ARG;
  if (hq % hkv != 0) return TG_ERR_UNSUPPORTED;
  const int G = hq / hkv;
  if (!(head_dim == 64 || head_dim == 128) || !(G == 1 || G == 2 || G == 4)) return TG_ERR_UNSUPPORTED;
  if (buffer_ranges && (int64_t)info->max_kept_len * hkv * head_dim * 2 >= 0xffffff00LL) return TG_ERR_UNSUPPORTED;
  return TG_OK;
}
}  // namespace

int tg_gated_attention_prefill(const void* q, const void* k, const void* v, const float* key_score,
                               const float* tau, const float* gain, const tg_segment* segs,
                               const tg_plan_info* info, int hq, int hkv, int head_dim, void* out, void* stream) {
  int st = check_attention_shapes(segs, info, hq, hkv, head_dim, true);
  if (st != TG_OK) return st;
  if (info->total_kept > 0 && (!q || !k || !v || !out)) return TG_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return TG_ERR_INVALID_ARG;
  if ((key_score && !aligned(key_score, 4)) || (tau && !aligned(tau, 4)) || (gain && !aligned(gain, 4)))
    return TG_ERR_INVALID_ARG;
  if (info->total_kept == 0) return TG_OK;
  st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_gated_attention(q, k, v, key_score, tau, gain, segs, *info, hq, hkv, head_dim,
                                               nullptr, 0, nullptr, nullptr, out,
                                               reinterpret_cast<hipStream_t>(stream)));
}

namespace {
// The split-tile workspace of an attention call: TG_ERR_WORKSPACE when one is needed and missing, misaligned or
// short; *use = the workspace, or nullptr when no tile is split.
int split_workspace(const tg_plan_info* info, int hq, int hkv, int head_dim, void* workspace, size_t workspace_bytes,
                    void** use) {
  const size_t need = tg::attention_prefill_workspace_bytes(*info, hq, hkv, head_dim);
  if (need > 0 && (!workspace || !aligned(workspace, 256) || workspace_bytes < need)) return TG_ERR_WORKSPACE;
  *use = need > 0 ? workspace : nullptr;
  return TG_OK;
}
}  // namespace

size_t tg_attention_prefill_workspace_bytes(const tg_plan_info* info, int hq, int hkv, int head_dim) {
  if (!info || hq <= 0 || hkv <= 0 || head_dim <= 0 || info->n_seg < 1 || info->total_kept < 0) return 0;
  return tg::attention_prefill_workspace_bytes(*info, hq, hkv, head_dim);
}

int tg_attention_workspace_status(const void* workspace, int* status, void* stream) {
  if (!workspace || !status || !aligned(workspace, 256)) return TG_ERR_INVALID_ARG;
  const int st = check_device();
  if (st != TG_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int word = 0;
  if (hipMemcpyAsync(&word, workspace, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    (void)hipGetLastError();
    return TG_ERR_HIP;
  }
  *status = word;
  return TG_OK;
}

int tg_gated_attention_prefill_ws(const void* q, const void* k, const void* v, const float* key_score,
                                  const float* tau, const float* gain, const tg_segment* segs,
                                  const tg_plan_info* info, int hq, int hkv, int head_dim, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  int st = check_attention_shapes(segs, info, hq, hkv, head_dim, true);
  if (st != TG_OK) return st;
  if (info->total_kept > 0 && (!q || !k || !v || !out)) return TG_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return TG_ERR_INVALID_ARG;
  if ((key_score && !aligned(key_score, 4)) || (tau && !aligned(tau, 4)) || (gain && !aligned(gain, 4)))
    return TG_ERR_INVALID_ARG;
  if (info->total_kept == 0) return TG_OK;
  st = check_device();
  if (st != TG_OK) return st;
  void* split_ws = nullptr;
  if ((st = split_workspace(info, hq, hkv, head_dim, workspace, workspace_bytes, &split_ws)) != TG_OK) return st;
  return hip_status(tg::launch_gated_attention(q, k, v, key_score, tau, gain, segs, *info, hq, hkv, head_dim,
                                               nullptr, 0, nullptr, nullptr, out,
                                               reinterpret_cast<hipStream_t>(stream), split_ws));
}

namespace {
// with_ws: the _ws entry point (workspace checked and passed on; split query tiles allowed)
int query_tau_impl(const void* q, const void* k, const void* v, const float* key_score,
                                         const float* sigma, const float* gain, const int32_t* positions,
                                         const tg_segment* segs, const tg_plan_info* info, int hq, int hkv,
                                         int head_dim, void* out, bool with_ws, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  if (!sigma) return TG_ERR_INVALID_ARG;
  int st = check_attention_shapes(segs, info, hq, hkv, head_dim, true);
  if (st != TG_OK) return st;
  if (info->total_kept > 0 && (!q || !k || !v || !out || !positions)) return TG_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return TG_ERR_INVALID_ARG;
  if ((key_score && !aligned(key_score, 4)) || !aligned(sigma, 4) || (gain && !aligned(gain, 4)) ||
      (positions && !aligned(positions, 4)))
    return TG_ERR_INVALID_ARG;
  if (info->total_kept == 0) return TG_OK;
  st = check_device();
  if (st != TG_OK) return st;
  void* split_ws = nullptr;
  if (with_ws && (st = split_workspace(info, hq, hkv, head_dim, workspace, workspace_bytes, &split_ws)) != TG_OK)
    return st;
  return hip_status(tg::launch_gated_attention(q, k, v, key_score, sigma, gain, segs, *info, hq, hkv, head_dim,
                                               nullptr, 0, positions, nullptr, out,
                                               reinterpret_cast<hipStream_t>(stream), split_ws));
}
}  // namespace

int tg_gated_attention_prefill_query_tau(const void* q, const void* k, const void* v, const float* key_score,
                                         const float* sigma, const float* gain, const int32_t* positions,
                                         const tg_segment* segs, const tg_plan_info* info, int hq, int hkv,
                                         int head_dim, void* out, void* stream) {
  return query_tau_impl(q, k, v, key_score, sigma, gain, positions, segs, info, hq, hkv, head_dim, out, false,
                        nullptr, 0, stream);
}

int tg_gated_attention_prefill_query_tau_ws(const void* q, const void* k, const void* v, const float* key_score,
                                            const float* sigma, const float* gain, const int32_t* positions,
                                            const tg_segment* segs, const tg_plan_info* info, int hq, int hkv,
                                            int head_dim, void* out, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  return query_tau_impl(q, k, v, key_score, sigma, gain, positions, segs, info, hq, hkv, head_dim, out, true,
                        workspace, workspace_bytes, stream);
}

namespace {
int gather_impl(const void* q, const void* k, const void* v, const float* key_score,
                                      const float* tau, const float* gain, const tg_segment* segs,
                                      const tg_plan_info* info, int hq, int hkv, int head_dim,
                                      const int32_t* kept_idx, int64_t n_src_rows, void* out, bool with_ws,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_info(segs, info);
  if (st != TG_OK) return st;
  if (hq <= 0 || hkv <= 0 || head_dim <= 0 || n_src_rows < 0) return TG_ERR_INVALID_ARG;
  if (info->total_kept > 0 && (!q || !k || !v || !out || !kept_idx || n_src_rows == 0)) return TG_ERR_INVALID_ARG;
  if (hq % hkv != 0) return TG_ERR_UNSUPPORTED;
  const int G = hq / hkv;
  if (!(head_dim == 64 || head_dim == 128) || !(G == 1 || G == 2 || G == 4)) return TG_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return TG_ERR_INVALID_ARG;
  if ((key_score && !aligned(key_score, 4)) || (tau && !aligned(tau, 4)) || (gain && !aligned(gain, 4)) ||
      (kept_idx && !aligned(kept_idx, 4)))
    return TG_ERR_INVALID_ARG;
  // indices of a prompt's kept rows live in LDS; K/V rows are addressed with 32-bit byte offsets
  if (info->max_kept_len > tg::kAttnMaxGatherRows) return TG_ERR_UNSUPPORTED;
  if (n_src_rows * (int64_t)hkv * head_dim * 2 >= 0xffffff00LL || n_src_rows * 4 >= 0xffffff00LL)
    return TG_ERR_UNSUPPORTED;
  if (info->total_kept == 0) return TG_OK;
  st = check_device();
  if (st != TG_OK) return st;
  void* split_ws = nullptr;
  if (with_ws && (st = split_workspace(info, hq, hkv, head_dim, workspace, workspace_bytes, &split_ws)) != TG_OK)
    return st;
  return hip_status(tg::launch_gated_attention(q, k, v, key_score, tau, gain, segs, *info, hq, hkv, head_dim,
                                               kept_idx, n_src_rows, nullptr, nullptr, out,
                                               reinterpret_cast<hipStream_t>(stream), split_ws));
}
}  // namespace

int tg_gated_attention_prefill_gather(const void* q, const void* k, const void* v, const float* key_score,
                                      const float* tau, const float* gain, const tg_segment* segs,
                                      const tg_plan_info* info, int hq, int hkv, int head_dim,
                                      const int32_t* kept_idx, int64_t n_src_rows, void* out, void* stream) {
  return gather_impl(q, k, v, key_score, tau, gain, segs, info, hq, hkv, head_dim, kept_idx, n_src_rows, out, false,
                     nullptr, 0, stream);
}

int tg_gated_attention_prefill_gather_ws(const void* q, const void* k, const void* v, const float* key_score,
                                         const float* tau, const float* gain, const tg_segment* segs,
                                         const tg_plan_info* info, int hq, int hkv, int head_dim,
                                         const int32_t* kept_idx, int64_t n_src_rows, void* out, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  return gather_impl(q, k, v, key_score, tau, gain, segs, info, hq, hkv, head_dim, kept_idx, n_src_rows, out, true,
                     workspace, workspace_bytes, stream);
}


int tg_gated_attention_prefill_lse(const void* q, const void* k, const void* v, const float* key_score,
                                   const float* tau, const float* gain, const tg_segment* segs,
                                   const tg_plan_info* info, int hq, int hkv, int head_dim, void* out, float* lse,
                                   void* stream) {
  int st = check_attention_shapes(segs, info, hq, hkv, head_dim, true);
  if (st != TG_OK) return st;
  if (info->total_kept > 0 && (!q || !k || !v || !out || !lse)) return TG_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
      (key_score && !aligned(key_score, 4)) || (tau && !aligned(tau, 4)) || (gain && !aligned(gain, 4)))
    return TG_ERR_INVALID_ARG;
  if (info->total_kept == 0) return TG_OK;
  st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_gated_attention(q, k, v, key_score, tau, gain, segs, *info, hq, hkv, head_dim,
                                               nullptr, 0, nullptr, lse, out,
                                               reinterpret_cast<hipStream_t>(stream)));
}

size_t tg_attention_backward_workspace_bytes(const tg_plan_info* info, int hq, int hkv, int head_dim) {
  if (!info || hq <= 0 || hkv <= 0 || head_dim <= 0 || info->n_seg < 1 || info->total_kept < 0) return 0;
  return tg::attention_backward_workspace_bytes(*info, hq, hkv, head_dim);
}

int tg_gated_attention_backward(const void* q, const void* k, const void* v, const float* key_score,
                                const float* tau, const float* gain, const tg_segment* segs,
                                const tg_plan_info* info, int hq, int hkv, int head_dim, const void* out,
                                const void* dout, const float* lse, float* dq, float* dk, float* dv, float* ds,
                                float* dgain, float* dtau, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_attention_shapes(segs, info, hq, hkv, head_dim, false);
  if (st != TG_OK) return st;
  if (info->total_kept > 0 && (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv))
    return TG_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(ds, 4) ||
      !aligned(dgain, 4) || !aligned(dtau, 4) || (key_score && !aligned(key_score, 4)) ||
      (tau && !aligned(tau, 4)) || (gain && !aligned(gain, 4)))
    return TG_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 16) ||
      workspace_bytes < tg::attention_backward_workspace_bytes(*info, hq, hkv, head_dim))
    return TG_ERR_WORKSPACE;
  st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_gated_attention_backward(q, k, v, key_score, tau, gain, segs, *info, hq, hkv, head_dim,
                                                        out, dout, lse, dq, dk, dv, ds, dgain, dtau, workspace,
                                                        reinterpret_cast<hipStream_t>(stream)));
}

size_t tg_decode_workspace_bytes(int batch, int hq, int head_dim, int64_t cache_rows) {
  if (batch <= 0 || hq <= 0 || head_dim <= 0 || cache_rows < 0) return 0;
  return tg::decode_workspace_bytes(batch, hq, head_dim, cache_rows);
}

int tg_gated_attention_decode(const void* q, const void* k_cache, const void* v_cache, const float* key_score,
                              const float* tau, int tau_per_query, const float* gain, const int32_t* lens,
                              int batch, int64_t cache_rows, int hq, int hkv, int head_dim, void* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || hq <= 0 || hkv <= 0 || head_dim <= 0 || cache_rows < 0) return TG_ERR_INVALID_ARG;
  if (tau_per_query != 0 && tau_per_query != 1) return TG_ERR_INVALID_ARG;
  if (batch == 0) return TG_OK;
  if (!q || !out || !lens || (cache_rows > 0 && (!k_cache || !v_cache))) return TG_ERR_INVALID_ARG;
  if (hq % hkv != 0) return TG_ERR_UNSUPPORTED;
  const int G = hq / hkv;
  if (!(head_dim == 64 || head_dim == 128) || !(G == 1 || G == 2 || G == 4)) return TG_ERR_UNSUPPORTED;
  if (batch > 65535 || hkv > 65535 || cache_rows > 65535LL * 256) return TG_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(lens, 4) || (key_score && !aligned(key_score, 4)) || (tau && !aligned(tau, 4)) ||
      (gain && !aligned(gain, 4)))
    return TG_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 16) ||
      workspace_bytes < tg::decode_workspace_bytes(batch, hq, head_dim, cache_rows))
    return TG_ERR_WORKSPACE;
  const int st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_gated_decode(q, k_cache, v_cache, key_score, tau, tau_per_query, gain, lens, batch,
                                            cache_rows, hq, hkv, head_dim, out, workspace,
                                            reinterpret_cast<hipStream_t>(stream)));
}

int tg_gemm_bf16(int epilogue, const void* x, int64_t ldx, const void* w, int64_t ldw, int64_t m, int n, int k,
                 const void* residual, int64_t ldr, void* y, int64_t ldy, void* stream) {
  if (epilogue < TG_GEMM_STORE || epilogue > TG_GEMM_SWIGLU || m < 0 || n <= 0 || k <= 0) return TG_ERR_INVALID_ARG;
  if (m > 0 && (!x || !w || !y || (epilogue == TG_GEMM_RESIDUAL && !residual))) return TG_ERR_INVALID_ARG;
  const int n_out = epilogue == TG_GEMM_SWIGLU ? n / 2 : n;
  if (ldx < k || ldw < k || ldy < n_out || (epilogue == TG_GEMM_RESIDUAL && ldr < n)) return TG_ERR_INVALID_ARG;
  if (n % 128 != 0 || k % 64 != 0 || ldx % 8 != 0 || ldw % 8 != 0 || ldy % 8 != 0 ||
      (epilogue == TG_GEMM_RESIDUAL && ldr % 8 != 0))
    return TG_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || (residual && !aligned(residual, 16)))
    return TG_ERR_UNSUPPORTED;
  if (m == 0) return TG_OK;
  int st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_gemm(epilogue, x, ldx, w, ldw, m, n, k, residual, ldr, y, ldy,
                                    reinterpret_cast<hipStream_t>(stream)));
}

int tg_rmsnorm_bf16(const void* x, int64_t ldx, int64_t m, int d, const void* weight, float eps, void* y, int64_t ldy,
                    void* stream) {
  if (m < 0 || d <= 0 || !(eps >= 0.0f)) return TG_ERR_INVALID_ARG;
  if (m > 0 && (!x || !weight || !y)) return TG_ERR_INVALID_ARG;
  if (ldx < d || ldy < d) return TG_ERR_INVALID_ARG;
  if (d % 8 != 0 || ldx % 8 != 0 || ldy % 8 != 0 || !aligned(x, 16) || !aligned(y, 16) || !aligned(weight, 16))
    return TG_ERR_UNSUPPORTED;
  if (m == 0) return TG_OK;
  int st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_rmsnorm(x, ldx, m, d, weight, eps, y, ldy, reinterpret_cast<hipStream_t>(stream)));
}

int tg_rope_split_bf16(const void* qkv, int64_t ldqkv, int64_t m, int hq, int hkv, int head_dim,
                       const int32_t* positions, float theta, void* q, void* k, void* v, void* stream) {
  if (m < 0 || hq <= 0 || hkv <= 0 || head_dim <= 0 || !(theta > 1.0f)) return TG_ERR_INVALID_ARG;
  if (m > 0 && (!qkv || !positions || !q || !k || !v)) return TG_ERR_INVALID_ARG;
  if (ldqkv < (int64_t)(hq + 2 * hkv) * head_dim) return TG_ERR_INVALID_ARG;
  if (head_dim % 2 != 0 || head_dim > 256) return TG_ERR_UNSUPPORTED;
  if (m == 0) return TG_OK;
  int st = check_device();
  if (st != TG_OK) return st;
  return hip_status(tg::launch_rope_split(qkv, ldqkv, m, hq, hkv, head_dim, positions, theta, q, k, v,
                                          reinterpret_cast<hipStream_t>(stream)));
}

namespace {
struct LayerWs {
  size_t xn, qkv, q, k, v, att, mid, total;
};
LayerWs layer_ws(int64_t m, int d, int hq, int hkv, int dh, int f) {
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  LayerWs w{};
  const size_t r = (size_t)(m > 0 ? m : 1);
  w.xn = al(r * d * 2);
  w.qkv = al(r * (size_t)(hq + 2 * hkv) * dh * 2);
  w.q = al(r * (size_t)hq * dh * 2);
  w.k = al(r * (size_t)hkv * dh * 2);
  w.v = w.k;
  w.att = w.q;
  w.mid = al(r * (size_t)f * 2);
  w.total = w.xn + w.qkv + w.q + w.k + w.v + w.att + w.mid;
  return w;
}
}  // namespace

size_t tg_decoder_layer_workspace_bytes(int64_t m, int d, int hq, int hkv, int head_dim, int f) {
  if (m < 0 || d <= 0 || hq <= 0 || hkv <= 0 || head_dim <= 0 || f <= 0) return 0;
  return layer_ws(m, d, hq, hkv, head_dim, f).total;
}

int tg_decoder_layer(void* hidden, const int32_t* positions, const float* key_score, const tg_segment* segs,
                     const tg_plan_info* info, int d, int hq, int hkv, int head_dim, int f, float rms_eps,
                     float rope_theta, const tg_layer_weights* w, void* post_attn_norm, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_info(segs, info);
  if (st != TG_OK) return st;
  if (!w || d <= 0 || hq <= 0 || hkv <= 0 || head_dim <= 0 || f <= 0 || !(rms_eps >= 0.0f) || !(rope_theta > 1.0f))
    return TG_ERR_INVALID_ARG;
  const int64_t m = info->total_kept;
  if (m > 0 && (!hidden || !positions || !w->attn_norm || !w->wqkv || !w->wo || !w->mlp_norm || !w->w_gate_up ||
                !w->w_down))
    return TG_ERR_INVALID_ARG;
  const int nqkv = (hq + 2 * hkv) * head_dim;
  if (hq % hkv != 0) return TG_ERR_UNSUPPORTED;
  const int G = hq / hkv;
  if (d % 128 != 0 || f % 64 != 0 || nqkv % 128 != 0 || (hq * head_dim) % 64 != 0 || (2 * f) % 128 != 0 ||
      !(head_dim == 64 || head_dim == 128) || !(G == 1 || G == 2 || G == 4))
    return TG_ERR_UNSUPPORTED;
  if ((int64_t)info->max_kept_len * hkv * head_dim * 2 >= 0xffffff00LL) return TG_ERR_UNSUPPORTED;  // attention ranges
  const LayerWs L = layer_ws(m, d, hq, hkv, head_dim, f);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total) return TG_ERR_WORKSPACE;
  if (!aligned(hidden, 16) || (post_attn_norm && !aligned(post_attn_norm, 16))) return TG_ERR_UNSUPPORTED;
  if (m == 0) return TG_OK;
  st = check_device();
  if (st != TG_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  void* xn = base;
  void* qkv = base + L.xn;
  void* q = static_cast<char*>(qkv) + L.qkv;
  void* k = static_cast<char*>(q) + L.q;
  void* v = static_cast<char*>(k) + L.k;
  void* att = static_cast<char*>(v) + L.v;
  void* mid = static_cast<char*>(att) + L.att;
  void* hn = post_attn_norm ? post_attn_norm : xn;
  hipError_t e;
#define TG_TRY(call)            \
  e = (call);                   \
  if (e != hipSuccess) return TG_ERR_HIP;
  TG_TRY(tg::launch_rmsnorm(hidden, d, m, d, w->attn_norm, rms_eps, xn, d, s));
  TG_TRY(tg::launch_gemm(0, xn, d, w->wqkv, d, m, nqkv, d, nullptr, 0, qkv, nqkv, s));
  TG_TRY(tg::launch_rope_split(qkv, nqkv, m, hq, hkv, head_dim, positions, rope_theta, q, k, v, s));
  TG_TRY(tg::launch_gated_attention(q, k, v, key_score, w->tau, w->gain, segs, *info, hq, hkv, head_dim, nullptr, 0,
                                    nullptr, nullptr, att, s));
  TG_TRY(tg::launch_gemm(1, att, (int64_t)hq * head_dim, w->wo, (int64_t)hq * head_dim, m, d, hq * head_dim, hidden,
                         d, hidden, d, s));
  TG_TRY(tg::launch_rmsnorm(hidden, d, m, d, w->mlp_norm, rms_eps, hn, d, s));
  TG_TRY(tg::launch_gemm(2, hn, d, w->w_gate_up, d, m, 2 * f, d, nullptr, 0, mid, f, s));
  TG_TRY(tg::launch_gemm(1, mid, f, w->w_down, f, m, d, f, hidden, d, hidden, d, s));
#undef TG_TRY
  return TG_OK;
}

}  // extern "C"
