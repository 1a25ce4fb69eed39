// Host-side driver of the C ABI for a build with AddressSanitizer and UndefinedBehaviorSanitizer on the host
// code.  No device is needed: every call either fails validation or reaches the device check, which fails
// without a GPU, so no kernel is launched.  Every host array is an exact-size heap allocation, so a read or
// write past one aborts the run; signed overflow or a bad shift in the sizing arithmetic aborts it too.
// Each check that a status is as expected prints the failing call and exits 1; "ok" and exit 0 otherwise.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "tokengate.h"

namespace {

void* const kFake = reinterpret_cast<void*>(0x10000);  // never dereferenced on the host
int g_fail = 0;

void expect(bool ok, const char* what, long a = 0, long b = 0) {
  if (!ok && g_fail++ < 20) std::printf("FAIL %s (%ld, %ld)\n", what, a, b);
}

bool error_before_launch(int st) {  // without a device a valid call ends at the device check
  return st == TG_ERR_NO_DEVICE || st == TG_ERR_INVALID_ARG || st == TG_ERR_UNSUPPORTED || st == TG_ERR_WORKSPACE ||
         st == TG_ERR_HIP;
}

struct Batch {
  std::vector<int32_t> seg_start, doc_begin, doc_end, k;
};

Batch random_batch(std::mt19937_64& rng, int n_seg, int max_len) {
  Batch b;
  b.seg_start.push_back(0);
  for (int i = 0; i < n_seg; ++i) {
    const int len = (int)(rng() % (uint64_t)(max_len + 1));
    const int lo = (int)(rng() % (uint64_t)(len + 1));
    const int hi = lo + (int)(rng() % (uint64_t)(len - lo + 1));
    b.seg_start.push_back(b.seg_start.back() + len);
    b.doc_begin.push_back(lo);
    b.doc_end.push_back(hi);
    b.k.push_back((int)(rng() % (uint64_t)(max_len + 2)));
  }
  return b;
}

// tg_plan_segments with every array in its own exact-size heap block
int plan(const Batch& b, tg_segment** table_out, tg_plan_info* info) {
  const int n = (int)b.doc_begin.size();
  int32_t* ss = new int32_t[n + 1];
  int32_t* db = new int32_t[n];
  int32_t* de = new int32_t[n];
  int32_t* kb = new int32_t[n];
  for (int i = 0; i <= n; ++i) ss[i] = b.seg_start[i];
  for (int i = 0; i < n; ++i) db[i] = b.doc_begin[i], de[i] = b.doc_end[i], kb[i] = b.k[i];
  tg_segment* table = new tg_segment[n > 0 ? n : 1];
  const int st = tg_plan_segments(n, ss, db, de, kb, table, info);
  delete[] ss;
  delete[] db;
  delete[] de;
  delete[] kb;
  *table_out = table;
  return st;
}

void check_plan(const Batch& b, const tg_segment* t, const tg_plan_info& info) {
  int64_t n_tok = 0, kept = 0;
  int ms = 0, md = 0, mk = 0;
  for (size_t i = 0; i < b.doc_begin.size(); ++i) {
    const int len = b.seg_start[i + 1] - b.seg_start[i], nd = b.doc_end[i] - b.doc_begin[i];
    const int ke = b.k[i] < nd ? b.k[i] : nd;
    expect(t[i].seg_start == b.seg_start[i] && t[i].seg_len == len && t[i].k_eff == ke &&
               t[i].kept_start == kept && t[i].kept_len == ke + len - nd,
           "plan entry", (long)i, t[i].kept_len);
    n_tok += len;
    kept += ke + len - nd;
    ms = len > ms ? len : ms;
    md = nd > md ? nd : md;
    mk = ke + len - nd > mk ? ke + len - nd : mk;
  }
  expect(info.n_tokens == n_tok && info.total_kept == kept && info.max_seg_len == ms && info.max_doc_len == md &&
             info.max_kept_len == mk,
         "plan totals", (long)info.total_kept, (long)kept);
}

void exercise(const tg_segment* segs, const tg_plan_info* info, std::mt19937_64& rng) {
  static const int kHeads[][3] = {{16, 8, 128}, {16, 16, 64}, {32, 8, 128}, {16, 6, 128}, {8, 8, 96},
                                  {1, 1, 64}, {0, 8, 128}, {64, 16, 128}};
  for (const auto& s : kHeads) {
    const int hq = s[0], hkv = s[1], dh = s[2];
    const size_t ws = tg_attention_prefill_workspace_bytes(info, hq, hkv, dh);
    const size_t wb = tg_attention_backward_workspace_bytes(info, hq, hkv, dh);
    expect(ws % 256 == 0, "split workspace size is a 256-byte multiple", (long)ws);
    void* wsp = ws ? kFake : nullptr;
    int st = tg_gated_attention_prefill(kFake, kFake, kFake, nullptr, nullptr, nullptr, segs, info, hq, hkv, dh, kFake,
                                        nullptr);
    expect(error_before_launch(st) || (st == TG_OK && info->total_kept == 0), "prefill", st);
    st = tg_gated_attention_prefill_ws(kFake, kFake, kFake, nullptr, nullptr, nullptr, segs, info, hq, hkv, dh, kFake,
                                       wsp, ws, nullptr);
    expect(error_before_launch(st) || (st == TG_OK && info->total_kept == 0), "prefill_ws", st);
    st = tg_gated_attention_prefill_gather(kFake, kFake, kFake, nullptr, nullptr, nullptr, segs, info, hq, hkv, dh,
                                           (const int32_t*)kFake, info->n_tokens, kFake, nullptr);
    expect(error_before_launch(st) || (st == TG_OK && info->total_kept == 0), "gather", st);
    st = tg_gated_attention_prefill_query_tau(kFake, kFake, kFake, nullptr, (const float*)kFake, nullptr,
                                              (const int32_t*)kFake, segs, info, hq, hkv, dh, kFake, nullptr);
    expect(error_before_launch(st) || (st == TG_OK && info->total_kept == 0), "query_tau", st);
    st = tg_gated_attention_prefill_lse(kFake, kFake, kFake, nullptr, nullptr, nullptr, segs, info, hq, hkv, dh, kFake,
                                        (float*)kFake, nullptr);
    expect(error_before_launch(st) || (st == TG_OK && info->total_kept == 0), "lse", st);
    float* f = (float*)kFake;
    st = tg_gated_attention_backward(kFake, kFake, kFake, f, f, f, segs, info, hq, hkv, dh, kFake, kFake, f, f, f, f, f,
                                     f, f, wb ? kFake : nullptr, wb, nullptr);
    expect(error_before_launch(st) || (st == TG_OK && info->total_kept == 0), "backward", st);
  }
  static const int kGate[][2] = {{2048, 256}, {4096, 128}, {64, 64}, {2040, 256}, {2048, 320}, {0, 256}};
  for (const auto& g : kGate) {
    const int d = g[0], h = g[1];
    const size_t ws = tg_gate_workspace_bytes(info, d, h);
    int st = tg_gate_score(kFake, d, d, kFake, nullptr, (const float*)kFake, 0.0f, h, segs, info, 1e-6f,
                           (float*)kFake, ws ? kFake : nullptr, ws, nullptr);
    expect(error_before_launch(st) || st == TG_OK, "gate", st);
    st = tg_gate_score_prepacked(kFake, d, d, kFake, nullptr, (const float*)kFake, 0.0f, h, segs, info, 1e-6f,
                                 (float*)kFake, ws ? kFake : nullptr, ws, nullptr);
    expect(error_before_launch(st) || st == TG_OK, "gate prepacked", st);
    st = tg_gate_score_prepacked_noalloc(kFake, d, d, kFake, nullptr, (const float*)kFake, 0.0f, h, segs, info, 1e-6f,
                                         (float*)kFake, nullptr);
    expect(error_before_launch(st) || st == TG_OK, "gate noalloc", st);
  }
  const size_t sw = tg_select_workspace_bytes(info);
  int st = tg_select_topk((const float*)kFake, segs, info, (int32_t*)kFake, sw ? kFake : nullptr, sw, nullptr);
  expect(error_before_launch(st) || st == TG_OK, "select", st);
  const int d = 256 << (rng() % 3), f = 512 << (rng() % 3);
  const size_t lw = tg_decoder_layer_workspace_bytes(info->total_kept, d, 16, 8, 128, f);
  tg_layer_weights w = {kFake, kFake, kFake, kFake, kFake, kFake, nullptr, nullptr};
  st = tg_decoder_layer(kFake, (const int32_t*)kFake, nullptr, segs, info, d, 16, 8, 128, f, 1e-6f, 1e6f, &w, nullptr,
                        lw ? kFake : nullptr, lw, nullptr);
  expect(error_before_launch(st) || st == TG_OK, "decoder layer", st);
}

void compact_calls(std::mt19937_64& rng) {
  for (int n = 0; n <= TG_COMPACT_MAX_TENSORS + 1; ++n) {
    const int cnt = n > 0 ? n : 1;
    const void** src = new const void*[cnt];
    void** dst = new void*[cnt];
    int64_t* rb = new int64_t[cnt];
    int64_t* ss = new int64_t[cnt];
    int64_t* ds = new int64_t[cnt];
    for (int t = 0; t < cnt; ++t) {
      src[t] = reinterpret_cast<const void*>(0x100000 + 0x10000 * t);
      dst[t] = reinterpret_cast<void*>(0x900000 + 0x10000 * t);
      rb[t] = (int64_t)(1 + rng() % 8192);
      ss[t] = rb[t] + (int64_t)(rng() % 64);
      ds[t] = rb[t] + (int64_t)(rng() % 3);
    }
    const int st = tg_compact_kept((const int32_t*)kFake, 1 + (int64_t)(rng() % 100000), 100000, n, src, dst, rb, ss,
                                   ds, nullptr);
    expect(n >= 1 && n <= TG_COMPACT_MAX_TENSORS ? error_before_launch(st) : st == TG_ERR_INVALID_ARG, "compact", n,
           st);
    delete[] src;
    delete[] dst;
    delete[] rb;
    delete[] ss;
    delete[] ds;
  }
}

void dense_calls(std::mt19937_64& rng) {
  for (int i = 0; i < 200; ++i) {
    const int64_t m = (int64_t)(rng() % 70000) - 2;
    const int n = (int)(rng() % 13000) - 2, k = (int)(rng() % 13000) - 2;
    const int ep = (int)(rng() % 5) - 1;
    int st = tg_gemm_bf16(ep, kFake, k, kFake, k, m, n, k, kFake, n, kFake, n, nullptr);
    expect(error_before_launch(st) || st == TG_OK, "gemm", st);
    st = tg_rmsnorm_bf16(kFake, n, m, n, kFake, 1e-6f, kFake, n, nullptr);
    expect(error_before_launch(st) || st == TG_OK, "rmsnorm", st);
    const int hq = 1 + (int)(rng() % 64), hkv = 1 + (int)(rng() % 16), dh = 32 << (rng() % 3);
    st = tg_rope_split_bf16(kFake, (int64_t)(hq + 2 * hkv) * dh, m, hq, hkv, dh, (const int32_t*)kFake, 1e6f, kFake,
                            kFake, kFake, nullptr);
    expect(error_before_launch(st) || st == TG_OK, "rope", st);
    const int batch = (int)(rng() % 300) - 2;
    const int64_t rows = (int64_t)(rng() % 300000) - 2;
    const size_t dw = tg_decode_workspace_bytes(batch, hq, dh, rows);
    int32_t* lens = new int32_t[batch > 0 ? batch : 1];
    for (int b = 0; b < (batch > 0 ? batch : 1); ++b) lens[b] = (int32_t)(rng() % 1000);
    st = tg_gated_attention_decode(kFake, kFake, kFake, nullptr, nullptr, 0, nullptr, lens, batch, rows, hq, hkv, dh,
                                   kFake, dw ? kFake : nullptr, dw, nullptr);
    expect(error_before_launch(st) || st == TG_OK, "decode", st);
    delete[] lens;
    const size_t pw = tg_gate_packed_w1_bytes(n, k);
    st = tg_gate_pack_w1(kFake, n, k, pw ? kFake : nullptr, nullptr);
    expect(error_before_launch(st) || st == TG_OK, "pack w1", st);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 300;
  std::mt19937_64 rng(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1);
  for (int s = -8; s <= 2; ++s) expect(tg_status_string(s) != nullptr, "status string", s);
  expect(tg_abi_version() == TG_ABI_VERSION, "abi version");
  expect(tg_kept_count(10, 3, 4) == 7 && tg_kept_count(10, 3, 40) == 13 && tg_kept_count(-1, 0, 0) == -1 &&
             tg_kept_count(INT64_MAX / 4, INT64_MAX / 4, INT64_MAX) == INT64_MAX / 4 * 2,
         "kept count");
  for (long it = 0; it < iters; ++it) {
    const int n_seg = 1 + (int)(rng() % 40);
    const int max_len = it % 10 == 0 ? 140000 : (int)(rng() % 5000);
    Batch b = random_batch(rng, n_seg, max_len);
    tg_segment* table = nullptr;
    tg_plan_info info{};
    int st = plan(b, &table, &info);
    expect(st == TG_OK, "plan", st);
    if (st == TG_OK) {
      check_plan(b, table, info);
      exercise(table, &info, rng);  // the table pointer stands in for the device copy: never read on the host
    }
    delete[] table;
    // invalid batches: each must be rejected without reading past its arrays
    Batch bad = b;
    switch (it % 4) {
      case 0: bad.k[0] = -1; break;
      case 1: bad.doc_end[0] = bad.seg_start[1] - bad.seg_start[0] + 1; break;
      case 2: bad.seg_start[0] = 1; break;
      default: bad.doc_begin[0] = bad.doc_end[0] + 1; break;
    }
    st = plan(bad, &table, &info);
    expect(st == TG_ERR_INVALID_ARG, "plan rejects", it % 4, st);
    delete[] table;
  }
  compact_calls(rng);
  dense_calls(rng);
  // the status query validates its arguments first
  int word = 0;
  expect(tg_attention_workspace_status(nullptr, &word, nullptr) == TG_ERR_INVALID_ARG, "status null");
  expect(tg_attention_workspace_status(kFake, nullptr, nullptr) == TG_ERR_INVALID_ARG, "status out null");
  if (g_fail) {
    std::printf("%d failures\n", g_fail);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
