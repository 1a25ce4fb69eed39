/*
 * tokengate.h -- C ABI of the TokenGate pruned-prefill hot path on AMD
 * Instinct MI355X (gfx950).
 *
 * TokenGate prunes the prompt inside the model: the layers below a gate layer
 * see every token; at the gate a small MLP scores every prunable (document)
 * token; the best K document tokens plus every non-prunable token
 * (instruction, question) form the kept set; the layers above the gate run on
 * the kept rows only, with token-gated attention.  Sources, cited by page and
 * section:
 *   [reading] "TokenGate 与 T2Quant：LLM/DLM 推理效率双子星 精读"
 *             (inkeast.github.io paper reading), sections 3.1 and 4.1;
 *   [news]    news.farwalk.ai translation of the MarkTechPost article on
 *             TokenGate, sections "TokenGate 的可学习 token 剪枝如何工作？",
 *             "什么是 token 门控注意力？" and "如何部署 TokenGate？".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every function returns a tg_status (0 = TG_OK, negative = error); no
 *   exception or abort crosses the ABI.  All arguments are validated before
 *   any kernel is launched; on error nothing is launched.
 * - Device pointers are plain HIP device addresses owned by the caller.  The
 *   library never allocates or frees device memory and never synchronises
 *   the stream: every launch is asynchronous on `stream` (a hipStream_t;
 *   NULL = the legacy default stream).  The one exception is
 *   tg_attention_workspace_status, whose purpose is to read a word back.
 * - Host pointers (marked "host") are read during the call only.
 * - bf16 tensors are IEEE bfloat16 bit patterns (uint16), row-major,
 *   token-major ([tokens, heads, head_dim]).  Scores and parameters are fp32.
 * - A packed batch of prompts ("segments") is described by a segment table
 *   built on the host with tg_plan_segments() and copied by the caller to the
 *   device; the host validates the table's totals (tg_plan_info) and sizes
 *   every grid and buffer from them, and the kernels read the device copy
 *   (the library cannot read it back without a synchronisation).  Each kernel
 *   clamps the fields of its entry into those totals (seg_start + seg_len <=
 *   n_tokens, seg_len <= max_seg_len, the document span inside the prompt and
 *   at most max_doc_len long, k_eff <= that length, kept_start + kept_len <=
 *   total_kept, kept_len <= max_kept_len), so a table that disagrees with its
 *   info gives wrong results, never an access outside the arrays; build it
 *   with tg_plan_segments, and pass the info returned with it.
 * - Results are deterministic: the same inputs give bit-identical outputs
 *   (fixed-order reductions, integer-only atomics).
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_ABI_VERSION 1

typedef enum tg_status {
  TG_OK = 0,
  TG_ERR_INVALID_ARG = -1, /* null pointer, negative size or budget, bad segment table */
  TG_ERR_UNSUPPORTED = -2, /* shape the kernels do not implement (see each function) */
  TG_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or smaller than required */
  TG_ERR_NO_DEVICE = -4,   /* no HIP device, or the current device is not gfx950 */
  TG_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed */
} tg_status;

/* Human-readable text of a status code (static storage). */
const char* tg_status_string(int status);

/* TG_ABI_VERSION of the library that was loaded. */
int tg_abi_version(void);

/* ------------------------------------------------------------------------ */
/* Segment table                                                             */
/* ------------------------------------------------------------------------ */

/* One prompt of a packed batch.  The prompt is x = [x_R, x_D]: a request and
 * a document that arrives with it ([reading] section 3.1); only the document
 * span [doc_begin, doc_end) is prunable, every other token is always kept
 * ([reading] section 4.1 component one; [news] "TokenGate 的可学习 token 剪枝如何
 * 工作？": the question is never pruned).  32 bytes, 4-byte aligned. */
typedef struct tg_segment {
  int32_t seg_start;  /* first token of the prompt in the packed token arrays */
  int32_t seg_len;    /* tokens in the prompt */
  int32_t doc_begin;  /* document span, relative to seg_start, 0 <= b <= e <= seg_len */
  int32_t doc_end;
  int32_t k_eff;      /* kept documents = min(K, doc_end - doc_begin) */
  int32_t kept_start; /* first row of this prompt in the compacted (kept) arrays */
  int32_t kept_len;   /* k_eff + seg_len - (doc_end - doc_begin) */
  int32_t reserved;   /* 0 */
} tg_segment;

/* Totals of a segment table, used on the host to size grids and buffers. */
typedef struct tg_plan_info {
  int64_t n_tokens;     /* sum of seg_len */
  int64_t total_kept;   /* sum of kept_len (= rows of every compacted array) */
  int32_t n_seg;
  int32_t max_seg_len;
  int32_t max_doc_len;
  int32_t max_kept_len;
} tg_plan_info;

/* Builds the segment table of a packed batch (host only, no GPU needed).
 *   seg_start [n_seg + 1] (host): prefix offsets, seg_start[0] = 0, non-decreasing.
 *   doc_begin, doc_end [n_seg] (host): document span of each prompt, relative.
 *   k_budget [n_seg] (host): document budget K ("max_kept_prefill_tokens",
 *     [news] "如何部署 TokenGate？"); K > document length keeps the whole
 *     document, K = 0 keeps only the non-document tokens, K < 0 is an error.
 *   table [n_seg] (host, out), info (host, out).
 * Errors: TG_ERR_INVALID_ARG for n_seg < 1, null pointers, a span outside its
 * prompt, a negative budget, or more than 2^31 - 1 tokens. */
int tg_plan_segments(int n_seg, const int32_t* seg_start, const int32_t* doc_begin, const int32_t* doc_end,
                     const int32_t* k_budget, tg_segment* table, tg_plan_info* info);

/* Kept rows of one prompt (host only): min(k, n_doc) + n_other, the size of
 * S = top-K(document) plus every non-document token ([reading] section 4.1;
 * the budget "max_kept_prefill_tokens", [news] "如何部署 TokenGate？").  It is
 * the kept_len that tg_plan_segments writes for the prompt.  Returns -1 for a
 * negative argument. */
int64_t tg_kept_count(int64_t n_doc, int64_t n_other, int64_t k);

/* ------------------------------------------------------------------------ */
/* (1) Gate score                                                            */
/* ------------------------------------------------------------------------ */

/* Device workspace (bytes) tg_gate_score needs for this plan and MLP shape
 * (per-tile sums of squares, and W1 re-ordered into MFMA fragment order). */
size_t tg_gate_workspace_bytes(const tg_plan_info* info, int d, int h);

/* Gate score of every token ([reading] section 4.1 component one): a small MLP
 * reads the hidden row x_j of every prunable token and outputs one scalar,
 *   r_j = w2 . GELU(W1 x_j + b1) + b2      (exact erf GELU),
 * the scores are RMS-normalised along each prompt's document,
 *   s_j = r_j / sqrt(mean_{j in doc} r_j^2 + rms_eps),
 * and every non-document token gets s_j = 0 exactly.
 *   x   bf16 [n_tokens, ld_x] (device): hidden rows; only the first d columns are read.
 *   w1  bf16 [h, d] (device, row-major); b1 fp32 [h] (device) or NULL (= 0);
 *   w2  fp32 [h] (device); b2 scalar.
 *   segs (device) / info (host): tg_plan_segments output.
 *   rms_eps: >= 0 normalises; < 0 skips the normalisation (s_j = r_j on the document).
 *   scores fp32 [n_tokens] (device, out): every token of every prompt is written.
 *   workspace (device, tg_gate_workspace_bytes(info, d, h), 256-byte aligned).
 * The first layer runs on bf16 MFMA with fp32 accumulation; GELU, the h -> 1
 * dot and the normalisation are fp32 (the sum of squares is accumulated in
 * fp64, in a fixed order).
 * Supported: d % 64 == 0, d <= 65536, h % 64 == 0, 64 <= h <= 256, ld_x >= d,
 * x and w1 16-byte aligned, ld_x % 8 == 0; otherwise TG_ERR_UNSUPPORTED. */
int tg_gate_score(const void* x, int64_t ld_x, int d, const void* w1, const float* b1, const float* w2, float b2,
                  int h, const tg_segment* segs, const tg_plan_info* info, float rms_eps, float* scores,
                  void* workspace, size_t workspace_bytes, void* stream);

/* The gate's first-layer weights are constant across calls, so their
 * re-ordering into MFMA fragment order (done inside every tg_gate_score call)
 * can be done once at load time instead:
 *   tg_gate_pack_w1: w1 bf16 [h, d] (device) -> w1_packed (device,
 *     tg_gate_packed_w1_bytes(d, h) bytes, 16-byte aligned), an opaque layout
 *     valid only for tg_gate_score_prepacked with the same d and h;
 *   tg_gate_score_prepacked: tg_gate_score with the packed weights (same
 *     results bit for bit, one launch fewer).  Same arguments, shapes and
 *     workspace otherwise. */
size_t tg_gate_packed_w1_bytes(int d, int h);
int tg_gate_pack_w1(const void* w1, int d, int h, void* w1_packed, void* stream);
int tg_gate_score_prepacked(const void* x, int64_t ld_x, int d, const void* w1_packed, const float* b1,
                            const float* w2, float b2, int h, const tg_segment* segs, const tg_plan_info* info,
                            float rms_eps, float* scores, void* workspace, size_t workspace_bytes, void* stream);

/* tg_gate_score_prepacked for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace, the same results
 * bit for bit.  The per-tile sums of squares go to a fixed scratch array
 * that the library holds on each GPU it runs on (512 KiB, until the process
 * ends); nothing is allocated or freed and no allocating routine is called.
 * The array holds n_seg x ceil(max_doc_len / 64) tiles at most,
 * tg_gate_noalloc_max_tiles() of them (65536: e.g. one prompt of 4M document
 * tokens, or 64 prompts of 64K); a plan needing more returns
 * TG_ERR_WORKSPACE.  All calls on one GPU share that array and nothing in it
 * needs to start at zero, but calls that overlap on one GPU (other streams,
 * other threads) race on it and must not be issued.  The first call on each
 * GPU looks up the address of that GPU's copy (with the GPU current). */
int tg_gate_score_prepacked_noalloc(const void* x, int64_t ld_x, int d, const void* w1_packed, const float* b1,
                                    const float* w2, float b2, int h, const tg_segment* segs,
                                    const tg_plan_info* info, float rms_eps, float* scores, void* stream);
size_t tg_gate_noalloc_max_tiles(void);

/* ------------------------------------------------------------------------ */
/* (2) Top-K select                                                          */
/* ------------------------------------------------------------------------ */

/* Device workspace (bytes) tg_select_topk needs for this plan: 0 when every
 * prompt has at most 16384 tokens (one workgroup per prompt keeps its state
 * on chip; workspace may then be NULL); otherwise room for the radix
 * histograms and per-slice counts of the multi-workgroup path (no initial
 * contents required). */
size_t tg_select_workspace_bytes(const tg_plan_info* info);

/* Kept set of every prompt, S = top-K(s_j over the document) ∪ (every
 * non-document token) ([reading] sections 3.1 and 4.1: |S ∩ P| = K).
 * Order among documents: higher score first; equal scores (IEEE equality, so
 * -0.0 == +0.0) go to the lower token index; NaN ranks below every number,
 * NaNs among themselves by index; +-inf are ordinary values.
 *   scores fp32 [n_tokens] (device).
 *   kept_idx int32 [info->total_kept] (device, out): global token indices,
 *     ascending; prompt i fills rows [kept_start, kept_start + kept_len).
 *   workspace (device, tg_select_workspace_bytes, 256-byte aligned; may be
 *     NULL when that size is 0).
 * Exact integer algorithm (radix select on order-preserving 32-bit keys,
 * then an index-ordered scan): identical results on every run.  One launch
 * with one workgroup per prompt up to 16384 tokens; longer prompts use six
 * launches over 512-token slices, or 4096-token slices when the batch has
 * enough of them to fill the GPU (integer atomics only). */
int tg_select_topk(const float* scores, const tg_segment* segs, const tg_plan_info* info, int32_t* kept_idx,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* (3) Compaction                                                            */
/* ------------------------------------------------------------------------ */

#define TG_COMPACT_MAX_TENSORS 8

/* Row gather of up to TG_COMPACT_MAX_TENSORS tensors in one launch:
 *   dst_t[r] = src_t[kept_idx[r]] for r < n_kept, row_bytes[t] bytes, bit-exact.
 * Pruned tokens never reach the layers above the gate, which create no KV
 * entries for them ([reading] section 4.1; [news] "剪枝前向").
 *   kept_idx int32 [n_kept] (device), each in [0, n_src_rows).  An index
 *     outside that range is a caller error; its row is skipped (dst row left
 *     as it was), never read out of bounds.
 *   n_src_rows: rows of every src tensor.
 *   src, dst [n_tensors] (host arrays of device pointers).
 *   row_bytes, src_stride, dst_stride [n_tensors] (host): bytes per row copied
 *     and the byte distance between rows; dst_stride >= row_bytes.
 * Rows are moved 16 bytes at a time when every pointer, stride and row size
 * of a tensor is a multiple of 16, else 4 bytes, else 1 byte.
 * src and dst of a tensor must not overlap.
 * Errors: TG_ERR_INVALID_ARG (null, negative sizes, dst_stride < row_bytes,
 * n_tensors outside 1..TG_COMPACT_MAX_TENSORS, src == dst). */
int tg_compact_kept(const int32_t* kept_idx, int64_t n_kept, int64_t n_src_rows, int n_tensors, const void* const* src,
                    void* const* dst, const int64_t* row_bytes, const int64_t* src_stride,
                    const int64_t* dst_stride, void* stream);

/* ------------------------------------------------------------------------ */
/* (4) Token-gated attention, prefill                                       */
/* ------------------------------------------------------------------------ */

/* Causal token-gated GQA attention over the kept rows of every prompt
 * ([reading] section 4.1 component two: the kept token's score enters the
 * attention logits as a bias, scaled by a per-(layer, head) gain, with a
 * temperature on q.k; [news] "什么是 token 门控注意力？").  For query head h,
 * key/value head c = h / (hq / hkv), kept rows r and t <= r of one prompt:
 *   z_rt = tau_h * (q_r . k_t) / sqrt(head_dim) + gain_h * s_t
 *   out[r, h] = sum_t softmax_t(z_r.) v_t
 *   q   bf16 [total_kept, hq, head_dim] (device, contiguous)
 *   k,v bf16 [total_kept, hkv, head_dim] (device, contiguous)
 *   key_score fp32 [total_kept] (device) or NULL (no bias)
 *   tau  fp32 [hq] (device) or NULL (= 1); gain fp32 [hq] (device) or NULL (no bias)
 *   segs (device) / info (host): rows of prompt i are [kept_start, kept_start + kept_len).
 *   out bf16 [total_kept, hq, head_dim] (device, out).
 * bf16 MFMA for q.k and p.v, fp32 softmax and accumulation; the softmax
 * denominator sums the bf16-rounded probabilities that the p.v product uses.
 * NaN anywhere in q, k, v, key_score, tau or gain gives unspecified output
 * values (no error); +-inf scores act as ordinary logit biases.
 * Supported: head_dim in {64, 128}; hq % hkv == 0 with hq / hkv in {1, 2, 4};
 * kept_len * hkv * head_dim * 2 < 2^32 - 256 for every prompt (32-bit buffer
 * ranges); all pointers 16-byte aligned; otherwise TG_ERR_UNSUPPORTED /
 * INVALID_ARG. */
int tg_gated_attention_prefill(const void* q, const void* k, const void* v, const float* key_score,
                               const float* tau, const float* gain, const tg_segment* segs,
                               const tg_plan_info* info, int hq, int hkv, int head_dim, void* out, void* stream);

/* tg_gated_attention_prefill with a workspace that lets the library split
 * the longest query tiles of a prompt over two workgroups when the prompt is
 * too short to fill the GPU (one prompt whose query tiles are few against the
 * CUs per KV head).  Each half publishes its partial softmax state (running
 * maximum, denominator, unnormalised output) to the workspace and the second
 * half to finish merges both; the merge is symmetric, so results are
 * deterministic.  Output: as tg_gated_attention_prefill up to fp32 rounding
 * of the merge (within the same tolerance against exact arithmetic).
 *   workspace: device, 256-byte aligned, at least
 *     tg_attention_prefill_workspace_bytes(info, hq, hkv, head_dim) bytes,
 *     zero-filled before its first use; every call leaves it reusable (its
 *     counters back at zero).  Calls sharing a workspace must not overlap (use
 *     one stream).  When the size is 0 no tile is split and workspace may be NULL.
 *   The second half waits for the first half's record a bounded time (2^22
 *   polls, each a load that bypasses the L2 plus a short sleep: 134 ns per
 *   poll measured on MI355X, so about 0.56 s; a workgroup that has already
 *   started only has to store its record, so the wait normally takes
 *   microseconds).  The first 4 bytes of
 *   the workspace are a status word, 0 while the workspace is consistent.
 *   Should the wait ever run out (the first half stalled, e.g. preempted), or
 *   should a call find a tile's counters already set when it starts (a
 *   workspace that was not zero-filled, or left by such a failed call, or
 *   shared by calls that overlapped), the rows of that tile are written as
 *   NaN (and NaN log-sum-exp) instead of a merge of a stale record, the status
 *   word gets bit 1 (counters already set) or bit 2 (wait ran out), and the
 *   counters are left as they are, so every later call reports the same until
 *   the caller zero-fills the workspace.  tg_attention_workspace_status reads
 *   the word.
 * Errors as tg_gated_attention_prefill, and TG_ERR_WORKSPACE when the
 * workspace is missing, misaligned or too small. */
size_t tg_attention_prefill_workspace_bytes(const tg_plan_info* info, int hq, int hkv, int head_dim);

/* Status word of a split-tile attention workspace (see above): *status = 0
 * when every call on it merged normally; otherwise bit 1 (a call found
 * counters already set) and/or bit 2 (a wait ran out), and the outputs of
 * those calls hold NaN rows.  Unlike every other entry point this one
 * synchronises `stream` (it copies the word to the host after the work
 * queued there).  workspace: device, 256-byte aligned, non-NULL; status: host.
 * Errors: TG_ERR_INVALID_ARG, TG_ERR_NO_DEVICE, TG_ERR_HIP. */
int tg_attention_workspace_status(const void* workspace, int* status, void* stream);
int tg_gated_attention_prefill_ws(const void* q, const void* k, const void* v, const float* key_score,
                                  const float* tau, const float* gain, const tg_segment* segs,
                                  const tg_plan_info* info, int hq, int hkv, int head_dim, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* The same attention reading the kept rows where they are (gather on load)
 * instead of from compacted copies: q [n_src_rows, hq, head_dim], k and v
 * [n_src_rows, hkv, head_dim] (bf16, device) and key_score [n_src_rows]
 * (fp32, device, or NULL) hold every token, and kept row r of prompt i is
 * source row kept_idx[kept_start_i + r] (int32 [info->total_kept], device,
 * as tg_select_topk writes it).  The output is compacted exactly as above:
 * out [info->total_kept, hq, head_dim].  The compaction step then only has to
 * move the rows the next layer needs (hidden state, scores), not Q, K and V.
 * An index outside [0, n_src_rows) is a caller error: its K/V row and score
 * read as zeros and its Q row as row 0 (no access outside the arrays).
 * Supported in addition: at most 16384 kept rows per prompt and
 * n_src_rows * hkv * head_dim * 2 < 2^32 (else TG_ERR_UNSUPPORTED). */
int tg_gated_attention_prefill_gather(const void* q, const void* k, const void* v, const float* key_score,
                                      const float* tau, const float* gain, const tg_segment* segs,
                                      const tg_plan_info* info, int hq, int hkv, int head_dim,
                                      const int32_t* kept_idx, int64_t n_src_rows, void* out, void* stream);
/* tg_gated_attention_prefill_gather with the split-tile workspace of
 * tg_gated_attention_prefill_ws (same sizing, zero-fill, reuse and error
 * rules; outputs equal to the gather call up to fp32 rounding of the merge). */
int tg_gated_attention_prefill_gather_ws(const void* q, const void* k, const void* v, const float* key_score,
                                         const float* tau, const float* gain, const tg_segment* segs,
                                         const tg_plan_info* info, int hq, int hkv, int head_dim,
                                         const int32_t* kept_idx, int64_t n_src_rows, void* out, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* The same attention with a temperature per query row ([reading] section 4.1
 * component two, second refinement: pruning shrinks the keys a query sees
 * from its original position to its rank among the kept tokens, and a
 * learnable temperature recalibrates the sharpened softmax).  For kept row r
 * (0-based inside its prompt) with original 0-based position positions[r]:
 *   tau_rh = softplus(sigma_h) * log(r + 1) / log(max(2, positions[r] + 1))
 *   z_rt = tau_rh * (q_r . k_t) / sqrt(head_dim) + gain_h * s_t
 * (the bias is not scaled by the temperature).
 *   sigma     fp32 [hq] (device, required): softplus(sigma_h) is the head's scale
 *   positions int32 [total_kept] (device): original position of every kept row
 *             inside its prompt, in kept order (what tg_compact_kept makes of
 *             the per-token positions); a value below 1 counts as 1
 * Everything else, the precision and the supported shapes are as for
 * tg_gated_attention_prefill.  NULL sigma, or NULL positions with kept rows,
 * is TG_ERR_INVALID_ARG. */
int tg_gated_attention_prefill_query_tau(const void* q, const void* k, const void* v, const float* key_score,
                                         const float* sigma, const float* gain, const int32_t* positions,
                                         const tg_segment* segs, const tg_plan_info* info, int hq, int hkv,
                                         int head_dim, void* out, void* stream);
/* tg_gated_attention_prefill_query_tau with the split-tile workspace of
 * tg_gated_attention_prefill_ws (same sizing, zero-fill, reuse and error
 * rules). */
int tg_gated_attention_prefill_query_tau_ws(const void* q, const void* k, const void* v, const float* key_score,
                                            const float* sigma, const float* gain, const int32_t* positions,
                                            const tg_segment* segs, const tg_plan_info* info, int hq, int hkv,
                                            int head_dim, void* out, void* workspace, size_t workspace_bytes,
                                            void* stream);

/* ------------------------------------------------------------------------ */
/* (4a) Token-gated attention, backward                                     */
/* ------------------------------------------------------------------------ */

/* The forward of tg_gated_attention_prefill that also writes the natural-log
 * log-sum-exp of every row's logits, lse[r * hq + h] = ln sum_t exp(z_rt)
 * (fp32 [total_kept, hq], device), which the backward needs. */
int tg_gated_attention_prefill_lse(const void* q, const void* k, const void* v, const float* key_score,
                                   const float* tau, const float* gain, const tg_segment* segs,
                                   const tg_plan_info* info, int hq, int hkv, int head_dim, void* out, float* lse,
                                   void* stream);

/* Gradients of tg_gated_attention_prefill ([reading] section 4.1,
 * engineering notes: the biased attention kernel runs backwards too and
 * carries the bias gradient back into the gate's scorer).  With P the
 * attention weights and dout [total_kept, hq, head_dim] (bf16) the upstream
 * gradient of out:
 *   dv = P^T dout, dZ = P o (dout v^T - rowsum(dout o out)),
 *   dq = tau_h / sqrt(D) dZ k,  dk = tau_h / sqrt(D) dZ^T q  (dk, dv summed over
 *   the hq / hkv heads sharing a KV head),
 *   ds_t = sum_h gain_h sum_r dZ_rt  (the key-score gradient, to the scorer),
 *   dgain_h = sum dZ_rt s_t,  dtau_h = sum dZ_rt (q_r . k_t) / sqrt(D).
 * Inputs as for the forward, plus out (its bf16 output) and lse (from
 * tg_gated_attention_prefill_lse).  Outputs, all fp32 and overwritten:
 *   dq [total_kept, hq, head_dim], dk and dv [total_kept, hkv, head_dim] (16-byte aligned);
 *   ds [total_kept], dgain [hq], dtau [hq]: each may be NULL (not written);
 *   without a bias (key_score or gain NULL) ds and dgain come out 0.
 * workspace: device, 16-byte aligned, >= tg_attention_backward_workspace_bytes
 *   (row terms, and fp32 dk / dv / ds partials of up to five query chunks).
 * bf16 MFMA products (P and the scaled dZ rounded to bf16), fp32
 * accumulation; results are deterministic.  Shapes as for the forward. */
size_t tg_attention_backward_workspace_bytes(const tg_plan_info* info, int hq, int hkv, int head_dim);
int tg_gated_attention_backward(const void* q, const void* k, const void* v, const float* key_score,
                                const float* tau, const float* gain, const tg_segment* segs,
                                const tg_plan_info* info, int hq, int hkv, int head_dim, const void* out,
                                const void* dout, const float* lse, float* dq, float* dk, float* dv, float* ds,
                                float* dgain, float* dtau, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* (4b) Token-gated attention, one decode step over a pruned KV cache        */
/* ------------------------------------------------------------------------ */

/* [reading] section 4.1: pruned tokens leave no KV entry, and the tokens
 * being generated are not prunable (score 0); the engineering notes of the
 * same section fold the gate term into an additive attention mask at decode
 * time.  Sequence b's new query attends to its cache rows j < lens[b] (its
 * own K/V row appended by the caller beforehand):
 *   z_j = tau_h * (q_h . k_j) / sqrt(head_dim) + gain_h * s_j
 *   out[b, h] = sum_j softmax_j(z) v_j          (0 when lens[b] == 0)
 *   q        bf16 [batch, hq, head_dim] (device)
 *   k_cache, v_cache bf16 [batch, cache_rows, hkv, head_dim] (device, contiguous)
 *   key_score fp32 [batch, cache_rows] (device) or NULL (no mask); 0 for
 *             generated and question rows
 *   tau      fp32 [hq] (tau_per_query = 0), [batch, hq] (tau_per_query = 1:
 *            a temperature per query, e.g. the per-query form of
 *            tg_gated_attention_prefill_query_tau evaluated on the host) or NULL (= 1)
 *   gain     fp32 [hq] (device) or NULL (no mask)
 *   lens     int32 [batch] (device): valid rows; values outside [0, cache_rows]
 *            are clamped into it (no access outside the caches)
 *   out      bf16 [batch, hq, head_dim] (device, out)
 *   workspace: device, 16-byte aligned, >= tg_decode_workspace_bytes(...)
 *            (split-KV partials; no state is kept between calls)
 * fp32 arithmetic on bf16 inputs; the key scores must be finite.
 * Supported: head_dim in {64, 128}, hq / hkv in {1, 2, 4}, batch and hkv at
 * most 65535, cache_rows at most 65535 * 256 (else TG_ERR_UNSUPPORTED). */
size_t tg_decode_workspace_bytes(int batch, int hq, int head_dim, int64_t cache_rows);
int tg_gated_attention_decode(const void* q, const void* k_cache, const void* v_cache, const float* key_score,
                              const float* tau, int tau_per_query, const float* gain, const int32_t* lens,
                              int batch, int64_t cache_rows, int hq, int hkv, int head_dim, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* (5) Dense decoder-layer support (the layers below and above the gate)    */
/* ------------------------------------------------------------------------ */

/* The layers below the gate process every token; the layers above it process
 * only the kept tokens ([reading] section 4.1: three-stage forward).  These
 * entry points run a Qwen3-shaped pre-norm decoder layer so the whole pruned
 * prefill can run on this library:
 *   h = x + Wo . Attn(RoPE(Wqkv . RMSNorm(x)))      (token-gated above the gate)
 *   y = h + Wdown . (silu(Wgate . RMSNorm(h)) * (Wup . RMSNorm(h)))
 * bf16 tensors, fp32 accumulation; every tensor between two steps is bf16. */

#define TG_GEMM_STORE 0    /* y = x . w^T */
#define TG_GEMM_RESIDUAL 1 /* y = x . w^T + residual (residual may be y itself) */
#define TG_GEMM_SWIGLU 2   /* w rows interleaved in groups of 8: gate 8j..8j+7, then up 8j..8j+7;
                              y[:, c] = silu(gate_c) * up_c, n / 2 output columns */

/* y [m, n] (or [m, n / 2] for SWIGLU) = x [m, k] . w [n, k]^T with the chosen
 * epilogue; row strides ldx, ldw, ldr, ldy in elements.  All bf16, device.
 * Supported: n % 128 == 0, k % 64 == 0, row strides % 8 == 0, 16-byte aligned
 * pointers; otherwise TG_ERR_UNSUPPORTED.  m may be any size >= 0. */
int tg_gemm_bf16(int epilogue, const void* x, int64_t ldx, const void* w, int64_t ldw, int64_t m, int n, int k,
                 const void* residual, int64_t ldr, void* y, int64_t ldy, void* stream);

/* y = x / sqrt(mean(x^2) + eps) * weight per row (fp32 math).  x, y bf16 [m, d]
 * (row strides ldx, ldy), weight bf16 [d].  d % 8 == 0. */
int tg_rmsnorm_bf16(const void* x, int64_t ldx, int64_t m, int d, const void* weight, float eps, void* y, int64_t ldy,
                    void* stream);

/* Splits a fused QKV row [q (hq heads) | k (hkv heads) | v (hkv heads)] x head_dim
 * into token-major q [m, hq, head_dim], k, v [m, hkv, head_dim], applying the
 * rotate-half rotary embedding to q and k at position positions[r] (int32,
 * device): pair (i, i + head_dim/2) rotates by positions[r] * theta^(-2i/head_dim)
 * (angle and its sine/cosine in fp64).  Above the gate the positions are the
 * original token positions of the kept rows. */
int tg_rope_split_bf16(const void* qkv, int64_t ldqkv, int64_t m, int hq, int hkv, int head_dim,
                       const int32_t* positions, float theta, void* q, void* k, void* v, void* stream);

/* Weights of one decoder layer (device pointers, bf16 unless noted). */
typedef struct tg_layer_weights {
  const void* attn_norm; /* [d] */
  const void* wqkv;      /* [(hq + 2 hkv) head_dim, d] */
  const void* wo;        /* [d, hq head_dim] */
  const void* mlp_norm;  /* [d] */
  const void* w_gate_up; /* [2 f, d], gate/up rows interleaved in groups of 8 (TG_GEMM_SWIGLU) */
  const void* w_down;    /* [d, f] */
  const float* tau;      /* fp32 [hq] temperature, or NULL (= 1) */
  const float* gain;     /* fp32 [hq] gate gain, or NULL (no bias) */
} tg_layer_weights;

/* Device workspace (bytes) of tg_decoder_layer for m rows. */
size_t tg_decoder_layer_workspace_bytes(int64_t m, int d, int hq, int hkv, int head_dim, int f);

/* One decoder layer over the rows described by segs / info (kept rows of every
 * prompt: kept_start, kept_len; below the gate plan with K >= document length
 * so that every token is a kept row).  hidden bf16 [total_kept, d] is updated
 * in place.  positions int32 [total_kept] (device): RoPE positions.
 * key_score fp32 [total_kept] or NULL: the gate scores of the kept rows (the
 * attention bias, with w->gain).  post_attn_norm bf16 [total_kept, d] or NULL:
 * if given, receives RMSNorm(h) (the MLP input, the tensor the gate reads).
 * Supported: d % 128 == 0, f % 64 == 0, head_dim 64 or 128, hq / hkv in
 * {1, 2, 4}, (hq + 2 hkv) head_dim % 128 == 0, hq head_dim % 64 == 0. */
int tg_decoder_layer(void* hidden, const int32_t* positions, const float* key_score, const tg_segment* segs,
                     const tg_plan_info* info, int d, int hq, int hkv, int head_dim, int f, float rms_eps,
                     float rope_theta, const tg_layer_weights* w, void* post_attn_norm, void* workspace,
                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_H */
