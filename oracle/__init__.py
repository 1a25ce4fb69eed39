"""CPU oracle for TokenGate's pruned prefill -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy code that states what the hot path computes, step
by step, in the order and notation of the TokenGate write-ups.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it.
The HIP library never calls into it and shares no code with it.

Sources, cited by page title and section throughout:

* [reading]  "TokenGate 与 T2Quant：LLM/DLM 推理效率双子星 精读"
  (inkeast.github.io paper reading), section 4.1 (three-stage forward,
  component one: gate module; component two: token-gated attention).
* [insight]  kg.zhiyong.dev insight article on TokenGate ("把机制串起来").
* [news]     news.farwalk.ai translation of the MarkTechPost article
  "斯坦福与 UC Berkeley 提出 TokenGate ..." (sections "TokenGate 的可学习 token
  剪枝如何工作？", "什么是 token 门控注意力？", "如何部署 TokenGate？").

Parity status of each function is recorded in its docstring ("pinned by").
"""

from .tokengate_ref import (  # noqa: F401
    gelu_erf,
    gate_raw_scores,
    sequence_rms_normalize,
    gate_scores,
    kept_count,
    select_doc_topk,
    select_doc_topk_by_rank,
    select_doc_topk_by_sort,
    kept_indices,
    compact_rows,
    gated_attention,
    softplus,
    query_temperature,
    gated_attention_decode,
    gated_attention_backward,
    attention_logsumexp,
)
from .stack_ref import (  # noqa: F401,E402
    round_bf16,
    rmsnorm,
    rope,
    silu,
    LayerWeights,
    decoder_layer,
    pruned_stack,
)
