"""CPU oracle for blended prefill (CacheBlend-style selective KV recompute).

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package. The product path never calls
it, and it shares no code with the GPU library: it imports numpy and the seeded input
generators (``synth``) and nothing else of this repository.

It is written plainly and slowly, one step of the method after another, in fp32 numpy by
default (fp64 where a step says so, and fp64 throughout when asked), following:

* QCFuse: Query-Aware Cache Fusion via Compressed View for Efficient RAG Serving, §2.1
  (Table 1 notation; Eq. 2 full prefill, Eq. 3 per-chunk cache, Eq. 4 position remapping and
  stitching, Eq. 6 recompute ratio, Eq. 7 fused cache),
* CacheBlend: Reusing KV Caches When Your Text Isn't a Prefix, sections "Quantifying the
  Damage" (KV deviation, HKVD tokens), "Selective Recompute Without Skipping" (the per-layer
  blend pass) and "The Chicken-and-Egg Problem" (select once on an early layer, or narrow the
  set layer by layer: gradual filtering),
* Request Order Matters: Cache-History Sensitivity in Selective KV-Cache Reuse for Rolling
  Agents, §2.2 Eq. 1 (deviation), Eq. 2 (budget), §2.3 Eq. 3 (span score and the
  document-aligned policy), §4.1 (rolling window).
"""
from .model import (rms_norm, rope, rope_angles, causal_attention, layer_rows, full_prefill, bf16_round,
                    chunk_prefill, k_rows, kv_rows, attention_at, layer_rows_over)
from .blend import (budget, reposition, stitch, kv_deviation, select_topk, select_doc_spans,
                    blend_prefill, direct_reuse, RollingWindow, BlendResult, narrow, gradual_schedule,
                    loading_ratio, single_window_bounds, fixed_chunk_bounds, select_ranked_spans,
                    select_span_heads, selection_stats, query_attention_mass, query_scores, anchor_count,
                    key_norms, select_anchors, anchored_query_scores)

__all__ = [
    "bf16_round", "rms_norm", "rope", "rope_angles", "causal_attention", "layer_rows", "full_prefill", "k_rows",
    "kv_rows", "attention_at", "layer_rows_over",
    "chunk_prefill", "budget", "reposition", "stitch", "kv_deviation", "select_topk",
    "select_doc_spans", "blend_prefill", "direct_reuse", "RollingWindow", "BlendResult", "narrow",
    "gradual_schedule", "loading_ratio", "single_window_bounds", "fixed_chunk_bounds",
    "select_ranked_spans", "select_span_heads", "selection_stats", "query_attention_mass", "query_scores",
    "anchor_count", "key_norms", "select_anchors", "anchored_query_scores",
]
