"""CPU float64 oracle of the token-skipping step. Test infrastructure only.

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg.
"""
from .dllm_ref import (DELTA_COS, DELTA_L1N, DELTA_L2R, SEL_THRESHOLD, SEL_TOPK, as_f64,
                       commit_step, confidence_argmax, context_all, decode_bf16, delta_variation,
                       dense_layer, embed_rows, flags_from_rows, gather_ffn_scatter,
                       gather_kv_rows, gather_qkv_scatter_kv, max_softmax_confidence, partial_attn,
                       rms_norm, salient_attention, saliency, select_compact, selected_layer,
                       silu)

__all__ = [
    "DELTA_COS", "DELTA_L1N", "DELTA_L2R", "SEL_THRESHOLD", "SEL_TOPK", "as_f64", "commit_step",
    "confidence_argmax", "context_all", "embed_rows", "flags_from_rows",
    "decode_bf16", "delta_variation", "dense_layer", "gather_ffn_scatter", "gather_kv_rows",
    "gather_qkv_scatter_kv", "max_softmax_confidence", "partial_attn", "rms_norm",
    "salient_attention", "saliency", "select_compact", "selected_layer", "silu",
]
