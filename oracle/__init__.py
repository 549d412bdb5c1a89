"""CPU oracle of the token-skipping step. TEST INFRASTRUCTURE ONLY.

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg; the HIP
library never routes through it.

The names exported here are the C++17 oracle (oracle/dllm_oracle.cpp, float64, std::thread over
rows, its own bfloat16 decoding and rounding) through its ctypes binding (oracle/cpp.py).
`oracle.numpy_ref` is the float64 numpy oracle written first (oracle/dllm_ref.py): a second,
independently written checker that the pins run against as well.
"""
from . import dllm_ref as numpy_ref
from .cpp import (DELTA_COS, DELTA_L1N, DELTA_L2R, SEL_THRESHOLD, SEL_TOPK, as_f64, commit_step,
                  confidence_argmax, context_all, decode_bf16, delta_variation, dense_layer,
                  embed_rows, flags_from_rows, gather_ffn_scatter, gather_kv_rows,
                  gather_qkv_scatter_kv, max_softmax_confidence, partial_attn, rms_norm,
                  round_bf16, salient_attention, saliency, select_compact, selected_layer,
                  set_threads, silu, threads)

__all__ = [
    "DELTA_COS", "DELTA_L1N", "DELTA_L2R", "SEL_THRESHOLD", "SEL_TOPK", "as_f64", "commit_step",
    "confidence_argmax", "context_all", "decode_bf16", "delta_variation", "dense_layer",
    "embed_rows", "flags_from_rows", "gather_ffn_scatter", "gather_kv_rows",
    "gather_qkv_scatter_kv", "max_softmax_confidence", "numpy_ref", "partial_attn", "rms_norm",
    "round_bf16", "salient_attention", "saliency", "select_compact", "selected_layer",
    "set_threads", "silu", "threads",
]
