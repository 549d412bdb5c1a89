"""Seeded input recipes of the five synthetic workloads (shapes + value distributions only).

  tiny_f32      : fp32, B=1, S=64 (32 prompt + 32 masked), d=256, 4 heads x 64, FFN 1024;
                  16 of 64 tokens perturbed by N(0, 0.5^2), the rest by N(0, (1e-3)^2); no logits.
  llada_layer   : bf16, one LLaDA-8B-shaped layer, B=1, S=1024 (512 + 512), d=4096,
                  32 heads x 128 (MHA), FFN 12288, vocab 126464; 154 of 1024 tokens (15%) get
                  N(0, 0.5^2) deltas, 870 get N(0, (1e-3)^2); logits N(0, 3^2); top-128.
  llada_step    : bf16, 32 LLaDA-8B layers, B=8, S=1024, early skip at layer 4, top-205 per
                  sequence (~20%), perturbation as llada_layer, cumulative across 16 steps.
  llada_long    : bf16, B=1, S=4096 (3584 prompt + 16 blocks of 32), 32 LLaDA-8B layers; the
                  active block is forced, 64 other positions chosen by delta.
  dream_gqa     : bf16, Dream-7B shape, B=16, S=2048, d=3584, 28 query / 4 kv heads x 128,
                  FFN 18944, 28 layers; selected fraction 5/10/25/50%.

These stand in for the pages' evaluation runs (trained weights and benchmark suites are not
available): weights are random N(0, 0.02^2), hidden states N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import layer_weights, logits as draw_logits, perturbed_pair


@dataclass(frozen=True)
class Dims:
    B: int
    S: int
    d: int
    H: int
    Hkv: int
    hd: int
    F: int
    V: int = 0
    dtype: torch.dtype = torch.bfloat16


TINY_F32 = Dims(B=1, S=64, d=256, H=4, Hkv=4, hd=64, F=1024, V=0, dtype=torch.float32)
LLADA_LAYER = Dims(B=1, S=1024, d=4096, H=32, Hkv=32, hd=128, F=12288, V=126464)
LLADA_STEP = Dims(B=8, S=1024, d=4096, H=32, Hkv=32, hd=128, F=12288, V=126464)
LLADA_LONG = Dims(B=1, S=4096, d=4096, H=32, Hkv=32, hd=128, F=12288, V=126464)
DREAM_GQA = Dims(B=16, S=2048, d=3584, H=28, Hkv=4, hd=128, F=18944, V=0)

TINY_LARGE = 16      # 25% of 64
LLADA_LARGE = 154    # round(0.15 * 1024)
LLADA_TOPK = 128
STEP_TOPK = 205      # round(0.2 * 1024)
STEP_SKIP = 4        # L / 8 for L = 32


def layer_inputs(dims: Dims, n_large: int, seed: int, device="cpu", with_logits=True):
    """(h_prev, h_cur, large_mask, logits or None, weights) of one single-layer workload."""
    h_prev, h_cur, large = perturbed_pair(dims.B, dims.S, dims.d, n_large, seed=seed,
                                          dtype=dims.dtype, device=device)
    lg = None
    if with_logits and dims.V:
        lg = draw_logits(dims.B, dims.S, dims.V, seed=seed * 7 + 3, dtype=dims.dtype,
                         device=device)
    w = layer_weights(dims.d, dims.H, dims.Hkv, dims.hd, dims.F, seed=seed * 11 + 5,
                      dtype=dims.dtype, device=device)
    return h_prev, h_cur, large, lg, w
