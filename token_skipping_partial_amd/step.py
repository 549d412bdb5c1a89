"""Step drivers over the five library calls: buffer plumbing only, no arithmetic.

A selected layer is qkv+scatter -> partial attention -> ffn+scatter on the rows that
`dllm_select_compact` produced. A single-layer step (the LLaDA-8B-shaped layer workload) is
saliency -> selection -> one selected layer. A multi-layer early-skip step runs layers below the
skip layer on every token, scores tokens at the skip layer, selects once, and runs the remaining
layers on the selected rows against the cached K/V (ES-dLLM, German summary page §2.B: skipping
at early layers such as 1/8 of the depth; the selection is reused by the layers above it).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

from . import (OP_ATTN, OP_FFN, OP_QKV, SEL_THRESHOLD, SEL_TOPK, Shape, dllm_gather_ffn_scatter,
               dllm_gather_qkv_scatter_kv, dllm_partial_attn, dllm_saliency,
               dllm_select_compact, workspace)


@dataclass
class LayerWeights:
    g_attn: torch.Tensor
    w_qkv: torch.Tensor
    w_o: torch.Tensor
    g_ffn: torch.Tensor
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor

    @classmethod
    def from_dict(cls, d: dict, device="cuda"):
        return cls(**{k: d[k].to(device).contiguous() for k in
                      ("g_attn", "w_qkv", "w_o", "g_ffn", "w_gate", "w_up", "w_down")})


@dataclass
class LayerScratch:
    """Per-(shape, m_cap) buffers of one selected layer: q_sel, o_sel and three workspaces."""
    shape: Shape
    m_cap: int
    device: str = "cuda"
    q_sel: torch.Tensor = field(init=False)
    o_sel: torch.Tensor = field(init=False)
    ws_qkv: torch.Tensor = field(init=False)
    ws_attn: torch.Tensor = field(init=False)
    ws_ffn: torch.Tensor = field(init=False)

    def __post_init__(self):
        s, dt = self.shape, self.shape.torch_dtype
        rows = max(1, self.m_cap)
        self.q_sel = torch.empty(rows, s.H * s.hd, dtype=dt, device=self.device)
        self.o_sel = torch.empty(rows, s.H * s.hd, dtype=dt, device=self.device)
        self.ws_qkv = workspace(OP_QKV, s, self.m_cap, self.device)
        self.ws_attn = workspace(OP_ATTN, s, self.m_cap, self.device)
        self.ws_ffn = workspace(OP_FFN, s, self.m_cap, self.device)


def attn_scale(shape: Shape) -> float:
    return 1.0 / math.sqrt(shape.hd)


def selected_layer(shape: Shape, w: LayerWeights, h_in, k_cache, v_cache, h_out, sel_idx, row_ptr,
                   scratch: LayerScratch, stream=None):
    """qkv + K/V scatter, partial attention, FFN + hidden scatter for the selected rows."""
    m = scratch.m_cap
    dllm_gather_qkv_scatter_kv(shape, h_in, w.g_attn, w.w_qkv, sel_idx, row_ptr, m,
                               scratch.q_sel, k_cache, v_cache, scratch.ws_qkv, stream)
    dllm_partial_attn(shape, attn_scale(shape), scratch.q_sel, k_cache, v_cache, sel_idx, row_ptr,
                      m, scratch.o_sel, scratch.ws_attn, stream)
    dllm_gather_ffn_scatter(shape, h_in, scratch.o_sel, w.w_o, w.g_ffn, w.w_gate, w.w_up,
                            w.w_down, sel_idx, row_ptr, m, h_out, scratch.ws_ffn, stream)


def all_rows(shape: Shape, device="cuda"):
    """Selection of every position: sel_idx = 0..B*S-1, row_ptr = 0, S, 2S, ..."""
    sel = torch.arange(shape.B * shape.S, dtype=torch.int32, device=device)
    rp = torch.arange(0, shape.B * shape.S + 1, shape.S, dtype=torch.int32, device=device)
    return sel, rp


@dataclass
class SelectConfig:
    mode: int = SEL_TOPK
    k: int = 0
    tau: float = 0.0
    alpha: float = 0.5
    delta_kind: int = 0


class SingleLayerStep:
    """saliency -> select -> selected layer, with every buffer preallocated.

    Inputs of one call: h_cur/h_prev [B,S,d], logits [B,S,V] or None, layer weights, the layer's
    K/V caches and hidden-state output (updated in place on the selected rows).
    """

    def __init__(self, shape: Shape, sel: SelectConfig, m_cap: int, device="cuda"):
        self.shape, self.sel, self.m_cap = shape, sel, m_cap
        B, S = shape.B, shape.S
        self.score = torch.empty(B, S, dtype=torch.float32, device=device)
        self.sel_idx = torch.empty(B * S, dtype=torch.int32, device=device)
        self.row_ptr = torch.empty(B + 1, dtype=torch.int32, device=device)
        self.scratch = LayerScratch(shape, m_cap, device)

    def score_and_select(self, h_cur, h_prev, logits, force=None, stream=None):
        c = self.sel
        dllm_saliency(self.shape, c.delta_kind, c.alpha, h_cur, h_prev, logits, self.score,
                      stream=stream)
        dllm_select_compact(self.shape, c.mode, c.tau, c.k, self.score, force, self.sel_idx,
                            self.row_ptr, stream=stream)

    def __call__(self, w: LayerWeights, h_cur, h_prev, logits, k_cache, v_cache, h_out,
                 force=None, stream=None):
        self.score_and_select(h_cur, h_prev, logits, force, stream)
        selected_layer(self.shape, w, h_cur, k_cache, v_cache, h_out, self.sel_idx, self.row_ptr,
                       self.scratch, stream)


class EarlySkipModel:
    """L-layer early-skip step with per-layer K/V caches and per-boundary hidden-state caches.

    hidden[l] is the input of layer l (hidden[0] = embeddings); layer l writes hidden[l + 1].
    Layers [0, skip) run on every token; the saliency of hidden[skip] against its value at the
    previous step picks the rows for layers [skip, L).
    """

    def __init__(self, shape: Shape, layers: list, skip: int, sel: SelectConfig, m_cap: int,
                 device="cuda"):
        self.shape, self.layers, self.skip, self.sel, self.m_cap = shape, layers, skip, sel, m_cap
        B, S, d, Hkv, hd = shape.B, shape.S, shape.d, shape.Hkv, shape.hd
        dt = shape.torch_dtype
        L = len(layers)
        self.k = [torch.zeros(B, Hkv, S, hd, dtype=dt, device=device) for _ in range(L)]
        self.v = [torch.zeros(B, Hkv, S, hd, dtype=dt, device=device) for _ in range(L)]
        self.hidden = [torch.zeros(B, S, d, dtype=dt, device=device) for _ in range(L + 1)]
        self.h_ref = torch.zeros(B, S, d, dtype=dt, device=device)  # hidden[skip] at step t-1
        self.all_sel, self.all_rp = all_rows(shape, device)
        self.dense = LayerScratch(shape, B * S, device)
        self.step1 = SingleLayerStep(shape, sel, m_cap, device)  # score/select buffers
        self.sparse = self.step1.scratch

    def fill(self, x0, stream=None):
        """Step 0: every layer on every token; primes caches and the skip-layer reference."""
        self.hidden[0].copy_(x0)
        for l, w in enumerate(self.layers):
            selected_layer(self.shape, w, self.hidden[l], self.k[l], self.v[l], self.hidden[l + 1],
                           self.all_sel, self.all_rp, self.dense, stream)
        self.h_ref.copy_(self.hidden[self.skip])

    def step(self, x, logits=None, force=None, stream=None):
        self.hidden[0].copy_(x)
        for l in range(self.skip):
            selected_layer(self.shape, self.layers[l], self.hidden[l], self.k[l], self.v[l],
                           self.hidden[l + 1], self.all_sel, self.all_rp, self.dense, stream)
        s = self.step1
        s.score_and_select(self.hidden[self.skip], self.h_ref, logits, force, stream)
        self.h_ref.copy_(self.hidden[self.skip])
        for l in range(self.skip, len(self.layers)):
            selected_layer(self.shape, self.layers[l], self.hidden[l], self.k[l], self.v[l],
                           self.hidden[l + 1], s.sel_idx, s.row_ptr, self.sparse, stream)
        return s.sel_idx, s.row_ptr
