"""Step drivers over the five library calls: buffer plumbing only, no arithmetic.

A selected layer is qkv+scatter -> partial attention -> ffn+scatter on the rows that
`dllm_select_compact` produced. A single-layer step (the LLaDA-8B-shaped layer workload) is
saliency -> selection -> one selected layer. A multi-layer early-skip step runs layers below the
skip layer on every token, scores tokens at the skip layer, selects once, and runs the remaining
layers on the selected rows against the cached K/V (ES-dLLM, German summary page §2.B: skipping
at early layers such as 1/8 of the depth; the selection is reused by the layers above it).
A layer-adaptive step (DyLLM, French summary page §2.A and §2.B) keeps the attention context of
every token in every layer and lets each layer pick, by the cosine change of the contexts, the
tokens whose FFN is recomputed; those tokens' changed outputs decide the next layer's rows.
Every driver can write its carried state to a file and resume from it (`save_state`,
`load_state`).
"""
from __future__ import annotations

import contextlib
import math
from dataclasses import dataclass, field

import torch

from . import (DELTA_COS, DELTA_L1N, OP_ATTN, OP_COMMIT, OP_FFN, OP_QKV, SEL_THRESHOLD, SEL_TOPK,
               Shape, dllm_commit, dllm_embed_rows, dllm_flags_from_rows, dllm_gather_ffn_scatter,
               dllm_gather_kv_rows,
               dllm_gather_qkv_scatter_kv, dllm_gather_rows, dllm_partial_attn, dllm_saliency,
               dllm_salient_attn, dllm_select_compact, workspace)


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


def _no_mark(tag):
    pass


def selected_layer(shape: Shape, w: LayerWeights, h_in, k_cache, v_cache, h_out, sel_idx, row_ptr,
                   scratch: LayerScratch, stream=None, mark=_no_mark, tag=""):
    """qkv + K/V scatter, partial attention, FFN + hidden scatter for the selected rows.
    mark(name) is called after each call is enqueued (name = tag + "qkv" / "attn" / "ffn"), so a
    caller can record a timing event at every call boundary."""
    m = scratch.m_cap
    dllm_gather_qkv_scatter_kv(shape, h_in, w.g_attn, w.w_qkv, sel_idx, row_ptr, m,
                               scratch.q_sel, k_cache, v_cache, scratch.ws_qkv, stream)
    mark(tag + "qkv")
    dllm_partial_attn(shape, attn_scale(shape), scratch.q_sel, k_cache, v_cache, sel_idx, row_ptr,
                      m, scratch.o_sel, scratch.ws_attn, stream)
    mark(tag + "attn")
    dllm_gather_ffn_scatter(shape, h_in, scratch.o_sel, w.w_o, w.g_ffn, w.w_gate, w.w_up,
                            w.w_down, sel_idx, row_ptr, m, h_out, scratch.ws_ffn, stream)
    mark(tag + "ffn")


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

    def score_and_select(self, h_cur, h_prev, logits, force=None, stream=None, conf=None,
                         mark=_no_mark):
        """conf: [B, S] float32; with logits the confidence is also written there, without
        logits (alpha != 0) it is read from there."""
        c = self.sel
        dllm_saliency(self.shape, c.delta_kind, c.alpha, h_cur, h_prev, logits, self.score,
                      conf, stream=stream)
        mark("saliency")
        dllm_select_compact(self.shape, c.mode, c.tau, c.k, self.score, force, self.sel_idx,
                            self.row_ptr, stream=stream)
        mark("select")

    def __call__(self, w: LayerWeights, h_cur, h_prev, logits, k_cache, v_cache, h_out,
                 force=None, stream=None):
        self.score_and_select(h_cur, h_prev, logits, force, stream)
        selected_layer(self.shape, w, h_cur, k_cache, v_cache, h_out, self.sel_idx, self.row_ptr,
                       self.scratch, stream)


# ---------------------------------------------------------------- checkpoint / resume
# A step driver's state is what its next step reads from the steps before it: the K/V and hidden
# caches, the skip-layer references, and for the layer-adaptive driver the attention states,
# contexts and launch plans. `state_dict` copies it to host memory (after the device has
# finished), `load_state_dict` copies it back into the driver's own buffers in place, so HIP
# graphs captured on the driver stay valid. A resumed driver's next step is bit-identical to the
# uninterrupted one's. Files hold plain tensors, numbers and strings (`torch.load(...,
# weights_only=True)` reads them).
STATE_FORMAT = "dllm-step-state/1"


def _shape_key(shape: Shape) -> list:
    return [shape.B, shape.S, shape.d, shape.H, shape.Hkv, shape.hd, shape.F, shape.V,
            "bf16" if shape.torch_dtype == torch.bfloat16 else "f32"]


def _snapshot(config: dict, tensors: dict, scalars: dict) -> dict:
    if any(t.is_cuda for t in tensors.values()):
        torch.cuda.synchronize()
    return {"format": STATE_FORMAT, "config": dict(config),
            "tensors": {n: t.detach().to("cpu", copy=True) for n, t in tensors.items()},
            "scalars": dict(scalars)}


def _restore(state: dict, config: dict, tensors: dict) -> dict:
    """Checks the state against the driver's configuration and buffers, copies the tensors in
    place and returns the scalars."""
    if not isinstance(state, dict) or state.get("format") != STATE_FORMAT:
        raise ValueError(f"not a {STATE_FORMAT} state")
    got = state["config"]
    for key in sorted(set(config) | set(got)):
        if got.get(key) != config.get(key):
            raise ValueError(f"state was saved with {key} = {got.get(key)!r}, this driver has "
                             f"{config.get(key)!r}")
    saved = state["tensors"]
    if set(saved) != set(tensors):
        raise ValueError(f"state tensors {sorted(set(saved) ^ set(tensors))} do not match")
    for n, t in tensors.items():
        if saved[n].shape != t.shape or saved[n].dtype != t.dtype:
            raise ValueError(f"state tensor {n}: {tuple(saved[n].shape)} {saved[n].dtype}, "
                             f"buffer {tuple(t.shape)} {t.dtype}")
    for n, t in tensors.items():
        t.copy_(saved[n])
    if any(t.is_cuda for t in tensors.values()):
        torch.cuda.synchronize()
    return dict(state["scalars"])


def save_state(driver, path) -> None:
    """Writes `driver.state_dict()` to `path`."""
    torch.save(driver.state_dict(), path)


def load_state(driver, path) -> None:
    """Restores a state written by `save_state` into `driver` (same configuration and shapes)."""
    driver.load_state_dict(torch.load(path, map_location="cpu", weights_only=True))


class EarlySkipModel:
    """L-layer early-skip step with per-layer K/V caches and per-boundary hidden-state caches.

    hidden[l] is the input of layer l (hidden[0] = embeddings); layer l writes hidden[l + 1].
    Layers [0, skip) run on every token; the saliency of hidden[skip] against its value at the
    previous step picks the rows for layers [skip, L).

    Optional second skip point (ES-dLLM German summary page §2.B names 1/8 and 1/4 of the depth):
    at layer skip2 the rows of the first selection are ranked again by the same score on
    hidden[skip2] (its change against the previous step, the confidence of the first stage reused)
    and only the top-k2 of them (plus the forced ones) go on through layers [skip2, L).
    """

    def __init__(self, shape: Shape, layers: list, skip: int, sel: SelectConfig, m_cap: int,
                 device="cuda", skip2: int = 0, k2: int = 0):
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
        if skip2 and not skip < skip2 < L:
            raise ValueError(f"second skip point {skip2} not inside ({skip}, {L})")
        self.skip2, self.k2 = int(skip2), int(k2)
        self.conf = torch.zeros(B, shape.S, dtype=torch.float32, device=device)
        if self.skip2:
            self.h_ref2 = torch.zeros(B, shape.S, d, dtype=dt, device=device)
            self.flags2 = torch.zeros(B, shape.S, dtype=torch.uint8, device=device)
            # the second stage keeps top-k2 per sequence plus forced rows: its layers are planned
            # for B * k2 rows (workspaces sized for any plan)
            self.shape2 = shape.with_plan(max(1, min(m_cap, B * self.k2)))
            self.step2 = SingleLayerStep(shape.with_plan(1), SelectConfig(
                mode=SEL_TOPK, k=self.k2, alpha=sel.alpha, delta_kind=sel.delta_kind), m_cap,
                device)

    def fill(self, x0, stream=None):
        """Step 0: every layer on every token; primes caches and the skip-layer reference."""
        self.hidden[0].copy_(x0)
        for l, w in enumerate(self.layers):
            selected_layer(self.shape, w, self.hidden[l], self.k[l], self.v[l], self.hidden[l + 1],
                           self.all_sel, self.all_rp, self.dense, stream)
        self.h_ref.copy_(self.hidden[self.skip])
        if self.skip2:
            self.h_ref2.copy_(self.hidden[self.skip2])

    def step(self, x, logits=None, force=None, stream=None, mark=_no_mark):
        """Returns the rows of the last layers: the first selection's, or with a second skip point
        the second one's (the first is in step1.sel_idx / step1.row_ptr).
        mark(name) is called after every call is enqueued ("copy", "dense_qkv", "dense_attn",
        "dense_ffn", "saliency", "select", "sel_qkv", "sel_attn", "sel_ffn")."""
        self.hidden[0].copy_(x)
        mark("copy")
        for l in range(self.skip):
            selected_layer(self.shape, self.layers[l], self.hidden[l], self.k[l], self.v[l],
                           self.hidden[l + 1], self.all_sel, self.all_rp, self.dense, stream,
                           mark, "dense_")
        s = self.step1
        s.score_and_select(self.hidden[self.skip], self.h_ref, logits, force, stream,
                           conf=self.conf if (self.skip2 and logits is not None) else None,
                           mark=mark)
        self.h_ref.copy_(self.hidden[self.skip])
        mark("copy")
        last = self.skip2 or len(self.layers)
        for l in range(self.skip, last):
            selected_layer(self.shape, self.layers[l], self.hidden[l], self.k[l], self.v[l],
                           self.hidden[l + 1], s.sel_idx, s.row_ptr, self.sparse, stream,
                           mark, "sel_")
        if not self.skip2:
            return s.sel_idx, s.row_ptr
        s2 = self.step2
        dllm_flags_from_rows(self.shape, force, s.sel_idx, s.row_ptr, self.m_cap, self.flags2,
                             stream)
        s2.score_and_select(self.hidden[self.skip2], self.h_ref2, None, self.flags2, stream,
                            conf=self.conf if self.sel.alpha != 0.0 else None, mark=mark)
        self.h_ref2.copy_(self.hidden[self.skip2])
        mark("copy")
        for l in range(self.skip2, len(self.layers)):
            selected_layer(self.shape2, self.layers[l], self.hidden[l], self.k[l], self.v[l],
                           self.hidden[l + 1], s2.sel_idx, s2.row_ptr, s2.scratch, stream,
                           mark, "sel2_")
        return s2.sel_idx, s2.row_ptr


    def _carried(self) -> dict:
        t = {}
        for l in range(len(self.layers)):
            t[f"k.{l}"], t[f"v.{l}"] = self.k[l], self.v[l]
        for l, h in enumerate(self.hidden):
            t[f"hidden.{l}"] = h
        t["h_ref"] = self.h_ref
        if self.skip2:
            t["h_ref2"] = self.h_ref2
        return t

    def _config(self) -> dict:
        return {"driver": "EarlySkipModel", "shape": _shape_key(self.shape),
                "layers": len(self.layers), "skip": self.skip, "skip2": self.skip2,
                "k2": self.k2, "m_cap": self.m_cap}

    def state_dict(self) -> dict:
        """K/V caches, hidden-state caches and skip-layer references, copied to the host."""
        return _snapshot(self._config(), self._carried(), {})

    def load_state_dict(self, state: dict) -> None:
        _restore(state, self._config(), self._carried())


class LayerAdaptiveModel:
    """L-layer step that keeps the attention context of every token (DyLLM, French summary page
    §2.A layer-adaptive saliency, §2.B salient / approximate attention).

    Per layer l and step t, with A_l the tokens whose layer input changed:
      copies of the K/V rows of A_l; QKV of A_l into the caches; contexts of every token
      (`dllm_salient_attn`: exact for A_l, changed-key update for the rest); the cosine change of
      each token's context against step t-1 (`dllm_saliency`, cosine kind, alpha 0); the tokens
      above the threshold (`dllm_select_compact`, threshold mode) get W_o + FFN and write their
      row of hidden[l + 1]; the others keep last step's row. A_{l+1} is that set. A_0 is chosen
      by the L1-normalised change of the layer-0 input against step t-1 (threshold `tau_in`).
    Buffers are sized for every token (the thresholded counts are only known on the device).
    The calls are told how many rows to plan for (`m_plan`): each row set's count of the last
    step of the same kind whose counts have reached the host, with a 1/8 margin. Counts come back
    by an asynchronous copy, so no step waits for the device; a wrong guess costs speed, never
    rows.

    Response-only steps (DyLLM §2.C), when `prompt_len` P > 0: positions 0..P-1 of every
    sequence hold the prompt. A response-only step leaves them out of every row set (selection
    flag "excluded") and out of the changed-key update of the contexts (`q_first` = P): their
    caches, states, contexts and hidden rows keep what they held. Every `inject_every`-th step
    (0 = never) re-injects the prompt: its positions are forced into every row set, so they are
    recomputed exactly, layer by layer.
    """

    def __init__(self, shape: Shape, layers: list, tau_in: float, tau_ctx, scale=None,
                 device="cuda", prompt_len: int = 0, inject_every: int = 0):
        self.shape, self.layers = shape, layers
        self.tau_in = tau_in
        if not 0 <= prompt_len <= shape.S:
            raise ValueError(f"prompt_len {prompt_len} outside [0, S]")
        self.prompt_len, self.inject_every = int(prompt_len), int(inject_every)
        self.t = 0                                    # steps since fill
        self.scale = attn_scale(shape) if scale is None else scale
        L = len(layers)
        self.tau_ctx = list(tau_ctx) if isinstance(tau_ctx, (list, tuple)) else [tau_ctx] * L
        B, S, d, H, Hkv, hd = shape.B, shape.S, shape.d, shape.H, shape.Hkv, shape.hd
        dt = shape.torch_dtype
        ntok, nq = B * S, H * hd
        z = lambda *sh, dtype=dt: torch.zeros(*sh, dtype=dtype, device=device)  # noqa: E731
        self.k = [z(B, Hkv, S, hd) for _ in range(L)]
        self.v = [z(B, Hkv, S, hd) for _ in range(L)]
        self.hidden = [z(B, S, d) for _ in range(L + 1)]
        self.x_ref = z(B, S, d)                       # layer-0 input at step t-1
        self.q_all = [z(ntok, nq) for _ in range(L)]
        self.st_m = [z(ntok, H, dtype=torch.float32) for _ in range(L)]
        self.st_l = [z(ntok, H, dtype=torch.float32) for _ in range(L)]
        self.st_o = [z(ntok, nq, dtype=torch.float32) for _ in range(L)]
        self.ctx = [[z(ntok, nq), z(ntok, nq)] for _ in range(L)]  # contexts at t and t-1
        self.cur = 0                                  # index of the step-t context buffer
        self.ctx_shape = Shape(B=B, S=S, d=nq, H=H, Hkv=Hkv, hd=hd, F=shape.F,
                               dtype=shape.dtype, V=0)
        # workspaces sized for any m_plan (a nonzero m_plan in the shape asks for that size)
        self.scratch = LayerScratch(shape.with_plan(1), ntok, device)
        self.plan = [0] * (L + 1)                      # m_plan per row set (0: every token)
        self._plans = {}                               # step kind (inject?) -> m_plan per set
        self._shapes = {}
        self._counts_kind = False
        flags = torch.zeros(B, S, dtype=torch.uint8, device=device)
        flags[:, :prompt_len] = 2
        self._flags_resp = flags if prompt_len else None     # prompt excluded
        self._flags_inject = (flags // 2) if prompt_len else None  # prompt forced
        self._counts = torch.zeros(L + 1, dtype=torch.int32, device=device)
        self._counts_host = torch.zeros(L + 1, dtype=torch.int32,
                                        pin_memory=torch.device(device).type == "cuda")
        self._counts_evt = None
        self.k_old = z(ntok, Hkv * hd)
        self.v_old = z(ntok, Hkv * hd)
        self.o_rows = z(ntok, nq)
        self.score = torch.empty(B, S, dtype=torch.float32, device=device)
        # row sets: [0] input-change set, then one per layer (its FFN set = next layer's input set)
        self.sel = [torch.empty(ntok, dtype=torch.int32, device=device) for _ in range(L + 1)]
        self.rp = [torch.empty(B + 1, dtype=torch.int32, device=device) for _ in range(L + 1)]
        self.all_sel, self.all_rp = all_rows(shape, device)
        self.layer_scores = None  # per-layer copies of the context scores (step(record=True))

    def _planned(self, m_plan):
        sh = self._shapes.get(m_plan)
        if sh is None:
            sh = self._shapes[m_plan] = self.shape.with_plan(m_plan)
        return sh

    def _layer(self, l, sel_a, rp_a, sel_f, rp_f, tau, stream, flags=None):
        w, sc, n = self.layers[l], self.scratch, self.shape.B * self.shape.S
        sh = self._planned(self.plan[l])       # rows of set l: projection and attention
        sh_f = self._planned(self.plan[l + 1])  # rows of set l + 1: output projection and FFN
        cur, prev = self.ctx[l][self.cur], self.ctx[l][1 - self.cur]
        dllm_gather_kv_rows(sh, self.k[l], self.v[l], sel_a, rp_a, n, self.k_old, self.v_old,
                            stream)
        dllm_gather_qkv_scatter_kv(sh, self.hidden[l], w.g_attn, w.w_qkv, sel_a, rp_a, n,
                                   sc.q_sel, self.k[l], self.v[l], sc.ws_qkv, stream)
        dllm_salient_attn(sh, self.scale, sc.q_sel, self.q_all[l], self.k[l], self.v[l],
                          self.k_old, self.v_old, sel_a, rp_a, n, self.st_m[l], self.st_l[l],
                          self.st_o[l], sc.o_sel, cur, sc.ws_attn, stream,
                          q_first=self.prompt_len)
        if tau is None:   # every token (fill)
            sel_f.copy_(self.all_sel)
            rp_f.copy_(self.all_rp)
        else:
            dllm_saliency(self.ctx_shape, DELTA_COS, 0.0, cur, prev, None, self.score,
                          stream=stream)
            if self.layer_scores is not None:
                self.layer_scores[l].copy_(self.score)
            dllm_select_compact(sh, SEL_THRESHOLD, tau, 0, self.score, flags, sel_f, rp_f,
                                stream=stream)
        dllm_gather_rows(self.ctx_shape, cur, self.ctx_shape.d, sel_f, rp_f, n, self.o_rows,
                         stream)
        dllm_gather_ffn_scatter(sh_f, self.hidden[l], self.o_rows, w.w_o, w.g_ffn, w.w_gate,
                                w.w_up, w.w_down, sel_f, rp_f, n, self.hidden[l + 1], sc.ws_ffn,
                                stream)

    def fill(self, x0, stream=None):
        """Step 0: every layer on every token; primes caches, states and both context buffers."""
        self.plan = [0] * len(self.plan)
        self._plans = {}
        self._counts_evt = None
        self.t = 0
        self.hidden[0].copy_(x0)
        self.x_ref.copy_(x0)
        for l in range(len(self.layers)):
            self._layer(l, self.all_sel, self.all_rp, self.sel[l + 1], self.rp[l + 1], None,
                        stream)
            self.ctx[l][1 - self.cur].copy_(self.ctx[l][self.cur])

    def step(self, x, tau_ctx=None, record=False, stream=None):
        """One denoising step on layer-0 input x (optionally with this step's per-layer context
        thresholds); returns the row sets: [0] input change, [l + 1] FFN rows of layer l.
        record=True keeps each layer's context scores in `layer_scores`."""
        taus = self.tau_ctx if tau_ctx is None else list(tau_ctx)
        if record and self.layer_scores is None:
            self.layer_scores = [torch.empty_like(self.score) for _ in self.layers]
        elif not record:
            self.layer_scores = None
        self.cur = 1 - self.cur
        self.t += 1
        inject = self.inject_every > 0 and self.t % self.inject_every == 0
        flags = None
        if self.prompt_len:
            flags = self._flags_inject if inject else self._flags_resp
        if self._counts_evt is not None and self._counts_evt.query():
            self._plans[self._counts_kind] = [c + c // 8 + 1 for c in self._counts_host.tolist()]
            self._counts_evt = None
        self.plan = self._plans.get(inject, [0] * len(self.plan))
        self.hidden[0].copy_(x)
        dllm_saliency(self.shape, DELTA_L1N, 0.0, self.hidden[0], self.x_ref, None, self.score,
                      stream=stream)
        dllm_select_compact(self.shape, SEL_THRESHOLD, self.tau_in, 0, self.score, flags,
                            self.sel[0], self.rp[0], stream=stream)
        self.x_ref.copy_(x)
        for l in range(len(self.layers)):
            self._layer(l, self.sel[l], self.rp[l], self.sel[l + 1], self.rp[l + 1], taus[l],
                        stream, flags)
        if self._counts_evt is None:   # the previous copy has been read: send this step's counts
            B = self.shape.B
            with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
                torch.stack([r[B] for r in self.rp], out=self._counts)
                self._counts_host.copy_(self._counts, non_blocking=True)
                self._counts_evt = torch.cuda.Event()
                self._counts_evt.record()
                self._counts_kind = inject
        return self.sel, self.rp


    def _settle_counts(self) -> None:
        """Waits for the row counts in flight and folds them into the plans, as the next step
        would once they have arrived (so that step's plans no longer depend on timing)."""
        if self._counts_evt is not None:
            self._counts_evt.synchronize()
            self._plans[self._counts_kind] = [c + c // 8 + 1 for c in self._counts_host.tolist()]
            self._counts_evt = None

    def _carried(self) -> dict:
        t = {"x_ref": self.x_ref}
        for l in range(len(self.layers)):
            t[f"k.{l}"], t[f"v.{l}"], t[f"q_all.{l}"] = self.k[l], self.v[l], self.q_all[l]
            t[f"st_m.{l}"], t[f"st_l.{l}"], t[f"st_o.{l}"] = self.st_m[l], self.st_l[l], self.st_o[l]
            t[f"ctx.{l}.0"], t[f"ctx.{l}.1"] = self.ctx[l]
        for l, h in enumerate(self.hidden):
            t[f"hidden.{l}"] = h
        return t

    def _config(self) -> dict:
        return {"driver": "LayerAdaptiveModel", "shape": _shape_key(self.shape),
                "layers": len(self.layers), "prompt_len": self.prompt_len,
                "inject_every": self.inject_every}

    def state_dict(self) -> dict:
        """Caches, attention states and contexts, the step counter, the index of the current
        context buffer and the launch plans (row counts still in flight are waited for)."""
        self._settle_counts()
        plans = {("inject" if k else "response"): list(v) for k, v in self._plans.items()}
        return _snapshot(self._config(), self._carried(),
                         {"t": self.t, "cur": self.cur, "plans": plans})

    def load_state_dict(self, state: dict) -> None:
        sc = _restore(state, self._config(), self._carried())
        self.t, self.cur = int(sc["t"]), int(sc["cur"])
        self._plans = {k == "inject": [int(c) for c in v] for k, v in sc["plans"].items()}
        self._counts_evt = None
        self.plan = [0] * len(self.plan)


class BlockDecoder:
    """Semi-autoregressive block decoding that stays on the device: the early-skip step
    (ES-dLLM, German summary page §2.B) with the active block forced into the selection, then the
    commit of the active block from this step's logits (SlowFast, German summary page,
    "Der SlowFast-Algorithmus" item 2: threshold commit, top-k update when too few pass; block
    advance) and the embeddings of the committed tokens written into the next step's input.

    Token ids, block indices, the selection flags and the input rows live on the device and are
    updated by the library calls, so `step` never waits for the device and can be captured in a
    HIP graph (`capture`) and replayed. `refresh` is the periodic full refresh: every layer on
    every token (the caches and the skip-layer reference rebuilt from the current input)
    (ES-dLLM, Dutch summary page, "Methodologie" item 3: caches refreshed periodically). `run_step` is
    one step, eager or replayed from a graph, followed by the refresh every `refresh_every` steps
    (0 = only when called).

    model: EarlySkipModel whose m_cap covers B x (top-k + one block); emb [V, d] and mask_emb
    [d] in the model's dtype; the model's shape carries V (the logits' vocabulary).
    """

    def __init__(self, model, emb, mask_emb, prompt_len: int, block_len: int, tau: float,
                 k_min: int, device="cuda", refresh_every: int = 0):
        sh = model.shape
        if emb.shape != (sh.V, sh.d):
            raise ValueError(f"embedding table {tuple(emb.shape)} is not [V={sh.V}, d={sh.d}]")
        if model.m_cap < sh.B * (model.sel.k + block_len):
            raise ValueError("the model's m_cap must hold, per sequence, the top-k plus one "
                             "forced block")
        self.model, self.emb, self.mask_emb = model, emb, mask_emb
        self.P, self.L, self.tau, self.k_min = int(prompt_len), int(block_len), tau, int(k_min)
        if refresh_every < 0:
            raise ValueError(f"refresh_every {refresh_every} < 0")
        self.refresh_every, self.steps_done = int(refresh_every), 0
        B, S = sh.B, sh.S
        self.nblk = -(-(S - self.P) // self.L)
        self.tok = torch.full((B, S), -1, dtype=torch.int32, device=device)
        self.blk = torch.zeros(B, dtype=torch.int32, device=device)
        self.flags = torch.zeros(B, S, dtype=torch.uint8, device=device)
        self.cidx = torch.zeros(B * self.L, dtype=torch.int32, device=device)
        self.crp = torch.zeros(B + 1, dtype=torch.int32, device=device)
        self.ws = workspace(OP_COMMIT, sh, self.L, device)
        self.x = torch.zeros(B, S, sh.d, dtype=sh.torch_dtype, device=device)
        self.all_sel, self.all_rp = all_rows(sh, device)

    def start(self, prompt, stream=None):
        """prompt: int32 [B, P] token ids. Every later position is masked; block 0 is active."""
        sh = self.model.shape
        self.steps_done = 0
        self.tok.fill_(-1)
        self.tok[:, :self.P] = prompt
        self.blk.zero_()
        self.flags.zero_()
        if self.nblk > 0:
            self.flags[:, self.P:min(sh.S, self.P + self.L)] = 1
        dllm_embed_rows(sh, self.emb, self.mask_emb, self.tok, self.all_sel, self.all_rp,
                        sh.B * sh.S, self.x, stream)
        self.model.fill(self.x, stream)

    def step(self, logits, stream=None):
        """One decoding step; `logits` [B, S, V] stand for this step's output of the model."""
        sh = self.model.shape
        self.model.step(self.x, force=self.flags, stream=stream)
        dllm_commit(sh, logits, self.P, self.L, self.tau, self.k_min, self.tok, self.blk,
                    self.cidx, self.crp, self.flags, self.ws, stream)
        dllm_embed_rows(sh, self.emb, self.mask_emb, self.tok, self.cidx, self.crp,
                        sh.B * self.L, self.x, stream)

    def refresh(self, stream=None):
        self.model.fill(self.x, stream)

    def run_step(self, logits=None, graph=None, stream=None):
        """One step: eager on `logits`, or the replay of `graph` (from `capture`); then the full
        refresh if this is a multiple of `refresh_every` steps since `start`."""
        if graph is None:
            self.step(logits, stream)
        else:
            graph.replay()
        self.steps_done += 1
        if self.refresh_every and self.steps_done % self.refresh_every == 0:
            self.refresh(stream)

    def capture(self, logits):
        """A HIP graph of one `step` reading `logits` (replay with .replay())."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                self.step(logits)
        torch.cuda.current_stream().wait_stream(side)
        return g

    def _config(self) -> dict:
        return {"driver": "BlockDecoder", "prompt_len": self.P, "block_len": self.L,
                "tau": float(self.tau), "k_min": self.k_min, "refresh_every": self.refresh_every}

    def _carried(self) -> dict:
        return {"tok": self.tok, "blk": self.blk, "flags": self.flags, "x": self.x}

    def state_dict(self) -> dict:
        """Token ids, block indices, selection flags and the next step's input rows, with the
        model's state under "model"."""
        st = _snapshot(self._config(), self._carried(), {"steps_done": self.steps_done})
        st["model"] = self.model.state_dict()
        return st

    def load_state_dict(self, state: dict) -> None:
        sc = _restore(state, self._config(), self._carried())
        self.model.load_state_dict(state["model"])
        self.steps_done = int(sc["steps_done"])
