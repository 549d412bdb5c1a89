"""Plain CPU oracle of one token-skipping denoising step. TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import or call this
module. The HIP library never routes through it, and it imports nothing from the HIP package.

It computes, slowly and in float64, what the five library calls compute:

  saliency            ES-dLLM (German summary page) §2.A, importance-score equation:
                      I = alpha * c^(t-1) + (1 - alpha) * ||H^t - H^(t-1)||_1 / (sqrt(d) ||H^(t-1)||_2),
                      alpha = 0.5 in the experiments; higher I = more likely selected.
                      DyLLM (French summary page) §2.A: cosine similarity of a token's vector at
                      step t and t-1, salient when it falls below a threshold tau.
  select_compact      ES-dLLM (German page) §2.B / Dutch page "Methodologie" item 2: only the
                      top-k positions go on; DyLLM §2.A: threshold rule. Output: ascending ids.
  gather_qkv_scatter  ES-dLLM (German page) §2.B and Dutch "Methodologie" item 3: keys, values
                      and hidden states are cached; selected tokens update the caches in place,
                      skipped tokens keep the old entries.
  partial_attn        DyLLM (French page) §2.B: for salient tokens the attention row is
                      recomputed exactly; §1: attention is bidirectional (no causal mask).
  gather_ffn_scatter  DyLLM (French page) §2.A: FFN runs for salient tokens only, the others
                      reuse cached activations.
  salient_attention   DyLLM (French page) §2.B, both paths: exact rows for salient tokens; for
                      stable tokens the weights of unchanged keys are reused and only the changed
                      keys' contributions are replaced, which equals attention of the reused query
                      against the updated cache (see the function); gather_kv_rows copies the K/V
                      rows that a step is about to overwrite. DyLLM §2.C response-only steps:
                      select_compact's excluded flag and salient_attention's q_first leave the
                      prompt out of a step.
  commit_step         SlowFast (German page) "Der SlowFast-Algorithmus" item 2: threshold commit
                      of the active block with a top-k fallback; block advance; embed_rows writes
                      the embeddings of the committed tokens (the next step's input rows).

Readings where the pages are silent (all listed in the design notes): confidence c is the maximum
softmax probability of the previous-step logits at temperature 1; the transformer block is
pre-norm with RMSNorm (gain g, epsilon eps), fused QKV weight rows ordered Q|K|V, grouped KV heads
mapped in blocks (kv head = h // (H / Hkv)), attention scale 1/sqrt(hd), no positional rotation,
SwiGLU FFN silu(hn W_gate^T) * (hn W_up^T) W_down^T, and residual adds around attention and FFN.
Top-k ranks by (score descending, position ascending); NaN ranks below -inf; -0 == +0.
Threshold selection is strict (score > tau).

Arithmetic is float64 throughout. Inputs arrive as float64 arrays (see `decode_bf16` for bf16
bit patterns); the only rounding is of the score to float32, because the score is the float32
array on which the selection decision is taken.

Pins: every function here is checked in tests/test_oracle_pins.py against closed forms,
brute force on tiny inputs, and invariants (select-all equals an independently written dense
layer; select-none leaves caches unchanged). `max_softmax_confidence` on real-valued logits
and the composed multi-layer step have no worked example on the pages: their end-to-end values
are "parity unpinned" beyond those checks.
"""
from __future__ import annotations

import math

import numpy as np

DELTA_L1N, DELTA_COS, DELTA_L2R = 0, 1, 2
SEL_THRESHOLD, SEL_TOPK = 0, 1


# ----------------------------------------------------------------------------------------------
# representation helpers (no arithmetic of the method)
# ----------------------------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64. bf16 is the top half of an IEEE float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(x) -> np.ndarray:
    """float32/float64 arrays -> float64; uint16 arrays are taken as bf16 bit patterns."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return x.astype(np.float64)


# ----------------------------------------------------------------------------------------------
# (1) saliency
# ----------------------------------------------------------------------------------------------
def delta_variation(h_cur: np.ndarray, h_prev: np.ndarray, kind: int = DELTA_L1N) -> np.ndarray:
    """Per-token change between step t and t-1 over the last axis (length d).

    L1N: ||x - y||_1 / (sqrt(d) ||y||_2)       ES-dLLM (German page) §2.A equation
    COS: 1 - <x, y> / (||x||_2 ||y||_2)         DyLLM (French page) §2.A cosine rule, as a
                                                 dissimilarity so that larger = more salient
    L2R: ||x - y||_2 / ||y||_2                   relative L2 change (the L2 variant of the same)
    """
    x = np.asarray(h_cur, dtype=np.float64)
    y = np.asarray(h_prev, dtype=np.float64)
    d = x.shape[-1]
    norm_y = np.sqrt(np.sum(y * y, axis=-1))
    if kind == DELTA_L1N:
        return np.sum(np.abs(x - y), axis=-1) / (math.sqrt(d) * norm_y)
    if kind == DELTA_COS:
        norm_x = np.sqrt(np.sum(x * x, axis=-1))
        return 1.0 - np.sum(x * y, axis=-1) / (norm_x * norm_y)
    if kind == DELTA_L2R:
        return np.sqrt(np.sum((x - y) ** 2, axis=-1)) / norm_y
    raise ValueError(f"unknown delta kind {kind}")


def max_softmax_confidence(logits: np.ndarray) -> np.ndarray:
    """c = max_v softmax(z)_v over the last axis = 1 / sum_v exp(z_v - max_v z_v).

    ES-dLLM (Dutch page, "Methodologie" 1; German page §2.A): the confidence of the previous
    iteration, a probability. Read here as the largest softmax probability at temperature 1.
    """
    z = np.asarray(logits, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    return 1.0 / np.sum(np.exp(z - m), axis=-1)


def saliency(h_cur, h_prev, logits, alpha: float, kind: int = DELTA_L1N, conf=None):
    """Importance score per token, ES-dLLM (German page) §2.A equation.

    h_cur, h_prev: [..., d] (may be None when alpha == 1); logits: [..., V] (None when alpha == 0,
    or when `conf`, the confidence of the same logits computed earlier, is given: the score at a
    second skip point, §2.B, reuses the previous step's confidence).
    Returns (score float32 [...], conf float64 [...] or None, delta float64 [...] or None).
    """
    if logits is not None:
        conf = max_softmax_confidence(logits)
    elif conf is not None:
        conf = np.asarray(conf, dtype=np.float64)
    delta = delta_variation(h_cur, h_prev, kind) if h_cur is not None else None
    c = conf if conf is not None else 0.0
    v = delta if delta is not None else 0.0
    score = alpha * c + (1.0 - alpha) * v
    return np.asarray(score, dtype=np.float64).astype(np.float32), conf, delta


# ----------------------------------------------------------------------------------------------
# (2) selection + compaction
# ----------------------------------------------------------------------------------------------
def _rank_key(value: float, pos: int):
    """Top-k order: larger score first, NaN after everything, ties by lower position."""
    if math.isnan(value):
        return (1, 0.0, pos)
    return (0, -value, pos)  # -(+0.0) == -(-0.0) in comparisons, so +-0 tie on position


def select_compact(score, force, mode: int, tau: float = 0.0, k: int = 0):
    """Per sequence: forced positions plus top-k (or score > tau) of the candidates, ascending.

    tau is taken as a float32, the type of the score array, so the comparison is float32.

    score: float32 [B, S]; force: integer flags [B, S] or None: bit 0 forced, else bit 1
    excluded (never selected: the prompt of a response-only step, DyLLM French summary page
    §2.C), else a candidate. A bool array is forced / candidate.
    Returns (sel_idx int32 [M] with flat ids b*S + s, row_ptr int32 [B+1]).
    """
    score = np.asarray(score, dtype=np.float32)
    B, S = score.shape
    flags = None if force is None else np.asarray(force).astype(np.int64)
    sel, row_ptr = [], [0]
    for b in range(B):
        forced = [bool(flags[b, s] & 1) if flags is not None else False for s in range(S)]
        excluded = [bool(flags[b, s] & 2) and not forced[s] if flags is not None else False
                    for s in range(S)]
        cand = [s for s in range(S) if not forced[s] and not excluded[s]]
        if mode == SEL_TOPK:
            ranked = sorted(cand, key=lambda s: _rank_key(float(score[b, s]), s))
            chosen = ranked[: max(0, int(k))]
        elif mode == SEL_THRESHOLD:
            tau32 = np.float32(tau)  # the threshold is a float32, compared in float32
            chosen = [s for s in cand if score[b, s] > tau32]
        else:
            raise ValueError(f"unknown selection mode {mode}")
        rows = sorted(set(chosen) | {s for s in range(S) if forced[s]})
        sel.extend(b * S + s for s in rows)
        row_ptr.append(len(sel))
    return np.asarray(sel, dtype=np.int32), np.asarray(row_ptr, dtype=np.int32)


# ----------------------------------------------------------------------------------------------
# (3) gathered QKV projection + K/V cache scatter
# ----------------------------------------------------------------------------------------------
def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def gather_qkv_scatter_kv(h_in, g_attn, w_qkv, sel_idx, row_ptr, k_cache, v_cache,
                          H: int, Hkv: int, hd: int, eps: float):
    """For each selected token r = (b, s): qkv = RMSNorm(h_in[b, s]) W_qkv^T.

    The query part goes to q_sel[r]; the key/value parts overwrite k_cache[b, :, s, :] and
    v_cache[b, :, s, :]. Caches are [B, Hkv, S, hd]; unselected entries are left as they were.
    Returns (q_sel [M, H*hd], k_cache', v_cache') as new arrays.
    """
    h_in = np.asarray(h_in, dtype=np.float64)
    B, S, d = h_in.shape
    M = int(row_ptr[-1])
    nq, nkv = H * hd, Hkv * hd
    k_new = np.array(k_cache, dtype=np.float64, copy=True)
    v_new = np.array(v_cache, dtype=np.float64, copy=True)
    ids = np.asarray(sel_idx[:M], dtype=np.int64)
    bs, ss = ids // S, ids % S
    x = h_in[bs, ss]                                   # [M, d] gathered rows
    qkv = rms_norm(x, g_attn, eps) @ np.asarray(w_qkv, np.float64).T
    q_sel = qkv[:, :nq]
    k_rows = qkv[:, nq:nq + nkv].reshape(M, Hkv, hd)
    v_rows = qkv[:, nq + nkv:].reshape(M, Hkv, hd)
    for r in range(M):
        k_new[bs[r], :, ss[r], :] = k_rows[r]
        v_new[bs[r], :, ss[r], :] = v_rows[r]
    return q_sel, k_new, v_new


# ----------------------------------------------------------------------------------------------
# (4) partial attention: selected queries against every cached key, no mask
# ----------------------------------------------------------------------------------------------
def partial_attn(q_sel, k_cache, v_cache, sel_idx, row_ptr, H: int, Hkv: int, hd: int,
                 scale: float):
    """o[r, h] = softmax_t(scale * q[r, h] . k[b, hk, t]) . v[b, hk, t] over all t in [0, S).

    b = batch row of selected token r, hk = h // (H / Hkv). Returns o_sel [M, H*hd].
    """
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    B, _, S, _ = k_cache.shape
    M = int(row_ptr[-1])
    G = H // Hkv
    q = np.asarray(q_sel, dtype=np.float64)[:M].reshape(M, H, hd)
    out = np.zeros((M, H, hd))
    for b in range(B):
        rows = np.arange(int(row_ptr[b]), int(row_ptr[b + 1]))
        if rows.size == 0:
            continue
        for h in range(H):
            hk = h // G
            s = (q[rows, h, :] @ k_cache[b, hk].T) * scale          # [m_b, S]
            p = np.exp(s - np.max(s, axis=1, keepdims=True))
            p /= np.sum(p, axis=1, keepdims=True)
            out[rows, h, :] = p @ v_cache[b, hk]
    return out.reshape(M, H * hd)


# ----------------------------------------------------------------------------------------------
# attention context of every token: exact rows for the salient tokens, reused rows for the rest
# ----------------------------------------------------------------------------------------------
def gather_kv_rows(k_cache, v_cache, sel_idx, row_ptr):
    """Copies of the K/V cache rows at the selected positions, taken before a projection call
    overwrites them: k_rows[r] = k_cache[b, :, s, :] for selected token r = (b, s).

    Returns (k_rows [M, Hkv, hd], v_rows [M, Hkv, hd]).
    """
    k_cache = np.asarray(k_cache)
    v_cache = np.asarray(v_cache)
    S = k_cache.shape[2]
    M = int(row_ptr[-1])
    ids = np.asarray(sel_idx[:M], dtype=np.int64)
    return k_cache[ids // S, :, ids % S, :].copy(), v_cache[ids // S, :, ids % S, :].copy()


def context_all(q_all, k_cache, v_cache, H: int, Hkv: int, hd: int, scale: float):
    """Attention context of every token's query against every cached key (no mask).

    o[b, s, h] = softmax_t(scale * q[b, s, h] . k[b, hk, t]) . v[b, hk, t], hk = h // (H / Hkv),
    and lse[b, s, h] = ln sum_t exp(scale * q[b, s, h] . k[b, hk, t]).
    Returns (o [B, S, H*hd], lse [B, S, H]).
    """
    q = np.asarray(q_all, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    B, _, S, _ = k_cache.shape
    G = H // Hkv
    q = q.reshape(B, S, H, hd)
    o = np.zeros((B, S, H, hd))
    lse = np.zeros((B, S, H))
    for b in range(B):
        for h in range(H):
            s = (q[b, :, h, :] @ k_cache[b, h // G].T) * scale              # [S queries, S keys]
            mx = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - mx)
            tot = np.sum(e, axis=1, keepdims=True)
            o[b, :, h, :] = (e / tot) @ v_cache[b, h // G]
            lse[b, :, h] = (mx + np.log(tot))[:, 0]
    return o.reshape(B, S, H * hd), lse


def salient_attention(q_sel, q_all, k_cache, v_cache, sel_idx, row_ptr, H: int, Hkv: int,
                      hd: int, scale: float, q_first: int = 0, o_prev=None, lse_prev=None):
    """DyLLM (French page) §2.B, both paths of one step, given the caches after the projection
    call of the step overwrote the K/V rows of the selected tokens:
      salient tokens (selected): their query is the one just projected and their attention row
        is recomputed exactly against every cached key;
      stable tokens (the rest): their query from the step that last projected them is reused,
        and their context takes in the changed K/V rows. Reusing the previous step's weights of
        the unchanged keys and replacing only the changed keys' contributions gives, exactly, the
        attention of the reused query against the updated cache.
    So the context of every token is the attention of the query cache, with the selected rows
    replaced, against the updated K/V cache.
    Response-only steps (§2.C): unselected positions s < q_first are not processed; they keep
    o_prev and lse_prev (their context and log-sum-exp before the step).

    Returns (q_all' [B, S, H*hd], o [B, S, H*hd], lse [B, S, H]).
    """
    q_new = np.array(q_all, dtype=np.float64, copy=True)
    B, S = q_new.shape[:2]
    M = int(row_ptr[-1])
    ids = np.asarray(sel_idx[:M], dtype=np.int64)
    q_new[ids // S, ids % S] = np.asarray(q_sel, dtype=np.float64)[:M]
    o, lse = context_all(q_new, k_cache, v_cache, H, Hkv, hd, scale)
    if q_first > 0:
        skip = np.zeros((B, S), dtype=bool)
        skip[:, :q_first] = True
        skip[ids // S, ids % S] = False
        if skip.any():   # (o_prev / lse_prev may be None when every position there is selected)
            o[skip] = np.asarray(o_prev, dtype=np.float64)[skip]
            lse[skip] = np.asarray(lse_prev, dtype=np.float64)[skip]
    return q_new, o, lse


# ----------------------------------------------------------------------------------------------
# (5) gathered output projection + SwiGLU FFN + hidden-state scatter
# ----------------------------------------------------------------------------------------------
def silu(x):
    return x / (1.0 + np.exp(-x))


def gather_ffn_scatter(h_in, o_sel, w_o, g_ffn, w_gate, w_up, w_down, sel_idx, row_ptr,
                       h_out, eps: float):
    """For each selected token r = (b, s):
         h = h_in[b, s] + o_sel[r] W_o^T
         y = h + (silu(RMSNorm(h) W_gate^T) * (RMSNorm(h) W_up^T)) W_down^T
       and h_out[b, s] = y. Unselected rows of h_out keep their values. Returns h_out' [B, S, d].
    """
    h_in = np.asarray(h_in, dtype=np.float64)
    B, S, d = h_in.shape
    M = int(row_ptr[-1])
    out = np.array(h_out, dtype=np.float64, copy=True)
    ids = np.asarray(sel_idx[:M], dtype=np.int64)
    bs, ss = ids // S, ids % S
    x = h_in[bs, ss]
    h = x + np.asarray(o_sel, np.float64)[:M] @ np.asarray(w_o, np.float64).T
    hn = rms_norm(h, g_ffn, eps)
    z = silu(hn @ np.asarray(w_gate, np.float64).T) * (hn @ np.asarray(w_up, np.float64).T)
    y = h + z @ np.asarray(w_down, np.float64).T
    out[bs, ss] = y
    return out


# ----------------------------------------------------------------------------------------------
# dense block over every token (written separately; pins "select all == full recompute")
# ----------------------------------------------------------------------------------------------
def dense_layer(h, wts: dict, H: int, Hkv: int, hd: int, eps: float, scale: float):
    """The same pre-norm block applied to every token with full bidirectional attention.

    Returns (k_cache [B,Hkv,S,hd], v_cache [B,Hkv,S,hd], h_out [B,S,d]).
    """
    h = np.asarray(h, dtype=np.float64)
    B, S, d = h.shape
    G = H // Hkv
    f = {k: np.asarray(v, dtype=np.float64) for k, v in wts.items()}
    ms = np.mean(h ** 2, axis=2, keepdims=True)
    xn = h * (1.0 / np.sqrt(ms + eps)) * f["g_attn"]
    qkv = (xn.reshape(B * S, d) @ f["w_qkv"].T).reshape(B, S, -1)
    q = qkv[..., : H * hd].reshape(B, S, H, hd).transpose(0, 2, 1, 3)          # [B,H,S,hd]
    k = qkv[..., H * hd: (H + Hkv) * hd].reshape(B, S, Hkv, hd).transpose(0, 2, 1, 3)
    v = qkv[..., (H + Hkv) * hd:].reshape(B, S, Hkv, hd).transpose(0, 2, 1, 3)
    o = np.zeros((B, S, H, hd))
    for b in range(B):
        for hh in range(H):
            logit = (q[b, hh] @ k[b, hh // G].T) * scale                           # [S, S]
            w = np.exp(logit - logit.max(axis=1, keepdims=True))
            w = w / w.sum(axis=1, keepdims=True)
            o[b, :, hh, :] = w @ v[b, hh // G]
    h1 = h + (o.reshape(B * S, H * hd) @ f["w_o"].T).reshape(B, S, d)
    ms1 = np.mean(h1 ** 2, axis=2, keepdims=True)
    hn = (h1 * (1.0 / np.sqrt(ms1 + eps)) * f["g_ffn"]).reshape(B * S, d)
    gate = hn @ f["w_gate"].T
    up = hn @ f["w_up"].T
    act = gate / (1.0 + np.exp(-gate)) * up
    y = h1 + (act @ f["w_down"].T).reshape(B, S, d)
    return k, v, y


# ----------------------------------------------------------------------------------------------
# one selected layer as the five calls compose it
# ----------------------------------------------------------------------------------------------
def selected_layer(h_in, wts: dict, sel_idx, row_ptr, k_cache, v_cache, h_out,
                   H: int, Hkv: int, hd: int, eps: float, scale: float):
    """qkv+scatter -> partial attention -> ffn+scatter for the selected rows.

    Returns (q_sel, o_sel, k_cache', v_cache', h_out').
    """
    q_sel, k_new, v_new = gather_qkv_scatter_kv(h_in, wts["g_attn"], wts["w_qkv"], sel_idx,
                                                row_ptr, k_cache, v_cache, H, Hkv, hd, eps)
    o_sel = partial_attn(q_sel, k_new, v_new, sel_idx, row_ptr, H, Hkv, hd, scale)
    out = gather_ffn_scatter(h_in, o_sel, wts["w_o"], wts["g_ffn"], wts["w_gate"], wts["w_up"],
                             wts["w_down"], sel_idx, row_ptr, h_out, eps)
    return q_sel, o_sel, k_new, v_new, out


# ----------------------------------------------------------------------------------------------
# device-side decode loop: commit rule, block advance, embeddings of committed tokens
# ----------------------------------------------------------------------------------------------
def confidence_argmax(logits_row):
    """(largest softmax probability at temperature 1, index of the largest logit; the lowest
    index among equal maxima) of one logit row: the token a masked position would take."""
    z = np.asarray(logits_row, dtype=np.float64)
    arg = int(np.argmax(z))          # numpy returns the first maximal index
    return float(max_softmax_confidence(z[None])[0]), arg


def commit_step(logits, tok, blk, prompt_len: int, block_len: int, tau: float, k_min: int):
    """One commit of semi-autoregressive block decoding (SlowFast, German summary page,
    "Der SlowFast-Algorithmus" item 2: tokens of the current region whose confidence is above a
    high threshold are decoded together; when too few are, a top-k update keeps progress).

    Per sequence b, with the active block [P + blk[b] L, P + (blk[b] + 1) L) (clipped to S):
      m = its masked positions (tok < 0); for s in m, conf_s and arg_s from the logit row
      (conf rounded to float32, the precision the decision is taken in);
      commit C = the n best of m by (conf descending, position ascending), where
      n = max(#{conf_s > tau}, min(k_min, |m|)); tok[b, s] = arg_s for s in C.
    When the active block has no masked position left, blk[b] advances by one (at most to the
    number of blocks, which means done). The next step's selection flags force the positions of
    the (possibly new) active block.

    logits [B, S, V] (anything indexable as logits[b, s] -> a row; only active-block rows are
    read); tok int [B, S] (-1 = masked); blk int [B].
    Returns (tok', blk', committed ids (flat b S + s, ascending per sequence), row_ptr,
             flags uint8 [B, S]).
    """
    tok = np.array(tok, dtype=np.int64, copy=True)
    blk = np.array(blk, dtype=np.int64, copy=True)
    B, S = tok.shape
    nblk = -(-(S - prompt_len) // block_len)
    tau32 = np.float32(tau)
    sel, rp = [], [0]
    flags = np.zeros((B, S), dtype=np.uint8)
    for b in range(B):
        if blk[b] < nblk:
            lo = prompt_len + int(blk[b]) * block_len
            hi = min(S, lo + block_len)
            masked = [s for s in range(lo, hi) if tok[b, s] < 0]
            conf, arg = {}, {}
            for s in masked:
                c, a = confidence_argmax(logits[b, s])
                conf[s], arg[s] = np.float32(c), a
            n_above = sum(1 for s in masked if conf[s] > tau32)
            n = max(n_above, min(int(k_min), len(masked)))
            order = sorted(masked, key=lambda s: (-float(conf[s]), s))
            chosen = sorted(order[:n])
            for s in chosen:
                tok[b, s] = arg[s]
            sel.extend(b * S + s for s in chosen)
            if all(tok[b, s] >= 0 for s in range(lo, hi)):
                blk[b] += 1
        rp.append(len(sel))
        if blk[b] < nblk:
            lo = prompt_len + int(blk[b]) * block_len
            flags[b, lo:min(S, lo + block_len)] = 1
    return tok, blk, np.asarray(sel, np.int32), np.asarray(rp, np.int32), flags


def embed_rows(emb, mask_emb, tok, sel_idx, row_ptr, x):
    """x[b, s] = emb[tok[b, s]] for a committed token, the mask embedding for a masked one
    (tok < 0), for the listed positions; other rows of x keep their values. Returns x'."""
    x = np.array(x, dtype=np.float64, copy=True)
    S = x.shape[1]
    for flat in np.asarray(sel_idx[:int(row_ptr[-1])], dtype=np.int64):
        b, s = int(flat) // S, int(flat) % S
        t = int(tok[b, s])
        x[b, s] = np.asarray(emb[t] if t >= 0 else mask_emb, dtype=np.float64)
    return x


def flags_from_rows(force, sel_idx, row_ptr, B: int, S: int):
    """Selection flags that restrict a later selection to the listed rows (ES-dLLM, German
    summary page §2.B: the second skip point ranks only the tokens still being computed): a
    listed position is a candidate, or forced if bit 0 of its `force` flag is set; every other
    position is excluded (flag 2)."""
    flags = np.full((B, S), 2, dtype=np.uint8)
    for flat in np.asarray(sel_idx[:int(row_ptr[-1])], dtype=np.int64):
        b, s = int(flat) // S, int(flat) % S
        flags[b, s] = (int(force[b, s]) & 1) if force is not None else 0
    return flags
