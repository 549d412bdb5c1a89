"""ctypes binding of the C++ oracle (oracle/dllm_oracle.cpp). TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this module.
The functions carry the names and signatures of the float64 numpy oracle (oracle/dllm_ref.py),
which stays as a second, independently written checker. Arrays go to the C++ code as they are:
uint16 arrays are bfloat16 bit patterns (decoded there), float32 and float64 arrays are passed
in their own type; everything else is converted to float64 first.

`store` (projection, attention, FFN and layer calls): the type the library stores q rows, K/V
cache rows, attention outputs and hidden rows in -- "f64" (default: no rounding), "f32" or
"bf16" (round to nearest even). The rounded values come back as float64 arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .dllm_ref import DELTA_COS, DELTA_L1N, DELTA_L2R, SEL_THRESHOLD, SEL_TOPK, as_f64, decode_bf16

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle_dllm.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python oracle/build.py` "
                      "(or __graft_entry__.build())")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_i32, _i64, _f32, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
_STORE = {"f32": 0, "bf16": 1, "f64": 2, None: 2}


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "S", "d", "H", "Hkv", "hd", "F")]


def _sig(name, args, res=None):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_sig("ora_set_threads", [ctypes.c_int])
_sig("ora_threads", [], ctypes.c_int)
_sig("ora_round_bf16", [_f64], _f64)
_sig("ora_delta", [_i64, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int, _P, ctypes.c_int, _P])
_sig("ora_confidence", [_i64, _i64, _P, ctypes.c_int, _P, _P])
_sig("ora_saliency", [_i64, ctypes.c_int, _i64, ctypes.c_int, _f64, _P, ctypes.c_int, _P,
                      ctypes.c_int, _P, ctypes.c_int, _P, _P, _P, _P])
_sig("ora_select", [ctypes.c_int, ctypes.c_int, ctypes.c_int, _f32, ctypes.c_int, _P, _P, _P, _P])
_sig("ora_flags_from_rows", [ctypes.c_int, ctypes.c_int, _P, _P, _P, _P])
_sig("ora_rms_norm", [_i64, ctypes.c_int, _P, _P, _f64, _P])
_sig("ora_silu", [_i64, _P, _P])
_sig("ora_qkv", [_P, _f64, ctypes.c_int, _P, ctypes.c_int, _P, ctypes.c_int, _P, ctypes.c_int,
                 _P, _P, _P, _P, _P])
_sig("ora_attn", [_P, _f64, ctypes.c_int, _P, _P, _P, _P, _P, _P])
_sig("ora_ffn", [_P, _f64, ctypes.c_int, _P, ctypes.c_int, _P, _P, _P, ctypes.c_int, _P, _P, _P,
                 ctypes.c_int, _P, _P, _P])
_sig("ora_dense_layer", [_P, _f64, _f64] + [_P] * 11)
_sig("ora_gather_kv_rows", [_P, _P, _P, _P, _P, _P, _P])
_sig("ora_context_all", [_P, _f64, _P, _P, _P, _P, _P])
_sig("ora_salient_attention", [_P, _f64, _P, _P, _P, _P, _P, _P, ctypes.c_int, _P, _P, _P, _P])
_sig("ora_confidence_argmax", [_i64, _P, ctypes.c_int, _P, _P])
_sig("ora_commit", [ctypes.c_int, ctypes.c_int, _i64, _P, ctypes.c_int, _P, ctypes.c_int,
                    ctypes.c_int, _f32, ctypes.c_int, _P, _P, _P, _P, _P])
_sig("ora_embed_rows", [ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int, _P,
                        ctypes.c_int, _P, _P, _P, _P])


def set_threads(n: int) -> None:
    """Worker threads of the C++ oracle (0 = one per hardware thread)."""
    _lib.ora_set_threads(int(n))


def threads() -> int:
    return int(_lib.ora_threads())


def round_bf16(x: float) -> float:
    """The oracle's own round-to-nearest-even of a float64 to bfloat16 (value as float64)."""
    return float(_lib.ora_round_bf16(float(x)))


# ------------------------------------------------------------------ marshalling (no arithmetic)
def _typed(x):
    """(contiguous array, type code): uint16 -> bfloat16 bits (1), float32 (0), float64 (2)."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return np.ascontiguousarray(a), 1
    if a.dtype == np.float32:
        return np.ascontiguousarray(a), 0
    return np.ascontiguousarray(a, dtype=np.float64), 2


def _f64a(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32a(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(B, S, d, H, Hkv, hd, F):
    return _Dims(int(B), int(S), int(d), int(H), int(Hkv), int(hd), int(F))


def _sel(sel_idx, row_ptr):
    rp = _i32a(row_ptr)
    M = int(rp[-1])
    sel = _i32a(np.asarray(sel_idx)[:M]) if M else np.zeros(1, dtype=np.int32)
    return sel, rp, M


# ------------------------------------------------------------------ (1) saliency
def delta_variation(h_cur, h_prev, kind: int = DELTA_L1N) -> np.ndarray:
    x, xt = _typed(h_cur)
    y, yt = _typed(h_prev)
    d = x.shape[-1]
    out = np.empty(x.shape[:-1], dtype=np.float64)
    _lib.ora_delta(x.size // d, d, int(kind), _ptr(x), xt, _ptr(y), yt, _ptr(out))
    return out


def max_softmax_confidence(logits) -> np.ndarray:
    z, zt = _typed(logits)
    V = z.shape[-1]
    out = np.empty(z.shape[:-1], dtype=np.float64)
    _lib.ora_confidence(z.size // V, V, _ptr(z), zt, _ptr(out), None)
    return out


def saliency(h_cur, h_prev, logits, alpha: float, kind: int = DELTA_L1N, conf=None):
    """(score float32 [...], conf float64 or None, delta float64 or None), as the numpy oracle."""
    x = y = z = cin = None
    xt = yt = zt = 2
    if h_cur is not None:
        x, xt = _typed(h_cur)
        y, yt = _typed(h_prev)
    if logits is not None:
        z, zt = _typed(logits)
    elif conf is not None:
        cin = _f64a(conf)
    if x is not None:
        shape = x.shape[:-1]
    elif z is not None:
        shape = z.shape[:-1]
    else:
        shape = cin.shape
    ntok = int(np.prod(shape)) if shape else 1
    d = x.shape[-1] if x is not None else 0
    V = z.shape[-1] if z is not None else 0
    score = np.empty(shape, dtype=np.float32)
    c_out = np.empty(shape, dtype=np.float64)
    v_out = np.empty(shape, dtype=np.float64)
    _lib.ora_saliency(ntok, d, V, int(kind), float(alpha), _ptr(x), xt, _ptr(y), yt, _ptr(z), zt,
                      _ptr(cin), _ptr(score), _ptr(c_out), _ptr(v_out))
    has_conf = z is not None or cin is not None
    return score, (c_out if has_conf else None), (v_out if x is not None else None)


# ------------------------------------------------------------------ (2) selection
def select_compact(score, force, mode: int, tau: float = 0.0, k: int = 0):
    sc = np.ascontiguousarray(np.asarray(score, dtype=np.float32))
    B, S = sc.shape
    fl = None if force is None else np.ascontiguousarray(np.asarray(force).astype(np.uint8))
    sel = np.empty(B * S + 1, dtype=np.int32)
    rp = np.empty(B + 1, dtype=np.int32)
    _lib.ora_select(B, S, int(mode), float(np.float32(tau)), int(k), _ptr(sc), _ptr(fl),
                    _ptr(sel), _ptr(rp))
    return sel[: rp[-1]].copy(), rp


def flags_from_rows(force, sel_idx, row_ptr, B: int, S: int):
    sel, rp, _ = _sel(sel_idx, row_ptr)
    fl = None if force is None else np.ascontiguousarray(np.asarray(force).astype(np.uint8))
    out = np.empty((B, S), dtype=np.uint8)
    _lib.ora_flags_from_rows(B, S, _ptr(fl), _ptr(sel), _ptr(rp), _ptr(out))
    return out


def rms_norm(x, g, eps: float):
    x = _f64a(x)
    d = x.shape[-1]
    g = _f64a(np.broadcast_to(np.asarray(g, dtype=np.float64), (d,)))
    out = np.empty_like(x)
    _lib.ora_rms_norm(x.size // d, d, _ptr(x), _ptr(g), float(eps), _ptr(out))
    return out


def silu(x):
    a = _f64a(x)
    out = np.empty_like(a)
    _lib.ora_silu(a.size, _ptr(a), _ptr(out))
    return out if out.ndim else float(out)


# ------------------------------------------------------------------ (3)-(5) layer calls
def _common_weights(*ws):
    """Weights of one call in one type: bfloat16 bits if all are, else float64."""
    if all(np.asarray(w).dtype == np.uint16 for w in ws):
        return [np.ascontiguousarray(w) for w in ws], 1
    return [_f64a(as_f64(w)) for w in ws], 2


def gather_qkv_scatter_kv(h_in, g_attn, w_qkv, sel_idx, row_ptr, k_cache, v_cache,
                          H: int, Hkv: int, hd: int, eps: float, store=None):
    h, ht = _typed(h_in)
    g, gt = _typed(g_attn)
    w, wt = _typed(w_qkv)
    B, S, d = h.shape
    sel, rp, M = _sel(sel_idx, row_ptr)
    q = np.empty((M, H * hd), dtype=np.float64)
    k_new = np.array(as_f64(k_cache), dtype=np.float64, copy=True)
    v_new = np.array(as_f64(v_cache), dtype=np.float64, copy=True)
    dm = _dims(B, S, d, H, Hkv, hd, 0)
    _lib.ora_qkv(ctypes.byref(dm), float(eps), _STORE[store], _ptr(h), ht, _ptr(g), gt, _ptr(w),
                 wt, _ptr(sel), _ptr(rp), _ptr(q), _ptr(k_new), _ptr(v_new))
    return q, k_new, v_new


def partial_attn(q_sel, k_cache, v_cache, sel_idx, row_ptr, H: int, Hkv: int, hd: int,
                 scale: float, store=None):
    kc, vc = _f64a(as_f64(k_cache)), _f64a(as_f64(v_cache))
    B, _, S, _ = kc.shape
    sel, rp, M = _sel(sel_idx, row_ptr)
    q = _f64a(as_f64(q_sel))[:M] if M else np.zeros((1, H * hd))
    q = np.ascontiguousarray(q)
    out = np.empty((M, H * hd), dtype=np.float64)
    dm = _dims(B, S, 0, H, Hkv, hd, 0)
    _lib.ora_attn(ctypes.byref(dm), float(scale), _STORE[store], _ptr(q), _ptr(kc), _ptr(vc),
                  _ptr(sel), _ptr(rp), _ptr(out))
    return out


def gather_ffn_scatter(h_in, o_sel, w_o, g_ffn, w_gate, w_up, w_down, sel_idx, row_ptr,
                       h_out, eps: float, store=None):
    h, ht = _typed(h_in)
    B, S, d = h.shape
    sel, rp, M = _sel(sel_idx, row_ptr)
    (wo, wg, wu, wd), wt = _common_weights(w_o, w_gate, w_up, w_down)
    g, gt = _typed(g_ffn)
    o = np.ascontiguousarray(_f64a(as_f64(o_sel))[:M]) if M else np.zeros((1, wo.shape[1]))
    out = np.array(as_f64(h_out), dtype=np.float64, copy=True)
    F = wg.shape[0]
    H_hd = wo.shape[1]
    dm = _dims(B, S, d, 1, 1, H_hd, F)   # H * hd is all the FFN call needs
    _lib.ora_ffn(ctypes.byref(dm), float(eps), _STORE[store], _ptr(h), ht, _ptr(o), _ptr(wo),
                 _ptr(g), gt, _ptr(wg), _ptr(wu), _ptr(wd), wt, _ptr(sel), _ptr(rp), _ptr(out))
    return out


def selected_layer(h_in, wts: dict, sel_idx, row_ptr, k_cache, v_cache, h_out,
                   H: int, Hkv: int, hd: int, eps: float, scale: float, store=None):
    """qkv+scatter -> partial attention -> ffn+scatter; returns (q_sel, o_sel, k', v', h_out')."""
    q, k_new, v_new = gather_qkv_scatter_kv(h_in, wts["g_attn"], wts["w_qkv"], sel_idx, row_ptr,
                                            k_cache, v_cache, H, Hkv, hd, eps, store)
    o = partial_attn(q, k_new, v_new, sel_idx, row_ptr, H, Hkv, hd, scale, store)
    out = gather_ffn_scatter(h_in, o, wts["w_o"], wts["g_ffn"], wts["w_gate"], wts["w_up"],
                             wts["w_down"], sel_idx, row_ptr, h_out, eps, store)
    return q, o, k_new, v_new, out


def dense_layer(h, wts: dict, H: int, Hkv: int, hd: int, eps: float, scale: float):
    hh = _f64a(as_f64(h))
    B, S, d = hh.shape
    f = {k: _f64a(as_f64(v)) for k, v in wts.items()}
    F = f["w_gate"].shape[0]
    k = np.empty((B, Hkv, S, hd))
    v = np.empty((B, Hkv, S, hd))
    y = np.empty((B, S, d))
    dm = _dims(B, S, d, H, Hkv, hd, F)
    _lib.ora_dense_layer(ctypes.byref(dm), float(eps), float(scale), _ptr(hh),
                         _ptr(_f64a(np.broadcast_to(f["g_attn"], (d,)))), _ptr(f["w_qkv"]),
                         _ptr(f["w_o"]), _ptr(_f64a(np.broadcast_to(f["g_ffn"], (d,)))),
                         _ptr(f["w_gate"]), _ptr(f["w_up"]), _ptr(f["w_down"]), _ptr(k), _ptr(v),
                         _ptr(y))
    return k, v, y


# ------------------------------------------------------------------ context of every token
def gather_kv_rows(k_cache, v_cache, sel_idx, row_ptr):
    kc, vc = _f64a(as_f64(k_cache)), _f64a(as_f64(v_cache))
    B, Hkv, S, hd = kc.shape
    sel, rp, M = _sel(sel_idx, row_ptr)
    kr = np.empty((M, Hkv, hd))
    vr = np.empty((M, Hkv, hd))
    dm = _dims(B, S, 0, Hkv, Hkv, hd, 0)
    _lib.ora_gather_kv_rows(ctypes.byref(dm), _ptr(kc), _ptr(vc), _ptr(sel), _ptr(rp), _ptr(kr),
                            _ptr(vr))
    return kr, vr


def context_all(q_all, k_cache, v_cache, H: int, Hkv: int, hd: int, scale: float):
    kc, vc = _f64a(as_f64(k_cache)), _f64a(as_f64(v_cache))
    B, _, S, _ = kc.shape
    q = _f64a(as_f64(q_all)).reshape(B, S, H * hd)
    o = np.empty((B, S, H * hd))
    lse = np.empty((B, S, H))
    dm = _dims(B, S, 0, H, Hkv, hd, 0)
    _lib.ora_context_all(ctypes.byref(dm), float(scale), _ptr(q), _ptr(kc), _ptr(vc), _ptr(o),
                         _ptr(lse))
    return o, lse


def salient_attention(q_sel, q_all, k_cache, v_cache, sel_idx, row_ptr, H: int, Hkv: int,
                      hd: int, scale: float, q_first: int = 0, o_prev=None, lse_prev=None):
    """Returns (q_all' [B, S, H*hd], o [B, S, H*hd], lse [B, S, H]) as the numpy oracle."""
    kc, vc = _f64a(as_f64(k_cache)), _f64a(as_f64(v_cache))
    B, _, S, _ = kc.shape
    sel, rp, M = _sel(sel_idx, row_ptr)
    qa = np.array(as_f64(q_all), dtype=np.float64, copy=True).reshape(B, S, H * hd)
    qs = np.ascontiguousarray(_f64a(as_f64(q_sel))[:M]) if M else np.zeros((1, H * hd))
    o = np.empty((B, S, H * hd))
    lse = np.empty((B, S, H))
    op = _f64a(as_f64(o_prev)).reshape(B, S, H * hd) if o_prev is not None else np.zeros((B, S, H * hd))
    lp = _f64a(as_f64(lse_prev)).reshape(B, S, H) if lse_prev is not None else np.zeros((B, S, H))
    dm = _dims(B, S, 0, H, Hkv, hd, 0)
    _lib.ora_salient_attention(ctypes.byref(dm), float(scale), _ptr(qs), _ptr(qa), _ptr(kc),
                               _ptr(vc), _ptr(sel), _ptr(rp), int(q_first), _ptr(op), _ptr(lp),
                               _ptr(o), _ptr(lse))
    return qa, o, lse


# ------------------------------------------------------------------ decode loop
def confidence_argmax(logits_row):
    z, zt = _typed(logits_row)
    conf = ctypes.c_double()
    arg = ctypes.c_int64()
    _lib.ora_confidence_argmax(z.size, _ptr(z), zt, ctypes.byref(conf), ctypes.byref(arg))
    return float(conf.value), int(arg.value)


def commit_step(logits, tok, blk, prompt_len: int, block_len: int, tau: float, k_min: int):
    """Returns (tok', blk', committed ids, row_ptr, flags uint8 [B, S]) as the numpy oracle.
    logits: an array [B, S, V], or any object indexable as logits[b, s] -> one row (then only
    the rows of the active blocks are read)."""
    t = np.array(tok, dtype=np.int32, copy=True)
    b = np.array(blk, dtype=np.int32, copy=True)
    B, S = t.shape
    row_of = None
    if hasattr(logits, "shape") and hasattr(logits, "dtype"):
        z, zt = _typed(logits)
    else:   # rows on demand: gather the active blocks' rows into one array
        nblk = -(-(S - prompt_len) // block_len)
        pos = [(bb, s) for bb in range(B) if b[bb] < nblk
               for s in range(prompt_len + b[bb] * block_len,
                              min(S, prompt_len + (b[bb] + 1) * block_len))]
        rows = [np.asarray(logits[bb, s]) for bb, s in pos]
        z, zt = _typed(np.stack(rows) if rows else np.zeros((1, 1)))
        row_of = np.full(B * S, -1, dtype=np.int32)
        for i, (bb, s) in enumerate(pos):
            row_of[bb * S + s] = i
    V = z.shape[-1]
    cidx = np.empty(max(1, B * block_len), dtype=np.int32)
    crp = np.empty(B + 1, dtype=np.int32)
    flags = np.empty((B, S), dtype=np.uint8)
    _lib.ora_commit(B, S, V, _ptr(z), zt, _ptr(row_of), int(prompt_len), int(block_len),
                    float(np.float32(tau)), int(k_min), _ptr(t), _ptr(b), _ptr(cidx), _ptr(crp),
                    _ptr(flags))
    return t.astype(np.int64), b.astype(np.int64), cidx[: crp[-1]].copy(), crp, flags


def embed_rows(emb, mask_emb, tok, sel_idx, row_ptr, x):
    e, et = _typed(emb)
    mk, mt = _typed(mask_emb)
    out = np.array(as_f64(x), dtype=np.float64, copy=True)
    B, S, d = out.shape
    t = _i32a(tok)
    sel, rp, _ = _sel(sel_idx, row_ptr)
    rp_b = rp if rp.size == B + 1 else np.array([0] * B + [int(rp[-1])], dtype=np.int32)
    _lib.ora_embed_rows(B, S, d, _ptr(e), et, _ptr(mk), mt, _ptr(t), _ptr(sel), _ptr(rp_b),
                        _ptr(out))
    return out


__all__ = [
    "DELTA_COS", "DELTA_L1N", "DELTA_L2R", "SEL_THRESHOLD", "SEL_TOPK", "as_f64", "commit_step",
    "confidence_argmax", "context_all", "decode_bf16", "delta_variation", "dense_layer",
    "embed_rows", "flags_from_rows", "gather_ffn_scatter", "gather_kv_rows",
    "gather_qkv_scatter_kv", "max_softmax_confidence", "partial_attn", "rms_norm", "round_bf16",
    "salient_attention", "saliency", "select_compact", "selected_layer", "set_threads", "silu",
    "threads",
]
