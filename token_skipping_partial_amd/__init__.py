"""Python binding of libdllm.so, the gfx950 HIP library of the token-skipping denoising step.

Argument marshalling only: every function forwards device pointers of torch tensors to the C ABI
declared in include/dllm.h and raises DllmError on a non-OK status. There is no fallback: if the
library is not built, importing this package raises.

    import token_skipping_partial_amd as tsp
    shape = tsp.Shape(B=1, S=1024, d=4096, H=32, Hkv=32, hd=128, F=12288, dtype="bf16", V=126464)
    tsp.dllm_saliency(shape, tsp.DELTA_L1N, 0.5, h_cur, h_prev, logits, score)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdllm.so")

DLLM_OK, DLLM_ERR_INVALID_ARG, DLLM_ERR_UNSUPPORTED, DLLM_ERR_WORKSPACE, DLLM_ERR_HIP = range(5)
F32, BF16 = 0, 1
DELTA_L1N, DELTA_COS, DELTA_L2R = 0, 1, 2
SEL_THRESHOLD, SEL_TOPK = 0, 1
OP_SALIENCY, OP_SELECT, OP_QKV, OP_ATTN, OP_FFN, OP_COMMIT = range(6)
MAX_SELECT_S = 8192
MAX_SALIENT_S = 8192
MAX_BLOCK_LEN = 256
COMMIT_NOALLOC_MAX_ROWS = 65536

EXPORTS = ("dllm_saliency", "dllm_select_compact", "dllm_gather_qkv_scatter_kv",
           "dllm_partial_attn", "dllm_gather_ffn_scatter", "dllm_gather_kv_rows",
           "dllm_salient_attn", "dllm_gather_rows", "dllm_commit", "dllm_commit_noalloc",
           "dllm_embed_rows",
           "dllm_flags_from_rows",
           "dllm_workspace_bytes", "dllm_status_string", "dllm_version")


class DllmError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call} returned {status_string(status)}")
        self.status = status


class Shape(ctypes.Structure):
    """dllm_shape: B, S, d, H, Hkv, hd, F, dtype, V, rms_eps, m_plan (48 bytes).
    m_plan: rows the layer calls tune their launch plans for (0 = m_cap); results cover every
    selected row whatever its value."""
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("d", ctypes.c_int32),
                ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("hd", ctypes.c_int32),
                ("F", ctypes.c_int32), ("dtype", ctypes.c_int32), ("V", ctypes.c_int64),
                ("rms_eps", ctypes.c_float), ("m_plan", ctypes.c_int32)]

    def __init__(self, B=1, S=1, d=64, H=1, Hkv=1, hd=64, F=64, dtype="bf16", V=0,
                 rms_eps=1e-5, m_plan=0):
        dt = {"bf16": BF16, "f32": F32, BF16: BF16, F32: F32}[dtype]
        super().__init__(B, S, d, H, Hkv, hd, F, dt, V, rms_eps, m_plan)

    def with_plan(self, m_plan: int) -> "Shape":
        """A copy of this shape with another m_plan."""
        s = Shape()
        ctypes.pointer(s)[0] = self
        s.m_plan = int(m_plan)
        return s

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == BF16 else torch.float32

    def __repr__(self):
        return (f"Shape(B={self.B}, S={self.S}, d={self.d}, H={self.H}, Hkv={self.Hkv}, "
                f"hd={self.hd}, F={self.F}, dtype={'bf16' if self.dtype == BF16 else 'f32'}, "
                f"V={self.V}, rms_eps={self.rms_eps}, m_plan={self.m_plan})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python token_skipping_partial_amd/build.py`"
                          " (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    SP = ctypes.POINTER(Shape)
    sigs = {
        "dllm_saliency": (I32, [SP, I32, F, P, P, P, P, P, P, P]),
        "dllm_select_compact": (I32, [SP, I32, F, I32, P, P, P, P, P, SZ, P]),
        "dllm_gather_qkv_scatter_kv": (I32, [SP, P, P, P, P, P, I32, P, P, P, P, SZ, P]),
        "dllm_partial_attn": (I32, [SP, F, P, P, P, P, P, I32, P, P, SZ, P]),
        "dllm_gather_ffn_scatter": (I32, [SP, P, P, P, P, P, P, P, P, P, I32, P, P, SZ, P]),
        "dllm_gather_kv_rows": (I32, [SP, P, P, P, P, I32, P, P, P]),
        "dllm_salient_attn": (I32, [SP, F, P, P, P, P, P, P, P, P, I32, I32, P, P, P, P, P, P, SZ,
                                    P]),
        "dllm_gather_rows": (I32, [SP, P, I32, P, P, I32, P, P]),
        "dllm_commit": (I32, [SP, P, I32, I32, F, I32, P, P, P, P, P, P, SZ, P]),
        "dllm_commit_noalloc": (I32, [SP, P, I32, I32, F, I32, P, P, P, P, P, P]),
        "dllm_embed_rows": (I32, [SP, P, P, P, P, P, I32, P, P]),
        "dllm_flags_from_rows": (I32, [SP, P, P, P, I32, P, P]),
        "dllm_workspace_bytes": (SZ, [I32, SP, I32]),
        "dllm_status_string": (ctypes.c_char_p, [I32]),
        "dllm_version": (I32, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.dllm_status_string(int(status)).decode()


def version() -> int:
    return _lib.dllm_version()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, call: str):
    if status != DLLM_OK:
        raise DllmError(status, call)


def dllm_workspace_bytes(op: int, shape: Shape, m_cap: int) -> int:
    n = _lib.dllm_workspace_bytes(op, ctypes.byref(shape), int(m_cap))
    if n == ctypes.c_size_t(-1).value:
        raise DllmError(DLLM_ERR_INVALID_ARG, "dllm_workspace_bytes")
    return n


def workspace(op: int, shape: Shape, m_cap: int, device="cuda") -> torch.Tensor:
    """Allocate the workspace a call needs (at least 256 bytes so the pointer is never NULL)."""
    n = max(256, dllm_workspace_bytes(op, shape, m_cap))
    return torch.empty(n, dtype=torch.uint8, device=device)


def dllm_saliency(shape, delta_kind, alpha, h_cur, h_prev, logits, score, conf_out=None,
                  delta_out=None, stream=None):
    _check(_lib.dllm_saliency(ctypes.byref(shape), int(delta_kind), float(alpha), _ptr(h_cur),
                              _ptr(h_prev), _ptr(logits), _ptr(score), _ptr(conf_out),
                              _ptr(delta_out), _stream(stream)), "dllm_saliency")


def dllm_select_compact(shape, mode, tau, k, score, force, sel_idx, row_ptr, ws=None,
                        stream=None):
    nbytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(_lib.dllm_select_compact(ctypes.byref(shape), int(mode), float(tau), int(k),
                                    _ptr(score), _ptr(force), _ptr(sel_idx), _ptr(row_ptr),
                                    _ptr(ws), nbytes, _stream(stream)), "dllm_select_compact")


def _ws(ws):
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


def dllm_gather_qkv_scatter_kv(shape, h_in, g_attn, w_qkv, sel_idx, row_ptr, m_cap, q_sel,
                               k_cache, v_cache, ws, stream=None):
    wp, wn = _ws(ws)
    _check(_lib.dllm_gather_qkv_scatter_kv(ctypes.byref(shape), _ptr(h_in), _ptr(g_attn),
                                           _ptr(w_qkv), _ptr(sel_idx), _ptr(row_ptr), int(m_cap),
                                           _ptr(q_sel), _ptr(k_cache), _ptr(v_cache), wp, wn,
                                           _stream(stream)), "dllm_gather_qkv_scatter_kv")


def dllm_partial_attn(shape, scale, q_sel, k_cache, v_cache, sel_idx, row_ptr, m_cap, o_sel, ws,
                      stream=None):
    wp, wn = _ws(ws)
    _check(_lib.dllm_partial_attn(ctypes.byref(shape), float(scale), _ptr(q_sel), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(sel_idx), _ptr(row_ptr), int(m_cap),
                                  _ptr(o_sel), wp, wn, _stream(stream)), "dllm_partial_attn")


def dllm_gather_ffn_scatter(shape, h_in, o_sel, w_o, g_ffn, w_gate, w_up, w_down, sel_idx,
                            row_ptr, m_cap, h_out, ws, stream=None):
    wp, wn = _ws(ws)
    _check(_lib.dllm_gather_ffn_scatter(ctypes.byref(shape), _ptr(h_in), _ptr(o_sel), _ptr(w_o),
                                        _ptr(g_ffn), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                        _ptr(sel_idx), _ptr(row_ptr), int(m_cap), _ptr(h_out),
                                        wp, wn, _stream(stream)), "dllm_gather_ffn_scatter")


def dllm_gather_kv_rows(shape, k_cache, v_cache, sel_idx, row_ptr, m_cap, k_rows, v_rows,
                        stream=None):
    _check(_lib.dllm_gather_kv_rows(ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(sel_idx), _ptr(row_ptr), int(m_cap), _ptr(k_rows),
                                    _ptr(v_rows), _stream(stream)), "dllm_gather_kv_rows")


def dllm_salient_attn(shape, scale, q_sel, q_all, k_cache, v_cache, k_old, v_old, sel_idx,
                      row_ptr, m_cap, st_m, st_l, st_o, o_sel, o_all, ws, stream=None, q_first=0):
    """q_first (keyword here, after m_cap in the C call): unselected positions before it are
    left out of the step (response-only steps)."""
    wp, wn = _ws(ws)
    _check(_lib.dllm_salient_attn(ctypes.byref(shape), float(scale), _ptr(q_sel), _ptr(q_all),
                                  _ptr(k_cache), _ptr(v_cache), _ptr(k_old), _ptr(v_old),
                                  _ptr(sel_idx), _ptr(row_ptr), int(m_cap), int(q_first),
                                  _ptr(st_m),
                                  _ptr(st_l), _ptr(st_o), _ptr(o_sel), _ptr(o_all), wp, wn,
                                  _stream(stream)), "dllm_salient_attn")


def dllm_gather_rows(shape, src, width, sel_idx, row_ptr, m_cap, dst, stream=None):
    _check(_lib.dllm_gather_rows(ctypes.byref(shape), _ptr(src), int(width), _ptr(sel_idx),
                                 _ptr(row_ptr), int(m_cap), _ptr(dst), _stream(stream)),
           "dllm_gather_rows")


def dllm_commit(shape, logits, prompt_len, block_len, tau, k_min, tok, blk, committed_idx,
                committed_rp, flags, ws, stream=None):
    wp, wn = _ws(ws)
    _check(_lib.dllm_commit(ctypes.byref(shape), _ptr(logits), int(prompt_len), int(block_len),
                            float(tau), int(k_min), _ptr(tok), _ptr(blk), _ptr(committed_idx),
                            _ptr(committed_rp), _ptr(flags), wp, wn, _stream(stream)),
           "dllm_commit")


def dllm_commit_noalloc(shape, logits, prompt_len, block_len, tau, k_min, tok, blk,
                        committed_idx, committed_rp, flags, stream=None):
    """dllm_commit with the library's static device scratch instead of a workspace."""
    _check(_lib.dllm_commit_noalloc(ctypes.byref(shape), _ptr(logits), int(prompt_len),
                                    int(block_len), float(tau), int(k_min), _ptr(tok), _ptr(blk),
                                    _ptr(committed_idx), _ptr(committed_rp), _ptr(flags),
                                    _stream(stream)), "dllm_commit_noalloc")


def dllm_embed_rows(shape, emb, mask_emb, tok, sel_idx, row_ptr, m_cap, x, stream=None):
    _check(_lib.dllm_embed_rows(ctypes.byref(shape), _ptr(emb), _ptr(mask_emb), _ptr(tok),
                                _ptr(sel_idx), _ptr(row_ptr), int(m_cap), _ptr(x),
                                _stream(stream)), "dllm_embed_rows")


def dllm_flags_from_rows(shape, force, sel_idx, row_ptr, m_cap, flags, stream=None):
    _check(_lib.dllm_flags_from_rows(ctypes.byref(shape), _ptr(force), _ptr(sel_idx),
                                     _ptr(row_ptr), int(m_cap), _ptr(flags), _stream(stream)),
           "dllm_flags_from_rows")
