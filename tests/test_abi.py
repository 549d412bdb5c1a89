"""C-ABI checks that need no GPU: the library loads, exports what include/dllm.h declares, sizes
workspaces on the host, and rejects bad arguments before enqueuing anything.

The pointers passed below are fake (aligned integers): every case is rejected by host-side
validation, so nothing is ever dereferenced or launched.
"""
import ctypes
import os
import re

import pytest

import token_skipping_partial_amd as tsp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dllm.h")

P = 0x10000  # fake, 16-byte aligned "device" pointer


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dllm_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("dllm_saliency", "dllm_select_compact", "dllm_gather_qkv_scatter_kv",
              "dllm_partial_attn", "dllm_gather_ffn_scatter"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tsp.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(tsp.EXPORTS) == set(declared_functions())


def test_shape_struct_layout():
    assert ctypes.sizeof(tsp.Shape) == 48
    assert tsp.Shape.V.offset == 32 and tsp.Shape.rms_eps.offset == 40
    assert tsp.Shape.m_plan.offset == 44


def test_status_strings_and_version():
    assert tsp.status_string(0) == "DLLM_OK"
    assert tsp.status_string(3) == "DLLM_ERR_WORKSPACE"
    assert tsp.status_string(99) == "DLLM_ERR_UNKNOWN"
    assert tsp.version() >= 100


def llada(B=1, S=1024, dtype="bf16"):
    return tsp.Shape(B=B, S=S, d=4096, H=32, Hkv=32, hd=128, F=12288, dtype=dtype, V=126464)


def test_workspace_sizes():
    s = llada()
    assert tsp.dllm_workspace_bytes(tsp.OP_SALIENCY, s, 128) == 0
    assert tsp.dllm_workspace_bytes(tsp.OP_SELECT, s, 128) == 0
    q = tsp.dllm_workspace_bytes(tsp.OP_QKV, s, 128)
    f = tsp.dllm_workspace_bytes(tsp.OP_FFN, s, 128)
    assert q >= 128 * 4096 * 2                       # normalised rows
    assert f >= 128 * 4096 * 4 + 128 * 4096 * 2 + 128 * 12288 * 2
    assert tsp.dllm_workspace_bytes(tsp.OP_QKV, s, 0) == 0
    with pytest.raises(tsp.DllmError):
        tsp.dllm_workspace_bytes(7, s, 128)
    with pytest.raises(tsp.DllmError):
        tsp.dllm_workspace_bytes(tsp.OP_QKV, s, 1025)  # m_cap > B*S


def test_workspace_covers_every_planned_row_count():
    """With m_plan > 0 the size does not depend on m_plan and covers the m_cap plan, so a caller
    may change m_plan between calls; m_plan above m_cap plans for m_cap."""
    for s, cap in ((llada(), 1024), (llada(B=8), 1640),
                   (tsp.Shape(B=16, S=2048, d=3584, H=28, Hkv=4, hd=128, F=18944), 16384),
                   (tsp.Shape(B=2, S=160, d=256, H=8, Hkv=2, hd=64, F=512), 320)):
        for op in (tsp.OP_QKV, tsp.OP_ATTN, tsp.OP_FFN):
            base = tsp.dllm_workspace_bytes(op, s, cap)
            sizes = {tsp.dllm_workspace_bytes(op, s.with_plan(p), cap)
                     for p in (1, 2, 64, 65, 100, 128, 129, 200, 256, 257, 300, 1000, cap, 10 * cap)}
            assert len(sizes) == 1 and sizes.pop() >= base
            assert tsp.dllm_workspace_bytes(op, s.with_plan(0), cap) == base


def rc(fn, *args):
    with pytest.raises(tsp.DllmError) as e:
        fn(*args)
    return e.value.status


def test_saliency_validation():
    s = llada()
    f = tsp.dllm_saliency
    assert rc(f, s, 0, 0.5, P, P, None, P) == tsp.DLLM_ERR_INVALID_ARG      # alpha>0, no logits
    assert rc(f, s, 0, 0.5, None, None, P, P) == tsp.DLLM_ERR_INVALID_ARG   # alpha<1, no h
    assert rc(f, s, 0, 1.5, P, P, P, P) == tsp.DLLM_ERR_INVALID_ARG         # alpha > 1
    assert rc(f, s, 0, float("nan"), P, P, P, P) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(f, s, 3, 0.5, P, P, P, P) == tsp.DLLM_ERR_INVALID_ARG         # bad delta kind
    assert rc(f, s, 0, 0.5, P, P, P, None) == tsp.DLLM_ERR_INVALID_ARG      # no score
    assert rc(f, s, 0, 0.5, P, None, P, P) == tsp.DLLM_ERR_INVALID_ARG      # h_prev missing
    assert rc(f, s, 0, 0.0, P, P, None, P, P) == tsp.DLLM_ERR_INVALID_ARG   # conf_out w/o logits
    assert rc(f, s, 0, 0.5, None, None, None, P, P) == tsp.DLLM_ERR_INVALID_ARG  # conf in, no h
    assert rc(f, s, 0, 0.5, P + 2, P, P, P) == tsp.DLLM_ERR_INVALID_ARG     # misaligned
    bad = llada(); bad.V = 1001
    assert rc(f, bad, 0, 0.5, P, P, P, P) == tsp.DLLM_ERR_UNSUPPORTED      # V % 8
    bad = llada(); bad.B = 0
    assert rc(f, bad, 0, 0.0, P, P, None, P) == tsp.DLLM_ERR_INVALID_ARG


def test_select_validation():
    s = llada()
    f = tsp.dllm_select_compact
    assert rc(f, s, tsp.SEL_TOPK, 0.0, -1, P, None, P, P) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(f, s, 5, 0.0, 1, P, None, P, P) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(f, s, tsp.SEL_THRESHOLD, float("nan"), 1, P, None, P, P) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(f, s, tsp.SEL_TOPK, 0.0, 1, None, None, P, P) == tsp.DLLM_ERR_INVALID_ARG
    big = llada(S=tsp.MAX_SELECT_S + 1)
    assert rc(f, big, tsp.SEL_TOPK, 0.0, 1, P, None, P, P) == tsp.DLLM_ERR_UNSUPPORTED


def test_layer_call_validation():
    s = llada()
    q, a, ff = tsp.dllm_gather_qkv_scatter_kv, tsp.dllm_partial_attn, tsp.dllm_gather_ffn_scatter
    ws = None
    # NULL required pointer
    assert rc(q, s, None, P, P, P, P, 128, P, P, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(a, s, 0.1, P, P, P, P, None, 128, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(ff, s, P, P, P, P, P, P, P, P, P, 128, None, ws) == tsp.DLLM_ERR_INVALID_ARG
    # m_cap outside [0, B*S]
    assert rc(q, s, P, P, P, P, P, -1, P, P, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(q, s, P, P, P, P, P, 1025, P, P, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    # H % Hkv
    bad = llada(); bad.Hkv = 5
    assert rc(a, bad, 0.1, P, P, P, P, P, 128, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    # unsupported head width / model width
    bad = llada(); bad.hd = 96
    assert rc(a, bad, 0.1, P, P, P, P, P, 128, P, ws) == tsp.DLLM_ERR_UNSUPPORTED
    bad = llada(); bad.d = 4000
    assert rc(ff, bad, P, P, P, P, P, P, P, P, P, 128, P, ws) == tsp.DLLM_ERR_UNSUPPORTED
    # non-finite scale, bad dtype, negative m_plan
    assert rc(a, s, float("inf"), P, P, P, P, P, 128, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    bad = llada(); bad.dtype = 7
    assert rc(q, bad, P, P, P, P, P, 128, P, P, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    bad = llada(); bad.m_plan = -1
    assert rc(q, bad, P, P, P, P, P, 128, P, P, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    # workspace too small (reported before any launch)
    lib = tsp.library()
    need = tsp.dllm_workspace_bytes(tsp.OP_QKV, s, 128)
    st = lib.dllm_gather_qkv_scatter_kv(ctypes.byref(s), P, P, P, P, P, 128, P, P, P, P,
                                        need - 1, None)
    assert st == tsp.DLLM_ERR_WORKSPACE
    need = tsp.dllm_workspace_bytes(tsp.OP_FFN, s, 128)
    st = lib.dllm_gather_ffn_scatter(ctypes.byref(s), P, P, P, P, P, P, P, P, P, 128, P, P,
                                     need - 1, None)
    assert st == tsp.DLLM_ERR_WORKSPACE
    need = tsp.dllm_workspace_bytes(tsp.OP_ATTN, s, 128)
    assert need > 0  # batch 1, M = 128 splits the key range
    st = lib.dllm_partial_attn(ctypes.byref(s), 0.1, P, P, P, P, P, 128, P, P, need - 1, None)
    assert st == tsp.DLLM_ERR_WORKSPACE


def test_context_call_validation():
    s = llada()
    g, c = tsp.dllm_gather_kv_rows, tsp.dllm_salient_attn
    ws = None
    assert rc(g, s, None, P, P, P, 128, P, P) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(g, s, P, P, P, P, 1025, P, P) == tsp.DLLM_ERR_INVALID_ARG      # m_cap > B*S
    assert rc(g, s, P, P, P, P, 128, P + 4, P) == tsp.DLLM_ERR_INVALID_ARG   # misaligned
    bad = llada(); bad.hd = 96
    assert rc(g, bad, P, P, P, P, 128, P, P) == tsp.DLLM_ERR_UNSUPPORTED
    full = (P,) * 6  # q_sel, q_all, k_cache, v_cache, k_old, v_old
    assert rc(c, s, 0.1, *full, None, P, 128, P, P, P, P, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(c, s, 0.1, *full, P, P, 128, P, None, P, P, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(c, s, float("nan"), *full, P, P, 128, P, P, P, P, P, ws) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(c, s, 0.1, P, P + 2, *(P,) * 4, P, P, 128, P, P, P, P, P, ws) == \
        tsp.DLLM_ERR_INVALID_ARG
    f32 = llada(dtype="f32")
    assert rc(c, f32, 0.1, *full, P, P, 128, P, P, P, P, P, ws) == tsp.DLLM_ERR_UNSUPPORTED
    long = llada(S=tsp.MAX_SALIENT_S + 8)
    assert rc(c, long, 0.1, *full, P, P, 128, P, P, P, P, P, ws) == tsp.DLLM_ERR_UNSUPPORTED
    lib = tsp.library()
    need = tsp.dllm_workspace_bytes(tsp.OP_ATTN, s, 128)
    st = lib.dllm_salient_attn(ctypes.byref(s), 0.1, P, P, P, P, P, P, P, P, 128, 0, P, P, P, P,
                               P, P, need - 1, None)
    assert st == tsp.DLLM_ERR_WORKSPACE
    for q_first in (-1, s.S + 1):   # outside [0, S]
        st = lib.dllm_salient_attn(ctypes.byref(s), 0.1, P, P, P, P, P, P, P, P, 128, q_first, P,
                                   P, P, P, P, P, need, None)
        assert st == tsp.DLLM_ERR_INVALID_ARG


def test_gather_rows_validation():
    s = llada()
    g = tsp.dllm_gather_rows
    assert rc(g, s, None, 4096, P, P, 128, P) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(g, s, P, 0, P, P, 128, P) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(g, s, P, 4096, P, P, 1025, P) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(g, s, P, 4, P, P, 128, P) == tsp.DLLM_ERR_UNSUPPORTED   # 8-byte rows


def test_commit_and_embed_validation():
    s = llada()
    c, e = tsp.dllm_commit, tsp.dllm_embed_rows
    need = tsp.dllm_workspace_bytes(tsp.OP_COMMIT, s, 32)
    assert need >= 2 * 32 * 4
    with pytest.raises(tsp.DllmError):
        tsp.dllm_workspace_bytes(tsp.OP_COMMIT, s, tsp.MAX_BLOCK_LEN + 1)
    args = lambda **k: [k.get("shape", s), k.get("logits", P), k.get("prompt", 512),  # noqa: E731
                        k.get("block", 32), k.get("tau", 0.9), k.get("k", 1), P, P, P, P, P, P]
    lib = tsp.library()
    call = lambda a, wsb=need: lib.dllm_commit(ctypes.byref(a[0]), *a[1:], wsb, None)  # noqa
    assert call(args(logits=None)) == tsp.DLLM_ERR_INVALID_ARG
    assert call(args(prompt=-1)) == tsp.DLLM_ERR_INVALID_ARG
    assert call(args(prompt=1025)) == tsp.DLLM_ERR_INVALID_ARG
    assert call(args(block=0)) == tsp.DLLM_ERR_INVALID_ARG
    assert call(args(k=-1)) == tsp.DLLM_ERR_INVALID_ARG
    assert call(args(tau=float("nan"))) == tsp.DLLM_ERR_INVALID_ARG
    assert call(args(logits=P + 4)) == tsp.DLLM_ERR_INVALID_ARG          # misaligned
    assert call(args(block=tsp.MAX_BLOCK_LEN + 1)) == tsp.DLLM_ERR_UNSUPPORTED
    odd = llada(); odd.V = 126460
    assert call(args(shape=odd)) == tsp.DLLM_ERR_UNSUPPORTED            # V % 8 != 0
    assert call(args(), need - 1) == tsp.DLLM_ERR_WORKSPACE
    assert rc(e, s, None, P, P, P, P, 128, P) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(e, s, P, P, P, P, P, 1025, P) == tsp.DLLM_ERR_INVALID_ARG
    assert rc(e, s, P + 8, P, P, P, P, 128, P) == tsp.DLLM_ERR_INVALID_ARG  # misaligned
    small = tsp.Shape(B=1, S=16, d=4, H=1, Hkv=1, hd=64, F=64, dtype="bf16", V=10)
    assert rc(e, small, P, P, P, P, P, 4, P) == tsp.DLLM_ERR_UNSUPPORTED  # 8-byte rows


def test_commit_noalloc_validation():
    """The allocation-free commit rejects what dllm_commit rejects, and a batch whose active-block
    rows exceed its static scratch, before touching the device."""
    lib = tsp.library()
    s = llada()
    args = lambda **k: [k.get("shape", s), k.get("logits", P), k.get("prompt", 512),  # noqa: E731
                        k.get("block", 32), k.get("tau", 0.9), k.get("k", 1), P, P, P, P, P]
    call = lambda a: lib.dllm_commit_noalloc(ctypes.byref(a[0]), *a[1:], None)  # noqa: E731
    assert call(args(logits=None)) == tsp.DLLM_ERR_INVALID_ARG
    assert call(args(block=0)) == tsp.DLLM_ERR_INVALID_ARG
    assert call(args(tau=float("nan"))) == tsp.DLLM_ERR_INVALID_ARG
    assert call(args(logits=P + 4)) == tsp.DLLM_ERR_INVALID_ARG
    assert call(args(block=tsp.MAX_BLOCK_LEN + 1)) == tsp.DLLM_ERR_UNSUPPORTED
    big = tsp.Shape(B=tsp.COMMIT_NOALLOC_MAX_ROWS // 256 + 1, S=1024, d=4096, H=32, Hkv=32,
                    hd=128, F=12288, dtype="bf16", V=126464)
    assert call(args(shape=big, block=256)) == tsp.DLLM_ERR_WORKSPACE
    with pytest.raises(tsp.DllmError, match="DLLM_ERR_WORKSPACE"):
        tsp.dllm_commit_noalloc(big, P, 512, 256, 0.9, 1, P, P, P, P, P)
