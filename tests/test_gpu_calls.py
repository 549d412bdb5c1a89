"""Per-call parity of the HIP library against the CPU oracle on identical seeded inputs.

Shapes span several tiles with ragged tails (odd S, odd M per sequence, empty sequences), the
three head layouts (multi-head, grouped 7:1 and 2:1, single kv head), both head widths, both
storage types, the split-key and split-K launch plans, and the capacity edge cases (m_cap above
and below the selected count).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import TOL, assert_close, host, random_selection, same_bits, to_dev

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def shape_of(tsp, dtype, B, S, d, H, Hkv, hd, F, V=0):
    return tsp.Shape(B=B, S=S, d=d, H=H, Hkv=Hkv, hd=hd, F=F,
                     dtype="bf16" if dtype == BF16 else "f32", V=V)


# ----------------------------------------------------------------------------- (1) saliency
@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("kind", [O.DELTA_L1N, O.DELTA_COS, O.DELTA_L2R])
@pytest.mark.parametrize("alpha,use_h,use_logits", [(0.0, True, False), (0.5, True, True),
                                                    (1.0, False, True), (0.0, True, True),
                                                    (0.25, True, True)])
def test_saliency(lib, dtype, kind, alpha, use_h, use_logits):
    B, S, d, V = 2, 37, 264, 1000
    print(f"saliency dtype={dtype} kind={kind} alpha={alpha} h={use_h} logits={use_logits}",
          flush=True)
    h_prev, h_cur, _ = synth.perturbed_pair(B, S, d, 9, seed=101, dtype=dtype)
    logits = synth.logits(B, S, V, seed=102, dtype=dtype) if use_logits else None
    shape = shape_of(lib, dtype, B, S, d, 4, 4, 64, 64, V)
    score = torch.full((B, S), -7.0, device="cuda")
    conf = torch.full((B, S), -7.0, device="cuda") if use_logits else None
    delta = torch.full((B, S), -7.0, device="cuda") if use_h else None
    lib.dllm_saliency(shape, kind, alpha, to_dev(h_cur) if use_h else None,
                      to_dev(h_prev) if use_h else None,
                      to_dev(logits) if use_logits else None, score, conf, delta)
    torch.cuda.synchronize()
    r_score, r_conf, r_delta = O.saliency(host(h_cur) if use_h else None,
                                          host(h_prev) if use_h else None,
                                          host(logits) if use_logits else None, alpha, kind)
    assert_close(host(score), r_score, 1e-4, "score")
    if use_logits:
        assert_close(host(conf), r_conf, 1e-4, "confidence")
    if use_h:
        assert_close(host(delta), r_delta, 1e-4, "delta")


def test_saliency_llada_vocab(lib):
    """Full LLaDA vocabulary (126464) on 64 tokens: the confidence stream at its real length."""
    B, S, d, V = 1, 64, 4096, 126464
    h_prev, h_cur, _ = synth.perturbed_pair(B, S, d, 10, seed=103, dtype=BF16)
    logits = synth.logits(B, S, V, seed=104, dtype=BF16)
    shape = shape_of(lib, BF16, B, S, d, 32, 32, 128, 12288, V)
    score = torch.empty(B, S, device="cuda")
    conf = torch.empty(B, S, device="cuda")
    lib.dllm_saliency(shape, O.DELTA_L1N, 0.5, to_dev(h_cur), to_dev(h_prev), to_dev(logits),
                      score, conf)
    torch.cuda.synchronize()
    r_score, r_conf, _ = O.saliency(host(h_cur), host(h_prev), host(logits), 0.5)
    assert_close(host(conf), r_conf, 1e-4, "confidence")
    assert_close(host(score), r_score, 1e-4, "score")


# ----------------------------------------------------------------------------- (2) selection
def run_select(lib, score, force, mode, tau, k):
    B, S = score.shape
    shape = lib.Shape(B=B, S=S, d=64)
    sel = torch.full((B * S + 5,), -7, dtype=torch.int32, device="cuda")
    rp = torch.full((B + 1,), -7, dtype=torch.int32, device="cuda")
    lib.dllm_select_compact(shape, mode, tau, k, to_dev(score),
                            to_dev(force.astype(np.uint8)) if force is not None else None, sel, rp)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), rp.cpu().numpy()


def check_select(lib, score_t, force, mode, tau=0.0, k=0):
    score = score_t.numpy().astype(np.float32)
    sel, rp = run_select(lib, score, force, mode, tau, k)
    r_sel, r_rp = O.select_compact(score, force, mode, tau, k)
    assert np.array_equal(rp, r_rp), (rp, r_rp)
    M = int(r_rp[-1])
    assert np.array_equal(sel[:M], r_sel), "selected ids differ"
    assert np.all(sel[M:] == -7), "entries past row_ptr[B] were written"


@pytest.mark.parametrize("kind", ["mixed", "equal", "ties", "random"])
@pytest.mark.parametrize("B,S", [(1, 1), (3, 40), (2, 1000), (1, 8192), (4, 2048)])
@pytest.mark.parametrize("k", [0, 1, 37, 128, 10 ** 6])
def test_select_topk_bit_exact(lib, kind, B, S, k):
    print(f"select topk kind={kind} B={B} S={S} k={k}", flush=True)
    score = synth.adversarial_scores(B, S, seed=200 + S + k, kind=kind)
    rng = np.random.default_rng(S + k)
    force = rng.random((B, S)) < 0.05
    if B > 1:
        force[-1, :] = True  # one sequence entirely forced
    check_select(lib, score, None, O.SEL_TOPK, k=k)
    check_select(lib, score, force, O.SEL_TOPK, k=k)


@pytest.mark.parametrize("kind", ["mixed", "ties", "random"])
@pytest.mark.parametrize("B,S,k", [(1, 1024, 128), (3, 40, 5), (2, 1000, 37), (1, 8192, 64),
                                   (4, 2048, 10 ** 6)])
def test_select_excluded_positions_bit_exact(lib, kind, B, S, k):
    """Flags: bit 0 forced, bit 1 excluded (a prompt half, random holes), forced wins, other bits
    ignored; top-k and threshold."""
    print(f"select flags kind={kind} B={B} S={S} k={k}", flush=True)
    score = synth.adversarial_scores(B, S, seed=700 + S + k, kind=kind)
    rng = np.random.default_rng(S + k + 1)
    flags = np.zeros((B, S), dtype=np.uint8)
    flags[:, : S // 2] = 2
    flags[rng.random((B, S)) < 0.05] |= 1
    flags[rng.random((B, S)) < 0.05] |= 2
    flags[rng.random((B, S)) < 0.05] |= 4
    if B > 1:
        flags[-1, :] = 2
    check_select(lib, score, flags, O.SEL_TOPK, k=k)
    check_select(lib, score, flags, O.SEL_THRESHOLD, tau=0.0)


@pytest.mark.parametrize("kind", ["mixed", "ties", "random"])
@pytest.mark.parametrize("tau", [0.0, 0.5, -0.25, float("inf"), -float("inf")])
def test_select_threshold_bit_exact(lib, kind, tau):
    B, S = 3, 1500
    score = synth.adversarial_scores(B, S, seed=300, kind=kind)
    force = np.random.default_rng(1).random((B, S)) < 0.02
    check_select(lib, score, None, O.SEL_THRESHOLD, tau=tau)
    check_select(lib, score, force, O.SEL_THRESHOLD, tau=tau)


def test_select_deterministic(lib):
    score = synth.adversarial_scores(4, 4096, seed=5, kind="ties").numpy()
    a = run_select(lib, score, None, O.SEL_TOPK, 0.0, 700)
    b = run_select(lib, score, None, O.SEL_TOPK, 0.0, 700)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ----------------------------------------------------------------------------- layer cases
LAYER_CASES = {
    # name: dtype, B, S, d, H, Hkv, hd, F, selected per sequence
    "tiny_f32": (F32, 1, 64, 256, 4, 4, 64, 1024, [16]),
    "f32_gqa_ragged": (F32, 2, 77, 128, 4, 2, 128, 192, [13, 77]),
    "bf16_gqa_ragged": (BF16, 2, 100, 256, 4, 2, 128, 512, [37, 100]),
    "bf16_mqa_hd64": (BF16, 3, 300, 384, 6, 1, 64, 640, [0, 1, 299]),
    "bf16_dream_group7": (BF16, 2, 160, 256, 7, 1, 128, 384, [70, 33]),
    "bf16_llada_layer": (BF16, 1, 1024, 4096, 32, 32, 128, 12288, [128]),
}


def layer_inputs(case, seed):
    dtype, B, S, d, H, Hkv, hd, F, counts = LAYER_CASES[case]
    w = synth.layer_weights(d, H, Hkv, hd, F, seed=seed, dtype=dtype)
    # non-unit norm gains so the gain is exercised
    w["g_attn"] = (1.0 + synth.normal((d,), 0.1, seed + 7)).to(dtype)
    w["g_ffn"] = (1.0 + synth.normal((d,), 0.1, seed + 8)).to(dtype)
    h_in = synth.normal((B, S, d), 1.0, seed + 1, dtype)
    kc = synth.normal((B, Hkv, S, hd), 1.0, seed + 2, dtype)
    vc = synth.normal((B, Hkv, S, hd), 1.0, seed + 3, dtype)
    sel, rp = random_selection(B, S, counts, seed + 4)
    return dtype, (B, S, d, H, Hkv, hd, F), w, h_in, kc, vc, sel, rp


def truncated(sel, rp, m_cap):
    """The selection a capacity of m_cap rows processes: the first m_cap ids."""
    M = min(int(rp[-1]), m_cap)
    return sel[:M], np.minimum(rp, M).astype(np.int32)


# ----------------------------------------------------------------------------- (3) QKV
@pytest.mark.parametrize("case", list(LAYER_CASES))
@pytest.mark.parametrize("cap", ["exact", "over", "under"])
def test_qkv_scatter(lib, case, cap):
    dtype, (B, S, d, H, Hkv, hd, F), w, h_in, kc, vc, sel, rp = layer_inputs(case, 400)
    M = int(rp[-1])
    m_cap = {"exact": M, "over": min(B * S, M + 13), "under": max(0, M - 5)}[cap]
    print(f"qkv case={case} M={M} m_cap={m_cap}", flush=True)
    shape = shape_of(lib, dtype, B, S, d, H, Hkv, hd, F)
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    q_sel = torch.full((max(1, m_cap), H * hd), -3.0, dtype=dtype, device="cuda")
    ws = lib.workspace(lib.OP_QKV, shape, m_cap)
    lib.dllm_gather_qkv_scatter_kv(shape, to_dev(h_in), to_dev(w["g_attn"]), to_dev(w["w_qkv"]),
                                   to_dev(sel), to_dev(rp), m_cap, q_sel, kc_d, vc_d, ws)
    torch.cuda.synchronize()
    s2, rp2 = truncated(sel, rp, m_cap)
    Mt = int(rp2[-1])
    rq, rk, rv = O.gather_qkv_scatter_kv(host(h_in), host(w["g_attn"]), host(w["w_qkv"]), s2, rp2,
                                         host(kc), host(vc), H, Hkv, hd, 1e-5)
    tol = TOL[dtype]
    assert_close(host(q_sel)[:Mt], rq, tol, "q_sel")
    if m_cap > Mt:
        assert np.all(host(q_sel)[Mt:m_cap] == -3.0), "q_sel rows past M were written"
    touched = np.zeros((B, S), dtype=bool)
    touched[s2 // S, s2 % S] = True
    gk, gv = host(kc_d), host(vc_d)
    for name, got, ref, orig in (("k_cache", gk, rk, host(kc)), ("v_cache", gv, rv, host(vc))):
        got_t = got.transpose(0, 2, 1, 3)[touched]   # [rows, Hkv, hd]
        ref_t = ref.transpose(0, 2, 1, 3)[touched]
        assert_close(got_t, ref_t, tol, name)
        assert np.array_equal(got.transpose(0, 2, 1, 3)[~touched],
                              orig.transpose(0, 2, 1, 3)[~touched]), f"{name}: unselected rows"


# ----------------------------------------------------------------------------- (4) attention
ATTN_CASES = {
    # dtype, B, S, H, Hkv, hd, counts, q scale[, softmax scale (default 1/sqrt(hd)), key ramp]
    "f32_tiny": (F32, 1, 64, 4, 4, 64, [16], 1.0),
    "f32_gqa": (F32, 2, 130, 4, 2, 128, [5, 9], 1.0),
    "llada_b1_m128": (BF16, 1, 1024, 32, 32, 128, [128], 1.0),
    "llada_b2_m205": (BF16, 2, 1024, 32, 32, 128, [205, 205], 1.0),
    "dream_gqa7": (BF16, 2, 300, 28, 4, 128, [50, 7], 1.0),
    "hd64_ragged": (BF16, 3, 100, 8, 2, 64, [1, 0, 100], 1.0),
    "seq_len_1": (BF16, 3, 1, 4, 4, 128, [1, 1, 0], 1.0),
    "peaked": (BF16, 1, 777, 4, 1, 128, [65], 6.0),
    "long_4096": (BF16, 1, 4096, 8, 8, 128, [96], 1.0),
    # scores that rise by about one (base 2) per 64-key tile: the running maximum creeps up by
    # less than the rescaling slack at each tile, so unnormalised probabilities far above 1
    # accumulate between rescalings
    "rising_keys": (BF16, 2, 1000, 8, 2, 128, [40, 130], 1.0, None, True),
    "negative_scale": (BF16, 2, 200, 8, 4, 128, [30, 77], 1.0, -0.2),
    "zero_scale": (BF16, 1, 150, 4, 4, 64, [20], 1.0, 0.0),
}


@pytest.mark.parametrize("case", list(ATTN_CASES))
def test_partial_attn(lib, case):
    dtype, B, S, H, Hkv, hd, counts, qs, *extra = ATTN_CASES[case]
    sc = extra[0] if extra and extra[0] is not None else 1.0 / math.sqrt(hd)
    ramp = len(extra) > 1 and extra[1]
    print(f"attn case={case}", flush=True)
    sel, rp = random_selection(B, S, counts, 500)
    M = int(rp[-1])
    q = synth.normal((max(1, M), H * hd), qs, 501, F32)
    kc = synth.normal((B, Hkv, S, hd), 1.0, 502, F32)
    if ramp:  # every entry of q shifted by +1 and of key t by t / S: q.k grows by ~hd t / S
        q = q + 1.0
        kc = kc + torch.linspace(0.0, 1.0, S)[None, None, :, None]
    q, kc = q.to(dtype), kc.to(dtype)
    vc = synth.normal((B, Hkv, S, hd), 1.0, 503, dtype)
    shape = shape_of(lib, dtype, B, S, 64, H, Hkv, hd, 64)
    o = torch.full((max(1, M), H * hd), -3.0, dtype=dtype, device="cuda")
    ws = lib.workspace(lib.OP_ATTN, shape, M)
    scale = sc
    lib.dllm_partial_attn(shape, scale, to_dev(q), to_dev(kc), to_dev(vc), to_dev(sel), to_dev(rp),
                          M, o, ws)
    torch.cuda.synchronize()
    ref = O.partial_attn(host(q), host(kc), host(vc), sel, rp, H, Hkv, hd, scale)
    assert_close(host(o)[:M], ref, TOL[dtype], "o_sel")


# ----------------------------------------------------------------------------- (5) FFN
@pytest.mark.parametrize("case", list(LAYER_CASES))
@pytest.mark.parametrize("alias", [False, True])
def test_ffn_scatter(lib, case, alias):
    dtype, (B, S, d, H, Hkv, hd, F), w, h_in, kc, vc, sel, rp = layer_inputs(case, 600)
    M = int(rp[-1])
    print(f"ffn case={case} M={M} alias={alias}", flush=True)
    shape = shape_of(lib, dtype, B, S, d, H, Hkv, hd, F)
    o_sel = synth.normal((max(1, M), H * hd), 1.0, 601, dtype)
    h_prev_out = synth.normal((B, S, d), 1.0, 602, dtype)
    h_in_d = to_dev(h_in)
    h_out = h_in_d if alias else to_dev(h_prev_out)
    ws = lib.workspace(lib.OP_FFN, shape, M)
    lib.dllm_gather_ffn_scatter(shape, h_in_d, to_dev(o_sel), to_dev(w["w_o"]),
                                to_dev(w["g_ffn"]), to_dev(w["w_gate"]), to_dev(w["w_up"]),
                                to_dev(w["w_down"]), to_dev(sel), to_dev(rp), M, h_out, ws)
    torch.cuda.synchronize()
    base = h_in if alias else h_prev_out
    ref = O.gather_ffn_scatter(host(h_in), host(o_sel), host(w["w_o"]), host(w["g_ffn"]),
                               host(w["w_gate"]), host(w["w_up"]), host(w["w_down"]), sel, rp,
                               host(base), 1e-5)
    touched = np.zeros((B, S), dtype=bool)
    touched[sel // S, sel % S] = True
    got = host(h_out)
    assert_close(got[touched], ref[touched], TOL[dtype], "h_out")
    assert np.array_equal(got[~touched], host(base)[~touched]), "unselected hidden rows changed"


def test_empty_selection_writes_nothing(lib):
    dtype, (B, S, d, H, Hkv, hd, F), w, h_in, kc, vc, _, _ = layer_inputs("bf16_gqa_ragged", 700)
    shape = shape_of(lib, dtype, B, S, d, H, Hkv, hd, F)
    sel = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    rp = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    m_cap = 64  # capacity above the (zero) count: the kernels must read row_ptr and write nothing
    kc_d, vc_d, h_out = to_dev(kc), to_dev(vc), to_dev(h_in).clone()
    q = torch.full((m_cap, H * hd), -3.0, dtype=dtype, device="cuda")
    o = torch.full((m_cap, H * hd), -3.0, dtype=dtype, device="cuda")
    lib.dllm_gather_qkv_scatter_kv(shape, to_dev(h_in), to_dev(w["g_attn"]), to_dev(w["w_qkv"]),
                                   sel, rp, m_cap, q, kc_d, vc_d,
                                   lib.workspace(lib.OP_QKV, shape, m_cap))
    lib.dllm_partial_attn(shape, 0.1, q, kc_d, vc_d, sel, rp, m_cap, o,
                          lib.workspace(lib.OP_ATTN, shape, m_cap))
    lib.dllm_gather_ffn_scatter(shape, to_dev(h_in), o, to_dev(w["w_o"]), to_dev(w["g_ffn"]),
                                to_dev(w["w_gate"]), to_dev(w["w_up"]), to_dev(w["w_down"]), sel,
                                rp, m_cap, h_out, lib.workspace(lib.OP_FFN, shape, m_cap))
    torch.cuda.synchronize()
    assert same_bits(kc_d, kc) and same_bits(vc_d, vc) and same_bits(h_out, h_in)
    assert torch.all(q.float() == -3.0) and torch.all(o.float() == -3.0)
