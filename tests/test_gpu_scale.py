"""Per-call parity at the full workload sizes, on sampled rows.

Inputs are drawn by the seeded generators directly on the GPU (the logits of the batched LLaDA step
alone are 2 GB); each call runs on every selected row exactly as the step runs it, and the oracle
recomputes a deterministic sample of rows from the same generator outputs. Rows are independent
given their inputs, so a sampled row is compared with its full-size result.

Workloads: LLaDA-8B step (B=8, S=1024, 205 selected per sequence), long context (B=1, S=4096,
32 forced + 64 selected), Dream-7B GQA (B=16, S=2048, 28/4 heads, 5%, 10%, 25% and 50% selected).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import TOL, assert_close, host, same_bits, to_dev
from synth import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
BF16 = torch.bfloat16
NSAMPLE = 48


def shape_of(lib, d, V=0):
    return lib.Shape(B=d.B, S=d.S, d=d.d, H=d.H, Hkv=d.Hkv, hd=d.hd, F=d.F, dtype="bf16", V=V)


def even_selection(B, S, per_row, seed):
    rng = np.random.default_rng(seed)
    sel, rp = [], [0]
    for b in range(B):
        pos = np.sort(rng.choice(S, size=per_row, replace=False))
        sel.extend(b * S + int(p) for p in pos)
        rp.append(len(sel))
    return np.asarray(sel, np.int32), np.asarray(rp, np.int32)


def sample_rows(M, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(M, size=min(NSAMPLE, M), replace=False))


def subset(sel, rows, S, B):
    """Selection of only `rows` (indices into sel), as (sel_sub, row_ptr_sub)."""
    sub = sel[rows]
    rp = np.zeros(B + 1, np.int32)
    for b in range(B):
        rp[b + 1] = rp[b] + int(np.sum(sub // S == b))
    return sub.astype(np.int32), rp


CASES = {
    # name: dims, selected per sequence
    "llada_step": (W.LLADA_STEP, W.STEP_TOPK),
    "llada_long": (W.LLADA_LONG, 96),
    "dream_5pct": (W.DREAM_GQA, 102),
    "dream_10pct": (W.DREAM_GQA, 205),
    "dream_25pct": (W.DREAM_GQA, 512),
    "dream_50pct": (W.DREAM_GQA, 1024),
}


def weights_gpu(d, seed):
    w = synth.layer_weights(d.d, d.H, d.Hkv, d.hd, d.F, seed=seed, dtype=BF16, device="cuda")
    w["g_attn"] = (1.0 + synth.normal((d.d,), 0.1, seed + 7, device="cuda")).to(BF16)
    w["g_ffn"] = (1.0 + synth.normal((d.d,), 0.1, seed + 8, device="cuda")).to(BF16)
    return w


@pytest.mark.parametrize("case", list(CASES))
def test_qkv_full_size(lib, case):
    d, per = CASES[case]
    print(f"qkv full-size {case}", flush=True)
    sel, rp = even_selection(d.B, d.S, per, 11)
    M = int(rp[-1])
    w = weights_gpu(d, 900)
    h_in = synth.normal((d.B, d.S, d.d), 1.0, 901, BF16, "cuda")
    kc = synth.normal((d.B, d.Hkv, d.S, d.hd), 1.0, 902, BF16, "cuda")
    vc = synth.normal((d.B, d.Hkv, d.S, d.hd), 1.0, 903, BF16, "cuda")
    kc0, vc0 = kc.clone(), vc.clone()
    shape = shape_of(lib, d)
    q = torch.empty(M, d.H * d.hd, dtype=BF16, device="cuda")
    lib.dllm_gather_qkv_scatter_kv(shape, h_in, w["g_attn"], w["w_qkv"], to_dev(sel), to_dev(rp), M,
                                   q, kc, vc, lib.workspace(lib.OP_QKV, shape, M))
    torch.cuda.synchronize()
    rows = sample_rows(M, 12)
    s_sub, rp_sub = subset(sel, rows, d.S, d.B)
    bs, ss = s_sub // d.S, s_sub % d.S
    # oracle on the sampled rows (host copies of the generator outputs)
    zeros = np.zeros((d.B, d.Hkv, d.S, d.hd))
    rq, rk, rv = O.gather_qkv_scatter_kv(host(h_in), host(w["g_attn"]), host(w["w_qkv"]), s_sub,
                                         rp_sub, zeros, zeros, d.H, d.Hkv, d.hd, 1e-5)
    tol = TOL[BF16]
    rows_t = torch.from_numpy(rows).cuda()
    bs_t, ss_t = torch.from_numpy(bs).cuda(), torch.from_numpy(ss).cuda()
    assert_close(host(q[rows_t]), rq, tol, "q_sel (sampled)")
    assert_close(host(kc[bs_t, :, ss_t, :]), rk[bs, :, ss, :], tol, "k_cache rows (sampled)")
    assert_close(host(vc[bs_t, :, ss_t, :]), rv[bs, :, ss, :], tol, "v_cache rows (sampled)")
    # every unselected position keeps its cache entry
    mask = torch.ones(d.B, d.S, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(sel // d.S).cuda().long(), torch.from_numpy(sel % d.S).cuda().long()] = False
    assert same_bits(kc.permute(0, 2, 1, 3)[mask], kc0.permute(0, 2, 1, 3)[mask])
    assert same_bits(vc.permute(0, 2, 1, 3)[mask], vc0.permute(0, 2, 1, 3)[mask])


@pytest.mark.parametrize("case", list(CASES))
def test_attention_full_size(lib, case):
    d, per = CASES[case]
    print(f"attention full-size {case}", flush=True)
    sel, rp = even_selection(d.B, d.S, per, 21)
    M = int(rp[-1])
    q = synth.normal((M, d.H * d.hd), 1.0, 911, BF16, "cuda")
    kc = synth.normal((d.B, d.Hkv, d.S, d.hd), 1.0, 912, BF16, "cuda")
    vc = synth.normal((d.B, d.Hkv, d.S, d.hd), 1.0, 913, BF16, "cuda")
    shape = shape_of(lib, d)
    o = torch.empty(M, d.H * d.hd, dtype=BF16, device="cuda")
    scale = 1.0 / math.sqrt(d.hd)
    lib.dllm_partial_attn(shape, scale, q, kc, vc, to_dev(sel), to_dev(rp), M, o,
                          lib.workspace(lib.OP_ATTN, shape, M))
    torch.cuda.synchronize()
    rows = sample_rows(M, 22)
    s_sub, rp_sub = subset(sel, rows, d.S, d.B)
    ref = O.partial_attn(host(q[torch.from_numpy(rows).cuda()]), host(kc), host(vc), s_sub, rp_sub,
                         d.H, d.Hkv, d.hd, scale)
    assert_close(host(o[torch.from_numpy(rows).cuda()]), ref, TOL[BF16], "o_sel (sampled)")


@pytest.mark.parametrize("case", list(CASES))
def test_ffn_full_size(lib, case):
    d, per = CASES[case]
    print(f"ffn full-size {case}", flush=True)
    sel, rp = even_selection(d.B, d.S, per, 31)
    M = int(rp[-1])
    w = weights_gpu(d, 920)
    h_in = synth.normal((d.B, d.S, d.d), 1.0, 921, BF16, "cuda")
    o_sel = synth.normal((M, d.H * d.hd), 1.0, 922, BF16, "cuda")
    h_out = synth.normal((d.B, d.S, d.d), 1.0, 923, BF16, "cuda")
    h_out0 = h_out.clone()
    shape = shape_of(lib, d)
    lib.dllm_gather_ffn_scatter(shape, h_in, o_sel, w["w_o"], w["g_ffn"], w["w_gate"], w["w_up"],
                                w["w_down"], to_dev(sel), to_dev(rp), M, h_out,
                                lib.workspace(lib.OP_FFN, shape, M))
    torch.cuda.synchronize()
    rows = sample_rows(M, 32)
    s_sub, rp_sub = subset(sel, rows, d.S, d.B)
    bs, ss = s_sub // d.S, s_sub % d.S
    ref = O.gather_ffn_scatter(host(h_in), host(o_sel[torch.from_numpy(rows).cuda()]),
                               host(w["w_o"]), host(w["g_ffn"]), host(w["w_gate"]), host(w["w_up"]),
                               host(w["w_down"]), s_sub, rp_sub, np.zeros((d.B, d.S, d.d)), 1e-5)
    got = host(h_out[torch.from_numpy(bs).cuda(), torch.from_numpy(ss).cuda()])
    assert_close(got, ref[bs, ss], TOL[BF16], "h_out rows (sampled)")
    mask = torch.ones(d.B, d.S, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(sel // d.S).cuda().long(), torch.from_numpy(sel % d.S).cuda().long()] = False
    assert same_bits(h_out[mask], h_out0[mask])


def test_saliency_batched_step_size(lib):
    """B=8 x 1024 tokens with the full 126464 vocabulary (2 GB of logits), sampled tokens."""
    d = W.LLADA_STEP
    h_prev, h_cur, _ = synth.perturbed_pair(d.B, d.S, d.d, W.LLADA_LARGE, seed=41, dtype=BF16,
                                            device="cuda")
    logits = synth.logits(d.B, d.S, d.V, seed=42, dtype=BF16, device="cuda")
    shape = shape_of(lib, d, d.V)
    score = torch.empty(d.B, d.S, device="cuda")
    conf = torch.empty(d.B, d.S, device="cuda")
    lib.dllm_saliency(shape, O.DELTA_L1N, 0.5, h_cur, h_prev, logits, score, conf)
    torch.cuda.synchronize()
    rng = np.random.default_rng(43)
    toks = rng.choice(d.B * d.S, size=64, replace=False)
    tb, ts = toks // d.S, toks % d.S
    idx = (torch.from_numpy(tb).cuda(), torch.from_numpy(ts).cuda())
    r_score, r_conf, _ = O.saliency(host(h_cur[idx]), host(h_prev[idx]), host(logits[idx]), 0.5)
    assert_close(host(score[idx]), r_score, 1e-4, "score (sampled)")
    assert_close(host(conf[idx]), r_conf, 1e-4, "confidence (sampled)")


def test_select_batched_step_size(lib):
    """B=8 x 1024, top-205 per sequence, plus the long-context forced block + top-64."""
    from test_gpu_calls import check_select
    score = synth.adversarial_scores(8, 1024, seed=51, kind="random")
    check_select(lib, score, None, O.SEL_TOPK, k=W.STEP_TOPK)
    score = synth.adversarial_scores(1, 4096, seed=52, kind="random")
    force = np.zeros((1, 4096), dtype=bool)
    force[0, 3584 + 32 * 5: 3584 + 32 * 6] = True   # the active block of 32
    check_select(lib, score, force, O.SEL_TOPK, k=64)
    score = synth.adversarial_scores(16, 2048, seed=53, kind="ties")
    check_select(lib, score, None, O.SEL_TOPK, k=1024)


PLANNED = [("llada", p) for p in (1, 128, 200, 300, 700, 1640, 5000)] + \
          [("dream", p) for p in (320, 656, 3280)]


@pytest.mark.parametrize("shape_name,m_plan", PLANNED, ids=[f"{n}-{p}" for n, p in PLANNED])
def test_planned_rows_do_not_change_results(lib, shape_name, m_plan):
    """A layer with 200 selected rows per sequence, capacity every token, and the calls planned
    for other row counts: every selected row is still computed and matches the oracle, and nothing
    else is written. LLaDA-8B: the planned counts reach every GEMM plan class at this shape: 1
    (64-row weight-streaming tiles, 4 row tiles), 128, 200 (256-row tiles); then the 32x32x16
    tiles chosen by their estimated time: 300 (128 x 256, unsplit and 4 K splits), 700 (256 x 256
    unsplit and with 4 splits, 128 x 256 with 2), 1640 (256 x 256 with 2 splits) and 5000
    (256 x 256 unsplit); up to 1024 planned rows the layer is one sequence of 1024 tokens, above it
    8 sequences (plans are capped at the capacity). Dream-7B (GQA 28/4, d 3584, FFN 18944, 16 x
    2048 tokens): 320 (128 x 256 with 4 splits over K = 3584), 656 (128 x 256 with 2 splits;
    256 x 256 with 4 splits over K = 18944) and 3280 (256 x 256). Each call takes its inputs from
    the generators."""
    if shape_name == "llada":
        d = W.LLADA_LAYER if m_plan <= 1024 else W.LLADA_STEP
    else:
        d = W.DREAM_GQA
    print(f"planned rows {m_plan}, {shape_name} B={d.B}", flush=True)
    sel, rp = even_selection(d.B, d.S, 200, 61)
    M, cap = int(rp[-1]), d.B * d.S
    w = weights_gpu(d, 930)
    h_in = synth.normal((d.B, d.S, d.d), 1.0, 931, BF16, "cuda")
    kc = synth.normal((d.B, d.Hkv, d.S, d.hd), 1.0, 932, BF16, "cuda")
    vc = synth.normal((d.B, d.Hkv, d.S, d.hd), 1.0, 933, BF16, "cuda")
    kc0 = kc.clone()
    q_in = synth.normal((cap, d.H * d.hd), 1.0, 935, BF16, "cuda")
    o_in = synth.normal((cap, d.H * d.hd), 1.0, 936, BF16, "cuda")
    h_out = synth.normal((d.B, d.S, d.d), 1.0, 934, BF16, "cuda")
    h_out0 = h_out.clone()
    shape = shape_of(lib, d).with_plan(m_plan)
    sel_d, rp_d = to_dev(sel), to_dev(rp)
    q = torch.zeros(cap, d.H * d.hd, dtype=BF16, device="cuda")
    o = torch.zeros(cap, d.H * d.hd, dtype=BF16, device="cuda")
    scale = 1.0 / math.sqrt(d.hd)
    lib.dllm_partial_attn(shape, scale, q_in, kc, vc, sel_d, rp_d, cap, o,
                          lib.workspace(lib.OP_ATTN, shape, cap))
    lib.dllm_gather_ffn_scatter(shape, h_in, o_in, w["w_o"], w["g_ffn"], w["w_gate"], w["w_up"],
                                w["w_down"], sel_d, rp_d, cap, h_out,
                                lib.workspace(lib.OP_FFN, shape, cap))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(M, 62)[:24], [M - 1]]))  # M-1: ragged tile
    s_sub, rp_sub = subset(sel, rows, d.S, d.B)
    bs, ss = s_sub // d.S, s_sub % d.S
    rows_t = torch.from_numpy(rows).cuda()
    bs_t, ss_t = torch.from_numpy(bs).cuda(), torch.from_numpy(ss).cuda()
    tol = TOL[BF16]
    ra = O.partial_attn(host(q_in[rows_t]), host(kc), host(vc), s_sub, rp_sub, d.H, d.Hkv, d.hd,
                        scale)
    assert_close(host(o[rows_t]), ra, tol, "o_sel (sampled)")
    rf = O.gather_ffn_scatter(host(h_in), host(o_in[rows_t]), host(w["w_o"]), host(w["g_ffn"]),
                              host(w["w_gate"]), host(w["w_up"]), host(w["w_down"]), s_sub, rp_sub,
                              np.zeros((d.B, d.S, d.d)), 1e-5)
    assert_close(host(h_out[bs_t, ss_t]), rf[bs, ss], tol, "h_out rows (sampled)")
    # the projection last: it rewrites the cache rows the attention above read
    lib.dllm_gather_qkv_scatter_kv(shape, h_in, w["g_attn"], w["w_qkv"], sel_d, rp_d, cap, q, kc,
                                   vc, lib.workspace(lib.OP_QKV, shape, cap))
    torch.cuda.synchronize()
    zeros = np.zeros((d.B, d.Hkv, d.S, d.hd))
    rq, rk, _ = O.gather_qkv_scatter_kv(host(h_in), host(w["g_attn"]), host(w["w_qkv"]), s_sub,
                                        rp_sub, zeros, zeros, d.H, d.Hkv, d.hd, 1e-5)
    assert_close(host(q[rows_t]), rq, tol, "q_sel (sampled)")
    assert_close(host(kc[bs_t, :, ss_t, :]), rk[bs, :, ss, :], tol, "k_cache rows (sampled)")
    # rows past M of the compact outputs and unselected cache / hidden rows are untouched
    assert not q[M:].any() and not o[M:].any()
    mask = torch.ones(d.B, d.S, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(sel // d.S).cuda().long(), torch.from_numpy(sel % d.S).cuda().long()] = False
    assert same_bits(kc.permute(0, 2, 1, 3)[mask], kc0.permute(0, 2, 1, 3)[mask])
    assert same_bits(h_out[mask], h_out0[mask])
