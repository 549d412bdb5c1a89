"""Parity of the attention context of every token (DyLLM French summary page §2.B, both paths)
against the oracle: dllm_gather_kv_rows copies the rows a step overwrites, dllm_salient_attn
recomputes the selected tokens exactly and updates every other token's stored softmax state with
the changed keys only.

Each case starts from the exact state (the oracle's context of the query cache against the
cache), then runs several steps: new selection, copies of the old rows, new K/V rows written at
the selected positions, new queries for the selected tokens. After every step the library's
context, state and query cache must match the oracle's context of the updated query cache against
the updated cache, so errors of the carried state would show up as growth over the steps.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import TOL, assert_close, host, random_selection, same_bits, to_dev

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
LN2 = math.log(2.0)


def exact_state(q_all, kc, vc, H, Hkv, hd, scale):
    """State holding the exact context: m = base-2 log-sum-exp, l = 1, o = context."""
    o, lse = O.context_all(host(q_all), host(kc), host(vc), H, Hkv, hd, scale)
    B, S = q_all.shape[:2]
    st_m = to_dev(lse / LN2, torch.float32)
    st_l = torch.ones(B, S, H, device="cuda")
    st_o = to_dev(o, torch.float32).reshape(B, S, H * hd).contiguous()
    return st_m, st_l, st_o


CASES = {
    # name: B, S, H, Hkv, hd, selected per sequence for each step, scale (None = 1/sqrt(hd))
    "mha_ragged_and_unchanged_row": (2, 200, 4, 4, 128, [[37, 0], [5, 64], [0, 1]], None),
    "gqa_4to1_hd64": (2, 160, 8, 2, 64, [[16, 45], [33, 2]], None),
    "many_changed_split_keys": (1, 512, 2, 2, 128, [[300], [40]], None),
    "negative_scale": (1, 128, 2, 1, 64, [[20], [7]], -0.2),
}


@pytest.mark.parametrize("case", list(CASES))
def test_salient_attention_steps(lib, case):
    B, S, H, Hkv, hd, steps, scale = CASES[case]
    scale = 1.0 / math.sqrt(hd) if scale is None else scale
    print(f"salient attention {case}", flush=True)
    Nq = H * hd
    shape = lib.Shape(B=B, S=S, d=Nq, H=H, Hkv=Hkv, hd=hd, F=64, dtype="bf16")
    q_all = synth.normal((B, S, Nq), 1.0, 700, BF16, "cuda")
    kc = synth.normal((B, Hkv, S, hd), 1.0, 701, BF16, "cuda")
    vc = synth.normal((B, Hkv, S, hd), 1.0, 702, BF16, "cuda")
    st_m, st_l, st_o = exact_state(q_all, kc, vc, H, Hkv, hd, scale)
    o_all = torch.empty(B, S, Nq, dtype=BF16, device="cuda")
    for t, counts in enumerate(steps):
        sel, rp = random_selection(B, S, counts, 710 + t)
        M = int(rp[-1])
        m_cap = max(M, 1)
        sel_d = to_dev(sel if M else np.zeros(1, np.int32))
        rp_d = to_dev(rp)
        k_old = torch.empty(m_cap, Hkv, hd, dtype=BF16, device="cuda")
        v_old = torch.empty_like(k_old)
        lib.dllm_gather_kv_rows(shape, kc, vc, sel_d, rp_d, m_cap, k_old, v_old)
        torch.cuda.synchronize()
        bs = torch.from_numpy(sel // S).long().cuda()
        ss = torch.from_numpy(sel % S).long().cuda()
        if M:
            assert same_bits(k_old[:M], kc[bs, :, ss, :]) and same_bits(v_old[:M], vc[bs, :, ss, :])
            kc[bs, :, ss, :] = synth.normal((M, Hkv, hd), 1.0, 720 + t, BF16, "cuda")
            vc[bs, :, ss, :] = synth.normal((M, Hkv, hd), 1.0, 730 + t, BF16, "cuda")
        q_sel = synth.normal((m_cap, Nq), 1.0, 740 + t, BF16, "cuda")
        q_before = q_all.clone()
        o_sel = torch.empty(m_cap, Nq, dtype=BF16, device="cuda")
        ws = lib.workspace(lib.OP_ATTN, shape, m_cap)
        lib.dllm_salient_attn(shape, scale, q_sel, q_all, kc, vc, k_old, v_old, sel_d, rp_d,
                              m_cap, st_m, st_l, st_o, o_sel, o_all, ws)
        torch.cuda.synchronize()
        q_ref, o_ref, lse_ref = O.salient_attention(host(q_sel)[:M], host(q_before), host(kc),
                                                    host(vc), sel, rp, H, Hkv, hd, scale)
        # query cache: selected rows replaced bit for bit, the others untouched
        keep = torch.ones(B, S, dtype=torch.bool, device="cuda")
        if M:
            keep[bs, ss] = False
            assert same_bits(q_all[bs, ss], q_sel[:M])
        assert same_bits(q_all[keep], q_before[keep])
        assert_close(host(o_all), o_ref, TOL[BF16], f"step {t} o_all")
        assert_close(host(st_o), o_ref, TOL[BF16], f"step {t} state o")
        lse = (host(st_m) + np.log2(host(st_l))) * LN2
        assert_close(lse, lse_ref, 1e-3, f"step {t} log-sum-exp")
        if M:
            want = O.partial_attn(host(q_sel)[:M], host(kc), host(vc), sel, rp, H, Hkv, hd, scale)
            assert_close(host(o_sel)[:M], want, TOL[BF16], f"step {t} o_sel")


def test_select_all_initialises_the_state(lib):
    """Every position selected: the state comes out exact whatever it held before."""
    B, S, H, Hkv, hd = 2, 96, 4, 2, 128
    Nq = H * hd
    scale = 1.0 / math.sqrt(hd)
    shape = lib.Shape(B=B, S=S, d=Nq, H=H, Hkv=Hkv, hd=hd, F=64, dtype="bf16")
    q_all = torch.zeros(B, S, Nq, dtype=BF16, device="cuda")
    kc = synth.normal((B, Hkv, S, hd), 1.0, 750, BF16, "cuda")
    vc = synth.normal((B, Hkv, S, hd), 1.0, 751, BF16, "cuda")
    st_m = torch.zeros(B, S, H, device="cuda")
    st_l = torch.zeros(B, S, H, device="cuda")          # not a valid state
    st_o = torch.full((B, S, Nq), 7.0, device="cuda")
    sel = np.arange(B * S, dtype=np.int32)
    rp = np.array([0, S, 2 * S], np.int32)
    M = B * S
    q_sel = synth.normal((M, Nq), 1.0, 752, BF16, "cuda")
    k_old = kc.permute(0, 2, 1, 3).reshape(M, Hkv, hd).contiguous()
    v_old = vc.permute(0, 2, 1, 3).reshape(M, Hkv, hd).contiguous()
    o_sel = torch.empty(M, Nq, dtype=BF16, device="cuda")
    o_all = torch.empty(B, S, Nq, dtype=BF16, device="cuda")
    lib.dllm_salient_attn(shape, scale, q_sel, q_all, kc, vc, k_old, v_old, to_dev(sel),
                          to_dev(rp), M, st_m, st_l, st_o, o_sel, o_all,
                          lib.workspace(lib.OP_ATTN, shape, M))
    torch.cuda.synchronize()
    o_ref, lse_ref = O.context_all(host(q_sel).reshape(B, S, Nq), host(kc), host(vc), H, Hkv, hd,
                                   scale)
    assert same_bits(q_all.reshape(M, Nq), q_sel)
    assert_close(host(o_all), o_ref, TOL[BF16], "o_all")
    assert_close(host(st_o), o_ref, TOL[BF16], "state o")
    assert_close((host(st_m) + np.log2(host(st_l))) * LN2, lse_ref, 1e-3, "log-sum-exp")


def test_no_selection_keeps_every_context(lib):
    """m_cap = 0: no key changed, every token keeps its context (up to the state's rounding)."""
    B, S, H, Hkv, hd = 1, 64, 2, 2, 64
    Nq = H * hd
    scale = 1.0 / math.sqrt(hd)
    shape = lib.Shape(B=B, S=S, d=Nq, H=H, Hkv=Hkv, hd=hd, F=64, dtype="bf16")
    q_all = synth.normal((B, S, Nq), 1.0, 760, BF16, "cuda")
    kc = synth.normal((B, Hkv, S, hd), 1.0, 761, BF16, "cuda")
    vc = synth.normal((B, Hkv, S, hd), 1.0, 762, BF16, "cuda")
    st_m, st_l, st_o = exact_state(q_all, kc, vc, H, Hkv, hd, scale)
    o0 = host(st_o)
    one = torch.zeros(1, dtype=torch.int32, device="cuda")
    rp = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    dummy = torch.zeros(1, Nq, dtype=BF16, device="cuda")
    dkv = torch.zeros(1, Hkv, hd, dtype=BF16, device="cuda")
    o_all = torch.empty(B, S, Nq, dtype=BF16, device="cuda")
    lib.dllm_salient_attn(shape, scale, dummy, q_all, kc, vc, dkv, dkv, one, rp, 0, st_m, st_l,
                          st_o, dummy, o_all, None)
    torch.cuda.synchronize()
    assert_close(host(st_o), o0, 1e-6, "state o")
    assert_close(host(o_all), o0, TOL[BF16], "o_all")


def test_response_only_steps_leave_the_prompt_alone(lib):
    """DyLLM §2.C: with q_first = P the unselected prompt positions are not processed (query,
    state and context bit-identical to before), response positions are updated, and a step that
    selects every prompt position (the prompt re-injected) brings the prompt rows back to the
    exact context of the updated cache. The oracle carries its own previous context for the
    rows a step leaves out."""
    B, S, H, Hkv, hd, P = 2, 160, 4, 2, 128, 96
    Nq = H * hd
    scale = 1.0 / math.sqrt(hd)
    shape = lib.Shape(B=B, S=S, d=Nq, H=H, Hkv=Hkv, hd=hd, F=64, dtype="bf16")
    q_all = synth.normal((B, S, Nq), 1.0, 770, BF16, "cuda")
    kc = synth.normal((B, Hkv, S, hd), 1.0, 771, BF16, "cuda")
    vc = synth.normal((B, Hkv, S, hd), 1.0, 772, BF16, "cuda")
    st_m, st_l, st_o = exact_state(q_all, kc, vc, H, Hkv, hd, scale)
    o_all = st_o.to(BF16).reshape(B, S, Nq).contiguous()
    o_prev, lse_prev = O.context_all(host(q_all), host(kc), host(vc), H, Hkv, hd, scale)
    rng = np.random.default_rng(773)
    # per step: (response positions per sequence, prompt positions per sequence)
    plan = [([20, 9], [0, 0]), ([5, 30], [1, 0]), ([12, 3], [P, P]), ([0, 7], [0, 0])]
    for t, (n_resp, n_prompt) in enumerate(plan):
        ids = []
        for b in range(B):
            pos = np.concatenate([rng.choice(P, n_prompt[b], replace=False),
                                  P + rng.choice(S - P, n_resp[b], replace=False)])
            ids.append(b * S + np.sort(pos))
        sel = np.concatenate(ids).astype(np.int32)
        rp = np.array([0] + list(np.cumsum([len(i) for i in ids])), np.int32)
        M = int(rp[-1])
        print(f"response-only step {t}: {M} selected ({sum(n_prompt)} prompt)", flush=True)
        m_cap = max(M, 1)
        sel_d = to_dev(sel if M else np.zeros(1, np.int32))
        rp_d = to_dev(rp)
        k_old = torch.empty(m_cap, Hkv, hd, dtype=BF16, device="cuda")
        v_old = torch.empty_like(k_old)
        lib.dllm_gather_kv_rows(shape, kc, vc, sel_d, rp_d, m_cap, k_old, v_old)
        bs = torch.from_numpy(sel // S).long().cuda()
        ss = torch.from_numpy(sel % S).long().cuda()
        if M:
            kc[bs, :, ss, :] = synth.normal((M, Hkv, hd), 1.0, 780 + t, BF16, "cuda")
            vc[bs, :, ss, :] = synth.normal((M, Hkv, hd), 1.0, 790 + t, BF16, "cuda")
        q_sel = synth.normal((m_cap, Nq), 1.0, 800 + t, BF16, "cuda")
        q_before = q_all.clone()
        before = [x.clone() for x in (st_m, st_l, st_o, o_all)]
        o_sel = torch.empty(m_cap, Nq, dtype=BF16, device="cuda")
        lib.dllm_salient_attn(shape, scale, q_sel, q_all, kc, vc, k_old, v_old, sel_d, rp_d,
                              m_cap, st_m, st_l, st_o, o_sel, o_all,
                              lib.workspace(lib.OP_ATTN, shape, m_cap), q_first=P)
        torch.cuda.synchronize()
        q_ref, o_ref, lse_ref = O.salient_attention(host(q_sel)[:M], host(q_before), host(kc),
                                                    host(vc), sel, rp, H, Hkv, hd, scale,
                                                    q_first=P, o_prev=o_prev, lse_prev=lse_prev)
        skip = torch.zeros(B, S, dtype=torch.bool, device="cuda")
        skip[:, :P] = True
        if M:
            skip[bs, ss] = False
        for x, x0 in zip((st_m, st_l, st_o, o_all), before):
            assert same_bits(x.reshape(B, S, -1)[skip], x0.reshape(B, S, -1)[skip])
        assert same_bits(q_all[skip], q_before[skip])
        assert_close(host(o_all), o_ref, TOL[BF16], f"step {t} o_all")
        assert_close(host(st_o), o_ref, TOL[BF16], f"step {t} state o")
        lse = (host(st_m) + np.log2(host(st_l))) * LN2
        assert_close(lse, lse_ref, 1e-3, f"step {t} log-sum-exp")
        o_prev, lse_prev = o_ref, lse_ref
    # after the re-injection step every prompt row is exact again (and stays so in the last step,
    # which changed keys but left the prompt out: the oracle keeps its step-3 rows as well)


@pytest.mark.parametrize("hd", [64, 128])
def test_changed_key_that_held_most_of_the_weight(lib, hd):
    """A stable token whose attention sat almost wholly (>= 0.9, here about 0.99) on one key that
    a step changes: the incremental update would subtract nearly all of its stored mass, so the
    leftover carries the rounding of the removed exponentials magnified by 1 / (1 - w). The
    library recomputes such a token's state exactly; its context must match the oracle row by
    row (each row against its own magnitude), in that step and in the next one, which builds on
    the recomputed state."""
    B, S, H, Hkv = 1, 160, 2, 2
    Nq = H * hd
    scale = 1.0 / math.sqrt(hd)
    p0, key = 5, 100                       # the stable token and the key it attends to
    shape = lib.Shape(B=B, S=S, d=Nq, H=H, Hkv=Hkv, hd=hd, F=64, dtype="bf16")
    q_all = synth.normal((B, S, Nq), 1.0, 840, BF16, "cuda")
    kc = synth.normal((B, Hkv, S, hd), 1.0, 841, BF16, "cuda")
    vc = synth.normal((B, Hkv, S, hd), 1.0, 842, BF16, "cuda")
    for h in range(H):                     # scaled score of about 10 for (p0, h) against `key`
        qv = q_all[0, p0, h * hd:(h + 1) * hd].float()
        kc[0, h, key] = (qv * (10.0 / (scale * float(qv.dot(qv))))).to(BF16)
    qh, kh = host(q_all), host(kc)
    for h in range(H):
        z = scale * kh[0, h] @ qh[0, p0, h * hd:(h + 1) * hd]
        w = np.exp(z - z.max())
        assert w[key] / w.sum() >= 0.9, "the case must put most of the weight on one key"
    st_m, st_l, st_o = exact_state(q_all, kc, vc, H, Hkv, hd, scale)
    o_all = torch.empty(B, S, Nq, dtype=BF16, device="cuda")
    for t, extra in enumerate([[key, 40, 41], [7, 90, 150]]):
        print(f"dominant-key step {t}: selected {extra}", flush=True)
        sel = np.array(sorted(extra), np.int32)
        rp = np.array([0, len(sel)], np.int32)
        M = len(sel)
        sel_d, rp_d = to_dev(sel), to_dev(rp)
        k_old = torch.empty(M, Hkv, hd, dtype=BF16, device="cuda")
        v_old = torch.empty_like(k_old)
        lib.dllm_gather_kv_rows(shape, kc, vc, sel_d, rp_d, M, k_old, v_old)
        bs = torch.zeros(M, dtype=torch.long, device="cuda")
        ss = torch.from_numpy(sel).long().cuda()
        kc[bs, :, ss, :] = synth.normal((M, Hkv, hd), 1.0, 850 + t, BF16, "cuda")
        vc[bs, :, ss, :] = synth.normal((M, Hkv, hd), 1.0, 860 + t, BF16, "cuda")
        q_sel = synth.normal((M, Nq), 1.0, 870 + t, BF16, "cuda")
        q_before = q_all.clone()
        o_sel = torch.empty(M, Nq, dtype=BF16, device="cuda")
        lib.dllm_salient_attn(shape, scale, q_sel, q_all, kc, vc, k_old, v_old, sel_d, rp_d, M,
                              st_m, st_l, st_o, o_sel, o_all, lib.workspace(lib.OP_ATTN, shape, M))
        torch.cuda.synchronize()
        _, o_ref, lse_ref = O.salient_attention(host(q_sel), host(q_before), host(kc), host(vc),
                                                sel, rp, H, Hkv, hd, scale)
        got, got_st = host(o_all), host(st_o)
        for h in range(H):
            cols = slice(h * hd, (h + 1) * hd)
            assert_close(got[0, p0, cols], o_ref[0, p0, cols], TOL[BF16], f"step {t} token row h{h}")
            assert_close(got_st[0, p0, cols], o_ref[0, p0, cols], TOL[BF16], f"step {t} state row h{h}")
        assert_close(got, o_ref, TOL[BF16], f"step {t} o_all")
        lse = (host(st_m) + np.log2(host(st_l))) * LN2
        assert_close(lse, lse_ref, 1e-3, f"step {t} log-sum-exp")
