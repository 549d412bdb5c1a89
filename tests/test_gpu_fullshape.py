"""Whole-step parity of the multi-layer workloads at their full shape, teacher-forced per layer.

Three steps at the shapes of the workloads they stand for, each a fill step (every layer on
every token) and two early-skip steps with every cache carried (ES-dLLM, German summary page,
§2.A equation and §2.B; SlowFast, German summary page, for the forced active block):
  * the batched LLaDA-8B step: 32 layers (d = 4096, 32 x 128 MHA, FFN 12288), B = 8, S = 1024,
    alpha 0.5 against the full 126464-entry vocabulary, top-205 per sequence;
  * the Dream-7B GQA step: 28 layers (d = 3584, 28 query heads on 4 kv heads, FFN 18944),
    B = 16, S = 2048, alpha 0, top-10% and top-25% per sequence;
  * long-context block decoding: 32 LLaDA-8B layers, B = 1, S = 4096, the active block of 32
    forced plus the top-64 by change;
  * the layer-adaptive step (every token's context kept, per-layer FFN rows): 32 LLaDA-8B layers,
    B = 1, S = 1024 (its own checks are listed in its docstring).

After each step the oracle checks, for one or two sequences:
  * the selection: the oracle's scores from the library's own stored bf16 inputs of the skip
    layer (this step's and the previous step's) and the logits, the top-k bit-identical to the
    library's rows, every candidate score at least 1e-4 from the boundary;
  * every layer (dense and selected): 8 sampled rows per sequence recomputed by the oracle from
    the library's stored bf16 input of that layer and the layer's K/V cache after the step (the
    other selected rows' new K/V entries are the library's), rounding to bf16 where the library
    stores bf16; the rows' K/V cache entries and output hidden rows must agree within the bf16
    tolerance.
Teacher forcing keeps the check at full size affordable (the oracle computes 8-16 rows per
layer, not thousands) while every layer of the real shape, caches and selection take part.

Inputs: one set of random N(0, 0.02^2) weights for all layers (non-unit norm gains), X0 N(0, 1),
per step the moving tokens (154, k or 64 per sequence) moved by N(0, 0.5^2) and the rest by
N(0, (1e-3)^2); for the LLaDA step logits N(0, 1) with one logit raised by 30 on 51 other tokens
per sequence, so the top-205 are those 205 tokens by a wide margin.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import TOL, assert_close, host
from synth import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
BF16 = torch.bfloat16
EPS = 1e-5
SEQS = (0, 5)      # sequences the oracle checks
PER_SEQ = 8        # sampled rows per sequence and layer


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint16).numpy()


def topk_margin(score, k):
    s = -np.sort(-score.astype(np.float64), axis=1)
    thr = 0.5 * (s[:, k - 1] + s[:, k])
    return float(np.min(np.abs(score - thr[:, None])))


def shared_weights(dims, seed):
    w = synth.layer_weights(dims.d, dims.H, dims.Hkv, dims.hd, dims.F, seed=seed)
    w["g_attn"] = (1.0 + synth.normal((dims.d,), 0.1, seed + 1)).to(BF16)
    w["g_ffn"] = (1.0 + synth.normal((dims.d,), 0.1, seed + 2)).to(BF16)
    return w


def make_model(lib, dims, L, skip, k, alpha, m_cap, w):
    from token_skipping_partial_amd.step import EarlySkipModel, LayerWeights, SelectConfig
    lw = LayerWeights.from_dict({n: t.cuda() for n, t in w.items()})
    shape = lib.Shape(B=dims.B, S=dims.S, d=dims.d, H=dims.H, Hkv=dims.Hkv, hd=dims.hd, F=dims.F,
                      dtype="bf16", V=dims.V)
    return EarlySkipModel(shape, [lw] * L, skip, SelectConfig(mode=lib.SEL_TOPK, k=k, alpha=alpha),
                          m_cap=m_cap)


def check_step(model, dims, wbits, tag, seqs, k, h_prev, logits, alpha, force, rng):
    """Selection of `seqs` from the library's stored inputs, then sampled rows of every layer."""
    B, S, H, Hkv, hd = dims.B, dims.S, dims.H, dims.Hkv, dims.hd
    L, skip = len(model.layers), model.skip
    rp = model.step1.row_ptr.cpu().numpy()
    sel_gpu = model.step1.sel_idx.cpu().numpy()[: rp[-1]]
    rows_of = {}
    for b in seqs:
        score, _, _ = O.saliency(bits(model.hidden[skip][b:b + 1]), bits(h_prev[b:b + 1]),
                                 None if logits is None else bits(logits[b:b + 1]), alpha)
        fl = None if force is None else force[b:b + 1]
        cand = score if fl is None else score[fl == 0].reshape(1, -1)
        margin = topk_margin(cand, k)
        print(f"{tag} sequence {b}: oracle score margin {margin:.3e}", flush=True)
        assert margin >= 1e-4, "inputs too close to the selection boundary"
        osel, orp = O.select_compact(score, fl, O.SEL_TOPK, k=k)
        mine = sel_gpu[rp[b]:rp[b + 1]] - b * S
        assert np.array_equal(mine, osel[: orp[-1]]), f"{tag} sequence {b} selection"
        rows_of[b] = mine
    idx = torch.tensor(seqs, device="cuda")
    scale = 1.0 / math.sqrt(hd)
    for l in range(L):
        picks = []
        for b in seqs:
            pool = np.arange(S) if l < skip else rows_of[b]
            picks.append(np.sort(rng.choice(pool, PER_SEQ, replace=False)).astype(np.int32))
        sel = np.concatenate([i * S + p for i, p in enumerate(picks)]).astype(np.int32)
        srp = np.arange(0, PER_SEQ * (len(seqs) + 1), PER_SEQ, dtype=np.int32)
        _, _, k2, v2, y2 = O.selected_layer(
            bits(model.hidden[l][idx]), wbits, sel, srp, bits(model.k[l][idx]),
            bits(model.v[l][idx]), bits(model.hidden[l + 1][idx]), H, Hkv, hd, EPS, scale,
            store="bf16")
        kg, vg, yg = host(model.k[l][idx]), host(model.v[l][idx]), host(model.hidden[l + 1][idx])
        for i, p in enumerate(picks):
            where = f"{tag} layer {l} sequence {seqs[i]}"
            assert_close(kg[i][:, p], k2[i][:, p], TOL[BF16], f"{where} K rows")
            assert_close(vg[i][:, p], v2[i][:, p], TOL[BF16], f"{where} V rows")
            assert_close(yg[i][p], y2[i][p], TOL[BF16], f"{where} hidden rows")
    print(f"{tag}: selection and {L} layers checked", flush=True)


def test_llada_step_full_shape_teacher_forced(lib):
    """The batched LLaDA-8B step (the default bench line): 32 layers, B = 8, alpha 0.5 with the
    full vocabulary, top-205, sequences 0 and 5 checked."""
    dims, L, skip, k = W.LLADA_STEP, 32, W.STEP_SKIP, W.STEP_TOPK
    B, S, d, V = dims.B, dims.S, dims.d, dims.V
    print(f"full-shape batched step: {dims}, {L} layers", flush=True)
    w = shared_weights(dims, 9100)
    wbits = {n: bits(t) for n, t in w.items()}
    model = make_model(lib, dims, L, skip, k, 0.5, B * k, w)
    x = synth.normal((B, S, d), 1.0, 9200, BF16, "cuda")
    model.fill(x)
    rng = np.random.default_rng(9700)
    for t in range(2):
        large = synth.large_positions(B, S, W.LLADA_LARGE, seed=9300 + t)
        spike = synth.large_positions(B, S, k - W.LLADA_LARGE, seed=9400 + t, exclude=large)
        x = synth.perturb(x, large.cuda(), seed=9500 + t)
        logits = synth.normal((B, S, V), 1.0, 9600 + t, BF16, "cuda")
        sb, ss = torch.nonzero(spike, as_tuple=True)
        sv = torch.from_numpy(rng.integers(0, V, sb.numel()))
        logits[sb.cuda(), ss.cuda(), sv.cuda()] += 30.0
        h_prev = model.h_ref.clone()
        model.step(x, logits)
        torch.cuda.synchronize()
        assert int(model.step1.row_ptr[-1]) == B * k
        check_step(model, dims, wbits, f"step {t}", SEQS, k, h_prev, logits, 0.5, None, rng)
        del logits


@pytest.mark.parametrize("frac", [0.10, 0.25])
def test_dream_step_full_shape_teacher_forced(lib, frac):
    """The Dream-7B GQA step: 28 layers, d = 3584, 28 query heads on 4 kv heads of 128, FFN
    18944, B = 16, S = 2048, alpha 0 (change only), exactly k tokens moved per sequence and
    step, top-k at 10% and 25%; sequences 3 and 12 checked."""
    dims, L, skip = W.DREAM_GQA, 28, 4
    B, S, d = dims.B, dims.S, dims.d
    k = round(frac * S)
    print(f"full-shape Dream step at {frac:.0%} (k = {k}): {dims}", flush=True)
    w = shared_weights(dims, 9800)
    wbits = {n: bits(t) for n, t in w.items()}
    model = make_model(lib, dims, L, skip, k, 0.0, B * k, w)
    x = synth.normal((B, S, d), 1.0, 9810, BF16, "cuda")
    model.fill(x)
    rng = np.random.default_rng(9820)
    for t in range(2):
        large = synth.large_positions(B, S, k, seed=9830 + t)
        x = synth.perturb(x, large.cuda(), seed=9840 + t)
        h_prev = model.h_ref.clone()
        model.step(x)
        torch.cuda.synchronize()
        check_step(model, dims, wbits, f"step {t}", (3, 12), k, h_prev, None, 0.0, None, rng)


def test_long_context_step_full_shape_teacher_forced(lib):
    """Long-context block decoding: 32 LLaDA-8B layers, B = 1, S = 4096 (3584 prompt + 16 blocks
    of 32), alpha 0, the active block forced plus the top-64 by change among the other positions
    (SlowFast, German summary page, "Der SlowFast-Algorithmus" item 2); the block advances by
    one between the two steps."""
    dims, L, skip, k, P, BL = W.LLADA_LONG, 32, 4, 64, 3584, 32
    S, d = dims.S, dims.d
    print(f"full-shape long-context step: {dims}, {L} layers", flush=True)
    w = shared_weights(dims, 9900)
    wbits = {n: bits(t) for n, t in w.items()}
    model = make_model(lib, dims, L, skip, k, 0.0, k + BL, w)
    x = synth.normal((1, S, d), 1.0, 9910, BF16, "cuda")
    model.fill(x)
    rng = np.random.default_rng(9920)
    for t in range(2):
        flags = np.zeros((1, S), np.uint8)
        flags[0, P + t * BL:P + (t + 1) * BL] = 1
        block = torch.from_numpy(flags.astype(bool))
        large = synth.large_positions(1, S, k, seed=9930 + t, exclude=block) | block
        x = synth.perturb(x, large.cuda(), seed=9940 + t)
        h_prev = model.h_ref.clone()
        model.step(x, force=torch.from_numpy(flags).cuda())
        torch.cuda.synchronize()
        assert int(model.step1.row_ptr[-1]) == k + BL
        check_step(model, dims, wbits, f"step {t}", (0,), k, h_prev, None, 0.0, flags, rng)


@pytest.mark.parametrize("P", [0, 512])
def test_layer_adaptive_full_shape_teacher_forced(lib, P):
    """The layer-adaptive step at the LLaDA-8B shape (DyLLM, French summary page §2.A and §2.B):
    32 layers, B = 1, S = 1024, every token's attention context kept, context thresholds at the
    80th percentile of an untimed calibration step (as in the bench). Two steps after a fill; per
    step the layer-0 input set against the oracle's L1-normalised change, then per layer, on 8
    sampled rows each:
      * input set: K/V cache rows and query cache from the library's stored input of the layer;
      * contexts of input-set rows and of stable tokens: the exact softmax over every key of the
        layer's cache with the token's cached query (stable tokens come from the changed-key
        update of their stored state, carried across the steps);
      * cosine scores of every token from the library's contexts (this and the previous step),
        and the FFN set equal to the tokens above the layer's threshold by those scores;
      * FFN set: output rows from the library's stored input and context; the other rows keep
        the previous step's bits.
    P = 512 (DyLLM §2.C): positions 0-511 are a prompt, step 1 is response-only (the prompt is
    left out of every row set and of the context update: its contexts keep their bits) and step 2
    re-injects it (forced into every row set)."""
    from token_skipping_partial_amd.step import LayerAdaptiveModel, LayerWeights
    dims, L = W.LLADA_LAYER, 32
    B, S, d, H, Hkv, hd = dims.B, dims.S, dims.d, dims.H, dims.Hkv, dims.hd
    nq = H * hd
    print(f"full-shape layer-adaptive step: {dims}, {L} layers, prompt {P}", flush=True)
    w = shared_weights(dims, 9950)
    wbits = {n: bits(t) for n, t in w.items()}
    lw = LayerWeights.from_dict({n: t.cuda() for n, t in w.items()})
    shape = lib.Shape(B=B, S=S, d=d, H=H, Hkv=Hkv, hd=hd, F=dims.F, dtype="bf16")
    model = LayerAdaptiveModel(shape, [lw] * L, 0.05, [0.0] * L, prompt_len=P,
                               inject_every=2 if P else 0)
    prompt = torch.zeros(B, S, dtype=torch.bool)
    prompt[:, :P] = True
    x = [synth.normal((B, S, d), 1.0, 9960, BF16, "cuda")]
    for t in (1, 2):
        large = synth.large_positions(B, S, W.LLADA_LARGE, seed=9970 + t,
                                      exclude=prompt if P else None)
        x.append(synth.perturb(x[-1], large.cuda(), seed=9980 + t))
    model.fill(x[0])
    taus = []
    for l in range(L):   # calibration: each layer's 80th percentile, every later layer takes all
        model.step(x[1], tau_ctx=taus + [-1.0] * (L - l), record=True)
        taus.append(float(torch.quantile(model.layer_scores[l][:, P:].flatten(), 0.8).item()))
        model.fill(x[0])
    torch.cuda.synchronize()
    rng = np.random.default_rng(9990)
    scale = 1.0 / math.sqrt(hd)
    pick = lambda pool, n=PER_SEQ: np.sort(rng.choice(pool, min(n, len(pool)), replace=False)).astype(np.int32)  # noqa: E731
    for t in (1, 2):
        inject = P > 0 and t % 2 == 0
        flags = None
        if P:
            flags = np.zeros((B, S), np.uint8)
            flags[:, :P] = 1 if inject else 2
        prev_hidden = [h.clone() for h in model.hidden]
        x_prev = model.x_ref.clone()
        sets, rps = model.step(x[t], tau_ctx=taus, record=True)
        torch.cuda.synchronize()
        score0, _, _ = O.saliency(bits(x[t]), bits(x_prev), None, 0.0, O.DELTA_L1N)
        cand0 = score0 if flags is None else score0[flags == 0]
        margin = float(np.min(np.abs(cand0 - 0.05)))
        assert margin >= 1e-4, f"step {t}: input-change margin {margin:.2e}"
        osel, orp = O.select_compact(score0, flags, O.SEL_THRESHOLD, tau=0.05)
        n0 = int(rps[0][-1])
        assert n0 == int(orp[-1]) and np.array_equal(sets[0][:n0].cpu().numpy(), osel[:n0]), t
        counts = []
        for l in range(L):
            tag = f"step {t} layer {l}"
            A = sets[l][:int(rps[l][-1])].cpu().numpy()
            Fs = sets[l + 1][:int(rps[l + 1][-1])].cpu().numpy()
            counts.append(len(Fs))
            cur, prev = model.ctx[l][model.cur], model.ctx[l][1 - model.cur]
            kb, vb = bits(model.k[l]), bits(model.v[l])
            # input set: K/V and query rows from the stored layer input
            pa = pick(A)
            q, k2, v2 = O.gather_qkv_scatter_kv(bits(model.hidden[l]), wbits["g_attn"],
                                                wbits["w_qkv"], pa, np.array([0, len(pa)], np.int32),
                                                kb, vb, H, Hkv, hd, EPS, store="bf16")
            assert_close(host(model.k[l])[0][:, pa], k2[0][:, pa], TOL[BF16], f"{tag} K rows")
            assert_close(host(model.v[l])[0][:, pa], v2[0][:, pa], TOL[BF16], f"{tag} V rows")
            assert_close(host(model.q_all[l])[pa], q, TOL[BF16], f"{tag} query cache rows")
            # contexts: exact softmax over every key with the cached query; in a response-only
            # step the prompt's contexts keep their bits
            lo = P if (P and not inject) else 0
            rows = np.sort(np.concatenate([pa, pick(np.setdiff1d(np.arange(lo, S), A))])).astype(np.int32)
            o = O.partial_attn(bits(model.q_all[l])[rows], kb, vb, rows,
                               np.array([0, len(rows)], np.int32), H, Hkv, hd, scale)
            assert_close(host(cur)[rows], o, TOL[BF16], f"{tag} contexts (input set + stable)")
            if lo:
                pp = pick(np.arange(P))
                assert np.array_equal(bits(cur)[pp], bits(prev)[pp]), f"{tag}: prompt contexts"
            # cosine scores from the library's contexts; the FFN set by the threshold
            sc, _, _ = O.saliency(bits(cur).reshape(B, S, nq), bits(prev).reshape(B, S, nq), None,
                                  0.0, O.DELTA_COS)
            lib_sc = model.layer_scores[l].cpu().numpy()
            err = float(np.max(np.abs(lib_sc.astype(np.float64) - sc)))
            assert err <= 1e-4, f"{tag}: context scores differ by {err:.2e}"
            fsel, frp = O.select_compact(lib_sc, flags, O.SEL_THRESHOLD, tau=taus[l])
            assert np.array_equal(Fs, fsel[:int(frp[-1])]), f"{tag}: FFN set"
            # FFN rows from the stored input and context; the other rows untouched
            pf = pick(Fs)
            out = O.gather_ffn_scatter(bits(model.hidden[l]), bits(cur)[pf], wbits["w_o"],
                                       wbits["g_ffn"], wbits["w_gate"], wbits["w_up"],
                                       wbits["w_down"], pf, np.array([0, len(pf)], np.int32),
                                       bits(model.hidden[l + 1]), EPS, store="bf16")
            assert_close(host(model.hidden[l + 1])[0][pf], out[0][pf], TOL[BF16],
                         f"{tag} output rows")
            rest = pick(np.setdiff1d(np.arange(S), Fs))
            assert np.array_equal(bits(model.hidden[l + 1])[0][rest],
                                  bits(prev_hidden[l + 1])[0][rest]), f"{tag}: untouched rows"
        print(f"step {t}{' (inject)' if inject else ''}: input rows {n0}, FFN rows per layer "
              f"{counts}", flush=True)
