"""Whole-step parity of the batched LLaDA-8B step at its full shape, teacher-forced per layer.

The step: 32 layers (d = 4096, 32 x 128 MHA, FFN 12288), B = 8, S = 1024, layers 0-3 on every
token, saliency of layer 4's input against its previous-step value blended with the previous
step's max-softmax confidence over the 126464-entry vocabulary (alpha = 0.5), top-205 per
sequence, layers 4-31 on those rows against the cached K/V (ES-dLLM, German summary page,
§2.A equation and §2.B). The GPU runs a fill step and two early-skip steps with every cache
carried.

After each step the oracle checks, for two of the eight sequences:
  * the selection: the oracle's scores from the library's own stored bf16 inputs of layer 4
    (this step's and the previous step's) and the logits, top-205 bit-identical to the
    library's rows, every score at least 1e-4 from the boundary;
  * every layer (dense and selected): sampled rows recomputed by the oracle from the library's
    stored bf16 input of that layer and the layer's K/V cache after the step (the other selected
    rows' new K/V entries are the library's), rounding to bf16 where the library stores bf16;
    the rows' K/V cache entries and output hidden rows must agree within the bf16 tolerance.
Teacher forcing keeps the check at full size affordable (the oracle computes 16 rows per layer,
not 8192) while every layer of the real shape, caches and selection of each step take part.

Inputs: one set of random N(0, 0.02^2) weights for all layers (non-unit norm gains), X0 N(0, 1),
per step 154 tokens per sequence moved by N(0, 0.5^2) and the rest by N(0, (1e-3)^2); logits
N(0, 1) with one logit raised by 30 on 51 other tokens per sequence, so the top-205 are those
205 tokens by a wide margin.
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


def test_llada_step_full_shape_teacher_forced(lib):
    from token_skipping_partial_amd.step import EarlySkipModel, LayerWeights, SelectConfig

    dims, L, skip, k = W.LLADA_STEP, 32, W.STEP_SKIP, W.STEP_TOPK
    B, S, d, H, Hkv, hd, V = dims.B, dims.S, dims.d, dims.H, dims.Hkv, dims.hd, dims.V
    scale = 1.0 / math.sqrt(hd)
    print(f"full-shape batched step: {dims}, {L} layers", flush=True)
    w = synth.layer_weights(d, H, Hkv, hd, dims.F, seed=9100)
    w["g_attn"] = (1.0 + synth.normal((d,), 0.1, 9101)).to(BF16)
    w["g_ffn"] = (1.0 + synth.normal((d,), 0.1, 9102)).to(BF16)
    wbits = {n: bits(t) for n, t in w.items()}
    lw = LayerWeights.from_dict({n: t.cuda() for n, t in w.items()})
    shape = lib.Shape(B=B, S=S, d=d, H=H, Hkv=Hkv, hd=hd, F=dims.F, dtype="bf16", V=V)
    model = EarlySkipModel(shape, [lw] * L, skip, SelectConfig(mode=lib.SEL_TOPK, k=k, alpha=0.5),
                           m_cap=B * k)
    x = synth.normal((B, S, d), 1.0, 9200, BF16, "cuda")
    model.fill(x)
    idx = torch.tensor(SEQS, device="cuda")
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
        print(f"step {t}: checking the selection", flush=True)
        rp = model.step1.row_ptr.cpu().numpy()
        assert rp[-1] == B * k
        sel_gpu = model.step1.sel_idx.cpu().numpy()[: rp[-1]]
        rows_of = {}
        for b in SEQS:
            score, _, _ = O.saliency(bits(model.hidden[skip][b:b + 1]), bits(h_prev[b:b + 1]),
                                     bits(logits[b:b + 1]), 0.5)
            assert topk_margin(score, k) >= 1e-4, "inputs too close to the selection boundary"
            osel, orp = O.select_compact(score, None, O.SEL_TOPK, k=k)
            mine = sel_gpu[rp[b]:rp[b + 1]] - b * S
            assert np.array_equal(mine, osel[: orp[-1]]), f"step {t} sequence {b} selection"
            rows_of[b] = mine
        del logits
        for l in range(L):
            # rows to check: any positions in the dense layers, selected ones above
            picks = []
            for b in SEQS:
                pool = np.arange(S) if l < skip else rows_of[b]
                picks.append(np.sort(rng.choice(pool, PER_SEQ, replace=False)).astype(np.int32))
            sel = np.concatenate([i * S + p for i, p in enumerate(picks)]).astype(np.int32)
            srp = np.array([0, PER_SEQ, 2 * PER_SEQ], np.int32)
            _, _, k2, v2, y2 = O.selected_layer(
                bits(model.hidden[l][idx]), wbits, sel, srp, bits(model.k[l][idx]),
                bits(model.v[l][idx]), bits(model.hidden[l + 1][idx]), H, Hkv, hd, EPS, scale,
                store="bf16")
            kg, vg, yg = host(model.k[l][idx]), host(model.v[l][idx]), host(model.hidden[l + 1][idx])
            for i, p in enumerate(picks):
                tag = f"step {t} layer {l} sequence {SEQS[i]}"
                assert_close(kg[i][:, p], k2[i][:, p], TOL[BF16], f"{tag} K rows")
                assert_close(vg[i][:, p], v2[i][:, p], TOL[BF16], f"{tag} V rows")
                assert_close(yg[i][p], y2[i][p], TOL[BF16], f"{tag} hidden rows")
        print(f"step {t}: {L} layers checked", flush=True)
