"""Whole-step parity of the layer-adaptive step (DyLLM French summary page §2.A: per layer, the
tokens whose attention context moved by more than a cosine threshold get their FFN recomputed;
§2.B: contexts of every token, exact for tokens whose layer input changed, changed-key update for
the rest) against the same composition of oracle functions.

Thresholds: every context threshold is taken by the oracle in the widest gap of its own scores
(middle 20-80% of the tokens), so both sides select the same rows; the test asserts that the gap
leaves a margin well above the rounding of bf16 contexts. Attention is made peaked (a larger
score scale) so that the contexts of different tokens move by clearly different amounts.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import TOL, assert_close, host, same_bits, to_dev

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
B, S, d, H, Hkv, hd, F, L = 2, 64, 256, 4, 2, 64, 512, 3
EPS = 1e-5
SCALE = 16.0 / math.sqrt(hd)
TAU_IN = 0.05          # input L1N change: large perturbations ~0.4, small ~8e-4
MARGIN = 2e-3          # minimum distance of every oracle score from its threshold


def inputs():
    x = [synth.normal((B, S, d), 1.0, 850, BF16)]
    for t in range(1, 3):
        large = synth.large_positions(B, S, 16, seed=860 + t)
        x.append(synth.perturb(x[-1], large, seed=870 + t))
    w = [synth.layer_weights(d, H, Hkv, hd, F, seed=880 + l, dtype=BF16) for l in range(L)]
    for l, wl in enumerate(w):
        wl["g_attn"] = (1.0 + synth.normal((d,), 0.1, 890 + l)).to(BF16)
        wl["g_ffn"] = (1.0 + synth.normal((d,), 0.1, 895 + l)).to(BF16)
    return x, w


def widest_gap_threshold(scores, cand=None):
    s = np.sort(scores.ravel() if cand is None else scores[cand])
    lo, hi = int(0.2 * (s.size - 1)), int(0.8 * (s.size - 1))
    gaps = s[lo + 1: hi + 1] - s[lo: hi]
    i = int(np.argmax(gaps))
    return 0.5 * (s[lo + i] + s[lo + i + 1]), 0.5 * float(gaps[i])


class OracleAdaptive:
    """The layer-adaptive step composed of oracle functions (float64)."""

    def __init__(self, w, prompt_len=0):
        self.P = prompt_len
        self.w = [{k: host(v) for k, v in wl.items()} for wl in w]
        self.all_sel = np.arange(B * S, dtype=np.int32)
        self.all_rp = np.arange(0, B * S + 1, S, dtype=np.int32)
        self.k = [np.zeros((B, Hkv, S, hd)) for _ in range(L)]
        self.v = [np.zeros((B, Hkv, S, hd)) for _ in range(L)]
        self.q = [np.zeros((B, S, H * hd)) for _ in range(L)]
        self.ctx = [None] * L
        self.lse = [None] * L
        self.hidden = [None] + [np.zeros((B, S, d)) for _ in range(L)]
        self.flags = None      # selection flags of the current step (response-only steps)

    def layer(self, l, sel, rp, tau):
        w = self.w[l]
        q_sel, self.k[l], self.v[l] = O.gather_qkv_scatter_kv(self.hidden[l], w["g_attn"],
                                                              w["w_qkv"], sel, rp, self.k[l],
                                                              self.v[l], H, Hkv, hd, EPS)
        self.q[l], o, lse = O.salient_attention(q_sel, self.q[l], self.k[l], self.v[l], sel, rp,
                                                H, Hkv, hd, SCALE, q_first=self.P,
                                                o_prev=self.ctx[l], lse_prev=self.lse[l])
        if tau is None:
            fs, frp, margin = self.all_sel, self.all_rp, None
        else:
            score, _, _ = O.saliency(o, self.ctx[l], None, 0.0, O.DELTA_COS)
            cand = None if self.flags is None else self.flags == 0
            if tau == "auto":
                tau, margin = widest_gap_threshold(score, cand)
            else:
                margin = float(np.min(np.abs(score - tau)))
            fs, frp = O.select_compact(score, self.flags, O.SEL_THRESHOLD, tau=tau)
        M = int(frp[-1])
        rows = o.reshape(B * S, -1)[fs[:M]]
        self.hidden[l + 1] = O.gather_ffn_scatter(self.hidden[l], rows, w["w_o"], w["g_ffn"],
                                                  w["w_gate"], w["w_up"], w["w_down"], fs, frp,
                                                  self.hidden[l + 1], EPS)
        self.ctx[l], self.lse[l] = o, lse
        return fs[:M].copy(), frp, tau, margin

    def fill(self, x0):
        self.hidden[0] = x0
        self.x_ref = x0
        for l in range(L):
            self.layer(l, self.all_sel, self.all_rp, None)

    def step(self, x, inject=False):
        if self.P:
            self.flags = np.zeros((B, S), np.uint8)
            self.flags[:, :self.P] = 1 if inject else 2
        score, _, _ = O.saliency(x, self.x_ref, None, 0.0, O.DELTA_L1N)
        sel, rp = O.select_compact(score, self.flags, O.SEL_THRESHOLD, tau=TAU_IN)
        self.hidden[0] = x
        self.x_ref = x
        sets, taus = [(sel[:int(rp[-1])].copy(), rp)], []
        for l in range(L):
            fs, frp, tau, margin = self.layer(l, sel, rp, "auto")
            assert margin >= MARGIN, f"layer {l}: oracle score margin {margin:.2e} too small"
            sets.append((fs, frp))
            taus.append(tau)
            sel, rp = fs, frp
        return sets, taus


def test_layer_adaptive_steps_match_the_oracle(lib):
    from token_skipping_partial_amd.step import LayerAdaptiveModel, LayerWeights
    print("layer-adaptive step: fill + 2 steps, 3 layers", flush=True)
    x, w = inputs()
    ref = OracleAdaptive(w)
    ref.fill(host(x[0]))
    shape = lib.Shape(B=B, S=S, d=d, H=H, Hkv=Hkv, hd=hd, F=F, dtype="bf16")
    layers = [LayerWeights.from_dict(wl, "cuda") for wl in w]
    model = LayerAdaptiveModel(shape, layers, TAU_IN, [0.0] * L, scale=SCALE)
    model.fill(x[0].cuda())
    torch.cuda.synchronize()
    assert_close(host(model.hidden[L]), ref.hidden[L], TOL[BF16], "fill output")
    for t in (1, 2):
        sets, taus = ref.step(host(x[t]))
        print(f"  step {t}: rows per layer input {[len(s) for s, _ in sets]}, thresholds "
              f"{[round(v, 4) for v in taus]}", flush=True)
        sel, rp = model.step(x[t].cuda(), tau_ctx=taus)
        torch.cuda.synchronize()
        for i, (want, want_rp) in enumerate(sets):
            got_rp = rp[i].cpu().numpy()
            assert np.array_equal(got_rp, want_rp), (t, i, got_rp, want_rp)
            assert np.array_equal(sel[i][:len(want)].cpu().numpy(), want), (t, i)
        for l in range(L):
            ctx = host(model.ctx[l][model.cur]).reshape(B, S, -1)
            assert_close(ctx, ref.ctx[l], TOL[BF16], f"step {t} layer {l} contexts")
        assert_close(host(model.hidden[L]), ref.hidden[L], TOL[BF16], f"step {t} output")


def test_response_only_steps_match_the_oracle(lib):
    """DyLLM §2.C on top of the layer-adaptive step: a 32-token prompt at the front of each
    sequence is left out of the row sets and of the context update in response-only steps
    (steps 1 and 3) and forced into every row set when it is re-injected (step 2). Inputs move
    at response positions only."""
    from token_skipping_partial_amd.step import LayerAdaptiveModel, LayerWeights
    P = 32
    print("response-only steps: fill + 3 steps, 3 layers, prompt 32 of 64", flush=True)
    _, w = inputs()
    x = [synth.normal((B, S, d), 1.0, 851, BF16)]
    prompt = torch.zeros(B, S, dtype=torch.bool)
    prompt[:, :P] = True
    for t in range(1, 4):
        large = synth.large_positions(B, S, 12, seed=865 + t, exclude=prompt)
        x.append(synth.perturb(x[-1], large, seed=875 + t))
    ref = OracleAdaptive(w, prompt_len=P)
    ref.fill(host(x[0]))
    shape = lib.Shape(B=B, S=S, d=d, H=H, Hkv=Hkv, hd=hd, F=F, dtype="bf16")
    layers = [LayerWeights.from_dict(wl, "cuda") for wl in w]
    model = LayerAdaptiveModel(shape, layers, TAU_IN, [0.0] * L, scale=SCALE, prompt_len=P,
                               inject_every=2)
    model.fill(x[0].cuda())
    for t in (1, 2, 3):
        inject = t == 2
        prompt_ctx = [host(model.ctx[l][model.cur]).reshape(B, S, -1)[:, :P] for l in range(L)]
        sets, taus = ref.step(host(x[t]), inject=inject)
        print(f"  step {t} ({'inject' if inject else 'response-only'}): rows per layer input "
              f"{[len(s) for s, _ in sets]}", flush=True)
        sel, rp = model.step(x[t].cuda(), tau_ctx=taus)
        torch.cuda.synchronize()
        for i, (want, want_rp) in enumerate(sets):
            got_rp = rp[i].cpu().numpy()
            assert np.array_equal(got_rp, want_rp), (t, i, got_rp, want_rp)
            got = sel[i][:len(want)].cpu().numpy()
            assert np.array_equal(got, want), (t, i)
            if inject:
                assert np.isin(np.arange(B * S)[(np.arange(B * S) % S) < P], got).all()
            else:
                assert np.all(got % S >= P)
        for l in range(L):
            ctx = host(model.ctx[l][model.cur]).reshape(B, S, -1)
            assert_close(ctx, ref.ctx[l], TOL[BF16], f"step {t} layer {l} contexts")
            if not inject:   # the prompt's contexts are the previous step's, bit for bit
                assert np.array_equal(ctx[:, :P], prompt_ctx[l]), (t, l)
        assert_close(host(model.hidden[L]), ref.hidden[L], TOL[BF16], f"step {t} output")
