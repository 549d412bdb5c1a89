"""Whole-step parity over chains of steps: the early-skip step driver on the GPU against the same
chain run by the oracle alone.

Both sides start from the same seeded inputs (weights, layer-0 input, per-step perturbations,
logits, all drawn on the host) and run a fill step (every layer on every token) and then several
early-skip steps with every cache carried from step to step: layers below the skip layer on every
token, saliency of the skip layer's input against its previous-step value, one selection reused by
every later layer (ES-dLLM, German summary page §2.B). The oracle never sees a GPU value: it runs
its own chain, rounding to bfloat16 exactly where the library stores bfloat16 tensors (q rows,
K/V cache rows, attention outputs, hidden rows). After every step the selection must be
bit-identical, and every layer's K/V cache and output hidden state must agree within the bf16
tolerance; the rows a selected layer does not write must be bit-identical to their previous-step
values on the GPU.

The chains have the depth and structure of the three multi-layer workloads, at a width the oracle
finishes in seconds:
  batched step   32 layers, B = 8, skip at 4, alpha = 0.5, top-20% per sequence;
  long context   32 layers, B = 1, S = 4096 (3584 prompt + 16 blocks of 32), skip at 4, the
                 active block forced + top-64 by change, commit of the active block after every
                 step (SlowFast, German summary page, "Der SlowFast-Algorithmus" item 2);
  Dream GQA      28 layers, B = 16, 7 query heads per kv head, skip at 4, alpha = 0, top-10% and
                 top-25% per sequence.
Inputs keep every oracle score far from the selection boundary: the moving tokens get N(0, 0.5^2)
perturbations (the rest N(0, (1e-3)^2)), and with alpha = 0.5 the remaining top-k slots go to
tokens whose logit row carries one raised logit (confidence ~1) while every other row is
N(0, 1) over 1024 entries (confidence < 0.03); the margin is asserted on the oracle's scores.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import TOL, assert_close, host, same_bits
from synth import workloads as W

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
EPS = 1e-5


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint16).numpy()


def chain_weights(dims, L, seed):
    out = []
    for l in range(L):
        w = synth.layer_weights(dims.d, dims.H, dims.Hkv, dims.hd, dims.F, seed=seed + l)
        w["g_attn"] = (1.0 + synth.normal((dims.d,), 0.1, seed + 1000 + l)).to(BF16)
        w["g_ffn"] = (1.0 + synth.normal((dims.d,), 0.1, seed + 2000 + l)).to(BF16)
        out.append(w)
    return out


def spiked_logits(B, S, V, spike_pos, seed):
    """N(0, 1) logits [B, S, V] (bf16); rows at spike_pos [B, S] get one logit raised by 30."""
    z = synth.normal((B, S, V), 1.0, seed)
    rng = np.random.default_rng(seed)
    b, s = np.nonzero(spike_pos.numpy())
    z[torch.from_numpy(b), torch.from_numpy(s), torch.from_numpy(rng.integers(0, V, len(b)))] += 30.0
    return z.to(BF16)


def topk_margin(score, k):
    """Smallest distance of a score to its sequence's top-k boundary (midpoint of the k-th and
    (k+1)-th largest)."""
    s = -np.sort(-score.astype(np.float64), axis=1)
    thr = 0.5 * (s[:, k - 1] + s[:, k])
    return float(np.min(np.abs(score - thr[:, None])))


class OracleChain:
    """The early-skip step driver written with the oracle's calls (bf16 stores)."""

    def __init__(self, dims, weights, skip, k, alpha):
        self.d, self.skip, self.k, self.alpha = dims, skip, k, alpha
        self.w = [{n: bits(t) for n, t in w.items()} for w in weights]
        L = len(weights)
        B, S = dims.B, dims.S
        self.K = [np.zeros((B, dims.Hkv, S, dims.hd)) for _ in range(L)]
        self.V = [np.zeros((B, dims.Hkv, S, dims.hd)) for _ in range(L)]
        self.h = [np.zeros((B, S, dims.d)) for _ in range(L + 1)]
        self.all_sel = np.arange(B * S, dtype=np.int32)
        self.all_rp = np.arange(0, B * S + 1, S, dtype=np.int32)
        self.scale = 1.0 / math.sqrt(dims.hd)

    def _layer(self, l, sel, rp):
        d = self.d
        _, _, self.K[l], self.V[l], self.h[l + 1] = O.selected_layer(
            self.h[l], self.w[l], sel, rp, self.K[l], self.V[l], self.h[l + 1], d.H, d.Hkv, d.hd,
            EPS, self.scale, store="bf16")

    def fill(self, x0):
        self.h[0] = O.decode_bf16(x0)
        for l in range(len(self.w)):
            self._layer(l, self.all_sel, self.all_rp)
        self.h_ref = self.h[self.skip]

    def lower(self, x):
        """Layers below the skip layer on every token; returns the skip layer's input."""
        self.h[0] = O.decode_bf16(x)
        for l in range(self.skip):
            self._layer(l, self.all_sel, self.all_rp)
        return self.h[self.skip]

    def score(self, logits):
        return O.saliency(self.h[self.skip], self.h_ref, logits, self.alpha)[0]

    def upper(self, force, score):
        sel, rp = O.select_compact(score, force, O.SEL_TOPK, k=self.k)
        self.h_ref = self.h[self.skip]
        for l in range(self.skip, len(self.w)):
            self._layer(l, sel, rp)
        return sel, rp


def gpu_model(lib, dims, weights, skip, k, alpha, m_cap):
    from token_skipping_partial_amd.step import EarlySkipModel, LayerWeights, SelectConfig
    shape = lib.Shape(B=dims.B, S=dims.S, d=dims.d, H=dims.H, Hkv=dims.Hkv, hd=dims.hd, F=dims.F,
                      dtype="bf16", V=dims.V)
    layers = [LayerWeights.from_dict(w) for w in weights]
    return EarlySkipModel(shape, layers, skip, SelectConfig(mode=lib.SEL_TOPK, k=k, alpha=alpha),
                          m_cap=m_cap), shape


def compare_layers(model, ora, tag, sel=None, rp=None, before=None):
    """Every layer's K/V cache and output hidden state against the oracle chain; with `before`
    (GPU tensors of the selected layers taken before the step), rows outside the selection are
    bit-identical to them."""
    tol = TOL[BF16]
    L = len(model.layers)
    for l in range(L):
        assert_close(host(model.k[l]), ora.K[l], tol, f"{tag} layer {l} K")
        assert_close(host(model.v[l]), ora.V[l], tol, f"{tag} layer {l} V")
        assert_close(host(model.hidden[l + 1]), ora.h[l + 1], tol, f"{tag} layer {l} hidden out")
    if before is None:
        return
    d = ora.d
    keep = torch.ones(d.B, d.S, dtype=torch.bool)
    ids = sel[: rp[-1]]
    keep[torch.from_numpy(ids // d.S).long(), torch.from_numpy(ids % d.S).long()] = False
    for l, (k0, v0, h0) in before.items():
        assert same_bits(model.k[l].cpu().permute(0, 2, 1, 3)[keep], k0.cpu().permute(0, 2, 1, 3)[keep])
        assert same_bits(model.v[l].cpu().permute(0, 2, 1, 3)[keep], v0.cpu().permute(0, 2, 1, 3)[keep])
        assert same_bits(model.hidden[l + 1].cpu()[keep], h0.cpu()[keep])


def snapshot(model, skip):
    return {l: (model.k[l].clone(), model.v[l].clone(), model.hidden[l + 1].clone())
            for l in range(skip, len(model.layers))}


def check_selection(model, ora_sel, ora_rp):
    s1 = model.step1
    rp = s1.row_ptr.cpu().numpy()
    assert np.array_equal(rp, ora_rp), (rp, ora_rp)
    assert np.array_equal(s1.sel_idx.cpu().numpy()[: rp[-1]], ora_sel)


@pytest.mark.slow
def test_batched_step_chain(lib):
    """Structure of the batched LLaDA-8B step: 32 layers, B = 8, skip at 4, alpha = 0.5 with
    previous-step logits, top-20% per sequence, 3 steps after the fill."""
    dims = W.Dims(B=8, S=128, d=256, H=2, Hkv=2, hd=128, F=512, V=1024)
    L, skip, k, n_large = 32, 4, 26, 19
    print(f"batched step chain: {dims}", flush=True)
    weights = chain_weights(dims, L, 6100)
    model, shape = gpu_model(lib, dims, weights, skip, k, 0.5, dims.B * k)
    ora = OracleChain(dims, weights, skip, k, 0.5)
    x = synth.normal((dims.B, dims.S, dims.d), 1.0, 6200, BF16)
    model.fill(x.cuda())
    ora.fill(bits(x))
    torch.cuda.synchronize()
    compare_layers(model, ora, "fill")
    for t in range(1, 4):
        large = synth.large_positions(dims.B, dims.S, n_large, seed=6300 + t)
        spikes = synth.large_positions(dims.B, dims.S, k - n_large, seed=6400 + t, exclude=large)
        x = synth.perturb(x, large, seed=6500 + t)
        logits = spiked_logits(dims.B, dims.S, dims.V, spikes, 6600 + t)
        ora.lower(bits(x))
        score = ora.score(bits(logits))
        margin = topk_margin(score, k)
        print(f"step {t}: oracle score margin {margin:.3e}", flush=True)
        assert margin > 1e-4
        sel, rp = ora.upper(None, score)
        before = snapshot(model, skip)
        model.step(x.cuda(), logits.cuda())
        torch.cuda.synchronize()
        # the score is computed from bf16 hidden states: the bf16 tolerance applies
        assert_close(model.step1.score.cpu().numpy(), score, TOL[BF16], f"step {t} scores")
        check_selection(model, sel, rp)
        compare_layers(model, ora, f"step {t}", sel, rp, before)


@pytest.mark.slow
def test_long_context_decode_chain(lib):
    """Structure of long-context block decoding: 32 layers, B = 1, S = 4096 (3584 prompt + 16
    blocks of 32), skip at 4, alpha = 0: the active block forced plus the top-64 by change; after
    every step the commit of the active block (confidence > 0.9, else the best one) decides the
    next step's forced block. The second step's logits raise one logit in every row of the
    block, so it completes and the next block becomes the forced one."""
    dims = W.Dims(B=1, S=4096, d=64, H=1, Hkv=1, hd=64, F=128, V=512)
    L, skip, k, P, BL = 32, 4, 64, 3584, 32
    print(f"long-context chain: {dims}", flush=True)
    weights = chain_weights(dims, L, 7100)
    model, shape = gpu_model(lib, dims, weights, skip, k, 0.0, dims.B * (k + BL))
    ora = OracleChain(dims, weights, skip, k, 0.0)
    x = synth.normal((dims.B, dims.S, dims.d), 1.0, 7200, BF16)
    model.fill(x.cuda())
    ora.fill(bits(x))
    torch.cuda.synchronize()
    compare_layers(model, ora, "fill")
    tok = np.full((1, dims.S), -1, np.int32)
    tok[0, :P] = np.random.default_rng(7).integers(0, dims.V, P)
    blk = np.zeros(1, np.int32)
    flags = np.zeros((1, dims.S), np.uint8)
    flags[0, P:P + BL] = 1
    tok_d, blk_d = torch.from_numpy(tok).cuda(), torch.from_numpy(blk).cuda()
    flags_d = torch.from_numpy(flags).cuda()
    cidx = torch.zeros(BL, dtype=torch.int32, device="cuda")
    crp = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws = lib.workspace(lib.OP_COMMIT, shape, BL)
    for t in range(1, 4):
        block = torch.from_numpy(flags.astype(bool))
        large = synth.large_positions(1, dims.S, k, seed=7300 + t, exclude=block) | block
        x = synth.perturb(x, large, seed=7400 + t)
        ora.lower(bits(x))
        score = ora.score(None)
        cand = score[~flags.astype(bool)].reshape(1, -1)
        margin = topk_margin(cand, k)
        print(f"step {t}: oracle score margin {margin:.3e}", flush=True)
        assert margin > 1e-4
        sel, rp = ora.upper(flags, score)
        before = snapshot(model, skip)
        model.step(x.cuda(), force=flags_d)
        torch.cuda.synchronize()
        check_selection(model, sel, rp)
        compare_layers(model, ora, f"step {t}", sel, rp, before)
        # commit: spikes in some rows of the block (every row at step 2), confidence < 0.3 elsewhere
        spike = np.zeros((1, dims.S), bool)
        lo = P + int(blk[0]) * BL
        rows = np.arange(lo, lo + BL) if t == 2 else lo + np.array([3, 17])
        spike[0, rows] = True
        logits = spiked_logits(1, dims.S, dims.V, torch.from_numpy(spike), 7500 + t)
        lib.dllm_commit(shape, logits.cuda(), P, BL, 0.9, 1, tok_d, blk_d, cidx, crp, flags_d, ws)
        tok, blk, c_sel, c_rp, flags = O.commit_step(bits(logits), tok, blk, P, BL, 0.9, 1)
        tok, blk = tok.astype(np.int32), blk.astype(np.int32)
        torch.cuda.synchronize()
        assert np.array_equal(crp.cpu().numpy(), c_rp)
        assert np.array_equal(cidx.cpu().numpy()[: c_rp[-1]], c_sel)
        assert np.array_equal(tok_d.cpu().numpy(), tok)
        assert np.array_equal(blk_d.cpu().numpy(), blk)
        assert np.array_equal(flags_d.cpu().numpy(), flags)
    assert int(blk[0]) == 1, "the second step's commit completes the first block"


@pytest.mark.slow
@pytest.mark.parametrize("frac", [0.10, 0.25])
def test_dream_gqa_chain(lib, frac):
    """Structure of the Dream-7B GQA workload: 28 layers, B = 16, 7 query heads per kv head,
    skip at 4, alpha = 0, exactly k moving tokens per sequence and step, top-k (10% or 25%)."""
    dims = W.Dims(B=16, S=128, d=448, H=7, Hkv=1, hd=64, F=576, V=0)
    L, skip = 28, 4
    k = round(frac * dims.S)
    print(f"Dream GQA chain at {frac:.0%} (k = {k}): {dims}", flush=True)
    weights = chain_weights(dims, L, 8100)
    model, shape = gpu_model(lib, dims, weights, skip, k, 0.0, dims.B * k)
    ora = OracleChain(dims, weights, skip, k, 0.0)
    x = synth.normal((dims.B, dims.S, dims.d), 1.0, 8200, BF16)
    model.fill(x.cuda())
    ora.fill(bits(x))
    torch.cuda.synchronize()
    compare_layers(model, ora, "fill")
    for t in range(1, 3):
        large = synth.large_positions(dims.B, dims.S, k, seed=8300 + t)
        x = synth.perturb(x, large, seed=8400 + t)
        ora.lower(bits(x))
        score = ora.score(None)
        margin = topk_margin(score, k)
        print(f"step {t}: oracle score margin {margin:.3e}", flush=True)
        assert margin > 1e-4
        sel, rp = ora.upper(None, score)
        before = snapshot(model, skip)
        model.step(x.cuda())
        torch.cuda.synchronize()
        check_selection(model, sel, rp)
        compare_layers(model, ora, f"step {t}", sel, rp, before)
