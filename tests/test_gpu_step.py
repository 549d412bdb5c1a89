"""Whole-step parity: saliency -> selection -> qkv/attention/ffn, GPU chain vs oracle chain.

Both sides start from the same seeded inputs and compute everything themselves, including the
step t-1 state of the caches (the block applied to h_prev on every token). The selection must be
identical (the inputs keep every score more than 1e-4 from the selection boundary); every float
output must agree within the fp32 / bf16 tolerance.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from parity import TOL, assert_close, host, same_bits, to_dev
from synth import workloads as W

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def oracle_weights(w):
    return {k: host(v) for k, v in w.items()}


def gpu_step(lib, dims, w_cpu, h_prev, h_cur, logits, sel_cfg, m_cap):
    from token_skipping_partial_amd.step import (LayerScratch, LayerWeights, SingleLayerStep,
                                                 all_rows, selected_layer)
    shape = lib.Shape(B=dims.B, S=dims.S, d=dims.d, H=dims.H, Hkv=dims.Hkv, hd=dims.hd, F=dims.F,
                      dtype="bf16" if dims.dtype == torch.bfloat16 else "f32", V=dims.V)
    w = LayerWeights.from_dict(w_cpu)
    hp, hc = to_dev(h_prev), to_dev(h_cur)
    lg = to_dev(logits) if logits is not None else None
    k = torch.zeros(dims.B, dims.Hkv, dims.S, dims.hd, dtype=dims.dtype, device="cuda")
    v = torch.zeros_like(k)
    h_out = torch.zeros(dims.B, dims.S, dims.d, dtype=dims.dtype, device="cuda")
    # step t-1: every token through the layer
    sel_all, rp_all = all_rows(shape)
    selected_layer(shape, w, hp, k, v, h_out, sel_all, rp_all, LayerScratch(shape, dims.B * dims.S))
    prior = (k.clone(), v.clone(), h_out.clone())
    step = SingleLayerStep(shape, sel_cfg, m_cap)
    step(w, hc, hp, lg, k, v, h_out)
    torch.cuda.synchronize()
    return step, prior, (k, v, h_out)


def check_chain(dims, step, prior, post, ref_prior, ref_sel, ref_rp, ref_post, r_score):
    tol = TOL[dims.dtype]
    M = int(ref_rp[-1])
    assert np.array_equal(step.row_ptr.cpu().numpy(), ref_rp)
    assert np.array_equal(step.sel_idx.cpu().numpy()[:M], ref_sel)
    assert_close(host(step.score), r_score, 1e-4, "score")
    rk0, rv0, ry0 = ref_prior
    assert_close(host(prior[0]), rk0, tol, "prior k")
    assert_close(host(prior[1]), rv0, tol, "prior v")
    assert_close(host(prior[2]), ry0, tol, "prior h_out")
    rq, ro, rk, rv, ry = ref_post
    assert_close(host(step.scratch.q_sel)[:M], rq, tol, "q_sel")
    assert_close(host(step.scratch.o_sel)[:M], ro, tol, "o_sel")
    assert_close(host(post[0]), rk, tol, "k_cache")
    assert_close(host(post[1]), rv, tol, "v_cache")
    assert_close(host(post[2]), ry, tol, "h_out")
    # rows outside the selection are bit-identical to the step t-1 state
    S = dims.S
    untouched = np.ones((dims.B, S), dtype=bool)
    untouched[ref_sel // S, ref_sel % S] = False
    ut = torch.from_numpy(untouched)
    assert same_bits(post[2].cpu()[ut], prior[2].cpu()[ut])
    assert same_bits(post[0].cpu().permute(0, 2, 1, 3)[ut], prior[0].cpu().permute(0, 2, 1, 3)[ut])
    assert same_bits(post[1].cpu().permute(0, 2, 1, 3)[ut], prior[1].cpu().permute(0, 2, 1, 3)[ut])


def test_tiny_f32_step(lib):
    """64 tokens, fp32, threshold at the midpoint of the 16th/17th scores -> 16 selected."""
    from token_skipping_partial_amd.step import SelectConfig
    dims = W.TINY_F32
    h_prev, h_cur, large, _, w = W.layer_inputs(dims, W.TINY_LARGE, seed=31)
    r_score, _, _ = O.saliency(host(h_cur), host(h_prev), None, 0.0)
    s = np.sort(r_score.astype(np.float64).ravel())[::-1]
    tau = float(np.float32(0.5 * (s[15] + s[16])))
    assert np.min(np.abs(r_score.astype(np.float64) - tau)) > 1e-4
    ref_sel, ref_rp = O.select_compact(r_score, None, O.SEL_THRESHOLD, tau=tau)
    assert len(ref_sel) == 16
    assert np.array_equal(np.sort(ref_sel), np.flatnonzero(large.numpy().ravel()))
    w64 = oracle_weights(w)
    scale = 1.0 / math.sqrt(dims.hd)
    ref_prior = O.dense_layer(host(h_prev), w64, dims.H, dims.Hkv, dims.hd, 1e-5, scale)
    ref_post = O.selected_layer(host(h_cur), w64, ref_sel, ref_rp, ref_prior[0], ref_prior[1],
                                ref_prior[2], dims.H, dims.Hkv, dims.hd, 1e-5, scale)
    cfg = SelectConfig(mode=O.SEL_THRESHOLD, tau=tau, alpha=0.0)
    step, prior, post = gpu_step(lib, dims, w, h_prev, h_cur, None, cfg, m_cap=16)
    check_chain(dims, step, prior, post, ref_prior, ref_sel, ref_rp, ref_post, r_score)


@pytest.mark.parametrize("kind", [O.DELTA_COS, O.DELTA_L2R])
def test_tiny_f32_step_other_deltas(lib, kind):
    from token_skipping_partial_amd.step import SelectConfig
    dims = W.TINY_F32
    h_prev, h_cur, large, _, w = W.layer_inputs(dims, W.TINY_LARGE, seed=32)
    r_score, _, _ = O.saliency(host(h_cur), host(h_prev), None, 0.0, kind)
    ref_sel, ref_rp = O.select_compact(r_score, None, O.SEL_TOPK, k=16)
    w64 = oracle_weights(w)
    scale = 1.0 / math.sqrt(dims.hd)
    ref_prior = O.dense_layer(host(h_prev), w64, dims.H, dims.Hkv, dims.hd, 1e-5, scale)
    ref_post = O.selected_layer(host(h_cur), w64, ref_sel, ref_rp, ref_prior[0], ref_prior[1],
                                ref_prior[2], dims.H, dims.Hkv, dims.hd, 1e-5, scale)
    cfg = SelectConfig(mode=O.SEL_TOPK, k=16, alpha=0.0, delta_kind=kind)
    step, prior, post = gpu_step(lib, dims, w, h_prev, h_cur, None, cfg, m_cap=16)
    check_chain(dims, step, prior, post, ref_prior, ref_sel, ref_rp, ref_post, r_score)


def llada_layer_seed():
    with open(os.path.join(GOLDEN, "llada_layer_seed.json")) as f:
        return json.load(f)["seed"]


@pytest.mark.slow
def test_llada_layer_step(lib):
    """LLaDA-8B-shaped layer, bf16, alpha = 0.5 with the full-vocabulary confidence, top-128."""
    from token_skipping_partial_amd.step import SelectConfig
    dims = W.LLADA_LAYER
    seed = llada_layer_seed()
    print(f"llada layer step seed={seed}", flush=True)
    h_prev, h_cur, large, logits, w = W.layer_inputs(dims, W.LLADA_LARGE, seed=seed)
    r_score, _, _ = O.saliency(host(h_cur[0]), host(h_prev[0]), host(logits[0]), 0.5)
    r_score = r_score.reshape(1, -1)
    ref_sel, ref_rp = O.select_compact(r_score, None, O.SEL_TOPK, k=W.LLADA_TOPK)
    w64 = oracle_weights(w)
    scale = 1.0 / math.sqrt(dims.hd)
    ref_prior = O.dense_layer(host(h_prev), w64, dims.H, dims.Hkv, dims.hd, 1e-5, scale)
    ref_post = O.selected_layer(host(h_cur), w64, ref_sel, ref_rp, ref_prior[0], ref_prior[1],
                                ref_prior[2], dims.H, dims.Hkv, dims.hd, 1e-5, scale)
    cfg = SelectConfig(mode=O.SEL_TOPK, k=W.LLADA_TOPK, alpha=0.5)
    step, prior, post = gpu_step(lib, dims, w, h_prev, h_cur, logits, cfg, m_cap=W.LLADA_TOPK)
    check_chain(dims, step, prior, post, ref_prior, ref_sel, ref_rp, ref_post, r_score)
    # determinism: the same step again gives the same bits
    step2, prior2, post2 = gpu_step(lib, dims, w, h_prev, h_cur, logits, cfg, m_cap=W.LLADA_TOPK)
    for a, b in zip(post, post2):
        assert same_bits(a, b)
    assert same_bits(step.scratch.o_sel, step2.scratch.o_sel)


def test_select_all_equals_dense_bf16(lib):
    """Selecting every token reproduces the dense block (oracle), GQA 2:1, B = 2."""
    from token_skipping_partial_amd.step import LayerScratch, LayerWeights, all_rows, selected_layer
    dims = W.Dims(B=2, S=96, d=256, H=4, Hkv=2, hd=128, F=512)
    _, h, _, _, w = W.layer_inputs(dims, 8, seed=41, with_logits=False)
    shape = lib.Shape(B=dims.B, S=dims.S, d=dims.d, H=dims.H, Hkv=dims.Hkv, hd=dims.hd, F=dims.F)
    k = torch.full((dims.B, dims.Hkv, dims.S, dims.hd), 9.0, dtype=dims.dtype, device="cuda")
    v = torch.full_like(k, -9.0)
    out = torch.zeros(dims.B, dims.S, dims.d, dtype=dims.dtype, device="cuda")
    sel, rp = all_rows(shape)
    selected_layer(shape, LayerWeights.from_dict(w), to_dev(h), k, v, out, sel, rp,
                   LayerScratch(shape, dims.B * dims.S))
    torch.cuda.synchronize()
    rk, rv, ry = O.dense_layer(host(h), oracle_weights(w), dims.H, dims.Hkv, dims.hd, 1e-5,
                               1.0 / math.sqrt(dims.hd))
    assert_close(host(k), rk, TOL[dims.dtype], "k")
    assert_close(host(v), rv, TOL[dims.dtype], "v")
    assert_close(host(out), ry, TOL[dims.dtype], "h_out")
