"""The C++ oracle's own pieces (no GPU): its bfloat16 rounding against a library routine, the
rounding applied only at the tensors the library stores, and agreement with the independently
written numpy oracle on random inputs of every call."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle as O

R = oracle.numpy_ref


def _torch_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 values rounded to bfloat16 by torch (round to nearest, ties to even)."""
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_library_rounding():
    rng = np.random.default_rng(3)
    vals = [rng.standard_normal(2000).astype(np.float32),
            (rng.standard_normal(500) * 1e-38).astype(np.float32),    # subnormal range
            (rng.standard_normal(500) * 1e38).astype(np.float32)]
    # exact ties: a bfloat16 value plus half its spacing (upper 16 bits, then bit 15 set)
    exp = rng.integers(1, 255, 1000, dtype=np.uint32)          # finite, normal bfloat16
    frac = rng.integers(0, 128, 1000, dtype=np.uint32)
    sign = rng.integers(0, 2, 1000, dtype=np.uint32)
    base = ((sign << 15) | (exp << 7) | frac) << 16
    ties = (base | 0x8000).view(np.float32)
    near = (base | 0x7FFF).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.4028235e38, -3.39e38,
                        1e-45, -1e-45, 1.17549435e-38], dtype=np.float32)
    for x in vals + [ties, near, special]:
        got = np.array([O.round_bf16(float(v)) for v in x])
        ref = _torch_bf16(x)
        assert np.array_equal(got, ref) and np.array_equal(np.signbit(got), np.signbit(ref))
    assert math.isnan(O.round_bf16(float("nan")))


def test_round_bf16_of_float64_values():
    # a float64 between two bfloat16 neighbours goes to the nearer one (no detour via float32):
    # 1 + 2^-8 + 2^-30 lies just above the tie 1 + 2^-8 and rounds up to 1 + 2^-7
    assert O.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0                 # the tie itself: to even
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie between odd and even


def _layer_inputs(B=2, S=24, d=64, H=4, Hkv=2, hd=16, F=96, seed=5):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((B, S, d))
    w = {"g_attn": 1.0 + 0.1 * rng.standard_normal(d),
         "w_qkv": 0.1 * rng.standard_normal(((H + 2 * Hkv) * hd, d)),
         "w_o": 0.1 * rng.standard_normal((d, H * hd)),
         "g_ffn": 1.0 + 0.1 * rng.standard_normal(d),
         "w_gate": 0.1 * rng.standard_normal((F, d)),
         "w_up": 0.1 * rng.standard_normal((F, d)),
         "w_down": 0.1 * rng.standard_normal((d, F))}
    kc = rng.standard_normal((B, Hkv, S, hd))
    vc = rng.standard_normal((B, Hkv, S, hd))
    y = rng.standard_normal((B, S, d))
    sel, rp = R.select_compact(rng.standard_normal((B, S)).astype(np.float32), None, R.SEL_TOPK,
                               k=7)
    return h, w, kc, vc, y, sel, rp


@pytest.mark.parametrize("store", ["bf16", "f32"])
def test_rounding_only_at_stored_tensors(store):
    """Each call with store=X returns exactly the rounding of the unrounded result of the same
    inputs: nothing before the store is rounded."""
    h, w, kc, vc, y, sel, rp = _layer_inputs()
    rnd = ((lambda a: np.vectorize(O.round_bf16)(a)) if store == "bf16"
           else (lambda a: a.astype(np.float32).astype(np.float64)))
    q64, k64, v64 = O.gather_qkv_scatter_kv(h, w["g_attn"], w["w_qkv"], sel, rp, kc, vc, 4, 2,
                                            16, 1e-5)
    q, k, v = O.gather_qkv_scatter_kv(h, w["g_attn"], w["w_qkv"], sel, rp, kc, vc, 4, 2, 16,
                                      1e-5, store=store)
    assert np.array_equal(q, rnd(q64))
    ids = sel[: rp[-1]]
    b, s = ids // 24, ids % 24
    assert np.array_equal(k[b, :, s], rnd(k64[b, :, s])) and np.array_equal(v[b, :, s], rnd(v64[b, :, s]))
    untouched = np.ones((2, 24), bool)
    untouched[b, s] = False
    assert np.array_equal(k.transpose(0, 2, 1, 3)[untouched], kc.transpose(0, 2, 1, 3)[untouched])
    o64 = O.partial_attn(q, k, v, sel, rp, 4, 2, 16, 0.25)
    o = O.partial_attn(q, k, v, sel, rp, 4, 2, 16, 0.25, store=store)
    assert np.array_equal(o, rnd(o64))
    y64 = O.gather_ffn_scatter(h, o, w["w_o"], w["g_ffn"], w["w_gate"], w["w_up"], w["w_down"],
                               sel, rp, y, 1e-5)
    yr = O.gather_ffn_scatter(h, o, w["w_o"], w["g_ffn"], w["w_gate"], w["w_up"], w["w_down"],
                              sel, rp, y, 1e-5, store=store)
    assert np.array_equal(yr[b, s], rnd(y64[b, s]))
    assert np.array_equal(yr[untouched], y[untouched])


def test_agrees_with_numpy_oracle_on_every_call():
    h, w, kc, vc, y, sel, rp = _layer_inputs(seed=9)
    H, Hkv, hd, eps, scale = 4, 2, 16, 1e-5, 0.25
    for kind in (R.DELTA_L1N, R.DELTA_COS, R.DELTA_L2R):
        assert np.allclose(O.delta_variation(h, y, kind), R.delta_variation(h, y, kind),
                           rtol=1e-12, atol=0)
    z = np.random.default_rng(1).standard_normal((2, 24, 300)) * 3
    assert np.allclose(O.max_softmax_confidence(z), R.max_softmax_confidence(z), rtol=1e-12)
    a = O.saliency(h, y, z, 0.5)
    b = R.saliency(h, y, z, 0.5)
    assert np.array_equal(a[0], b[0]) or np.max(np.abs(a[0] - b[0])) <= 1e-7
    got = O.selected_layer(h, w, sel, rp, kc, vc, y, H, Hkv, hd, eps, scale)
    ref = R.selected_layer(h, w, sel, rp, kc, vc, y, H, Hkv, hd, eps, scale)
    for g, r in zip(got, ref):
        assert np.allclose(g, r, rtol=1e-10, atol=1e-12)
    kd, vd, yd = O.dense_layer(h, w, H, Hkv, hd, eps, scale)
    kr, vr, yr = R.dense_layer(h, w, H, Hkv, hd, eps, scale)
    for g, r in ((kd, kr), (vd, vr), (yd, yr)):
        assert np.allclose(g, r, rtol=1e-10, atol=1e-12)
    q_all = np.random.default_rng(2).standard_normal((2, 24, H * hd))
    oc, lc = O.context_all(q_all, kc, vc, H, Hkv, hd, scale)
    orf, lrf = R.context_all(q_all, kc, vc, H, Hkv, hd, scale)
    assert np.allclose(oc, orf, rtol=1e-10, atol=1e-12) and np.allclose(lc, lrf, rtol=1e-12)
    q_sel = np.random.default_rng(4).standard_normal((int(rp[-1]), H * hd))
    got = O.salient_attention(q_sel, q_all, kc, vc, sel, rp, H, Hkv, hd, scale, q_first=10,
                              o_prev=oc, lse_prev=lc)
    ref = R.salient_attention(q_sel, q_all, kc, vc, sel, rp, H, Hkv, hd, scale, q_first=10,
                              o_prev=oc, lse_prev=lc)
    for g, r in zip(got, ref):
        assert np.allclose(g, r, rtol=1e-10, atol=1e-12)


def test_threads_do_not_change_results():
    h, w, kc, vc, y, sel, rp = _layer_inputs(seed=13)
    O.set_threads(1)
    try:
        one = O.selected_layer(h, w, sel, rp, kc, vc, y, 4, 2, 16, 1e-5, 0.25, store="bf16")
    finally:
        O.set_threads(0)
    many = O.selected_layer(h, w, sel, rp, kc, vc, y, 4, 2, 16, 1e-5, 0.25, store="bf16")
    for a, b in zip(one, many):
        assert np.array_equal(a, b)
