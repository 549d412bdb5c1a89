"""Pins of the CPU oracle against closed forms, brute force and invariants (no GPU).

Each test fixes something a plausible mistake in the oracle would break: a dropped sqrt(d), a
swapped norm, a missing residual, a transposed weight, a wrong KV-head map, a missing attention
scale, an off-by-one in compaction, a wrong tie-break or NaN policy.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# Every pin runs against both oracles: the C++ one the tests use (oracle.*) and the numpy one
# written first (oracle.numpy_ref), so each is pinned on its own.
_IMPLS = {"cpp": oracle, "numpy": oracle.numpy_ref}


@pytest.fixture(params=sorted(_IMPLS), autouse=True)
def _oracle_impl(request, monkeypatch):
    import sys
    monkeypatch.setattr(sys.modules[__name__], "O", _IMPLS[request.param])
    return request.param


# ------------------------------------------------------------------------------ saliency
@pytest.mark.parametrize("t", [0.3, -0.7, 2.5])
def test_l1n_and_l2r_closed_form_on_uniform_shift(t):
    d = 16
    y = np.ones((1, d))
    x = (1.0 + t) * np.ones((1, d))
    assert O.delta_variation(x, y, O.DELTA_L1N)[0] == pytest.approx(abs(t), rel=1e-14)
    assert O.delta_variation(x, y, O.DELTA_L2R)[0] == pytest.approx(abs(t), rel=1e-14)


def test_cosine_closed_forms():
    rng = np.random.default_rng(1)
    y = rng.standard_normal((3, 32))
    assert np.allclose(O.delta_variation(3.5 * y, y, O.DELTA_COS), 0.0, atol=1e-14)
    assert np.allclose(O.delta_variation(-y, y, O.DELTA_COS), 2.0, atol=1e-14)
    a = np.zeros((1, 4)); a[0, 0] = 2.0
    b = np.zeros((1, 4)); b[0, 1] = 5.0
    assert O.delta_variation(a, b, O.DELTA_COS)[0] == pytest.approx(1.0, abs=1e-15)


@pytest.mark.parametrize("V", [2, 7, 126464])
def test_confidence_closed_forms(V):
    # a float64 sum of V terms in sequence is within about V * 2^-53 of the exact sum (plus the
    # rounding of e^a and of ln(9 (V - 1))): the bound the pins below allow
    rel = max(1e-12, 4.0 * V * 2.0 ** -53)
    assert O.max_softmax_confidence(np.zeros(V)) == pytest.approx(1.0 / V, rel=rel)
    assert O.max_softmax_confidence(np.full(V, 1000.0)) == pytest.approx(1.0 / V, rel=rel)
    a = 2.0
    z = np.zeros(V); z[V // 2] = a
    assert O.max_softmax_confidence(z) == pytest.approx(math.exp(a) / (math.exp(a) + V - 1),
                                                        rel=rel)
    # one logit at ln(9 (V - 1)) puts exactly 0.9 of the mass on it
    z[V // 2] = math.log(9.0 * (V - 1))
    assert O.max_softmax_confidence(z) == pytest.approx(0.9, rel=rel)


def test_worked_example_golden():
    with open(os.path.join(GOLDEN, "saliency_worked_example.json")) as f:
        g = json.load(f)
    x = np.array([g["h_cur"]]); y = np.array([g["h_prev"]]); z = np.array([g["logits"]])
    e = g["expected"]
    assert O.delta_variation(x, y, O.DELTA_L1N)[0] == pytest.approx(e["variation_l1n"], rel=1e-14)
    assert O.delta_variation(x, y, O.DELTA_COS)[0] == pytest.approx(e["variation_cos"], rel=1e-13)
    assert O.delta_variation(x, y, O.DELTA_L2R)[0] == pytest.approx(e["variation_l2r"], rel=1e-14)
    assert O.max_softmax_confidence(z)[0] == pytest.approx(e["confidence"], rel=1e-14)
    score, conf, delta = O.saliency(x, y, z, g["alpha"], O.DELTA_L1N)
    assert score.dtype == np.float32
    assert float(score[0]) == np.float32(e["score_alpha_0.5"])
    # alpha = 0 keeps only the variation, alpha = 1 only the confidence
    assert float(O.saliency(x, y, None, 0.0)[0][0]) == np.float32(e["variation_l1n"])
    assert float(O.saliency(None, None, z, 1.0)[0][0]) == np.float32(e["confidence"])


@pytest.mark.parametrize("sigma", [0.5, 1e-3])
def test_statistical_l1n_of_generator(sigma):
    """E[L1N] = sigma sqrt(2/pi) for h_prev ~ N(0,1)^d and a N(0, sigma^2) perturbation."""
    B, S, d = 1, 64, 4096
    h_prev, h_cur, large = synth.perturbed_pair(B, S, d, S, seed=7, dtype=torch.float32,
                                                std_large=sigma)
    v = O.delta_variation(h_cur.double().numpy(), h_prev.double().numpy(), O.DELTA_L1N)
    assert float(v.mean()) == pytest.approx(sigma * math.sqrt(2 / math.pi), rel=0.01)
    c = O.delta_variation(h_cur.double().numpy(), h_prev.double().numpy(), O.DELTA_COS)
    if sigma == 0.5:
        assert float(c.mean()) == pytest.approx(1 - (1 + sigma ** 2) ** -0.5, rel=0.03)


# ------------------------------------------------------------------------------ selection
def _check_topk(score, force, k, sel, row_ptr):
    B, S = score.shape
    assert row_ptr[0] == 0 and len(row_ptr) == B + 1
    for b in range(B):
        ids = sel[row_ptr[b]:row_ptr[b + 1]]
        assert np.all(np.diff(ids) > 0), "ascending, no duplicates"
        pos = set(int(i) - b * S for i in ids)
        assert all(0 <= p < S for p in pos)
        fl = [int(force[b, s]) if force is not None else 0 for s in range(S)]
        forced = {s for s in range(S) if fl[s] & 1}
        excluded = {s for s in range(S) if fl[s] & 2 and not fl[s] & 1}
        cand = [s for s in range(S) if s not in forced and s not in excluded]
        assert forced <= pos and not (excluded & pos)
        chosen = pos - forced
        assert len(chosen) == min(k, len(cand))

        def better(s, u):  # s strictly ahead of u in the top-k order
            a, c = float(score[b, s]), float(score[b, u])
            if math.isnan(a) or math.isnan(c):
                return (not math.isnan(a) and math.isnan(c)) or (
                    math.isnan(a) and math.isnan(c) and s < u)
            return a > c or (a == c and s < u)

        for s in chosen:
            for u in cand:
                if u not in chosen:
                    assert better(s, u), (b, s, u, score[b, s], score[b, u])


@pytest.mark.parametrize("kind", ["mixed", "equal", "ties", "random"])
@pytest.mark.parametrize("k", [0, 1, 5, 17, 40, 64])
def test_topk_is_the_best_k_by_pairwise_order(kind, k):
    score = synth.adversarial_scores(3, 40, seed=11 + k, kind=kind).numpy()
    force = np.zeros((3, 40), dtype=bool)
    force[1, [0, 7, 39]] = True
    force[2, :] = True
    sel, row_ptr = O.select_compact(score, force, O.SEL_TOPK, k=k)
    _check_topk(score, force, k, sel, row_ptr)


@pytest.mark.parametrize("kind", ["mixed", "equal", "ties", "random"])
@pytest.mark.parametrize("k", [0, 1, 5, 17, 40])
def test_topk_with_excluded_positions(kind, k):
    """Flag bit 1 takes a position out of the candidates (a response-only step's prompt),
    bit 0 (forced) wins over it, other bits are ignored."""
    score = synth.adversarial_scores(4, 40, seed=31 + k, kind=kind).numpy()
    flags = np.zeros((4, 40), dtype=np.uint8)
    flags[0, :20] = 2                 # a 20-token prompt
    flags[1, 10:30] = 2
    flags[1, [3, 12]] = 3             # forced wins
    flags[2, :] = 6                   # every position excluded (bit 2 ignored)
    flags[3, ::3] = 4                 # ignored bit: still candidates
    flags[3, 1] = 5                   # forced
    sel, row_ptr = O.select_compact(score, flags, O.SEL_TOPK, k=k)
    _check_topk(score, flags, k, sel, row_ptr)
    assert row_ptr[3] == row_ptr[2]   # nothing from the fully excluded sequence


def test_threshold_with_excluded_positions():
    score = np.array([[0.9, 0.8, 0.1, 0.7, 0.95, 0.0]], dtype=np.float32)
    flags = np.array([[2, 3, 2, 0, 0, 1]], dtype=np.uint8)
    sel, rp = O.select_compact(score, flags, O.SEL_THRESHOLD, tau=0.5)
    assert list(sel) == [1, 3, 4, 5] and list(rp) == [0, 4]


def test_topk_signed_zero_and_nan_ties():
    score = np.array([[-0.0, 0.0, np.nan, -np.inf, np.nan]], dtype=np.float32)
    sel, rp = O.select_compact(score, None, O.SEL_TOPK, k=1)
    assert list(sel) == [0]          # -0 == +0, lower index wins
    sel, rp = O.select_compact(score, None, O.SEL_TOPK, k=3)
    assert list(sel) == [0, 1, 3]    # -inf ranks above NaN
    sel, rp = O.select_compact(score, None, O.SEL_TOPK, k=4)
    assert list(sel) == [0, 1, 2, 3]  # first NaN by position


def test_threshold_rule():
    score = np.array([[0.5, 0.2, np.nan, 0.2000001, np.inf, -np.inf],
                      [0.1, 0.3, 0.3, 0.0, -0.0, 1.0]], dtype=np.float32)
    force = np.zeros_like(score, dtype=bool)
    force[1, 0] = True
    sel, rp = O.select_compact(score, force, O.SEL_THRESHOLD, tau=0.2)
    assert list(sel) == [0, 3, 4, 6 + 0, 6 + 1, 6 + 2, 6 + 5]   # strict '>', NaN never
    assert list(rp) == [0, 3, 7]
    sel, rp = O.select_compact(score, force, O.SEL_THRESHOLD, tau=float("inf"))
    assert list(sel) == [6] and list(rp) == [0, 0, 1]
    sel, rp = O.select_compact(score, None, O.SEL_THRESHOLD, tau=-float("inf"))
    assert list(rp) == [0, 4, 10]     # everything except NaN and -inf


# ------------------------------------------------------------------------------ QKV projection
def test_rms_norm_closed_form():
    g = np.arange(1.0, 9.0)          # the gain multiplies each component
    for c in (0.01, -3.0, 7.5):
        for eps in (1e-5, 0.0, 0.25):
            out = O.rms_norm(np.full((1, 8), c), g, eps)
            want = g * math.copysign(1.0, c) / math.sqrt(1.0 + eps / c ** 2)
            assert np.allclose(out, want, rtol=1e-14)


def test_qkv_order_and_scatter_slots():
    """W_qkv = [I; 2I; 3I] with H = Hkv = 1, hd = d: q = xn, k = 2 xn, v = 3 xn at (b, 0, s)."""
    B, S, d, eps = 2, 5, 8, 1e-5
    c = -2.0
    h_in = np.random.default_rng(0).standard_normal((B, S, d))
    h_in[1, 3] = c
    w = np.concatenate([np.eye(d), 2 * np.eye(d), 3 * np.eye(d)])
    kc = np.random.default_rng(1).standard_normal((B, 1, S, d))
    vc = np.random.default_rng(2).standard_normal((B, 1, S, d))
    sel = np.array([1 * S + 3], dtype=np.int32)
    rp = np.array([0, 0, 1], dtype=np.int32)
    g = np.linspace(0.5, 2.0, d)
    q, k2, v2 = O.gather_qkv_scatter_kv(h_in, g, w, sel, rp, kc, vc, 1, 1, d, eps)
    n = g * math.copysign(1.0, c) / math.sqrt(1.0 + eps / c ** 2)
    assert np.allclose(q, n, rtol=1e-14)
    assert np.allclose(k2[1, 0, 3], 2 * n, rtol=1e-14)
    assert np.allclose(v2[1, 0, 3], 3 * n, rtol=1e-14)
    untouched = np.ones((B, 1, S), dtype=bool); untouched[1, 0, 3] = False
    assert np.array_equal(k2[untouched], kc[untouched])
    assert np.array_equal(v2[untouched], vc[untouched])


def test_qkv_kv_head_rows():
    """Key rows for head hk are rows H*hd + hk*hd .. of W_qkv and land in cache[b, hk, s]."""
    B, S, d, H, Hkv, hd = 1, 3, 4, 4, 2, 2
    nq, nkv = H * hd, Hkv * hd
    w = np.zeros((nq + 2 * nkv, d))
    for r in range(nq + 2 * nkv):
        w[r, 0] = r + 1.0           # output r = (r + 1) * xn[0]
    h_in = np.ones((B, S, d))       # xn = 1/sqrt(1 + eps) everywhere
    eps = 1e-5
    n = 1.0 / math.sqrt(1.0 + eps)
    sel = np.array([2], dtype=np.int32); rp = np.array([0, 1], dtype=np.int32)
    kc = np.zeros((B, Hkv, S, hd)); vc = np.zeros((B, Hkv, S, hd))
    q, k2, v2 = O.gather_qkv_scatter_kv(h_in, np.ones(d), w, sel, rp, kc, vc, H, Hkv, hd, eps)
    assert np.allclose(q[0], (np.arange(nq) + 1) * n)
    for hk in range(Hkv):
        assert np.allclose(k2[0, hk, 2], (nq + hk * hd + np.arange(hd) + 1) * n)
        assert np.allclose(v2[0, hk, 2], (nq + nkv + hk * hd + np.arange(hd) + 1) * n)


# ------------------------------------------------------------------------------ attention
def _attn_case(B, S, H, Hkv, hd, M_rows, seed=0):
    rng = np.random.default_rng(seed)
    kc = rng.standard_normal((B, Hkv, S, hd))
    vc = rng.standard_normal((B, Hkv, S, hd))
    sel = np.array(M_rows, dtype=np.int32)
    rp = [0] + [int(np.sum(sel // S <= b)) for b in range(B)]
    q = rng.standard_normal((len(sel), H * hd))
    return q, kc, vc, sel, np.array(rp, dtype=np.int32)


def test_attention_brute_force_python_loops():
    B, S, H, Hkv, hd = 2, 5, 4, 2, 3
    q, kc, vc, sel, rp = _attn_case(B, S, H, Hkv, hd, [1, 4, 5, 9])
    scale = 0.37
    o = O.partial_attn(q, kc, vc, sel, rp, H, Hkv, hd, scale)
    G = H // Hkv
    for r, flat in enumerate(sel):
        b = int(flat) // S
        for h in range(H):
            hk = h // G
            logit = [scale * sum(q[r, h * hd + e] * kc[b, hk, t, e] for e in range(hd))
                     for t in range(S)]
            mx = max(logit)
            w = [math.exp(x - mx) for x in logit]
            tot = sum(w)
            for e in range(hd):
                want = sum(w[t] * vc[b, hk, t, e] for t in range(S)) / tot
                assert o[r, h * hd + e] == pytest.approx(want, rel=1e-12, abs=1e-14)


def test_attention_two_key_closed_form():
    """scale * q.k0 = ln 3, q.k1 = 0 -> weights 3/4, 1/4."""
    hd = 4
    scale = 1.0 / math.sqrt(hd)
    kc = np.zeros((1, 1, 2, hd)); vc = np.zeros((1, 1, 2, hd))
    kc[0, 0, 0, 0] = 2.0 * math.log(3.0)
    vc[0, 0, 0, 0] = 4.0
    vc[0, 0, 1, 1] = 8.0
    q = np.array([[1.0, 0.0, 0.0, 0.0]])
    o = O.partial_attn(q, kc, vc, np.array([1], np.int32), np.array([0, 1], np.int32),
                       1, 1, hd, scale)
    assert np.allclose(o[0], [3.0, 2.0, 0.0, 0.0], rtol=1e-14)


def test_attention_special_cases():
    B, S, H, Hkv, hd = 1, 6, 2, 1, 4
    q, kc, vc, sel, rp = _attn_case(B, S, H, Hkv, hd, [0, 2, 5])
    same_k = np.broadcast_to(kc[:, :, :1], kc.shape).copy()
    o = O.partial_attn(q, same_k, vc, sel, rp, H, Hkv, hd, 0.5)
    assert np.allclose(o.reshape(3, H, hd), vc[0, 0].mean(axis=0), rtol=1e-13)
    row = np.array([1.0, -2.0, 0.5, 3.0])
    const_v = np.broadcast_to(row, vc.shape).copy()
    o = O.partial_attn(q, kc, const_v, sel, rp, H, Hkv, hd, 0.5)
    assert np.allclose(o.reshape(3, H, hd), row, rtol=1e-13)
    o = O.partial_attn(q[:1], kc[:, :, :1], vc[:, :, :1], np.array([0], np.int32),
                       np.array([0, 1], np.int32), H, Hkv, hd, 0.5)
    assert np.allclose(o.reshape(H, hd), vc[0, 0, 0], rtol=1e-14)


def test_attention_grouped_heads_are_blocked():
    """H = 4, Hkv = 2: heads 0,1 read kv head 0 and heads 2,3 read kv head 1."""
    B, S, H, Hkv, hd = 1, 3, 4, 2, 2
    q, kc, vc, sel, rp = _attn_case(B, S, H, Hkv, hd, [1])
    vc[0, 0] = [5.0, 6.0]
    vc[0, 1] = [-1.0, 2.0]
    o = O.partial_attn(q, kc, vc, sel, rp, H, Hkv, hd, 1.0).reshape(H, hd)
    assert np.allclose(o[0], [5, 6]) and np.allclose(o[1], [5, 6])
    assert np.allclose(o[2], [-1, 2]) and np.allclose(o[3], [-1, 2])


# --------------------------------------------------- context of every token (DyLLM §2.B paths)
def test_context_all_brute_force_python_loops():
    B, S, H, Hkv, hd = 2, 4, 4, 2, 3
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, S, H * hd))
    kc = rng.standard_normal((B, Hkv, S, hd))
    vc = rng.standard_normal((B, Hkv, S, hd))
    scale = 0.61
    o, lse = O.context_all(q, kc, vc, H, Hkv, hd, scale)
    G = H // Hkv
    for b in range(B):
        for s_ in range(S):
            for h in range(H):
                hk = h // G
                logit = [scale * sum(q[b, s_, h * hd + e] * kc[b, hk, t, e] for e in range(hd))
                         for t in range(S)]
                w = [math.exp(x) for x in logit]
                tot = sum(w)
                assert lse[b, s_, h] == pytest.approx(math.log(tot), rel=1e-12, abs=1e-13)
                for e in range(hd):
                    want = sum(w[t] * vc[b, hk, t, e] for t in range(S)) / tot
                    assert o[b, s_, h * hd + e] == pytest.approx(want, rel=1e-12, abs=1e-14)


def test_context_all_special_cases():
    B, S, H, Hkv, hd = 1, 5, 2, 1, 4
    rng = np.random.default_rng(6)
    q = rng.standard_normal((B, S, H * hd))
    kc = rng.standard_normal((B, Hkv, S, hd))
    vc = rng.standard_normal((B, Hkv, S, hd))
    # identical keys: uniform weights, lse = scale q.k + ln S
    same_k = np.broadcast_to(kc[:, :, :1], kc.shape).copy()
    o, lse = O.context_all(q, same_k, vc, H, Hkv, hd, 0.5)
    assert np.allclose(o.reshape(S, H, hd), vc[0, 0].mean(axis=0), rtol=1e-13)
    qk = q.reshape(S, H, hd) @ kc[0, 0, 0]
    assert np.allclose(lse[0], 0.5 * qk + math.log(S), rtol=1e-13)
    # one key: o = v0, lse = scale q.k0
    o, lse = O.context_all(q[:, :1], kc[:, :, :1], vc[:, :, :1], H, Hkv, hd, 0.5)
    assert np.allclose(o.reshape(H, hd), vc[0, 0, 0], rtol=1e-14)
    assert np.allclose(lse[0, 0], 0.5 * (q[0, 0].reshape(H, hd) @ kc[0, 0, 0]), rtol=1e-14)


def test_gather_kv_rows_copies_the_selected_positions():
    B, Hkv, S, hd = 2, 3, 5, 2
    kc = np.arange(B * Hkv * S * hd, dtype=np.float64).reshape(B, Hkv, S, hd)
    vc = -kc
    sel = np.array([1, 4, 7], np.int32)   # (0,1), (0,4), (1,2)
    rp = np.array([0, 2, 3], np.int32)
    kr, vr = O.gather_kv_rows(kc, vc, sel, rp)
    for r, (b, s_) in enumerate([(0, 1), (0, 4), (1, 2)]):
        for hk in range(Hkv):
            assert list(kr[r, hk]) == list(kc[b, hk, s_])
            assert list(vr[r, hk]) == list(vc[b, hk, s_])


def test_salient_attention_rows_use_the_right_query():
    """Selected rows attend with the new query, the rest with the cached one (compared with the
    separately written partial_attn, itself pinned by brute force above)."""
    B, S, H, Hkv, hd = 2, 6, 4, 2, 3
    rng = np.random.default_rng(7)
    q_all = rng.standard_normal((B, S, H * hd))
    kc = rng.standard_normal((B, Hkv, S, hd))
    vc = rng.standard_normal((B, Hkv, S, hd))
    sel = np.array([2, 3, 7], np.int32)
    rp = np.array([0, 2, 3], np.int32)
    q_sel = rng.standard_normal((3, H * hd))
    q_new, o, _ = O.salient_attention(q_sel, q_all, kc, vc, sel, rp, H, Hkv, hd, 0.4)
    want_sel = O.partial_attn(q_sel, kc, vc, sel, rp, H, Hkv, hd, 0.4)
    for r, flat in enumerate(sel):
        assert np.allclose(o[flat // S, flat % S], want_sel[r], rtol=1e-13)
        assert np.array_equal(q_new[flat // S, flat % S], q_sel[r])
    rest = np.array([i for i in range(B * S) if i not in set(sel.tolist())], np.int32)
    rp_rest = np.array([0, int(np.sum(rest < S)), len(rest)], np.int32)
    q_rest = q_all.reshape(B * S, -1)[rest]
    want_rest = O.partial_attn(q_rest, kc, vc, rest, rp_rest, H, Hkv, hd, 0.4)
    for r, flat in enumerate(rest):
        assert np.allclose(o[flat // S, flat % S], want_rest[r], rtol=1e-13)
        assert np.array_equal(q_new[flat // S, flat % S], q_all[flat // S, flat % S])


def test_response_only_rows_before_q_first():
    """q_first: unselected positions before it keep the given previous context and log-sum-exp,
    selected ones there are exact, positions from q_first on are as without it."""
    B, S, H, Hkv, hd, P = 2, 7, 2, 1, 3, 4
    rng = np.random.default_rng(8)
    q_all = rng.standard_normal((B, S, H * hd))
    kc = rng.standard_normal((B, Hkv, S, hd))
    vc = rng.standard_normal((B, Hkv, S, hd))
    o_prev = rng.standard_normal((B, S, H * hd))
    lse_prev = rng.standard_normal((B, S, H))
    sel = np.array([1, 5, 7 + 6], np.int32)          # a prompt position of sequence 0
    rp = np.array([0, 2, 3], np.int32)
    q_sel = rng.standard_normal((3, H * hd))
    q0, o0, l0 = O.salient_attention(q_sel, q_all, kc, vc, sel, rp, H, Hkv, hd, 0.3)
    q1, o1, l1 = O.salient_attention(q_sel, q_all, kc, vc, sel, rp, H, Hkv, hd, 0.3, q_first=P,
                                     o_prev=o_prev, lse_prev=lse_prev)
    assert np.array_equal(q0, q1)
    for b in range(B):
        for s in range(S):
            if s < P and b * S + s not in (1, 5, 13):
                assert np.array_equal(o1[b, s], o_prev[b, s])
                assert np.array_equal(l1[b, s], lse_prev[b, s])
            else:
                assert np.array_equal(o1[b, s], o0[b, s]) and np.array_equal(l1[b, s], l0[b, s])
    # q_first = S and nothing selected: the previous contexts come back unchanged
    _, o2, l2 = O.salient_attention(q_sel[:0], q_all, kc, vc, sel[:0], np.zeros(3, np.int32), H,
                                    Hkv, hd, 0.3, q_first=S, o_prev=o_prev, lse_prev=lse_prev)
    assert np.array_equal(o2, o_prev) and np.array_equal(l2, lse_prev)


def test_stable_rows_equal_reused_weights_plus_changed_contributions():
    """DyLLM §2.B, non-salient path, done incrementally in this test: keep the previous step's
    softmax numerator and denominator of a stable token, take out the old rows of the changed
    keys, put in the new ones. The result must be the oracle's context of the reused query
    against the updated cache."""
    S, hd, scale = 7, 4, 0.45
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, S, hd))
    k_old = rng.standard_normal((1, 1, S, hd))
    v_old = rng.standard_normal((1, 1, S, hd))
    changed = [1, 4, 5]
    k_new, v_new = k_old.copy(), v_old.copy()
    k_new[0, 0, changed] = rng.standard_normal((3, hd))
    v_new[0, 0, changed] = rng.standard_normal((3, hd))
    o_new, lse_new = O.context_all(q, k_new, v_new, 1, 1, hd, scale)
    for i in range(S):
        w = [math.exp(scale * float(q[0, i] @ k_old[0, 0, t])) for t in range(S)]
        den = sum(w)
        num = [sum(w[t] * v_old[0, 0, t, e] for t in range(S)) for e in range(hd)]
        for t in changed:
            w_old = math.exp(scale * float(q[0, i] @ k_old[0, 0, t]))
            w_new = math.exp(scale * float(q[0, i] @ k_new[0, 0, t]))
            den += w_new - w_old
            for e in range(hd):
                num[e] += w_new * v_new[0, 0, t, e] - w_old * v_old[0, 0, t, e]
        assert lse_new[0, i, 0] == pytest.approx(math.log(den), rel=1e-12)
        for e in range(hd):
            assert o_new[0, i, e] == pytest.approx(num[e] / den, rel=1e-11, abs=1e-13)


# ------------------------------------------------------------------------------ FFN
def test_ffn_zero_projections_copy_rows_exactly():
    B, S, d, F = 2, 4, 8, 16
    rng = np.random.default_rng(3)
    h_in = rng.standard_normal((B, S, d)); h_out = rng.standard_normal((B, S, d))
    sel = np.array([1, 6], np.int32); rp = np.array([0, 1, 2], np.int32)
    o_sel = rng.standard_normal((2, d))
    out = O.gather_ffn_scatter(h_in, o_sel, np.zeros((d, d)), np.ones(d),
                               rng.standard_normal((F, d)), rng.standard_normal((F, d)),
                               np.zeros((d, F)), sel, rp, h_out, 1e-5)
    assert np.array_equal(out[0, 1], h_in[0, 1]) and np.array_equal(out[1, 2], h_in[1, 2])
    keep = np.ones((B, S), bool); keep[0, 1] = keep[1, 2] = False
    assert np.array_equal(out[keep], h_out[keep])


def test_ffn_closed_form_gate_up_down_routing():
    """x = c*1, W_o = 0: y = x + silu(a n) (beta n) e_2 with n = RMSNorm(c*1) component."""
    d, F, eps, c, beta = 4, 2, 1e-5, 1.5, 0.8
    a = math.log(3.0) * math.sqrt(1 + eps / c ** 2)
    h_in = np.full((1, 1, d), c)
    w_gate = np.zeros((F, d)); w_gate[0, 0] = a
    w_up = np.zeros((F, d)); w_up[0, 1] = beta
    w_down = np.zeros((d, F)); w_down[2, 0] = 1.0
    out = O.gather_ffn_scatter(h_in, np.zeros((1, d)), np.zeros((d, d)), np.ones(d), w_gate, w_up,
                               w_down, np.array([0], np.int32), np.array([0, 1], np.int32),
                               np.zeros((1, 1, d)), eps)
    n = 1.0 / math.sqrt(1.0 + eps / c ** 2)
    g = a * n                                           # = ln 3 -> silu = 0.75 ln 3
    want = np.full(d, c); want[2] += 0.75 * math.log(3.0) * beta * n
    assert g == pytest.approx(math.log(3.0), rel=1e-14)
    assert np.allclose(out[0, 0], want, rtol=1e-14)


def test_ffn_attention_residual_through_w_o():
    """h = x + o W_o^T with a non-symmetric W_o (W_o[0, 2] = 3 routes o[2] into h[0])."""
    d, F = 4, 3
    h_in = np.zeros((1, 2, d)); h_in[0, 1] = [1.0, 2.0, 3.0, 4.0]
    o_sel = np.array([[0.5, 0.0, -1.0, 0.0]])
    w_o = np.zeros((d, d)); w_o[0, 2] = 3.0; w_o[1, 0] = 2.0
    out = O.gather_ffn_scatter(h_in, o_sel, w_o, np.ones(d), np.ones((F, d)), np.ones((F, d)),
                               np.zeros((d, F)), np.array([1], np.int32),
                               np.array([0, 1], np.int32), np.zeros((1, 2, d)), 1e-5)
    assert np.allclose(out[0, 1], [1.0 - 3.0, 2.0 + 1.0, 3.0, 4.0], rtol=1e-15)


def test_ffn_norm_gain_applies():
    """g_ffn scales RMSNorm(h) per component: with W_gate picking component 1 and g_ffn[1] = 0
    the gate is silu(0) = 0 and y = h exactly."""
    d, F = 4, 1
    h_in = np.full((1, 1, d), 2.0)
    g = np.ones(d); g[1] = 0.0
    w_gate = np.zeros((F, d)); w_gate[0, 1] = 5.0
    w_up = np.ones((F, d))
    w_down = np.ones((d, F))
    out = O.gather_ffn_scatter(h_in, np.zeros((1, d)), np.zeros((d, d)), g, w_gate, w_up,
                               w_down, np.array([0], np.int32), np.array([0, 1], np.int32),
                               np.zeros((1, 1, d)), 1e-5)
    assert np.array_equal(out[0, 0], h_in[0, 0])
    g[1] = 1.0
    out = O.gather_ffn_scatter(h_in, np.zeros((1, d)), np.zeros((d, d)), g, w_gate, w_up,
                               w_down, np.array([0], np.int32), np.array([0, 1], np.int32),
                               np.zeros((1, 1, d)), 1e-5)
    assert not np.array_equal(out[0, 0], h_in[0, 0])


def test_silu_closed_form():
    assert O.silu(0.0) == 0.0
    assert O.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    assert O.silu(-math.log(3.0)) == pytest.approx(-0.25 * math.log(3.0), rel=1e-15)


# ------------------------------------------------------------------------------ layer invariants
def _tiny_layer(B=2, S=6, d=8, H=2, Hkv=1, hd=4, F=16, seed=5):
    w = {k: v.double().numpy() for k, v in synth.layer_weights(d, H, Hkv, hd, F, seed=seed,
                                                               dtype=torch.float32,
                                                               std=0.3).items()}
    h = synth.normal((B, S, d), 1.0, seed + 100, torch.float32).double().numpy()
    return w, h


@pytest.mark.parametrize("H,Hkv", [(2, 1), (2, 2), (4, 2)])
def test_select_all_equals_dense_layer(H, Hkv):
    B, S, d, hd, F, eps = 2, 6, 8, 4, 16, 1e-5
    w, h = _tiny_layer(B, S, d, H, Hkv, hd, F)
    scale = 1.0 / math.sqrt(hd)
    k_d, v_d, y_d = O.dense_layer(h, w, H, Hkv, hd, eps, scale)
    sel = np.arange(B * S, dtype=np.int32)
    rp = np.array([0, S, 2 * S], np.int32)
    junk = np.full((B, Hkv, S, hd), 1e3)
    q, o, k_s, v_s, y_s = O.selected_layer(h, w, sel, rp, junk, junk, np.zeros((B, S, d)),
                                           H, Hkv, hd, eps, scale)
    assert np.allclose(k_s, k_d, rtol=1e-12, atol=1e-13)
    assert np.allclose(v_s, v_d, rtol=1e-12, atol=1e-13)
    assert np.allclose(y_s, y_d, rtol=1e-12, atol=1e-13)


def test_select_none_leaves_caches_unchanged():
    B, S, d, H, Hkv, hd, F, eps = 2, 6, 8, 2, 1, 4, 16, 1e-5
    w, h = _tiny_layer(B, S, d, H, Hkv, hd, F)
    rng = np.random.default_rng(9)
    kc = rng.standard_normal((B, Hkv, S, hd)); vc = rng.standard_normal((B, Hkv, S, hd))
    ho = rng.standard_normal((B, S, d))
    q, o, k2, v2, y2 = O.selected_layer(h, w, np.zeros(0, np.int32), np.zeros(B + 1, np.int32),
                                        kc, vc, ho, H, Hkv, hd, eps, 0.5)
    assert q.shape[0] == 0 and o.shape[0] == 0
    assert np.array_equal(k2, kc) and np.array_equal(v2, vc) and np.array_equal(y2, ho)


def test_rows_are_independent_in_projection_calls():
    B, S, d, H, Hkv, hd, F, eps = 1, 6, 8, 2, 1, 4, 16, 1e-5
    w, h = _tiny_layer(B, S, d, H, Hkv, hd, F)
    kc = np.zeros((B, Hkv, S, hd)); vc = np.zeros((B, Hkv, S, hd))
    q_all, k_all, _ = O.gather_qkv_scatter_kv(h, w["g_attn"], w["w_qkv"],
                                              np.array([0, 2, 3], np.int32),
                                              np.array([0, 3], np.int32), kc, vc, H, Hkv, hd, eps)
    q_one, k_one, _ = O.gather_qkv_scatter_kv(h, w["g_attn"], w["w_qkv"],
                                              np.array([2], np.int32), np.array([0, 1], np.int32),
                                              kc, vc, H, Hkv, hd, eps)
    # equal up to the library matmul's summation order, which may depend on the row count
    assert np.allclose(q_all[1], q_one[0], rtol=1e-13, atol=1e-15)
    assert np.allclose(k_all[0, :, 2], k_one[0, :, 2], rtol=1e-13, atol=1e-15)


def test_kv_cache_sizing_matches_quoted_memory():
    """ES-dLLM (German page) §4 quotes about 644 MB of cache per sample for LLaDA-8B at 1024
    prompt + 256 generated tokens. A bf16 [Hkv=32, S, hd=128] K and V cache per layer over 32
    layers and 1280 positions is 2*32*1280*4096*2 bytes = 640 MiB (671 MB): the same size
    within 5%, which supports the per-layer [B, Hkv, S, hd] bf16 layout at that shape."""
    bytes_kv = 2 * 32 * 1280 * 32 * 128 * 2
    assert abs(bytes_kv / 644e6 - 1.0) < 0.05


# ---- decode loop: commit rule and block advance (SlowFast German page, "Der SlowFast-Algorithmus"
# item 2: threshold commit with a top-k fallback), worked by hand on a 6-token vocabulary. One
# logit a above five zeros gives the confidence e^a / (e^a + 5): a = 5 -> 0.967, 2 -> 0.596,
# 1 -> 0.352 (tau = 0.9 needs a > ln 45 = 3.81).
def _spike_logits(B, S, V, spikes):
    z = np.zeros((B, S, V))
    for (b, s), (a, idx) in spikes.items():
        z[b, s, idx] = a
    return z


def test_confidence_argmax_closed_form_and_ties():
    c, a = O.confidence_argmax(np.array([0.0, 0.0, 5.0, 0.0, 0.0, 0.0]))
    assert a == 2 and abs(c - math.exp(5) / (math.exp(5) + 5)) < 1e-15
    c, a = O.confidence_argmax(np.array([1.0, 3.0, 0.0, 3.0]))
    assert a == 1 and abs(c - math.exp(3) / (2 * math.exp(3) + math.exp(1) + 1)) < 1e-15


def test_commit_threshold_fallback_and_block_advance():
    B, S, V, P, L = 2, 10, 6, 2, 4            # blocks [2, 6) and [6, 10)
    tok = np.full((B, S), -1)
    tok[:, :P] = [[1, 2], [4, 0]]
    tok[1, 2:7] = [1, 1, 1, 1, 2]             # sequence 1: block 0 done, block 1 at position 6
    blk = np.array([0, 1])
    z = _spike_logits(B, S, V, {(0, 2): (5, 3), (0, 3): (2, 1), (0, 4): (5, 0), (0, 5): (1, 4),
                                (1, 7): (1, 5), (1, 8): (2, 2), (1, 9): (1, 1)})
    # two above the threshold in sequence 0 (k_min 1): both; none in sequence 1: the best one
    t1, b1, sel, rp, fl = O.commit_step(z, tok, blk, P, L, 0.9, 1)
    assert list(sel) == [2, 4, 10 + 8] and list(rp) == [0, 2, 3]
    assert t1[0, 2] == 3 and t1[0, 4] == 0 and t1[1, 8] == 2 and t1[0, 3] == -1
    assert list(b1) == [0, 1]
    assert fl[0].tolist() == [0, 0, 1, 1, 1, 1, 0, 0, 0, 0] and fl[1].tolist() == [0] * 6 + [1] * 4
    # k_min 2: sequence 0 completes block 0 (3 then 5 by confidence) and moves to block 1;
    # sequence 1 takes 7 and 9 (equal confidence: both, as only two are left) and is done
    t2, b2, sel, rp, fl = O.commit_step(z, t1, b1, P, L, 0.9, 2)
    assert list(sel) == [3, 5, 10 + 7, 10 + 9] and list(rp) == [0, 2, 4]
    assert t2[0, 3] == 1 and t2[0, 5] == 4 and t2[1, 7] == 5 and t2[1, 9] == 1
    assert list(b2) == [1, 2]
    assert fl[0].tolist() == [0] * 6 + [1] * 4 and not fl[1].any()
    # a done sequence commits nothing and stays done
    t3, b3, sel, rp, fl = O.commit_step(z, t2, b2, P, L, 0.9, 2)
    assert list(rp) == [0, 0, 0] or rp[2] == rp[1]
    assert b3[1] == 2 and np.array_equal(t3[1], t2[1])


def test_commit_ties_go_to_the_lower_position_and_ragged_last_block():
    B, S, V, P, L = 1, 9, 6, 2, 4             # blocks [2, 6), [6, 9)
    tok = np.full((B, S), -1)
    tok[0, :6] = [0, 0, 1, 1, 1, 1]
    z = _spike_logits(B, S, V, {(0, 6): (1, 2), (0, 7): (1, 3), (0, 8): (1, 4)})
    t, b, sel, rp, fl = O.commit_step(z, tok, np.array([1]), P, L, 0.9, 2)
    assert list(sel) == [6, 7] and t[0, 6] == 2 and t[0, 7] == 3 and b[0] == 1
    assert fl[0].tolist() == [0] * 6 + [1] * 3
    t, b, sel, rp, fl = O.commit_step(z, t, b, P, L, 0.9, 2)
    assert list(sel) == [8] and b[0] == 2 and not fl.any()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_commit_invariants_on_random_logits(seed):
    rng = np.random.default_rng(seed)
    B, S, V, P, L = 3, 40, 17, 8, 8
    tok = np.full((B, S), -1)
    tok[:, :P] = rng.integers(0, V, (B, P))
    blk = np.array([0, 2, 3])
    for b in range(B):
        tok[b, P:P + blk[b] * L] = rng.integers(0, V, blk[b] * L)
    z = rng.normal(0, 3, (B, S, V))
    z[rng.random((B, S)) < 0.2, 0] += 30      # some rows far above the threshold
    tok[1, P + 2 * L + 1] = 5                 # an already committed position inside a block
    for k_min in (1, 3):
        t, bl, sel, rp, fl = O.commit_step(z, tok, blk, P, L, 0.9, k_min)
        for b in range(B):
            lo, hi = P + blk[b] * L, min(S, P + (blk[b] + 1) * L)
            masked = [s for s in range(lo, hi) if tok[b, s] < 0]
            ids = [int(i) - b * S for i in sel[rp[b]:rp[b + 1]]]
            conf = {s: np.float32(O.confidence_argmax(z[b, s])[0]) for s in masked}
            above = [s for s in masked if conf[s] > np.float32(0.9)]
            assert set(ids) <= set(masked)
            assert len(ids) == max(len(above), min(k_min, len(masked)))
            for s in ids:
                assert t[b, s] == int(np.argmax(z[b, s]))
                for u in set(masked) - set(ids):
                    assert conf[s] > conf[u] or (conf[s] == conf[u] and s < u)
            others = np.ones(S, bool)
            others[ids] = False
            assert np.array_equal(t[b][others], tok[b][others])
            done = all(t[b, s] >= 0 for s in range(lo, hi))
            assert bl[b] == blk[b] + (1 if done else 0)


def test_embed_rows_copies_the_listed_rows():
    rng = np.random.default_rng(3)
    emb, mask = rng.standard_normal((7, 5)), rng.standard_normal(5)
    tok = np.array([[3, -1, 6, 0]])
    x = rng.standard_normal((1, 4, 5))
    y = O.embed_rows(emb, mask, tok, np.array([1, 2], np.int32), np.array([0, 2], np.int32), x)
    assert np.array_equal(y[0, 1], mask) and np.array_equal(y[0, 2], emb[6])
    assert np.array_equal(y[0, 0], x[0, 0]) and np.array_equal(y[0, 3], x[0, 3])


def test_saliency_with_earlier_confidence_equals_the_logits_path():
    """A second skip point reuses the previous step's confidence: the score from the stored
    confidence equals the score computed from the logits themselves."""
    rng = np.random.default_rng(5)
    h1, h0 = rng.standard_normal((2, 6, 16)), rng.standard_normal((2, 6, 16))
    z = rng.normal(0, 3, (2, 6, 40))
    s_a, conf, _ = O.saliency(h1, h0, z, 0.5)
    s_b, conf_b, _ = O.saliency(h1, h0, None, 0.5, conf=conf)
    assert np.array_equal(s_a, s_b) and np.array_equal(conf, conf_b)
    s_c, _, d = O.saliency(h1, h0, None, 0.0)
    assert np.array_equal(s_c, d.astype(np.float32))


def test_flags_from_rows_restrict_to_the_listed_rows():
    force = np.array([[3, 0, 1, 0], [0, 2, 0, 1]], np.uint8)
    sel = np.array([0, 1, 5, 7], np.int32)
    rp = np.array([0, 2, 4], np.int32)
    f = O.flags_from_rows(force, sel, rp, 2, 4)
    assert f.tolist() == [[1, 0, 2, 2], [2, 0, 2, 1]]
    assert O.flags_from_rows(None, sel, rp, 2, 4).tolist() == [[0, 0, 2, 2], [2, 0, 2, 0]]
