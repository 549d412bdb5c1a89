"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This module draws random tensors and nothing else: it holds none of the method's arithmetic
(no saliency, no selection, no normalisation, no projection). Every function takes an explicit
integer seed and returns the same values for the same seed on the same device, so a test can
hand identical bytes to the HIP library and to the oracle.

Workload shapes and value distributions follow the synthetic LLaDA-8B / Dream-7B stand-ins for the
pages' evaluation runs (trained weights and benchmark suites are not available):
  * linear weights ~ N(0, 0.02^2), norm gains = 1;
  * hidden states at step t-1 ~ N(0, 1);
  * step-t hidden = step-(t-1) hidden + a per-token perturbation: a chosen subset of tokens per
    sequence gets N(0, 0.5^2), every other token N(0, (1e-3)^2);
  * previous-step logits ~ N(0, 3^2) over the vocabulary.

Generation happens in float32 and is then rounded to the requested storage dtype by torch's
round-to-nearest-even conversion.
"""
from __future__ import annotations

import torch

__all__ = [
    "generator",
    "normal",
    "layer_weights",
    "perturbed_pair",
    "perturb",
    "logits",
    "large_positions",
    "adversarial_scores",
]


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def normal(shape, std: float, seed: int, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """N(0, std^2) samples of `shape`, drawn in float32 and stored as `dtype`."""
    g = generator(seed, device)
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def layer_weights(d: int, H: int, Hkv: int, hd: int, F: int, *, seed: int,
                  dtype=torch.bfloat16, device="cpu", std: float = 0.02) -> dict:
    """Random-init weights of one pre-norm transformer block, [out, in] row-major.

    w_qkv stacks the query rows (H*hd), then key rows (Hkv*hd), then value rows (Hkv*hd).
    """
    nq, nkv = H * hd, Hkv * hd
    return {
        "g_attn": torch.ones(d, dtype=dtype, device=device),
        "w_qkv": normal((nq + 2 * nkv, d), std, seed * 16 + 1, dtype, device),
        "w_o": normal((d, nq), std, seed * 16 + 2, dtype, device),
        "g_ffn": torch.ones(d, dtype=dtype, device=device),
        "w_gate": normal((F, d), std, seed * 16 + 3, dtype, device),
        "w_up": normal((F, d), std, seed * 16 + 4, dtype, device),
        "w_down": normal((d, F), std, seed * 16 + 5, dtype, device),
    }


def large_positions(B: int, S: int, n_large: int, *, seed: int, exclude=None,
                    device="cpu") -> torch.Tensor:
    """Bool mask [B, S] with exactly `n_large` True entries per row, drawn uniformly.

    Positions where `exclude` ([B, S] bool) is True are never drawn.
    """
    g = generator(seed, "cpu")
    mask = torch.zeros(B, S, dtype=torch.bool)
    for b in range(B):
        pool = torch.arange(S)
        if exclude is not None:
            pool = pool[~exclude[b].cpu()]
        pick = pool[torch.randperm(pool.numel(), generator=g)[:n_large]]
        mask[b, pick] = True
    return mask.to(device)


def perturb(h: torch.Tensor, large: torch.Tensor, *, seed: int, std_large: float = 0.5,
            std_small: float = 1e-3) -> torch.Tensor:
    """h + delta, delta ~ N(0, std_large^2) on tokens where `large` is True, else N(0, std_small^2).

    h: [B, S, d]; large: [B, S] bool. Returned in h's dtype.
    """
    B, S, d = h.shape
    z = normal((B, S, d), 1.0, seed, torch.float32, h.device)
    scale = torch.where(large.to(h.device), std_large, std_small).to(torch.float32)
    z.mul_(scale.unsqueeze(-1))
    z.add_(h.to(torch.float32))
    return z.to(h.dtype)


def perturbed_pair(B: int, S: int, d: int, n_large: int, *, seed: int, dtype=torch.bfloat16,
                   device="cpu", std_large: float = 0.5, std_small: float = 1e-3):
    """(h_prev, h_cur, large): h_prev ~ N(0,1) [B,S,d]; h_cur = h_prev + per-token perturbation."""
    h_prev = normal((B, S, d), 1.0, seed * 8 + 1, dtype, device)
    large = large_positions(B, S, n_large, seed=seed * 8 + 2, device=device)
    h_cur = perturb(h_prev, large, seed=seed * 8 + 3, std_large=std_large, std_small=std_small)
    return h_prev, h_cur, large


def logits(B: int, S: int, V: int, *, seed: int, std: float = 3.0, dtype=torch.bfloat16,
           device="cpu") -> torch.Tensor:
    """Previous-step logits ~ N(0, std^2), [B, S, V]."""
    return normal((B, S, V), std, seed, dtype, device)


def adversarial_scores(B: int, S: int, *, seed: int, kind: str = "mixed") -> torch.Tensor:
    """float32 score rows that stress a top-k / threshold selector.

    kinds: "mixed" (heavy ties, +-0, NaN, +-inf, denormals, random values), "equal" (all equal),
    "ties" (values from a 4-element set), "random" (plain N(0,1)).
    """
    g = generator(seed)
    if kind == "random":
        return torch.randn(B, S, generator=g)
    if kind == "equal":
        return torch.full((B, S), 0.25)
    if kind == "ties":
        vals = torch.tensor([-1.0, 0.0, 0.5, 2.0])
        return vals[torch.randint(0, 4, (B, S), generator=g)]
    special = torch.tensor([float("nan"), float("inf"), float("-inf"), 0.0, -0.0,
                            1.0e-45, -1.0e-45, 3.0e38, -3.0e38, 1.0, 1.0, 0.5, 0.5])
    base = torch.randn(B, S, generator=g)
    base = torch.round(base * 4) / 4  # coarse grid -> many exact ties
    pick = torch.rand(B, S, generator=g) < 0.3
    idx = torch.randint(0, special.numel(), (B, S), generator=g)
    return torch.where(pick, special[idx], base)
