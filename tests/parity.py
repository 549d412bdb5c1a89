"""Helpers for comparing the HIP library's outputs with the CPU oracle."""
import numpy as np
import torch

import oracle as O

# per output tensor: max|gpu - ref| <= tol * max|ref| over the rows the call writes
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def host(t) -> np.ndarray:
    """Tensor (any device) -> float64 numpy; bf16 is decoded by the oracle's own decoder."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return O.decode_bf16(t.view(torch.uint16).numpy())
    return t.numpy().astype(np.float64)


def assert_close(got, ref, tol: float, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    print(f"  {what}: max|err| = {err:.3e}, max|ref| = {scale:.3e}, ratio = {err / max(scale, 1e-300):.2e}")
    assert err <= tol * scale, f"{what}: max|err| {err:.3e} > {tol} * max|ref| {scale:.3e}"


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    a = a.detach().cpu().contiguous()
    b = b.detach().cpu().contiguous()
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def random_selection(B: int, S: int, counts, seed: int):
    """Ascending flat ids with counts[b] positions drawn in sequence b; returns (sel, row_ptr)."""
    rng = np.random.default_rng(seed)
    sel, rp = [], [0]
    for b in range(B):
        c = counts[b] if b < len(counts) else counts[-1]
        pos = np.sort(rng.choice(S, size=c, replace=False))
        sel.extend(b * S + int(p) for p in pos)
        rp.append(len(sel))
    return np.asarray(sel, dtype=np.int32), np.asarray(rp, dtype=np.int32)


def to_dev(x, dtype=None, device="cuda"):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(x)
    if dtype is not None:
        x = x.to(dtype)
    return x.to(device).contiguous()
