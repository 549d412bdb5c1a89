"""The allocation-free commit (dllm_commit_noalloc, static device scratch) against dllm_commit
(caller workspace), through the C ABI: identical token ids, blocks, committed lists and flags over
two calls in a row, the second with a smaller batch and block, each followed by more commit steps
on the same state."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def logits_with_spikes(B, S, V, seed):
    """N(0, 3^2) logits; a quarter of the rows get one logit raised by 30 (confidence ~1)."""
    z = synth.normal((B, S, V), 3.0, seed, torch.float32, "cuda")
    rng = np.random.default_rng(seed)
    rows = np.argwhere(rng.random((B, S)) < 0.25)
    if len(rows):
        z[torch.from_numpy(rows[:, 0]).cuda(), torch.from_numpy(rows[:, 1]).cuda(),
          torch.from_numpy(rng.integers(0, V, len(rows))).cuda()] += 30.0
    return z.to(torch.bfloat16)


def commit_both(lib, B, S, V, P, L, k_min, seed, steps=3):
    shape = lib.Shape(B=B, S=S, d=64, H=1, Hkv=1, hd=64, F=64, dtype="bf16", V=V)
    rng = np.random.default_rng(seed)
    tok = np.full((B, S), -1, np.int32)
    tok[:, :P] = rng.integers(0, V, (B, P))
    state = []
    for _ in range(2):   # [0]: dllm_commit with a workspace, [1]: dllm_commit_noalloc
        state.append(dict(
            tok=torch.from_numpy(tok.copy()).cuda(),
            blk=torch.zeros(B, dtype=torch.int32, device="cuda"),
            cidx=torch.full((B * L,), -5, dtype=torch.int32, device="cuda"),
            crp=torch.full((B + 1,), -5, dtype=torch.int32, device="cuda"),
            flags=torch.full((B, S), 7, dtype=torch.uint8, device="cuda")))
    ws = lib.workspace(lib.OP_COMMIT, shape, L)
    for step in range(steps):
        logits = logits_with_spikes(B, S, V, seed + 100 * step)
        a, b = state
        lib.dllm_commit(shape, logits, P, L, 0.9, k_min, a["tok"], a["blk"], a["cidx"], a["crp"],
                        a["flags"], ws)
        lib.dllm_commit_noalloc(shape, logits, P, L, 0.9, k_min, b["tok"], b["blk"], b["cidx"],
                                b["crp"], b["flags"])
        torch.cuda.synchronize()
        n = int(a["crp"][-1].item())
        print(f"B={B} L={L} step {step}: {n} committed", flush=True)
        for name in ("tok", "blk", "crp", "flags"):
            assert torch.equal(a[name], b[name]), (name, step)
        assert torch.equal(a["cidx"][:n], b["cidx"][:n]), step


def test_noalloc_commit_matches_commit(lib):
    commit_both(lib, B=6, S=700, V=2048, P=60, L=128, k_min=2, seed=41)
    commit_both(lib, B=2, S=90, V=512, P=10, L=16, k_min=1, seed=42)   # smaller, same scratch
