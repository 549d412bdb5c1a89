"""Resume from a checkpoint: a step driver restored from `save_state` into a fresh driver (same
weights, same configuration) takes the next steps bit-identically to the driver that was never
interrupted, for the early-skip step with a second skip point, the layer-adaptive step with
response-only and prompt-injecting steps, and the block decoder (whose restored state is also
read by a HIP graph captured before the restore).
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
B, S, d, H, Hkv, hd, F, V, L = 2, 64, 256, 4, 2, 64, 512, 128, 4


def weights(seed):
    from token_skipping_partial_amd.step import LayerWeights
    return [LayerWeights.from_dict(synth.layer_weights(d, H, Hkv, hd, F, seed=seed + l,
                                                       dtype=BF16), "cuda") for l in range(L)]


def inputs(n, seed):
    x = [synth.normal((B, S, d), 1.0, seed, BF16)]
    for t in range(1, n):
        large = synth.large_positions(B, S, 12, seed=seed + 10 + t)
        x.append(synth.perturb(x[-1], large, seed=seed + 20 + t))
    return [t.cuda() for t in x]


def logits(seed):
    z = synth.normal((B, S, V), 3.0, seed, torch.float32, "cuda")
    rng = np.random.default_rng(seed)
    rows = np.argwhere(rng.random((B, S)) < 0.2)
    z[torch.from_numpy(rows[:, 0]).cuda(), torch.from_numpy(rows[:, 1]).cuda(),
      torch.from_numpy(rng.integers(0, V, len(rows))).cuda()] += 30.0
    return z.to(BF16)


def same(a: dict, b: dict, where):
    for n in a:
        x, y = a[n], b[n]
        if x.dtype == BF16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), f"{where}: {n}"


def test_early_skip_resume_is_bit_identical(lib, tmp_path):
    from token_skipping_partial_amd.step import EarlySkipModel, SelectConfig, load_state, save_state
    print("early-skip resume: 4 layers, skip 1 / 2, top-16 / top-8, 2 + 2 steps", flush=True)
    shape = lib.Shape(B=B, S=S, d=d, H=H, Hkv=Hkv, hd=hd, F=F, dtype="bf16", V=V)
    w = weights(1200)
    mk = lambda: EarlySkipModel(shape, w, 1, SelectConfig(mode=lib.SEL_TOPK, k=16, alpha=0.5),  # noqa: E731
                                B * 16, skip2=2, k2=8)
    x = inputs(5, 1300)
    a = mk()
    a.fill(x[0])
    for t in (1, 2):
        a.step(x[t], logits(1400 + t))
    save_state(a, tmp_path / "es.pt")
    b = mk()
    b.fill(x[4])          # a different history, overwritten by the restore
    load_state(b, tmp_path / "es.pt")
    for t in (3, 4):
        lg = logits(1400 + t)
        sa, ra = a.step(x[t], lg)
        sb, rb = b.step(x[t], lg)
        torch.cuda.synchronize()
        assert torch.equal(ra, rb) and torch.equal(sa[:int(ra[-1])], sb[:int(rb[-1])]), t
        same(a._carried(), b._carried(), f"step {t}")


def test_layer_adaptive_resume_is_bit_identical(lib, tmp_path):
    from token_skipping_partial_amd.step import LayerAdaptiveModel, load_state, save_state
    print("layer-adaptive resume: 4 layers, prompt 16, inject every 2nd step, 3 + 3 steps",
          flush=True)
    shape = lib.Shape(B=B, S=S, d=d, H=H, Hkv=Hkv, hd=hd, F=F, dtype="bf16")
    w = weights(1500)
    mk = lambda: LayerAdaptiveModel(shape, w, 0.05, [0.02] * L, prompt_len=16,  # noqa: E731
                                    inject_every=2)
    x = inputs(7, 1600)
    a = mk()
    a.fill(x[0])
    for t in (1, 2, 3):
        a.step(x[t])
    save_state(a, tmp_path / "ad.pt")
    b = mk()
    load_state(b, tmp_path / "ad.pt")
    for t in (4, 5, 6):
        sa, ra = a.step(x[t])
        sb, rb = b.step(x[t])
        torch.cuda.synchronize()
        assert a.plan == b.plan, t
        for i in range(L + 1):
            assert torch.equal(ra[i], rb[i]), (t, i)
            assert torch.equal(sa[i][:int(ra[i][-1])], sb[i][:int(rb[i][-1])]), (t, i)
        same(a._carried(), b._carried(), f"step {t}")


def test_decoder_resume_is_bit_identical_with_a_graph(lib, tmp_path):
    from token_skipping_partial_amd.step import (BlockDecoder, EarlySkipModel, SelectConfig,
                                                 load_state, save_state)
    print("block decoder resume: 4 layers, prompt 16, blocks of 8, 3 steps, then 3 graph "
          "replays on the restored decoder", flush=True)
    shape = lib.Shape(B=B, S=S, d=d, H=H, Hkv=Hkv, hd=hd, F=F, dtype="bf16", V=V)
    w = weights(1700)
    emb = synth.normal((V, d), 1.0, 1750, BF16, "cuda")
    mask = synth.normal((d,), 1.0, 1751, BF16, "cuda")
    prompt = torch.from_numpy(np.random.default_rng(1752).integers(0, V, (B, 16))).int().cuda()

    def mk():
        m = EarlySkipModel(shape, w, 0, SelectConfig(mode=lib.SEL_TOPK, k=4, alpha=0.0),
                           B * (4 + 8))
        dec = BlockDecoder(m, emb, mask, 16, 8, 0.9, 1)
        dec.start(prompt)
        return dec

    bufs = [logits(1800 + i) for i in range(3)]
    a = mk()
    for t in range(3):
        a.step(bufs[t % 3])
    save_state(a, tmp_path / "dec.pt")
    b = mk()
    graphs = [b.capture(buf) for buf in bufs]
    torch.cuda.synchronize()
    load_state(b, tmp_path / "dec.pt")
    for t in range(3, 6):
        a.step(bufs[t % 3])
        graphs[t % 3].replay()
        torch.cuda.synchronize()
        same(a._carried(), b._carried(), f"step {t}")
        same(a.model._carried(), b.model._carried(), f"step {t} model")
    assert int(a.tok.ge(0).sum()) > B * 16   # tokens were committed
