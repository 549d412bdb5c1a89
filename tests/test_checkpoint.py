"""Checkpoint / resume of the step drivers (host side; no kernel runs).

A driver's state is what its next step reads from the steps before it. These tests fill every
carried buffer of a CPU-allocated driver with seeded values, write the state with `save_state`,
read it into a fresh driver with `load_state` (plain `torch.load(..., weights_only=True)`
underneath) and check that every buffer holds the same bits, in place, and that a state saved
under another configuration is refused. The GPU test `test_gpu_resume.py` checks that a resumed
driver's next steps are bit-identical to the uninterrupted ones.
"""
import pytest
import torch

import token_skipping_partial_amd as tsp
from token_skipping_partial_amd.step import (BlockDecoder, EarlySkipModel, LayerAdaptiveModel,
                                             SelectConfig, load_state, save_state)

B, S, d, H, Hkv, hd, F, V, L = 2, 32, 256, 4, 2, 64, 512, 64, 4


def shape(S_=S):
    return tsp.Shape(B=B, S=S_, d=d, H=H, Hkv=Hkv, hd=hd, F=F, dtype="bf16", V=V)


def early_skip(skip=1, skip2=2, S_=S):
    return EarlySkipModel(shape(S_), [None] * L, skip, SelectConfig(mode=tsp.SEL_TOPK, k=8,
                                                                    alpha=0.5),
                          B * 16, device="cpu", skip2=skip2, k2=4)


def randomise(tensors, seed):
    g = torch.Generator().manual_seed(seed)
    for t in tensors.values():
        if t.dtype in (torch.bfloat16, torch.float32):
            t.copy_(torch.randn(t.shape, generator=g).to(t.dtype))
        else:
            t.copy_(torch.randint(0, 100, t.shape, generator=g).to(t.dtype))


def assert_same(a: dict, b: dict):
    assert set(a) == set(b)
    for n in a:
        assert torch.equal(a[n].view(torch.uint8) if a[n].dtype == torch.bfloat16 else a[n],
                           b[n].view(torch.uint8) if b[n].dtype == torch.bfloat16 else b[n]), n


def test_early_skip_state_round_trips(tmp_path):
    a, b = early_skip(), early_skip()
    randomise(a._carried(), 1)
    ptrs = {n: t.data_ptr() for n, t in b._carried().items()}
    save_state(a, tmp_path / "es.pt")
    load_state(b, tmp_path / "es.pt")
    assert_same(a._carried(), b._carried())
    assert {n: t.data_ptr() for n, t in b._carried().items()} == ptrs   # copied in place
    assert "h_ref2" in b._carried()


def test_adaptive_state_round_trips(tmp_path):
    mk = lambda: LayerAdaptiveModel(shape(), [None] * L, 0.05, 0.1, device="cpu",  # noqa: E731
                                    prompt_len=8, inject_every=3)
    a, b = mk(), mk()
    randomise(a._carried(), 2)
    a.t, a.cur = 7, 1
    a._plans = {False: [40, 30, 20, 20, 10], True: [64, 64, 64, 64, 64]}
    save_state(a, tmp_path / "ad.pt")
    load_state(b, tmp_path / "ad.pt")
    assert_same(a._carried(), b._carried())
    assert (b.t, b.cur) == (7, 1)
    assert b._plans == a._plans


def test_decoder_state_round_trips(tmp_path):
    def mk():
        m = early_skip(skip=0, skip2=0)
        emb = torch.zeros(V, d, dtype=torch.bfloat16)
        return BlockDecoder(m, emb, torch.zeros(d, dtype=torch.bfloat16), 8, 8, 0.9, 1,
                            device="cpu")
    a, b = mk(), mk()
    randomise(a._carried(), 3)
    randomise(a.model._carried(), 4)
    save_state(a, tmp_path / "dec.pt")
    load_state(b, tmp_path / "dec.pt")
    assert_same(a._carried(), b._carried())
    assert_same(a.model._carried(), b.model._carried())


def test_state_file_holds_plain_data(tmp_path):
    a = early_skip()
    save_state(a, tmp_path / "es.pt")
    st = torch.load(tmp_path / "es.pt", map_location="cpu", weights_only=True)
    assert st["format"] == "dllm-step-state/1"
    assert st["config"]["skip"] == 1 and st["config"]["layers"] == L
    assert all(t.device.type == "cpu" for t in st["tensors"].values())


@pytest.mark.parametrize("other, key", [(lambda: early_skip(skip=2, skip2=3), "skip"),
                                        (lambda: early_skip(S_=48), "shape"),
                                        (lambda: early_skip(skip2=0), "skip2")])
def test_state_of_another_configuration_is_refused(tmp_path, other, key):
    save_state(early_skip(), tmp_path / "es.pt")
    with pytest.raises(ValueError, match=key):
        load_state(other(), tmp_path / "es.pt")


def test_state_of_another_driver_is_refused(tmp_path):
    ad = LayerAdaptiveModel(shape(), [None] * L, 0.05, 0.1, device="cpu")
    save_state(ad, tmp_path / "ad.pt")
    with pytest.raises(ValueError, match="driver"):
        load_state(early_skip(), tmp_path / "ad.pt")
    with pytest.raises(ValueError, match="not a"):
        early_skip().load_state_dict({"tensors": {}})
