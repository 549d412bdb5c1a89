"""Benchmark of the token-skipping denoising step on one MI355X.

    python bench.py [--gpus 1] [--steps 16] [--warmup 3] [--workload llada_step]

Default workload (llada_step): one full denoising step of 32 LLaDA-8B-shaped layers (bf16, B=8,
S=1024, d=4096, 32 heads x 128, FFN 12288, vocabulary 126464) with early skip at layer 4: layers
0-3 on every token, saliency of the layer-4 input against the previous step (alpha = 0.5,
L1-normalised delta + max-softmax confidence of fresh previous-step logits), top-205 selection per
sequence, layers 4-31 on the 1640 selected rows against the cached K/V; the layer-0 input moves
from step to step and every cache is carried across steps. Inputs are resident in HBM before the
timed region.

Metric: selected-token layer-steps per second (rows x layers run per second: 4 x 8192 + 28 x
1640 per step). Rank 0 prints one JSON line with the step rate, the roofline of the call that
takes the most time per step (HIP events at every call boundary inside the timed region), the
partial-attention HBM rate inside the step, and the CPU oracle timed on sampled rows of the
same workload. `--workload llada_layer` runs the single-layer configuration (B=1, top-128).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix peak, published
METRIC = "selected-token layer-steps/sec at 8B shape; partial-attn HBM GB/s % peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=16)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="llada_step",
                   choices=["llada_layer", "llada_step", "llada_context", "llada_adaptive",
                            "llada_response", "llada_decode", "dream_sweep"],
                   help="llada_step (default): the full 32-layer early-skip step, B=8, S=1024, "
                        "top-205 per sequence; llada_layer: one LLaDA-8B-shaped layer, B=1; "
                        "llada_context: the llada_layer step keeping the attention context of "
                        "every token (exact rows for the selected, changed-key update for the rest); "
                        "llada_adaptive: 32 LLaDA-8B layers, B=1, S=1024, per-layer FFN rows chosen "
                        "by the cosine change of every token's attention context; "
                        "llada_response: llada_adaptive with a 512-token prompt left out of "
                        "response-only steps and re-injected every --inject-every steps; "
                        "llada_decode: long-context block decoding (S=4096, 3584 prompt + 16 "
                        "blocks of 32, 32 layers, early skip at layer 4, top-64 + the active "
                        "block), commit at confidence 0.9 with a top-1 fallback, every step "
                        "replayed from a HIP graph; dream_sweep: 28 Dream-7B-shaped layers (GQA "
                        "28/4), B=16, S=2048, early skip at layer 4, top-k by delta at 1, 2, 5, 10, "
                        "25 and 50%% of the tokens: step time and per-call rates")
    p.add_argument("--second-skip", type=int, default=0,
                   help="llada_step: a second skip point at this layer (0 = none; the pages name "
                        "1/8 and 1/4 of the depth: 4 and 8)")
    p.add_argument("--second-k", type=int, default=0,
                   help="llada_step: rows per sequence kept at the second skip point "
                        "(0 = half of the first top-k)")
    p.add_argument("--inject-every", type=int, default=8,
                   help="llada_response: every n-th step re-injects the prompt")
    p.add_argument("--sets", type=int, default=16, help="rotated input/weight sets")
    p.add_argument("--context-seq", type=int, default=1024, choices=[1024, 4096],
                   help="llada_context: sequence length (1024: top-128 of the llada_layer "
                        "recipe; 4096: the long-context shape with the top-96)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="budget of the CPU oracle sample (0 = skip)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run 5 plain device copies of 1 GiB (reference for rocprofv3 "
                        "FETCH_SIZE / WRITE_SIZE scaling) and exit")
    return p.parse_args()


def calibrate_copy():
    """Five device-to-device copies of exactly 1 GiB (read 1 GiB + write 1 GiB per launch)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": 5}), flush=True)


def kernel_traffic(kernel: str, source: str):
    """Measured HBM bytes per launch from profiles/traffic.json, or None when the kernel's
    source has changed since the counters were taken (hash mismatch) or none were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec:
        return None
    with open(os.path.join(ROOT, source), "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if rec.get("source_sha256") != digest:
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build runs the token-skipping step on a single "
              "MI355X (no collectives). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return

    if args.workload == "llada_step":
        run_llada_step(args)
        return
    if args.workload == "llada_context":
        run_llada_context(args)
        return
    if args.workload == "llada_decode":
        run_llada_decode(args)
        return
    if args.workload == "dream_sweep":
        run_dream_sweep(args)
        return
    if args.workload in ("llada_adaptive", "llada_response"):
        run_llada_adaptive(args, response=args.workload == "llada_response")
        return
    run_llada_layer(args)


def run_llada_layer(args):
    """One LLaDA-8B-shaped layer step, B=1, S=1024, top-128 of 1024 tokens, 16 rotated sets of
    weights, logits, hidden states and caches (so no set is still in the last-level cache)."""
    import token_skipping_partial_amd as tsp  # raises if libdllm.so is not built
    from synth import workloads as W
    from token_skipping_partial_amd.step import (LayerScratch, LayerWeights, SelectConfig,
                                                 SingleLayerStep, all_rows, selected_layer)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    dims = W.LLADA_LAYER
    k_sel = W.LLADA_TOPK
    shape = tsp.Shape(B=dims.B, S=dims.S, d=dims.d, H=dims.H, Hkv=dims.Hkv, hd=dims.hd,
                      F=dims.F, dtype="bf16", V=dims.V)
    print(f"[bench] building {args.sets} input sets of {shape}", file=sys.stderr, flush=True)

    sets = []
    fill = LayerScratch(shape, dims.B * dims.S, dev)
    sel_all, rp_all = all_rows(shape, dev)
    for i in range(args.sets):
        h_prev, h_cur, _, logits, w = W.layer_inputs(dims, W.LLADA_LARGE, seed=9000 + i,
                                                     device=dev)
        wd = LayerWeights.from_dict(w, dev)
        kc = torch.zeros(dims.B, dims.Hkv, dims.S, dims.hd, dtype=dims.dtype, device=dev)
        vc = torch.zeros_like(kc)
        h_out = torch.zeros(dims.B, dims.S, dims.d, dtype=dims.dtype, device=dev)
        # step t-1 state: the layer on every token of h_prev (untimed)
        selected_layer(shape, wd, h_prev, kc, vc, h_out, sel_all, rp_all, fill)
        sets.append((wd, h_prev, h_cur, logits, kc, vc, h_out))
    del fill
    torch.cuda.synchronize()

    step = SingleLayerStep(shape, SelectConfig(mode=tsp.SEL_TOPK, k=k_sel, alpha=0.5), k_sel, dev)
    stream = torch.cuda.current_stream()

    def run(i, ev=None, sal_ev=None):
        wd, h_prev, h_cur, logits, kc, vc, h_out = sets[i % len(sets)]
        sc = step.scratch
        if ev is not None:
            ev[0].record(stream)
        if sal_ev is not None:
            sal_ev[0].record(stream)
        tsp.dllm_saliency(shape, tsp.DELTA_L1N, 0.5, h_cur, h_prev, logits, step.score)
        if sal_ev is not None:
            sal_ev[1].record(stream)
        if ev is not None:
            ev[1].record(stream)
        tsp.dllm_select_compact(shape, tsp.SEL_TOPK, 0.0, k_sel, step.score, None, step.sel_idx,
                                step.row_ptr)
        if ev is not None:
            ev[2].record(stream)
        tsp.dllm_gather_qkv_scatter_kv(shape, h_cur, wd.g_attn, wd.w_qkv, step.sel_idx,
                                       step.row_ptr, k_sel, sc.q_sel, kc, vc, sc.ws_qkv)
        if ev is not None:
            ev[3].record(stream)
        tsp.dllm_partial_attn(shape, 1.0 / math.sqrt(dims.hd), sc.q_sel, kc, vc, step.sel_idx,
                              step.row_ptr, k_sel, sc.o_sel, sc.ws_attn)
        if ev is not None:
            ev[4].record(stream)
        tsp.dllm_gather_ffn_scatter(shape, h_cur, sc.o_sel, wd.w_o, wd.g_ffn, wd.w_gate, wd.w_up,
                                    wd.w_down, step.sel_idx, step.row_ptr, k_sel, h_out, sc.ws_ffn)
        if ev is not None:
            ev[5].record(stream)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()

    # timed region: the steps back to back; inside it, events only around the saliency launch
    # (the roofline kernel), whose duration is measured live here
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sal_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        run(args.warmup + i, sal_ev=sal_evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    M = int(step.row_ptr[-1].item())
    value = M * args.steps / (total_ms / 1e3)

    # per-call breakdown from a separate pass with an event between calls (untimed region)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        run(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    names = ["saliency", "select_compact", "gather_qkv_scatter_kv", "partial_attn",
             "gather_ffn_scatter"]
    per_call = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps
                for j, n in enumerate(names)}
    per_call["saliency"] = sum(e[0].elapsed_time(e[1]) for e in sal_evs) / args.steps

    # algorithmic bytes / flops per launch (what the method must move or compute)
    b = 2
    ntok = dims.B * dims.S
    nq, nkv = dims.H * dims.hd, dims.Hkv * dims.hd
    sal_bytes = ntok * (2 * dims.d * b + dims.V * b + 4)
    attn_bytes = (M * nq * b * 2 + 2 * dims.B * dims.S * nkv * b + M * 4 + (dims.B + 1) * 4)
    qkv_bytes = (nq + 2 * nkv) * dims.d * b + M * (dims.d * b + (nq + 2 * nkv) * b) + dims.d * b
    ffn_bytes = (dims.d * nq + 3 * dims.F * dims.d) * b + M * (nq * b + 2 * dims.d * b) + dims.d * b
    qkv_flops = 2.0 * M * (nq + 2 * nkv) * dims.d
    ffn_flops = 2.0 * M * (dims.d * nq + 3 * dims.F * dims.d)
    attn_flops = 4.0 * M * dims.S * nq
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9  # noqa: E731

    kernels = {
        "saliency": {"ms": per_call["saliency"], "bytes": sal_bytes,
                     "GB/s": gbs(sal_bytes, per_call["saliency"])},
        "select_compact": {"ms": per_call["select_compact"]},
        "gather_qkv_scatter_kv": {"ms": per_call["gather_qkv_scatter_kv"], "bytes": qkv_bytes,
                                  "GB/s": gbs(qkv_bytes, per_call["gather_qkv_scatter_kv"]),
                                  "TFLOP/s": qkv_flops / per_call["gather_qkv_scatter_kv"] / 1e9},
        "partial_attn": {"ms": per_call["partial_attn"], "bytes": attn_bytes,
                         "GB/s": gbs(attn_bytes, per_call["partial_attn"]),
                         "TFLOP/s": attn_flops / per_call["partial_attn"] / 1e9},
        "gather_ffn_scatter": {"ms": per_call["gather_ffn_scatter"], "bytes": ffn_bytes,
                               "GB/s": gbs(ffn_bytes, per_call["gather_ffn_scatter"]),
                               "TFLOP/s": ffn_flops / per_call["gather_ffn_scatter"] / 1e9},
    }
    sal_gbs = kernels["saliency"]["GB/s"]
    roofline = {"kernel": "saliency_logits_kernel (dllm_saliency: one launch per call)",
                "bound": "hbm", "achieved": round(sal_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(sal_gbs / HBM_PEAK_GBS, 4),
                "traffic": kernel_traffic("saliency_logits_kernel",
                                          "token_skipping_partial_amd/csrc/saliency.hip")}
    attn_gbs = kernels["partial_attn"]["GB/s"]
    partial_attn = {"achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                    "launches": "attention kernel + split-key merge kernel"}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(sets[0], dims, k_sel, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "selected-token layer-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: hidden N(0,1); 15% of tokens + N(0,0.5^2), the rest + N(0,(1e-3)^2); "
                "logits N(0,3^2); random-init weights N(0,0.02^2)",
        "config": {"workload": "llada_layer: one LLaDA-8B-shaped layer step, B=1, S=1024, "
                               "d=4096, 32x128 MHA, FFN 12288, V=126464, alpha=0.5, top-128",
                   "selected_per_step": M, "rotated_sets": args.sets},
        "roofline": roofline,
        "partial_attn": partial_attn,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


class CallMarks:
    """HIP events recorded at every call boundary of a step (on the stream the calls run on).
    After a synchronisation, durations() gives, per call name, the sum and count of the
    intervals that end at that name's events."""

    def __init__(self, stream, capacity: int):
        self.stream = stream
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        self.tags = []

    def start(self):
        self.tags = ["start"]
        self.events[0].record(self.stream)

    def __call__(self, tag):
        self.events[len(self.tags)].record(self.stream)
        self.tags.append(tag)

    def durations(self, into: dict):
        for i in range(1, len(self.tags)):
            ms = self.events[i - 1].elapsed_time(self.events[i])
            tot, n = into.get(self.tags[i], (0.0, 0))
            into[self.tags[i]] = (tot + ms, n + 1)


def call_work(dims, rows: int):
    """Algorithmic flops and HBM bytes of one launch of each layer call on `rows` selected rows
    (what the method must compute and move: weights once, each selected row's activations, the
    K/V cache read once per (sequence, kv head)), bf16 storage."""
    b = 2
    nq, nkv = dims.H * dims.hd, dims.Hkv * dims.hd
    nqkv = nq + 2 * nkv
    return {
        "qkv": {"flops": 2.0 * rows * nqkv * dims.d,
                "bytes": b * (nqkv * dims.d + dims.d + rows * (dims.d + nqkv)) + 4 * rows},
        "attn": {"flops": 4.0 * rows * dims.S * nq,
                 "bytes": b * (2 * rows * nq + 2 * dims.B * dims.S * nkv) + 4 * (rows + dims.B + 1)},
        "ffn": {"flops": 2.0 * rows * (dims.d * nq + 3 * dims.F * dims.d),
                "bytes": b * (dims.d * nq + 3 * dims.F * dims.d + 2 * dims.d
                              + rows * (nq + 2 * dims.d)) + 4 * rows},
    }


def run_llada_step(args):
    """32 LLaDA-8B layers, B=8, S=1024: layers 0-3 on every token, saliency at layer 4 (alpha 0.5,
    fresh previous-step logits), top-205 per sequence, layers 4-31 on the selected rows against the
    cached K/V. Hidden input X^t = X^(t-1) + per-step perturbation; caches carried across steps.
    The timed region holds the steps back to back with an event before and after it (value,
    ms_per_step). The per-call figures (calls, roofline, partial_attn) come from the next `steps`
    steps, run the same way with an event at every call boundary: those events cost GPU time of
    their own, so they stay out of the step time."""
    import synth
    import token_skipping_partial_amd as tsp
    from synth import workloads as W
    from token_skipping_partial_amd.step import EarlySkipModel, LayerWeights, SelectConfig

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dims, L, skip, k_sel = W.LLADA_STEP, 32, W.STEP_SKIP, W.STEP_TOPK
    shape = tsp.Shape(B=dims.B, S=dims.S, d=dims.d, H=dims.H, Hkv=dims.Hkv, hd=dims.hd,
                      F=dims.F, dtype="bf16", V=dims.V)
    print(f"[bench] llada_step: {L} layers of {shape}", file=sys.stderr, flush=True)
    layers = [LayerWeights.from_dict(synth.layer_weights(dims.d, dims.H, dims.Hkv, dims.hd, dims.F,
                                                         seed=7000 + l, device="cuda"))
              for l in range(L)]
    k2 = (args.second_k or k_sel // 2) if args.second_skip else 0
    model = EarlySkipModel(shape, layers, skip, SelectConfig(mode=tsp.SEL_TOPK, k=k_sel, alpha=0.5),
                           m_cap=dims.B * k_sel, skip2=args.second_skip, k2=k2)
    nsteps = args.warmup + 2 * args.steps
    xs = [synth.normal((dims.B, dims.S, dims.d), 1.0, 7500, torch.bfloat16, "cuda")]
    for t in range(1, nsteps + 1):
        large = synth.large_positions(dims.B, dims.S, W.LLADA_LARGE, seed=7600 + t, device="cuda")
        xs.append(synth.perturb(xs[-1], large, seed=7700 + t))
    logits = [synth.logits(dims.B, dims.S, dims.V, seed=7800 + i, device="cuda") for i in range(4)]
    print("[bench] inputs resident; fill step", file=sys.stderr, flush=True)
    model.fill(xs[0])
    for t in range(args.warmup):
        model.step(xs[1 + t], logits[t % 4])
    torch.cuda.synchronize()
    print("[bench] warm; timing", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for t in range(args.steps):
        i = args.warmup + t
        model.step(xs[1 + i], logits[i % 4])
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    print(f"[bench] {ms:.3f} ms per step; per-call pass", file=sys.stderr, flush=True)
    marks = [CallMarks(stream, 8 * L + 16) for _ in range(args.steps)]
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    m0.record(stream)
    for t in range(args.steps):
        i = args.warmup + args.steps + t
        marks[t].start()
        model.step(xs[1 + i], logits[i % 4], mark=marks[t])
    m1.record(stream)
    torch.cuda.synchronize()
    ms_marked = m0.elapsed_time(m1) / args.steps
    M = int(model.step1.row_ptr[-1].item())
    skip2 = args.second_skip or L
    M2 = int(model.step2.row_ptr[-1].item()) if args.second_skip else M
    units = skip * dims.B * dims.S + (skip2 - skip) * M + (L - skip2) * M2

    # per call class: total per step, launches per step, mean per launch, algorithmic rates
    acc = {}
    for mk in marks:
        mk.durations(acc)
    rows_of = {"dense": dims.B * dims.S, "sel": M, "sel2": M2}
    calls = {}
    for tag, (tot, n) in acc.items():
        entry = {"ms_per_step": round(tot / args.steps, 4), "launches_per_step": n // args.steps,
                 "us_per_launch": round(tot / n * 1e3, 2)}
        kind, _, call = tag.partition("_")
        if call in ("qkv", "attn", "ffn"):
            w = call_work(dims, rows_of[kind])[call]
            us = tot / n * 1e3
            entry.update({"rows": rows_of[kind], "flops_per_launch": w["flops"],
                          "bytes_per_launch": w["bytes"],
                          "TFLOP/s": round(w["flops"] / us / 1e6, 1),
                          "GB/s": round(w["bytes"] / us / 1e3, 1)})
        calls[tag] = entry
    # roofline: the layer call that takes the most time per step
    dom = max((t for t in calls if "flops_per_launch" in calls[t]),
              key=lambda t: calls[t]["ms_per_step"])
    d = calls[dom]
    ai = d["flops_per_launch"] / d["bytes_per_launch"]
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai >= ridge:
        roof = {"bound": "mfma", "achieved": d["TFLOP/s"], "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(d["TFLOP/s"] / MFMA_BF16_PEAK_TFS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": d["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(d["GB/s"] / HBM_PEAK_GBS, 4)}
    roofline = {"kernel": f"{dom}: {CALL_KERNELS[dom.partition('_')[2]]}",
                **roof, "traffic": call_traffic(dom)}
    pa = calls.get("sel_attn")
    partial_attn = None
    if pa:
        partial_attn = {"achieved": pa["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(pa["GB/s"] / HBM_PEAK_GBS, 4), "rows": M,
                        "us_per_launch": pa["us_per_launch"],
                        "kernel": CALL_KERNELS["attn"], "traffic": call_traffic("sel_attn")}
    cpu = None
    if args.cpu_seconds > 0 and not args.second_skip:
        cpu = cpu_baseline_step(dims, L, skip, M, args.cpu_seconds)
    out = {
        "metric": METRIC, "value": round(units / (ms * 1e-3), 1),
        "unit": "selected-token layer-steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: X0 N(0,1), per step 154 tokens per sequence + N(0,0.5^2), rest + "
                "N(0,(1e-3)^2); logits N(0,3^2); random-init weights N(0,0.02^2)",
        "config": {"workload": "llada_step: 32 LLaDA-8B-shaped layers, B=8, S=1024, d=4096, 32x128 "
                               "MHA, FFN 12288, V=126464, early skip at layer 4, alpha=0.5, "
                               "top-205 per sequence",
                   "units_per_step": units, "selected_per_step": M,
                   "ms_per_step_with_call_events": round(ms_marked, 3)},
        "roofline": roofline,
        "partial_attn": partial_attn,
        "calls": calls,
        "cpu_baseline": cpu,
    }
    if args.second_skip:
        out["config"]["workload"] += (f", second skip point at layer {args.second_skip} keeping "
                                      f"top-{k2} of those per sequence")
        out["config"]["selected_after_second_skip"] = M2
    print(json.dumps(out), flush=True)


# kernels each layer call launches (bf16, the planned shapes of the llada_step workload)
CALL_KERNELS = {
    "qkv": "dllm_gather_qkv_scatter_kv (gather + RMSNorm, then the QKV GEMM whose epilogue writes "
           "q rows and scatters K/V rows into the cache)",
    "attn": "dllm_partial_attn (attention over every cached key; split-key merge when planned)",
    "ffn": "dllm_gather_ffn_scatter (W_o GEMM + residual, RMSNorm, gate/up GEMM with SwiGLU, "
           "W_down GEMM + residual + scatter)",
}


def call_traffic(tag: str):
    """Measured HBM bytes per launch of a call class from profiles/traffic.json (FETCH_SIZE and
    WRITE_SIZE of the call's kernels, scaled by the copy calibration), or None when a source
    file has changed since the counters were taken or none were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("llada_step/" + tag)
    if not rec:
        return None
    for src, digest in rec.get("sources", {}).items():
        with open(os.path.join(ROOT, src), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return rec.get("bytes_per_launch")


def cpu_baseline_step(dims, L: int, skip: int, M: int, budget_s: float):
    """The C++ CPU oracle on the llada_step workload, extrapolated from sampled rows: the three
    layer calls (QKV + K/V scatter, attention over every key, FFN + scatter) on 64 rows,
    saliency of one sequence's 1024 tokens over the full vocabulary, and the selection of every
    sequence. Rows are independent given their inputs, so the step's time is the sample's scaled
    to 4 x 8192 + 28 x M layer rows and 8 x 1024 scored tokens. The sample runs on synthetic
    inputs of the same shapes drawn on the host; bf16 tensors go to the oracle as bit patterns."""
    import numpy as np

    import oracle as O
    import synth

    bits = lambda t: t.contiguous().view(torch.uint16).numpy()  # noqa: E731
    rows = 64
    scale = 1.0 / math.sqrt(dims.hd)
    w = {k: bits(v) for k, v in synth.layer_weights(dims.d, dims.H, dims.Hkv, dims.hd, dims.F,
                                                    seed=5000).items()}
    h = bits(synth.normal((1, dims.S, dims.d), 1.0, 5001, torch.bfloat16))
    kc = bits(synth.normal((1, dims.Hkv, dims.S, dims.hd), 1.0, 5002, torch.bfloat16))
    vc = bits(synth.normal((1, dims.Hkv, dims.S, dims.hd), 1.0, 5003, torch.bfloat16))
    sel = np.arange(0, dims.S, dims.S // rows, dtype=np.int32)[:rows]
    rp = np.array([0, sel.size], dtype=np.int32)
    t0 = time.perf_counter()
    n_layer = 0
    while True:
        O.selected_layer(h, w, sel, rp, kc, vc, h, dims.H, dims.Hkv, dims.hd, 1e-5, scale,
                         store="bf16")
        n_layer += 1
        if time.perf_counter() - t0 >= budget_s * 0.6:
            break
    t_layer = (time.perf_counter() - t0) / n_layer
    hc = bits(synth.normal((dims.S, dims.d), 1.0, 5004, torch.bfloat16))
    hp = bits(synth.normal((dims.S, dims.d), 1.0, 5005, torch.bfloat16))
    lg = bits(synth.logits(1, dims.S, dims.V, seed=5006))[0]
    t0 = time.perf_counter()
    O.saliency(hc, hp, lg, 0.5)
    t_sal = time.perf_counter() - t0
    score = np.random.default_rng(5007).standard_normal((dims.B, dims.S)).astype(np.float32)
    t0 = time.perf_counter()
    O.select_compact(score, None, O.SEL_TOPK, k=M // dims.B)
    t_sel = time.perf_counter() - t0
    layer_rows = skip * dims.B * dims.S + (L - skip) * M
    t_step = layer_rows / rows * t_layer + dims.B * t_sal + t_sel
    return {"value": round(layer_rows / t_step, 2), "unit": "selected-token layer-steps/s",
            "cores": O.threads(), "kind": "oracle",
            "sample": f"extrapolated: {n_layer} C++ oracle layer calls (QKV + K/V scatter, "
                      f"attention over every key, FFN + scatter) on {rows} rows ({t_layer:.2f} s "
                      f"each), saliency of {dims.S} tokens over the full vocabulary "
                      f"({t_sal:.2f} s), selection of {dims.B} sequences; scaled to {layer_rows} "
                      f"layer rows and {dims.B * dims.S} scored tokens per step (float64, "
                      f"std::thread over rows on {O.threads()} threads)"}


def run_llada_decode(args):
    """Long-context semi-autoregressive block decoding, B=1, S=4096 (3584 prompt + 16 blocks of
    32), 32 LLaDA-8B layers: every step is the early-skip step (layers 0-3 on every token, L1
    change of the layer-4 input ranks the rest, alpha 0: top-64 + the active block forced), the
    commit of the active block (confidence > 0.9, else the best one) from that step's logits, and
    the embeddings of the committed tokens; all on the device, replayed from one HIP graph per
    logits buffer (4 rotating N(0, 3^2) buffers in which 10% of the rows carry one logit raised by
    30, confidence ~1). Token and embedding tables are random."""
    import synth
    import token_skipping_partial_amd as tsp
    from synth import workloads as W
    from token_skipping_partial_amd.step import (BlockDecoder, EarlySkipModel, LayerWeights,
                                                 SelectConfig)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dims, L, skip, k_sel, P, blk_len = W.LLADA_LONG, 32, 4, 64, 3584, 32
    shape = tsp.Shape(B=dims.B, S=dims.S, d=dims.d, H=dims.H, Hkv=dims.Hkv, hd=dims.hd,
                      F=dims.F, dtype="bf16", V=dims.V)
    print(f"[bench] llada_decode: {L} layers of {shape}", file=sys.stderr, flush=True)
    layers = [LayerWeights.from_dict(synth.layer_weights(dims.d, dims.H, dims.Hkv, dims.hd, dims.F,
                                                         seed=7000 + l, device="cuda"))
              for l in range(L)]
    model = EarlySkipModel(shape, layers, skip, SelectConfig(mode=tsp.SEL_TOPK, k=k_sel, alpha=0.0),
                           m_cap=dims.B * (k_sel + blk_len))
    emb = synth.normal((dims.V, dims.d), 1.0, 7900, torch.bfloat16, "cuda")
    mask = synth.normal((dims.d,), 1.0, 7901, torch.bfloat16, "cuda")
    dec = BlockDecoder(model, emb, mask, P, blk_len, 0.9, 1)
    bufs = []
    for i in range(4):
        z = synth.normal((dims.B, dims.S, dims.V), 3.0, 7800 + i, torch.float32, "cuda")
        rows = synth.large_positions(dims.B, dims.S, dims.S // 10, seed=7850 + i, device="cuda")
        g = torch.Generator(device="cuda").manual_seed(7860 + i)
        idx = torch.randint(0, dims.V, (dims.B, dims.S), generator=g, device="cuda")
        z.view(-1, dims.V)[torch.arange(dims.B * dims.S, device="cuda"),
                           idx.view(-1)] += 30.0 * rows.view(-1).float()
        bufs.append(z.to(torch.bfloat16))
        del z
    prompt = torch.randint(0, dims.V, (dims.B, P), generator=torch.Generator().manual_seed(7870),
                           dtype=torch.int32).cuda()
    dec.start(prompt)
    torch.cuda.synchronize()
    graphs = [dec.capture(b) for b in bufs]
    for t in range(args.warmup):
        graphs[t % 4].replay()
    torch.cuda.synchronize()
    tok0 = int(dec.tok.ge(0).sum().item())
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    counts = torch.zeros(args.steps, dtype=torch.int32, device="cuda")
    t0.record(stream)
    for t in range(args.steps):
        graphs[(args.warmup + t) % 4].replay()
        counts[t] = model.step1.row_ptr[-1]
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    M = float(counts.float().mean().item())
    committed = int(dec.tok.ge(0).sum().item()) - tok0
    # one periodic full refresh (every layer on every token), timed on its own
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    dec.refresh()
    r1.record(stream)
    torch.cuda.synchronize()
    units = skip * dims.B * dims.S + (L - skip) * M
    out = {
        "metric": METRIC, "value": round(units / (ms * 1e-3), 1),
        "unit": "selected-token layer-steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: random token ids and embedding table N(0,1); logits N(0,3^2) with "
                "10% of rows spiked by +30 on one logit; random-init weights N(0,0.02^2)",
        "config": {"workload": "llada_decode: B=1, S=4096 (3584 prompt + 16 blocks of 32), 32 "
                               "LLaDA-8B-shaped layers, early skip at layer 4, top-64 by delta + "
                               "the active block, commit at confidence 0.9 with a top-1 fallback, "
                               "steps replayed from HIP graphs",
                   "units_per_step": units, "selected_per_step": M,
                   "tokens_committed": committed,
                   "tokens_per_s": round(committed / (ms * 1e-3 * args.steps), 1),
                   "blocks_done": int(dec.blk[0].item()),
                   "refresh_ms": round(r0.elapsed_time(r1), 3)},
    }
    print(json.dumps(out), flush=True)


def run_dream_sweep(args):
    """28 Dream-7B-shaped layers (d 3584, 28 query / 4 kv heads x 128, FFN 18944), B=16, S=2048:
    layers 0-3 on every token, the L1 change of the layer-4 input (alpha 0) picks the top-k of
    every sequence for layers 4-27. For each selected fraction (1, 2, 5, 10, 25, 50%: the last
    four are the workload's, the first two show where the products stop being bound by the
    weight stream): a fill, then timed steps, and the three layer calls of one selected layer
    timed one by one with their algorithmic flops and bytes. Inputs move by N(0, 0.5^2) at
    exactly k tokens of every sequence per step, N(0, (1e-3)^2) elsewhere."""
    import synth
    import token_skipping_partial_amd as tsp
    from synth import workloads as W
    from token_skipping_partial_amd.step import EarlySkipModel, LayerWeights, SelectConfig

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dims, L, skip = W.DREAM_GQA, 28, 4
    shape = tsp.Shape(B=dims.B, S=dims.S, d=dims.d, H=dims.H, Hkv=dims.Hkv, hd=dims.hd,
                      F=dims.F, dtype="bf16", V=0)
    print(f"[bench] dream_sweep: {L} layers of {shape}", file=sys.stderr, flush=True)
    layers = [LayerWeights.from_dict(synth.layer_weights(dims.d, dims.H, dims.Hkv, dims.hd, dims.F,
                                                         seed=8000 + l, device="cuda"))
              for l in range(L)]
    Nq, Nkv = dims.H * dims.hd, dims.Hkv * dims.hd
    w_bytes = 2 * (dims.d * (Nq + 2 * Nkv) + dims.d * Nq + 3 * dims.d * dims.F)
    stream = torch.cuda.current_stream()
    steps = max(1, min(args.steps, 8))
    points = []
    x0 = synth.normal((dims.B, dims.S, dims.d), 1.0, 8500, torch.bfloat16, "cuda")
    for frac in (0.01, 0.02, 0.05, 0.10, 0.25, 0.50):
        k = max(1, round(frac * dims.S))
        M = dims.B * k
        model = EarlySkipModel(shape, layers, skip, SelectConfig(mode=tsp.SEL_TOPK, k=k, alpha=0.0),
                               m_cap=M)
        xs = [x0]
        for t in range(1, 3 + steps + 1):
            large = synth.large_positions(dims.B, dims.S, k, seed=8600 + t, device="cuda")
            xs.append(synth.perturb(xs[-1], large, seed=8700 + t))
        model.fill(xs[0])
        for t in range(2):
            model.step(xs[1 + t])
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for t in range(steps):
            model.step(xs[3 + t])
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        # the three calls of layer `skip` on this step's rows, one event pair around 20 repeats of
        # each (enough for the host to run ahead of the GPU, so launch latency is not timed)
        s1, sc, w = model.step1, model.sparse, layers[skip]
        calls = {
            "gather_qkv_scatter_kv": lambda: tsp.dllm_gather_qkv_scatter_kv(
                shape, model.hidden[skip], w.g_attn, w.w_qkv, s1.sel_idx, s1.row_ptr, M, sc.q_sel,
                model.k[skip], model.v[skip], sc.ws_qkv),
            "partial_attn": lambda: tsp.dllm_partial_attn(
                shape, 1.0 / math.sqrt(dims.hd), sc.q_sel, model.k[skip], model.v[skip],
                s1.sel_idx, s1.row_ptr, M, sc.o_sel, sc.ws_attn),
            "gather_ffn_scatter": lambda: tsp.dllm_gather_ffn_scatter(
                shape, model.hidden[skip], sc.o_sel, w.w_o, w.g_ffn, w.w_gate, w.w_up, w.w_down,
                s1.sel_idx, s1.row_ptr, M, model.hidden[skip + 1], sc.ws_ffn),
        }
        flops = {"gather_qkv_scatter_kv": 2.0 * M * dims.d * (Nq + 2 * Nkv),
                 "partial_attn": 4.0 * M * dims.S * Nq,
                 "gather_ffn_scatter": 2.0 * M * dims.d * (Nq + 3 * dims.F)}
        nbytes = {"gather_qkv_scatter_kv": 2 * dims.d * (Nq + 2 * Nkv) + 2 * M * (dims.d + Nq + 2 * Nkv),
                  "partial_attn": 2 * dims.B * dims.S * 2 * Nkv + 2 * M * 2 * Nq,
                  "gather_ffn_scatter": 2 * dims.d * (Nq + 3 * dims.F) + 2 * M * (Nq + 3 * dims.d)}
        per = {}
        for name, fn in calls.items():
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / 20 * 1e3
            per[name] = {"us": round(us, 1), "TFLOP/s": round(flops[name] / us / 1e6, 1),
                         "GB/s": round(nbytes[name] / us / 1e3, 1),
                         "flop_per_byte": round(flops[name] / nbytes[name], 1)}
        units = skip * dims.B * dims.S + (L - skip) * M
        points.append({"fraction": frac, "k_per_sequence": k, "rows": M, "ms_per_step": round(ms, 3),
                       "units_per_s": round(units / (ms * 1e-3), 1), "layer_calls": per})
        print(f"[bench] dream_sweep {frac:.0%}: {ms:.2f} ms/step", file=sys.stderr, flush=True)
        del model
        torch.cuda.empty_cache()
    ref = next(p for p in points if p["fraction"] == 0.10)
    out = {
        "metric": METRIC, "value": ref["units_per_s"], "unit": "selected-token layer-steps/s",
        "n_gpus": 1, "steps": steps, "warmup": 2, "ms_per_step": ref["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: X0 N(0,1), per step k tokens per sequence + N(0,0.5^2), rest + "
                "N(0,(1e-3)^2); random-init weights N(0,0.02^2)",
        "config": {"workload": "dream_sweep: 28 Dream-7B-shaped layers (GQA 28/4 x 128, FFN "
                               "18944), B=16, S=2048, early skip at layer 4, alpha 0, top-k per "
                               "sequence; value and ms_per_step at 10%", "weight_bytes_per_layer":
                   w_bytes, "points": points},
    }
    print(json.dumps(out), flush=True)


def run_llada_context(args):
    """The llada_layer step with the attention context of every token kept (DyLLM §2.B): copies
    of the rows about to change, the projection, then exact rows for the 128 selected tokens and
    the changed-key update of the other 896 tokens' softmax state, then the FFN of the selected.
    16 rotated sets, each with its own caches, query cache and state (initialised untimed by a
    select-all call)."""
    import token_skipping_partial_amd as tsp
    from synth import workloads as W
    from token_skipping_partial_amd.step import (LayerScratch, LayerWeights, SelectConfig,
                                                 SingleLayerStep, all_rows, selected_layer)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    if args.context_seq == 4096:
        dims, k_sel, n_large = W.LLADA_LONG, 96, round(0.15 * 4096)
    else:
        dims, k_sel, n_large = W.LLADA_LAYER, W.LLADA_TOPK, W.LLADA_LARGE
    shape = tsp.Shape(B=dims.B, S=dims.S, d=dims.d, H=dims.H, Hkv=dims.Hkv, hd=dims.hd,
                      F=dims.F, dtype="bf16", V=dims.V)
    ntok, nq, nkv = dims.B * dims.S, dims.H * dims.hd, dims.Hkv * dims.hd
    scale = 1.0 / math.sqrt(dims.hd)
    print(f"[bench] llada_context: building {args.sets} sets of {shape}", file=sys.stderr,
          flush=True)
    fill = LayerScratch(shape, ntok, dev)
    sel_all, rp_all = all_rows(shape, dev)
    ws_all = tsp.workspace(tsp.OP_ATTN, shape, ntok)
    sets = []
    for i in range(args.sets):
        h_prev, h_cur, _, logits, w = W.layer_inputs(dims, n_large, seed=9000 + i, device=dev)
        wd = LayerWeights.from_dict(w, dev)
        kc = torch.zeros(dims.B, dims.Hkv, dims.S, dims.hd, dtype=dims.dtype, device=dev)
        vc = torch.zeros_like(kc)
        h_out = torch.zeros(dims.B, dims.S, dims.d, dtype=dims.dtype, device=dev)
        selected_layer(shape, wd, h_prev, kc, vc, h_out, sel_all, rp_all, fill)
        q_all = torch.empty(ntok, nq, dtype=dims.dtype, device=dev)
        st_m = torch.empty(ntok, dims.H, device=dev)
        st_l = torch.empty(ntok, dims.H, device=dev)
        st_o = torch.empty(ntok, nq, device=dev)
        o_all = torch.empty(ntok, nq, dtype=dims.dtype, device=dev)
        # state of step t-1: every token's context from its query of the fill pass
        kv_rows = torch.empty(2, ntok, nkv, dtype=dims.dtype, device=dev)
        tsp.dllm_salient_attn(shape, scale, fill.q_sel, q_all, kc, vc, kv_rows[0], kv_rows[1],
                              sel_all, rp_all, ntok, st_m, st_l, st_o, fill.o_sel, o_all, ws_all)
        sets.append((wd, h_prev, h_cur, logits, kc, vc, h_out, q_all, st_m, st_l, st_o, o_all))
    del fill, kv_rows
    torch.cuda.synchronize()
    step = SingleLayerStep(shape, SelectConfig(mode=tsp.SEL_TOPK, k=k_sel, alpha=0.5), k_sel, dev)
    sc = step.scratch
    k_old = torch.empty(k_sel, nkv, dtype=dims.dtype, device=dev)
    v_old = torch.empty_like(k_old)
    stream = torch.cuda.current_stream()

    def run(i, ev=None):
        wd, h_prev, h_cur, logits, kc, vc, h_out, q_all, st_m, st_l, st_o, o_all = \
            sets[i % len(sets)]
        rec = (lambda j: ev[j].record(stream)) if ev is not None else (lambda j: None)
        rec(0)
        tsp.dllm_saliency(shape, tsp.DELTA_L1N, 0.5, h_cur, h_prev, logits, step.score)
        tsp.dllm_select_compact(shape, tsp.SEL_TOPK, 0.0, k_sel, step.score, None, step.sel_idx,
                                step.row_ptr)
        rec(1)
        tsp.dllm_gather_kv_rows(shape, kc, vc, step.sel_idx, step.row_ptr, k_sel, k_old, v_old)
        rec(2)
        tsp.dllm_gather_qkv_scatter_kv(shape, h_cur, wd.g_attn, wd.w_qkv, step.sel_idx,
                                       step.row_ptr, k_sel, sc.q_sel, kc, vc, sc.ws_qkv)
        rec(3)
        tsp.dllm_salient_attn(shape, scale, sc.q_sel, q_all, kc, vc, k_old, v_old, step.sel_idx,
                              step.row_ptr, k_sel, st_m, st_l, st_o, sc.o_sel, o_all, sc.ws_attn)
        rec(4)
        tsp.dllm_gather_ffn_scatter(shape, h_cur, sc.o_sel, wd.w_o, wd.g_ffn, wd.w_gate, wd.w_up,
                                    wd.w_down, step.sel_idx, step.row_ptr, k_sel, h_out, sc.ws_ffn)
        rec(5)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        run(args.warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    M = int(step.row_ptr[-1].item())
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        run(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    names = ["saliency+select", "gather_kv_rows", "gather_qkv_scatter_kv", "salient_attn",
             "gather_ffn_scatter"]
    per = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps
           for j, n in enumerate(names)}
    # what the same contexts cost by exact recomputation of every row (dllm_partial_attn, all
    # 1024 queries against all keys), timed on one set
    wd, h_prev, h_cur, logits, kc, vc, h_out, q_all, st_m, st_l, st_o, o_all = sets[0]
    o_full = torch.empty(ntok, nq, dtype=dims.dtype, device=dev)
    for _ in range(3):
        tsp.dllm_partial_attn(shape, scale, q_all, kc, vc, sel_all, rp_all, ntok, o_full, ws_all)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        tsp.dllm_partial_attn(shape, scale, q_all, kc, vc, sel_all, rp_all, ntok, o_full, ws_all)
    e1.record(stream)
    torch.cuda.synchronize()
    full_ms = e0.elapsed_time(e1) / 10
    b = 2
    ctx_bytes = (ntok * nq * b                       # query cache
                 + 2 * ntok * nq * 4 + 4 * ntok * dims.H * 4   # state read + write
                 + ntok * nq * b                     # context of every token
                 + 2 * 2 * M * nkv * b               # old and new rows of the changed keys
                 + M * nq * b * 3                    # new queries, their cache rows, o_sel
                 + 2 * dims.B * dims.S * nkv * b)    # exact rows: the cache once per kv head
    gbs = ctx_bytes / (per["salient_attn"] * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(M * args.steps / (ms * args.steps * 1e-3), 1),
        "unit": "selected-token layer-steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: as llada_layer",
        "config": {"workload": f"llada_context: LLaDA-8B-shaped layer step, B=1, S={dims.S}, "
                               f"top-{k_sel}, keeping the attention context of every token "
                               f"({k_sel} exact rows, {ntok - k_sel} changed-key updates)",
                   "selected_per_step": M, "rotated_sets": args.sets},
        "salient_attn": {"ms": round(per["salient_attn"], 4), "bytes": ctx_bytes,
                         "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "all_rows_exact_ms": round(full_ms, 4)},
        "kernels": {k: round(v, 4) for k, v in per.items()},
    }
    print(json.dumps(out), flush=True)


def run_llada_adaptive(args, response=False):
    """32 LLaDA-8B layers, B=1, S=1024, layer-adaptive (DyLLM §2.A/§2.B): the 154 tokens whose
    layer-0 input moved (L1-normalised change > 0.05) are the first layer's rows; in every layer
    the contexts of all tokens are kept and the tokens whose context moved most (cosine change
    above a per-layer threshold, set from an untimed calibration step at the 80th percentile of
    that layer's scores) get W_o + FFN and become the next layer's rows. Inputs cumulative as in
    llada_step.
    response=True (DyLLM §2.C): positions 0-511 are the prompt (512 prompt + 512 generation);
    the 154 moving tokens are drawn among the generation positions, response-only steps leave
    the prompt out, every --inject-every-th step re-injects it; thresholds from the response
    positions' scores."""
    import synth
    import token_skipping_partial_amd as tsp
    from synth import workloads as W
    from token_skipping_partial_amd.step import LayerAdaptiveModel, LayerWeights

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dims, L = W.LLADA_LAYER, 32
    shape = tsp.Shape(B=dims.B, S=dims.S, d=dims.d, H=dims.H, Hkv=dims.Hkv, hd=dims.hd,
                      F=dims.F, dtype="bf16", V=dims.V)
    print(f"[bench] llada_adaptive: {L} layers of {shape}", file=sys.stderr, flush=True)
    layers = [LayerWeights.from_dict(synth.layer_weights(dims.d, dims.H, dims.Hkv, dims.hd, dims.F,
                                                         seed=7000 + l, device="cuda"))
              for l in range(L)]
    P = dims.S // 2 if response else 0
    inject = args.inject_every if response else 0
    model = LayerAdaptiveModel(shape, layers, 0.05, [0.0] * L, prompt_len=P, inject_every=inject)
    nsteps = args.warmup + args.steps + 1
    xs = [synth.normal((dims.B, dims.S, dims.d), 1.0, 7500, torch.bfloat16, "cuda")]
    prompt = torch.zeros(dims.B, dims.S, dtype=torch.bool)
    prompt[:, :P] = True
    for t in range(1, nsteps + 1):
        large = synth.large_positions(dims.B, dims.S, W.LLADA_LARGE, seed=7600 + t,
                                      exclude=prompt if P else None, device="cuda")
        xs.append(synth.perturb(xs[-1], large, seed=7700 + t))
    model.fill(xs[0])
    # calibration (untimed): context thresholds at the 80th percentile of each layer's scores
    taus = []
    model.layer_scores = None
    for l in range(L):
        model.step(xs[1], tau_ctx=taus + [-1.0] * (L - l), record=True)
        taus.append(float(torch.quantile(model.layer_scores[l][:, P:].flatten(), 0.8).item()))
        model.fill(xs[0])
    model.tau_ctx = taus
    for t in range(args.warmup):
        model.step(xs[1 + t])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    counts, kinds = [], []
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0.record(stream)
    evs[0].record(stream)
    for t in range(args.steps):
        sel, rp = model.step(xs[1 + args.warmup + t])
        evs[t + 1].record(stream)
        kinds.append(bool(inject) and model.t % inject == 0)
        counts.append(torch.stack([r[-1] for r in rp]))
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    per = [evs[t].elapsed_time(evs[t + 1]) for t in range(args.steps)]
    c = torch.stack(counts).float().mean(0).cpu().tolist()   # [input rows, FFN rows per layer]
    ffn_rows = sum(c[1:])
    qkv_rows = sum(c[:-1])
    out = {
        "metric": METRIC, "value": round(ffn_rows / (ms * 1e-3), 1),
        "unit": "selected-token layer-steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: X0 N(0,1), per step 154 tokens + N(0,0.5^2), rest + N(0,(1e-3)^2); "
                "random-init weights N(0,0.02^2)",
        "config": {"workload": "llada_adaptive: 32 LLaDA-8B-shaped layers, B=1, S=1024, "
                               "layer-adaptive FFN rows (cosine change of every token's context, "
                               "per-layer threshold at the calibrated 80th percentile)",
                   "ffn_rows_per_step": round(ffn_rows, 1),
                   "projection_rows_per_step": round(qkv_rows, 1),
                   "rows_per_layer": [round(v, 1) for v in c]},
    }
    if response:
        out["config"]["workload"] = (
            f"llada_response: llada_adaptive with positions 0-{P - 1} a prompt, left out of "
            f"response-only steps, re-injected every {inject}th step; 154 moving tokens among "
            f"the generation positions")
        ri = [p for p, k in zip(per, kinds) if not k]
        ij = [p for p, k in zip(per, kinds) if k]
        out["config"]["ms_response_only_step"] = round(sum(ri) / max(1, len(ri)), 3)
        out["config"]["ms_inject_step"] = round(sum(ij) / max(1, len(ij)), 3) if ij else None
        out["config"]["inject_steps_timed"] = len(ij)
    print(json.dumps(out), flush=True)


def cpu_baseline(one_set, dims, k_sel, budget_s):
    """The CPU oracle on the same workload: whole steps (saliency over every token and the full
    vocabulary, selection, then the layer on the selected rows) until the budget is used."""
    import numpy as np

    import oracle as O

    import synth

    # the generator outputs of set 0 (weights, hidden states, logits) as bf16 bit patterns; the
    # step t-1 caches and hidden rows are fresh synthetic tensors of their shapes (the oracle's
    # time does not depend on their values)
    wd, h_prev, h_cur, logits = one_set[:4]
    bits = lambda t: t.detach().cpu().contiguous().view(torch.uint16).numpy()  # noqa: E731
    hp, hc, lg = bits(h_prev[0]), bits(h_cur[0]), bits(logits[0])
    w = {n: bits(getattr(wd, n)) for n in ("g_attn", "w_qkv", "w_o", "g_ffn", "w_gate", "w_up",
                                             "w_down")}
    k0 = bits(synth.normal((dims.B, dims.Hkv, dims.S, dims.hd), 1.0, 5101, torch.bfloat16))
    v0 = bits(synth.normal((dims.B, dims.Hkv, dims.S, dims.hd), 1.0, 5102, torch.bfloat16))
    y0 = bits(synth.normal((dims.B, dims.S, dims.d), 1.0, 5103, torch.bfloat16))
    scale = 1.0 / math.sqrt(dims.hd)
    steps, t0 = 0, time.perf_counter()
    while True:
        score, _, _ = O.saliency(hc, hp, lg, 0.5)
        sel, rp = O.select_compact(score.reshape(1, -1), None, O.SEL_TOPK, k=k_sel)
        O.selected_layer(hc[None], w, sel, rp, k0, v0, y0, dims.H, dims.Hkv, dims.hd, 1e-5, scale,
                         store="bf16")
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 200:
            break
    return {"value": round(k_sel * steps / el, 2), "unit": "selected-token layer-steps/s",
            "cores": O.threads(), "kind": "oracle",
            "sample": f"{steps} whole C++ oracle steps of the same workload (set 0), {el:.1f} s; "
                      f"float64, std::thread over rows on {O.threads()} threads"}


if __name__ == "__main__":
    main()
