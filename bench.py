"""Decode-step benchmark of the packed K6/V4 KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2|3|4|5]

A step is one pass of the hot path for one layer: quantise-and-append the
new token of every sequence, then split-K decode attention of one query per
sequence over the whole packed cache, then the merge of the split partials.
With one segment and a uniform batch (workloads 2, 4) that is
lkv_append_decode_merged, one launch: the split kernel writes each
sequence's new row itself and merges the splits (--two-launch:
lkv_append_decode, the split kernel then lkv_decode_combine).  The tiered
workload 3 (two segments) is one launch too: lkv_append_decode_merged over
both segments, the new row going to HIGH (--two-launch: lkv_quant_append,
then lkv_decode_split and lkv_decode_combine).  The ragged workload 5 runs
lkv_append_decode_merged in compact order (--two-launch: lkv_append_decode,
its split kernel in compact order, then the merge kernel).  Every workload
with --unfused runs lkv_quant_append, lkv_decode_split and
lkv_decode_combine.  Steps rotate over several layer caches so that
consecutive steps stream from HBM, not from the 256 MB last-level cache.

  workload 2 (default) and 4: every step re-appends the row of the last
    position and attends over all N positions, the same work as the step
    that brings the context to N tokens (--fp16-layer: the fp16 format of
    workload 4's sensitive layers).
  workload 3: the cache is appended at K6V6 and tiered once per layer
    (untimed) into a HIGH (K6V6) and a MID (K6V4) segment; a step re-appends
    the last HIGH row and decodes over both segments with the sparse-V skip
    at tau_low.
  workload 5: 64 ragged sequences in a permuted paged pool; decode step s of
    a layer appends the token at position len_b + s of every sequence and
    decodes over len_b + s + 1 tokens (the positions and lengths of every
    step are prepared on the device beforehand).

Prints one JSON line.  `value` is packed-KV GB/s: counted bytes per step
(packed codes + fp32 scales + uint8 zero points of every live token and KV
head, plus Q and O, plus the appended rows) over the measured step time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, 8 TB/s
METRIC = "packed-KV decode attention GB/s (% of HBM peak); decode tokens/s at 32K ctx"
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # after every synchronisation (the GPU idle) the step time of workload 2
    # ran fast for ~30 steps, then up to 40% slower for a few hundred, then
    # steady: the default run times enough steps for the steady part to
    # dominate
    p.add_argument("--steps", type=int, default=10000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5])
    p.add_argument("--layers", type=int, default=4, help="layer caches rotated over (HBM, not cache)")
    p.add_argument("--split-tokens", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seqs", type=int, default=8, help="sequences in the oracle's timed sample")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="least oracle time in the CPU baseline")
    p.add_argument("--copy-probe", action="store_true",
                   help="after the timed steps, stream 1 GiB in and 1 GiB out (counter scaling reference)")
    p.add_argument("--fp16-layer", action="store_true", help="time the fp16 sensitive-layer format")
    p.add_argument("--no-tier", action="store_true", help="skip the tier-update and re-tiering secondary figures")
    p.add_argument("--no-secondary", action="store_true",
                   help="skip every secondary figure but the prefill append (counter passes: only the step's kernels run)")
    p.add_argument("--graph", action="store_true",
                   help="replay each step as a captured HIP graph instead of launching its kernels from the host")
    p.add_argument("--kv-heads", type=int, default=0,
                   help="workloads 2 and 4: this many KV heads (query heads scaled to keep the GQA group), e.g. 1 "
                        "for one GPU's share of a cache sharded by KV head over 8 GPUs")
    p.add_argument("--probe-only", action="store_true",
                   help="only the HBM read probe (a streaming read of 4 GiB; profiling)")
    p.add_argument("--tier-only", action="store_true",
                   help="only the tier-update and re-tier figures at the tiered workload's shape (profiling)")
    p.add_argument("--two-launch", action="store_true",
                   help="the split kernel, then the merge kernel, instead of one launch that merges in the split "
                        "kernel (workloads 2 to 5)")
    p.add_argument("--unfused", action="store_true",
                   help="three launches per step: the append kernel, the split kernel, the merge")
    return p.parse_args()


def measured_traffic(kernel: str, workload: str, fused: bool, merged: bool = False):
    """HBM bytes of the split kernel and the merge per step, from the
    committed counter summary, if it was taken on the current kernel sources
    with the same step; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    from quantized_kv_cache_token_amd.profsum import kernel_source_hash

    if (rec.get("source_hash") != kernel_source_hash() or bool(rec.get("fused")) != fused or
            bool(rec.get("merged")) != merged):
        return None
    return rec.get("hbm_bytes_per_step")


class Setup:
    """What the timing loop needs from a workload: the prepared stages of
    each step ((append, split, combine), or (append + split, combine) when
    the split kernel appends), the counted bytes of step i, the split
    kernel's algorithmic bytes, and the JSON config."""

    def __init__(self):
        self.calls = []          # stages per rotation slot
        self.fused = False       # the split stage also appends the new rows
        self.merged = None       # ... and merges its own splits (one launch per step)
        self.keep = []           # tensors the prepared calls point at
        self.step_bytes = None   # i -> counted bytes of step i
        self.split_alg = None    # i -> algorithmic bytes of the split launch of step i (KV + Q)
        self.append_bytes = 0    # counted bytes of a step's append (rows in, packed rows out)
        self.out_bytes = 0       # bytes of O the merge writes
        self.sequences = 0
        self.config = {}
        self.later = []          # (name, figure) secondary figures run after the timed steps
        self.secondary = {}
        self.per_token_head = 0
        self.q_bytes = 2


def _event():
    import torch

    return torch.cuda.Event(enable_timing=True)


def fused_step(args, S, cache, view, k, v, q, sm, split, out, ws, counters, merged: bool):
    """The stages of one fused step: lkv_append_decode_merged (one launch)
    when asked for (merged) and the library takes that form, else the split
    kernel with the append and the merge kernel (lkv_append_decode's two
    stages)."""
    from quantized_kv_cache_token_amd import lkv

    if S.merged is None:  # decided once, by whether the library takes the merged form
        S.merged = False
        if merged:
            try:
                lkv.append_decode_merged(cache, view, k, v, q, sm, 0.0, split, counters, out, ws)
                S.merged = True
            except lkv.LkvError as e:
                if e.status != lkv.EUNSUPPORTED:
                    raise
    if S.merged:
        return (lkv.prepare_append_decode_merged(cache, view, k, v, q, sm, 0.0, split, out, counters, ws),)
    return lkv.prepare_append_decode(cache, view, k, v, q, sm, 0.0, split, out, ws)


def setup_uniform(args, wl, dev) -> Setup:
    """Workloads 2 and 4: every sequence at N tokens, identity block tables."""
    import numpy as np
    import torch

    from quantized_kv_cache_token_amd import inputs, lkv

    kb, vb = (16, 16) if args.fp16_layer else (wl.k_bits, wl.v_bits)
    B, Hq, Hkv, D, N = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.n_ctx
    name = wl.name if not args.fp16_layer else wl.name.replace("k6v4", "fp16")
    if args.kv_heads:  # one GPU's share of a cache sharded by KV head: the same GQA group
        Hq, Hkv = Hq // Hkv * args.kv_heads, args.kv_heads
        name = name.replace(f"hq{wl.num_q_heads}_hkv{wl.num_kv_heads}", f"hq{Hq}_hkv{Hkv}")
    nblk = (N + 63) // 64
    bt = torch.arange(B * nblk, dtype=torch.int32, device=dev).view(B, nblk)
    lens = torch.full((B,), N, dtype=torch.int32, device=dev)
    outl = inputs.outlier_channels(wl.seed, Hkv, D) if wl.outliers else None
    S = Setup()
    # layer caches, filled by the append kernel (prefill; each call timed with
    # events for the secondary figures, outside the timed steps)
    caches, prefill = [], []
    for layer in range(args.layers):
        c = lkv.Cache(D, wl.group_size, kb, vb, Hkv, B * nblk, device=dev)
        for b in range(B):
            k, v = inputs.kv_rows(wl.seed, b, N - 1, Hkv, D, dtype=wl.dtype, outliers=outl, layer=layer,
                                  device=dev)
            cu = torch.tensor([0, N - 1], dtype=torch.int32, device=dev)
            sp0 = torch.zeros(1, dtype=torch.int32, device=dev)
            e0, e1 = _event(), _event()
            e0.record()
            lkv.quant_append(c, k, v, cu, sp0, bt[b:b + 1], N - 1)
            e1.record()
            prefill.append((e0, e1))
            del k, v
        caches.append(c)
    torch.cuda.synchronize()
    prefill_ms = [a.elapsed_time(b) for a, b in prefill]
    view = lkv.View(bt, lens, N)
    cu1 = torch.arange(B + 1, dtype=torch.int32, device=dev)
    last = torch.full((B,), N - 1, dtype=torch.int32, device=dev)
    sm = float(np.float32(1.0 / np.sqrt(D)))
    split = args.split_tokens or lkv.decode_plan([caches[0]], [view], B, Hq)
    ws = lkv.decode_workspace([caches[0]], [view], B, Hq, split, dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    S.fused = not args.unfused
    counters = lkv.merge_counters(caches[0], B, dev)
    for layer in range(args.layers):
        k, v = inputs.kv_rows(wl.seed, 1000, B, Hkv, D, dtype=wl.dtype, outliers=outl, layer=layer, step=1,
                              device=dev)
        q = inputs.queries(wl.seed, B, Hq, D, dtype=wl.dtype, layer=layer, device=dev)
        if S.fused:  # the new row of each sequence is position N - 1: lengths are N
            S.calls.append(fused_step(args, S, caches[layer], view, k, v, q, sm, split, out, ws, counters,
                                      not args.two_launch))
        else:
            app = lkv.prepare_append(caches[layer], k, v, cu1, last, bt, 1)
            spl, comb = lkv.prepare_decode([caches[layer]], [view], q, sm, 0.0, split, out, ws)
            S.calls.append((app, spl, comb))
        S.keep += [k, v, q]
    S.keep += [caches, bt, lens, view, cu1, last, ws, out, counters]
    ptk = caches[0].chunk_bytes // 64
    if not args.fp16_layer and not args.no_secondary:
        # measured after the timed steps, so that their buffers and launches
        # are not around while the steps run
        keep = S.keep
        S.later += [("decode_with_scores", lambda: scores_figure(caches, view, keep, B, Hq, Hkv, D, N, sm, split, dev)),
                    ("multi_token", lambda: multi_figure(caches, view, keep, B, Hq, Hkv, D, N, sm, ptk, dev)),
                    ("k_norm", lambda: knorm_figure(args, wl, bt, view, keep, sm, dev))]
    qb = 2 if wl.dtype == "bf16" else 4
    kv = B * Hkv * N * ptk
    S.per_token_head, S.q_bytes = ptk, qb
    S.step_bytes = lambda i: kv + B * Hq * D * (qb + 4) + B * Hkv * (2 * D * qb + ptk)
    S.split_alg = lambda i: kv + B * Hq * D * qb
    S.append_bytes, S.out_bytes = B * Hkv * (2 * D * qb + ptk), B * Hq * D * 4
    S.sequences = B
    S.config = {"workload": name, "batch": B,
                "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "ctx_tokens": N,
                "group_size": wl.group_size, "k_bits": kb, "v_bits": vb, "q_dtype": wl.dtype,
                "split_tokens": split, "layers_rotated": args.layers, "append_in_split_kernel": S.fused,
                "merge_in_split_kernel": bool(S.merged)}
    pre_bytes = (N - 1) * Hkv * (2 * D * qb + ptk)
    pre_s = float(np.median(prefill_ms)) / 1e3
    S.secondary["append_prefill"] = {"GB/s": round(pre_bytes / pre_s / 1e9, 1),
                                     "us_per_call": round(pre_s * 1e6, 1), "rows_per_call": N - 1,
                                     "counted": "bf16 K/V rows in + packed rows out"}
    return S


def scores_figure(caches, view, keep, B, Hq, Hkv, D, N, sm, split, dev):
    """lkv_decode_attn_scores against lkv_decode_attn over the same layer
    caches: 32 calls of each, back to back, between one event pair."""
    import torch

    from quantized_kv_cache_token_amd import lkv

    acc = torch.zeros((1, B, N), dtype=torch.float32, device=dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    ws_s = lkv.decode_scores_workspace([caches[0]], [view], B, Hq, split, dev)
    ws = lkv.decode_workspace([caches[0]], [view], B, Hq, split, dev)
    qs = [torch.randn(B, Hq, D, device=dev).to(torch.bfloat16) for _ in caches]
    with_s = [lkv.prepare_decode_scores([c], [view], q, sm, 0.0, split, out, acc, ws_s) for c, q in zip(caches, qs)]
    plain = []
    for c, q in zip(caches, qs):
        spl, comb = lkv.prepare_decode([c], [view], q, sm, 0.0, split, out, ws)
        plain.append((spl, comb))

    def run(fn):
        for i in range(8):
            fn(i)
        e0, e1 = _event(), _event()
        e0.record()
        for i in range(32):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 32 * 1e3

    t_s = run(lambda i: with_s[i % len(with_s)]())
    t_p = run(lambda i: [f() for f in plain[i % len(plain)]])
    keep += [acc, out, ws_s, ws, qs, with_s, plain]
    extra = B * Hq * N * 4 * 2 + B * N * 4 * 2
    return {"us_per_call": round(t_s, 1), "plain_us_per_call": round(t_p, 1),
            "extra_bytes_per_call": extra,
            "counted": "score rows written and read (B x Hq x N fp32) plus the accumulator read and written"}


def multi_figure(caches, view, keep, B, Hq, Hkv, D, N, sm, ptk, dev):
    """lkv_decode_attn_multi over the same layer caches: T query tokens per
    sequence (the last T of the N cached ones, causal), T = 4 and 16, with
    the library's split plan; 32 calls rotated over the layers between one
    event pair after 8 untimed ones.  Counted bytes: the cache once, Q and
    the fp32 output."""
    import torch

    from quantized_kv_cache_token_amd import lkv

    fig = {}
    for T in (4, 16):
        split = lkv.decode_plan_multi([caches[0]], [view], B, T, Hq)
        ws = lkv.decode_workspace([caches[0]], [view], B * T, Hq, split, dev)
        out = torch.empty(B, T, Hq, D, dtype=torch.float32, device=dev)
        qs = [torch.randn(B, T, Hq, D, device=dev).to(torch.bfloat16) for _ in caches]

        def call(i):
            lkv.decode_attn_multi([caches[i % len(caches)]], [view], qs[i % len(caches)], sm, 0.0, split, out, ws)

        for i in range(8):
            call(i)
        e0, e1 = _event(), _event()
        e0.record()
        for i in range(32):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 32 / 1e3
        nbytes = B * Hkv * N * ptk + B * T * Hq * D * (2 + 4)
        fig[f"T{T}"] = {"us_per_call": round(t * 1e6, 1), "GB/s": round(nbytes / t / 1e9, 1),
                        "query_tokens_per_s": round(B * T / t, 1), "split_tokens": split}
        keep += [ws, out, qs]
    fig["counted"] = "the layer's packed cache once, bf16 Q and fp32 output"
    return fig


def knorm_figure(args, wl, bt, view, keep, sm, dev):
    """The direction-preserving K codec at the same shape: layer caches
    appended with k_norm = 1 (each prefill timed with events), then 32
    decode calls rotated over them between one event pair after 8 untimed
    ones.  Counted bytes per token-head: the plain format's plus the 4-byte
    norm factor."""
    import numpy as np
    import torch

    from quantized_kv_cache_token_amd import inputs, lkv

    B, Hq, Hkv, D, N = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.n_ctx
    outl = inputs.outlier_channels(wl.seed, Hkv, D) if wl.outliers else None
    caches, pre = [], []
    for layer in range(args.layers):
        c = lkv.Cache(D, wl.group_size, wl.k_bits, wl.v_bits, Hkv, bt.numel(), device=dev, k_norm=1)
        for b in range(B):
            k, v = inputs.kv_rows(wl.seed, b, N, Hkv, D, dtype=wl.dtype, outliers=outl, layer=layer, device=dev)
            e0, e1 = _event(), _event()
            e0.record()
            lkv.quant_append(c, k, v, torch.tensor([0, N], dtype=torch.int32, device=dev),
                             torch.zeros(1, dtype=torch.int32, device=dev), bt[b:b + 1], N)
            e1.record()
            pre.append((e0, e1))
            del k, v
        caches.append(c)
    split = lkv.decode_plan([caches[0]], [view], B, Hq)
    ws = lkv.decode_workspace([caches[0]], [view], B, Hq, split, dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    qs = [inputs.queries(wl.seed, B, Hq, D, dtype=wl.dtype, layer=layer, device=dev) for layer in range(args.layers)]
    calls = [lkv.prepare_decode([c], [view], q, sm, 0.0, split, out, ws) for c, q in zip(caches, qs)]
    for i in range(8):
        for f in calls[i % len(calls)]:
            f()
    e0, e1 = _event(), _event()
    e0.record()
    for i in range(32):
        for f in calls[i % len(calls)]:
            f()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 32 / 1e3
    ptk = caches[0].chunk_bytes // 64
    nbytes = B * Hkv * N * ptk + B * Hq * D * (2 + 4)
    pre_s = float(np.median([a.elapsed_time(b) for a, b in pre])) / 1e3
    pre_bytes = N * Hkv * (2 * D * 2 + ptk)
    keep += [caches, ws, out, qs, calls]
    return {"decode_us_per_call": round(t * 1e6, 1), "decode_GB/s": round(nbytes / t / 1e9, 1),
            "bytes_per_token_head": ptk, "append_prefill_us": round(pre_s * 1e6, 1),
            "append_prefill_GB/s": round(pre_bytes / pre_s / 1e9, 1),
            "counted": "codes, scales, zeros and norm factors once, bf16 Q and fp32 output"}


def setup_tiered(args, wl, dev) -> Setup:
    """Workload 3: K6V6 append and one tier update per layer (untimed), then
    steps of (re-append the last HIGH row, decode over HIGH + MID with the
    skip at tau_low)."""
    import numpy as np
    import torch

    from quantized_kv_cache_token_amd import inputs, lkv

    B, Hq, Hkv, D, N = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.n_ctx
    nblk = (N + 63) // 64
    bt = torch.arange(B * nblk, dtype=torch.int32, device=dev).view(B, nblk)
    outl = inputs.outlier_channels(wl.seed, Hkv, D) if wl.outliers else None
    tl, th = lkv.default_thresholds(N)
    scores = torch.stack([inputs.tier_scores(wl.seed, b, N, tl, th) for b in range(B)]).to(dev)
    S = Setup()
    segs = []
    for layer in range(args.layers):
        src = lkv.Cache(D, wl.group_size, 6, 6, Hkv, B * nblk, device=dev)
        for b in range(B):
            k, v = inputs.kv_rows(wl.seed, b, N, Hkv, D, dtype=wl.dtype, outliers=outl, layer=layer, device=dev)
            lkv.quant_append(src, k, v, torch.tensor([0, N], dtype=torch.int32, device=dev),
                             torch.zeros(1, dtype=torch.int32, device=dev), bt[b:b + 1], N)
            del k, v
        h = lkv.Cache(D, wl.group_size, 6, 6, Hkv, B * nblk, device=dev)
        m = lkv.Cache(D, wl.group_size, 6, 4, Hkv, B * nblk, device=dev)
        nh = torch.zeros(B, dtype=torch.int32, device=dev)
        nm = torch.zeros_like(nh)
        tiers = torch.zeros((B, N), dtype=torch.uint8, device=dev)
        lkv.tier_update(src, lkv.View(bt, torch.full((B,), N, dtype=torch.int32, device=dev), N), scores, tl, th,
                        h, bt, m, bt, nh, nm, tiers)
        torch.cuda.synchronize()
        del src, tiers
        torch.cuda.empty_cache()
        segs.append((h, m, nh, nm))
    nh_h, nm_h = segs[0][2].cpu().numpy(), segs[0][3].cpu().numpy()
    max_h, max_m = int(nh_h.max()), int(nm_h.max())
    sm = float(np.float32(1.0 / np.sqrt(D)))
    views0 = [lkv.View(bt, segs[0][2], max_h), lkv.View(bt, segs[0][3], max_m)]
    split = args.split_tokens or lkv.decode_plan([segs[0][0], segs[0][1]], views0, B, Hq)
    ws = lkv.decode_workspace([segs[0][0], segs[0][1]], views0, B, Hq, split, dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    cu1 = torch.arange(B + 1, dtype=torch.int32, device=dev)
    counters = lkv.merge_counters(segs[0][0], B, dev)
    S.fused = S.merged = not args.two_launch and not args.unfused
    for layer, (h, m, nh, nm) in enumerate(segs):
        lv = [lkv.View(bt, nh, max_h), lkv.View(bt, nm, max_m)]
        last = (nh - 1).contiguous()
        k, v = inputs.kv_rows(wl.seed, 1000, B, Hkv, D, dtype=wl.dtype, outliers=outl, layer=layer, step=1,
                              device=dev)
        q = inputs.queries(wl.seed, B, Hq, D, dtype=wl.dtype, layer=layer, device=dev)
        if S.merged:  # one launch: append into HIGH, split over both segments, merge
            S.calls.append((lkv.prepare_append_decode_merged([h, m], lv, k, v, q, sm, tl, split, out, counters,
                                                             ws),))
        else:
            app = lkv.prepare_append(h, k, v, cu1, last, bt, 1)
            spl, comb = lkv.prepare_decode([h, m], lv, q, sm, tl, split, out, ws)
            S.calls.append((app, spl, comb))
        S.keep += [k, v, q, last, lv]
    S.keep += [segs, bt, scores, views0, ws, out, cu1, counters]
    qb = 2 if wl.dtype == "bf16" else 4
    kv = int(Hkv * (int(nh_h.sum()) * 212 + int(nm_h.sum()) * 180))
    S.per_token_head, S.q_bytes = 212, qb
    S.step_bytes = lambda i: kv + B * Hq * D * (qb + 4) + B * Hkv * (2 * D * qb + 212)
    S.split_alg = lambda i: kv + B * Hq * D * qb
    S.append_bytes, S.out_bytes = B * Hkv * (2 * D * qb + 212), B * Hq * D * 4
    S.sequences = B
    S.config = {"workload": wl.name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                "ctx_tokens": N, "high_tokens": int(nh_h[0]), "mid_tokens": int(nm_h[0]),
                "group_size": wl.group_size, "segments": "K6V6 + K6V4", "tau_low": tl, "q_dtype": wl.dtype,
                "split_tokens": split, "layers_rotated": args.layers, "append_in_split_kernel": S.fused,
                "merge_in_split_kernel": S.merged}
    return S


def setup_ragged(args, wl, dev) -> Setup:
    """Workload 5: ragged lengths in a permuted paged pool; decode step s of
    each layer appends one token per sequence at len_b + s, then decodes over
    len_b + s + 1 tokens.  Positions and lengths of all steps are device
    tensors prepared beforehand; every step's max_len is the final one."""
    import numpy as np
    import torch

    from quantized_kv_cache_token_amd import inputs, lkv

    B, Hq, Hkv, D = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lens = inputs.ragged_lengths(wl.seed, B, *wl.ragged).numpy().astype(np.int64)
    n_steps = wl.steps
    cap = lens + n_steps
    nblk = (cap + 63) // 64
    max_blocks = int(nblk.max())
    total = int(nblk.sum())
    perm = inputs.block_permutation(wl.seed, total).numpy()
    bt_h = np.zeros((B, max_blocks), np.int32)
    at = 0
    for b in range(B):
        bt_h[b, :nblk[b]] = perm[at:at + nblk[b]]
        at += nblk[b]
    bt = torch.tensor(bt_h, device=dev)
    pos = torch.tensor(lens[None, :] + np.arange(n_steps)[:, None], dtype=torch.int32, device=dev)  # [steps][B]
    after = (pos + 1).contiguous()
    max_len = int(cap.max())
    S = Setup()
    caches = []
    for layer in range(args.layers):
        c = lkv.Cache(D, wl.group_size, wl.k_bits, wl.v_bits, Hkv, total, device=dev)
        for b0 in range(0, B, 16):
            ks, vs = [], []
            for b in range(b0, b0 + 16):
                k, v = inputs.kv_rows(wl.seed, b, int(lens[b]), Hkv, D, dtype=wl.dtype, layer=layer, device=dev)
                ks.append(k)
                vs.append(v)
            cu = torch.tensor(np.concatenate([[0], np.cumsum(lens[b0:b0 + 16])]), dtype=torch.int32, device=dev)
            lkv.quant_append(c, torch.cat(ks), torch.cat(vs), cu, torch.zeros(16, dtype=torch.int32, device=dev),
                             bt[b0:b0 + 16].contiguous(), int(lens[b0:b0 + 16].max()))
            del ks, vs
        caches.append(c)
    torch.cuda.synchronize()
    sm = float(np.float32(1.0 / np.sqrt(D)))
    live = [int((lens + s + 1).sum()) for s in range(n_steps)]
    # the host knows the batch's lengths: they size the splits (sum_len hint,
    # and the last step's lengths, which every step's work items fit)
    view_last = lkv.View(bt, after[-1], max_len, live[-1])
    split = args.split_tokens or lkv.decode_plan_lens(caches[0], view_last, cap, Hq)
    ws = lkv.decode_workspace([caches[0]], [view_last], B, Hq, split, dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    cu1 = torch.arange(B + 1, dtype=torch.int32, device=dev)
    kvs = [inputs.kv_rows(wl.seed, 2000, B, Hkv, D, dtype=wl.dtype, layer=layer, step=1, device=dev)
           for layer in range(args.layers)]
    qs = [inputs.queries(wl.seed, B, Hq, D, dtype=wl.dtype, layer=layer, device=dev) for layer in range(args.layers)]
    views = [lkv.View(bt, after[s], max_len, live[s]) for s in range(n_steps)]
    # rotation slot i = s * layers + layer: decode step s of that layer
    S.fused = not args.unfused
    counters = lkv.merge_counters(caches[0], B, dev)
    for s in range(n_steps):
        for layer in range(args.layers):
            k, v = kvs[layer]
            if S.fused:  # the new row of sequence b is position len_b + s: the step's lengths count it
                S.calls.append(fused_step(args, S, caches[layer], views[s], k, v, qs[layer], sm, split, out, ws,
                                          counters, not args.two_launch))
            else:
                app = lkv.prepare_append(caches[layer], k, v, cu1, pos[s], bt, 1)
                spl, comb = lkv.prepare_decode([caches[layer]], [views[s]], qs[layer], sm, 0.0, split, out, ws)
                S.calls.append((app, spl, comb))
    S.keep += [caches, bt, pos, after, views, ws, out, cu1, kvs, qs, counters]
    qb = 2 if wl.dtype == "bf16" else 4
    L = args.layers
    S.per_token_head, S.q_bytes = 180, qb
    S.step_bytes = lambda i: live[(i // L) % n_steps] * Hkv * 180 + B * Hq * D * (qb + 4) + B * Hkv * (
        2 * D * qb + 180)
    S.split_alg = lambda i: live[(i // L) % n_steps] * Hkv * 180 + B * Hq * D * qb
    S.append_bytes, S.out_bytes = B * Hkv * (2 * D * qb + 180), B * Hq * D * 4
    S.sequences = B
    S.config = {"workload": wl.name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                "ctx_tokens_min": int(lens.min()), "ctx_tokens_max": int(cap.max()),
                "ctx_tokens_mean": round(float(lens.mean()), 1), "decode_steps": n_steps,
                "group_size": wl.group_size, "k_bits": wl.k_bits, "v_bits": wl.v_bits, "q_dtype": wl.dtype,
                "split_tokens": split, "layers_rotated": L, "paged": "seeded permutation of pool blocks",
                "append_in_split_kernel": S.fused, "merge_in_split_kernel": bool(S.merged)}
    return S


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; its kernels run on one "
              "GPU's share of a cache sharded by KV head.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_kv_cache_token_amd import workloads

    wl = workloads.BY_INDEX[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.tier_only:
        tier, retier = tier_figure(workloads.BY_INDEX[3], dev)
        if args.copy_probe:
            copy_probe(dev)
        print(json.dumps({"tier_update": tier, "retier": retier}), flush=True)
        return
    if args.probe_only:
        print(json.dumps({"hbm_read_probe": probe_figure(dev)}), flush=True)
        return
    # one stream (default priority) for every prepared call and graph
    run_stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(run_stream):
        if args.workload == 3:
            S = setup_tiered(args, wl, dev)
        elif args.workload == 5:
            S = setup_ragged(args, wl, dev)
            args.steps = min(args.steps, len(S.calls))
        else:
            S = setup_uniform(args, wl, dev)
    torch.cuda.synchronize()
    n_calls = len(S.calls)

    def step(i, ev=None):
        stages = S.calls[i % n_calls]
        if ev is not None:
            ev[0].record(run_stream)
        for j, fn in enumerate(stages):
            fn()
            if ev is not None:
                ev[j + 1].record(run_stream)

    # warmup, then the timed steps; workload 5 times its decode steps from
    # the first (its warmup replays the first slots, appending the same rows)
    first = 0 if args.workload == 5 else args.warmup
    import gc
    with torch.cuda.stream(run_stream):
        for i in range(args.warmup):
            step(i)
    if not args.graph:
        # the host's own preparation of the timed region runs while the
        # warmup steps do, so that the GPU does not idle before the timed
        # steps: the cycle collector, and the timed region's events
        gc.collect()
        gc.disable()  # no cycle-collector pause inside the timed steps
    g0, g1 = _event(), _event()
    nwin = min(10, args.steps)  # an event at each tenth of the timed steps: the step time by window
    wev = [_event() for _ in range(nwin - 1)]
    torch.cuda.synchronize()
    n_stages = len(S.calls[0])
    # the step of each rotation slot as a HIP graph (its launches replayed
    # without host work in between, as a serving loop runs a decode step)
    graphs = None
    if args.graph:
        graphs = []
        for i in range(n_calls):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=run_stream):
                step(i)
            graphs.append(g)
        torch.cuda.synchronize()
        with torch.cuda.stream(run_stream):
            for i in range(args.warmup):
                graphs[i % n_calls].replay()
        torch.cuda.synchronize()
    # timed region: K steps between synchronisations; HIP events on the
    # run stream bracket all of them (the steps' GPU time)
    if args.graph:
        gc.collect()
        gc.disable()  # no cycle-collector pause inside the timed steps
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(run_stream):
        g0.record(run_stream)
        for i in range(args.steps):
            if i * nwin % args.steps < nwin and 0 < i * nwin // args.steps:
                wev[i * nwin // args.steps - 1].record(run_stream)
            if graphs is not None:
                graphs[(first + i) % n_calls].replay()
            else:
                step(first + i)
        g1.record(run_stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    gpu_step_s = g0.elapsed_time(g1) / 1e3 / args.steps
    bounds = [g0] + wev + [g1]
    edges = [0] + [next(i for i in range(args.steps) if i * nwin // args.steps == w) for w in range(1, nwin)] + [args.steps]
    window_us = [round(bounds[w].elapsed_time(bounds[w + 1]) * 1e3 / (edges[w + 1] - edges[w]), 1) for w in range(nwin)]
    # then, outside the timed region, HIP events before and after each stage
    # of the first (at most 2000) timed steps, replayed launch by launch over
    # the same rotation: the split kernel's and the merge's own durations
    timed = list(range(min(args.steps, 2000)))
    evs = {i: tuple(_event() for _ in range(n_stages + 1)) for i in timed}
    with torch.cuda.stream(run_stream):
        for i in timed:
            step(first + i, evs[i])
    torch.cuda.synchronize()
    if args.copy_probe:
        copy_probe(dev)

    step_s = (t1 - t0) / args.steps
    total_bytes = sum(S.step_bytes(first + i) for i in range(args.steps))
    value = total_bytes / (t1 - t0) / 1e9
    # stage times: the split stage (K2; with the fused append it also writes
    # the new rows) and the merge (K3), from the events around them
    if n_stages == 1:  # one launch: the split kernel appends and merges
        split_ms = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in timed])
        comb_ms = np.zeros_like(split_ms)
    else:
        si = n_stages - 2  # the split stage is the one before the merge
        split_ms = np.array([evs[i][si].elapsed_time(evs[i][si + 1]) for i in timed])
        comb_ms = np.array([evs[i][si + 1].elapsed_time(evs[i][si + 2]) for i in timed])
    split_alg = np.array([S.split_alg(first + i) for i in timed], dtype=np.float64)
    if S.fused:
        split_alg = split_alg + S.append_bytes
    k23_alg = split_alg + S.out_bytes
    split_s = float(split_ms.mean()) / 1e3
    split_achieved = float(split_alg.sum() / (split_ms.sum() / 1e3)) / 1e9
    if S.fused:
        # a step is the split kernel and the merge (one kernel when it merges
        # its own splits): its GPU time over the timed region is K2 + K3
        # (with any gap between them)
        k23_alg = np.array([S.split_alg(first + i) + S.append_bytes + S.out_bytes for i in range(args.steps)],
                           dtype=np.float64)
        k23_s = gpu_step_s
        k23_src = ("hip events around the timed steps (a step is one kernel that appends, splits and merges)"
                   if S.merged else "hip events around the timed steps (a step is the split kernel and the merge)")
    else:
        k23_s = float((split_ms + comb_ms).mean()) / 1e3
        k23_src = "hip events around each kernel, one step in every rotation cycle"
    achieved = float(k23_alg.mean() / k23_s) / 1e9
    kname = ("append_split_merged" if S.merged else "append_split+combine") if S.fused else "decode_split+combine"
    traffic = measured_traffic("decode_step", S.config["workload"], S.fused, bool(S.merged))

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "gpu_ms_per_step": round(gpu_step_s * 1e3, 4),
        "step_us_by_tenth": window_us,
        "graph_replay": graphs is not None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f16x2-mfma/f32-acc" if S.config.get("k_bits") == 16 else "bf16x2-mfma/f32-acc")
        if S.config.get("q_dtype") == "bf16" else "f32",
        "data": "synthetic",
        "config": S.config,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(S.sequences / step_s, 1),
        "bytes_per_step": int(round(total_bytes / args.steps)),
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": int(round(k23_alg.mean())),
                     "avg_launch_us": round(k23_s * 1e6, 2), "timing": k23_src,
                     "split_only": {"kernel": ("append_split_merged" if S.merged else "append_split") if S.fused
                                    else "decode_split",
                                    "achieved": round(split_achieved, 2),
                                    "frac": round(split_achieved / HBM_PEAK_GBS, 4),
                                    "alg_bytes_per_launch": int(round(split_alg.mean())),
                                    "avg_launch_us": round(split_s * 1e6, 2)},
                     "combine_us": round(float(comb_ms.mean()) * 1e3, 2)},
    }
    secondary = dict(S.secondary)
    with torch.cuda.stream(run_stream):
        for name, fig in S.later:
            secondary[name] = fig()
    torch.cuda.synchronize()
    ptk, qb = S.per_token_head, S.q_bytes
    kb, vb = S.config.get("k_bits"), S.config.get("v_bits")
    if args.workload == 4 and not args.fp16_layer and not args.kv_heads and not args.no_secondary:
        secondary["stack_32_layers"] = stack_figure(args, wl, dev, gpu_step_s)
    if args.workload == 2 and not args.fp16_layer and not args.no_tier and not args.no_secondary:
        del S
        torch.cuda.empty_cache()
        secondary["tier_update"], secondary["retier"] = tier_figure(workloads.BY_INDEX[3], dev)
    if args.workload in (2, 5) and not args.fp16_layer and not args.no_tier and not args.no_secondary:
        S = None
        torch.cuda.empty_cache()
        secondary["serving_tiered"] = serving_figure(workloads.BY_INDEX[5], dev)
    if not args.no_secondary:
        secondary["hbm_read_probe"] = probe_figure(dev)
    if secondary:
        rec["secondary"] = secondary
    if not args.no_cpu_baseline and args.workload in (2, 4):
        rec["cpu_baseline"] = cpu_baseline(wl, kb, vb, min(args.cpu_seqs, wl.batch), ptk, qb, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def stack_figure(args, wl, dev, quant_step_s):
    """The whole decode stack of workload 4 (2 of every 32 layers held in
    fp16): the fp16 layer's step (append + decode at the same shape, two
    layer caches rotated, 64 steps between one event pair after 8 untimed
    ones), then per token step 30 quantised layers at the timed step's GPU
    time and 2 fp16 layers."""
    import copy

    import torch

    a16 = copy.copy(args)
    a16.fp16_layer, a16.no_secondary, a16.layers, a16.kv_heads = True, True, 2, 0
    run_stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(run_stream):
        S16 = setup_uniform(a16, wl, dev)
    torch.cuda.synchronize()

    def step(i):
        for fn in S16.calls[i % len(S16.calls)]:
            fn()

    with torch.cuda.stream(run_stream):
        for i in range(8):
            step(i)
    torch.cuda.synchronize()
    e0, e1 = _event(), _event()
    with torch.cuda.stream(run_stream):
        e0.record(run_stream)
        for i in range(64):
            step(i)
        e1.record(run_stream)
    torch.cuda.synchronize()
    f16_s = e0.elapsed_time(e1) / 64 / 1e3
    nf = wl.fp16_layers
    nq = wl.layers_per_stack - nf
    stack_s = nq * quant_step_s + nf * f16_s
    del S16
    torch.cuda.empty_cache()
    return {"layers": wl.layers_per_stack, "fp16_layers": nf, "quantised_layer_us": round(quant_step_s * 1e6, 2),
            "fp16_layer_us": round(f16_s * 1e6, 2), "stack_us_per_token_step": round(stack_s * 1e6, 1),
            "decode_tokens_per_s": round(wl.batch / stack_s, 1),
            "counted": "attention of every layer (append + decode), nothing else of the model"}


def copy_probe(dev):
    """A plain streaming kernel of known traffic (reads 1 GiB, writes 1 GiB),
    three launches: the reference that scales the HBM byte counters."""
    import torch

    src = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def tier_figure(wl, dev):
    """One lkv_tier_update at the tiered workload's shape (the batch and
    context of `wl`, K6V6 source, scores with 10% high / 30% mid / 60% low),
    then one lkv_retier of its segments with fresh scores of the same mix,
    each timed with events after one untimed call.  Counted bytes: source
    rows and scores read, survivors' rows, tiers and counts written."""
    import torch

    from quantized_kv_cache_token_amd import inputs, lkv

    B, Hkv, D, N = wl.batch, wl.num_kv_heads, wl.head_dim, wl.n_ctx
    nblk = (N + 63) // 64
    bt = torch.arange(B * nblk, dtype=torch.int32, device=dev).view(B, nblk)
    src = lkv.Cache(D, wl.group_size, 6, 6, Hkv, B * nblk, device=dev)
    outl = inputs.outlier_channels(wl.seed, Hkv, D) if wl.outliers else None
    for b in range(B):
        k, v = inputs.kv_rows(wl.seed, b, N, Hkv, D, dtype=wl.dtype, outliers=outl, device=dev)
        lkv.quant_append(src, k, v, torch.tensor([0, N], dtype=torch.int32, device=dev),
                         torch.zeros(1, dtype=torch.int32, device=dev), bt[b:b + 1], N)
        del k, v
    tl, th = lkv.default_thresholds(N)
    scores = torch.stack([inputs.tier_scores(wl.seed, b, N, tl, th) for b in range(B)]).to(dev)
    hdst = lkv.Cache(D, wl.group_size, 6, 6, Hkv, B * nblk, device=dev)
    mdst = lkv.Cache(D, wl.group_size, 6, 4, Hkv, B * nblk, device=dev)
    tiers = torch.zeros((B, N), dtype=torch.uint8, device=dev)
    nh = torch.zeros(B, dtype=torch.int32, device=dev)
    nm = torch.zeros_like(nh)
    view = lkv.View(bt, torch.full((B,), N, dtype=torch.int32, device=dev), N)
    ws = torch.empty(lkv.tier_workspace_bytes(B, N), dtype=torch.uint8, device=dev)
    call = lambda: lkv.tier_update(src, view, scores, tl, th, hdst, bt, mdst, bt, nh, nm, tiers, ws)
    call()
    e0, e1 = _event(), _event()
    e0.record()
    call()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    n_h, n_m = int(nh.sum()), int(nm.sum())
    nbytes = B * N * Hkv * 212 + B * N * 4 + (n_h * 212 + n_m * 180) * Hkv + B * N + 8 * B
    tier = {"GB/s": round(nbytes / t / 1e9, 1), "us_per_call": round(t * 1e6, 1), "high": n_h, "mid": n_m,
            "evicted": B * N - n_h - n_m, "counted": "K6V6 rows and scores in, HIGH/MID rows and tiers out"}
    # re-tiering of those segments with fresh scores (same tier fractions)
    del src
    nh_h, nm_h = nh.cpu().numpy(), nm.cpu().numpy()
    hs = torch.zeros(B, N, device=dev)
    ms = torch.zeros(B, N, device=dev)
    for b in range(B):
        hs[b, :nh_h[b]] = inputs.tier_scores(wl.seed + 1, b, int(nh_h[b]), tl, th).to(dev)
        ms[b, :nm_h[b]] = inputs.tier_scores(wl.seed + 2, b, int(nm_h[b]), tl, th).to(dev)
    h2 = lkv.Cache(D, wl.group_size, 6, 6, Hkv, B * nblk, device=dev)
    m2 = lkv.Cache(D, wl.group_size, 6, 4, Hkv, B * nblk, device=dev)
    nh2, nm2 = torch.zeros_like(nh), torch.zeros_like(nh)
    ht = torch.zeros((B, N), dtype=torch.uint8, device=dev)
    mt = torch.zeros((B, N), dtype=torch.uint8, device=dev)
    hv = lkv.View(bt, nh, int(nh_h.max()))
    mv = lkv.View(bt, nm, int(nm_h.max()))
    ws2 = torch.empty(lkv.retier_workspace_bytes(B, N, N), dtype=torch.uint8, device=dev)
    call = lambda: lkv.retier(hdst, hv, hs, mdst, mv, ms, tl, th, h2, bt, m2, bt, nh2, nm2, ht, mt, ws2)
    call()
    e0.record()
    call()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    n_h2, n_m2 = int(nh2.sum()), int(nm2.sum())
    nbytes = (n_h * 212 + n_m * 180) * Hkv + (n_h + n_m) * 5 + (n_h2 * 212 + n_m2 * 180) * Hkv + 8 * B
    retier = {"GB/s": round(nbytes / t / 1e9, 1), "us_per_call": round(t * 1e6, 1), "high": n_h2, "mid": n_m2,
              "evicted": n_h + n_m - n_h2 - n_m2,
              "counted": "HIGH/MID rows and their scores in, new HIGH/MID rows and tiers out"}
    # the same re-tier in place, each segment compacted within its own
    # blocks (one timed call: it consumes its input; an untimed one on
    # copies first, so that the in-place kernels are loaded and warm)
    hc = lkv.Cache(D, wl.group_size, 6, 6, Hkv, B * nblk, pool=hdst.pool.clone())
    mc = lkv.Cache(D, wl.group_size, 6, 4, Hkv, B * nblk, pool=mdst.pool.clone())
    nhc, nmc = torch.zeros_like(nh), torch.zeros_like(nh)
    htc, mtc = torch.zeros_like(ht), torch.zeros_like(mt)
    lkv.retier(hc, hv, hs, mc, mv, ms, tl, th, hc, bt, mc, bt, nhc, nmc, htc, mtc, ws2)
    torch.cuda.synchronize()
    del hc, mc
    e0.record()
    lkv.retier(hdst, hv, hs, mdst, mv, ms, tl, th, hdst, bt, mdst, bt, nh2, nm2, ht, mt, ws2)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    retier["in_place_us_per_call"] = round(t * 1e6, 1)
    retier["in_place_GB/s"] = round(nbytes / t / 1e9, 1)
    assert int(nh2.sum()) == n_h2 and int(nm2.sum()) == n_m2
    return tier, retier


def probe_figure(dev, gib=4, reps=20):
    """lkv_hbm_read_probe over a zero-filled buffer of `gib` GiB, plain and
    non-temporal loads, each timed with HIP events over `reps` launches after
    two untimed ones: the read bandwidth a streaming kernel reaches."""
    import torch

    from quantized_kv_cache_token_amd import lkv

    buf = torch.zeros(gib << 28, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {"bytes": buf.numel() * 4, "launches": reps}
    for nt in (False, True):
        for _ in range(2):
            lkv.hbm_read_probe(buf, sink, nt)
        e0, e1 = _event(), _event()
        e0.record()
        for _ in range(reps):
            lkv.hbm_read_probe(buf, sink, nt)
        e1.record()
        torch.cuda.synchronize()
        res["nt_GB/s" if nt else "GB/s"] = round(buf.numel() * 4 * reps / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)
    assert int(sink.item()) == 0
    del buf
    torch.cuda.empty_cache()
    return res


def serving_figure(wl, dev, every=32, tl_rel=0.35, th_rel=1.9):
    """The loop below, with Python's cycle collector off: a collection that
    falls between a re-tier's opening event and its launches would count as
    GPU time (such a pause once added 40 ms to one re-tier)."""
    import gc

    gc.collect()
    gc.disable()
    try:
        return _serving_loop(wl, dev, every, tl_rel, th_rel)
    finally:
        gc.enable()


def _serving_loop(wl, dev, every, tl_rel, th_rel):
    """The tiered serving loop at the ragged workload's shape: the cache is
    prefilled at K6V6 (all HIGH); each step appends one row per sequence to
    HIGH and decodes over HIGH + MID with the sparse-V skip, accumulating
    every token's weight (lkv_decode_attn_scores); every `every` steps the
    segments are re-tiered in place (lkv_retier with each destination its
    own source) on the weights scaled per sequence to weight x live tokens
    (1 = the uniform weight; tl_rel, th_rel on that scale).  Blocks come from
    host free lists: HIGH blocks for the epoch's appends beforehand, MID rows
    grown for every HIGH token before a re-tier, and the blocks past each new
    length returned after it.  GPU time from HIP events around each epoch's
    steps and around each re-tier; the wall time includes the host's block
    bookkeeping and the synchronisation that reads the new counts."""
    import numpy as np
    import torch

    from quantized_kv_cache_token_amd import inputs, lkv

    B, Hq, Hkv, D = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    steps = wl.steps
    blocks = lambda n: -(-int(n) // 64)
    lens = inputs.ragged_lengths(wl.seed, B, *wl.ragged).numpy().astype(np.int64)
    width = blocks(lens.max() + steps) + 1
    nh_pool = int(sum(blocks(n) for n in lens)) + B * (blocks(steps) + 1)
    nm_pool = int(sum(blocks(n + steps) for n in lens)) + B
    h = lkv.Cache(D, wl.group_size, 6, 6, Hkv, nh_pool, device=dev)
    m = lkv.Cache(D, wl.group_size, 6, 4, Hkv, nm_pool, device=dev)
    free_h, free_m = list(range(nh_pool - 1, -1, -1)), list(range(nm_pool - 1, -1, -1))
    hbt = np.zeros((B, width), np.int32)
    mbt = np.zeros((B, width), np.int32)
    for b in range(B):
        for i in range(blocks(lens[b])):
            hbt[b, i] = free_h.pop()
    hb, mb = torch.tensor(hbt, device=dev), torch.tensor(mbt, device=dev)
    outl = inputs.outlier_channels(wl.seed, Hkv, D)
    for b in range(B):
        k, v = inputs.kv_rows(wl.seed, b, int(lens[b]), Hkv, D, dtype=wl.dtype, outliers=outl, device=dev)
        lkv.quant_append(h, k, v, torch.tensor([0, int(lens[b])], dtype=torch.int32, device=dev),
                         torch.zeros(1, dtype=torch.int32, device=dev), hb[b:b + 1].contiguous(), int(lens[b]))
        del k, v
    hl, ml = lens.astype(np.int32), np.zeros(B, np.int32)
    stride = int(lens.max()) + steps + 64
    acc = torch.zeros((2, B, stride), dtype=torch.float32, device=dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    cu1 = torch.arange(B + 1, dtype=torch.int32, device=dev)
    sm = float(np.float32(1.0 / np.sqrt(D)))
    tau = lkv.default_thresholds(int(lens.max()))[0]
    rows = [inputs.kv_rows(wl.seed, 7000, B, Hkv, D, dtype=wl.dtype, outliers=outl, step=s + 1, device=dev)
            for s in range(every)]
    qs = [inputs.queries(wl.seed, B, Hq, D, dtype=wl.dtype, step=s, device=dev) for s in range(every)]
    n_high = torch.zeros(B, dtype=torch.int32, device=dev)
    n_mid = torch.zeros_like(n_high)
    torch.cuda.synchronize()
    step_ms, retier_ms, live, growth, recycled = [], [], [], [], 0
    freed_h, freed_m = set(), set()
    t0 = time.perf_counter()
    done = 0
    while done < steps:
        n = min(every, steps - done)
        for b in range(B):  # HIGH blocks for this epoch's rows
            for i in range(blocks(hl[b]), blocks(hl[b] + n)):
                hbt[b, i] = free_h.pop()
                recycled += int(hbt[b, i]) in freed_h
        hb.copy_(torch.from_numpy(hbt))
        pos = [torch.tensor(hl + s, device=dev) for s in range(n)]
        hlen = [torch.tensor(hl + s + 1, device=dev) for s in range(n)]
        mlen = torch.tensor(ml, device=dev)
        views = [[lkv.View(hb, hlen[s], int(hl.max()) + s + 1, int(hl.sum()) + B * (s + 1)),
                  lkv.View(mb, mlen, max(int(ml.max()), 1), int(ml.sum()))] for s in range(n)]
        split = lkv.decode_plan([h, m], views[-1], B, Hq)
        ws = lkv.decode_scores_workspace([h, m], views[-1], B, Hq, split, dev)
        calls = []
        for s in range(n):
            k, v = rows[s]
            calls.append(lkv.prepare_append(h, k, v, cu1, pos[s], hb, 1))
            calls.append(lkv.prepare_decode_scores([h, m], views[s], qs[s], sm, tau, split, out, acc, ws))
        e0, e1, e2 = _event(), _event(), _event()
        e0.record()
        for c in calls:
            c()
        e1.record()
        hl = hl + n
        done += n
        # re-tier in place on the epoch's weights
        scale = torch.tensor((hl + ml).astype(np.float64) / (n * Hq), dtype=torch.float32, device=dev)
        rel = acc * scale[None, :, None]
        hs = rel[0, :, :max(int(hl.max()), 1)].contiguous()
        ms = rel[1, :, :max(int(ml.max()), 1)].contiguous()
        grown = 0
        for b in range(B):
            for i in range(blocks(ml[b]), blocks(ml[b] + hl[b])):
                mbt[b, i] = free_m.pop()
                recycled += int(mbt[b, i]) in freed_m
                grown += 1
        mb.copy_(torch.from_numpy(mbt))
        ht = torch.empty(hs.shape, dtype=torch.uint8, device=dev)
        mt = torch.empty(ms.shape, dtype=torch.uint8, device=dev)
        hv = lkv.View(hb, torch.tensor(hl, device=dev), int(hl.max()))
        mv = lkv.View(mb, torch.tensor(ml, device=dev), max(int(ml.max()), 1))
        ws2 = torch.empty(lkv.retier_workspace_bytes(B, hs.shape[1], ms.shape[1]), dtype=torch.uint8, device=dev)
        e1b = _event()
        e1b.record()
        lkv.retier(h, hv, hs, m, mv, ms, tl_rel, th_rel, h, hb, m, mb, n_high, n_mid, ht, mt, ws2)
        e2.record()
        nh, nm = n_high.cpu().numpy(), n_mid.cpu().numpy()  # synchronises
        if (nh < 0).any() or (nm < 0).any():
            raise RuntimeError("serving loop: a re-tier found no room")
        step_ms.append(e0.elapsed_time(e1) / n)
        retier_ms.append(e1b.elapsed_time(e2))
        live.append(int(hl.sum() + ml.sum()))
        growth.append(grown)
        for b in range(B):
            for blk in hbt[b, blocks(nh[b]):blocks(hl[b])]:
                free_h.append(int(blk))
                freed_h.add(int(blk))
            for blk in mbt[b, blocks(nm[b]):blocks(ml[b] + hl[b])]:
                free_m.append(int(blk))
                freed_m.add(int(blk))
        hl, ml = nh.astype(np.int32), nm.astype(np.int32)
        acc.zero_()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = (sum(x * every for x in step_ms[:-1]) + step_ms[-1] * (steps - every * (len(step_ms) - 1)) +
             sum(retier_ms)) / 1e3
    return {"workload": wl.name + "_tiered", "steps": steps, "retier_every": every, "retier_in_place": True,
            "tau_rel": [tl_rel, th_rel], "tau_skip": tau,
            "decode_step_us": [round(x * 1e3, 1) for x in step_ms],
            "retier_us": [round(x * 1e3, 1) for x in retier_ms],
            "tokens_per_s_gpu": round(B * steps / gpu_s, 1), "tokens_per_s_wall": round(B * steps / wall, 1),
            "live_tokens_at_retier": live, "final_high_mid": [int(hl.sum()), int(ml.sum())],
            "mid_blocks_grown_per_retier": growth, "recycled_blocks_taken": recycled,
            "blocks_in_use_after": [nh_pool - len(free_h), nm_pool - len(free_m)],
            "pool_blocks": [nh_pool, nm_pool],
            "timing": "hip events around each epoch's append+decode launches and each re-tier; wall includes "
                      "host block bookkeeping and the count read-back"}


def cpu_baseline(wl, kb, vb, nseq, per_token_head, q_bytes, min_seconds):
    """The oracle, as it stands, on a bounded sample of the same workload:
    `nseq` sequences with all their query heads; one step appends one row per
    sequence and decodes over N tokens.  Steps repeat until `min_seconds` have
    passed.  GB/s over the same counted bytes as the GPU line."""
    import numpy as np

    from oracle import oracle as O
    from quantized_kv_cache_token_amd import inputs

    B, Hq, Hkv, D, N = nseq, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.n_ctx
    nblk = (N + 63) // 64
    outl = inputs.outlier_channels(wl.seed, Hkv, D) if wl.outliers else None
    cache = O.Cache(D, wl.group_size, kb, vb, Hkv, B * nblk)
    bt = np.arange(B * nblk, dtype=np.int32).reshape(B, nblk)
    for b in range(B):
        k, v = inputs.kv_rows(wl.seed, b, N - 1, Hkv, D, dtype=wl.dtype, outliers=outl)
        O.append(cache, k.float().numpy(), v.float().numpy(), [0, N - 1], [0], bt[b:b + 1])
    k, v = inputs.kv_rows(wl.seed, 1000, B, Hkv, D, dtype=wl.dtype, outliers=outl, step=1)
    k, v = k.float().numpy(), v.float().numpy()
    q = inputs.queries(wl.seed, B, Hq, D, dtype=wl.dtype).float().numpy()
    sm = float(np.float32(1.0 / np.sqrt(D)))
    cu, last, lens = np.arange(B + 1), np.full(B, N - 1), np.full(B, N, np.int32)
    steps = 0
    t0 = time.perf_counter()
    while True:
        O.append(cache, k, v, cu, last, bt)
        O.decode([cache], [bt], [lens], q, sm, 0.0, 0)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    nbytes = B * Hkv * N * per_token_head + B * Hq * D * (q_bytes + 4) + B * Hkv * (2 * D * q_bytes + per_token_head)
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(steps * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": O.num_threads(),
            "kind": "oracle", "cpu_model": model, "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"{B} of {wl.batch} sequences, all {Hq} query heads; {steps} steps of (append 1 row per "
                      f"sequence + fp64 decode over {N} tokens) in {dt:.2f} s"}


if __name__ == "__main__":
    main()
