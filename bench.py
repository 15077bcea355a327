"""Decode-step benchmark of the packed K6/V4 KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

A step is one pass of the hot path for one layer: quantise-and-append the
new token of every sequence (lkv_quant_append), then split-K decode
attention of one query per sequence over the whole packed cache
(lkv_decode_split + lkv_decode_combine, i.e. lkv_decode_attn).  Steps rotate
over several layer caches so that consecutive steps stream from HBM, not
from the 256 MB last-level cache.  Every step re-appends the row of the last
position and attends over all N positions, the same work as the step that
brings the context to N tokens.

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
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--workload", type=int, default=2, choices=[2, 4])
    p.add_argument("--layers", type=int, default=4, help="layer caches rotated over (HBM, not cache)")
    p.add_argument("--split-tokens", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seqs", type=int, default=8, help="sequences in the oracle's timed sample")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="least oracle time in the CPU baseline")
    p.add_argument("--copy-probe", action="store_true",
                   help="after the timed steps, stream 1 GiB in and 1 GiB out (counter scaling reference)")
    p.add_argument("--fp16-layer", action="store_true", help="time the fp16 sensitive-layer format")
    p.add_argument("--no-tier", action="store_true", help="skip the tier-update secondary figure")
    return p.parse_args()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    from quantized_kv_cache_token_amd.profsum import kernel_source_hash

    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the kernel runs on one GPU's share; see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_kv_cache_token_amd import inputs, lkv, workloads

    wl = workloads.BY_INDEX[args.workload]
    if args.fp16_layer:
        kb, vb = 16, 16
    else:
        kb, vb = wl.k_bits, wl.v_bits
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    B, Hq, Hkv, D, N = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.n_ctx
    nblk = (N + 63) // 64
    bt = torch.arange(B * nblk, dtype=torch.int32, device=dev).view(B, nblk)
    lens = torch.full((B,), N, dtype=torch.int32, device=dev)
    outl = inputs.outlier_channels(wl.seed, Hkv, D) if wl.outliers else None

    # ---- layer caches, filled by the append kernel (prefill; each call timed
    # with events for the secondary figures, outside the timed steps)
    caches = []
    prefill_ms = []
    for layer in range(args.layers):
        c = lkv.Cache(D, wl.group_size, kb, vb, Hkv, B * nblk, device=dev)
        for b in range(B):
            k, v = inputs.kv_rows(wl.seed, b, N - 1, Hkv, D, dtype=wl.dtype, outliers=outl, layer=layer,
                                  device=dev)
            cu = torch.tensor([0, N - 1], dtype=torch.int32, device=dev)
            sp0 = torch.zeros(1, dtype=torch.int32, device=dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            lkv.quant_append(c, k, v, cu, sp0, bt[b:b + 1], N - 1)
            e1.record()
            prefill_ms.append((e0, e1))
            del k, v
        caches.append(c)
    torch.cuda.synchronize()
    prefill_ms = [a.elapsed_time(b) for a, b in prefill_ms]
    chunk = caches[0].chunk_bytes
    view = lkv.View(bt, lens, N)

    # ---- per-step inputs: the new token's K/V and the query, per layer
    new_k, new_v, qs = [], [], []
    for layer in range(args.layers):
        k, v = inputs.kv_rows(wl.seed, 1000, B, Hkv, D, dtype=wl.dtype, outliers=outl, layer=layer, step=1,
                              device=dev)
        new_k.append(k.contiguous())
        new_v.append(v.contiguous())
        qs.append(inputs.queries(wl.seed, B, Hq, D, dtype=wl.dtype, layer=layer, device=dev))
    cu1 = torch.arange(B + 1, dtype=torch.int32, device=dev)
    last = torch.full((B,), N - 1, dtype=torch.int32, device=dev)
    sm = float(np.float32(1.0 / np.sqrt(D)))
    split = args.split_tokens or lkv.decode_plan([caches[0]], [view], B, Hq)
    ws = lkv.decode_workspace([caches[0]], [view], B, Hq, split, dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)

    # pre-marshalled calls (one set per layer cache)
    calls = []
    for layer in range(args.layers):
        app = lkv.prepare_append(caches[layer], new_k[layer], new_v[layer], cu1, last, bt, 1)
        spl, comb = lkv.prepare_decode([caches[layer]], [view], qs[layer], sm, 0.0, split, out, ws)
        calls.append((app, spl, comb))

    def step(i, ev=None):
        app, spl, comb = calls[i % args.layers]
        app()
        if ev is not None:
            ev[0].record()
        spl()
        if ev is not None:
            ev[1].record()
        comb()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # HIP events bracket the split kernel on one step of every rotation
    # cycle (an event between kernels adds a small gap to that step only)
    timed = [i for i in range(args.steps) if i % args.layers == 0]
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in timed}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if args.copy_probe:
        # a plain streaming kernel of known traffic: reads 1 GiB, writes 1 GiB
        src = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    step_s = (t1 - t0) / args.steps
    split_ms = [a.elapsed_time(b) for a, b in evs.values()]
    split_s = float(np.mean(split_ms)) / 1e3

    per_token_head = chunk // 64
    q_bytes = 2 if wl.dtype == "bf16" else 4
    kv_bytes = B * Hkv * N * per_token_head
    decode_bytes = kv_bytes + B * Hq * D * q_bytes + B * Hq * D * 4
    append_bytes = B * Hkv * (2 * D * q_bytes + per_token_head)
    step_bytes = decode_bytes + append_bytes
    value = step_bytes / step_s / 1e9
    split_alg = kv_bytes + B * Hq * D * q_bytes
    achieved = split_alg / split_s / 1e9
    kname = "decode_split"
    wname = wl.name if not args.fp16_layer else wl.name.replace("k6v4", "fp16")
    traffic = measured_traffic(kname, wname)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wname, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "ctx_tokens": N, "group_size": wl.group_size, "k_bits": kb, "v_bits": vb,
                   "q_dtype": wl.dtype, "split_tokens": split, "layers_rotated": args.layers},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(B / step_s, 1),
        "bytes_per_step": step_bytes,
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": split_alg,
                     "avg_launch_us": round(split_s * 1e6, 2)},
    }
    in_bytes = 2 if wl.dtype in ("bf16", "f16") else 4
    pre_bytes = (N - 1) * Hkv * (2 * D * in_bytes + per_token_head)
    pre_s = float(np.median(prefill_ms)) / 1e3
    rec["secondary"] = {
        "append_prefill": {"GB/s": round(pre_bytes / pre_s / 1e9, 1), "us_per_call": round(pre_s * 1e6, 1),
                           "rows_per_call": N - 1, "counted": "bf16 K/V rows in + packed rows out"},
    }
    if not args.fp16_layer and not args.no_tier:
        del caches, calls
        torch.cuda.empty_cache()
        rec["secondary"]["tier_update"] = tier_figure(wl, dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, kb, vb, min(args.cpu_seqs, B), per_token_head, q_bytes,
                                           args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def tier_figure(wl, dev):
    """One lkv_tier_update at the tiered workload's shape (the batch and
    context of `wl`, K6V6 source, scores with 10% high / 30% mid / 60% low),
    timed with events after one untimed call.  Counted bytes: source rows and
    scores read, survivors' rows, tiers and counts written."""
    import numpy as np
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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    call()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    n_h, n_m = int(nh.sum()), int(nm.sum())
    nbytes = B * N * Hkv * 212 + B * N * 4 + (n_h * 212 + n_m * 180) * Hkv + B * N + 8 * B
    return {"GB/s": round(nbytes / t / 1e9, 1), "us_per_call": round(t * 1e6, 1), "high": n_h, "mid": n_m,
            "evicted": B * N - n_h - n_m, "counted": "K6V6 rows and scores in, HIGH/MID rows and tiers out"}


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
    return {"value": round(steps * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"{B} of {wl.batch} sequences, all {Hq} query heads; {steps} steps of (append 1 row per "
                      f"sequence + fp64 decode over {N} tokens) in {dt:.2f} s"}


if __name__ == "__main__":
    main()
