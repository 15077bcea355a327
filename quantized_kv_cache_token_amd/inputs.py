"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and shapes them like the workloads the
pages describe; it holds none of the method's arithmetic (no quantisation,
packing, attention or tiering), so both the HIP path and the oracle can
consume its arrays.

Recipe:
  * every stream has its own torch generator, seeded from the workload seed
    and a tuple of integer keys (stream id, sequence, layer, step), so any
    single sequence can be regenerated on its own;
  * values are drawn as fp32 N(0, 1) and rounded once (round to nearest even)
    to the workload dtype;
  * K outlier channels: for each KV head the first 4 entries of a seeded
    permutation of the head_dim channels are multiplied by 12 in fp32 before
    the rounding;
  * tier scores: a fixed count of high (10%), mid (30%) and low (60%) tokens
    placed by a seeded permutation, with values uniform in [tau_high,
    2 tau_high), [tau_low, tau_high) and [0, tau_low);
  * ragged lengths: uniform integers in [lo, hi];
  * paged pools: blocks handed out in the order of a seeded permutation.
"""
from __future__ import annotations

import torch

# stream ids
K_STREAM, V_STREAM, Q_STREAM, OUTLIER_STREAM, SCORE_STREAM, LEN_STREAM, PERM_STREAM = range(1, 8)

_MIX = 1_000_003
_MASK = (1 << 63) - 1

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def seed_of(base: int, *keys: int) -> int:
    s = base & _MASK
    for k in keys:
        s = (s * _MIX + (k & 0xFFFFFFFF) + 1) & _MASK
    return s


def generator(base: int, *keys: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(base, *keys))
    return g


def normal(shape, base: int, *keys: int, dtype="bf16", device="cpu") -> torch.Tensor:
    """fp32 N(0,1) draws rounded once to `dtype`."""
    g = generator(base, *keys, device=device)
    x = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    return x.to(DTYPES[dtype])


def outlier_channels(base: int, num_kv_heads: int, head_dim: int, count: int = 4) -> torch.Tensor:
    """int64 [Hkv][count]: the outlier channels of each KV head."""
    rows = []
    for h in range(num_kv_heads):
        g = generator(base, OUTLIER_STREAM, h)
        rows.append(torch.randperm(head_dim, generator=g)[:count])
    return torch.stack(rows)


def kv_rows(base: int, seq: int, n_tokens: int, num_kv_heads: int, head_dim: int,
            dtype="bf16", outliers: torch.Tensor | None = None, outlier_gain: float = 12.0,
            layer: int = 0, step: int = 0, device="cpu"):
    """K and V rows [n_tokens][Hkv][D] of one sequence, in `dtype`.

    `step` distinguishes rows appended at different decode steps."""
    shape = (n_tokens, num_kv_heads, head_dim)
    gk = generator(base, K_STREAM, seq, layer, step, device=device)
    gv = generator(base, V_STREAM, seq, layer, step, device=device)
    k = torch.randn(*shape, generator=gk, dtype=torch.float32, device=device)
    v = torch.randn(*shape, generator=gv, dtype=torch.float32, device=device)
    if outliers is not None:
        gain = torch.ones(num_kv_heads, head_dim, dtype=torch.float32)
        for h in range(num_kv_heads):
            gain[h, outliers[h]] = outlier_gain
        k = k * gain.to(device)
    return k.to(DTYPES[dtype]), v.to(DTYPES[dtype])


def queries(base: int, batch: int, num_q_heads: int, head_dim: int, dtype="bf16",
            layer: int = 0, step: int = 0, device="cpu") -> torch.Tensor:
    g = generator(base, Q_STREAM, layer, step, device=device)
    x = torch.randn(batch, num_q_heads, head_dim, generator=g, dtype=torch.float32, device=device)
    return x.to(DTYPES[dtype])


def tier_scores(base: int, seq: int, n_tokens: int, tau_low: float, tau_high: float,
                frac_high: float = 0.1, frac_mid: float = 0.3) -> torch.Tensor:
    """fp32 [n_tokens] accumulated attention scores with fixed tier fractions."""
    g = generator(base, SCORE_STREAM, seq)
    n_h = int(round(frac_high * n_tokens))
    n_m = int(round(frac_mid * n_tokens))
    n_l = n_tokens - n_h - n_m
    if n_l < 0:
        raise ValueError("frac_high + frac_mid must not exceed 1")
    u = torch.rand(n_tokens, generator=g, dtype=torch.float32)
    lo = torch.empty(n_tokens, dtype=torch.float32)
    width = torch.empty(n_tokens, dtype=torch.float32)
    lo[:n_h], width[:n_h] = tau_high, tau_high
    lo[n_h:n_h + n_m], width[n_h:n_h + n_m] = tau_low, tau_high - tau_low
    lo[n_h + n_m:], width[n_h + n_m:] = 0.0, tau_low
    vals = lo + u * width
    perm = torch.randperm(n_tokens, generator=g)
    out = torch.empty(n_tokens, dtype=torch.float32)
    out[perm] = vals
    return out


def ragged_lengths(base: int, batch: int, lo: int, hi: int) -> torch.Tensor:
    g = generator(base, LEN_STREAM)
    return torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64).to(torch.int32)


def block_permutation(base: int, num_blocks: int) -> torch.Tensor:
    g = generator(base, PERM_STREAM)
    return torch.randperm(num_blocks, generator=g).to(torch.int32)
