"""Helpers of the GPU parity tests: run the same seeded inputs through the
HIP path (C ABI) and through the oracle, and compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import oracle as O
from quantized_kv_cache_token_amd import lkv
from tests import np_reference as R

BT = 64


def say(*a):
    """Name the case before each GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def max_abs_vhat(cache: O.Cache, batch: int = 256) -> float:
    """max |v_hat| over every slot of a host pool (unwritten slots are 0),
    taken over batches of chunks so that large pools stay cheap."""
    D, g, vb = cache.head_dim, cache.group_size, cache.v_bits
    off = cache.layout
    ch_all = cache.pool.reshape(-1, cache.chunk_bytes)
    vbytes = D * BT * vb // 8
    ng = D // g
    gi = np.arange(D) // g
    best = 0.0
    for c0 in range(0, ch_all.shape[0], batch):
        ch = ch_all[c0:c0 + batch]
        bits = np.unpackbits(ch[:, off[1]:off[1] + vbytes], axis=1, bitorder="little")
        bits = bits.reshape(ch.shape[0], D * BT, vb).astype(np.uint32)
        codes = (bits << np.arange(vb, dtype=np.uint32)).sum(-1).reshape(ch.shape[0], D, BT)
        if vb == 16:
            vals = codes.astype(np.uint16).view(np.float16).astype(np.float64)
        else:
            s = ch[:, off[3]:off[3] + ng * BT * 4].copy().view(np.float32).reshape(-1, ng, BT).astype(np.float64)
            z = ch[:, off[5]:off[5] + ng * BT].reshape(-1, ng, BT).astype(np.float64)
            vals = (codes - z[:, gi, :]) * s[:, gi, :]
        best = max(best, float(np.abs(vals).max()))
    return best


def max_abs_vhat_live(cache: O.Cache, block_table, lens) -> float:
    """max |v_hat| over the live tokens of a host pool only (pools that hold
    stale bytes in other slots), read with the independent numpy unpacking."""
    from tests import np_reference as R

    best = 0.0
    for b, n in enumerate(np.asarray(lens)):
        if int(n) <= 0:
            continue
        _, V = R.dequant_sequence(cache.pool, cache.chunk_bytes, cache.num_kv_heads, cache.head_dim,
                                  cache.group_size, cache.k_bits, cache.v_bits, np.asarray(block_table)[b], int(n))
        best = max(best, float(np.abs(V).max()))
    return best


def assert_attention_close(got: np.ndarray, want: np.ndarray, vmax: float, what: str = ""):
    """max|d| <= 1e-3 max|v_hat| and ||d||_2 / ||want||_2 <= 1e-4."""
    got = np.asarray(got, np.float64)
    d = got - want
    maxd = float(np.abs(d).max()) if d.size else 0.0
    nrm = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(d)) / nrm if nrm > 0 else float(np.linalg.norm(d))
    assert np.all(np.isfinite(got)), what
    assert maxd <= 1e-3 * vmax, f"{what}: max|d| {maxd:.3e} > 1e-3 * {vmax:.3e}"
    assert rel <= 1e-4, f"{what}: rel L2 {rel:.3e}"
    return maxd, rel


def to_f32_host(t: torch.Tensor) -> np.ndarray:
    """Exact widening of fp32/bf16/fp16 tensors to fp32 numpy."""
    return t.detach().to("cpu").to(torch.float32).numpy()


class Pair:
    """A GPU cache and an oracle cache with the same format and block table."""

    def __init__(self, D, g, kb, vb, Hkv, num_blocks):
        self.gpu = lkv.Cache(D, g, kb, vb, Hkv, num_blocks)
        self.ref = O.Cache(D, g, kb, vb, Hkv, num_blocks)

    def append(self, k: torch.Tensor, v: torch.Tensor, cu_new, start_pos, block_table: np.ndarray):
        cu = torch.tensor(np.asarray(cu_new), dtype=torch.int32)
        sp = torch.tensor(np.asarray(start_pos), dtype=torch.int32)
        bt = torch.tensor(np.asarray(block_table), dtype=torch.int32)
        max_new = int((cu[1:] - cu[:-1]).max()) if len(cu) > 1 else 0
        lkv.quant_append(self.gpu, k.cuda().contiguous(), v.cuda().contiguous(), cu.cuda(), sp.cuda(), bt.cuda(),
                         max_new)
        O.append(self.ref, to_f32_host(k), to_f32_host(v), cu.numpy(), sp.numpy(), bt.numpy())

    def pool_equal(self) -> bool:
        torch.cuda.synchronize()
        return np.array_equal(self.gpu.pool.cpu().numpy(), self.ref.pool)

    def first_pool_mismatch(self):
        g = self.gpu.pool.cpu().numpy()
        bad = np.nonzero(g != self.ref.pool)[0]
        if bad.size == 0:
            return None
        i = int(bad[0])
        chunk, off = divmod(i, self.ref.chunk_bytes)
        return dict(count=int(bad.size), chunk=chunk, offset=off, gpu=int(g[i]), ref=int(self.ref.pool[i]),
                    layout=self.ref.layout)


def sm_scale(D: int) -> float:
    return float(np.float32(1.0 / math.sqrt(D)))


# Relative band of the sparse-V skip decisions that may go either way: the
# GPU evaluates exp(s - m) and tau_low * L in fp32, where a score carries a
# relative error of order 1e-5 of its terms (bf16-exact products, fp32
# accumulation over 128 channels against an offset of 128 per code) and L
# one of order n * 2^-24; pairs whose exact margin is within 2^-10 of the
# bound are taken as the GPU decides.
SKIP_BAND = 2.0 ** -10


def mask_to_given(mask: torch.Tensor, max_lens, max_tok: int) -> np.ndarray:
    """GPU skip mask int32 [E][Hq][words] -> the oracle's layout uint8
    [E][Hq][nseg][max_tok] (segment s's columns start at the sum of the
    earlier segments' max_len rounded up to 64)."""
    m = mask.cpu().numpy()
    bits = np.unpackbits(m.view(np.uint8), axis=-1, bitorder="little")
    E, Hq = m.shape[:2]
    given = np.zeros((E, Hq, len(max_lens), max_tok), np.uint8)
    col = 0
    for s, ml in enumerate(max_lens):
        given[:, :, s, :ml] = bits[:, :, col:col + ml]
        assert not bits[:, :, col + ml:col + -(-ml // BT) * BT].any(), "mask bits past max_len"
        col += -(-ml // BT) * BT
    return given


def resolved_reference(ref_caches, ref_bts, ref_lens, q_host: np.ndarray, sm: float, tau: float, split: int,
                       mask: torch.Tensor, max_lens, what: str = ""):
    """The oracle's decode with the GPU's skip decisions taken inside
    SKIP_BAND; every decision outside the band must equal the exact one, bit
    for bit, and no column without a live token may be marked.  Returns the
    oracle output and (live pairs, pairs whose GPU decision differs from the
    exact one, the largest relative margin among those)."""
    max_tok = max(np.asarray(bt).shape[1] for bt in ref_bts) * BT
    given = mask_to_given(mask, max_lens, max_tok)
    out, skip, amb, margin = O.decode_resolved(ref_caches, ref_bts, ref_lens, q_host, sm, tau, split, given,
                                               SKIP_BAND)
    E, Hq = given.shape[:2]
    live = np.zeros(given.shape, bool)
    for s, ln in enumerate(ref_lens):
        ln = np.asarray(ln)
        for e in range(E):
            live[e, :, s, :int(ln[e])] = True
    assert not (given.astype(bool) & ~live).any(), f"{what}: skip bits on columns without a live token"
    bad = (given != skip) & live
    assert not bad.any(), (f"{what}: {int(bad.sum())} skip decisions differ outside the band; relative margins "
                           f"{margin[bad][:8]}")
    flips = live & (given.astype(bool) != (margin < 0)) if tau > 0 else np.zeros_like(live)
    worst = float(np.abs(margin[flips]).max()) if flips.any() else 0.0
    return out, (int(live.sum()), int(flips.sum()), worst)
