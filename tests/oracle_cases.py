"""Small host-side cases built with the oracle (test helpers, CPU only)."""
from __future__ import annotations

import numpy as np

from oracle import oracle as O

BT = 64


def block_tables(lens, rng=None, extra_blocks=0):
    """Block table [B][max_blocks] and pool size; blocks handed out in a
    random order when rng is given, else contiguously."""
    nblk = [-(-int(n) // BT) for n in lens]
    max_blocks = max(max(nblk), 1) + extra_blocks
    total = sum(nblk) + 1
    order = rng.permutation(total) if rng is not None else np.arange(total)
    bt = np.zeros((len(lens), max_blocks), np.int32)
    at = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = order[at:at + n]
        at += n
    return bt, total


def build_cache(K, V, D, g, kb, vb, rng=None, lens=None, k_norm=0):
    """Append per-sequence rows K[b], V[b] (fp32 [n_b][Hkv][D]) into a fresh
    oracle cache.  Returns (cache, block_table, lens)."""
    B = len(K)
    Hkv = K[0].shape[1]
    lens = np.array([k.shape[0] for k in K], np.int32) if lens is None else np.asarray(lens, np.int32)
    bt, total = block_tables(lens, rng)
    cache = O.Cache(D, g, kb, vb, Hkv, total, k_norm=k_norm)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    O.append(cache, np.concatenate(K), np.concatenate(V), cu, np.zeros(B, np.int32), bt)
    return cache, bt, lens
