"""Pins of the oracle's multi-token queries (T query tokens per sequence
with a causal mask over the packed cache; the attention that FlashAttention-
style kernels compute, which the TurboQuant page states the cache is
compatible with).  CPU only."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from tests import np_reference as R
from tests.oracle_cases import build_cache


def _case(seed, lens, Hkv, D, g, kb, vb, G, T):
    rng = np.random.default_rng(seed)
    K = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    V = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    cache, bt, lens = build_cache(K, V, D, g, kb, vb, rng=rng)
    q = rng.standard_normal((len(lens), T, Hkv * G, D)).astype(np.float32)
    return cache, bt, lens, q


@pytest.mark.parametrize("fmt,G,T", [((128, 64, 6, 4), 4, 3), ((64, 32, 6, 6), 1, 5), ((64, 16, 16, 16), 2, 2)])
def test_multi_matches_numpy_causal_attention(fmt, G, T):
    """Every query token equals brute-force softmax attention over the
    dequantised prefix up to its own position (independent unpacking)."""
    D, g, kb, vb = fmt
    Hkv = 2
    cache, bt, lens, q = _case(11, [T, 70, 130], Hkv, D, g, kb, vb, G, T)
    sm = float(np.float32(1 / math.sqrt(D)))
    got = O.decode_multi([cache], [bt], [lens], q, sm)
    for b, n in enumerate(lens):
        Kh, Vh = R.dequant_sequence(cache.pool, cache.chunk_bytes, Hkv, D, g, kb, vb, bt[b], n)
        for i in range(T):
            p = n - T + i + 1
            want = R.attention(q[b, i], Kh[:, :p], Vh[:, :p], sm)
            assert np.allclose(got[b, i], want, rtol=1e-12, atol=1e-13)


def test_single_query_is_decode():
    cache, bt, lens, q = _case(12, [1, 64, 300], 2, 128, 64, 6, 4, 4, 1)
    for tau, split in [(0.0, 0), (1e-3, 128)]:
        a = O.decode_multi([cache], [bt], [lens], q, 0.09, tau, split)
        b = O.decode([cache], [bt], [lens], q[:, 0], 0.09, tau, split)
        assert np.array_equal(a[:, 0], b)


def test_last_query_sees_everything_and_later_tokens_are_invisible():
    """Query T-1 is plain decode over the whole sequence; changing the
    cached rows of the newest token leaves every earlier query unchanged,
    bit for bit."""
    T, Hkv, D, g, G = 4, 1, 64, 32, 4
    cache, bt, lens, q = _case(13, [90, 129], Hkv, D, g, 6, 4, G, T)
    sm = 0.125
    a = O.decode_multi([cache], [bt], [lens], q, sm, 1e-4, 64)
    full = O.decode([cache], [bt], [lens], q[:, T - 1], sm, 1e-4, 64)
    assert np.array_equal(a[:, T - 1], full)
    # overwrite each sequence's newest token with other rows
    rng = np.random.default_rng(14)
    k = rng.standard_normal((2, Hkv, D)).astype(np.float32) * 5
    O.append(cache, k, -k, [0, 1, 2], [n - 1 for n in lens], bt)
    b2 = O.decode_multi([cache], [bt], [lens], q, sm, 1e-4, 64)
    assert np.array_equal(a[:, :T - 1], b2[:, :T - 1])
    assert not np.array_equal(a[:, T - 1], b2[:, T - 1])


def test_two_segments_mask_only_the_first():
    """With tiered segments the new tokens are the tail of the first one;
    every token of the second precedes them."""
    T, Hkv, D, g, G = 3, 2, 128, 64, 4
    rng = np.random.default_rng(15)
    lh, lm = [5, 64], [40, 1]
    Kh = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lh]
    Vh = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lh]
    Km = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lm]
    Vm = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lm]
    ch, bth, lh = build_cache(Kh, Vh, D, g, 6, 6, rng=rng)
    cm, btm, lm = build_cache(Km, Vm, D, g, 6, 4, rng=rng)
    q = rng.standard_normal((2, T, Hkv * G, D)).astype(np.float32)
    sm = float(np.float32(0.088))  # the oracle takes the scale as fp32
    got = O.decode_multi([ch, cm], [bth, btm], [lh, lm], q, sm)
    for b in range(2):
        K1, V1 = R.dequant_sequence(ch.pool, ch.chunk_bytes, Hkv, D, g, 6, 6, bth[b], lh[b])
        K2, V2 = R.dequant_sequence(cm.pool, cm.chunk_bytes, Hkv, D, g, 6, 4, btm[b], lm[b])
        for i in range(T):
            p = lh[b] - T + i + 1
            K = np.concatenate([K1[:, :p], K2], axis=1)
            V = np.concatenate([V1[:, :p], V2], axis=1)
            assert np.allclose(got[b, i], R.attention(q[b, i], K, V, sm), rtol=1e-12, atol=1e-13)


def test_multi_rejects_sequences_shorter_than_their_queries():
    cache, bt, lens, q = _case(16, [2, 10], 1, 64, 32, 6, 4, 1, 3)
    with pytest.raises(ValueError):
        O.decode_multi([cache], [bt], [lens], q, 0.1)
