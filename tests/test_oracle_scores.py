"""Pins of the oracle's accumulated attention scores (the per-token signal of
the attention-aware tiers, Super KV Compression page, second layer): the
softmax weight of every live token, summed over the query heads, added to
score_acc[segment][b][token]."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from tests import np_reference as R
from tests.oracle_cases import build_cache


def _rand_kv(rng, lens, Hkv, D):
    K = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    V = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    return K, V


def _numpy_scores(cache, bt, lens, q, sm, fmt):
    """Sum over heads of numpy softmax weights, [B][max(lens)]."""
    D, g, kb, vb = fmt
    Hq = q.shape[1]
    Hkv = cache.num_kv_heads
    G = Hq // Hkv
    out = np.zeros((len(lens), max(lens)))
    for b, n in enumerate(lens):
        if n == 0:
            continue
        Kh, _ = R.dequant_sequence(cache.pool, cache.chunk_bytes, Hkv, D, g, kb, vb, bt[b], n)
        for h in range(Hq):
            s = (Kh[h // G] @ q[b, h].astype(np.float64)) * sm
            w = np.exp(s - s.max())
            out[b, :n] += w / w.sum()
    return out


@pytest.mark.parametrize("fmt", [(64, 32, 6, 4), (128, 64, 6, 6), (64, 16, 16, 16)])
@pytest.mark.parametrize("G", [1, 4])
def test_scores_match_numpy_weights(fmt, G):
    """Each token's score equals the numpy softmax weights summed over the
    heads (independent dequantisation), for paged ragged batches."""
    D, g, kb, vb = fmt
    rng = np.random.default_rng(200 + G)
    lens = [1, 64, 130, 257]
    Hkv = 2
    K, V = _rand_kv(rng, lens, Hkv, D)
    cache, bt, lens = build_cache(K, V, D, g, kb, vb, rng=rng)
    q = rng.standard_normal((len(lens), Hkv * G, D)).astype(np.float32)
    sm = float(np.float32(1.0 / math.sqrt(D)))
    acc = np.zeros((1, len(lens), 300))
    O.decode([cache], [bt], [lens], q, sm, 0.0, 64, score_acc=acc)
    ref = _numpy_scores(cache, bt, lens, q, sm, fmt)
    for b, n in enumerate(lens):
        assert np.allclose(acc[0, b, :n], ref[b, :n], rtol=1e-12, atol=1e-15)
        assert np.all(acc[0, b, n:] == 0.0)  # past the end: untouched


@pytest.mark.parametrize("tau", [0.0, 1e-3])
def test_scores_sum_to_the_head_count_over_segments(tau):
    """Every head's weights sum to 1 over all live tokens of all segments, so
    a sequence's scores sum to Hq; the skip does not change the weights."""
    D, g, Hkv, G = 128, 64, 2, 4
    rng = np.random.default_rng(7)
    lens_h, lens_m = [40, 0, 300], [129, 77, 1]
    Kh, Vh = _rand_kv(rng, lens_h, Hkv, D)
    Km, Vm = _rand_kv(rng, lens_m, Hkv, D)
    ch, bth, lh = build_cache(Kh, Vh, D, g, 6, 6, rng=rng)
    cm, btm, lm = build_cache(Km, Vm, D, g, 6, 4, rng=rng)
    q = rng.standard_normal((3, Hkv * G, D)).astype(np.float32)
    acc = np.zeros((2, 3, 400))
    O.decode([ch, cm], [bth, btm], [lh, lm], q, 0.088, tau, 64, score_acc=acc)
    totals = acc.sum(axis=(0, 2))
    assert np.allclose(totals, Hq := Hkv * G, rtol=0, atol=1e-12), totals
    acc0 = np.zeros_like(acc)
    O.decode([ch, cm], [bth, btm], [lh, lm], q, 0.088, 0.0, 64, score_acc=acc0)
    assert np.array_equal(acc, acc0)  # weights do not depend on the skip
    assert Hq == 8


def test_scores_accumulate_and_single_token():
    """score_acc is added to, not overwritten; a lone token takes every
    head's whole weight."""
    D, g = 64, 32
    rng = np.random.default_rng(3)
    K, V = _rand_kv(rng, [1, 90], 1, D)
    cache, bt, lens = build_cache(K, V, D, g, 6, 4)
    q = rng.standard_normal((2, 4, D)).astype(np.float32)
    acc = np.zeros((1, 2, 128))
    O.decode([cache], [bt], [lens], q, 0.125, 0.0, 0, score_acc=acc)
    assert acc[0, 0, 0] == 4.0 and np.all(acc[0, 0, 1:] == 0)
    once = acc.copy()
    O.decode([cache], [bt], [lens], q, 0.125, 0.0, 0, score_acc=acc)
    assert np.allclose(acc, 2 * once, rtol=1e-15, atol=0)


def test_scores_reject_a_short_stride():
    rng = np.random.default_rng(4)
    K, V = _rand_kv(rng, [70], 1, 64)
    cache, bt, lens = build_cache(K, V, 64, 32, 6, 4)
    q = rng.standard_normal((1, 1, 64)).astype(np.float32)
    with pytest.raises(ValueError):
        O.decode([cache], [bt], [lens], q, 0.125, 0.0, 0, score_acc=np.zeros((1, 1, 69)))
