"""Pins of the oracle's resolution of near-threshold sparse-V skip decisions
(Super KV Compression page, third layer: V terms of tokens under the
threshold are skipped).  The rule compares exp(s - m) with tau_low * L per
block; where the two are within a relative band, either decision is
correct and the oracle takes the one it is given.  CPU only."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from tests import np_reference as R
from tests.oracle_cases import build_cache

BT = 64


def _one_block(rng, n=64, D=64, g=32, kb=6, vb=4):
    K = [rng.standard_normal((n, 1, D)).astype(np.float32)]
    V = [rng.standard_normal((n, 1, D)).astype(np.float32)]
    cache, bt, lens = build_cache(K, V, D, g, kb, vb)
    _, Vh = R.dequant_sequence(cache.pool, cache.chunk_bytes, 1, D, g, kb, vb, bt[0], n)
    return cache, bt, lens, Vh[0]


def test_exact_tie_is_ambiguous_and_follows_the_given_decision():
    """q = 0: every score is 0, so in the first block exp(s - m) = 1 and
    L = 64; tau_low = 1/64 puts every token exactly on the bound."""
    rng = np.random.default_rng(1)
    cache, bt, lens, Vh = _one_block(rng)
    q = np.zeros((1, 1, 64), np.float32)
    tau = 1.0 / 64
    mean = Vh.mean(axis=0)
    out, skip, amb, margin = O.decode_resolved([cache], [bt], [lens], q, 0.125, tau, 64, None, 0.0)
    assert np.all(amb[0, 0, 0, :64] == 1) and np.all(margin[0, 0, 0, :64] == 0.0)
    assert np.all(skip[0, 0, 0, :64] == 0)  # 1 < 1 is false: the exact decision keeps
    assert np.allclose(out[0, 0], mean, rtol=0, atol=1e-14)
    for given, want in ((1, np.zeros_like(mean)), (0, mean)):
        g = np.full(skip.shape, given, np.uint8)
        out, skip, amb, _ = O.decode_resolved([cache], [bt], [lens], q, 0.125, tau, 64, g, 0.0)
        assert np.all(skip[0, 0, 0, :64] == given)
        assert np.allclose(out[0, 0], want, rtol=0, atol=1e-14)


def test_band_edges():
    """tau_low = (1 + d)/64 with q = 0: the relative margin of every token is
    exactly -d / (1 + d).  A band of d covers it; a band of d/2 does not, and
    then the exact decision (skip) is kept whatever is given."""
    rng = np.random.default_rng(2)
    cache, bt, lens, Vh = _one_block(rng)
    q = np.zeros((1, 1, 64), np.float32)
    d = 2.0 ** -10
    tau = float(np.float32((1 + d) / 64))
    assert tau == (1 + d) / 64  # exact in fp32
    keep_all = np.zeros((1, 1, 1, 64), np.uint8)
    out, skip, amb, margin = O.decode_resolved([cache], [bt], [lens], q, 0.125, tau, 64, keep_all, d)
    assert np.all(amb[..., :64] == 1) and np.all(skip[..., :64] == 0)
    assert np.allclose(margin[..., :64], -d / (1 + d), rtol=1e-15, atol=0)
    assert np.allclose(out[0, 0], Vh.mean(axis=0), rtol=0, atol=1e-14)
    out, skip, amb, _ = O.decode_resolved([cache], [bt], [lens], q, 0.125, tau, 64, keep_all, d / 2)
    assert np.all(amb == 0) and np.all(skip[..., :64] == 1)
    assert np.all(out == 0.0)


def test_no_given_equals_plain_decode():
    """Without given decisions the resolved decode is the plain decode, bit
    for bit, whatever the band."""
    rng = np.random.default_rng(3)
    lens = [1, 64, 130, 257]
    K = [rng.standard_normal((n, 2, 128)).astype(np.float32) for n in lens]
    V = [rng.standard_normal((n, 2, 128)).astype(np.float32) for n in lens]
    cache, bt, lens = build_cache(K, V, 128, 64, 6, 4, rng=rng)
    q = rng.standard_normal((4, 8, 128)).astype(np.float32)
    for tau in (0.0, 1e-3, 5e-3):
        want, wskip = O.decode([cache], [bt], [lens], q, 0.088388, tau, 64, want_skip=True)
        for band in (0.0, 1e-3, 1e9):
            out, skip, _, _ = O.decode_resolved([cache], [bt], [lens], q, 0.088388, tau, 64, None, band)
            assert np.array_equal(out, want) and np.array_equal(skip, wskip)


@pytest.mark.parametrize("tau", [1e-3, 5e-3, 2e-2])
def test_any_given_decisions_give_numpy_attention_with_that_skip_set(tau):
    """An unbounded band makes every live pair ambiguous: the skip set is then
    exactly the given one, and the output is numpy softmax attention with
    those V terms dropped (denominator unchanged)."""
    rng = np.random.default_rng(4)
    lens = [5, 64, 200]
    Hkv, G, D = 2, 4, 64
    K = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    V = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    cache, bt, lens = build_cache(K, V, D, 32, 6, 4, rng=rng)
    q = rng.standard_normal((3, Hkv * G, D)).astype(np.float32)
    sm = float(np.float32(1 / math.sqrt(D)))
    max_tok = bt.shape[1] * BT
    given = rng.integers(0, 2, (3, Hkv * G, 1, max_tok)).astype(np.uint8)
    out, skip, amb, _ = O.decode_resolved([cache], [bt], [lens], q, sm, tau, 128, given, 1e300)
    for b, n in enumerate(lens):
        assert np.array_equal(skip[b, :, 0, :n], given[b, :, 0, :n])
        assert np.all(amb[b, :, 0, :n] == 1)
        Kh, Vh = R.dequant_sequence(cache.pool, cache.chunk_bytes, Hkv, D, 32, 6, 4, bt[b], n)
        ref = R.attention(q[b], Kh, Vh, sm, keep=given[b, :, 0, :n] == 0)
        assert np.allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def test_margin_of_a_one_block_split():
    """For a split of one block, the running (m, L) are the block's own: the
    margin of token j is exp(s_j - max s) / (tau L) - 1 with
    L = sum exp(s - max s), computed here with numpy."""
    rng = np.random.default_rng(5)
    cache, bt, lens, _ = _one_block(rng, n=50)
    q = rng.standard_normal((1, 1, 64)).astype(np.float32)
    sm = 0.125
    tau = float(np.float32(2e-2))  # the oracle takes tau_low in fp32
    _, _, _, margin = O.decode_resolved([cache], [bt], [lens], q, sm, tau, 64, None, 0.0)
    Kh, _ = R.dequant_sequence(cache.pool, cache.chunk_bytes, 1, 64, 32, 6, 4, bt[0], 50)
    s = (Kh[0] @ q[0, 0].astype(np.float64)) * sm
    w = np.exp(s - s.max())
    want = w / (tau * w.sum()) - 1.0
    assert np.allclose(margin[0, 0, 0, :50], want, rtol=1e-12, atol=1e-12)
    assert np.all(margin[0, 0, 0, 50:] == 0.0)


def test_resolved_decode_accumulates_the_same_scores():
    """The weights a resolved decode adds to score_acc are decode()'s: they
    do not depend on the skip decisions."""
    rng = np.random.default_rng(31)
    lens = [300, 70]
    K = [rng.standard_normal((n, 1, 64)).astype(np.float32) for n in lens]
    V = [rng.standard_normal((n, 1, 64)).astype(np.float32) for n in lens]
    cache, bt, lens = build_cache(K, V, 64, 32, 6, 4, rng=rng)
    q = rng.standard_normal((2, 2, 64)).astype(np.float32)
    a = np.zeros((1, 2, 320))
    b = np.zeros((1, 2, 320))
    O.decode([cache], [bt], [lens], q, 0.125, 0.02, 64, score_acc=a)
    given = np.ones((2, 2, 1, bt.shape[1] * 64), np.uint8)  # every ambiguous pair skipped
    O.decode_resolved([cache], [bt], [lens], q, 0.125, 0.02, 64, given, 0.5, score_acc=b)
    assert np.array_equal(a, b) and a.sum() > 0
