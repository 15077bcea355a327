"""Pins of the oracle's direction-preserving K codec (the norm-direction
page's insight: a key's direction matters more to attention than its
norm).  The group codes carry the direction; one fp32 factor per token
restores the norm, so the key read back is r * k_hat with |r * k_hat| =
|k|.  CPU only."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from tests import np_reference as R
from tests.oracle_cases import block_tables, build_cache

D, g, Hkv = 128, 64, 2


def _rows(seed, lens, outliers=True):
    rng = np.random.default_rng(seed)
    K, V = [], []
    for n in lens:
        k = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        if outliers:  # a few large channels, as in the workloads
            k[:, :, [3, 40, 77, 101]] *= 12
        K.append(k)
        V.append(rng.standard_normal((n, Hkv, D)).astype(np.float32))
    return K, V


def _factors(cache, bt, b, n):
    out = np.zeros((Hkv, n))
    for lb in range(-(-n // 64)):
        for h in range(Hkv):
            o = (int(bt[b, lb]) * Hkv + h) * cache.chunk_bytes + cache.knorm_offset
            m = min(64, n - lb * 64)
            out[h, lb * 64:lb * 64 + m] = cache.pool[o:o + 256].view(np.float32)[:m]
    return out


@pytest.mark.parametrize("kb,vb", [(6, 4), (4, 6)])
def test_codes_are_the_plain_codecs_and_the_norm_is_restored(kb, vb):
    lens = [1, 70, 129]
    K, V = _rows(1, lens)
    plain, bt, lens = build_cache(K, V, D, g, kb, vb)
    nd, bt2, _ = build_cache(K, V, D, g, kb, vb, k_norm=1)
    assert np.array_equal(bt, bt2) and nd.chunk_bytes == plain.chunk_bytes + 256
    for b, n in enumerate(lens):
        for lb in range(-(-n // 64)):
            for h in range(Hkv):
                cp = plain.chunk(int(bt[b, lb]), h)
                cn = nd.chunk(int(bt[b, lb]), h)
                assert np.array_equal(cp, cn[:plain.chunk_bytes])  # codes, scales, zeros unchanged
        Kp, _ = R.dequant_sequence(plain.pool, plain.chunk_bytes, Hkv, D, g, kb, vb, bt[b], n)
        Kn, _ = R.dequant_sequence(nd.pool, nd.chunk_bytes, Hkv, D, g, kb, vb, bt[b], n, nd.knorm_offset)
        k = K[b].transpose(1, 0, 2).astype(np.float64)
        nk, nn, np_ = (np.linalg.norm(a, axis=-1) for a in (k, Kn, Kp))
        assert np.allclose(nn, nk, rtol=2 ** -23, atol=0)        # the norm of k, to the fp32 factor
        assert np.max(np.abs(np_ - nk) / nk) > 1e-3              # the plain codec's norm is off
        cos = lambda a, c: np.sum(a * c, -1) / np.linalg.norm(a, axis=-1) / np.linalg.norm(c, axis=-1)
        assert np.allclose(cos(Kn, k), cos(Kp, k), rtol=1e-12)   # the direction is the codes'
        r = _factors(nd, bt, b, n)
        assert np.all(np.isfinite(r)) and np.all(r > 0)


def test_zero_key_takes_factor_one():
    K = [np.zeros((3, Hkv, D), np.float32)]
    V = [np.ones((3, Hkv, D), np.float32)]
    nd, bt, lens = build_cache(K, V, D, g, 6, 4, k_norm=1)
    assert np.all(_factors(nd, bt, 0, 3) == 1.0)


@pytest.mark.parametrize("G,tau,split", [(4, 0.0, 0), (8, 1e-3, 64)])
def test_decode_reads_the_scaled_keys(G, tau, split):
    """Decode over a direction-preserving cache equals numpy attention over
    r * k_hat (independent unpacking and scaling)."""
    lens = [65, 200]
    K, V = _rows(2, lens)
    nd, bt, lens = build_cache(K, V, D, g, 6, 4, k_norm=1)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, Hkv * G, D)).astype(np.float32)
    sm = float(np.float32(1 / math.sqrt(D)))
    got = O.decode([nd], [bt], [lens], q, sm, tau, split)
    for b, n in enumerate(lens):
        Kn, Vn = R.dequant_sequence(nd.pool, nd.chunk_bytes, Hkv, D, g, 6, 4, bt[b], n, nd.knorm_offset)
        if tau == 0.0:
            assert np.allclose(got[b], R.attention(q[b], Kn, Vn, sm), rtol=1e-12, atol=1e-13)
    if tau > 0.0:  # the skip follows the scaled scores: same as decode of the scaled rows in a plain cache
        plain_out = O.decode([nd], [bt], [lens], q, sm, 0.0, split)
        assert np.max(np.abs(got - plain_out)) <= 2 * tau * max(np.abs(Vn).max(), 1) * 64


def test_fp16_format_and_tiers_reject_the_codec():
    with pytest.raises(ValueError):
        c = O.Cache(D, g, 16, 16, 1, 1, k_norm=1)
        O.append(c, np.zeros((1, 1, D), np.float32), np.zeros((1, 1, D), np.float32), [0, 1], [0],
                 np.zeros((1, 1), np.int32))
    K, V = _rows(4, [64], outliers=False)
    src, bt, lens = build_cache(K, V, D, g, 6, 6, k_norm=1)
    h, m = O.Cache(D, g, 6, 6, Hkv, 2), O.Cache(D, g, 6, 4, Hkv, 2)
    with pytest.raises(ValueError):
        O.tier_update(src, bt, lens, np.ones((1, 64), np.float32), 0.1, 0.5, h, bt, m, bt)
