"""Pins of the oracle's append placement and decode attention (fp64),
including the sparse-V skip rule.  CPU only."""
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


FORMATS = [(64, 32, 6, 4), (128, 64, 6, 4), (128, 64, 6, 6), (128, 64, 4, 4), (64, 16, 16, 16)]


@pytest.mark.parametrize("fmt", FORMATS)
def test_append_places_rows_paged(fmt):
    """Every (sequence, token, KV head) row lands in its block-table chunk
    and slot: numpy unpacking of the pool reconstructs each original row
    within half a step (fp16: exactly its fp16 rounding)."""
    D, g, kb, vb = fmt
    rng = np.random.default_rng(11)
    lens = [1, 63, 64, 65, 200]
    K, V = _rand_kv(rng, lens, 2, D)
    cache, bt, lens = build_cache(K, V, D, g, kb, vb, rng=rng)
    for b, n in enumerate(lens):
        Kh, Vh = R.dequant_sequence(cache.pool, cache.chunk_bytes, 2, D, g, kb, vb, bt[b], n)
        for X, Xh, bits in ((K[b], Kh, kb), (V[b], Vh, vb)):
            X = X.transpose(1, 0, 2).astype(np.float64)
            if bits == 16:
                assert np.array_equal(Xh, X.astype(np.float16).astype(np.float64))
                continue
            G = X.reshape(2, n, D // g, g)
            rng_ = np.maximum(G.max(-1), 0) - np.minimum(G.min(-1), 0)
            step = (rng_ / ((1 << bits) - 1))[..., None]
            err = np.abs(Xh.reshape(G.shape) - G)
            assert np.all(err <= step * (0.5 + 2 ** -14))


def test_append_ragged_start_positions_do_not_touch_other_slots():
    """Appending at start_pos > 0 writes only the new slots."""
    D, g, kb, vb = 128, 64, 6, 4
    rng = np.random.default_rng(5)
    K, V = _rand_kv(rng, [100], 1, D)
    cache, bt, _ = build_cache(K, V, D, g, kb, vb)
    before = cache.pool.copy()
    k2, v2 = _rand_kv(rng, [3], 1, D)
    O.append(cache, k2[0], v2[0], [0, 3], [100], bt)
    Kh, _ = R.dequant_sequence(cache.pool, cache.chunk_bytes, 1, D, g, kb, vb, bt[0], 103)
    Kh0, _ = R.dequant_sequence(before, cache.chunk_bytes, 1, D, g, kb, vb, bt[0], 100)
    assert np.array_equal(Kh[:, :100], Kh0)
    assert np.max(np.abs(Kh[0, 100:] - k2[0][:, 0])) < 0.2


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("G", [1, 4])
def test_decode_matches_numpy_bruteforce(fmt, G):
    """fp64 decode equals an independent numpy softmax over the numpy
    dequantisation of the same pool, for paged ragged batches."""
    D, g, kb, vb = fmt
    rng = np.random.default_rng(100 + G)
    lens = [1, 64, 130, 257]
    Hkv = 2
    K, V = _rand_kv(rng, lens, Hkv, D)
    cache, bt, lens = build_cache(K, V, D, g, kb, vb, rng=rng)
    q = rng.standard_normal((len(lens), Hkv * G, D)).astype(np.float32)
    sm = float(np.float32(1.0 / math.sqrt(D)))  # the API takes an fp32 scale
    for split in (0, 64, 128):
        out = O.decode([cache], [bt], [lens], q, sm, 0.0, split)
        for b, n in enumerate(lens):
            Kh, Vh = R.dequant_sequence(cache.pool, cache.chunk_bytes, Hkv, D, g, kb, vb, bt[b], n)
            ref = R.attention(q[b], Kh, Vh, sm)
            assert np.allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def test_decode_special_cases():
    """N = 1 gives v_hat exactly; q = 0 gives the mean of v_hat; one
    dominant key gives its v_hat; token order does not matter."""
    D, g = 64, 32
    rng = np.random.default_rng(9)
    K, V = _rand_kv(rng, [1], 1, D)
    cache, bt, lens = build_cache(K, V, D, g, 6, 4)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    out = O.decode([cache], [bt], [lens], q, 0.125)
    _, Vh = R.dequant_sequence(cache.pool, cache.chunk_bytes, 1, D, g, 6, 4, bt[0], 1)
    assert np.array_equal(out[0, 0], Vh[0, 0])

    K, V = _rand_kv(rng, [300], 1, D)
    cache, bt, lens = build_cache(K, V, D, g, 6, 4)
    _, Vh = R.dequant_sequence(cache.pool, cache.chunk_bytes, 1, D, g, 6, 4, bt[0], 300)
    out = O.decode([cache], [bt], [lens], np.zeros((1, 1, D), np.float32), 0.125)
    assert np.allclose(out[0, 0], Vh[0].mean(0), rtol=0, atol=1e-13)

    K[0][:, 0, 0] = rng.standard_normal(300) * 0.1
    K[0][77, 0, 0] = 2000.0
    cache, bt, lens = build_cache(K, V, D, g, 6, 4)
    Kh, Vh = R.dequant_sequence(cache.pool, cache.chunk_bytes, 1, D, g, 6, 4, bt[0], 300)
    qe = np.zeros((1, 1, D), np.float32)
    qe[0, 0, 0] = 1.0
    sm = 1.0 / 8.0
    s = Kh[0] @ qe[0, 0].astype(np.float64) * sm
    gap = s[77] - np.delete(s, 77).max()
    assert gap > 100
    out = O.decode([cache], [bt], [lens], qe, sm)
    assert np.max(np.abs(out[0, 0] - Vh[0, 77])) <= 300 * math.exp(-gap) * np.abs(Vh).max() + 1e-15

    perm = rng.permutation(300)
    cache2, bt2, _ = build_cache([K[0][perm]], [V[0][perm]], D, g, 6, 4)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    a = O.decode([cache], [bt], [lens], q, sm)
    b = O.decode([cache2], [bt2], [lens], q, sm)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_gqa_head_mapping():
    """G = 1 is per-head attention; query heads of one group read one KV
    head: equal queries inside a group give equal outputs, across groups
    they do not."""
    D, g = 64, 32
    rng = np.random.default_rng(4)
    K, V = _rand_kv(rng, [150], 2, D)
    cache, bt, lens = build_cache(K, V, D, g, 6, 4)
    q1 = rng.standard_normal(D).astype(np.float32)
    q = np.stack([q1] * 8)[None]
    out = O.decode([cache], [bt], [lens], q, 0.125)[0]
    for h in range(4):
        assert np.array_equal(out[h], out[0]) and np.array_equal(out[4 + h], out[4])
    assert not np.allclose(out[0], out[4])
    mha = O.decode([cache], [bt], [lens], q[:, [0, 4]], 0.125)[0]
    assert np.array_equal(mha[0], out[0]) and np.array_equal(mha[1], out[4])


def test_split_plans_agree_without_skip():
    D, g = 128, 64
    rng = np.random.default_rng(2)
    K, V = _rand_kv(rng, [1000, 777], 1, D)
    cache, bt, lens = build_cache(K, V, D, g, 6, 4, rng=rng)
    q = rng.standard_normal((2, 4, D)).astype(np.float32)
    outs = [O.decode([cache], [bt], [lens], q, 0.09, 0.0, s) for s in (0, 64, 192, 1024)]
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=1e-12, atol=1e-14)


def _weights(q, Kh, sm, G):
    """Global softmax weights [Hq][n] from numpy."""
    a = []
    for h in range(q.shape[0]):
        s = (Kh[h // G] @ q[h].astype(np.float64)) * sm
        w = np.exp(s - s.max())
        a.append(w / w.sum())
    return np.array(a)


@pytest.mark.parametrize("tau", [1e-4, 1e-3, 5e-3])
@pytest.mark.parametrize("split", [64, 256, 0])
def test_skip_rule_soundness_and_bound(tau, split):
    """Every skipped (token, head) has true weight < tau; tau = 0 skips
    nothing; skipped tokens stay in the denominator (numpy brute force with
    the oracle's skip set agrees); the output moves by at most
    sum(skipped weights) * max|v_hat|."""
    D, g, G = 128, 64, 4
    rng = np.random.default_rng(int(tau * 1e6) + split)
    K, V = _rand_kv(rng, [700], 1, D)
    K[0][:, :, :4] *= 12.0
    cache, bt, lens = build_cache(K, V, D, g, 6, 4)
    q = rng.standard_normal((1, G, D)).astype(np.float32)
    sm = float(np.float32(1 / math.sqrt(D)))
    o_skip, sk = O.decode([cache], [bt], [lens], q, sm, tau, split, want_skip=True)
    o_full, sk0 = O.decode([cache], [bt], [lens], q, sm, 0.0, split, want_skip=True)
    assert sk0.sum() == 0
    Kh, Vh = R.dequant_sequence(cache.pool, cache.chunk_bytes, 1, D, g, 6, 4, bt[0], 700)
    a = _weights(q[0], Kh, sm, G)
    skipped = sk[0, :, 0, :700].astype(bool)
    assert skipped.sum() > 0
    assert np.all(a[skipped] < tau)
    ref = R.attention(q[0], Kh, Vh, sm, keep=~skipped)
    assert np.allclose(o_skip[0], ref, rtol=1e-12, atol=1e-14)
    vmax = np.abs(Vh).max()
    for h in range(G):
        assert np.max(np.abs(o_skip[0, h] - o_full[0, h])) <= a[h][skipped[h]].sum() * vmax * (1 + 1e-9)


def test_skip_rule_uses_the_running_block_bound():
    """Hand-built case: within one 64-token block, a token 25 below the
    maximum is skipped at tau = 1e-10 and one 5 below is kept; a token of an
    earlier block is judged against the running (m, L) of its own block, so
    a later, larger maximum does not make it skipped."""
    D, g = 64, 32
    n = 128
    K = np.zeros((n, 1, D), np.float32)
    V = np.ones((n, 1, D), np.float32)
    K[:, 0, 1] = 1.0        # a second channel keeps every group two-valued
    K[:64, 0, 0] = -5.0     # block 0: scores -5 ...
    K[10, 0, 0] = 0.0       # ... one at 0 ...
    K[20, 0, 0] = -30.0     # ... and one at -30
    K[64:, 0, 0] = -40.0    # block 1: scores -40 ...
    K[100, 0, 0] = 20.0     # ... and a new maximum at 20
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    cache, bt, lens = build_cache([K], [V], D, g, 6, 4)
    Kh, _ = R.dequant_sequence(cache.pool, cache.chunk_bytes, 1, D, g, 6, 4, bt[0], n)
    s = Kh[0, :, 0]
    assert s[10] == 0.0 and abs(s[100] - 20) < 1e-3 and abs(s[20] + 30) < 0.5 and abs(s[0] + 5) < 0.5
    _, sk = O.decode([cache], [bt], [lens], q, 1.0, 1e-10, 128, want_skip=True)
    sk = sk[0, 0, 0, :n].astype(bool)
    assert sk[20] and not sk[10] and not sk[0]
    # block 0's -5 tokens have true weight ~ e^-25 < 1e-10 once token 100 is
    # seen, but were judged against block 0's running bound: kept
    assert math.exp(s[0] - 20) < 1e-10 and not sk[:64][np.arange(64) != 20].any()
    # block 1's -40 tokens are skipped (e^-60 relative to the running max)
    assert sk[64:100].all() and not sk[100]
