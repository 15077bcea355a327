"""Pins of the oracle's attention-aware tier update (Super KV Compression
page, second layer).  CPU only."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from tests import np_reference as R
from tests.oracle_cases import block_tables, build_cache

D, g = 128, 64


def _case(seed, lens, Hkv=2, frac=(0.1, 0.3)):
    rng = np.random.default_rng(seed)
    K = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    V = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    src, sbt, lens = build_cache(K, V, D, g, 6, 6, rng=rng)
    stride = int(max(lens))
    tl, th = O.default_thresholds(stride)
    scores = np.zeros((len(lens), stride), np.float32)
    for b, n in enumerate(lens):
        u = rng.random(n)
        kind = rng.choice(3, n, p=[1 - sum(frac), frac[1], frac[0]])
        lo = np.array([0.0, tl, th])[kind]
        hi = np.array([tl, th, 2 * th])[kind]
        scores[b, :n] = (lo + u * (hi - lo)).astype(np.float32)
    # exact threshold values: equal to tau_low is MID, equal to tau_high is HIGH
    scores[0, 0], scores[0, 1] = tl, th
    hbt, hn = block_tables(lens, rng)
    mbt, mn = block_tables(lens, rng)
    dst_h = O.Cache(D, g, 6, 6, Hkv, hn)
    dst_m = O.Cache(D, g, 6, 4, Hkv, mn)
    tiers, nh, nm = O.tier_update(src, sbt, lens, scores, tl, th, dst_h, hbt, dst_m, mbt)
    return dict(src=src, sbt=sbt, lens=lens, scores=scores, tl=tl, th=th, dst_h=dst_h, hbt=hbt,
                dst_m=dst_m, mbt=mbt, tiers=tiers, nh=nh, nm=nm, Hkv=Hkv)


def test_tier_assignment_and_counts():
    c = _case(1, [300, 65, 1])
    for b, n in enumerate(c["lens"]):
        s = c["scores"][b, :n]
        t = c["tiers"][b, :n]
        assert np.array_equal(t == 2, s >= c["th"])
        assert np.array_equal(t == 0, s < c["tl"])           # eviction only below tau_low
        assert np.array_equal(t == 1, (s >= c["tl"]) & (s < c["th"]))
        assert c["nh"][b] == (t == 2).sum() and c["nm"][b] == (t == 1).sum()
        assert c["nh"][b] + c["nm"][b] + (t == 0).sum() == n
        assert np.all(c["tiers"][b, n:] == 255)              # past the length: untouched
    assert c["tiers"][0, 0] == 1 and c["tiers"][0, 1] == 2


def _rows(cache, bt, b, n, Hkv):
    """Raw codes/metadata of positions [0, n) of sequence b: dict of arrays
    [Hkv][n][...]."""
    out = {k: [] for k in ("kc", "vc", "ks", "vs", "kz", "vz")}
    for h in range(Hkv):
        acc = {k: [] for k in out}
        for lb in range(-(-n // 64)):
            o = (int(bt[b, lb]) * Hkv + h) * cache.chunk_bytes
            _, _, raw = R.dequant_chunk(cache.pool[o:o + cache.chunk_bytes], D, g, cache.k_bits, cache.v_bits)
            m = min(64, n - lb * 64)
            acc["kc"].append(raw["kc"][:m])
            acc["vc"].append(raw["vc"][:m])
            for k in ("ks", "vs", "kz", "vz"):
                acc[k].append(raw[k].T[:m])
        for k in out:
            out[k].append(np.concatenate(acc[k]) if acc[k] else np.zeros((0,)))
    return {k: np.array(v) for k, v in out.items()}


def test_compaction_is_stable_and_bit_exact():
    """HIGH rows (K6, V6, scales, zeros) and MID K rows are the source rows
    in increasing token order, bit for bit."""
    c = _case(2, [400, 130])
    for b, n in enumerate(c["lens"]):
        t = c["tiers"][b, :n]
        src = _rows(c["src"], c["sbt"], b, n, c["Hkv"])
        hi = _rows(c["dst_h"], c["hbt"], b, int(c["nh"][b]), c["Hkv"])
        mid = _rows(c["dst_m"], c["mbt"], b, int(c["nm"][b]), c["Hkv"])
        ih, im = np.nonzero(t == 2)[0], np.nonzero(t == 1)[0]
        for k in ("kc", "vc", "ks", "vs", "kz", "vz"):
            assert np.array_equal(hi[k], src[k][:, ih])
        for k in ("kc", "ks", "kz"):
            assert np.array_equal(mid[k], src[k][:, im])


def test_mid_v4_is_the_4bit_quantisation_of_dequantised_v6():
    """MID V4 codes are the nearest 4-bit codes of the fp32 dequantised V6
    values, within the half-step bound of each group."""
    c = _case(3, [500])
    n = c["lens"][0]
    t = c["tiers"][0, :n]
    im = np.nonzero(t == 1)[0]
    src = _rows(c["src"], c["sbt"], 0, n, c["Hkv"])
    mid = _rows(c["dst_m"], c["mbt"], 0, int(c["nm"][0]), c["Hkv"])
    gidx = np.arange(D) // g
    # fp32 round trip of V6: (q - z) * s, one fp32 rounding
    v6 = ((src["vc"][:, im].astype(np.float32) - src["vz"][:, im][..., gidx].astype(np.float32))
          * src["vs"][:, im][..., gidx].astype(np.float32)).astype(np.float32)
    v4 = (mid["vc"].astype(np.float64) - mid["vz"][..., gidx]) * mid["vs"][..., gidx].astype(np.float64)
    step = mid["vs"][..., gidx].astype(np.float64)
    assert np.all(np.abs(v4 - v6) <= step * (0.5 + 2 ** -14))
    grp = v6.reshape(v6.shape[0], v6.shape[1], D // g, g).astype(np.float64)
    rng_ = np.maximum(grp.max(-1), 0) - np.minimum(grp.min(-1), 0)
    assert np.allclose(mid["vs"], (rng_ / 15).astype(np.float32), rtol=2e-7, atol=0)


def test_evicted_tokens_cost_less_than_their_weight_bound():
    """When the scores are a query's own softmax weights, evicting the LOW
    tokens and requantising MID V moves that query's output by at most
    2 A_low max|v| + max_mid(s4/2) / (1 - A_low), where A_low is the evicted
    weight; with tau_low = eps4/N, A_low <= eps4."""
    rng = np.random.default_rng(8)
    n, Hkv = 640, 1
    K = [rng.standard_normal((n, Hkv, D)).astype(np.float32) * 2.5]
    V = [rng.standard_normal((n, Hkv, D)).astype(np.float32)]
    src, sbt, lens = build_cache(K, V, D, g, 6, 6)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    sm = float(np.float32(1 / math.sqrt(D)))
    Kh, Vh = R.dequant_sequence(src.pool, src.chunk_bytes, 1, D, g, 6, 6, sbt[0], n)
    s = Kh[0] @ q[0, 0].astype(np.float64) * sm
    a = np.exp(s - s.max())
    a /= a.sum()
    tl, th = O.default_thresholds(n)
    scores = a.astype(np.float32)[None]
    hbt, hn = block_tables([n])
    mbt, mn = block_tables([n])
    dh, dm = O.Cache(D, g, 6, 6, 1, hn), O.Cache(D, g, 6, 4, 1, mn)
    tiers, nh, nm = O.tier_update(src, sbt, lens, scores, tl, th, dh, hbt, dm, mbt)
    assert (tiers == 0).sum() > 0 and nh[0] > 0 and nm[0] > 0
    full = O.decode([src], [sbt], [lens], q, sm)
    tiered = O.decode([dh, dm], [hbt, mbt], [nh, nm], q, sm)
    a_low = a[tiers[0] == 0].sum()
    assert a_low <= n * tl
    assert n * tl <= 1 / 30 * (1 + 1e-6)
    mid = _rows(dm, mbt, 0, int(nm[0]), 1)
    bound = 2 * a_low * np.abs(Vh).max() + (mid["vs"].max() / 2) * (1 + 1e-6) / (1 - a_low)
    assert np.max(np.abs(full - tiered)) <= bound


def test_tier_update_rejects_bad_formats_and_capacity():
    c = _case(4, [100])
    with pytest.raises(ValueError):   # destination M must hold 4-bit V
        O.tier_update(c["src"], c["sbt"], c["lens"], c["scores"], c["tl"], c["th"],
                      c["dst_h"], c["hbt"], c["dst_h"], c["hbt"])
    small = np.zeros((1, 0), np.int32)
    with pytest.raises(ValueError):   # no room for the survivors
        O.tier_update(c["src"], c["sbt"], c["lens"], c["scores"], c["tl"], c["th"],
                      c["dst_h"], small, c["dst_m"], c["mbt"])
