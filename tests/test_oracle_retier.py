"""Pins of the oracle's re-tiering of a tiered cache (the periodic form of
the attention-aware tiers, Super KV Compression page, second layer).  CPU
only."""
import numpy as np
import pytest

from oracle import oracle as O
from tests import np_reference as R
from tests.oracle_cases import block_tables, build_cache

D, g, HKV = 128, 64, 2


def _scores(rng, lens, tl, th, frac=(0.2, 0.5), stride=None):
    """fp32 [B][stride] scores: LOW / MID / HIGH with the given fractions."""
    stride = stride or max(max(lens), 1)
    s = np.zeros((len(lens), stride), np.float32)
    for b, n in enumerate(lens):
        kind = rng.choice(3, n, p=[1 - sum(frac), frac[1], frac[0]])
        lo = np.array([0.0, tl, th])[kind]
        hi = np.array([tl, th, 2 * th])[kind]
        s[b, :n] = (lo + rng.random(n) * (hi - lo)).astype(np.float32)
    return s


def _tiered(seed, lens):
    """A tiered cache {H: K6V6, M: K6V4} made by the (pinned) tier update."""
    rng = np.random.default_rng(seed)
    K = [rng.standard_normal((n, HKV, D)).astype(np.float32) for n in lens]
    V = [rng.standard_normal((n, HKV, D)).astype(np.float32) for n in lens]
    src, sbt, lens = build_cache(K, V, D, g, 6, 6, rng=rng)
    tl, th = O.default_thresholds(int(max(lens)))
    sc = _scores(rng, lens, tl, th)
    hbt, hn = block_tables(lens, rng)
    mbt, mn = block_tables(lens, rng)
    h, m = O.Cache(D, g, 6, 6, HKV, hn), O.Cache(D, g, 6, 4, HKV, mn)
    _, nh, nm = O.tier_update(src, sbt, lens, sc, tl, th, h, hbt, m, mbt)
    return rng, h, hbt, nh, m, mbt, nm, tl, th


def _rows(cache, bt_row, n, vb):
    return R.dequant_sequence(cache.pool, cache.chunk_bytes, HKV, D, g, 6, vb, bt_row, n)


def _retier(rng, h, hbt, nh, m, mbt, nm, tl, th, hs=None, ms=None):
    B = len(nh)
    hs = _scores(rng, nh, tl, th) if hs is None else hs
    ms = _scores(rng, nm, tl, th) if ms is None else ms
    cap = [int(a + b) for a, b in zip(nh, nm)]
    dhb, dhn = block_tables([max(c, 1) for c in cap], rng)
    dmb, dmn = block_tables([max(c, 1) for c in cap], rng)
    dh, dm = O.Cache(D, g, 6, 6, HKV, dhn), O.Cache(D, g, 6, 4, HKV, dmn)
    ht, mt, nh2, nm2 = O.retier(h, hbt, nh, hs, m, mbt, nm, ms, tl, th, dh, dhb, dm, dmb)
    return dict(hs=hs, ms=ms, dh=dh, dhb=dhb, dm=dm, dmb=dmb, ht=ht, mt=mt, nh=nh2, nm=nm2, B=B)


def test_retier_with_an_empty_mid_segment_is_the_tier_update():
    """With no MID tokens, re-tiering HIGH is exactly the tier update of it:
    same tiers, counts and destination bytes."""
    rng, h, hbt, nh, m, mbt, nm, tl, th = _tiered(1, [300, 700, 65])
    zero = np.zeros_like(nm)
    r = _retier(rng, h, hbt, nh, m, mbt, zero, tl, th)
    dh2, dm2 = O.Cache(D, g, 6, 6, HKV, r["dh"].num_blocks), O.Cache(D, g, 6, 4, HKV, r["dm"].num_blocks)
    t, n1, n2 = O.tier_update(h, hbt, nh, r["hs"], tl, th, dh2, r["dhb"], dm2, r["dmb"])
    assert np.array_equal(r["nh"], n1) and np.array_equal(r["nm"], n2)
    for b, n in enumerate(nh):
        assert np.array_equal(r["ht"][b, :n], t[b, :n])
    assert np.array_equal(r["dh"].pool, dh2.pool) and np.array_equal(r["dm"].pool, dm2.pool)


def test_retier_counts_order_and_rows():
    rng, h, hbt, nh, m, mbt, nm, tl, th = _tiered(2, [400, 900, 130])
    r = _retier(rng, h, hbt, nh, m, mbt, nm, tl, th)
    for b in range(r["B"]):
        hs, ms = r["hs"][b, :nh[b]], r["ms"][b, :nm[b]]
        keep_h = np.nonzero(hs >= th)[0]
        demote = np.nonzero((hs >= tl) & (hs < th))[0]
        keep_m = np.nonzero(ms >= tl)[0]
        assert r["nh"][b] == len(keep_h) and r["nm"][b] == len(keep_m) + len(demote)
        assert np.array_equal(r["ht"][b, :nh[b]], np.where(hs >= th, 2, np.where(hs >= tl, 1, 0)))
        assert np.array_equal(r["mt"][b, :nm[b]], np.where(ms >= tl, 1, 0))
        Kh, Vh = _rows(h, hbt[b], int(nh[b]), 6)
        Km, Vm = _rows(m, mbt[b], int(nm[b]), 4)
        Kdh, Vdh = _rows(r["dh"], r["dhb"][b], int(r["nh"][b]), 6)
        Kdm, Vdm = _rows(r["dm"], r["dmb"][b], int(r["nm"][b]), 4)
        # HIGH kept, in order, bit for bit
        assert np.array_equal(Kdh, Kh[:, keep_h]) and np.array_equal(Vdh, Vh[:, keep_h])
        # MID kept first, in order, bit for bit; then the demoted tokens
        k = len(keep_m)
        assert np.array_equal(Kdm[:, :k], Km[:, keep_m]) and np.array_equal(Vdm[:, :k], Vm[:, keep_m])
        assert np.array_equal(Kdm[:, k:], Kh[:, demote])
        # a demoted V row is the 4-bit quantisation of its 6-bit values
        for kv in range(HKV):
            for i, j in enumerate(demote):
                for gi in range(D // g):
                    x = Vh[kv, j, gi * g:(gi + 1) * g].astype(np.float32)
                    s, z, codes = O.quantize_group(x, 4)
                    want = (codes.astype(np.float64) - z) * np.float64(s)
                    assert np.array_equal(Vdm[kv, k + i, gi * g:(gi + 1) * g], want)


def test_retier_never_promotes_a_mid_token():
    rng, h, hbt, nh, m, mbt, nm, tl, th = _tiered(3, [200, 500])
    ms = np.full((2, int(nm.max())), 4 * th, np.float32)  # every MID token far above tau_high
    hs = np.full((2, int(nh.max())), tl / 2, np.float32)   # every HIGH token evicted
    r = _retier(rng, h, hbt, nh, m, mbt, nm, tl, th, hs=hs, ms=ms)
    assert np.array_equal(r["nh"], [0, 0]) and np.array_equal(r["nm"], nm)
    for b in range(2):
        assert np.all(r["mt"][b, :nm[b]] == 1) and np.all(r["ht"][b, :nh[b]] == 0)


def test_retier_rejects_a_destination_without_room():
    rng, h, hbt, nh, m, mbt, nm, tl, th = _tiered(4, [1000])
    assert nh[0] > 64  # more HIGH survivors than one destination block holds
    hs = np.full((1, int(nh[0])), 2 * th, np.float32)
    ms = np.full((1, int(nm[0])), 2 * th, np.float32)
    small = O.Cache(D, g, 6, 6, HKV, 1)
    with pytest.raises(ValueError):
        O.retier(h, hbt, nh, hs, m, mbt, nm, ms, tl, th, small, np.zeros((1, 1), np.int32),
                 O.Cache(D, g, 6, 4, HKV, 8), np.arange(8, dtype=np.int32)[None])


def grow_rows(cache, bt, lens_now, lens_need, rng):
    """A copy of `cache` whose rows hold blocks for lens_need positions: the
    row's blocks for lens_now positions, then fresh blocks appended to the
    pool (filled with random bytes: stale data)."""
    have = [-(-int(n) // 64) for n in lens_now]
    need = [max(-(-int(n) // 64), h) for n, h in zip(lens_need, have)]
    extra = sum(n - h for n, h in zip(need, have))
    big = O.Cache(cache.head_dim, cache.group_size, cache.k_bits, cache.v_bits, cache.num_kv_heads,
                  cache.num_blocks + extra)
    big.pool[:cache.pool.size] = cache.pool
    big.pool[cache.pool.size:] = rng.integers(0, 256, big.pool.size - cache.pool.size, dtype=np.uint8)
    width = max(max(need), bt.shape[1], 1)
    out = np.zeros((len(have), width), np.int32)
    fresh = cache.num_blocks
    for b, (h, n) in enumerate(zip(have, need)):
        out[b, :h] = bt[b, :h]
        out[b, h:n] = np.arange(fresh, fresh + n - h)
        fresh += n - h
    return big, out


def _same_live(a, abt, b, bbt, lens, vb):
    for r, n in enumerate(lens):
        fa = R.token_fields(a.pool, a.chunk_bytes, HKV, D, g, 6, vb, abt[r], int(n))
        fb = R.token_fields(b.pool, b.chunk_bytes, HKV, D, g, 6, vb, bbt[r], int(n))
        for k in fa:
            assert np.array_equal(fa[k], fb[k]), (r, k)


def test_retier_in_place_equals_the_retier_into_new_blocks():
    """Destinations that are the sources themselves (same pools, same block
    tables; MID rows grown for the demoted tokens): tiers, counts and every
    live token's codes, scales and zeros as the re-tier into fresh blocks."""
    rng, h, hbt, nh, m, mbt, nm, tl, th = _tiered(5, [300, 1000, 65, 2100])
    r = _retier(rng, h, hbt, nh, m, mbt, nm, tl, th)
    h2 = O.Cache(D, g, 6, 6, HKV, h.num_blocks, pool=h.pool.copy())
    m2, mbt2 = grow_rows(m, mbt, nm, nm + nh, rng)
    ht, mt, n_h, n_m = O.retier(h2, hbt, nh, r["hs"], m2, mbt2, nm, r["ms"], tl, th, h2, hbt, m2, mbt2)
    assert np.array_equal(n_h, r["nh"]) and np.array_equal(n_m, r["nm"])
    assert np.array_equal(ht, r["ht"]) and np.array_equal(mt, r["mt"])
    assert 0 < int(n_h.sum()) and int(n_m.sum()) > int(nm.sum()) // 2  # kept, demoted and evicted tokens
    _same_live(h2, hbt, r["dh"], r["dhb"], n_h, 6)
    _same_live(m2, mbt2, r["dm"], r["dmb"], n_m, 4)


def test_tier_update_in_place_equals_the_update_into_new_blocks():
    """HIGH compacted within the K6V6 source's own blocks."""
    rng = np.random.default_rng(6)
    lens = [500, 64, 1300]
    K = [rng.standard_normal((n, HKV, D)).astype(np.float32) for n in lens]
    V = [rng.standard_normal((n, HKV, D)).astype(np.float32) for n in lens]
    src, sbt, lens = build_cache(K, V, D, g, 6, 6, rng=rng)
    tl, th = O.default_thresholds(int(max(lens)))
    sc = _scores(rng, lens, tl, th)
    hbt, hn = block_tables(lens, rng)
    mbt, mn = block_tables(lens, rng)
    h, m = O.Cache(D, g, 6, 6, HKV, hn), O.Cache(D, g, 6, 4, HKV, mn)
    t, nh, nm = O.tier_update(src, sbt, lens, sc, tl, th, h, hbt, m, mbt)
    m2 = O.Cache(D, g, 6, 4, HKV, mn)
    t2, nh2, nm2 = O.tier_update(src, sbt, lens, sc, tl, th, src, sbt, m2, mbt)
    assert np.array_equal(t, t2) and np.array_equal(nh, nh2) and np.array_equal(nm, nm2)
    assert np.array_equal(m.pool, m2.pool)
    _same_live(src, sbt, h, hbt, nh, 6)
