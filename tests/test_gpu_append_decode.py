"""lkv_append_decode (one decode step of a layer in one call) against
lkv_quant_append followed by lkv_decode_attn, and against the oracle.

The fused path (the split kernel writes each sequence's newest row) and the
fallback (the append kernel, then the split kernel) must leave the pool and
the output bit for bit as the two calls do; the pool is bit-exact with the
oracle's append and the output within max|d| <= 1e-3 max|v_hat| and rel L2
<= 1e-4 of the oracle's decode."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_kv_cache_token_amd import inputs, lkv
from tests.gpu_common import (Pair, assert_attention_close, max_abs_vhat, resolved_reference, say, sm_scale,
                              to_f32_host)
from tests.oracle_cases import block_tables
from tests.test_gpu_parity import _prefill

pytestmark = pytest.mark.gpu

CASES = [  # (format, G, q dtype, new-row dtype): fused (matrix-core) and fallback formats
    ((128, 64, 6, 4), 4, "bf16", "bf16"),
    ((128, 64, 6, 4), 8, "bf16", "bf16"),
    ((128, 64, 6, 6), 4, "bf16", "f32"),
    ((128, 64, 6, 6), 8, "bf16", "f16"),
    ((128, 64, 6, 4), 4, "f32", "bf16"),      # fp32 Q: generic kernel after the append kernel
    ((128, 64, 16, 16), 8, "bf16", "bf16"),   # fp16 layer
    ((64, 32, 6, 4), 2, "bf16", "f32"),
]
# lengths after the new token: slot 0 of a new block, a full block, split
# edges (with split 64 every split is one block: the row is written before
# that block is loaded), a single token, and an empty sequence
LENS = [1, 64, 65, 129, 1024, 1025, 2048, 1500, 0]


def _caches(fmt, lens, Hkv, seed):
    D, g, kb, vb = fmt
    rng = np.random.default_rng(seed)
    bt, nblk = block_tables([max(n, 1) for n in lens], rng)
    a = Pair(D, g, kb, vb, Hkv, nblk)
    _prefill(a, [max(n - 1, 0) for n in lens], Hkv, D, "bf16", seed, bt, outliers=True)
    b = lkv.Cache(D, g, kb, vb, Hkv, nblk, pool=a.gpu.pool.clone())
    return a, b, bt


@pytest.mark.parametrize("case", CASES, ids=lambda c: "D{}g{}k{}v{}".format(*c[0]) + f"G{c[1]}{c[2]}{c[3]}")
@pytest.mark.parametrize("split", [64, 1024])
def test_append_decode_equals_append_then_decode(case, split):
    fmt, G, qd, kvd = case
    D = fmt[0]
    Hkv = 2
    lens = LENS
    B = len(lens)
    pair, fused, bt = _caches(fmt, lens, Hkv, 41)
    k_new, v_new = inputs.kv_rows(42, 0, B, Hkv, D, dtype=kvd)
    q = inputs.queries(43, B, Hkv * G, D, dtype=qd).cuda()
    lt = torch.tensor(lens, dtype=torch.int32).cuda()
    view = lkv.View(torch.tensor(bt).cuda(), lt, max(lens))
    sm = sm_scale(D)
    say("append_decode", case, "split", split)
    got = lkv.append_decode(fused, view, k_new.cuda(), v_new.cuda(), q, sm, 0.0, split)
    # the two calls: rows of the non-empty sequences at seq_len - 1
    live = [b for b, n in enumerate(lens) if n > 0]
    cu = np.arange(len(live) + 1, dtype=np.int32)
    sp = np.array([lens[b] - 1 for b in live], np.int32)
    pair.append(k_new[live], v_new[live], cu, sp, bt[live])
    want = lkv.decode_attn([pair.gpu], [view], q, sm, 0.0, split)
    torch.cuda.synchronize()
    assert torch.equal(fused.pool, pair.gpu.pool), "pool differs from lkv_quant_append"
    assert torch.equal(got, want), f"output differs from lkv_decode_attn: max |d| {float((got - want).abs().max())}"
    assert pair.pool_equal(), pair.first_pool_mismatch()
    ref = O.decode([pair.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm, 0.0, split)
    assert_attention_close(got.cpu().numpy(), ref, max_abs_vhat(pair.ref), f"{case} split {split}")
    assert np.all(got.cpu().numpy()[lens.index(0)] == 0.0)


def test_append_decode_steps_with_skip_against_the_oracle():
    """Several decode steps in a row on a ragged paged batch, each with the
    sparse-V skip: every step's pool bit-exact and output within tolerance
    (skip decisions resolved through the debug entry point)."""
    from tests.gpu_common import resolved_reference

    fmt, G, Hkv, D = (128, 64, 6, 4), 8, 2, 128
    rng = np.random.default_rng(44)
    lens0 = [int(x) for x in rng.integers(60, 700, 6)]
    steps = 5
    bt, nblk = block_tables([n + steps for n in lens0], rng)
    pair = Pair(*fmt, Hkv, nblk)
    _prefill(pair, lens0, Hkv, D, "bf16", 44, bt)
    btd = torch.tensor(bt).cuda()
    tau = 2e-3
    for s in range(steps):
        lens = [n + s + 1 for n in lens0]
        k_new, v_new = inputs.kv_rows(45, 0, len(lens), Hkv, D, step=s + 1)
        q = inputs.queries(46 + s, len(lens), Hkv * G, D).cuda()
        view = lkv.View(btd, torch.tensor(lens, dtype=torch.int32).cuda(), max(lens), sum(lens))
        say("append_decode step", s, "lens", lens)
        out = lkv.append_decode(pair.gpu, view, k_new.cuda(), v_new.cuda(), q, sm_scale(D), tau)
        dbg, mask = lkv.decode_attn_debug([pair.gpu], [view], q, sm_scale(D), tau)
        O.append(pair.ref, to_f32_host(k_new), to_f32_host(v_new), np.arange(len(lens) + 1, dtype=np.int32),
                 np.array(lens, np.int32) - 1, bt)
        torch.cuda.synchronize()
        assert torch.equal(dbg, out)
        assert pair.pool_equal(), (s, pair.first_pool_mismatch())
        split = lkv.decode_plan([pair.gpu], [view], len(lens), Hkv * G)
        want, _ = resolved_reference([pair.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm_scale(D),
                                     tau, split, mask, [view.max_len], f"step {s}")
        assert_attention_close(out.cpu().numpy(), want, max_abs_vhat(pair.ref), f"step {s}")


MERGED = [c for c in CASES if c[0][:3] == (128, 64, 6) and c[0][3] in (4, 6) and c[2] == "bf16"]


@pytest.mark.parametrize("case", MERGED, ids=lambda c: "D{}g{}k{}v{}".format(*c[0]) + f"G{c[1]}{c[2]}{c[3]}")
@pytest.mark.parametrize("split", [64, 1024])
def test_append_decode_merged_equals_append_decode(case, split):
    """The split kernel that merges its own splits: three steps in a row, each
    with the pool bit for bit that of lkv_append_decode, the output within
    tolerance of the oracle (the splits are merged G at a time, then the
    groups, so the rounding differs from the merge kernel's within a few fp32
    ulps), and the counters back at zero after every call."""
    fmt, G, qd, kvd = case
    Hkv = 2
    # and one long sequence: 129 splits of 64 tokens, 33 (G 4) or 17 (G 8) workgroup partials
    lens0 = [max(n - 3, 0) for n in LENS] + [8197]
    B = len(lens0)
    rng = np.random.default_rng(47)
    bt, nblk = block_tables([n + 3 for n in lens0], rng)
    a = Pair(*fmt, Hkv, nblk)
    _prefill(a, lens0, Hkv, fmt[0], "bf16", 47, bt, outliers=True)
    b = lkv.Cache(*fmt, Hkv, nblk, pool=a.gpu.pool.clone())
    counters = lkv.merge_counters(b, B)
    btd = torch.tensor(bt).cuda()
    for s in range(3):
        lens = [n + s + 1 if n > 0 else 0 for n in lens0]
        view = lkv.View(btd, torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
        k_new, v_new = inputs.kv_rows(48, 0, B, Hkv, fmt[0], dtype=kvd, step=s)
        q = inputs.queries(49 + s, B, Hkv * G, fmt[0], dtype=qd).cuda()
        tau = 0.0 if s == 0 else 1e-4
        say("append_decode_merged", case, "split", split, "step", s)
        want = lkv.append_decode(a.gpu, view, k_new.cuda(), v_new.cuda(), q, sm_scale(fmt[0]), tau, split)
        got = lkv.append_decode_merged(b, view, k_new.cuda(), v_new.cuda(), q, sm_scale(fmt[0]), tau, split,
                                       counters)
        _, mask = lkv.decode_attn_debug([b], [view], q, sm_scale(fmt[0]), tau, split)
        live = [i for i, n in enumerate(lens) if n > 0]
        O.append(a.ref, to_f32_host(k_new[live]), to_f32_host(v_new[live]), np.arange(len(live) + 1, dtype=np.int32),
                 np.array([lens[i] - 1 for i in live], np.int32), bt[live])
        torch.cuda.synchronize()
        assert torch.equal(b.pool, a.gpu.pool), f"step {s}: pool differs from lkv_append_decode"
        assert a.pool_equal(), (s, a.first_pool_mismatch())
        d = (got - want).abs()
        assert float(d.max()) <= 1e-5 * max_abs_vhat(a.ref), f"step {s}: max |d| {float(d.max())}"
        assert int(counters.abs().sum()) == 0, f"step {s}: counters not back at zero"
        assert np.all(got.cpu().numpy()[lens.index(0)] == 0.0)
        ref, _ = resolved_reference([a.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm_scale(fmt[0]),
                                    tau, split, mask, [view.max_len], f"step {s}")
        assert_attention_close(got.cpu().numpy(), ref, max_abs_vhat(a.ref), f"{case} split {split} step {s}")


@pytest.mark.parametrize("G", [4, 8])
def test_append_decode_merged_many_workgroup_partials(G):
    """Rows with more than 64 workgroup partials (the last workgroup merges
    them in chunks of 64): one step, pool bit-exact, output within tolerance
    of the oracle, counters back at zero."""
    fmt, Hkv, split = (128, 64, 6, 4), 2, 64
    # 64 G + 1 and 130 G splits of 64 tokens (65 and 130 partials), and a short row
    lens0 = [64 * G * 64 + 63, 130 * G * 64 - 1, 300]
    B = len(lens0)
    rng = np.random.default_rng(53)
    bt, nblk = block_tables([n + 1 for n in lens0], rng)
    a = Pair(*fmt, Hkv, nblk)
    _prefill(a, lens0, Hkv, fmt[0], "bf16", 53, bt, outliers=True)
    counters = lkv.merge_counters(a.gpu, B)
    lens = [n + 1 for n in lens0]
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    k_new, v_new = inputs.kv_rows(54, 0, B, Hkv, fmt[0])
    q = inputs.queries(55, B, Hkv * G, fmt[0]).cuda()
    say("append_decode_merged many partials G", G, "lens", lens)
    got = lkv.append_decode_merged(a.gpu, view, k_new.cuda(), v_new.cuda(), q, sm_scale(fmt[0]), 0.0, split, counters)
    O.append(a.ref, to_f32_host(k_new), to_f32_host(v_new), np.arange(B + 1, dtype=np.int32), np.array(lens0, np.int32),
             bt)
    torch.cuda.synchronize()
    assert a.pool_equal(), a.first_pool_mismatch()
    assert int(counters.abs().sum()) == 0
    ref = O.decode([a.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm_scale(fmt[0]), 0.0, split)
    assert_attention_close(got.cpu().numpy(), ref, max_abs_vhat(a.ref), f"G {G}")


def test_append_decode_merged_rejects_more_than_256_workgroup_partials():
    fmt, G, Hkv = (128, 64, 6, 4), 4, 2
    lens = [1024 * 64 + 1, 100]  # 1025 splits of 64 tokens: 257 workgroups of 4
    bt, nblk = block_tables(lens, np.random.default_rng(50))
    c = lkv.Cache(*fmt, Hkv, nblk)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    k_new, v_new = inputs.kv_rows(51, 0, 2, Hkv, 128)
    q = inputs.queries(52, 2, Hkv * G, 128).cuda()
    counters = lkv.merge_counters(c, 2)
    with pytest.raises(lkv.LkvError) as e:
        lkv.append_decode_merged(c, view, k_new.cuda(), v_new.cuda(), q, sm_scale(128), 0.0, 64, counters)
    assert e.value.status == lkv.EUNSUPPORTED
    torch.cuda.synchronize()
    assert int(counters.abs().sum()) == 0 and not c.pool.any()  # nothing was launched


@pytest.mark.parametrize("case", CASES, ids=lambda c: "D{}g{}k{}v{}".format(*c[0]) + f"G{c[1]}{c[2]}{c[3]}")
@pytest.mark.parametrize("split", [64, 1024])
def test_ragged_hint_merge_equals_full_merge(case, split):
    """With a view's sum_len hint on a ragged batch the merge reads only the
    splits that hold tokens; the decode step's output and pool, and a decode
    over the same cache, are bit-equal to the calls without the hint, which
    read every split (an empty sequence, lengths on block and split edges)."""
    fmt, G, qd, kvd = case
    D = fmt[0]
    Hkv = 2
    lens = LENS
    B = len(lens)
    pair, hinted_cache, bt = _caches(fmt, lens, Hkv, 61)
    q = inputs.queries(62, B, Hkv * G, D, dtype=qd).cuda()
    btd, lt = torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda()
    plain = lkv.View(btd, lt, max(lens))
    hinted = lkv.View(btd, lt, max(lens), sum(lens))
    sm = sm_scale(D)
    k_new, v_new = inputs.kv_rows(63, 0, B, Hkv, D, dtype=kvd)
    say("ragged hint", case, "split", split)
    got = lkv.append_decode(hinted_cache, hinted, k_new.cuda(), v_new.cuda(), q, sm, 0.0, split)
    want = lkv.append_decode(pair.gpu, plain, k_new.cuda(), v_new.cuda(), q, sm, 0.0, split)
    again = lkv.decode_attn([hinted_cache], [hinted], q, sm, 0.0, split)
    base = lkv.decode_attn([hinted_cache], [plain], q, sm, 0.0, split)
    torch.cuda.synchronize()
    assert torch.equal(hinted_cache.pool, pair.gpu.pool)
    assert torch.equal(got, want), f"decode step: max |d| {float((got - want).abs().max())}"
    assert torch.equal(again, base), f"decode: max |d| {float((again - base).abs().max())}"
    assert torch.equal(again, got)


N_RAGGED = 120


def test_seeded_random_ragged_steps():
    """Seeded random decode steps of ragged batches (up to 64 sequences,
    empty ones and block and split edges among them) in the fused formats:
    with the sum_len hint (the compact order and the merge over the splits
    with tokens) the pool and the output are bit-equal to the calls without
    it (the full grid), with and without the skip; without the skip the
    output is within tolerance of the oracle.  Split sizes are drawn, or
    taken from lkv_decode_plan_lens."""
    rng = np.random.default_rng(4077)
    edge = [0, 1, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1024, 1025]
    for i in range(N_RAGGED):
        fmt = ((128, 64, 6, 4), (128, 64, 6, 6), (128, 32, 6, 4))[rng.integers(3)]
        G = int(rng.choice([4, 8]))
        Hkv = int(rng.choice([1, 2, 4]))
        B = int(rng.choice([2, 5, 17, 64])) if rng.random() < 0.5 else int(rng.integers(1, 65))
        lens = [int(rng.choice(edge)) if rng.random() < 0.4 else int(rng.integers(1, 3000)) for _ in range(B)]
        lens[0] = max(lens[0], 1)
        tau = float(rng.choice([0.0, 0.0, 1e-4, 2e-3]))
        seed = int(rng.integers(1, 10**6))
        pair, hinted_cache, bt = _caches(fmt, lens, Hkv, seed)
        D = fmt[0]
        q = inputs.queries(seed + 1, B, Hkv * G, D).cuda()
        btd, lt = torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda()
        plain = lkv.View(btd, lt, max(lens))
        hinted = lkv.View(btd, lt, max(lens), sum(lens))
        if rng.random() < 0.4:
            split = lkv.decode_plan_lens(hinted_cache, hinted, lens, Hkv * G)
        else:
            split = int(rng.choice([64, 128, 256, 512, 1024]))
        what = f"case {i}: {fmt} G{G} Hkv{Hkv} B{B} lens {lens} split {split} tau {tau} seed {seed}"
        say(what)
        k_new, v_new = inputs.kv_rows(seed + 2, 0, B, Hkv, D)
        sm = sm_scale(D)
        got = lkv.append_decode(hinted_cache, hinted, k_new.cuda(), v_new.cuda(), q, sm, tau, split)
        want = lkv.append_decode(pair.gpu, plain, k_new.cuda(), v_new.cuda(), q, sm, tau, split)
        torch.cuda.synchronize()
        assert torch.equal(hinted_cache.pool, pair.gpu.pool), what
        assert torch.equal(got, want), f"{what}: max |d| {float((got - want).abs().max())}"
        if tau == 0.0:
            live = [b for b, n in enumerate(lens) if n > 0]
            O.append(pair.ref, to_f32_host(k_new[live]), to_f32_host(v_new[live]),
                     np.arange(len(live) + 1, dtype=np.int32), np.array([lens[b] - 1 for b in live], np.int32),
                     bt[live])
            assert pair.pool_equal(), (what, pair.first_pool_mismatch())
            ref = O.decode([pair.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm, 0.0, split)
            assert_attention_close(got.cpu().numpy(), ref, max_abs_vhat(pair.ref), what)


@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("tau,split", [(0.0, 64), (1e-4, 256)])
def test_append_decode_merged_tiered_segments(G, tau, split):
    """The one-launch step over a tiered cache: HIGH (K6V6) takes the new
    rows, HIGH and MID (K6V4) are read, the splits merged in the kernel.
    Ragged lengths, a sequence with no HIGH token (nothing appended), one
    whose only HIGH token is the new one and whose MID is empty.  Both pools
    bit-exact with the oracle's append, the output within tolerance of the
    oracle's decode over both segments (skip decisions resolved through the
    debug entry point) and within 1e-5 max|v_hat| of lkv_decode_attn over
    the same pools, the counters back at zero."""
    from tests.gpu_common import resolved_reference

    D, g, Hkv = 128, 64, 2
    rng = np.random.default_rng(61)
    lens_h = [0, 131, 701, 65, 1]  # after the new row
    lens_m = [900, 1, 2100, 65, 0]
    B = len(lens_h)
    pairs, views, bts = [], [], []
    for vb, lens, pre, seed in ((6, lens_h, [max(n - 1, 0) for n in lens_h], 62), (4, lens_m, lens_m, 63)):
        bt, nblk = block_tables([max(n, 1) for n in lens], rng)
        pair = Pair(D, g, 6, vb, Hkv, nblk)
        _prefill(pair, pre, Hkv, D, "bf16", seed, bt, outliers=True)
        pairs.append(pair)
        bts.append(bt)
        views.append(lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(max(lens), 1)))
    k_new, v_new = inputs.kv_rows(64, 0, B, Hkv, D)
    q = inputs.queries(65, B, Hkv * G, D).cuda()
    counters = lkv.merge_counters(pairs[0].gpu, B)
    say("append_decode_merged tiered G", G, "tau", tau, "split", split)
    got = lkv.append_decode_merged([p.gpu for p in pairs], views, k_new.cuda(), v_new.cuda(), q, sm_scale(D), tau,
                                   split, counters)
    again, mask = lkv.decode_attn_debug([p.gpu for p in pairs], views, q, sm_scale(D), tau, split)
    live = [b for b in range(B) if lens_h[b] > 0]
    O.append(pairs[0].ref, to_f32_host(k_new[live]), to_f32_host(v_new[live]), np.arange(len(live) + 1, dtype=np.int32),
             np.array([lens_h[b] - 1 for b in live], np.int32), bts[0][live])
    torch.cuda.synchronize()
    assert pairs[0].pool_equal(), pairs[0].first_pool_mismatch()
    assert pairs[1].pool_equal(), pairs[1].first_pool_mismatch()
    assert int(counters.abs().sum()) == 0
    vmax = max(max_abs_vhat(p.ref) for p in pairs)
    assert float((got - again).abs().max()) <= 1e-5 * vmax
    want, _ = resolved_reference([p.ref for p in pairs], bts, [np.array(lens_h, np.int32), np.array(lens_m, np.int32)],
                                 to_f32_host(q), sm_scale(D), tau, split, mask, [v.max_len for v in views],
                                 f"tiered G {G}")
    assert_attention_close(got.cpu().numpy(), want, vmax, f"tiered G {G} tau {tau}")


def test_append_decode_merged_rejects_other_segment_pairs():
    """Two segments must be {K6V6, K6V4}: another pair is LKV_EUNSUPPORTED
    with nothing launched; three segments are LKV_EINVAL."""
    D, g, Hkv, G = 128, 64, 2, 4
    lens = [100, 300]
    bt, nblk = block_tables(lens, np.random.default_rng(66))
    a, b = lkv.Cache(D, g, 6, 4, Hkv, nblk), lkv.Cache(D, g, 6, 4, Hkv, nblk)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    k_new, v_new = inputs.kv_rows(67, 0, 2, Hkv, D)
    q = inputs.queries(68, 2, Hkv * G, D).cuda()
    counters = lkv.merge_counters(a, 2)
    with pytest.raises(lkv.LkvError) as e:
        lkv.append_decode_merged([a, b], [view, view], k_new.cuda(), v_new.cuda(), q, sm_scale(D), 0.0, 64, counters)
    assert e.value.status == lkv.EUNSUPPORTED
    with pytest.raises(lkv.LkvError) as e:
        lkv.append_decode_merged([a, b, a], [view, view, view], k_new.cuda(), v_new.cuda(), q, sm_scale(D), 0.0, 64,
                                 counters)
    assert e.value.status == lkv.EINVAL
    torch.cuda.synchronize()
    assert int(counters.abs().sum()) == 0 and not a.pool.any() and not b.pool.any()


N_RAGGED_MERGED = 40


def test_seeded_random_ragged_steps_one_launch():
    """Seeded random decode steps of ragged batches (up to 64 sequences,
    empty ones and block and split edges among them) through the one-launch
    step in compact order (the sum_len hint): pool bit-equal to the two-launch
    step's, output within 1e-5 max|v_hat| of it (the same skip decisions, the
    splits merged in another order) and, without the skip, within tolerance
    of the oracle; counters back at zero.  Split sizes are drawn, or taken
    from lkv_decode_plan_lens."""
    rng = np.random.default_rng(4099)
    edge = [0, 1, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1024, 1025]
    for i in range(N_RAGGED_MERGED):
        fmt = ((128, 64, 6, 4), (128, 64, 6, 6))[rng.integers(2)]
        G = int(rng.choice([4, 8]))
        Hkv = int(rng.choice([1, 2, 4]))
        B = int(rng.choice([2, 5, 17, 64])) if rng.random() < 0.5 else int(rng.integers(1, 65))
        lens = [int(rng.choice(edge)) if rng.random() < 0.4 else int(rng.integers(1, 3000)) for _ in range(B)]
        lens[0] = max(lens[0], 1)
        tau = float(rng.choice([0.0, 0.0, 1e-4, 2e-3]))
        seed = int(rng.integers(1, 10**6))
        pair, cache, bt = _caches(fmt, lens, Hkv, seed)
        D = fmt[0]
        q = inputs.queries(seed + 1, B, Hkv * G, D).cuda()
        btd, lt = torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda()
        hinted = lkv.View(btd, lt, max(lens), sum(lens))
        if rng.random() < 0.5:
            split = lkv.decode_plan_lens(cache, hinted, lens, Hkv * G)
        else:
            split = int(rng.choice([64, 128, 256, 512, 1024]))
        what = f"case {i}: {fmt} G{G} Hkv{Hkv} B{B} lens {lens} split {split} tau {tau} seed {seed}"
        say(what)
        k_new, v_new = inputs.kv_rows(seed + 2, 0, B, Hkv, D)
        sm = sm_scale(D)
        counters = lkv.merge_counters(cache, B)
        want = lkv.append_decode(cache, hinted, k_new.cuda(), v_new.cuda(), q, sm, tau, split)
        pool = cache.pool.clone()
        got = lkv.append_decode_merged(cache, hinted, k_new.cuda(), v_new.cuda(), q, sm, tau, split, counters)
        live = [b for b, n in enumerate(lens) if n > 0]
        O.append(pair.ref, to_f32_host(k_new[live]), to_f32_host(v_new[live]), np.arange(len(live) + 1, dtype=np.int32),
                 np.array([lens[b] - 1 for b in live], np.int32), bt[live])
        torch.cuda.synchronize()
        assert torch.equal(cache.pool, pool), f"{what}: the re-appended rows changed the pool"
        assert int(counters.abs().sum()) == 0, f"{what}: counters not back at zero"
        vmax = max_abs_vhat(pair.ref)
        d = float((got - want).abs().max())
        assert d <= 1e-5 * vmax, f"{what}: max |d| {d} against the two-launch step"
        assert np.all(got.cpu().numpy()[[b for b, n in enumerate(lens) if n == 0]] == 0.0), what
        if tau == 0.0:
            pair.gpu.pool.copy_(cache.pool)
            assert pair.pool_equal(), (what, pair.first_pool_mismatch())
            ref = O.decode([pair.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm, 0.0, split)
            assert_attention_close(got.cpu().numpy(), ref, vmax, what)
