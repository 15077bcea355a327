"""Accumulated attention scores from decode (lkv_decode_attn_scores) against
the oracle: every live token's softmax weight summed over the query heads,
added to score_acc[segment][b][token]."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_kv_cache_token_amd import inputs, lkv
from tests.gpu_common import Pair, say, sm_scale, to_f32_host
from tests.oracle_cases import block_tables

pytestmark = pytest.mark.gpu


def _prefill(pair, lens, Hkv, D, seed, bt):
    rows = [inputs.kv_rows(seed, b, n, Hkv, D, dtype="bf16") for b, n in enumerate(lens)]
    k = torch.cat([r[0] for r in rows])
    v = torch.cat([r[1] for r in rows])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pair.append(k, v, cu, np.zeros(len(lens), np.int32), bt)


def assert_scores_close(got, want, what=""):
    """Per token: |d| <= 1e-4 * score + 1e-9 * (sum of the sequence's
    scores = Hq): fp32 exponentials of fp32 scores against fp64."""
    got = np.asarray(got, np.float64)
    d = np.abs(got - want)
    bound = 1e-4 * np.abs(want) + 1e-9 * want.sum(axis=-1, keepdims=True)
    assert np.all(np.isfinite(got)), what
    bad = np.argwhere(d > bound)
    assert bad.size == 0, f"{what}: {len(bad)} tokens off, first {tuple(bad[0])}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


CASES = [  # (D, g, kb, vb, G, q dtype): the matrix-core, fp16 and generic kernels
    (128, 64, 6, 4, 4, "bf16"),
    (128, 64, 6, 4, 8, "bf16"),
    (128, 64, 6, 6, 4, "bf16"),
    (128, 64, 16, 16, 8, "bf16"),
    (128, 64, 16, 16, 4, "f32"),
    (64, 32, 6, 4, 4, "bf16"),
    (128, 64, 6, 4, 4, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "d{}g{}k{}v{}G{}{}".format(*c))
@pytest.mark.parametrize("tau", [0.0, 1e-4])
def test_scores_one_segment(case, tau):
    D, g, kb, vb, G, qd = case
    Hkv = 2
    lens = [1, 64, 300, 1500, 0]
    rng = np.random.default_rng(60)
    bt, nblk = block_tables([max(n, 1) for n in lens], rng)
    pair = Pair(D, g, kb, vb, Hkv, nblk)
    _prefill(pair, lens, Hkv, D, 60, bt)
    q = inputs.queries(61, len(lens), Hkv * G, D, dtype=qd)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    stride = 1600
    sentinel = np.zeros((1, len(lens), stride))  # 0.25 past each sequence's end
    for b, n in enumerate(lens):
        sentinel[0, b, n:] = 0.25
    acc = torch.tensor(sentinel, dtype=torch.float32, device="cuda")
    split = 256
    say("decode scores", case, "tau", tau)
    out = lkv.decode_attn_scores([pair.gpu], [view], q.cuda(), acc, sm_scale(D), tau, split)
    ref_out = lkv.decode_attn([pair.gpu], [view], q.cuda(), sm_scale(D), tau, split)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)  # the output is exactly lkv_decode_attn's
    want = sentinel.copy()
    O.decode([pair.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm_scale(D), tau, split, score_acc=want)
    got = acc.cpu().numpy().astype(np.float64)
    for b, n in enumerate(lens):
        assert np.all(got[0, b, n:] == 0.25), "entries past the end must stay untouched"
    assert_scores_close(got - sentinel, want - sentinel, f"{case} tau {tau}")


@pytest.mark.parametrize("G", [4, 8])
def test_scores_tiered_segments_accumulate(G):
    """HIGH (K6V6) + MID (K6V4) segments in one launch, with the skip; two
    calls accumulate."""
    D, g, Hkv = 128, 64, 2
    rng = np.random.default_rng(70)
    lens_h, lens_m = [0, 130, 700, 64], [900, 1, 2100, 65]
    pairs, views, ref = [], [], []
    for vb, lens, seed in ((6, lens_h, 71), (4, lens_m, 72)):
        bt, nblk = block_tables([max(n, 1) for n in lens], rng)
        pair = Pair(D, g, 6, vb, Hkv, nblk)
        _prefill(pair, lens, Hkv, D, seed, bt)
        pairs.append(pair)
        views.append(lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens)))
        ref.append((bt, np.array(lens, np.int32)))
    q = inputs.queries(73, 4, Hkv * G, D)
    acc = torch.zeros((2, 4, 2200), dtype=torch.float32, device="cuda")
    say("decode scores tiered G", G)
    for _ in range(2):
        lkv.decode_attn_scores([p.gpu for p in pairs], views, q.cuda(), acc, sm_scale(D), 1e-5, 256)
    torch.cuda.synchronize()
    want = np.zeros((2, 4, 2200))
    for _ in range(2):
        O.decode([p.ref for p in pairs], [r[0] for r in ref], [r[1] for r in ref], to_f32_host(q), sm_scale(D), 1e-5,
                 256, score_acc=want)
    got = acc.cpu().numpy()
    assert_scores_close(got, want, f"tiered G{G}")
    # every head's weights sum to one over both segments: 2 calls x Hq
    assert np.allclose(got.sum(axis=(0, 2)), 2 * Hkv * G, rtol=1e-5)


def test_scores_reject_a_short_stride():
    D, g, Hkv = 128, 64, 1
    bt, nblk = block_tables([300])
    pair = Pair(D, g, 6, 4, Hkv, nblk)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor([300], dtype=torch.int32).cuda(), 300)
    q = torch.zeros((1, 4, D), dtype=torch.bfloat16, device="cuda")
    acc = torch.zeros((1, 1, 299), dtype=torch.float32, device="cuda")
    with pytest.raises(lkv.LkvError):
        lkv.decode_attn_scores([pair.gpu], [view], q, acc, sm_scale(D), 0.0, 64)


def test_scores_drive_the_tier_update():
    """The loop the tiers are for: decode with scores for three steps, tier
    the K6V6 cache on the accumulated scores, decode HIGH + MID.  The oracle
    tiers from the same fp32 scores: tiers, counts and pools bit-exact, then
    attention within tolerance."""
    from tests.gpu_common import assert_attention_close, max_abs_vhat

    D, g, Hkv, G = 128, 64, 2, 4
    lens = [700, 1300, 64]
    rng = np.random.default_rng(80)
    bt, nblk = block_tables(lens, rng)
    src = Pair(D, g, 6, 6, Hkv, nblk)
    _prefill(src, lens, Hkv, D, 81, bt)
    stride = 1408
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    acc = torch.zeros((1, len(lens), stride), dtype=torch.float32, device="cuda")
    want_acc = np.zeros((1, len(lens), stride))
    say("decode scores, three steps")
    for step in range(3):
        q = inputs.queries(82, len(lens), Hkv * G, D, step=step)
        lkv.decode_attn_scores([src.gpu], [view], q.cuda(), acc, sm_scale(D), 0.0, 256)
        O.decode([src.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm_scale(D), 0.0, 256,
                 score_acc=want_acc)
    torch.cuda.synchronize()
    assert_scores_close(acc.cpu().numpy(), want_acc, "three steps")
    # the thresholds bound one head's weight at one step: tier on the mean
    # weight per head and step.  Both sides read the oracle's scores,
    # rounded to fp32: no oracle input comes from the GPU
    scores_h = np.ascontiguousarray(want_acc[0] / (3 * Hkv * G), np.float32)
    scores = torch.from_numpy(scores_h).cuda()
    tl, th = lkv.default_thresholds(max(lens))
    hbt, hn = block_tables(lens, rng)
    mbt, mn = block_tables(lens, rng)
    h, m = Pair(D, g, 6, 6, Hkv, hn), Pair(D, g, 6, 4, Hkv, mn)
    tiers = torch.full((len(lens), stride), 255, dtype=torch.uint8, device="cuda")
    nh = torch.zeros(len(lens), dtype=torch.int32, device="cuda")
    nm = torch.zeros_like(nh)
    say("tier update on decode scores")
    lkv.tier_update(src.gpu, view, scores, tl, th, h.gpu, torch.tensor(hbt).cuda(), m.gpu, torch.tensor(mbt).cuda(),
                    nh, nm, tiers)
    torch.cuda.synchronize()
    t_ref, nh_ref, nm_ref = O.tier_update(src.ref, bt, np.array(lens, np.int32), scores_h, tl, th,
                                          h.ref, hbt, m.ref, mbt)
    assert np.array_equal(tiers.cpu().numpy(), t_ref)
    assert np.array_equal(nh.cpu().numpy(), nh_ref) and np.array_equal(nm.cpu().numpy(), nm_ref)
    assert 0 < int(nh_ref.sum()) < int(nm_ref.sum())  # HIGH and MID both occur
    assert h.pool_equal() and m.pool_equal()
    q = inputs.queries(83, len(lens), Hkv * G, D)
    views = [lkv.View(torch.tensor(hbt).cuda(), nh, int(nh_ref.max())),
             lkv.View(torch.tensor(mbt).cuda(), nm, int(nm_ref.max()))]
    say("decode the tiered segments")
    got = lkv.decode_attn([h.gpu, m.gpu], views, q.cuda(), sm_scale(D), tl, 128).cpu().numpy()
    want = O.decode([h.ref, m.ref], [hbt, mbt], [nh_ref, nm_ref], to_f32_host(q), sm_scale(D), tl, 128)
    assert_attention_close(got, want, max(max_abs_vhat(h.ref), max_abs_vhat(m.ref)), "tiered after scores")
