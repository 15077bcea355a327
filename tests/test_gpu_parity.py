"""GPU parity of the three calls against the oracle on small seeded cases
that still span several blocks and a ragged tail.  Codes, scales, zeros,
tiers and counts bit-exact; attention within max|d| <= 1e-3 max|v_hat| and
relative L2 <= 1e-4."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_kv_cache_token_amd import inputs, lkv
from tests.gpu_common import (Pair, assert_attention_close, max_abs_vhat, resolved_reference, say, sm_scale,
                              to_f32_host)
from tests.oracle_cases import block_tables

pytestmark = pytest.mark.gpu

FORMATS = [(64, 32, 6, 4), (128, 64, 6, 4), (128, 64, 6, 6), (128, 64, 4, 4), (128, 32, 4, 6),
           (64, 16, 6, 6), (128, 64, 16, 16), (64, 32, 16, 16)]


def _fmt_id(f):
    return "D{}g{}k{}v{}".format(*f)


def _prefill(pair: Pair, lens, Hkv, D, dtype, seed, bt, outliers=False):
    """Append every sequence's rows in one call, and return the inputs."""
    K, V = [], []
    out = inputs.outlier_channels(seed, Hkv, D) if outliers else None
    for b, n in enumerate(lens):
        k, v = inputs.kv_rows(seed, b, int(n), Hkv, D, dtype=dtype, outliers=out)
        K.append(k)
        V.append(v)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pair.append(torch.cat(K), torch.cat(V), cu, np.zeros(len(lens), np.int32), bt)
    return K, V


@pytest.mark.parametrize("fmt", FORMATS, ids=_fmt_id)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_append_pool_bit_exact(fmt, dtype):
    D, g, kb, vb = fmt
    rng = np.random.default_rng(1)
    lens = [1, 63, 64, 65, 300]
    Hkv = 2
    bt, nblk = block_tables([n + 70 for n in lens], rng)
    pair = Pair(D, g, kb, vb, Hkv, nblk)
    say("append prefill", fmt, dtype)
    _prefill(pair, lens, Hkv, D, dtype, 7, bt, outliers=True)
    assert pair.pool_equal(), pair.first_pool_mismatch()
    # then appends of 1 and of 5 rows at ragged positions into partial blocks
    for step, t in enumerate([1, 5, 1]):
        say("append step", step, t)
        k, v = inputs.kv_rows(7, 99, len(lens) * t, Hkv, D, dtype=dtype, step=step + 1)
        cu = np.arange(len(lens) + 1, dtype=np.int32) * t
        pair.append(k, v, cu, np.array(lens, np.int32), bt)
        lens = [n + t for n in lens]
        assert pair.pool_equal(), pair.first_pool_mismatch()


def test_append_special_groups_bit_exact():
    """Constant, one-sided, tie and zero groups (fp32 inputs)."""
    D, g = 128, 64
    rows = []
    consts = [0.0, -0.0, 1e-30, -1e-30, 1.0, -1.0, np.pi, 1e30, -1e30, 3.3895313892515355e38]
    for c in consts:
        rows.append(np.full(D, c, np.float32))
    rng = np.random.default_rng(3)
    rows.append(rng.uniform(0.5, 2.0, D).astype(np.float32))
    rows.append(-rng.uniform(0.5, 2.0, D).astype(np.float32))
    tie = np.zeros(D, np.float32)
    tie[:11] = [-7.75, 8.0, 0.125, 0.375, 0.625, 0.875, 1.0, -1.0, 0.0, -0.125, -0.375]
    tie[64:75] = tie[:11]
    rows.append(tie)
    rows.append((1.0 + 1e-6 * rng.standard_normal(D)).astype(np.float32))
    x = torch.tensor(np.stack(rows))[:, None, :]
    n = x.shape[0]
    for kb, vb in [(6, 4), (4, 6), (16, 16)]:
        pair = Pair(D, g, kb, vb, 1, 2)
        say("append special groups", kb, vb)
        pair.append(x, -x, [0, n], [0], np.array([[0, 1]], np.int32))
        assert pair.pool_equal(), pair.first_pool_mismatch()


def _tie_rows(D, g, bits, rng):
    """fp32 rows whose groups have power-of-two scales, so that -lo / s and
    x / s land exactly on half-integers (and a few ulps away from them),
    plus groups of subnormal values and groups whose range overflows."""
    qmax = (1 << bits) - 1
    rows = []
    for e in (-3, 0, 5):
        s = 2.0 ** e
        row = np.zeros(D, np.float32)
        for g0 in range(0, D, g):
            k = rng.integers(-qmax // 2, qmax // 2, g).astype(np.float64) + 0.5
            vals = (k * s).astype(np.float32)
            vals[0], vals[1] = -(qmax / 2) * s, (qmax / 2) * s  # range qmax * s: the scale is s, -lo / s a tie
            near = rng.random(g) < 0.3
            vals[2:][near[2:]] = np.nextafter(vals[2:][near[2:]], np.float32(np.inf) * rng.choice([-1, 1], near[2:].sum()))
            row[g0:g0 + g] = vals
        rows.append(row)
    rows.append((rng.standard_normal(D) * 1e-40).astype(np.float32))      # subnormal scales
    big = rng.uniform(-3.3e38, 3.3e38, D).astype(np.float32)
    big[::g] = -3.3e38
    big[1::g] = 3.3e38                                                     # hi - lo overflows
    rows.append(big)
    return rows


@pytest.mark.parametrize("D,g", [(128, 64), (128, 32), (128, 16), (64, 32), (64, 16)])
def test_append_quotient_ties_bit_exact(D, g):
    """Half-integer quotients (exact ties and their neighbours), subnormal
    scales and overflowing ranges: the lanes the fast quantiser defers to
    correctly rounded division."""
    rng = np.random.default_rng(31)
    for kb, vb in [(6, 4), (4, 6), (6, 6)]:
        rows = _tie_rows(D, g, kb, rng) + _tie_rows(D, g, vb, rng)
        x = torch.tensor(np.stack(rows))[:, None, :]
        n = x.shape[0]
        pair = Pair(D, g, kb, vb, 1, 1)
        say("append quotient ties", D, g, kb, vb)
        pair.append(x, -x, [0, n], [0], np.array([[0]], np.int32))
        assert pair.pool_equal(), pair.first_pool_mismatch()


def test_append_unaligned_inputs_bit_exact():
    """K and V views one element off their allocation's alignment."""
    D, g, Hkv = 128, 64, 2
    lens = [70, 3]
    rng = np.random.default_rng(32)
    bt, nblk = block_tables([n + 64 for n in lens], rng)
    for dtype in ("bf16", "f32"):
        pair = Pair(D, g, 6, 4, Hkv, nblk)
        k, v = inputs.kv_rows(33, 0, sum(lens), Hkv, D, dtype=dtype)
        kk = torch.empty(k.numel() + 1, dtype=k.dtype, device="cuda")[1:].view(k.shape)
        vv = torch.empty(v.numel() + 1, dtype=v.dtype, device="cuda")[1:].view(v.shape)
        kk.copy_(k.cuda())
        vv.copy_(v.cuda())
        cu = np.array([0, lens[0], sum(lens)], np.int32)
        say("append unaligned", dtype)
        lkv.quant_append(pair.gpu, kk, vv, torch.tensor(cu).cuda(), torch.zeros(2, dtype=torch.int32).cuda(),
                         torch.tensor(bt).cuda(), max(lens))
        O.append(pair.ref, to_f32_host(k), to_f32_host(v), cu, np.zeros(2, np.int32), bt)
        assert pair.pool_equal(), pair.first_pool_mismatch()


def _decode_case(fmt, G, qdtype, lens, tau, split, seed=5, Hkv=2, nseg=1):
    """fmt: one format for every segment, or a list with one per segment."""
    fmts = list(fmt) if isinstance(fmt, list) else [fmt] * nseg
    nseg = len(fmts)
    D = fmts[0][0]
    rng = np.random.default_rng(seed)
    pairs, views, ref_views = [], [], []
    for s in range(nseg):
        _, g, kb, vb = fmts[s]
        seg_lens = [max(0, n - 37 * s) for n in lens]
        bt, nblk = block_tables([max(n, 1) for n in seg_lens], rng)
        pair = Pair(D, g, kb, vb, Hkv, nblk)
        _prefill(pair, seg_lens, Hkv, D, "bf16", seed + s, bt, outliers=True)
        pairs.append(pair)
        lt = torch.tensor(seg_lens, dtype=torch.int32)
        views.append(lkv.View(torch.tensor(bt).cuda(), lt.cuda(), max(seg_lens)))
        ref_views.append((bt, np.array(seg_lens, np.int32)))
    q = inputs.queries(seed, len(lens), Hkv * G, D, dtype=qdtype)
    sm = sm_scale(D)
    say("decode", fmt, "G", G, qdtype, "lens", lens, "tau", tau, "split", split, "nseg", nseg)
    out = lkv.decode_attn([p.gpu for p in pairs], views, q.cuda(), sm, tau, split)
    torch.cuda.synchronize()
    if tau > 0:
        # the skip decisions too: the oracle takes the GPU's near the bound
        dbg, mask = lkv.decode_attn_debug([p.gpu for p in pairs], views, q.cuda(), sm, tau, split)
        torch.cuda.synchronize()
        assert torch.equal(dbg, out), "the debug entry point must give the production output bit for bit"
        want, stats = resolved_reference([p.ref for p in pairs], [v[0] for v in ref_views],
                                         [v[1] for v in ref_views], to_f32_host(q), sm, tau,
                                         split or lkv.decode_plan([p.gpu for p in pairs], views, len(lens),
                                                                  Hkv * G),
                                         mask, [v.max_len for v in views])
        say("  skip pairs live / flipped near the bound / largest flipped margin:", *stats)
    else:
        want = O.decode([p.ref for p in pairs], [v[0] for v in ref_views], [v[1] for v in ref_views],
                        to_f32_host(q), sm, tau, split)
    vmax = max(max_abs_vhat(p.ref) for p in pairs)
    return out.cpu().numpy(), want, vmax


@pytest.mark.parametrize("lens", [[2100, 64, 9], [4096, 1, 3000], [4100, 64, 9], [5, 2700, 9000]],
                         ids=["33_splits", "64_splits", "65_splits", "141_splits"])
@pytest.mark.parametrize("tau", [0.0, 1e-4])
def test_decode_parity_many_splits(lens, tau):
    """More than 32 splits of a sequence: at head_dim 128 one wave merges up
    to 64 (a split per lane), four waves up to 128, sixteen beyond."""
    got, want, vmax = _decode_case((128, 64, 6, 4), 4, "bf16", lens, tau, 64)
    assert_attention_close(got, want, vmax, f"{max(lens) // 64 + 1} splits tau {tau}")


@pytest.mark.parametrize("fmt", FORMATS, ids=_fmt_id)
@pytest.mark.parametrize("G", [1, 4, 8])
def test_decode_parity_formats(fmt, G):
    got, want, vmax = _decode_case(fmt, G, "bf16", [1, 64, 200, 777], 0.0, 128)
    assert_attention_close(got, want, vmax, f"{fmt} G{G}")


@pytest.mark.parametrize("qdtype", ["f32", "bf16"])
@pytest.mark.parametrize("split", [64, 256, 1024])
@pytest.mark.parametrize("tau", [0.0, 1e-5, 2e-4])
def test_decode_parity_splits_and_skip(qdtype, split, tau):
    got, want, vmax = _decode_case((128, 64, 6, 4), 4, qdtype, [5, 700, 1500, 2048], tau, split)
    assert_attention_close(got, want, vmax, f"split {split} tau {tau}")


SKIP_KERNELS = [  # (formats, G, q dtype): every split kernel that applies the skip
    ((128, 64, 6, 4), 4, "bf16"),                        # matrix cores, two-set layout
    ((128, 64, 6, 4), 8, "bf16"),                        # matrix cores, 8-head layout
    ((128, 64, 6, 6), 4, "bf16"),
    ([(128, 64, 6, 6), (128, 64, 6, 4)], 4, "bf16"),     # tiered {HIGH, MID} in one launch
    ([(128, 64, 6, 6), (128, 64, 6, 4)], 8, "bf16"),
    ((128, 64, 16, 16), 8, "bf16"),                      # fp16 layer
    ((128, 64, 16, 16), 4, "f32"),
    ((64, 32, 6, 4), 2, "bf16"),                         # generic kernel
    ((128, 64, 6, 4), 4, "f32"),
]


@pytest.mark.parametrize("case", SKIP_KERNELS, ids=lambda c: f"{c[0]}G{c[1]}{c[2]}".replace(" ", ""))
@pytest.mark.parametrize("tau", [1e-3, 5e-3, 3e-2])
def test_skip_decisions_bit_exact_outside_the_band(case, tau):
    """The skip mask of the debug entry point: every decision outside the
    band fp32 can take either way equals the exact one; with the GPU's
    decisions inside it, the oracle's output matches within tolerance."""
    fmts, G, qd = case
    got, want, vmax = _decode_case(fmts, G, qd, [5, 300, 1500, 2048], tau, 256)
    assert_attention_close(got, want, vmax, f"{case} tau {tau}")


def test_debug_mask_is_empty_without_a_threshold_and_clears_stale_bits():
    """tau_low = 0 skips nothing: the mask comes back all zero (the call
    clears it first), and the output is the production call's."""
    D, g, Hkv, G = 128, 64, 2, 4
    lens = [70, 1000]
    rng = np.random.default_rng(8)
    bt, nblk = block_tables(lens, rng)
    pair = Pair(D, g, 6, 4, Hkv, nblk)
    _prefill(pair, lens, Hkv, D, "bf16", 8, bt)
    q = inputs.queries(8, len(lens), Hkv * G, D).cuda()
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    say("debug mask at tau 0")
    _, m1 = lkv.decode_attn_debug([pair.gpu], [view], q, sm_scale(D), 0.05, 128)
    out0, m0 = lkv.decode_attn_debug([pair.gpu], [view], q, sm_scale(D), 0.0, 128)
    ref = lkv.decode_attn([pair.gpu], [view], q, sm_scale(D), 0.0, 128)
    torch.cuda.synchronize()
    assert int((m1 != 0).sum()) > 0          # at 0.05 most tokens are skipped
    assert int((m0 != 0).sum()) == 0
    assert torch.equal(out0, ref)


@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("qdtype", ["f32", "bf16"])
@pytest.mark.parametrize("split,tau", [(64, 0.0), (1024, 0.0), (256, 1e-5), (1024, 2e-4)])
def test_decode_parity_fp16_layer(G, qdtype, split, tau):
    """The fp16 sensitive-layer format on its matrix-core kernel."""
    got, want, vmax = _decode_case((128, 64, 16, 16), G, qdtype, [5, 700, 1500, 2048], tau, split)
    assert_attention_close(got, want, vmax, f"fp16 G{G} {qdtype} split {split} tau {tau}")


@pytest.mark.parametrize("fmt", [(128, 64, 6, 4), (128, 64, 6, 6), (128, 64, 16, 16), (64, 32, 6, 4)], ids=_fmt_id)
def test_decode_ignores_stale_bytes_past_the_end(fmt):
    """Slots past a sequence's end may hold any bytes (here all 0xFF: NaN
    scales, NaN fp16 values); they must not reach the output."""
    D, g, kb, vb = fmt
    lens = [1, 65, 200, 777]
    rng = np.random.default_rng(21)
    bt, nblk = block_tables(lens, rng)
    pair = Pair(D, g, kb, vb, 2, nblk)
    pair.gpu.pool.fill_(0xFF)
    pair.ref.pool[:] = 0xFF
    _prefill(pair, lens, 2, D, "bf16", 21, bt, outliers=True)
    for G in (4, 8):
        q = inputs.queries(21, len(lens), 2 * G, D)
        view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
        say("decode stale bytes", fmt, "G", G)
        got = lkv.decode_attn([pair.gpu], [view], q.cuda(), sm_scale(D), 0.0, 128).cpu().numpy()
        want = O.decode([pair.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm_scale(D), 0.0, 128)
        # v_hat over the live slots only (the stale ones decode to NaN)
        live = Pair(D, g, kb, vb, 2, nblk)
        _prefill(live, lens, 2, D, "bf16", 21, bt, outliers=True)
        assert_attention_close(got, want, max_abs_vhat(live.ref), f"stale bytes {fmt} G{G}")


@pytest.mark.parametrize("fmt", [(128, 64, 6, 4), (128, 64, 16, 16)], ids=_fmt_id)
def test_decode_split_longer_than_4096_tokens(fmt):
    got, want, vmax = _decode_case(fmt, 4, "bf16", [9000, 5000, 4097], 1e-5, 8192)
    assert_attention_close(got, want, vmax, f"split 8192 {fmt}")


@pytest.mark.parametrize("fmt", [(128, 64, 6, 4), (128, 64, 16, 16)], ids=_fmt_id)
def test_decode_query_not_16_byte_aligned(fmt):
    D, g, kb, vb = fmt
    lens = [300, 129]
    rng = np.random.default_rng(8)
    bt, nblk = block_tables(lens, rng)
    pair = Pair(D, g, kb, vb, 2, nblk)
    _prefill(pair, lens, 2, D, "bf16", 8, bt)
    q = inputs.queries(8, 2, 8, D)
    buf = torch.empty(q.numel() + 1, dtype=q.dtype, device="cuda")
    qv = buf[1:].view(q.shape)
    qv.copy_(q.cuda())
    assert qv.data_ptr() % 16 != 0
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    say("decode unaligned q", fmt)
    got = lkv.decode_attn([pair.gpu], [view], qv, sm_scale(D), 0.0, 64).cpu().numpy()
    want = O.decode([pair.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm_scale(D), 0.0, 64)
    assert_attention_close(got, want, max_abs_vhat(pair.ref), f"unaligned q {fmt}")


def test_decode_skip_changes_the_result_as_the_oracle_does():
    """With a large tau the skip moves the output well beyond the tolerance;
    the GPU follows the oracle with skip, not the oracle without."""
    fmt = (128, 64, 6, 4)
    got, want, vmax = _decode_case(fmt, 4, "bf16", [3000, 2500], 2e-4, 512, seed=9)
    assert_attention_close(got, want, vmax, "skip on")
    _, want0, _ = _decode_case(fmt, 4, "bf16", [3000, 2500], 0.0, 512, seed=9)
    assert np.linalg.norm(want - want0) / np.linalg.norm(want0) > 1e-3


@pytest.mark.parametrize("fmt", [(128, 64, 6, 6), (128, 64, 6, 4)], ids=_fmt_id)
def test_decode_two_segments(fmt):
    got, want, vmax = _decode_case(fmt, 4, "bf16", [40, 300, 129], 1e-5, 64, nseg=2)
    assert_attention_close(got, want, vmax, "two segments")


@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("tau", [0.0, 1e-5])
def test_decode_tiered_segments_one_launch(G, tau):
    """A HIGH (K6V6) and a MID (K6V4) segment, decoded in one matrix-core
    launch: ragged lengths, a sequence whose HIGH segment is empty, and one
    whose MID segment is a single token."""
    D, g, Hkv = 128, 64, 2
    rng = np.random.default_rng(31)
    lens_h = [0, 130, 700, 64]
    lens_m = [900, 1, 2100, 65]
    pairs, views, ref = [], [], []
    for fmt_v, lens, seed in ((6, lens_h, 40), (4, lens_m, 41)):
        bt, nblk = block_tables([max(n, 1) for n in lens], rng)
        pair = Pair(D, g, 6, fmt_v, Hkv, nblk)
        _prefill(pair, lens, Hkv, D, "bf16", seed, bt, outliers=True)
        pairs.append(pair)
        views.append(lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens)))
        ref.append((bt, np.array(lens, np.int32)))
    q = inputs.queries(42, len(lens_h), Hkv * G, D)
    sm = sm_scale(D)
    split = 256
    say("decode tiered one launch G", G, "tau", tau)
    got = lkv.decode_attn([p.gpu for p in pairs], views, q.cuda(), sm, tau, split).cpu().numpy()
    want = O.decode([p.ref for p in pairs], [r[0] for r in ref], [r[1] for r in ref], to_f32_host(q), sm, tau, split)
    vmax = max(max_abs_vhat(p.ref) for p in pairs)
    assert_attention_close(got, want, vmax, f"tiered G{G} tau {tau}")


@pytest.mark.parametrize("fmt", [(128, 64, 6, 4), (128, 64, 6, 6)], ids=_fmt_id)
@pytest.mark.parametrize("G", [4, 8])
def test_decode_one_token_past_a_full_block(fmt, G):
    """65 tokens in one 256-token split (a full block, then one live slot):
    the matrix-core kernels once gave non-finite rows here for K6V6, G 4,
    when the sequence length was held in vector registers."""
    got, want, vmax = _decode_case(fmt, G, "bf16", [65], 0.0, 256, seed=40)
    assert_attention_close(got, want, vmax, f"65 tokens {fmt} G{G}")


def test_decode_empty_and_degenerate():
    """Zero-length sequences give 0; a single token gives its v_hat."""
    fmt = (128, 64, 6, 4)
    got, want, vmax = _decode_case(fmt, 4, "bf16", [0, 1, 0, 65], 0.0, 64)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert_attention_close(got, want, vmax, "empty")


def test_decode_leaves_the_pool_unchanged():
    D, g, kb, vb = 128, 64, 6, 4
    rng = np.random.default_rng(2)
    bt, nblk = block_tables([500, 300], rng)
    pair = Pair(D, g, kb, vb, 2, nblk)
    _prefill(pair, [500, 300], 2, D, "bf16", 3, bt)
    before = pair.gpu.pool.clone()
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor([500, 300], dtype=torch.int32).cuda(), 500)
    q = inputs.queries(3, 2, 8, D).cuda()
    say("decode pool unchanged")
    lkv.decode_attn([pair.gpu], [view], q, sm_scale(D), 1e-4, 128)
    torch.cuda.synchronize()
    assert torch.equal(before, pair.gpu.pool)


def test_decode_is_deterministic():
    fmt = (128, 64, 6, 4)
    a, _, _ = _decode_case(fmt, 8, "bf16", [900, 1300], 1e-5, 256)
    b, _, _ = _decode_case(fmt, 8, "bf16", [900, 1300], 1e-5, 256)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("lens", [[300, 65, 1, 0], [2000, 1500]])
def test_tier_update_bit_exact(lens):
    D, g, Hkv = 128, 64, 2
    rng = np.random.default_rng(4)
    stride = max(lens) + 13
    bt, nblk = block_tables([max(n, 1) for n in lens], rng)
    src = Pair(D, g, 6, 6, Hkv, nblk)
    _prefill(src, lens, Hkv, D, "bf16", 11, bt, outliers=True)
    tl, th = O.default_thresholds(stride)
    scores = torch.zeros(len(lens), stride)
    for b, n in enumerate(lens):
        scores[b, :n] = inputs.tier_scores(11, b, n, tl, th)
    if lens[0] >= 2:
        scores[0, 0], scores[0, 1] = tl, th   # exact boundaries
    hbt, hn = block_tables([max(n, 1) for n in lens], rng)
    mbt, mn = block_tables([max(n, 1) for n in lens], rng)
    h, m = Pair(D, g, 6, 6, Hkv, hn), Pair(D, g, 6, 4, Hkv, mn)
    tiers = torch.full((len(lens), stride), 255, dtype=torch.uint8, device="cuda")
    nh = torch.zeros(len(lens), dtype=torch.int32, device="cuda")
    nm = torch.zeros_like(nh)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    say("tier update", lens)
    lkv.tier_update(src.gpu, view, scores.cuda(), tl, th, h.gpu, torch.tensor(hbt).cuda(), m.gpu,
                    torch.tensor(mbt).cuda(), nh, nm, tiers)
    torch.cuda.synchronize()
    t_ref, nh_ref, nm_ref = O.tier_update(src.ref, bt, np.array(lens, np.int32), scores.numpy(), tl, th,
                                          h.ref, hbt, m.ref, mbt)
    assert np.array_equal(nh.cpu().numpy(), nh_ref) and np.array_equal(nm.cpu().numpy(), nm_ref)
    assert np.array_equal(tiers.cpu().numpy(), t_ref)
    assert h.pool_equal(), h.first_pool_mismatch()
    assert m.pool_equal(), m.first_pool_mismatch()


def test_tier_update_without_room_writes_nothing():
    D, g, Hkv = 128, 64, 1
    lens = [400]
    bt, nblk = block_tables(lens)
    src = Pair(D, g, 6, 6, Hkv, nblk)
    _prefill(src, lens, Hkv, D, "bf16", 12, bt)
    tl, th = O.default_thresholds(400)
    scores = torch.full((1, 400), th)             # every token HIGH: 400 > 64 slots
    h, m = Pair(D, g, 6, 6, Hkv, 1), Pair(D, g, 6, 4, Hkv, 1)
    tiers = torch.zeros((1, 400), dtype=torch.uint8, device="cuda")
    nh = torch.zeros(1, dtype=torch.int32, device="cuda")
    nm = torch.zeros_like(nh)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), 400)
    one = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    say("tier update without room")
    lkv.tier_update(src.gpu, view, scores.cuda(), tl, th, h.gpu, one, m.gpu, one, nh, nm, tiers)
    torch.cuda.synchronize()
    assert nh.item() == -400 and nm.item() == 0
    assert int(h.gpu.pool.abs().sum()) == 0 and int(m.gpu.pool.abs().sum()) == 0
    assert bool((tiers == 2).all())
