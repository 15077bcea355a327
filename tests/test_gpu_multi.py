"""Multi-token queries (lkv_decode_attn_multi) against the oracle: T query
tokens per sequence with a causal mask over the packed cache, for every
split kernel, with and without the sparse-V skip, over one and two
segments.  Attention within max|d| <= 1e-3 max|v_hat| and rel L2 <= 1e-4."""
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


def _queries(seed, B, T, Hq, D, dtype):
    q = inputs.queries(seed, B * T, Hq, D, dtype=dtype)
    return q.reshape(B, T, Hq, D).contiguous()


def _multi_case(fmt, G, qdtype, lens, T, tau, split, seed=40, Hkv=2):
    D, g, kb, vb = fmt
    rng = np.random.default_rng(seed)
    bt, nblk = block_tables(lens, rng)
    pair = Pair(D, g, kb, vb, Hkv, nblk)
    _prefill(pair, lens, Hkv, D, "bf16", seed, bt, outliers=True)
    q = _queries(seed + 1, len(lens), T, Hkv * G, D, qdtype)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    say("multi", fmt, "G", G, qdtype, "T", T, "lens", lens, "tau", tau, "split", split)
    got_t = lkv.decode_attn_multi([pair.gpu], [view], q.cuda(), sm_scale(D), tau, split)
    got = got_t.cpu().numpy()
    if tau > 0:
        # the skip decisions too: the oracle takes the GPU's near the bound
        dbg, mask = lkv.decode_attn_debug([pair.gpu], [view], q.cuda(), sm_scale(D), tau, split)
        torch.cuda.synchronize()
        assert torch.equal(dbg, got_t), "the debug entry point must give the production output bit for bit"
        ebts, elens = O.multi_entries([bt], [np.array(lens, np.int32)], T)
        sp = split or lkv.decode_plan_multi([pair.gpu], [view], len(lens), T, Hkv * G)
        want, stats = resolved_reference([pair.ref], ebts, elens, to_f32_host(q.reshape(-1, Hkv * G, D)),
                                         sm_scale(D), tau, sp, mask, [view.max_len])
        want = want.reshape(q.shape)
        say("  skip pairs live / flipped near the bound / largest flipped margin:", *stats)
    else:
        want = O.decode_multi([pair.ref], [bt], [np.array(lens, np.int32)],
                              to_f32_host(q.reshape(-1, Hkv * G, D)).reshape(q.shape), sm_scale(D), tau, split)
    return got, want, max_abs_vhat(pair.ref), (pair, view, q, bt)


CASES = [  # (format, G, q dtype): the matrix-core, fp16 and generic kernels
    ((128, 64, 6, 4), 4, "bf16"),
    ((128, 64, 6, 4), 8, "bf16"),
    ((128, 64, 6, 6), 4, "bf16"),
    ((128, 64, 6, 6), 8, "bf16"),
    ((128, 64, 16, 16), 8, "bf16"),
    ((64, 32, 6, 4), 2, "bf16"),
    ((128, 64, 6, 4), 4, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "D{}g{}k{}v{}".format(*c[0]) + f"G{c[1]}{c[2]}")
@pytest.mark.parametrize("T", [2, 7, 16])
@pytest.mark.parametrize("tau", [0.0, 1e-4])
def test_multi_parity(case, T, tau):
    fmt, G, qd = case
    lens = [T, 64 + T - 1, 300, 1100]
    got, want, vmax, _ = _multi_case(fmt, G, qd, lens, T, tau, 256)
    assert_attention_close(got.reshape(-1, *got.shape[2:]), want.reshape(-1, *want.shape[2:]), vmax,
                           f"multi {case} T {T} tau {tau}")


def test_single_query_is_decode_bit_for_bit():
    fmt, G = (128, 64, 6, 4), 4
    got, _, _, (pair, view, q, bt) = _multi_case(fmt, G, "bf16", [1, 65, 700], 1, 1e-4, 128)
    dec = lkv.decode_attn([pair.gpu], [view], q[:, 0].contiguous().cuda(), sm_scale(128), 1e-4, 128)
    assert np.array_equal(got[:, 0], dec.cpu().numpy())


def test_multi_causal_prefix_and_plan():
    """The library's own split plan; query i of a sequence equals a decode
    over the first L - T + i + 1 tokens (same split size)."""
    fmt, G, T = (128, 64, 6, 4), 8, 5
    lens = [40, 513, 2000]
    got, want, vmax, (pair, view, q, bt) = _multi_case(fmt, G, "bf16", lens, T, 0.0, 0)
    assert_attention_close(got.reshape(-1, *got.shape[2:]), want.reshape(-1, *want.shape[2:]), vmax, "planned")
    split = lkv.decode_plan_multi([pair.gpu], [view], len(lens), T, 2 * G)
    for i in (0, T - 1):
        pre = torch.tensor([n - T + i + 1 for n in lens], dtype=torch.int32).cuda()
        dec = lkv.decode_attn([pair.gpu], [lkv.View(view.block_table, pre, max(lens))], q[:, i].contiguous().cuda(),
                              sm_scale(128), 0.0, split)
        assert np.array_equal(got[:, i], dec.cpu().numpy())


@pytest.mark.parametrize("vb", [4, 6])
@pytest.mark.parametrize("T", [2, 3, 5, 8])
@pytest.mark.parametrize("split", [64, 128])
def test_query_pairs_at_block_edges(vb, T, split):
    """4 query heads per KV head: query tokens run in pairs through the
    8-head matrix-core layout.  Prefixes that end on a block edge give the
    earlier token of a pair no live token in the split's last block (or in a
    whole split); an odd T pairs its last token with itself."""
    fmt = (128, 64, 6, vb)
    lens = [T, 64 + T - 1, 64 + T, 128 + T - 1, 129 + T, 300, 1100]
    got, want, vmax, (pair, view, q, bt) = _multi_case(fmt, 4, "bf16", lens, T, 1e-4, split, seed=45)
    assert np.all(np.isfinite(got))
    assert_attention_close(got.reshape(-1, *got.shape[2:]), want.reshape(-1, *want.shape[2:]), vmax,
                           f"pairs v{vb} T {T} split {split}")


@pytest.mark.parametrize("G", [4, 8])
def test_multi_tiered_segments(G):
    """HIGH (K6V6, holding the new tokens) + MID (K6V4) in one launch."""
    D, g, Hkv, T = 128, 64, 2, 4
    rng = np.random.default_rng(50)
    lens_h, lens_m = [4, 130, 700], [900, 0, 65]
    pairs, views, ref = [], [], []
    for vb, lens, seed in ((6, lens_h, 51), (4, lens_m, 52)):
        bt, nblk = block_tables([max(n, 1) for n in lens], rng)
        pair = Pair(D, g, 6, vb, Hkv, nblk)
        _prefill(pair, lens, Hkv, D, "bf16", seed, bt)
        pairs.append(pair)
        views.append(lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens)))
        ref.append((bt, np.array(lens, np.int32)))
    q = _queries(53, 3, T, Hkv * G, D, "bf16")
    say("multi tiered G", G)
    got = lkv.decode_attn_multi([p.gpu for p in pairs], views, q.cuda(), sm_scale(D), 1e-5, 128).cpu().numpy()
    want = O.decode_multi([p.ref for p in pairs], [r[0] for r in ref], [r[1] for r in ref],
                          to_f32_host(q.reshape(-1, Hkv * G, D)).reshape(q.shape), sm_scale(D), 1e-5, 128)
    vmax = max(max_abs_vhat(p.ref) for p in pairs)
    assert_attention_close(got.reshape(-1, *got.shape[2:]), want.reshape(-1, *want.shape[2:]), vmax, f"tiered G{G}")


def test_multi_rejects_short_views():
    D, g, Hkv = 128, 64, 1
    bt, nblk = block_tables([3])
    pair = Pair(D, g, 6, 4, Hkv, nblk)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor([3], dtype=torch.int32).cuda(), 3)
    q = torch.zeros((1, 4, 4, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lkv.LkvError):
        lkv.decode_attn_multi([pair.gpu], [view], q, sm_scale(D), 0.0, 64)
