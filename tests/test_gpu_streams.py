"""Calls issued on a side stream that is not torch's current stream.

The binding allocates workspaces and outputs for the caller when it passes
none; they must belong to the stream the kernels run on, or torch's caching
allocator could hand that memory to other work while the kernels are still
queued.  Each call here is queued behind a long-running kernel on the side
stream while the current stream allocates and fills memory; the results
must equal those of the same calls on the current stream."""
import numpy as np
import pytest
import torch

from quantized_kv_cache_token_amd import inputs, lkv
from tests.gpu_common import Pair, say, sm_scale
from tests.oracle_cases import block_tables
from tests.test_gpu_parity import _prefill

pytestmark = pytest.mark.gpu

D, G, HKV = 128, 4, 2


def _delay(stream):
    """Keep the side stream busy for a while (a few ms of elementwise work)."""
    x = torch.ones(1 << 24, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(40):
            x.mul_(1.0000001)
    return x


def _churn():
    """Allocate, fill and free memory on the current stream."""
    for i in range(64):
        t = torch.full((1 << 18,), float(i + 1), device="cuda")
        del t


def _case(seed, lens, vb=4):
    rng = np.random.default_rng(seed)
    bt, nblk = block_tables(lens, rng)
    pair = Pair(D, 64, 6, vb, HKV, nblk)
    _prefill(pair, lens, HKV, D, "bf16", seed, bt, outliers=True)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    return pair.gpu, view


def test_decode_calls_on_a_side_stream():
    cache, view = _case(170, [700, 3000, 65])
    q = inputs.queries(171, 3, HKV * G, D).cuda()
    qm = inputs.queries(172, 3 * 2, HKV * G, D).view(3, 2, HKV * G, D).cuda()
    sm = sm_scale(D)
    say("side stream: reference calls on the current stream")
    want = lkv.decode_attn([cache], [view], q, sm, 1e-4)
    want_m = lkv.decode_attn_multi([cache], [view], qm, sm, 1e-4)
    acc_want = torch.zeros((1, 3, 3008), device="cuda")
    want_s = lkv.decode_attn_scores([cache], [view], q, acc_want, sm, 1e-4)
    want_d, want_mask = lkv.decode_attn_debug([cache], [view], q, sm, 1e-4)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    say("side stream: the same calls queued behind a delay")
    acc = torch.zeros((1, 3, 3008), device="cuda")
    torch.cuda.synchronize()
    keep = _delay(s)
    got = lkv.decode_attn([cache], [view], q, sm, 1e-4, stream=s)
    got_m = lkv.decode_attn_multi([cache], [view], qm, sm, 1e-4, stream=s)
    got_s = lkv.decode_attn_scores([cache], [view], q, acc, sm, 1e-4, stream=s)
    got_d, got_mask = lkv.decode_attn_debug([cache], [view], q, sm, 1e-4, stream=s)
    _churn()
    torch.cuda.synchronize()
    del keep
    assert torch.equal(got, want)
    assert torch.equal(got_m, want_m)
    assert torch.equal(got_s, want_s) and torch.equal(acc, acc_want)
    assert torch.equal(got_d, want_d) and torch.equal(got_mask, want_mask)


def test_tier_calls_on_a_side_stream():
    lens = [900, 2100]
    src, view = _case(173, lens, vb=6)
    tl, th = lkv.default_thresholds(max(lens))
    scores = torch.stack([inputs.tier_scores(174, b, max(lens), tl, th) for b in range(2)]).cuda()
    nb = -(-max(lens) // 64)
    hbt = torch.arange(2 * nb, dtype=torch.int32).view(2, nb).cuda()

    def run(stream):
        h = lkv.Cache(D, 64, 6, 6, HKV, 2 * nb)
        m = lkv.Cache(D, 64, 6, 4, HKV, 2 * nb)
        nh = torch.zeros(2, dtype=torch.int32, device="cuda")
        nm = torch.zeros_like(nh)
        tiers = torch.zeros((2, max(lens)), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        keep = _delay(stream) if stream is not None else None
        lkv.tier_update(src, view, scores, tl, th, h, hbt, m, hbt, nh, nm, tiers, stream=stream)
        if stream is not None:
            _churn()
            stream.synchronize()
        torch.cuda.synchronize()
        del keep
        nh_h, nm_h = nh.cpu().numpy(), nm.cpu().numpy()
        hs = torch.stack([inputs.tier_scores(175, b, max(lens), tl, th) for b in range(2)]).cuda()
        ms = torch.stack([inputs.tier_scores(176, b, max(lens), tl, th) for b in range(2)]).cuda()
        h2 = lkv.Cache(D, 64, 6, 6, HKV, 2 * nb)
        m2 = lkv.Cache(D, 64, 6, 4, HKV, 2 * nb)
        nh2, nm2 = torch.zeros_like(nh), torch.zeros_like(nh)
        ht = torch.zeros((2, max(lens)), dtype=torch.uint8, device="cuda")
        mt = torch.zeros_like(ht)
        hv = lkv.View(hbt, nh, int(max(nh_h.max(), 1)))
        mv = lkv.View(hbt, nm, int(max(nm_h.max(), 1)))
        keep = _delay(stream) if stream is not None else None
        lkv.retier(h, hv, hs, m, mv, ms, tl, th, h2, hbt, m2, hbt, nh2, nm2, ht, mt, stream=stream)
        if stream is not None:
            _churn()
            stream.synchronize()
        torch.cuda.synchronize()
        del keep
        return [t.clone() for t in (h.pool, m.pool, nh, nm, tiers, h2.pool, m2.pool, nh2, nm2, ht, mt)]

    say("side stream: tier update and re-tier on the current stream")
    want = run(None)
    say("side stream: tier update and re-tier behind a delay")
    got = run(torch.cuda.Stream())
    for i, (g, w) in enumerate(zip(got, want)):
        assert torch.equal(g, w), f"result {i} differs on the side stream"


def test_hbm_read_probe_reads_the_whole_buffer():
    """The probe's fold is stored only for the magic value: a zero buffer
    leaves the sink alone; one word set at the very end (the grid-stride
    tail) reaches it, with plain and non-temporal loads."""
    buf = torch.zeros((1 << 22) + 4, dtype=torch.int32, device="cuda")  # 16 MiB + one 16-byte piece
    for nt in (False, True):
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        say("probe over zeros, nt", nt)
        lkv.hbm_read_probe(buf, sink, nt)
        torch.cuda.synchronize()
        assert int(sink.item()) == 0
        buf[-1] = np.int32(np.uint32(0x9E3779B9).view(np.int32))
        say("probe with the magic word at the end, nt", nt)
        lkv.hbm_read_probe(buf, sink, nt)
        torch.cuda.synchronize()
        assert int(sink.item()) == int(np.uint32(0x9E3779B9).view(np.int32))
        buf[-1] = 0
