"""The decode step captured in a HIP graph and replayed: every replay, with
the program's own eager work and synchronisations in between, must give
the eager result bit for bit (pool and output).  The calls launch kernels
only (no allocation, no memset node, no synchronisation), so a serving loop
can replay them."""
import numpy as np
import pytest
import torch

from quantized_kv_cache_token_amd import inputs, lkv
from tests.gpu_common import Pair, say, sm_scale
from tests.oracle_cases import block_tables
from tests.test_gpu_parity import _prefill

pytestmark = pytest.mark.gpu


def _setup(fmt, G, lens, seed):
    D, g, kb, vb = fmt
    Hkv = 2
    rng = np.random.default_rng(seed)
    bt, nblk = block_tables(lens, rng)
    pair = Pair(D, g, kb, vb, Hkv, nblk)
    _prefill(pair, [n - 1 for n in lens], Hkv, D, "bf16", seed, bt, outliers=True)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens), sum(lens))
    k_new, v_new = inputs.kv_rows(seed + 1, 0, len(lens), Hkv, D)
    q = inputs.queries(seed + 2, len(lens), Hkv * G, D).cuda()
    return pair.gpu, view, k_new.cuda(), v_new.cuda(), q


@pytest.mark.parametrize("fmt,G", [((128, 64, 6, 4), 4), ((128, 64, 6, 4), 8), ((128, 64, 16, 16), 8),
                                   ((64, 32, 6, 4), 2)])
def test_append_decode_graph_replays_match_eager(fmt, G):
    D = fmt[0]
    cache, view, k_new, v_new, q = _setup(fmt, G, [70, 1000, 2049, 64], 70)
    B, Hq = q.shape[0], q.shape[1]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        split = lkv.decode_plan([cache], [view], B, Hq)
        ws = lkv.decode_workspace([cache], [view], B, Hq, split, q.device)
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
        say("graph: eager append_decode", fmt, G)
        lkv.append_decode(cache, view, k_new, v_new, q, sm_scale(D), 1e-4, split, out, ws, stream)
    torch.cuda.synchronize()
    want_out, want_pool = out.clone(), cache.pool.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        lkv.append_decode(cache, view, k_new, v_new, q, sm_scale(D), 1e-4, split, out, ws, stream)
    for r in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()  # the program's own eager work between replays
        torch.cuda.synchronize()
        say("graph replay", r)
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out, want_out), f"replay {r}: output differs from the eager call"
        assert torch.equal(cache.pool, want_pool), f"replay {r}: pool differs from the eager call"


def test_noalloc_decode_graph_replays_match_eager():
    """lkv_decode_attn_noalloc under capture: its partials live in the
    library's static scratch, so the graph holds no allocation at all."""
    fmt, G, D = (128, 64, 6, 4), 4, 128
    cache, view, _, _, q = _setup(fmt, G, [300, 4000, 65], 71)
    B, Hq = q.shape[0], q.shape[1]
    stream = torch.cuda.Stream()
    split = lkv.decode_plan([cache], [view], B, Hq)
    with torch.cuda.stream(stream):
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
        want = lkv.decode_attn([cache], [view], q, sm_scale(D), 0.0, split, stream=stream)
        lkv.decode_attn_noalloc([cache], [view], q, sm_scale(D), 0.0, out=out, stream=stream)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        lkv.decode_attn_noalloc([cache], [view], q, sm_scale(D), 0.0, out=out, stream=stream)
    for r in range(4):
        out.zero_()
        other = lkv.decode_attn([cache], [view], q[:1].contiguous(), sm_scale(D), 0.0, split)  # eager work between
        torch.cuda.synchronize()
        say("noalloc graph replay", r)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(other, want[:1])
        assert torch.equal(out, want), f"replay {r}"


@pytest.mark.parametrize("G", [4, 8])
def test_append_decode_merged_graph_replays_match_eager(G):
    """The one-launch step (lkv_append_decode_merged) under capture: its
    counters come back to zero at the end of every launch, so the graph needs
    no clearing node; every replay equals the eager call bit for bit."""
    fmt, D = (128, 64, 6, 4), 128
    cache, view, k_new, v_new, q = _setup(fmt, G, [70, 1000, 2049, 64], 72)
    B, Hq = q.shape[0], q.shape[1]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        split = lkv.decode_plan([cache], [view], B, Hq)
        ws = lkv.decode_workspace([cache], [view], B, Hq, split, q.device)
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
        counters = lkv.merge_counters(cache, B)
        say("graph: eager append_decode_merged", G)
        lkv.append_decode_merged(cache, view, k_new, v_new, q, sm_scale(D), 1e-4, split, counters, out, ws, stream)
    torch.cuda.synchronize()
    want_out, want_pool = out.clone(), cache.pool.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        lkv.append_decode_merged(cache, view, k_new, v_new, q, sm_scale(D), 1e-4, split, counters, out, ws, stream)
    for r in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()  # the program's own eager work between replays
        torch.cuda.synchronize()
        say("graph replay", r)
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out, want_out), f"replay {r}: output differs from the eager call"
        assert torch.equal(cache.pool, want_pool), f"replay {r}: pool differs from the eager call"
        assert int(counters.abs().sum()) == 0, f"replay {r}: counters not back at zero"
