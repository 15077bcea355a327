"""The C ABI without a GPU: the library loads, exports every function
include/lkv.h declares, and rejects bad arguments on the host before any
launch.  No call here reaches a kernel."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import oracle as O
from quantized_kv_cache_token_amd import lkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "lkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = lkv.lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert sorted(lkv.EXPORTS) == names


def test_chunk_layout_matches_the_oracle():
    for fmt in [(128, 64, 6, 4), (64, 32, 6, 4), (128, 64, 6, 6), (128, 64, 4, 4), (128, 64, 16, 16),
                (64, 16, 6, 6), (128, 32, 4, 6)]:
        assert lkv.chunk_layout(*fmt) == O.chunk_layout(*fmt)
    for bad in [(96, 32, 6, 4), (128, 48, 6, 4), (128, 64, 5, 4), (128, 64, 16, 4), (128, 128, 6, 4)]:
        with pytest.raises(lkv.LkvError):
            lkv.chunk_layout(*bad)


def test_default_thresholds_bit_exact_with_the_oracle():
    for n in [1, 7, 256, 3277, 13107, 32768, 131072]:
        assert lkv.default_thresholds(n) == O.default_thresholds(n)


def _cache(pool=0x10000, **kw):
    d = dict(head_dim=128, group_size=64, k_bits=6, v_bits=4, num_kv_heads=8, block_tokens=64,
             num_blocks=16, pool=pool)
    d.update(kw)
    return lkv._Cache(**d)


def _view(max_len=1024, max_blocks=16, sum_len=0):
    return lkv._View(0x20000, 0x30000, max_blocks, max_len, sum_len)


def test_append_rejects_bad_arguments():
    L = lkv.lib()
    k = C.c_void_p(0x40000)
    args = lambda c, dt=1, bt=C.c_void_p(0x50000), mb=16, b=2, mn=4: L.lkv_quant_append(
        C.byref(c), k, k, dt, k, k, bt, mb, b, mn, None)
    assert args(_cache(head_dim=96)) == lkv.EUNSUPPORTED
    assert args(_cache(k_bits=5)) == lkv.EUNSUPPORTED
    assert args(_cache(block_tokens=32)) == lkv.EUNSUPPORTED
    assert args(_cache(pool=0)) == lkv.EINVAL
    assert args(_cache(pool=0x10010)) == lkv.EINVAL          # not 256-byte aligned
    assert args(_cache(num_kv_heads=0)) == lkv.EINVAL
    assert args(_cache(), dt=7) == lkv.EINVAL
    assert args(_cache(), bt=None) == lkv.EINVAL
    assert args(_cache(), mb=0) == lkv.EINVAL
    assert args(_cache(), b=-1) == lkv.EINVAL
    assert args(_cache(), b=0) == lkv.OK                      # nothing to do, nothing queued
    assert args(_cache(), mn=0) == lkv.OK


def test_decode_rejects_bad_arguments_and_plans_deterministically():
    L = lkv.lib()
    q = C.c_void_p(0x60000)

    def call(segs, views, n=1, Hq=32, dt=1, split=1024, ws=1 << 30, b=8, sm=0.088, tau=0.0):
        cs = (lkv._Cache * len(segs))(*segs)
        vs = (lkv._View * len(views))(*views)
        return L.lkv_decode_attn(cs, vs, n, q, dt, b, Hq, sm, tau, split, C.c_void_p(0x70000),
                                 C.c_void_p(0x80000), ws, None)

    assert call([_cache()], [_view()], n=0) == lkv.EINVAL
    assert call([_cache()] * 3, [_view()] * 3, n=3) == lkv.EINVAL
    assert call([_cache()], [_view()], Hq=12) == lkv.EINVAL            # not a multiple of Hkv
    assert call([_cache()], [_view()], Hq=8 * 3) == lkv.EUNSUPPORTED   # G = 3
    assert call([_cache()], [_view()], dt=2) == lkv.EINVAL             # fp16 queries
    assert call([_cache()], [_view()], split=100) == lkv.EINVAL
    assert call([_cache()], [_view(max_len=2000, max_blocks=16)]) == lkv.EINVAL
    assert call([_cache()], [_view()], ws=16) == lkv.EINVAL            # workspace too small
    assert call([_cache()], [_view()], sm=float("inf")) == lkv.EINVAL
    assert call([_cache(), _cache(head_dim=64, group_size=32)], [_view(), _view()], n=2) == lkv.EINVAL
    assert call([_cache()], [_view()], b=0) == lkv.OK

    cs = (lkv._Cache * 1)(_cache())
    vs = (lkv._View * 1)(_view(max_len=32768, max_blocks=512))
    out = C.c_int32()
    assert L.lkv_decode_plan(cs, vs, 1, 8, 32, C.byref(out)) == lkv.OK
    assert out.value == 1024               # 8 x 8 x 512 blocks / 2048 work items = 16 blocks
    ws = L.lkv_decode_workspace_bytes(cs, vs, 1, 8, 32, 1024)
    assert ws == 8 * 32 * 32 * 130 * 4
    vs1 = (lkv._View * 1)(_view(max_len=256, max_blocks=4))
    cs1 = (lkv._Cache * 1)(_cache(head_dim=64, group_size=32, num_kv_heads=1))
    assert L.lkv_decode_plan(cs1, vs1, 1, 1, 1, C.byref(out)) == lkv.OK and out.value == 64


def test_plan_uses_the_total_length_hint_of_a_ragged_batch():
    """64 ragged sequences, 2 KV heads, max_len 16512: counted at max_len
    they make 64 x 258 x 2 = 33024 blocks, 17 per work item.  With the
    batch's total length 557056 (8704 blocks), p blocks per split give at most
    2 x (ceil(8704 / p) + 64) splits with work; p = 10 is the smallest with at
    most 2048 (1870).  A hint above the dense count is capped by it: then
    2 x (ceil(16512 / p) + 64) <= 2048 needs p = 18."""
    L = lkv.lib()
    out = C.c_int32()
    cs = (lkv._Cache * 1)(_cache(num_kv_heads=2, num_blocks=10000))
    for hint, want in [(0, 17 * 64), (557056, 10 * 64), (10**9, 18 * 64)]:
        vs = (lkv._View * 1)(_view(max_len=16512, max_blocks=258, sum_len=hint))
        assert L.lkv_decode_plan(cs, vs, 1, 64, 16, C.byref(out)) == lkv.OK
        assert out.value == want, (hint, out.value)


def _items(lens, H, per, cap):
    """Splits with tokens of the decode step's compact order (an empty
    sequence counts one), written out."""
    return sum(H * max(1, -(-min(max(n, 0), cap) // (64 * per))) for n in lens)


def test_exact_length_plan_fits_the_compact_order_in_one_round():
    """lkv_decode_plan_lens: for a ragged batch of at most 64 sequences in a
    fused format, the smallest split (in 64-token blocks) whose splits with
    tokens over the KV heads number at most 2048, by brute force over the
    lengths; otherwise exactly lkv_decode_plan's choice."""
    L = lkv.lib()
    out, ref = C.c_int32(), C.c_int32()
    rng = np.random.default_rng(7)
    for trial in range(40):
        B = int(rng.integers(1, 65))
        H = int(rng.choice([1, 2, 4, 8]))
        cap = int(rng.integers(64, 40000))
        lens = rng.integers(0, cap + 1, B).astype(np.int32)
        lens[0] = cap
        total = int(lens.sum())
        cache = _cache(num_kv_heads=H, num_blocks=100000)
        view = _view(max_len=cap, max_blocks=-(-cap // 64), sum_len=total)
        st = L.lkv_decode_plan_lens(C.byref(cache), C.byref(view), lens.ctypes.data, B, 4 * H, C.byref(out))
        assert st == lkv.OK
        if total < B * cap:
            want = next((p for p in range(1, 64) if _items(lens, H, p, cap) <= 2048), 64)
        else:  # not ragged: the plan of lkv_decode_plan
            assert L.lkv_decode_plan(C.byref(cache), C.byref(view), 1, B, 4 * H, C.byref(ref)) == lkv.OK
            want = ref.value // 64
        assert out.value == 64 * want, (trial, B, H, cap, out.value, want)
    # the workload shape: 64 sequences of 1K to 16K (+128 steps), 2 KV heads
    lens = np.arange(64, dtype=np.int32) * 240 + 1152
    view = _view(max_len=int(lens.max()), max_blocks=-(-int(lens.max()) // 64), sum_len=int(lens.sum()))
    cache = _cache(num_kv_heads=2, num_blocks=100000)
    assert L.lkv_decode_plan_lens(C.byref(cache), C.byref(view), lens.ctypes.data, 64, 16, C.byref(out)) == lkv.OK
    assert _items(lens, 2, out.value // 64, int(lens.max())) <= 2048 < _items(lens, 2, out.value // 64 - 1,
                                                                              int(lens.max()))
    # no compact order: more than 64 sequences, the fp16 format, direction-preserving K, 2 query heads per KV head
    lens = np.full(65, 100, np.int32)
    lens[0] = 5000
    for cache, B, Hq in [(_cache(num_kv_heads=2, num_blocks=100000), 65, 8),
                         (_cache(num_kv_heads=2, num_blocks=100000, k_bits=16, v_bits=16), 64, 8),
                         (_cache(num_kv_heads=2, num_blocks=100000, k_norm=1), 64, 8),
                         (_cache(num_kv_heads=2, num_blocks=100000), 64, 4)]:
        view = _view(max_len=5000, max_blocks=79, sum_len=int(lens[:B].sum()))
        assert L.lkv_decode_plan_lens(C.byref(cache), C.byref(view), lens.ctypes.data, B, Hq, C.byref(out)) == lkv.OK
        assert L.lkv_decode_plan(C.byref(cache), C.byref(view), 1, B, Hq, C.byref(ref)) == lkv.OK
        assert out.value == ref.value
    assert L.lkv_decode_plan_lens(C.byref(cache), C.byref(view), None, 4, 8, C.byref(out)) == lkv.EINVAL


def test_tier_update_rejects_bad_formats():
    L = lkv.lib()
    p = C.c_void_p(0x90000)
    src, h, m = _cache(v_bits=6), _cache(v_bits=6), _cache(v_bits=4)
    v = _view(max_len=1024)

    def call(src=src, h=h, m=m, stride=1024, ws=1 << 20):
        return L.lkv_tier_update(C.byref(src), C.byref(v), p, stride, 1e-6, 1e-4, C.byref(h), p, 16,
                                 C.byref(m), p, 16, p, p, p, 8, p, ws, None)

    assert call(src=_cache(v_bits=4)) == lkv.EUNSUPPORTED     # the source must hold V6
    assert call(h=_cache(v_bits=4)) == lkv.EINVAL
    assert call(m=_cache(v_bits=6)) == lkv.EINVAL
    assert call(m=_cache(v_bits=4, group_size=32)) == lkv.EINVAL
    assert call(stride=512) == lkv.EINVAL                      # scores shorter than max_len
    assert call(ws=100) == lkv.EINVAL
    # (HIGH, MID) int32 counts per 2048-token scan chunk, then (HIGH, MID)
    # destination positions per 64-token block, then a ticket (8 bytes) and a
    # uint32 read count per 64-token block for in-place compaction
    assert L.lkv_tier_workspace_bytes(8, 32768) == 8 * (16 + 512) * 8 + 8 + 8 * 512 * 4
    assert L.lkv_tier_workspace_bytes(2, 300) == 2 * (1 + 5) * 8 + 8 + 2 * 5 * 4
    assert L.lkv_tier_workspace_bytes(1, 0) == 1 * (1 + 1) * 8 + 8 + 1 * 1 * 4


def test_in_place_tiering_needs_its_own_segment_and_row_width():
    """A destination with a source's pool and block table compacts that
    source in place: only its own segment, read with the source's row
    width; anything else is rejected before a launch."""
    L = lkv.lib()
    p = C.c_void_p(0x90000)
    h, m = _cache(v_bits=6, pool=0x11000), _cache(v_bits=4, pool=0x12000)
    hv = lkv._View(0x20000, 0x30000, 16, 1024, 0)
    mv = lkv._View(0x21000, 0x31000, 16, 1024, 0)

    def retier(dh=h, dh_bt=0x90000, dh_w=16, dm=m, dm_bt=0x91000, dm_w=16):
        return L.lkv_retier(C.byref(h), C.byref(hv), p, 1024, C.byref(m), C.byref(mv), p, 1024, 1e-6, 1e-4,
                            C.byref(dh), C.c_void_p(dh_bt), dh_w, C.byref(dm), C.c_void_p(dm_bt), dm_w, p, p, p, p,
                            8, p, 1 << 22, None)

    assert retier(dh_bt=0x20000, dh_w=8) == lkv.EINVAL                         # HIGH in place, narrower rows
    assert retier(dm_bt=0x21000, dm_w=32) == lkv.EINVAL                        # MID in place, wider rows
    assert retier(dh=_cache(v_bits=6, pool=0x12000), dh_bt=0x21000) == lkv.EINVAL  # HIGH onto MID's blocks
    assert retier(dm=_cache(v_bits=4, pool=0x11000), dm_bt=0x20000) == lkv.EINVAL  # MID onto HIGH's blocks

    def tier(dh=h, dh_bt=0x90000, dh_w=16, dm=m, dm_bt=0x91000):
        return L.lkv_tier_update(C.byref(h), C.byref(hv), p, 1024, 1e-6, 1e-4, C.byref(dh), C.c_void_p(dh_bt),
                                 dh_w, C.byref(dm), C.c_void_p(dm_bt), 16, p, p, p, 8, p, 1 << 20, None)

    assert tier(dh_bt=0x20000, dh_w=4) == lkv.EINVAL
    assert tier(dm=_cache(v_bits=4, pool=0x11000), dm_bt=0x20000) == lkv.EINVAL  # MID onto the source's blocks


def test_hbm_read_probe_rejects_bad_buffers():
    L = lkv.lib()
    p = C.c_void_p(0x90000)
    assert L.lkv_hbm_read_probe(None, 1 << 20, 0, p, None) == lkv.EINVAL
    assert L.lkv_hbm_read_probe(p, 0, 0, p, None) == lkv.EINVAL
    assert L.lkv_hbm_read_probe(p, 1000, 0, p, None) == lkv.EINVAL          # not a multiple of 16
    assert L.lkv_hbm_read_probe(C.c_void_p(0x90004), 1 << 20, 1, p, None) == lkv.EINVAL  # misaligned
    assert L.lkv_hbm_read_probe(p, 1 << 20, 0, None, None) == lkv.EINVAL


def test_retier_rejects_bad_formats():
    L = lkv.lib()
    p = C.c_void_p(0x90000)
    h, m = _cache(v_bits=6), _cache(v_bits=4)
    v = _view(max_len=1024)

    def call(h=h, m=m, dh=h, dm=m, hs=1024, ms=1024, ws=1 << 22):
        return L.lkv_retier(C.byref(h), C.byref(v), p, hs, C.byref(m), C.byref(v), p, ms, 1e-6, 1e-4,
                            C.byref(dh), p, 16, C.byref(dm), p, 16, p, p, p, p, 8, p, ws, None)

    assert call(h=_cache(v_bits=4)) == lkv.EUNSUPPORTED        # HIGH holds V6
    assert call(m=_cache(v_bits=6)) == lkv.EINVAL               # MID holds V4
    assert call(m=_cache(v_bits=4, k_bits=4)) == lkv.EINVAL     # the same K in every segment
    assert call(dh=_cache(v_bits=4)) == lkv.EINVAL
    assert call(dm=_cache(v_bits=4, num_kv_heads=2)) == lkv.EINVAL
    assert call(ms=512) == lkv.EINVAL                           # MID scores shorter than max_len
    assert call(ws=100) == lkv.EINVAL
    # (HIGH, MID) counts per 2048-token chunk and destination positions per
    # 64-token block, of each segment
    assert L.lkv_retier_workspace_bytes(8, 32768, 4096) == 8 * (16 + 2 + 512 + 64) * 8 + 8 + 8 * 512 * 4
    assert L.lkv_retier_workspace_bytes(2, 300, 0) == 2 * (1 + 1 + 5 + 1) * 8 + 8 + 2 * 5 * 4
    assert L.lkv_retier_workspace_bytes(-1, 1, 1) == lkv.EINVAL


def test_decode_multi_rejects_bad_arguments():
    L = lkv.lib()
    p = C.c_void_p(0x90000)
    cs = (lkv._Cache * 1)(_cache())
    vs = (lkv._View * 1)(_view(max_len=1024))

    def call(T=4, max_len=1024, q_dtype=lkv.BF16, ws=1 << 30):
        v = (lkv._View * 1)(_view(max_len=max_len))
        return L.lkv_decode_attn_multi(cs, v, 1, p, q_dtype, 8, T, 32, 0.088, 0.0, 256, p, p, ws, None)

    assert call(T=0) == lkv.EINVAL
    assert call(max_len=3) == lkv.EINVAL       # every sequence holds its T query tokens
    assert call(q_dtype=7) == lkv.EINVAL
    assert call(ws=100) == lkv.EINVAL          # partials for batch * T entries
    # the workspace is lkv_decode_workspace_bytes for batch * T entries
    assert L.lkv_decode_workspace_bytes(cs, vs, 1, 8 * 4, 32, 256) == 8 * 4 * 32 * 4 * 130 * 4


def test_decode_debug_rejects_bad_arguments_before_any_launch():
    """Every check of the skip-mask entry point runs before it clears the
    mask: a rejected call queues nothing (without a GPU, a queued kernel
    would report LKV_EHIP instead)."""
    L = lkv.lib()
    p = C.c_void_p(0x90000)
    cs = (lkv._Cache * 2)(_cache(v_bits=6), _cache())

    def call(T=1, nseg=1, words=None, q_dtype=lkv.BF16, ws=1 << 30, sm=0.088, tau=1e-3, mask=p, out=p):
        v = (lkv._View * 2)(_view(max_len=1000), _view(max_len=300))
        if words is None:
            words = (1024 + (320 if nseg == 2 else 0)) // 32
        return L.lkv_decode_attn_debug(cs, v, nseg, p, q_dtype, 8, T, 32, sm, tau, 256, out, mask, words, p, ws,
                                       None)

    assert call(words=31) == lkv.EINVAL              # 1000 tokens round up to 1024 columns: 32 words
    assert call(nseg=2, words=32) == lkv.EINVAL      # + 300 rounded up to 320: 42 words
    assert call(q_dtype=7) == lkv.EINVAL
    assert call(ws=100) == lkv.EINVAL
    assert call(sm=float("inf")) == lkv.EINVAL
    assert call(tau=float("nan")) == lkv.EINVAL
    assert call(T=0) == lkv.EINVAL
    assert call(mask=None) == lkv.EINVAL
    assert call(out=None) == lkv.EINVAL


def test_append_decode_rejects_bad_arguments_before_any_launch():
    L = lkv.lib()
    p = C.c_void_p(0x90000)
    vs = (lkv._View * 1)(_view(max_len=1000))

    def call(fn="lkv_append_decode", kvd=lkv.BF16, k=p, v=p, split=256, ws=1 << 30, q_dtype=lkv.BF16, knorm=0,
             out=p):
        cs = (lkv._Cache * 1)(_cache(k_norm=knorm))
        if fn == "lkv_append_decode":
            return L.lkv_append_decode(cs, vs, k, v, kvd, p, q_dtype, 8, 32, 0.088, 0.0, split, out, p, ws, None)
        return L.lkv_append_split(cs, vs, k, v, kvd, p, q_dtype, 8, 32, 0.088, 0.0, split, p, ws, None)

    for fn in ("lkv_append_decode", "lkv_append_split"):
        assert call(fn, kvd=7) == lkv.EINVAL
        assert call(fn, k=None) == lkv.EINVAL
        assert call(fn, v=None) == lkv.EINVAL
        assert call(fn, ws=100) == lkv.EINVAL
        assert call(fn, q_dtype=lkv.F16) == lkv.EINVAL
        assert call(fn, knorm=1, k=C.c_void_p(0x90002)) == lkv.EUNSUPPORTED  # k_norm: two-element alignment
    assert call("lkv_append_split", split=0) == lkv.EINVAL       # the split stage takes a resolved size
    assert call("lkv_append_decode", out=None) == lkv.EINVAL


def test_noalloc_rejects_partials_beyond_its_scratch_before_any_launch():
    L = lkv.lib()
    p = C.c_void_p(0x90000)
    cs = (lkv._Cache * 1)(_cache(num_blocks=1 << 20))
    vs = (lkv._View * 1)(_view(max_len=64, max_blocks=1))
    # 65536 sequences x 32 heads x 1 split x 130 floats = 1.09 GB of partials
    assert L.lkv_decode_attn_noalloc(cs, vs, 1, p, lkv.BF16, 65536, 32, 0.088, 0.0, 64, p, None) == lkv.ESCRATCH
    assert "scratch" in lkv.status_string(lkv.ESCRATCH)
    assert L.lkv_decode_attn_noalloc(cs, vs, 1, p, lkv.BF16, 8, 32, 0.088, 0.0, 48, p, None) == lkv.EINVAL


def test_multi_token_plan_counts_query_pairs_at_four_heads_per_kv_head():
    L = lkv.lib()
    out = C.c_int32()
    vs = (lkv._View * 1)(_view(max_len=32768, max_blocks=512))

    def plan(B, T, Hq, Hkv=8):
        cs = (lkv._Cache * 1)(_cache(num_kv_heads=Hkv))
        st = L.lkv_decode_plan_multi(cs, vs, 1, B, T, Hq, C.byref(out))
        return out.value if st == lkv.OK else st

    # G = 4: B * ceil(T / 2) pairs; G = 8: B * T query tokens (2048 work items)
    assert plan(8, 4, 32) == 2048      # 8 x 2 pairs x 8 heads x 512 blocks / 2048 = 32 blocks
    assert plan(8, 3, 32) == 2048      # ceil(3 / 2) = 2 pairs
    assert plan(8, 4, 64) == 4096      # 8 x 4 tokens x 8 heads x 512 / 2048 = 64 blocks
    assert plan(8, 1, 32) == 1024      # one token: the plain decode plan
    assert plan(8, 0, 32) == lkv.EINVAL
    assert plan(1 << 20, 1 << 12, 32) == lkv.EINVAL


def test_status_strings():
    assert lkv.status_string(lkv.OK) == "ok"
    assert "invalid" in lkv.status_string(lkv.EINVAL)


def test_binding_checks_raise_value_errors_before_any_call():
    """The binding's own argument checks are errors, not asserts, so they
    hold under python -O; none of these reaches the library's compute."""
    import torch

    with pytest.raises(ValueError):
        lkv.Cache(128, 64, 6, 4, 2, 1, pool=torch.zeros(3, dtype=torch.uint8), device="cpu")
    cache = lkv.Cache(128, 64, 6, 4, 2, 1, device="cpu")
    with pytest.raises(ValueError):
        lkv.View(torch.zeros(1, 1, dtype=torch.int64), torch.zeros(1, dtype=torch.int32), 0).c()
    k = torch.zeros(4, 2, 128)
    with pytest.raises(ValueError):
        lkv.quant_append(cache, k, torch.zeros(4, 2, 64), None, None, None, 4)
    view = lkv.View(torch.zeros(1, 1, dtype=torch.int32), torch.zeros(1, dtype=torch.int32), 0)
    with pytest.raises(ValueError):
        lkv._segs([cache], [view, view])
    with pytest.raises(ValueError):
        lkv.decode_attn([cache], [view], torch.zeros(1, 128, 8).transpose(1, 2), 1.0, split_tokens=64)
    scores = torch.zeros(1, 64)
    with pytest.raises(ValueError):
        lkv.tier_update(cache, view, scores, 0.0, 1.0, cache, None, cache, None, None, None,
                        torch.zeros(1, 64, dtype=torch.int32))
    from quantized_kv_cache_token_amd import inputs
    with pytest.raises(ValueError):
        inputs.tier_scores(1, 0, 10, 1e-4, 1e-3, frac_high=0.8, frac_mid=0.5)


def test_append_decode_merged_rejects_bad_arguments_before_any_launch():
    """lkv_append_decode_merged: one or two segments, counters, out and the
    new rows are checked on the host; nothing is launched when they fail."""
    L = lkv.lib()
    p = C.c_void_p(0x90000)

    def call(nseg=1, counters=p, out=p, k=p, kvd=lkv.BF16, ws=1 << 30):
        cs = (lkv._Cache * 3)(_cache(), _cache(), _cache())
        vs = (lkv._View * 3)(_view(max_len=1000), _view(max_len=1000), _view(max_len=1000))
        return L.lkv_append_decode_merged(cs, vs, nseg, k, p, kvd, p, lkv.BF16, 8, 32, 0.088, 0.0, 256, out,
                                          counters, p, ws, None)

    assert call(nseg=0) == lkv.EINVAL
    assert call(nseg=3) == lkv.EINVAL
    assert call(counters=None) == lkv.EINVAL
    assert call(counters=C.c_void_p(0x90002)) == lkv.EINVAL  # counters are 4-byte aligned
    assert call(out=None) == lkv.EINVAL
    assert call(k=None) == lkv.EINVAL
    assert call(kvd=7) == lkv.EINVAL
    assert call(ws=100) == lkv.EINVAL
