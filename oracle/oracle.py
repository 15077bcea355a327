"""ctypes view of the plain C oracle (oracle/lkv_oracle.c).

TEST INFRASTRUCTURE ONLY.  Imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg; the product package never imports it.

Every function takes and returns numpy arrays on the host.  Inputs of
narrower float types (bf16, fp16) are widened exactly to fp32 by the caller
before they get here.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblkv_oracle.so")
BLOCK_TOKENS = 64


class _Cache(C.Structure):
    _fields_ = [("head_dim", C.c_int32), ("group_size", C.c_int32),
                ("k_bits", C.c_int32), ("v_bits", C.c_int32),
                ("num_kv_heads", C.c_int32), ("num_blocks", C.c_int64),
                ("pool", C.c_void_p), ("k_norm", C.c_int32)]


class _View(C.Structure):
    _fields_ = [("block_table", C.c_void_p), ("seq_lens", C.c_void_p),
                ("max_blocks", C.c_int32)]


def build() -> None:
    """Compile the oracle with its Makefile (plain gcc)."""
    subprocess.run(["make", "-s", "-C", _HERE, "liblkv_oracle.so"], check=True)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        L.orc_chunk_layout.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_int64)]
        L.orc_chunk_layout.restype = C.c_int
        L.orc_quantize_group.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
        L.orc_quantize_group.restype = None
        L.orc_get_field.argtypes = [C.c_void_p, C.c_int64, C.c_int]
        L.orc_get_field.restype = C.c_uint32
        L.orc_put_field.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_uint32]
        L.orc_put_field.restype = None
        L.orc_f32_to_f16.argtypes = [C.c_float]
        L.orc_f32_to_f16.restype = C.c_uint16
        L.orc_f16_to_f64.argtypes = [C.c_uint16]
        L.orc_f16_to_f64.restype = C.c_double
        L.orc_append.argtypes = [C.POINTER(_Cache), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_int32, C.c_int32]
        L.orc_append.restype = C.c_int
        L.orc_decode.argtypes = [C.POINTER(_Cache), C.POINTER(_View), C.c_int32, C.c_void_p,
                                 C.c_int32, C.c_int32, C.c_float, C.c_float, C.c_int32,
                                 C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32]
        L.orc_decode.restype = C.c_int
        L.orc_decode_resolved.argtypes = [C.POINTER(_Cache), C.POINTER(_View), C.c_int32, C.c_void_p,
                                          C.c_int32, C.c_int32, C.c_float, C.c_float, C.c_int32,
                                          C.c_void_p, C.c_void_p, C.c_void_p, C.c_double, C.c_void_p, C.c_void_p,
                                          C.c_void_p, C.c_int32]
        L.orc_decode_resolved.restype = C.c_int
        L.orc_tier_update.argtypes = [C.POINTER(_Cache), C.POINTER(_View), C.c_void_p, C.c_int32,
                                      C.c_float, C.c_float,
                                      C.POINTER(_Cache), C.c_void_p, C.c_int32,
                                      C.POINTER(_Cache), C.c_void_p, C.c_int32,
                                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32]
        L.orc_tier_update.restype = C.c_int
        L.orc_retier.argtypes = [C.POINTER(_Cache), C.POINTER(_View), C.c_void_p, C.c_int32,
                                 C.POINTER(_Cache), C.POINTER(_View), C.c_void_p, C.c_int32, C.c_float, C.c_float,
                                 C.POINTER(_Cache), C.c_void_p, C.c_int32, C.POINTER(_Cache), C.c_void_p, C.c_int32,
                                 C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32]
        L.orc_retier.restype = C.c_int
        L.orc_default_thresholds.argtypes = [C.c_int32, C.POINTER(C.c_float), C.POINTER(C.c_float)]
        L.orc_default_thresholds.restype = None
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


# ------------------------------------------------------------------ format

def chunk_layout(D: int, g: int, kb: int, vb: int) -> list[int]:
    off = (C.c_int64 * 7)()
    if lib().orc_chunk_layout(D, g, kb, vb, off) != 0:
        raise ValueError(f"format D={D} g={g} kb={kb} vb={vb} is not defined")
    return list(off)


def quantize_group(x: np.ndarray, bits: int):
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.size, np.uint8)
    s = np.zeros(1, np.float32)
    z = np.zeros(1, np.uint8)
    lib().orc_quantize_group(_p(x), x.size, bits, _p(s), _p(z), _p(codes))
    return float(s[0]), int(z[0]), codes


def f32_to_f16_bits(x: float) -> int:
    return int(lib().orc_f32_to_f16(C.c_float(x)))


def f16_bits_to_f64(h: int) -> float:
    return float(lib().orc_f16_to_f64(h))


def put_fields(values, bits: int, nbytes: int) -> np.ndarray:
    buf = np.zeros(nbytes, np.uint8)
    for i, v in enumerate(values):
        lib().orc_put_field(_p(buf), i, bits, int(v))
    return buf


def get_fields(buf: np.ndarray, n: int, bits: int) -> np.ndarray:
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    return np.array([lib().orc_get_field(_p(buf), i, bits) for i in range(n)], np.uint32)


def default_thresholds(n_tokens: int) -> tuple[float, float]:
    lo, hi = C.c_float(), C.c_float()
    lib().orc_default_thresholds(n_tokens, C.byref(lo), C.byref(hi))
    return float(lo.value), float(hi.value)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_num_threads())


# ------------------------------------------------------------------ caches

@dataclass
class Cache:
    """A host cache: format and pool [num_blocks][Hkv][chunk] bytes."""
    head_dim: int
    group_size: int
    k_bits: int
    v_bits: int
    num_kv_heads: int
    num_blocks: int
    pool: np.ndarray = None
    k_norm: int = 0  # 1: direction-preserving K, one fp32 norm factor per slot after the six sections

    def __post_init__(self):
        self.layout = chunk_layout(self.head_dim, self.group_size, self.k_bits, self.v_bits)
        self.knorm_offset = self.layout[6]
        self.chunk_bytes = self.layout[6] + (BLOCK_TOKENS * 4 if self.k_norm else 0)
        if self.pool is None:
            self.pool = np.zeros(self.num_blocks * self.num_kv_heads * self.chunk_bytes, np.uint8)

    def c(self) -> _Cache:
        return _Cache(self.head_dim, self.group_size, self.k_bits, self.v_bits,
                      self.num_kv_heads, self.num_blocks, self.pool.ctypes.data, self.k_norm)

    def chunk(self, blk: int, kvh: int) -> np.ndarray:
        o = (blk * self.num_kv_heads + kvh) * self.chunk_bytes
        return self.pool[o:o + self.chunk_bytes]


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def append(cache: Cache, k: np.ndarray, v: np.ndarray, cu_new, start_pos, block_table) -> None:
    """Quantise rows k, v (fp32 [total_new][Hkv][D]) into the cache."""
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    cu = _i32(cu_new)
    sp = _i32(start_pos)
    bt = _i32(block_table)
    batch = len(sp)
    assert bt.ndim == 2 and bt.shape[0] == batch and len(cu) == batch + 1
    assert k.shape == (int(cu[-1]), cache.num_kv_heads, cache.head_dim) == v.shape
    cc = cache.c()
    rc = lib().orc_append(C.byref(cc), _p(k), _p(v), _p(cu), _p(sp), _p(bt), bt.shape[1], batch)
    if rc != 0:
        raise ValueError("oracle append rejected its arguments")


def decode(caches, block_tables, seq_lens, q: np.ndarray, sm_scale: float,
           tau_low: float = 0.0, split_tokens: int = 0, want_skip: bool = False,
           score_acc: np.ndarray | None = None):
    """fp64 attention of q (fp32 [B][Hq][D]) over one or more segments.

    Returns out (fp64 [B][Hq][D]) and, if want_skip, the skip flags
    (uint8 [B][Hq][nseg][max_tok]).  score_acc (fp64 [nseg][B][stride],
    C-contiguous) receives, added in place, every live token's softmax weight
    summed over the query heads."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, Hq, D = q.shape
    nseg = len(caches)
    bts = [_i32(t) for t in block_tables]
    lens = [_i32(n) for n in seq_lens]
    ccs = (_Cache * nseg)(*[c.c() for c in caches])
    views = (_View * nseg)(*[_View(bt.ctypes.data, ln.ctypes.data, bt.shape[1]) for bt, ln in zip(bts, lens)])
    out = np.zeros((B, Hq, D), np.float64)
    skip = None
    if want_skip:
        max_tok = max(bt.shape[1] for bt in bts) * BLOCK_TOKENS
        skip = np.zeros((B, Hq, nseg, max_tok), np.uint8)
    if score_acc is not None:
        assert score_acc.dtype == np.float64 and score_acc.flags.c_contiguous
        assert score_acc.ndim == 3 and score_acc.shape[:2] == (nseg, B)
    rc = lib().orc_decode(ccs, views, nseg, _p(q), B, Hq, sm_scale, tau_low, split_tokens,
                          _p(out), _p(skip) if skip is not None else None,
                          _p(score_acc) if score_acc is not None else None,
                          score_acc.shape[2] if score_acc is not None else 0)
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    return (out, skip) if want_skip else out


def decode_resolved(caches, block_tables, seq_lens, q: np.ndarray, sm_scale: float, tau_low: float,
                    split_tokens: int, given: np.ndarray | None, band: float, score_acc: np.ndarray | None = None):
    """decode() with the skip decisions near the threshold resolved.

    A (token, head) pair whose exact margin |exp(s - m) - tau_low L| is at
    most band * tau_low * L can take either decision in finite precision; for
    it the decision in `given` (uint8 [B][Hq][nseg][max_tok], 1 = skipped; None
    keeps the exact one) is taken.  Returns (out fp64 [B][Hq][D], skip,
    ambiguous, margin): skip and ambiguous uint8 in the layout of given, margin
    fp64 the relative margin (exp(s - m) - tau_low L) / (tau_low L) of every
    live pair (0 elsewhere).  score_acc: as in decode() (the weights do not
    depend on the skip)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, Hq, D = q.shape
    nseg = len(caches)
    bts = [_i32(t) for t in block_tables]
    lens = [_i32(n) for n in seq_lens]
    ccs = (_Cache * nseg)(*[c.c() for c in caches])
    views = (_View * nseg)(*[_View(bt.ctypes.data, ln.ctypes.data, bt.shape[1]) for bt, ln in zip(bts, lens)])
    max_tok = max(bt.shape[1] for bt in bts) * BLOCK_TOKENS
    shape = (B, Hq, nseg, max_tok)
    out = np.zeros((B, Hq, D), np.float64)
    skip = np.zeros(shape, np.uint8)
    amb = np.zeros(shape, np.uint8)
    margin = np.zeros(shape, np.float64)
    if given is not None:
        given = np.ascontiguousarray(given, dtype=np.uint8)
        if given.shape != shape:
            raise ValueError(f"given must be {shape}")
    if score_acc is not None:
        assert score_acc.dtype == np.float64 and score_acc.flags.c_contiguous
        assert score_acc.ndim == 3 and score_acc.shape[:2] == (nseg, B)
    rc = lib().orc_decode_resolved(ccs, views, nseg, _p(q), B, Hq, sm_scale, tau_low, split_tokens, _p(out),
                                   _p(skip), _p(given) if given is not None else None, float(band), _p(amb),
                                   _p(margin), _p(score_acc) if score_acc is not None else None,
                                   score_acc.shape[2] if score_acc is not None else 0)
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    return out, skip, amb, margin


def multi_entries(block_tables, seq_lens, T: int):
    """The decode entries of T query tokens per sequence: entry (b, i) reads
    sequence b's tables, with segment 0 cut to its causal prefix
    0 .. L - T + i.  Returns (tables, lens) per segment."""
    bts = [_i32(t) for t in block_tables]
    lens = [_i32(n) for n in seq_lens]
    if T < 1 or np.any(lens[0] < T):
        raise ValueError("every sequence must hold its T query tokens")
    B = len(lens[0])
    ebts = [np.repeat(bt, T, axis=0) for bt in bts]                  # entry (b, i): sequence b's table
    elens = [np.repeat(ln, T) for ln in lens]
    elens[0] = elens[0] - (T - 1) + np.tile(np.arange(T, dtype=np.int32), B)  # causal prefix in segment 0
    return ebts, elens


def decode_multi(caches, block_tables, seq_lens, q: np.ndarray, sm_scale: float,
                 tau_low: float = 0.0, split_tokens: int = 0):
    """Attention of T query tokens per sequence over the packed cache, with a
    causal mask (the queries of a chunked prefill, or tokens to verify).

    q: fp32 [B][T][Hq][D]; seq_lens count every cached token including the T
    new ones, which are the last T tokens of the first segment.  Query token
    i of sequence b sits at position L - T + i of that segment and attends to
    every token of the other segments and to the first segment's tokens
    0 .. L - T + i.  Each query token is therefore one decode query (decode
    above) over that causal prefix, with the same split size and sparse-V
    rule.  Returns fp64 [B][T][Hq][D]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, T, Hq, D = q.shape
    ebts, elens = multi_entries(block_tables, seq_lens, T)
    out = decode(caches, ebts, elens, q.reshape(B * T, Hq, D), sm_scale, tau_low, split_tokens)
    return out.reshape(B, T, Hq, D)


def tier_update(src: Cache, src_bt, src_lens, scores: np.ndarray, tau_low: float, tau_high: float,
                dst_h: Cache, h_bt, dst_m: Cache, m_bt):
    """Returns (tiers uint8 [B][stride], n_high int32 [B], n_mid int32 [B])."""
    sbt = _i32(src_bt)
    sl = _i32(src_lens)
    hb = _i32(h_bt)
    mb = _i32(m_bt)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    B, stride = scores.shape
    tiers = np.full((B, stride), 255, np.uint8)
    nh = np.zeros(B, np.int32)
    nm = np.zeros(B, np.int32)
    cs, ch, cm = src.c(), dst_h.c(), dst_m.c()
    view = _View(sbt.ctypes.data, sl.ctypes.data, sbt.shape[1])
    rc = lib().orc_tier_update(C.byref(cs), C.byref(view), _p(scores), stride, tau_low, tau_high,
                               C.byref(ch), _p(hb), hb.shape[1], C.byref(cm), _p(mb), mb.shape[1],
                               _p(nh), _p(nm), _p(tiers), B)
    if rc != 0:
        raise ValueError("oracle tier update rejected its arguments")
    return tiers, nh, nm


def retier(h: Cache, h_bt, h_lens, h_scores: np.ndarray, m: Cache, m_bt, m_lens, m_scores: np.ndarray,
           tau_low: float, tau_high: float, dst_h: Cache, dh_bt, dst_m: Cache, dm_bt):
    """Re-tiering of a tiered cache {h: K6V6, m: K6V4} with fresh scores.
    Returns (h_tiers uint8 [B][h_stride], m_tiers uint8 [B][m_stride],
    n_high int32 [B], n_mid int32 [B])."""
    hb, hl, mb, ml = _i32(h_bt), _i32(h_lens), _i32(m_bt), _i32(m_lens)
    dhb, dmb = _i32(dh_bt), _i32(dm_bt)
    hs = np.ascontiguousarray(h_scores, dtype=np.float32)
    ms = np.ascontiguousarray(m_scores, dtype=np.float32)
    B = hs.shape[0]
    ht = np.full(hs.shape, 255, np.uint8)
    mt = np.full(ms.shape, 255, np.uint8)
    nh = np.zeros(B, np.int32)
    nm = np.zeros(B, np.int32)
    ch, cm, cdh, cdm = h.c(), m.c(), dst_h.c(), dst_m.c()
    hv = _View(hb.ctypes.data, hl.ctypes.data, hb.shape[1])
    mv = _View(mb.ctypes.data, ml.ctypes.data, mb.shape[1])
    rc = lib().orc_retier(C.byref(ch), C.byref(hv), _p(hs), hs.shape[1], C.byref(cm), C.byref(mv), _p(ms),
                          ms.shape[1], tau_low, tau_high, C.byref(cdh), _p(dhb), dhb.shape[1], C.byref(cdm), _p(dmb),
                          dmb.shape[1], _p(nh), _p(nm), _p(ht), _p(mt), B)
    if rc != 0:
        raise ValueError("oracle retier rejected its arguments")
    return ht, mt, nh, nm
