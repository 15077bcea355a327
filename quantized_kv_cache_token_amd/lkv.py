"""Thin ctypes binding of the C ABI in include/lkv.h.

Argument marshalling only: every step of the path runs in the HIP kernels of
liblkv.so.  Tensors are torch tensors on the GPU (PyTorch provides device
memory and streams); work is queued on torch's current stream.  If the
library is missing, loading it raises -- there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblkv.so")
BLOCK_TOKENS = 64

OK, EINVAL, EUNSUPPORTED, EHIP, ESCRATCH = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 16 << 20  # LKV_NOALLOC_SCRATCH_BYTES
F32, BF16, F16 = 0, 1, 2
_DTYPE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class LkvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} ({status})")
        self.status = status


class _Cache(C.Structure):
    _fields_ = [("head_dim", C.c_int32), ("group_size", C.c_int32), ("k_bits", C.c_int32),
                ("v_bits", C.c_int32), ("num_kv_heads", C.c_int32), ("block_tokens", C.c_int32),
                ("num_blocks", C.c_int64), ("pool", C.c_void_p), ("k_norm", C.c_int32)]


class _View(C.Structure):
    _fields_ = [("block_table", C.c_void_p), ("seq_lens", C.c_void_p), ("max_blocks", C.c_int32),
                ("max_len", C.c_int32), ("sum_len", C.c_int64)]


_lib = None

EXPORTS = ["lkv_status_string", "lkv_chunk_layout", "lkv_quant_append", "lkv_decode_plan",
           "lkv_decode_workspace_bytes", "lkv_decode_attn", "lkv_decode_split", "lkv_decode_combine",
           "lkv_decode_scores_workspace_bytes", "lkv_decode_attn_scores",
           "lkv_default_thresholds", "lkv_tier_workspace_bytes", "lkv_tier_update",
           "lkv_retier_workspace_bytes", "lkv_retier", "lkv_decode_attn_multi", "lkv_decode_plan_multi",
           "lkv_decode_attn_debug", "lkv_decode_attn_noalloc", "lkv_append_decode", "lkv_append_split",
           "lkv_hbm_read_probe", "lkv_append_decode_merged", "lkv_decode_plan_lens"]


def lib():
    """Load liblkv.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"{LIB_PATH} is missing: build it with `python -m quantized_kv_cache_token_amd.build`")
    L = C.CDLL(LIB_PATH)
    P, I32, I64, F, V = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_void_p
    PC, PV = C.POINTER(_Cache), C.POINTER(_View)
    sig = {
        "lkv_status_string": ([C.c_int], C.c_char_p),
        "lkv_chunk_layout": ([I32, I32, I32, I32, C.POINTER(I64)], C.c_int),
        "lkv_quant_append": ([PC, P, P, I32, P, P, P, I32, I32, I32, V], C.c_int),
        "lkv_decode_plan": ([PC, PV, I32, I32, I32, C.POINTER(I32)], C.c_int),
        "lkv_decode_plan_lens": ([PC, PV, P, I32, I32, C.POINTER(I32)], C.c_int),
        "lkv_decode_workspace_bytes": ([PC, PV, I32, I32, I32, I32], I64),
        "lkv_decode_attn": ([PC, PV, I32, P, I32, I32, I32, F, F, I32, P, P, C.c_size_t, V], C.c_int),
        "lkv_decode_split": ([PC, PV, I32, P, I32, I32, I32, F, F, I32, P, C.c_size_t, V], C.c_int),
        "lkv_decode_combine": ([PC, PV, I32, I32, I32, I32, P, P, C.c_size_t, V], C.c_int),
        "lkv_decode_scores_workspace_bytes": ([PC, PV, I32, I32, I32, I32], I64),
        "lkv_decode_attn_scores": ([PC, PV, I32, P, I32, I32, I32, F, F, I32, P, P, I32, P, C.c_size_t, V],
                                   C.c_int),
        "lkv_default_thresholds": ([I32, C.POINTER(F), C.POINTER(F)], None),
        "lkv_tier_workspace_bytes": ([I32, I32], I64),
        "lkv_tier_update": ([PC, PV, P, I32, F, F, PC, P, I32, PC, P, I32, P, P, P, I32, P, C.c_size_t, V],
                            C.c_int),
        "lkv_retier_workspace_bytes": ([I32, I32, I32], I64),
        "lkv_decode_attn_multi": ([PC, PV, I32, P, I32, I32, I32, I32, F, F, I32, P, P, C.c_size_t, V], C.c_int),
        "lkv_decode_plan_multi": ([PC, PV, I32, I32, I32, I32, C.POINTER(I32)], C.c_int),
        "lkv_append_decode": ([PC, PV, P, P, I32, P, I32, I32, I32, F, F, I32, P, P, C.c_size_t, V], C.c_int),
        "lkv_append_split": ([PC, PV, P, P, I32, P, I32, I32, I32, F, F, I32, P, C.c_size_t, V], C.c_int),
        "lkv_append_decode_merged": ([PC, PV, I32, P, P, I32, P, I32, I32, I32, F, F, I32, P, P, P, C.c_size_t,
                                      V], C.c_int),
        "lkv_decode_attn_noalloc": ([PC, PV, I32, P, I32, I32, I32, F, F, I32, P, V], C.c_int),
        "lkv_hbm_read_probe": ([P, I64, I32, P, V], C.c_int),
        "lkv_decode_attn_debug": ([PC, PV, I32, P, I32, I32, I32, I32, F, F, I32, P, P, I32, P, C.c_size_t, V],
                                  C.c_int),
        "lkv_retier": ([PC, PV, P, I32, PC, PV, P, I32, F, F, PC, P, I32, PC, P, I32, P, P, P, P, I32, P,
                        C.c_size_t, V], C.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().lkv_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise LkvError(fn, status)


def _require(cond: bool, what: str) -> None:
    """Argument check of the binding; unlike assert it is kept under -O."""
    if not cond:
        raise ValueError(what)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _on(stream=None):
    """Context for the binding's own allocations (outputs, workspaces): on the
    stream the call's kernels run on, so that the caching allocator does not
    hand that memory to other work while they are queued."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def chunk_layout(head_dim: int, group_size: int, k_bits: int, v_bits: int) -> list[int]:
    off = (C.c_int64 * 7)()
    _check("lkv_chunk_layout", lib().lkv_chunk_layout(head_dim, group_size, k_bits, v_bits, off))
    return list(off)


@dataclass
class Cache:
    """A cache: format plus a device pool [num_blocks][Hkv][chunk] (uint8)."""
    head_dim: int
    group_size: int
    k_bits: int
    v_bits: int
    num_kv_heads: int
    num_blocks: int
    pool: torch.Tensor = None
    device: str = "cuda"
    k_norm: int = 0  # 1: direction-preserving K, one fp32 norm factor per slot after the six sections

    def __post_init__(self):
        self.knorm_offset = chunk_layout(self.head_dim, self.group_size, self.k_bits, self.v_bits)[6]
        self.chunk_bytes = self.knorm_offset + (BLOCK_TOKENS * 4 if self.k_norm else 0)
        nbytes = self.num_blocks * self.num_kv_heads * self.chunk_bytes
        if self.pool is None:
            self.pool = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        _require(self.pool.numel() == nbytes and self.pool.dtype == torch.uint8,
                 f"pool must be {nbytes} uint8 bytes")

    def c(self) -> _Cache:
        return _Cache(self.head_dim, self.group_size, self.k_bits, self.v_bits, self.num_kv_heads,
                      BLOCK_TOKENS, self.num_blocks, self.pool.data_ptr(), self.k_norm)


@dataclass
class View:
    """Which blocks and how many tokens of a cache a batch reads."""
    block_table: torch.Tensor   # int32 [B][max_blocks], device
    seq_lens: torch.Tensor      # int32 [B], device
    max_len: int                # host upper bound of seq_lens
    sum_len: int = 0            # host hint: total of seq_lens (0 = unknown); sizes splits, marks a batch ragged

    def c(self) -> _View:
        _require(self.block_table.dtype == torch.int32 and self.seq_lens.dtype == torch.int32,
                 "block_table and seq_lens must be int32")
        _require(self.block_table.is_contiguous() and self.seq_lens.is_contiguous(),
                 "block_table and seq_lens must be contiguous")
        return _View(self.block_table.data_ptr(), self.seq_lens.data_ptr(), self.block_table.shape[1],
                     int(self.max_len), int(self.sum_len))


def quant_append(cache: Cache, k: torch.Tensor, v: torch.Tensor, cu_new: torch.Tensor, start_pos: torch.Tensor,
                 block_table: torch.Tensor, max_new: int, stream=None) -> None:
    """lkv_quant_append: k, v [total_new][Hkv][D] (fp32, bf16 or fp16)."""
    _require(k.dtype == v.dtype and k.is_contiguous() and v.is_contiguous(), "k and v: one dtype, contiguous")
    _require(k.shape == v.shape and k.shape[1:] == (cache.num_kv_heads, cache.head_dim),
             "k and v must be [total_new][Hkv][D] of the cache")
    cc = cache.c()
    _check("lkv_quant_append", lib().lkv_quant_append(
        C.byref(cc), _ptr(k), _ptr(v), _DTYPE[k.dtype], _ptr(cu_new), _ptr(start_pos), _ptr(block_table),
        block_table.shape[1], start_pos.shape[0], int(max_new), _stream(stream)))


def _segs(caches, views):
    n = len(caches)
    _require(n == len(views), "one view per cache")
    return (_Cache * n)(*[c.c() for c in caches]), (_View * n)(*[v.c() for v in views]), n


def decode_plan(caches, views, batch: int, num_q_heads: int) -> int:
    cs, vs, n = _segs(caches, views)
    out = C.c_int32()
    _check("lkv_decode_plan", lib().lkv_decode_plan(cs, vs, n, batch, num_q_heads, C.byref(out)))
    return out.value


def decode_plan_lens(cache: Cache, view: View, host_lens, num_q_heads: int) -> int:
    """lkv_decode_plan_lens: the decode step's split size from the host's
    lengths (a sequence of ints, the new token counted)."""
    import numpy as np

    lens = np.ascontiguousarray(np.asarray(host_lens, dtype=np.int32))
    out = C.c_int32()
    cc, vc = cache.c(), view.c()
    _check("lkv_decode_plan_lens", lib().lkv_decode_plan_lens(C.byref(cc), C.byref(vc), lens.ctypes.data, lens.size,
                                                              num_q_heads, C.byref(out)))
    return out.value


def decode_plan_multi(caches, views, batch: int, q_per_seq: int, num_q_heads: int) -> int:
    """lkv_decode_plan_multi: the split size decode_attn_multi plans."""
    cs, vs, n = _segs(caches, views)
    out = C.c_int32()
    _check("lkv_decode_plan_multi", lib().lkv_decode_plan_multi(cs, vs, n, batch, q_per_seq, num_q_heads,
                                                                C.byref(out)))
    return out.value


def decode_workspace_bytes(caches, views, batch: int, num_q_heads: int, split_tokens: int) -> int:
    cs, vs, n = _segs(caches, views)
    r = lib().lkv_decode_workspace_bytes(cs, vs, n, batch, num_q_heads, split_tokens)
    if r < 0:
        raise LkvError("lkv_decode_workspace_bytes", r)
    return r


def decode_workspace(caches, views, batch, num_q_heads, split_tokens, device="cuda") -> torch.Tensor:
    nbytes = decode_workspace_bytes(caches, views, batch, num_q_heads, split_tokens)
    return torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=device)


def decode_attn(caches, views, q: torch.Tensor, sm_scale: float, tau_low: float = 0.0, split_tokens: int = 0,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """lkv_decode_attn: q [B][Hq][D] (fp32 or bf16) -> out fp32 [B][Hq][D]."""
    B, Hq, D = q.shape
    _require(q.is_contiguous(), "q must be contiguous")
    if split_tokens == 0:
        split_tokens = decode_plan(caches, views, B, Hq)
    with _on(stream):
        if workspace is None:
            workspace = decode_workspace(caches, views, B, Hq, split_tokens, q.device)
        if out is None:
            out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    cs, vs, n = _segs(caches, views)
    _check("lkv_decode_attn", lib().lkv_decode_attn(
        cs, vs, n, _ptr(q), _DTYPE[q.dtype], B, Hq, sm_scale, tau_low, split_tokens, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def append_decode(cache: Cache, view: View, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                  sm_scale: float, tau_low: float = 0.0, split_tokens: int = 0, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None):
    """lkv_append_decode: append each sequence's new row (k_new, v_new
    [B][Hkv][D]) at position seq_lens[b] - 1, then decode q [B][Hq][D] over
    seq_lens[b] tokens -> out fp32 [B][Hq][D]."""
    B, Hq, D = q.shape
    _require(q.is_contiguous() and k_new.is_contiguous() and v_new.is_contiguous(), "q, k_new, v_new contiguous")
    _require(k_new.dtype == v_new.dtype and k_new.shape == v_new.shape == (B, cache.num_kv_heads, cache.head_dim),
             "k_new and v_new must be [B][Hkv][D] of one dtype")
    if split_tokens == 0:
        split_tokens = decode_plan([cache], [view], B, Hq)
    with _on(stream):
        if workspace is None:
            workspace = decode_workspace([cache], [view], B, Hq, split_tokens, q.device)
        if out is None:
            out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    cc, vc = cache.c(), view.c()
    _check("lkv_append_decode", lib().lkv_append_decode(
        C.byref(cc), C.byref(vc), _ptr(k_new), _ptr(v_new), _DTYPE[k_new.dtype], _ptr(q), _DTYPE[q.dtype], B, Hq,
        sm_scale, tau_low, split_tokens, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor, nontemporal: bool = False, stream=None) -> None:
    """lkv_hbm_read_probe: a streaming read of buf (a device tensor)."""
    _require(buf.is_cuda and buf.is_contiguous() and sink.dtype in (torch.int32, torch.uint32) and sink.is_cuda,
             "buf: contiguous device tensor; sink: one device int32")
    _check("lkv_hbm_read_probe", lib().lkv_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(),
                                                          int(nontemporal), _ptr(sink), _stream(stream)))


def decode_attn_noalloc(caches, views, q: torch.Tensor, sm_scale: float, tau_low: float = 0.0,
                        split_tokens: int = 0, out: torch.Tensor | None = None, stream=None):
    """lkv_decode_attn_noalloc: decode_attn with the split partials in the
    library's static device scratch (no workspace).  With `out` given, the
    call allocates nothing at all."""
    B, Hq, D = q.shape
    _require(q.is_contiguous(), "q must be contiguous")
    if out is None:
        with _on(stream):
            out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    cs, vs, n = _segs(caches, views)
    _check("lkv_decode_attn_noalloc", lib().lkv_decode_attn_noalloc(
        cs, vs, n, _ptr(q), _DTYPE[q.dtype], B, Hq, sm_scale, tau_low, split_tokens, _ptr(out), _stream(stream)))
    return out


def decode_attn_multi(caches, views, q: torch.Tensor, sm_scale: float, tau_low: float = 0.0,
                      split_tokens: int = 0, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None):
    """lkv_decode_attn_multi: q [B][T][Hq][D] (fp32 or bf16), the last T
    tokens of the first segment -> out fp32 [B][T][Hq][D], causal."""
    B, T, Hq, D = q.shape
    _require(q.is_contiguous(), "q must be contiguous")
    if split_tokens == 0:
        split_tokens = decode_plan_multi(caches, views, B, T, Hq)
    with _on(stream):
        if workspace is None:
            workspace = decode_workspace(caches, views, B * T, Hq, split_tokens, q.device)
        if out is None:
            out = torch.empty(B, T, Hq, D, dtype=torch.float32, device=q.device)
    cs, vs, n = _segs(caches, views)
    _check("lkv_decode_attn_multi", lib().lkv_decode_attn_multi(
        cs, vs, n, _ptr(q), _DTYPE[q.dtype], B, T, Hq, sm_scale, tau_low, split_tokens, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def skip_mask_words(views) -> int:
    """Words per row of the skip mask of decode_attn_debug: every segment's
    max_len rounded up to 64 tokens, one bit per token."""
    return sum(-(-int(v.max_len) // BLOCK_TOKENS) * BLOCK_TOKENS for v in views) // 32


def decode_attn_debug(caches, views, q: torch.Tensor, sm_scale: float, tau_low: float = 0.0,
                      split_tokens: int = 0, stream=None):
    """lkv_decode_attn_debug: decode_attn (q [B][Hq][D]) or decode_attn_multi
    (q [B][T][Hq][D]) that also returns the sparse-V skip decisions.  Returns
    (out, mask): mask int32 [B*T][Hq][words], bit c set when score column c
    (the first segment's tokens, then the second's from its max_len rounded
    up to 64) had its V term skipped.  For tests."""
    if q.dim() == 3:
        B, Hq, D = q.shape
        T = 1
    else:
        B, T, Hq, D = q.shape
    _require(q.is_contiguous(), "q must be contiguous")
    if split_tokens == 0:
        split_tokens = decode_plan_multi(caches, views, B, T, Hq)
    words = max(skip_mask_words(views), 1)
    with _on(stream):
        workspace = decode_workspace(caches, views, B * T, Hq, split_tokens, q.device)
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        mask = torch.empty(B * T, Hq, words, dtype=torch.int32, device=q.device)
    cs, vs, n = _segs(caches, views)
    _check("lkv_decode_attn_debug", lib().lkv_decode_attn_debug(
        cs, vs, n, _ptr(q), _DTYPE[q.dtype], B, T, Hq, sm_scale, tau_low, split_tokens, _ptr(out), _ptr(mask),
        words, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, mask


def decode_scores_workspace(caches, views, batch, num_q_heads, split_tokens, device="cuda") -> torch.Tensor:
    cs, vs, n = _segs(caches, views)
    r = lib().lkv_decode_scores_workspace_bytes(cs, vs, n, batch, num_q_heads, split_tokens)
    if r < 0:
        raise LkvError("lkv_decode_scores_workspace_bytes", r)
    return torch.empty(max(r, 4), dtype=torch.uint8, device=device)


def decode_attn_scores(caches, views, q: torch.Tensor, score_acc: torch.Tensor, sm_scale: float,
                       tau_low: float = 0.0, split_tokens: int = 0, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, stream=None):
    """lkv_decode_attn_scores: decode as decode_attn, and add each live
    token's softmax weight summed over the query heads to score_acc
    (fp32 [nseg][B][stride])."""
    B, Hq, D = q.shape
    _require(q.is_contiguous() and score_acc.is_contiguous() and score_acc.dtype == torch.float32,
             "q and score_acc contiguous, score_acc fp32")
    _require(score_acc.dim() == 3 and score_acc.shape[:2] == (len(caches), B), "score_acc must be [nseg][B][stride]")
    if split_tokens == 0:
        split_tokens = decode_plan(caches, views, B, Hq)
    with _on(stream):
        if workspace is None:
            workspace = decode_scores_workspace(caches, views, B, Hq, split_tokens, q.device)
        if out is None:
            out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    cs, vs, n = _segs(caches, views)
    _check("lkv_decode_attn_scores", lib().lkv_decode_attn_scores(
        cs, vs, n, _ptr(q), _DTYPE[q.dtype], B, Hq, sm_scale, tau_low, split_tokens, _ptr(out), _ptr(score_acc),
        score_acc.shape[2], _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def decode_split(caches, views, q, sm_scale, tau_low, split_tokens, workspace, stream=None) -> None:
    B, Hq, _ = q.shape
    cs, vs, n = _segs(caches, views)
    _check("lkv_decode_split", lib().lkv_decode_split(
        cs, vs, n, _ptr(q), _DTYPE[q.dtype], B, Hq, sm_scale, tau_low, split_tokens, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_combine(caches, views, batch, num_q_heads, split_tokens, out, workspace, stream=None) -> None:
    cs, vs, n = _segs(caches, views)
    _check("lkv_decode_combine", lib().lkv_decode_combine(
        cs, vs, n, batch, num_q_heads, split_tokens, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def default_thresholds(n_tokens: int) -> tuple[float, float]:
    lo, hi = C.c_float(), C.c_float()
    lib().lkv_default_thresholds(n_tokens, C.byref(lo), C.byref(hi))
    return lo.value, hi.value


def tier_workspace_bytes(batch: int, scores_stride: int) -> int:
    r = lib().lkv_tier_workspace_bytes(batch, scores_stride)
    if r < 0:
        raise LkvError("lkv_tier_workspace_bytes", r)
    return r


def tier_update(src: Cache, src_view: View, scores: torch.Tensor, tau_low: float, tau_high: float,
                dst_h: Cache, h_block_table: torch.Tensor, dst_m: Cache, m_block_table: torch.Tensor,
                n_high: torch.Tensor, n_mid: torch.Tensor, tiers: torch.Tensor,
                workspace: torch.Tensor | None = None, stream=None) -> None:
    """lkv_tier_update: scores fp32 [B][stride]; tiers uint8 [B][stride]."""
    B, stride = scores.shape
    _require(scores.dtype == torch.float32 and tiers.dtype == torch.uint8 and tiers.shape == scores.shape,
             "scores fp32 and tiers uint8, both [B][stride]")
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(tier_workspace_bytes(B, stride), 4), dtype=torch.uint8,
                                    device=scores.device)
    cs, ch, cm, sv = src.c(), dst_h.c(), dst_m.c(), src_view.c()
    _check("lkv_tier_update", lib().lkv_tier_update(
        C.byref(cs), C.byref(sv), _ptr(scores), stride, tau_low, tau_high, C.byref(ch), _ptr(h_block_table),
        h_block_table.shape[1], C.byref(cm), _ptr(m_block_table), m_block_table.shape[1], _ptr(n_high),
        _ptr(n_mid), _ptr(tiers), B, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def retier_workspace_bytes(batch: int, h_stride: int, m_stride: int) -> int:
    r = lib().lkv_retier_workspace_bytes(batch, h_stride, m_stride)
    if r < 0:
        raise LkvError("lkv_retier_workspace_bytes", r)
    return r


def retier(h: Cache, h_view: View, h_scores: torch.Tensor, m: Cache, m_view: View, m_scores: torch.Tensor,
           tau_low: float, tau_high: float, dst_h: Cache, dh_block_table: torch.Tensor, dst_m: Cache,
           dm_block_table: torch.Tensor, n_high: torch.Tensor, n_mid: torch.Tensor, h_tiers: torch.Tensor,
           m_tiers: torch.Tensor, workspace: torch.Tensor | None = None, stream=None) -> None:
    """lkv_retier: scores fp32 [B][stride] per segment; tiers uint8 of the
    same shapes."""
    B, hs = h_scores.shape
    ms = m_scores.shape[1]
    _require(m_scores.shape[0] == B and h_scores.dtype == torch.float32 and m_scores.dtype == torch.float32,
             "scores fp32 [B][stride] per segment")
    _require(h_tiers.dtype == torch.uint8 and h_tiers.shape == h_scores.shape, "h_tiers uint8, shape of h_scores")
    _require(m_tiers.dtype == torch.uint8 and m_tiers.shape == m_scores.shape, "m_tiers uint8, shape of m_scores")
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(retier_workspace_bytes(B, hs, ms), 8), dtype=torch.uint8,
                                    device=h_scores.device)
    ch, cm, cdh, cdm, hv, mv = h.c(), m.c(), dst_h.c(), dst_m.c(), h_view.c(), m_view.c()
    _check("lkv_retier", lib().lkv_retier(
        C.byref(ch), C.byref(hv), _ptr(h_scores), hs, C.byref(cm), C.byref(mv), _ptr(m_scores), ms, tau_low,
        tau_high, C.byref(cdh), _ptr(dh_block_table), dh_block_table.shape[1], C.byref(cdm),
        _ptr(dm_block_table), dm_block_table.shape[1], _ptr(n_high), _ptr(n_mid), _ptr(h_tiers), _ptr(m_tiers), B,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


class Prepared:
    """Pre-marshalled calls for a fixed set of tensors, for loops that issue
    the same call many times (the ctypes structures are built once).  The
    tensors must stay alive and keep their storage while it is used."""

    def __init__(self, fn: str, *args):
        self._fn = getattr(lib(), fn)
        self._name = fn
        self._args = args

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != OK:
            raise LkvError(self._name, st)


def prepare_append(cache: Cache, k, v, cu_new, start_pos, block_table, max_new: int, stream=None) -> Prepared:
    cc = cache.c()
    return Prepared("lkv_quant_append", C.byref(cc), _ptr(k), _ptr(v), _DTYPE[k.dtype], _ptr(cu_new),
                    _ptr(start_pos), _ptr(block_table), block_table.shape[1], start_pos.shape[0], int(max_new),
                    _stream(stream))


def prepare_decode_scores(caches, views, q, sm_scale: float, tau_low: float, split_tokens: int, out, score_acc,
                          workspace, stream=None) -> Prepared:
    """lkv_decode_attn_scores as a prepared call."""
    B, Hq, _ = q.shape
    cs, vs, n = _segs(caches, views)
    call = Prepared("lkv_decode_attn_scores", cs, vs, n, _ptr(q), _DTYPE[q.dtype], B, Hq, sm_scale, tau_low,
                    split_tokens, _ptr(out), _ptr(score_acc), score_acc.shape[2], _ptr(workspace),
                    workspace.numel() * workspace.element_size(), _stream(stream))
    call._keep = (cs, vs)
    return call


def prepare_append_decode(cache: Cache, view: View, k_new, v_new, q, sm_scale: float, tau_low: float,
                          split_tokens: int, out, workspace, stream=None) -> tuple[Prepared, Prepared]:
    """(append + split, combine) stages of lkv_append_decode as prepared calls."""
    B, Hq, _ = q.shape
    cs, vs, n = _segs([cache], [view])
    nbytes = workspace.numel() * workspace.element_size()
    st = _stream(stream)
    split = Prepared("lkv_append_split", cs, vs, _ptr(k_new), _ptr(v_new), _DTYPE[k_new.dtype], _ptr(q),
                     _DTYPE[q.dtype], B, Hq, sm_scale, tau_low, split_tokens, _ptr(workspace), nbytes, st)
    comb = Prepared("lkv_decode_combine", cs, vs, n, B, Hq, split_tokens, _ptr(out), _ptr(workspace), nbytes, st)
    split._keep = comb._keep = (cs, vs)
    return split, comb


def merge_counters(cache: Cache, batch: int, device="cuda") -> torch.Tensor:
    """Zeroed counters for lkv_append_decode_merged: uint32 per (sequence, KV head)."""
    return torch.zeros(batch * cache.num_kv_heads, dtype=torch.int32, device=device)


def _seg_list(cache, view):
    """A cache and its view, or lists of them (a tiered cache's segments)."""
    caches = list(cache) if isinstance(cache, (list, tuple)) else [cache]
    views = list(view) if isinstance(view, (list, tuple)) else [view]
    return caches, views


def append_decode_merged(cache, view, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                         sm_scale: float, tau_low: float, split_tokens: int, counters: torch.Tensor,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """lkv_append_decode_merged: the decode step in one launch (the split
    kernel appends the new rows and merges its own splits); counters from
    merge_counters().  cache and view: one segment, or the lists [HIGH, MID]
    of a tiered cache (the new rows go to HIGH)."""
    caches, views = _seg_list(cache, view)
    B, Hq, D = q.shape
    _require(q.is_contiguous() and k_new.is_contiguous() and v_new.is_contiguous() and k_new.dtype == v_new.dtype,
             "q, k_new, v_new contiguous; k_new and v_new of one dtype")
    _require(counters.dtype == torch.int32 and counters.numel() >= B * caches[0].num_kv_heads and counters.is_cuda,
             "counters: int32 [batch * KV heads] on the device")
    with _on(stream):
        if workspace is None:
            workspace = decode_workspace(caches, views, B, Hq, split_tokens, q.device)
        if out is None:
            out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    cs, vs, n = _segs(caches, views)
    _check("lkv_append_decode_merged", lib().lkv_append_decode_merged(
        cs, vs, n, _ptr(k_new), _ptr(v_new), _DTYPE[k_new.dtype], _ptr(q), _DTYPE[q.dtype], B, Hq, sm_scale,
        tau_low, split_tokens, _ptr(out), _ptr(counters), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def prepare_append_decode_merged(cache, view, k_new, v_new, q, sm_scale: float, tau_low: float,
                                 split_tokens: int, out, counters, workspace, stream=None) -> Prepared:
    """lkv_append_decode_merged as a prepared call (cache and view as in
    append_decode_merged)."""
    caches, views = _seg_list(cache, view)
    B, Hq, _ = q.shape
    cs, vs, n = _segs(caches, views)
    call = Prepared("lkv_append_decode_merged", cs, vs, n, _ptr(k_new), _ptr(v_new), _DTYPE[k_new.dtype], _ptr(q),
                    _DTYPE[q.dtype], B, Hq, sm_scale, tau_low, split_tokens, _ptr(out), _ptr(counters),
                    _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    call._keep = (cs, vs)
    return call


def prepare_decode(caches, views, q, sm_scale: float, tau_low: float, split_tokens: int, out, workspace,
                   stream=None) -> tuple[Prepared, Prepared]:
    """(split, combine) stages of lkv_decode_attn as prepared calls."""
    B, Hq, _ = q.shape
    cs, vs, n = _segs(caches, views)
    nbytes = workspace.numel() * workspace.element_size()
    st = _stream(stream)
    split = Prepared("lkv_decode_split", cs, vs, n, _ptr(q), _DTYPE[q.dtype], B, Hq, sm_scale, tau_low,
                     split_tokens, _ptr(workspace), nbytes, st)
    comb = Prepared("lkv_decode_combine", cs, vs, n, B, Hq, split_tokens, _ptr(out), _ptr(workspace), nbytes, st)
    split._keep = comb._keep = (cs, vs)
    return split, comb
