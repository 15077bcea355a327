"""The allocation-free decode entry point (lkv_decode_attn_noalloc), for
callers that cannot allocate device memory, against lkv_decode_attn on the
same inputs: two calls in a row, the second with a smaller input, bit for
bit (same kernels, same split plan; only the partials' address differs)."""
import numpy as np
import pytest
import torch

from quantized_kv_cache_token_amd import inputs, lkv
from tests.gpu_common import Pair, say, sm_scale
from tests.oracle_cases import block_tables
from tests.test_gpu_parity import _prefill

pytestmark = pytest.mark.gpu


def _case(lens, Hkv, G, seed, fmt=(128, 64, 6, 4), qdtype="bf16"):
    D, g, kb, vb = fmt
    rng = np.random.default_rng(seed)
    bt, nblk = block_tables(lens, rng)
    pair = Pair(D, g, kb, vb, Hkv, nblk)
    _prefill(pair, lens, Hkv, D, "bf16", seed, bt, outliers=True)
    view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    q = inputs.queries(seed, len(lens), Hkv * G, D, dtype=qdtype).cuda()
    return pair, view, q


@pytest.mark.parametrize("fmt,G,qdtype", [((128, 64, 6, 4), 4, "bf16"), ((128, 64, 6, 4), 8, "bf16"),
                                          ((128, 64, 16, 16), 8, "bf16"), ((64, 32, 6, 4), 2, "f32")])
def test_noalloc_equals_decode_on_two_calls_in_a_row(fmt, G, qdtype):
    D = fmt[0]
    big = _case([3000, 64, 1, 2500, 777], 2, G, 90, fmt, qdtype)
    small = _case([100, 65], 1, G, 91, fmt, qdtype)
    for name, (pair, view, q), tau in (("larger", big, 1e-3), ("smaller", small, 0.0)):
        say("noalloc", fmt, "G", G, qdtype, name)
        want = lkv.decode_attn([pair.gpu], [view], q, sm_scale(D), tau)
        out = torch.full_like(want, float("nan"))
        got = lkv.decode_attn_noalloc([pair.gpu], [view], q, sm_scale(D), tau, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, want), f"{name}: max |d| {float((got - want).abs().max())}"


def test_noalloc_rejects_partials_beyond_its_scratch():
    """A call whose partials exceed the static scratch returns LKV_ESCRATCH
    and launches nothing; the workspace entry point still takes it."""
    pair, view, q = _case([128], 1, 4, 92)
    # 65536 sequences x 4 heads x 1 split x 130 floats = 136 MB of partials
    bt = view.block_table.expand(65536, -1).contiguous()
    lens = view.seq_lens.expand(65536).contiguous()
    big_view = lkv.View(bt, lens, 128)
    qq = q.expand(65536, -1, -1).contiguous()
    assert lkv.decode_workspace_bytes([pair.gpu], [big_view], 65536, 4, 128) > lkv.NOALLOC_SCRATCH_BYTES
    say("noalloc oversized call")
    with pytest.raises(lkv.LkvError) as e:
        lkv.decode_attn_noalloc([pair.gpu], [big_view], qq, sm_scale(128), 0.0, 128)
    assert e.value.status == lkv.ESCRATCH
