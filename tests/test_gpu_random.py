"""Seeded random cases against the oracle.

Decode and multi-token queries: every format, G, one or two segments,
ragged lengths drawn half from block and split edges, split sizes, skip
thresholds and query dtypes; attention within max|d| <= 1e-3 max|v_hat|
and rel L2 <= 1e-4.  Appends (a prefill, then more rows into partly filled
blocks) and tier updates followed by two re-tierings: bit-exact pools,
tiers and counts.  Accumulated scores (per token within 1e-4 relative) and
the direction-preserving K codec (bit-exact codes, factors within one ulp,
attention within the bounds above).  With a skip threshold the skip
decisions are compared bit for bit outside the band of decisions fp32 can
take either way.  The cases are fixed by the seeds."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_kv_cache_token_amd import inputs, lkv
from tests import np_reference as R
from tests import test_gpu_knorm as TK
from tests import test_gpu_retier as TR
from tests import test_gpu_scores as TS
from tests.gpu_common import Pair, assert_attention_close, resolved_reference, say, sm_scale, to_f32_host
from tests.oracle_cases import block_tables
from tests.test_gpu_multi import _multi_case
from tests.test_gpu_parity import FORMATS, _decode_case, _prefill

pytestmark = pytest.mark.gpu

EDGE = [1, 2, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257, 511, 1023, 1024, 1025]
N_CASES = 300
# Skip thresholds: tau_low = eps4 / N is 2e-4 at N = 167 tokens and 5e-3 at
# N = 7.  With tau > 0 the GPU's skip decisions are read back through the
# debug entry point: outside the band of decisions that fp32 can take either
# way they must equal the exact ones bit for bit, and inside it the oracle
# takes the GPU's (tests/gpu_common.py, resolved_reference).
TAUS = [0.0, 0.0, 1e-5, 1e-4, 2e-4, 1e-3, 5e-3]


def _case(rng):
    fmt = FORMATS[rng.integers(len(FORMATS))]
    D = fmt[0]
    G = int(rng.choice([1, 2, 4, 8, 16] if D == 64 else [1, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2]))
    B = int(rng.integers(1, 5))
    lens = [int(rng.choice(EDGE)) if rng.random() < 0.5 else int(rng.integers(1, 2500)) for _ in range(B)]
    split = int(rng.choice([64, 128, 192, 256, 512, 1024]))
    tau = float(rng.choice(TAUS))
    qd = str(rng.choice(["bf16", "bf16", "f32"]))
    seed = int(rng.integers(1, 10**6))
    T = int(rng.integers(2, 10)) if rng.random() < 0.35 else 1
    nseg = 2 if (T == 1 and rng.random() < 0.25 and fmt[2] != 16) else 1
    return fmt, G, Hkv, lens, split, tau, qd, seed, T, nseg


def test_seeded_random_cases():
    rng = np.random.default_rng(2026)
    for i in range(N_CASES):
        fmt, G, Hkv, lens, split, tau, qd, seed, T, nseg = _case(rng)
        what = f"case {i}: {fmt} G{G} Hkv{Hkv} lens {lens} split {split} tau {tau} {qd} seed {seed} T{T} nseg {nseg}"
        if T > 1:
            lens = [max(n, T) for n in lens]
            got, want, vmax, _ = _multi_case(fmt, G, qd, lens, T, tau, split, seed=seed, Hkv=Hkv)
            got, want = got.reshape(-1, *got.shape[2:]), want.reshape(-1, *want.shape[2:])
        else:
            got, want, vmax = _decode_case(fmt, G, qd, lens, tau, split, seed=seed, Hkv=Hkv, nseg=nseg)
        assert_attention_close(got, want, vmax, what)


N_BITEXACT = 120
APPEND_EDGE = [1, 2, 63, 64, 65, 127, 128, 129]
TIER_EDGE = APPEND_EDGE + [2047, 2048, 2049]


def test_seeded_random_appends_and_tiers_bit_exact():
    rng = np.random.default_rng(11)
    for i in range(N_BITEXACT):
        if rng.random() < 0.5:
            fmt = FORMATS[rng.integers(len(FORMATS))]
            D, g, kb, vb = fmt
            dtype = str(rng.choice(["f32", "bf16", "f16"]))
            Hkv = int(rng.choice([1, 2, 3]))
            B = int(rng.integers(1, 5))
            lens = [int(rng.choice(APPEND_EDGE)) if rng.random() < 0.5 else int(rng.integers(0, 700))
                    for _ in range(B)]
            extra = [int(rng.integers(0, 70)) for _ in range(B)]
            bt, nblk = block_tables([n + e + 1 for n, e in zip(lens, extra)], rng)
            pair = Pair(D, g, kb, vb, Hkv, nblk)
            seed = int(rng.integers(1, 10**6))
            say("case", i, "append", fmt, dtype, "Hkv", Hkv, "lens", lens, "extra", extra, "seed", seed)
            _prefill(pair, lens, Hkv, D, dtype, seed, bt, outliers=bool(rng.random() < 0.5))
            assert pair.pool_equal(), pair.first_pool_mismatch()
            K, V = [], []
            for b, e in enumerate(extra):
                k, v = inputs.kv_rows(seed + 1, b, e, Hkv, D, dtype=dtype)
                K.append(k)
                V.append(v)
            cu = np.concatenate([[0], np.cumsum(extra)]).astype(np.int32)
            pair.append(torch.cat(K), torch.cat(V), cu, np.array(lens, np.int32), bt)
            assert pair.pool_equal(), pair.first_pool_mismatch()
        else:
            Hkv = int(rng.choice([1, 2]))
            B = int(rng.integers(1, 4))
            lens = [int(rng.choice(TIER_EDGE)) if rng.random() < 0.4 else int(rng.integers(1, 3000))
                    for _ in range(B)]
            seed = int(rng.integers(1, 10**6))
            say("case", i, "tier", "Hkv", Hkv, "lens", lens, "seed", seed)
            h, hbt, nh, m, mbt, nm, tl, th = TR._tiered(lens, Hkv, seed, rng)
            for it in range(2):
                frac = (float(rng.uniform(0, 0.5)), float(rng.uniform(0, 0.5)))
                r = TR._retier_both(h, hbt, nh, m, mbt, nm, tl, th, seed + 7 * it + 1, rng, frac=frac,
                                    boundaries=bool(rng.random() < 0.5))
                TR._check_bit_exact(r)
                h, hbt, nh, m, mbt, nm = r["dh"], r["dhb"], r["ref"][2], r["dm"], r["dmb"], r["ref"][3]


N_SCORES_KNORM = 120


def test_seeded_random_scores_and_knorm():
    rng = np.random.default_rng(6)
    for i in range(N_SCORES_KNORM):
        fmt = FORMATS[rng.integers(len(FORMATS))]
        D, g, kb, vb = fmt
        G = int(rng.choice([1, 2, 4, 8, 16] if D == 64 else [1, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2]))
        B = int(rng.integers(1, 5))
        lens = [int(rng.choice(EDGE)) if rng.random() < 0.5 else int(rng.integers(0, 2000)) for _ in range(B)]
        split = int(rng.choice([64, 128, 256, 512, 1024]))
        tau = float(rng.choice(TAUS))
        qd = str(rng.choice(["bf16", "f32"]))
        seed = int(rng.integers(1, 10**6))
        what = f"case {i}: {fmt} G{G} Hkv{Hkv} lens {lens} split {split} tau {tau} {qd} seed {seed}"
        if kb != 16 and rng.random() < 0.5:
            dtype = str(rng.choice(["bf16", "f32"]))
            lens = [max(n, 1) for n in lens]
            say(what, "k_norm", dtype)
            bt, nblk = block_tables(lens, rng)
            pair = TK.NormPair(D, g, kb, vb, Hkv, nblk)
            TK._append(pair, lens, Hkv, D, seed, bt, dtype)
            pair.compare()
            q = inputs.queries(seed + 2, B, Hkv * G, D, dtype=qd)
            view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
            got_t = lkv.decode_attn([pair.gpu], [view], q.cuda(), sm_scale(D), tau, split)
            got = got_t.cpu().numpy()
            if tau > 0:
                dbg, mask = lkv.decode_attn_debug([pair.gpu], [view], q.cuda(), sm_scale(D), tau, split)
                torch.cuda.synchronize()
                assert torch.equal(dbg, got_t), what
                want, stats = resolved_reference([pair.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q),
                                                 sm_scale(D), tau, split, mask, [view.max_len], what)
                say("  skip pairs live / flipped near the bound / largest flipped margin:", *stats)
            else:
                want = O.decode([pair.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm_scale(D), tau,
                                split)
            vmax = max(float(np.abs(R.dequant_sequence(pair.ref.pool, pair.ref.chunk_bytes, Hkv, D, g, kb, vb,
                                                       bt[b], n)[1]).max()) for b, n in enumerate(lens))
            assert_attention_close(got, want, vmax, what)
        else:
            say(what, "scores")
            bt, nblk = block_tables([max(n, 1) for n in lens], rng)
            pair = Pair(D, g, kb, vb, Hkv, nblk)
            TS._prefill(pair, lens, Hkv, D, seed, bt)
            q = inputs.queries(seed + 1, B, Hkv * G, D, dtype=qd)
            view = lkv.View(torch.tensor(bt).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
            stride = max(lens) + int(rng.integers(0, 70))
            acc0 = rng.uniform(0, 1, (1, B, max(stride, 1))).astype(np.float32)
            for b, n in enumerate(lens):
                acc0[0, b, :n] = 0.0  # live positions start empty; the bytes past the end must stay
            acc = torch.tensor(acc0, device="cuda")
            out = lkv.decode_attn_scores([pair.gpu], [view], q.cuda(), acc, sm_scale(D), tau, split)
            ref_out = lkv.decode_attn([pair.gpu], [view], q.cuda(), sm_scale(D), tau, split)
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out), what
            want = acc0.astype(np.float64)
            O.decode([pair.ref], [bt], [np.array(lens, np.int32)], to_f32_host(q), sm_scale(D), tau, split,
                     score_acc=want)
            got = acc.cpu().numpy().astype(np.float64)
            for b, n in enumerate(lens):
                assert np.all(got[0, b, n:] == acc0[0, b, n:]), what
            TS.assert_scores_close(got - acc0, want - acc0, what)
