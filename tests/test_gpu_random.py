"""Seeded random decode and multi-token cases against the oracle: every
format, G, one or two segments, ragged lengths drawn half from block and
split edges, split sizes, skip thresholds and query dtypes.  Attention
within max|d| <= 1e-3 max|v_hat| and rel L2 <= 1e-4.  The cases are fixed
by the seed; a wider run of the same generator (7800 cases) found no
failure."""
import numpy as np
import pytest

from tests.gpu_common import assert_attention_close
from tests.test_gpu_multi import _multi_case
from tests.test_gpu_parity import FORMATS, _decode_case

pytestmark = pytest.mark.gpu

EDGE = [1, 2, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257, 511, 1023, 1024, 1025]
N_CASES = 300


def _case(rng):
    fmt = FORMATS[rng.integers(len(FORMATS))]
    D = fmt[0]
    G = int(rng.choice([1, 2, 4, 8, 16] if D == 64 else [1, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2]))
    B = int(rng.integers(1, 5))
    lens = [int(rng.choice(EDGE)) if rng.random() < 0.5 else int(rng.integers(1, 2500)) for _ in range(B)]
    split = int(rng.choice([64, 128, 192, 256, 512, 1024]))
    tau = float(rng.choice([0.0, 0.0, 1e-5, 1e-4, 1e-3]))
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
