"""Pins of the oracle's quantiser, packing, layout and fp16 conversion.

Each test checks the oracle against something other than itself: a closed
form, a printed figure of the pages, a hand-computed example, a numpy
library routine or an exhaustive search.  CPU only.
"""
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from tests import np_reference as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _groups(rng, kind, n_groups, g):
    if kind == "normal":
        return rng.standard_normal((n_groups, g)).astype(np.float32)
    if kind == "uniform_pos":
        return rng.uniform(0.5, 3.0, (n_groups, g)).astype(np.float32)
    if kind == "uniform_neg":
        return -rng.uniform(0.5, 3.0, (n_groups, g)).astype(np.float32)
    if kind == "outlier12":
        x = rng.standard_normal((n_groups, g)).astype(np.float32)
        x[:, :4] *= 12.0
        return x
    if kind == "tiny_range":
        return (1.0 + 1e-6 * rng.standard_normal((n_groups, g))).astype(np.float32)
    if kind == "bf16_normal":
        x = rng.standard_normal((n_groups, g)).astype(np.float32)
        u = x.view(np.uint32)
        u = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)  # RNE to bf16
        return u.view(np.float32)
    raise ValueError(kind)


KINDS = ["normal", "uniform_pos", "uniform_neg", "outlier12", "tiny_range", "bf16_normal"]


@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("kind", KINDS)
def test_roundtrip_error_bound_and_nearest_code(bits, g, kind):
    """|x - (q - z) s| <= s (1/2 + 2^-14) and q is the nearest of the 2^b
    grid points (the scale/2 bound of asymmetric quantisation)."""
    rng = np.random.default_rng(1000 * bits + 7 * g + KINDS.index(kind))
    X = _groups(rng, kind, 400, g)
    qmax = (1 << bits) - 1
    for x in X:
        s, z, q = O.quantize_group(x, bits)
        assert 0 <= z <= qmax and q.max() <= qmax
        assert s > 0
        xd = x.astype(np.float64)
        xh = (q.astype(np.float64) - z) * s
        assert np.all(np.abs(xd - xh) <= s * (0.5 + 2.0 ** -14)), (kind, bits, g)
        grid = (np.arange(qmax + 1, dtype=np.float64) - z) * s
        best = np.abs(xd[:, None] - grid[None, :]).min(axis=1)
        assert np.all(np.abs(xd - xh) <= best + 1e-5 * s)


@pytest.mark.parametrize("c", [0.0, -0.0, 1e-30, -1e-30, 1.0, -1.0, math.pi, -math.pi, 1e30, -1e30,
                               3.3895313892515355e38, -3.3895313892515355e38])
@pytest.mark.parametrize("bits", [4, 6])
def test_constant_groups_reconstruct_exactly(c, bits):
    """A constant group reconstructs to its value at every magnitude."""
    x = np.full(64, c, np.float32)
    s, z, q = O.quantize_group(x, bits)
    xh = (np.float64(q[0]) - z) * s
    assert np.all(q == q[0])
    assert xh == np.float64(np.float32(c))
    assert np.float32((np.float32(q[0]) - np.float32(z)) * np.float32(s)) == np.float32(c)


def test_worked_example_6bit():
    """Hand-computed codes of tests/golden/quant_worked_example.txt."""
    rows, meta = [], {}
    for line in open(os.path.join(GOLDEN, "quant_worked_example.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] in ("bits", "scale", "zero"):
            meta[line[0]] = float(line[1])
        else:
            rows.append((float(line[0]), int(line[3])))
    x = np.array([r[0] for r in rows], np.float32)
    s, z, q = O.quantize_group(x, int(meta["bits"]))
    assert s == meta["scale"] and z == meta["zero"]
    assert list(q) == [r[1] for r in rows]


@pytest.mark.parametrize("bits", [4, 6])
def test_zero_maps_to_zero_point(bits):
    rng = np.random.default_rng(7)
    for _ in range(200):
        x = rng.standard_normal(64).astype(np.float32)
        x[rng.integers(64)] = 0.0
        s, z, q = O.quantize_group(x, bits)
        assert np.all(q[x == 0.0] == z)


def test_pack_words_hand_computed():
    """Bitstream words match the hand-computed words of
    tests/golden/pack_words.txt (LSB-first fields)."""
    for line in open(os.path.join(GOLDEN, "pack_words.txt")):
        f = line.split("#")[0].split()
        if not f:
            continue
        bits, w, val = int(f[1]), int(f[3]), int(f[4], 16)
        codes = [d % (1 << bits) for d in range(64)]
        buf = O.put_fields(codes, bits, 64 * bits // 8)
        word = int.from_bytes(bytes(buf[4 * w:4 * w + 4]), "little")
        assert word == val, (bits, w, hex(word), hex(val))


@pytest.mark.parametrize("bits", [4, 6, 16])
def test_pack_unpack_bijection_against_bigint(bits):
    """The oracle's bit loop equals a big-integer construction of the stream,
    and numpy unpacking inverts it."""
    rng = np.random.default_rng(bits)
    n = 128
    codes = rng.integers(0, 1 << bits, n)
    buf = O.put_fields(codes, bits, n * bits // 8)
    stream = 0
    for i, c in enumerate(codes):
        stream |= int(c) << (bits * i)
    assert bytes(buf) == stream.to_bytes(n * bits // 8, "little")
    assert np.array_equal(R.unpack(buf, n, bits), codes.astype(np.uint32))
    assert np.array_equal(O.get_fields(buf, n, bits), codes.astype(np.uint32))


def test_straddling_6bit_codes():
    """6-bit codes 5 and 10 cross a 32-bit word boundary."""
    codes = [0] * 16
    codes[5], codes[10] = 0b111111, 0b101101
    buf = O.put_fields(codes, 6, 12)
    words = [int.from_bytes(bytes(buf[4 * i:4 * i + 4]), "little") for i in range(3)]
    assert (words[0] >> 30) & 3 == 0b11 and words[1] & 0xF == 0b1111
    assert (words[1] >> 28) & 0xF == 0b1101 and words[2] & 0x3 == 0b10


def test_chunk_layout_closed_form_and_page_ratio():
    """Chunk bytes equal the closed form; K6V4 codes give the page's 3.2x."""
    figs = {}
    for line in open(os.path.join(GOLDEN, "page_figures.txt")):
        f = line.split("#")[0].split()
        if f:
            figs[f[0]] = float(f[1])
    expect = {(128, 64, 6, 4): 11520, (64, 32, 6, 4): 6400, (128, 64, 6, 6): 13568, (128, 64, 16, 16): 32768}
    for (D, g, kb, vb), nbytes in expect.items():
        off = O.chunk_layout(D, g, kb, vb)
        assert off[6] == nbytes
        assert off == R.layout(D, g, kb, vb)
    # per token per KV head: 180, 100, 212, 512 bytes
    assert [O.chunk_layout(*f)[6] // 64 for f in expect] == [180, 100, 212, 512]
    # codes only, against 16-bit K and V: 512 / 160 = 3.2 (the page's figure)
    off = O.chunk_layout(128, 64, 6, 4)
    codes_per_token = (off[2] - off[0]) / 64
    assert (2 * 128 * 2) / codes_per_token == figs["k6v4_compression"]
    # with fp32 scales and uint8 zeros per 64-channel group
    assert round(512 / 180, 3) == 2.844
    # TurboQuant 6-bit 2.56x = 16 / 6.25 bits: 0.25 bit of metadata per element
    assert 16 / (6 + 0.25) == figs["turboquant_6bit_compression"]
    with pytest.raises(ValueError):
        O.chunk_layout(128, 48, 6, 4)
    with pytest.raises(ValueError):
        O.chunk_layout(128, 64, 5, 4)


def test_fp16_round_to_nearest_even_matches_numpy():
    """Software fp32 -> fp16 equals numpy's IEEE conversion (round to
    nearest even, subnormals kept, overflow to infinity)."""
    rng = np.random.default_rng(3)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-5).astype(np.float32),      # fp16 subnormal range
        (rng.standard_normal(2000) * 7e4).astype(np.float32),       # near overflow
        np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001,
                  3 * 2.0 ** -26, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, np.inf, -np.inf], np.float32),
        rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    vals = vals[np.isfinite(vals) | np.isinf(vals)]
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = np.array([O.f32_to_f16_bits(float(v)) for v in vals], np.uint16)
    nan = np.isnan(vals)
    assert np.array_equal(got[~nan], want[~nan])
    back = np.array([O.f16_bits_to_f64(int(h)) for h in got[~nan][:3000]])
    assert np.array_equal(back, want[~nan][:3000].view(np.float16).astype(np.float64))


def test_default_thresholds_closed_form():
    """tau_low = eps4 / N, tau_high = (eps4 / eps6) / N, eps_b = 1/(2(2^b-1))."""
    lo, hi = O.default_thresholds(32768)
    assert lo == np.float32((1 / 30) / 32768)
    assert hi == np.float32(4.2 / 32768)
    assert math.isclose(lo, 1.0172526e-6, rel_tol=1e-7) and math.isclose(hi, 1.2817383e-4, rel_tol=1e-7)


def test_memory_claims_of_the_pages():
    """KV footprints quoted on the pages, in closed form.  Layer counts are
    not on the pages: 32 layers x 8 KV heads for the 8B model, 80 layers x 8
    KV heads for the 70B model (both GQA, head_dim 128)."""
    figs = {}
    for line in open(os.path.join(GOLDEN, "page_figures.txt")):
        f = line.split("#")[0].split()
        if f:
            figs[f[0]] = float(f[1])
    gib = 2 * 32 * 8 * 128 * 2 * 32768 / 2 ** 30
    assert gib == 4.0
    assert figs["llama8b_32k_kv_gib_min"] <= gib <= figs["llama8b_32k_kv_gib_max"]
    gqa = 2 * 80 * 8 * 128 * 2 * 32768 / 1e9      # 10.7 GB per sequence
    mha = 2 * 80 * 64 * 128 * 2 * 32768 / 1e9     # 85.9 GB per sequence
    assert gqa < figs["llama70b_32k_kv_gb_min"] < mha
    assert 8 * gqa > figs["llama70b_32k_kv_gb_min"]   # or a batch of 8 with GQA
    # the K6V4 cache at 180 B per token per KV head: 8B model at 32K
    assert 32 * 8 * 32768 * 180 / 2 ** 30 == 1.40625
