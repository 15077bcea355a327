// quant_device.h -- device-side group quantiser and bitstream packing.
//
// Group-wise asymmetric integer quantisation with an fp32 scale and an integer
// zero point (TurboQuant page, core innovation; K at 6 bits and V at 4 bits,
// Super KV Compression page, first layer).  Files that include this header
// are compiled with -ffp-contract=off, and the quantiser functions also turn
// contraction off themselves (for the decode kernel that appends a row): the
// scale, zero point and codes are computed in IEEE fp32 with correctly
// rounded division and round-half-even rint, in a fixed order, so they are
// reproducible bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lkv {

// min / max over aligned segments of `seg` lanes (seg 16, 32 or 64), with
// lane exchanges that stay in the vector ALU: quad permutations (lane ^ 1,
// lane ^ 2), mirrors within 8 and 16 lanes (after the smaller steps every
// lane of the half holds its half's extreme), then swaps of 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <bool MAX>
__device__ __forceinline__ float seg_extreme(float x, int seg)
{
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
    x = op(x, dpp_mov<0xB1>(x));   // quad_perm [1,0,3,2]
    x = op(x, dpp_mov<0x4E>(x));   // quad_perm [2,3,0,1]
    x = op(x, dpp_mov<0x141>(x));  // row_half_mirror
    x = op(x, dpp_mov<0x140>(x));  // row_mirror
    if (seg >= 32) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
    }
    if (seg >= 64) {
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
    }
    return x;
}
__device__ __forceinline__ float seg_min(float x, int seg) { return seg_extreme<false>(x, seg); }
__device__ __forceinline__ float seg_max(float x, int seg) { return seg_extreme<true>(x, seg); }

// Quantise the value x held by this lane; the group is the aligned segment of
// g lanes that holds it.  Returns the code; *s, *z receive the group's scale
// and zero point (the same in every lane of the segment).
//   constant group c:  (s, z, q) = (c, 0, 1) | (-c, 1, 0) | (0, 0, 0)
//   otherwise:         lo = min(mn, 0), hi = max(mx, 0), s = (hi - lo) / qmax,
//                      z = clamp(rint(-lo / s)), q = clamp(rint(x / s) + z)
// The sign of a zero minimum or maximum never changes the result.
__device__ __forceinline__ int quantize_lane(float x, int g, int bits, float* s_out, int* z_out)
{
#pragma clang fp contract(off)
    const int qmax = (1 << bits) - 1;
    const float mn = seg_min(x, g);
    const float mx = seg_max(x, g);
    if (mn == mx) {
        if (mn > 0.0f) { *s_out = mn; *z_out = 0; return 1; }
        if (mn < 0.0f) { *s_out = -mn; *z_out = 1; return 0; }
        *s_out = 0.0f; *z_out = 0; return 0;
    }
    const float lo = mn < 0.0f ? mn : 0.0f;
    const float hi = mx > 0.0f ? mx : 0.0f;
    const float r = hi - lo;
    const float s = r / (float)qmax;
    const float neg_lo = -lo;
    int z = (int)rintf(neg_lo / s);
    z = z < 0 ? 0 : (z > qmax ? qmax : z);
    int q = (int)rintf(x / s) + z;
    q = q < 0 ? 0 : (q > qmax ? qmax : q);
    *s_out = s;
    *z_out = z;
    return q;
}

// ---- faster quantiser for rows held P consecutive channels per lane ----
//
// The same codes, scale and zero point as quantize_lane (finite inputs), with
// fewer operations:
//  - min / max by compares (no NaN handling) over the lane's P values, then
//    over the g / P lanes of the group;
//  - s = RN(r / qmax) as r * RN(1 / qmax) plus one fma correction, which is
//    the correctly rounded quotient for every finite r >= 0 when qmax is 15
//    or 63 (tests/native/quant_exact.c checks every finite fp32 r);
//  - rint(RN(x / s)) from an approximate reciprocal and one fma correction,
//    which gives the quotient to within an ulp: rint can differ only when
//    that quotient lies within a few ulps of a half-integer.  Such lanes
//    (and any scale that is not a finite normal number) are flagged and
//    recomputed with correctly rounded division (quantize_exact); the same
//    file checks the flagged bound on random and near-tie quotients with
//    reciprocals up to two ulps off.

// Order-preserving integer key of a finite float (the map is its own
// inverse): min / max of keys are single integer instructions, with no NaN
// handling.  -0 orders below +0; the quantiser treats both alike.
__device__ __forceinline__ int fkey(float x)
{
    const int i = __float_as_int(x);
    return i ^ ((i >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float fkey_value(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

template <bool MAX>
__device__ __forceinline__ int pick(int a, int b) { return MAX ? max(a, b) : min(a, b); }

// Extreme of keys over aligned segments of LANES lanes (8, 16, 32 or 64).
template <bool MAX, int LANES>
__device__ __forceinline__ int lanes_extreme(int k)
{
    static_assert(LANES == 8 || LANES == 16 || LANES == 32 || LANES == 64, "segment of 8 to 64 lanes");
    k = pick<MAX>(k, __builtin_amdgcn_update_dpp(0, k, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    k = pick<MAX>(k, __builtin_amdgcn_update_dpp(0, k, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    k = pick<MAX>(k, __builtin_amdgcn_update_dpp(0, k, 0x141, 0xF, 0xF, true));  // row_half_mirror
    if constexpr (LANES >= 16) k = pick<MAX>(k, __builtin_amdgcn_update_dpp(0, k, 0x140, 0xF, 0xF, true));  // row_mirror
    if constexpr (LANES >= 32) {
        const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)k, (uint32_t)k, false, false);
        k = pick<MAX>((int)a[0], (int)a[1]);
    }
    if constexpr (LANES >= 64) {
        const auto a = __builtin_amdgcn_permlane32_swap((uint32_t)k, (uint32_t)k, false, false);
        k = pick<MAX>((int)a[0], (int)a[1]);
    }
    return k;
}

// rint(RN(x / s)) for a finite normal s > 0 and |x / s| < 128, from rc
// within two ulps of 1 / s; sets `slow` when the result is not certain.
__device__ __forceinline__ float rint_quot(float x, float s, float rc, bool& slow)
{
#pragma clang fp contract(off)
    const float q0 = x * rc;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, x), rc, q0);
    const float r = rintf(q1);
    slow = slow || !(__builtin_fabsf(q1 - r) <= 0.5f - 0x1p-16f);
    return r;
}

// Group state of one row: the group's min / max and the lane's codes.
template <int P>
struct QRow {
    float mn, mx, s;
    int z;
    int q[P];
    bool slow;
};

// Quantise the lane's P values x (channels P * lane + p); the group of GS
// channels is the aligned segment of GS / P lanes.  bits is 4 or 6.  No
// branch: the rows a wave quantises together interleave.
template <int P, int GS>
__device__ __forceinline__ void quantize_fast(const float (&x)[P], int bits, QRow<P>& o)
{
#pragma clang fp contract(off)
    const int qmax = (1 << bits) - 1;
    const float fq = (float)qmax;
    const float C = bits == 6 ? 0x1.041042p-6f : 0x1.111112p-4f;  // RN(1/63), RN(1/15)
    int kn = fkey(x[0]), kx = kn;
#pragma unroll
    for (int p = 1; p < P; p++) {
        kn = pick<false>(kn, fkey(x[p]));
        kx = pick<true>(kx, fkey(x[p]));
    }
    const float mn = fkey_value(lanes_extreme<false, GS / P>(kn));
    const float mx = fkey_value(lanes_extreme<true, GS / P>(kx));
    const float lo = mn < 0.0f ? mn : 0.0f;
    const float hi = mx > 0.0f ? mx : 0.0f;
    const float r = hi - lo;
    const float s0 = r * C;
    const float s = __builtin_fmaf(__builtin_fmaf(-s0, fq, r), C, s0);
    const float rc = __builtin_amdgcn_rcpf(s);
    bool slow = !(s >= 0x1p-126f && s <= 0x1.fffffep127f);
    const float zf = rint_quot(-lo, s, rc, slow);
    int z = (int)zf;
    z = z < 0 ? 0 : (z > qmax ? qmax : z);
#pragma unroll
    for (int p = 0; p < P; p++) {
        int q = (int)rint_quot(x[p], s, rc, slow) + z;
        o.q[p] = q < 0 ? 0 : (q > qmax ? qmax : q);
    }
    o.mn = mn;
    o.mx = mx;
    o.s = s;
    o.z = z;
    o.slow = slow;
    if (mn == mx) {  // a constant group c: (c, 0, 1) | (-c, 1, 0) | (0, 0, 0)
        o.slow = false;
        o.s = mn > 0.0f ? mn : (mn < 0.0f ? -mn : 0.0f);
        o.z = mn < 0.0f ? 1 : 0;
#pragma unroll
        for (int p = 0; p < P; p++) o.q[p] = mn > 0.0f ? 1 : 0;
    }
}

// The same with correctly rounded division throughout, for flagged lanes.
template <int P>
__device__ __forceinline__ void quantize_exact(const float (&x)[P], int bits, QRow<P>& o)
{
#pragma clang fp contract(off)
    const int qmax = (1 << bits) - 1;
    const float lo = o.mn < 0.0f ? o.mn : 0.0f;
    const float hi = o.mx > 0.0f ? o.mx : 0.0f;
    const float s = (hi - lo) / (float)qmax;
    int z = (int)rintf(-lo / s);
    z = z < 0 ? 0 : (z > qmax ? qmax : z);
#pragma unroll
    for (int p = 0; p < P; p++) {
        int q = (int)rintf(x[p] / s) + z;
        o.q[p] = q < 0 ? 0 : (q > qmax ? qmax : q);
    }
    o.s = s;
    o.z = z;
    o.slow = false;
}

// NV values of NB bits (low bits of v, higher bits ignored) as NW words,
// LSB first.
template <int NB, int NV, int NW>
__device__ __forceinline__ void pack_values(const uint32_t (&v)[NV], uint32_t (&w)[NW])
{
    static_assert(NB * NV == 32 * NW, "whole words");
    uint64_t acc = 0;
    int nacc = 0, o = 0;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        acc |= (uint64_t)(v[i] & ((1u << NB) - 1u)) << nacc;
        nacc += NB;
        if (nacc >= 32) {
            w[o++] = (uint32_t)acc;
            acc >>= 32;
            nacc -= 32;
        }
    }
}

// Word w of a bitstream of `bits`-bit fields, field i read by get(i) for
// i in [0, n); fields outside [lo, hi) count as zero.
template <typename Get>
__device__ __forceinline__ uint32_t pack_word(int w, int bits, int lo, int hi, Get get)
{
    const int first = (32 * w) / bits;
    const int last = (32 * w + 31) / bits;
    uint32_t word = 0;
    for (int i = first; i <= last; i++) {
        if (i < lo || i >= hi) continue;
        const uint32_t v = get(i);
        const int sh = bits * i - 32 * w;
        word |= sh >= 0 ? (uint32_t)((uint64_t)v << sh) : (v >> (-sh));
    }
    return word;
}

// Mask of the bits of word w that belong to fields [lo, hi).
__device__ __forceinline__ uint32_t field_mask(int w, int bits, int lo, int hi)
{
    const int64_t a = (int64_t)bits * lo - 32 * w;
    const int64_t b = (int64_t)bits * hi - 32 * w;
    const int64_t a0 = a < 0 ? 0 : (a > 32 ? 32 : a);
    const int64_t b0 = b < 0 ? 0 : (b > 32 ? 32 : b);
    if (b0 <= a0) return 0u;
    const uint64_t m = ((1ull << (b0 - a0)) - 1ull) << a0;
    return (uint32_t)m;
}

// Channel-major staging of V codes: one byte per (channel, slot), rows 68
// bytes apart, so that a wave storing one slot of 64 consecutive channels
// hits distinct banks.
constexpr int VPITCH = 68;

// V words of channel rows: group m of NV slots -> NW words; only the words
// holding bits of slots [s0, s1) are written, shared words merged with
// atomics.
template <int NB, int NV, int NW, int D>
__device__ __forceinline__ void pack_v_rows(const uint8_t (*vt)[VPITCH], uint8_t* ch, int off_vc, int vrow, int s0,
                                            int s1)
{
    const int m0 = s0 / NV, m1 = (s1 - 1) / NV;
    const int ng = m1 - m0 + 1;
    for (int idx = threadIdx.x; idx < D * ng; idx += blockDim.x) {
        const int d = idx / ng, m = m0 + idx % ng;
        uint32_t v[NV], w[NW];
        const uint32_t* src = (const uint32_t*)(vt[d] + m * NV);
#pragma unroll
        for (int i = 0; i < NV / 4; i++) {
            const uint32_t t = src[i];
            v[4 * i] = t & 0xFFu;
            v[4 * i + 1] = (t >> 8) & 0xFFu;
            v[4 * i + 2] = (t >> 16) & 0xFFu;
            v[4 * i + 3] = t >> 24;
        }
        pack_values<NB, NV, NW>(v, w);
        uint32_t* row = (uint32_t*)(ch + off_vc + d * vrow) + m * NW;
#pragma unroll
        for (int i = 0; i < NW; i++) {
            const uint32_t mask = field_mask(m * NW + i, NB, s0, s1);
            if (mask == 0xFFFFFFFFu) {
                row[i] = w[i];
            } else if (mask != 0u) {
                atomicAnd(row + i, ~mask);
                atomicOr(row + i, w[i] & mask);
            }
        }
    }
}

// Field i of a bitstream held in global or shared memory (32-bit words).
__device__ __forceinline__ uint32_t get_field(const uint32_t* words, int i, int bits)
{
    const int bit = i * bits;
    const int w = bit >> 5, sh = bit & 31;
    uint64_t x = words[w];
    if (sh + bits > 32) x |= (uint64_t)words[w + 1] << 32;
    return (uint32_t)(x >> sh) & ((1u << bits) - 1u);
}

__device__ __forceinline__ float load_as_float(const void* p, int64_t i, int dtype)
{
    if (dtype == LKV_F32) return ((const float*)p)[i];
    const uint16_t u = ((const uint16_t*)p)[i];
    if (dtype == LKV_BF16) return __uint_as_float((uint32_t)u << 16);
    return __half2float(__ushort_as_half(u));
}

__device__ __forceinline__ uint32_t f16_bits(float x)
{
    return (uint32_t)__half_as_ushort(__float2half_rn(x));
}

}  // namespace lkv
