// quant_device.h -- device-side group quantiser and bitstream packing.
//
// Group-wise asymmetric integer quantisation with an fp32 scale and an integer
// zero point (TurboQuant page, core innovation; K at 6 bits and V at 4 bits,
// Super KV Compression page, first layer).  Files that include this header
// are compiled with -ffp-contract=off: the scale, zero point and codes are
// computed in IEEE fp32 with correctly rounded division and round-half-even
// rint, in a fixed order, so they are reproducible bit for bit.
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
