// merge128.h -- the merge of up to CH (at most 64) split partials (o, m, L) of
// one (sequence, query head) at head_dim 128, in one wave (the split step of
// the pages' decode: per-split running maximum and sum, then one rescaled
// sum).  Lane l holds channels 2l and 2l + 1 of every split's o row and
// split l's (m, L); splits past the count hold m = -inf.  The merge kernel
// and the split kernel that merges its own splits (a workgroup's splits
// first, then the workgroups' partials) use these functions, built without
// fp contraction.
#pragma once

#include <hip/hip_runtime.h>

namespace lkv {

__device__ __forceinline__ float merge_wave_max(float x)
{
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ float merge_wave_sum(float x)
{
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// M = max_i m_i, L = sum_i L_i 2^(m_i - M), o = sum_i o_i 2^(m_i - M) / L
// (splits in order; base 2).  Returns the lane's two output channels; M and
// 1 / L (0 when no split has a token) go to *M_out and *inv_out.
template <int CH>
__device__ __forceinline__ float2 merge128(const float2 (&ov)[CH], float mi, float li, float* M_out, float* inv_out)
{
#pragma clang fp contract(off)
    const float M = merge_wave_max(mi);
    float2 acc = {0.0f, 0.0f};
    float L = 0.0f;
    if (M != -INFINITY) {
        const float wi = mi == -INFINITY ? 0.0f : exp2f(mi - M);
        L = merge_wave_sum(li * wi);
#pragma unroll
        for (int i = 0; i < CH; i++) {
            // splits past the count have weight 0 (their lanes hold mi = -inf)
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wi), i));
            acc.x += w != 0.0f ? ov[i].x * w : 0.0f;
            acc.y += w != 0.0f ? ov[i].y * w : 0.0f;
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    *M_out = M;
    *inv_out = inv;
    return float2{acc.x * inv, acc.y * inv};
}

// The same merge without the final division: the partial (o, M, L) of the
// union of the splits, o = sum_i o_i 2^(m_i - M) and L = sum_i L_i 2^(m_i -
// M), to be merged again with other such partials.  M = -inf and L = 0 when
// no split has a token.
template <int CH>
__device__ __forceinline__ float2 merge128_partial(const float2 (&ov)[CH], float mi, float li, float* M_out,
                                                   float* L_out)
{
#pragma clang fp contract(off)
    const float M = merge_wave_max(mi);
    float2 acc = {0.0f, 0.0f};
    float L = 0.0f;
    if (M != -INFINITY) {
        const float wi = mi == -INFINITY ? 0.0f : exp2f(mi - M);
        L = merge_wave_sum(li * wi);
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wi), i));
            acc.x += w != 0.0f ? ov[i].x * w : 0.0f;
            acc.y += w != 0.0f ? ov[i].y * w : 0.0f;
        }
    }
    *M_out = M;
    *L_out = L;
    return acc;
}

// Folds the partial (Mc, Lc, oc) into the running partial (Mr, Lr, ar) of
// the same rows: M = max(Mr, Mc), each side weighted by 2^(its M - M).  A
// side with M = -inf (no token) has weight 0.
__device__ __forceinline__ void fold_partial(float& Mr, float& Lr, float2& ar, float Mc, float Lc, float2 oc)
{
#pragma clang fp contract(off)
    const float M = fmaxf(Mr, Mc);
    if (M == -INFINITY) return;
    const float wr = Mr == -INFINITY ? 0.0f : exp2f(Mr - M);
    const float wc = Mc == -INFINITY ? 0.0f : exp2f(Mc - M);
    Lr = Lr * wr + Lc * wc;
    ar.x = ar.x * wr + oc.x * wc;
    ar.y = ar.y * wr + oc.y * wc;
    Mr = M;
}

}  // namespace lkv
