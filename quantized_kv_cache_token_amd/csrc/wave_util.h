// wave_util.h -- matrix-core and cross-lane helpers shared by the
// matrix-core decode kernels (gfx950, wave64).
//
// MFMA 16x16x32 operand layout (bf16 and f16 alike): lane l holds
//   A[m][k] for m = l % 16, k = 8 (l / 16) + i, i = 0..7   (8 elements)
//   B[k][n] for n = l % 16, k = 8 (l / 16) + i, i = 0..7   (8 elements)
//   C[m][n] for n = l % 16, m = 4 (l / 16) + i, i = 0..3   (4 fp32 values)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// C += A B with bf16 operands (8 per lane, as 4 packed words).
__device__ __forceinline__ f32x4_t mfma_16x16x32(const uint32_t (&a)[4], const uint32_t (&b)[4], f32x4_t c)
{
    bf16x8_t av, bv;
    __builtin_memcpy(&av, a, 16);
    __builtin_memcpy(&bv, b, 16);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

// C += A B with f16 operands (8 per lane, as 4 packed words).
__device__ __forceinline__ f32x4_t mfma_16x16x32_f16(const uint32_t (&a)[4], const uint32_t (&b)[4], f32x4_t c)
{
    f16x8_t av, bv;
    __builtin_memcpy(&av, a, 16);
    __builtin_memcpy(&bv, b, 16);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
}

// Value of the neighbouring lane (lane ^ 1) -- DPP quad permutation.  Every
// lane is active where it is called; with bound_ctrl set the compiler folds
// the move into the instruction that consumes it (v_add_f32_dpp).
__device__ __forceinline__ float xor1(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// Value of lane ^ 8 within each 16-lane row -- DPP row rotation by 8.
__device__ __forceinline__ float xor8(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true));
}

// v + the value of lane ^ 32 (both halves end with the same sum).
__device__ __forceinline__ float halves_sum(float v)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows_max(float v)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace lkv
