// Device-side helpers shared by the CRISP HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "crisp_kernels.h"

namespace crisp {

constexpr int kWave = 64;    // CDNA wavefront

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// log2(e): softmax is evaluated as exp2(x * log2e - m)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// D = A(32x16) * B(16x32) + C on the bf16 matrix cores.  Operand layout
// (checked on gfx950): lane l holds A[l%32][8*(l/32) .. +7] and
// B[8*(l/32) .. +7][l%32]; C/D register r of lane l is element
// (8*(r/4) + 4*(l/32) + r%4, l%32).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value held by lane l ^ 32 (the other half of the wavefront).
__device__ __forceinline__ float swap_half(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float wave_max(float x)
{
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ double wave_sum(double x)
{
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ int wave_sum(int x)
{
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

}  // namespace crisp
