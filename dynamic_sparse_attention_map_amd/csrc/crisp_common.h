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

// D = A(16x32) * B(32x16) + C on the bf16 matrix cores.  Operand layout
// (checked on gfx950): lane l holds A[l%16][8*(l/16) .. +7] and
// B[8*(l/16) .. +7][l%16]; C/D register r of lane l is element
// (4*(l/16) + r, l%16).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// N independent wave sums with the butterfly of wave_sum (the same additions
// in the same order, so the same bits), their shuffles interleaved so that
// their latencies overlap.
template <int N>
__device__ __forceinline__ void wave_sum_n(double (&x)[N])
{
    for (int o = 32; o > 0; o >>= 1) {
        double y[N];
        for (int j = 0; j < N; ++j) y[j] = __shfl_xor(x[j], o);
        for (int j = 0; j < N; ++j) x[j] += y[j];
    }
}

// Float wave sums for short reductions (one value per lane, a 64-term sum)
// without a round trip through the LDS crossbar for every step: lanes xor 1
// and xor 2 by DPP quad permutes, xor 4, 8 and 16 by ds_swizzle (bit mode,
// within 32 lanes), xor 32 by the lane-half swap.  Every lane ends with the
// total; N independent sums run interleaved.  (The order of additions is
// fixed, so the same inputs give the same bits in every kernel using it.)
template <int N>
__device__ __forceinline__ void wave_sum_fast_n(float (&x)[N])
{
    for (int j = 0; j < N; ++j)
        x[j] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[j]), 0xB1, 0xF, 0xF, true));
    for (int j = 0; j < N; ++j)
        x[j] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[j]), 0x4E, 0xF, 0xF, true));
    for (int j = 0; j < N; ++j)
        x[j] += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x[j]), 0x101f));
    for (int j = 0; j < N; ++j)
        x[j] += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x[j]), 0x201f));
    for (int j = 0; j < N; ++j)
        x[j] += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x[j]), 0x401f));
    for (int j = 0; j < N; ++j) x[j] += swap_half(x[j]);
}

// Inclusive prefix sums over the 64 lanes of a wavefront (every lane
// active).  Within each row of 16 lanes, DPP row shifts by 1, 2, 4 and 8
// (lanes shifted in from outside the row add 0); then the row totals are
// carried across rows by DPP row broadcasts: lane 15 of each row to the
// next row (written only into rows 1 and 3), then lane 31 to rows 2 and 3.
template <int Ctrl, int RowMask>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, Ctrl, RowMask, 0xF, false);
}

template <int Ctrl, int RowMask>
__device__ __forceinline__ unsigned long long dpp_or_zero(unsigned long long x)
{
    const uint32_t lo = dpp_or_zero<Ctrl, RowMask>((uint32_t)x);
    const uint32_t hi = dpp_or_zero<Ctrl, RowMask>((uint32_t)(x >> 32));
    return ((unsigned long long)hi << 32) | lo;
}

template <typename T>
__device__ __forceinline__ T wave_scan_incl(T x)
{
    x += dpp_or_zero<0x111, 0xF>(x);     // row_shr:1
    x += dpp_or_zero<0x112, 0xF>(x);     // row_shr:2
    x += dpp_or_zero<0x114, 0xF>(x);     // row_shr:4
    x += dpp_or_zero<0x118, 0xF>(x);     // row_shr:8
    x += dpp_or_zero<0x142, 0xA>(x);     // row_bcast:15
    x += dpp_or_zero<0x143, 0xC>(x);     // row_bcast:31
    return x;
}

// Lane 63's value, in every lane (a wave-uniform result).
__device__ __forceinline__ uint32_t last_lane(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ unsigned long long last_lane(unsigned long long x)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 63);
    return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ int wave_sum(int x)
{
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds_addr + 16 l (lds_addr wave-uniform).  Written as inline asm so
// that the compiler, which cannot tell a ring's stages apart, does not put a
// full vmcnt(0) before every LDS read; completion is awaited explicitly
// (wait_copies) before the barrier that publishes the data.  M0 is set here
// and declared clobbered; the s_nop covers the M0 -> LDS-DMA hazard.  (M0 is
// otherwise unused by the kernels that call this.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* gptr, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory", "m0");
}
// The same with a wave-uniform 64-bit base (held in scalar registers) and a
// per-lane 32-bit byte offset, which costs one vector register instead of two.
__device__ __forceinline__ void copy16_to_lds(const void* sbase, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_copies()
{
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8));
}

// LDS byte address of a shared-memory pointer
template <typename T>
__device__ __forceinline__ uint32_t lds_address(T* p)
{
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) T*)p);
}

// V^T as LDS-ready images, one per 64-key sub-tile: image i of KV head g
// (keys 64 i .. 64 i + 63, at vt + (g n_img + i) kVImage) holds row d (the
// 64 keys' values of head dimension d) as 8 chunks of 8 keys, chunk c at
// slot c ^ ((d >> 1) & 7), and inside every group of 16 keys bits 2 and 3 of
// the key index are swapped.  A lane's 8 keys of a PV operand fragment,
// {4h .. 4h+3, 8+4h .. 8+4h+3} of a group for lane half h (the order the
// S^T accumulator holds them in), are then one 16-byte chunk.  Keys past n
// are zero.  One image takes 256 threads (tid 0..255) and a 64 x kVPitch
// LDS tile: v_image_stage reads the keys, and after a barrier
// v_image_write stores the image.
constexpr int kVPitch = kD + 8;

template <class R>
__device__ __forceinline__ void v_image_stage(const R& v, int n, int g, int i,
                                              uint16_t (*tile)[kVPitch], int tid)
{
    const int key0 = 64 * i;
    const uint16_t* src = v.row(g, key0);
    for (int x = 0; x < 4; ++x) {
        const int e = tid + 256 * x;
        const int row = e >> 4, ch = e & 15;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (key0 + row < n) val = *reinterpret_cast<const u32x4*>(src + row * v.st + 8 * ch);
        *reinterpret_cast<u32x4*>(&tile[row][8 * ch]) = val;
    }
}

__device__ __forceinline__ void v_image_write(const uint16_t (*tile)[kVPitch], uint16_t* __restrict__ img,
                                              int tid)
{
    for (int x = 0; x < 4; ++x) {
        const int e = tid + 256 * x;                    // slot e & 7 of row d
        const int d = e >> 3, c = (e & 7) ^ ((d >> 1) & 7);
        u32x4 val;
        for (int y = 0; y < 4; ++y) {
            const int p0 = 8 * c + 2 * y;               // positions p0, p0 + 1
            const int k0 = (p0 & ~12) | ((p0 & 4) << 1) | ((p0 & 8) >> 1);
            val[y] = (uint32_t)tile[k0][d] | ((uint32_t)tile[k0 + 1][d] << 16);
        }
        *reinterpret_cast<u32x4*>(img + 8 * e) = val;
    }
}

}  // namespace crisp
