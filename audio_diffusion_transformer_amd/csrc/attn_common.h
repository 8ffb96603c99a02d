// Device helpers shared by the attention kernels (bf16 and quantised):
// LDS swizzle, direct-to-LDS tile fills, the row exchange between the two
// 32-lane halves of a wave that hold one query row, and small packing and
// INT8 coding helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3_internal.h"

namespace h3 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// s_waitcnt immediate (gfx9 encoding): vmcnt(0), expcnt and lgkmcnt left at their maximum.
constexpr int kWaitVmcnt0 = 0x0F70;
// Word 3 of a raw (unformatted, stride 0) buffer descriptor on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;
// s_waitcnt immediate (gfx9 encoding): vmcnt = n < 64, lgkmcnt = 0, expcnt at its maximum.
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would wait for every direct-to-LDS fill in flight, including those of
// stages that are not read yet.  The caller has already waited for what the
// barrier hands over; the clobber keeps memory accesses on their side of it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    bf16x2_t v = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

// 16-byte chunk swizzle of an LDS row: rows of 256 bytes (16 chunks) XOR the
// chunk index with row % 16, rows of 128 bytes (8 chunks) with (row / 2) % 8,
// rows of 64 bytes (4 chunks) with (row / 4) % 4, rows of 32 bytes (2 chunks)
// with (row / 8) % 2, so that 16 consecutive rows read at one logical chunk
// cover all 64 banks.
template <int CPR>
__device__ __forceinline__ int swz(int row)
{
    return CPR == 16 ? (row & 15) : CPR == 8 ? ((row >> 1) & 7) : CPR == 4 ? ((row >> 2) & 3) : ((row >> 3) & 1);
}

// Direct-to-LDS tile fill (buffer_load_dwordx4 ... lds): a tile of ROWS x CPR
// 16-byte chunks lies contiguously in global memory; every wave instruction
// writes 1 KB of LDS, lane L the 16 bytes at offset 16 L, so lane L fetches
// the global chunk the swizzle places there.  The per-lane offsets do not
// depend on the tile and are computed once; the tile's offset is a scalar and
// the buffer descriptor bounds every access to the sequence's rows.
template <int ROWS, int CPR>
struct TileFill {
    static constexpr int KB = ROWS * CPR / 64;   // 1 KB pieces in the tile
    static constexpr int PER_WAVE = KB / 4;
    static constexpr int RPK = 64 / CPR;         // rows per piece
    uint32_t goff[PER_WAVE];                     // byte offsets in the global tile
    __device__ __forceinline__ void init(int wave, int lane)
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int row = (wave * PER_WAVE + i) * RPK + lane / CPR;
            goff[i] = (uint32_t)(row * CPR + ((lane % CPR) ^ swz<CPR>(row))) * 16u;
        }
    }
    // Piece i (< PER_WAVE) of this wave's share of the tile at byte offset
    // `toff` (wave-uniform) of the buffer `rsrc`.
    __device__ __forceinline__ void load_piece(__amdgpu_buffer_rsrc_t rsrc, uint32_t toff, void *lds, int wave,
                                               int i) const
    {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void *)(static_cast<char *>(lds) + (wave * PER_WAVE + i) * 1024),
            16, goff[i], toff, 0, 0);
    }
    // This wave's whole share at once.
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, uint32_t toff, void *lds, int wave) const
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc,
                (__attribute__((address_space(3))) void *)(static_cast<char *>(lds) + (wave * PER_WAVE + i) * 1024),
                16, goff[i], toff, 0, 0);
    }
};

// max / sum of a lane's value and the value of lane l ^ 32 (same query row).
__device__ __forceinline__ float row_max2(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum2(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// INT8 code of r: round half to even, clamped to [-127, 127].
__device__ __forceinline__ int32_t i8code(float r)
{
    return (int32_t)fminf(fmaxf(__builtin_rintf(r), -127.f), 127.f);
}

__device__ __forceinline__ uint32_t pack_i8x4(int32_t a, int32_t b, int32_t c, int32_t d)
{
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// Row maximum of the 32 scores a lane holds (16 of each 32-key block).
__device__ __forceinline__ float lane_max32(const f32x16 &s0, const f32x16 &s1)
{
    float a = max3f(s0[0], s0[1], s0[2]), b = max3f(s1[0], s1[1], s1[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
        a = max3f(a, s0[r], s0[r + 1]);
        b = max3f(b, s1[r], s1[r + 1]);
    }
    return max3f(a, b, fmaxf(s0[15], s1[15]));
}

}  // namespace h3
