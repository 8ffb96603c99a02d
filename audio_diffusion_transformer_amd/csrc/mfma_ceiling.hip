// Sustained matrix-core rate of the part, for the roofline of the attention
// kernels: register-only MFMA streams on every CU, operands changing from
// instruction to instruction like a real product (eight A and eight B
// fragments of hashed values), alone or with vector work beside them.  Under
// a sustained load the engine clock settles where the part's power limit
// puts it for this kind of work, so the measured rate, not the datasheet
// figure, is what a dense kernel can reach on the box.  Six mixes:
//   0  v_mfma_f32_32x32x16_bf16 alone;
//   1  the same with one v_exp_f32 and one FMA per MFMA (the vector work the
//      bf16 attention's softmax adds per MFMA);
//   2  v_mfma_i32_32x32x32_i8 alone;
//   3  the same with the quantised attention's vector work per 32 matrix-core
//      cycles: two FMAs, two v_exp_f32, one v_cvt_pk_fp8_f32 and one
//      v_max3_f32 (per 64-key tile and wave that kernel issues 544 cycles of
//      MFMA beside 32 FMAs, 32 exp2, 16 FP8 packs and the tile maximum), on
//      eight independent chains;
//   4  v_mfma_scale_f32_32x32x64_f8f6f4 on e2m1 (FP4) operands alone;
//   5  the same with the MXFP4 attention's vector work per 32 matrix-core
//      cycles: four v_exp_f32, two v_cvt_scalef32_pk_fp4_f32, two v_max3_f32
//      and one FMA (per 64-key tile and wave that kernel issues 272 cycles of
//      MFMA beside 32 exp2, 16 FP4 packs, the tile maximum and the block
//      scale).
// Mix 3 against mix 2 (5 against 4) shows how far the vector work of the
// quantised (MXFP4) path can hide under its matrix-core time on one SIMD.
#include "h3_internal.h"

namespace h3 {

typedef __bf16 bf16x8c __attribute__((ext_vector_type(8)));
typedef float f32x16c __attribute__((ext_vector_type(16)));
typedef int i32x4c __attribute__((ext_vector_type(4)));
typedef int i32x8c __attribute__((ext_vector_type(8)));
typedef int i32x16c __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float mix_hash(unsigned x)
{
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return (float)(int)(x & 0xFFFFu) / 32768.0f - 1.0f;
}

template <bool MIX>
__global__ __launch_bounds__(512) void mfma_ceiling_kernel(float *out, int iters)
{
    bf16x8c A[8], B[8];
    const unsigned t = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            A[j][i] = (__bf16)mix_hash(t * 131u + j * 17u + i);
            B[j][i] = (__bf16)mix_hash(t * 257u + j * 29u + i + 7777u);
        }
    f32x16c acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = (f32x16c){};
    float x = mix_hash(t) - 4.f, y = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[j], B[(3 * j + 1) & 7], acc[j & 3], 0, 0, 0);
            if (MIX) {
                x = __builtin_amdgcn_exp2f(x) - 4.f;
                y = fmaf(y, 0.999f, x);
            }
        }
    }
    float s = x + y;
#pragma unroll
    for (int k = 0; k < 4; ++k) s += acc[k][threadIdx.x & 15];
    out[t] = s;
}

template <bool MIX>
__global__ __launch_bounds__(512) void mfma_ceiling_i8_kernel(float *out, int iters, float cs, float c0)
{
    i32x4c A[8], B[8];
    const unsigned t = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            A[j][i] = __float_as_int(mix_hash(t * 131u + j * 17u + i)) ^ (int)(t * 2654435761u + 97u * j + i);
            B[j][i] = __float_as_int(mix_hash(t * 257u + j * 29u + i + 7777u)) ^ (int)(t * 40503u + 31u * j + i);
        }
    i32x16c acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = (i32x16c){};
    float sv[8], mx = -1.f;
    int w = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) sv[k] = -0.5f - 0.0625f * k;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc[j & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[j], B[(3 * j + 1) & 7], acc[j & 3], 0, 0, 0);
            if (MIX) {
                const int k = (2 * j) & 7;
                sv[k] = fmaf(sv[k], cs, c0);
                sv[k + 1] = fmaf(sv[k + 1], cs, c0);
                const float e0 = __builtin_amdgcn_exp2f(sv[k]), e1 = __builtin_amdgcn_exp2f(sv[k + 1]);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, w, false);
                mx = fmaxf(fmaxf(mx, e0), e1);
            }
        }
    }
    float s = mx + (float)w;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += sv[k];
#pragma unroll
    for (int k = 0; k < 4; ++k) s += (float)acc[k][threadIdx.x & 15];
    out[t] = s;
}

template <bool MIX>
__global__ __launch_bounds__(512) void mfma_ceiling_fp4_kernel(float *out, int iters, float cs)
{
    i32x8c A[8], B[8];
    const unsigned t = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // e2m1 codes: every nibble is a finite value; registers 4..7 are not read
            A[j][i] = i < 4 ? (int)(t * 2654435761u + 97u * j + 13u * i) : 0;
            B[j][i] = i < 4 ? (int)((t + 7777u) * 40503u + 31u * j + 29u * i) : 0;
        }
    f32x16c acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = (f32x16c){};
    float x[8], mx0 = 0.f, mx1 = 0.f, y = 0.f;
    uint32_t w = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = 0.5f + 0.01f * k;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc[j & 3] =
                __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[j], B[(3 * j + 1) & 7], acc[j & 3], 4, 4, 0, 127u, 0, 127u);
            if (MIX) {
                // x -> 2^-x stays near its fixed point 0.64, so the chains stay finite
                const int k = (4 * j) & 7;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[k + i] = __builtin_amdgcn_exp2f(-x[k + i]);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[k], x[k + 1], cs, 0);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[k + 2], x[k + 3], cs, 1);
                mx0 = fmaxf(fmaxf(mx0, x[k]), x[k + 1]);
                mx1 = fmaxf(fmaxf(mx1, x[k + 2]), x[k + 3]);
                y = fmaf(y, cs, x[k]);
            }
        }
    }
    float s = mx0 + mx1 + y + (float)w;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += x[k];
#pragma unroll
    for (int k = 0; k < 4; ++k) s += acc[k][threadIdx.x & 15];
    out[t] = s;
}

hipError_t launch_mfma_ceiling(int mix, int workgroups, int iters, float *out, hipStream_t st)
{
    const dim3 g((unsigned)workgroups), b(512);
    switch (mix) {
    case 0: hipLaunchKernelGGL((mfma_ceiling_kernel<false>), g, b, 0, st, out, iters); break;
    case 1: hipLaunchKernelGGL((mfma_ceiling_kernel<true>), g, b, 0, st, out, iters); break;
    case 2: hipLaunchKernelGGL((mfma_ceiling_i8_kernel<false>), g, b, 0, st, out, iters, 0.999f, -0.001f); break;
    case 3: hipLaunchKernelGGL((mfma_ceiling_i8_kernel<true>), g, b, 0, st, out, iters, 0.999f, -0.001f); break;
    case 4: hipLaunchKernelGGL((mfma_ceiling_fp4_kernel<false>), g, b, 0, st, out, iters, 1.0f); break;
    default: hipLaunchKernelGGL((mfma_ceiling_fp4_kernel<true>), g, b, 0, st, out, iters, 1.0f); break;
    }
    return hipGetLastError();
}

}  // namespace h3
