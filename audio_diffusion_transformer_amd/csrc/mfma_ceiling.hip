// Sustained bf16 matrix-core rate of the part, for the roofline of the
// attention kernels: register-only streams of v_mfma_f32_32x32x16_bf16 on
// every CU, operands changing from instruction to instruction like a real
// product (eight A and eight B fragments of hashed values), optionally with
// one v_exp_f32 and one FMA per MFMA beside them (the vector work the
// attention's softmax adds per MFMA).  Under a sustained load the engine
// clock settles where the part's power limit puts it for this kind of work,
// so the measured rate, not the datasheet figure, is what a dense bf16
// kernel can reach on the box.
#include "h3_internal.h"

namespace h3 {

typedef __bf16 bf16x8c __attribute__((ext_vector_type(8)));
typedef float f32x16c __attribute__((ext_vector_type(16)));

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

hipError_t launch_mfma_ceiling(int mix, int workgroups, int iters, float *out, hipStream_t st)
{
    if (mix)
        hipLaunchKernelGGL((mfma_ceiling_kernel<true>), dim3((unsigned)workgroups), dim3(512), 0, st, out, iters);
    else
        hipLaunchKernelGGL((mfma_ceiling_kernel<false>), dim3((unsigned)workgroups), dim3(512), 0, st, out, iters);
    return hipGetLastError();
}

}  // namespace h3
