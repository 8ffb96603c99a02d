// Output projection with the gated residual of a DiT-style block, for gfx950:
//   out[t][c] = resid[t][c] + gate[s(t)][c] * (attn[t] . W_o[c])
// where s(t) is the sequence of packed token t.
//
// The page "Buyer Questions: Current Evidence Status" (question 4) puts the
// block's GEMMs at about 27% and its "gates" at about 2% of block time; the
// page "Open-H3-Regenerate-2K" lists an adaLN table among the model files.
// The pages give no formula; this is the plain reading of an adaLN block's
// attention branch: the bias-free output projection of the attention output,
// scaled per channel by the sequence's gate and added to the residual stream,
// all in one pass, so the projected activations never go to memory on their
// own.  attn is read through its token stride (the [N, H, d] output of the
// attention kernel is a [N, H*d] matrix), the product runs on the matrix
// cores in the shared main loop of proj_gemm.h (256 tokens x 256 output
// channels per 8-wave workgroup), and the epilogue applies gate and residual
// in fp32 and rounds once to bf16.
#include "h3_internal.h"
#include "proj_gemm.h"

namespace h3 {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64 * kGemmWaves, 1) void out_proj_kernel(OutProjArgs a)
{
    constexpr int D = 128;                           // output channels per wave
    constexpr int FB = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t lx0[kGemmBM * kGemmBK], lx1[kGemmBM * kGemmBK],
        lx2[kGemmBM * kGemmBK], lx3[kGemmBM * kGemmBK];
    __shared__ __attribute__((aligned(16))) uint16_t lw0[2 * D * kGemmBK], lw1[2 * D * kGemmBK],
        lw2[2 * D * kGemmBK], lw3[2 * D * kGemmBK];
    const GemmStages<D> stages = {{lx0, lx1, lx2, lx3}, {lw0, lw1, lw2, lw3}};

    const int nfb = a.model_dim / D;
    int blk, F2;
    if (!gemm_tile<2>(a.nblk, (nfb + 1) / 2, blk, F2)) return;
    const int rows_blk = (int)min(a.N - (int64_t)kGemmBM * blk, (int64_t)kGemmBM);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, hh = lane >> 5;
    const int tw = wave & 3, fw = wave >> 2;
    const int F = 2 * F2 + fw;                       // this wave's 128-channel block
    const int nf_blk = min(2, nfb - 2 * F2);

    const uint32_t xrow = (uint32_t)(a.attn_stride * 2), wrow = (uint32_t)(a.K * 2);
    const uint16_t *xbase = a.attn + (int64_t)kGemmBM * blk * a.attn_stride;
    const uint16_t *wbase = a.w + (int64_t)2 * F2 * D * a.K;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(xbase), 0, (int)((uint32_t)(rows_blk - 1) * xrow + wrow), kBufferFlags);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(wbase), 0, (int)((uint32_t)(nf_blk * D) * wrow), kBufferFlags);

    f32x16 acc[2][FB];
    gemm_mainloop<D>(acc, stages, xrs, xrow, wrs, wrow, a.K / kGemmBK, wave, lane);
    if (F >= nfb) return;

    // ---- epilogue: gate and residual in fp32, one rounding to bf16
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int64_t tok = (int64_t)kGemmBM * blk + 64 * tw + 32 * tb + m;
        if (tok >= a.N) continue;
        int s = 0;
        while (s + 1 < a.S && tok >= a.cu[s + 1]) ++s;
        const float *g = a.gate ? a.gate + (int64_t)s * a.model_dim : nullptr;
        const uint16_t *r = a.resid ? a.resid + tok * a.resid_stride : nullptr;
        uint16_t *o = a.out + tok * a.out_stride;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f0 = D * F + 32 * fb + 8 * q + 4 * hh;
                f32x4 gv = {1.f, 1.f, 1.f, 1.f};
                if (g) gv = *reinterpret_cast<const f32x4 *>(g + f0);
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = acc[tb][fb][4 * q + e] * gv[e];
                if (r) {
                    const u32x2 rv = *reinterpret_cast<const u32x2 *>(r + f0);
                    y[0] += __uint_as_float(rv[0] << 16);
                    y[1] += __uint_as_float(rv[0] & 0xffff0000u);
                    y[2] += __uint_as_float(rv[1] << 16);
                    y[3] += __uint_as_float(rv[1] & 0xffff0000u);
                }
                *reinterpret_cast<u32x2 *>(o + f0) = (u32x2){pack2(y[0], y[1]), pack2(y[2], y[3])};
            }
        }
    }
}

hipError_t launch_out_proj(const OutProjArgs &a, hipStream_t st)
{
    const dim3 grid(gemm_grid(a.nblk, (a.model_dim / 128 + 1) / 2));
    hipLaunchKernelGGL(out_proj_kernel, grid, dim3(64 * kGemmWaves), 0, st, a);
    return hipGetLastError();
}

}  // namespace h3
