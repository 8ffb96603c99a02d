// Fused Q/K RMSNorm + RoPE + layout prologue for gfx950.
//
// The page "H3 Runtime Current State" counts a fused Q/K norm, RoPE and
// relayout kernel among the owed ones ("Owned Performance Kernels"); "Buyer Questions: Current
// Evidence Status" (question 4) measures norm/RoPE as about 4% of a block and
// the strided-NHD QKV copy as about 3.6%.  This kernel does all of it in one
// HBM pass: it reads q, k and v once through their token strides, normalises
// and rotates q and k in fp32, and writes the head-major bf16 copies the
// attention kernel streams (qhat, khat: [H][Npad][d]; vt: V transposed per
// 64-key tile).  Padding rows of every sequence are written as zeros, so the
// attention kernel never reads uninitialised memory.  qhat is stored already
// multiplied by softmax_scale * log2(e), so the attention kernel's scores come
// out of the matrix cores in base-2 exponent units.
//
// It also records, per 64-token tile and head, the largest 2-norm of the stored
// (bf16-rounded) khat rows.  With |qhat| this bounds every score of a query row
// (Cauchy-Schwarz), which lets the attention kernel fix its softmax shift up
// front.
//
// Work split: one workgroup (256 lanes) handles one 64-token tile of one head.
// d/8 lanes share a (token, head) row, 16 bytes (8 channels) per lane, so
// every global access is a coalesced 16-byte vector access and the RMSNorm
// reduction is a d/8-lane butterfly.  RoPE pairs (2j, 2j+1) sit inside one
// lane.  Workgroups are numbered so that all heads of one token tile run on
// the same XCD (dispatch is round-robin over the 8 XCDs): the RoPE table rows
// of the tile are then fetched into that XCD's L2 once.
#include "h3_internal.h"
#include "norm_rope.h"

namespace h3 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}

// Position of token r (0..63) inside its tile of the transposed V copy: bits
// 2 and 3 swapped, the order in which the attention kernel's P.V operand
// consumes keys (see attn_bf16.hip).
__device__ __forceinline__ int vt_pos(int r)
{
    return (r & ~0xC) | ((r >> 1) & 4) | ((r << 1) & 8);
}

template <int D>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a)
{
    constexpr int LPR = D / 8;          // lanes per (token, head) row
    constexpr int RPP = 256 / LPR;      // rows per pass
    __shared__ __attribute__((aligned(16))) uint16_t vl[D][64 + 8];
    __shared__ float kred[4];

    const int H = a.H;
    const int b = blockIdx.x;
    const int gt = 8 * ((b >> 3) / H) + (b & 7);    // padded tile index
    const int h = (b >> 3) % H;
    if (gt >= a.ntiles) return;
    int s, j, valid;
    tile_seq(a.seq.cu, a.seq.off, a.seq.S, gt, s, j, valid);
    if (a.natural && valid == 0) return;

    const int t = threadIdx.x;
    const int c = t % LPR;
    const int rr = t / LPR;
    const float inv_d = 1.0f / (float)D;
    float wq[8], wk[8];
    load_w8(a.norm_w, h, D, c, wq);
    load_w8(a.norm_w, H + h, D, c, wk);
    float kn2 = 0.f;                    // largest |khat|^2 of the rows this lane saw

#pragma unroll
    for (int pass = 0; pass < kTile / RPP; ++pass) {
        const int r = pass * RPP + rr;
        const bool ok = r < valid;
        const int64_t tok = (int64_t)a.seq.cu[s] + kTile * j + r;
        float cs[8] = {1.f, 0.f, 1.f, 0.f, 1.f, 0.f, 1.f, 0.f};
        if (ok) load_cs8(a.rope, tok, D, c, cs);
        const int64_t orow = a.natural ? tok : (int64_t)a.seq.off[s] + kTile * j + r;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const uint16_t *src = which ? a.k + tok * a.k_stride : a.q + tok * a.q_stride;
            u32x4_t raw = {0u, 0u, 0u, 0u};
            if (ok) raw = *reinterpret_cast<const u32x4_t *>(src + h * D + 8 * c);
            float x[8], y[8];
            unpack8(raw, x);
            norm_rope8<LPR>(x, which ? wk : wq, cs, inv_d, a.eps, y);
            if (!which) {
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] *= a.q_mult;
            }
            u32x4_t o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = pack_bf16(y[2 * i], y[2 * i + 1]);
            if (!ok) o = (u32x4_t){0u, 0u, 0u, 0u};
            if (which) {
                // squared norm of the stored row: the lane's 8 rounded values,
                // then a butterfly over the row's LPR lanes
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float lo = __uint_as_float(o[i] << 16), hi = __uint_as_float(o[i] & 0xffff0000u);
                    ss = fmaf(lo, lo, fmaf(hi, hi, ss));
                }
#pragma unroll
                for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
                kn2 = fmaxf(kn2, ss);
            }
            if (ok || !a.natural) {
                uint16_t *dst = (which ? a.khat : a.qhat) + h * a.out_hstride + orow * a.out_tstride + 8 * c;
                *reinterpret_cast<u32x4_t *>(dst) = o;
            }
        }
        if (!a.natural) {
            u32x4_t raw = {0u, 0u, 0u, 0u};
            if (ok) raw = *reinterpret_cast<const u32x4_t *>(a.v + tok * a.v_stride + h * D + 8 * c);
            const int p = vt_pos(r);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vl[8 * c + 2 * i][p] = (uint16_t)(raw[i] & 0xffffu);
                vl[8 * c + 2 * i + 1][p] = (uint16_t)(raw[i] >> 16);
            }
        }
    }
    if (a.natural) return;
#pragma unroll
    for (int m = 32; m >= LPR; m >>= 1) kn2 = fmaxf(kn2, __shfl_xor(kn2, m));
    if ((t & 63) == 0) kred[t >> 6] = kn2;
    __syncthreads();
    if (t == 0)
        a.knorm[(int64_t)h * a.ntiles + gt] = sqrtf(fmaxf(fmaxf(kred[0], kred[1]), fmaxf(kred[2], kred[3])));
    uint16_t *vt = a.vt + ((int64_t)h * a.ntiles + gt) * (D * kTile);
#pragma unroll
    for (int g = t; g < D * 8; g += 256) {
        const int row = g >> 3, cc = g & 7;
        *reinterpret_cast<u32x4_t *>(vt + row * kTile + 8 * cc) =
            *reinterpret_cast<const u32x4_t *>(&vl[row][8 * cc]);
    }
}

hipError_t launch_prologue(const PrologueArgs &a, int d, hipStream_t st)
{
    const int64_t groups = (a.ntiles + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * a.H));
    if (d == 128)
        hipLaunchKernelGGL(prologue_kernel<128>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(prologue_kernel<64>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace h3
