// Device helpers shared by the bf16 and quantised prologues: per-(token, head)
// RMSNorm over d channels followed by interleaved-pair RoPE, in fp32.
//
// A row of d channels is spread over d/8 consecutive lanes, 8 channels
// (16 bytes of bf16) per lane; the sum of squares is a butterfly over those
// lanes, and each RoPE pair (2j, 2j+1) lives inside one lane.  These are the
// norm and rotation of the fused norm/RoPE/relayout kernel that the page "H3
// Runtime Current State" counts among the owed kernels ("Owned Performance
// Kernels"):
//   y_c = x_c / sqrt(mean_c x_c^2 + eps) * w_c, then pair (y_2j, y_2j+1) turned
//   by the token's angle for pair j (cos, sin taken from the RoPE table).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Unpack 8 bf16 values (16 bytes) to fp32.
__device__ __forceinline__ void unpack8(u32x4_t raw, float x[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16lo(raw[i]);
        x[2 * i + 1] = bf16hi(raw[i]);
    }
}

// RMSNorm + RoPE of the 8 channels [8c, 8c+8) this lane holds; LPR lanes
// (a power of two, aligned) share the row.  w: the 8 weights; cs: the 4
// (cos, sin) pairs of this lane's channels.  Rows that are padding pass
// zeros and get zeros back.
template <int LPR>
__device__ __forceinline__ void norm_rope8(const float x[8], const float w[8], const float cs[8],
                                           float inv_d, float eps, float y[8])
{
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
#pragma unroll
    for (int msk = LPR / 2; msk >= 1; msk >>= 1) ss += __shfl_xor(ss, msk, LPR);
    const float rs = rsqrtf(fmaf(ss, inv_d, eps));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = x[2 * i] * rs * w[2 * i];
        const float b = x[2 * i + 1] * rs * w[2 * i + 1];
        const float co = cs[2 * i], si = cs[2 * i + 1];
        y[2 * i] = a * co - b * si;
        y[2 * i + 1] = a * si + b * co;
    }
}

// Load the 8 weights of channels [8c, 8c+8) of weight row `row` (q: h, k: H + h).
__device__ __forceinline__ void load_w8(const float *norm_w, int64_t row, int d, int c, float w[8])
{
    const f32x4_t *wp = reinterpret_cast<const f32x4_t *>(norm_w + row * d + 8 * c);
    const f32x4_t a = wp[0], b = wp[1];
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
}

// (cos, sin) of the 4 pairs of channels [8c, 8c+8) of packed token `tok`.
__device__ __forceinline__ void load_cs8(const float *rope, int64_t tok, int d, int c, float cs[8])
{
    const f32x4_t *rp = reinterpret_cast<const f32x4_t *>(rope + tok * d + 8 * c);
    const f32x4_t a = rp[0], b = rp[1];
    cs[0] = a[0]; cs[1] = a[1]; cs[2] = a[2]; cs[3] = a[3];
    cs[4] = b[0]; cs[5] = b[1]; cs[6] = b[2]; cs[7] = b[3];
}

// Padded 64-token tile -> (sequence, tile within it, valid tokens).
__device__ __forceinline__ void tile_seq(const int32_t *cu, const int32_t *off, int S, int gt,
                                         int &s, int &j, int &valid)
{
    s = 0;
    while (s + 1 < S && gt >= off[s + 1] / 64) ++s;
    j = gt - off[s] / 64;
    const int n_s = cu[s + 1] - cu[s];
    valid = min(max(n_s - 64 * j, 0), 64);
}

}  // namespace h3
