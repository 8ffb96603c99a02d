// Block-quantised attention for gfx950: INT8 Q.K^T and FP8 (e4m3) P.V on the
// CDNA4 matrix cores, fp32 accumulation.
//
// Role: the quantised attention backend of a MiniMax-H3 block.  The page "H3
// Runtime Current State" names SageAttention2 the default quality backend and
// lists approximate INT8 backends; "Buyer Questions: Current Evidence Status"
// (question 4) puts attention at about 58% of block time.  Those CUDA kernels
// are prior art only; this path is designed for the CDNA4 INT8/FP8 MFMAs.
//
// Steps (d = 128):
//  pass 1  per 64-token tile and head: RMSNorm + RoPE of q and k in fp32;
//          qhat -> INT8 with one scale per tile (scale = amax / 127, codes
//          round-half-even, clamped to +-127); per-channel partial sums of khat
//          and per-channel maxima of |v| for the tile.
//  reduce  per (sequence, head): mean of khat over the sequence's tokens and
//          V scale = amax / 448 per channel, in a fixed order.
//  pass 3  recompute khat exactly as in pass 1, subtract the mean (softmax is
//          unchanged by a per-sequence shift of every key), INT8 per tile;
//          v / scale -> FP8 e4m3, stored transposed per 64-key tile in the key
//          order the FP8 P.V operand consumes.
//  attention  S^T = K8 . Q8^T on v_mfma_i32_32x32x32_i8 (exact i32), scaled
//          by s_q * s_k * softmax_scale * log2(e); online softmax in base 2
//          with the running max raised only when a tile exceeds it by more
//          than 1, so p <= 2; P quantised to e4m3 as p * 224 (a fixed per-row
//          scale mapping the largest possible p to 448); O^T += V8^T . P8^T on
//          v_mfma_f32_32x32x64_f8f6f4; the row sum l is the sum of the
//          quantised P (one more, half-size FP8 MFMA against ones).  Finally
//          o_c = O_c * vscale_c / l.
#include "h3_internal.h"
#include "norm_rope.h"
#include "attn_common.h"
#include "h3_checked.h"

namespace h3 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int QD = 128;               // head dim of the quantised path
constexpr float kPScale = 224.0f;     // 448 / 2^kQ8Lazy
constexpr float kQ8Lazy = 1.0f;       // running max raised when a tile exceeds it by > 1 (log2 units)

// Four fp32 -> four OCP e4m3 bytes (round to nearest even), little-endian.  The
// first conversion's pass-through operand is arbitrary (its half is overwritten
// by the second); passing a dead input avoids materialising a zero.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Position of key r (0..63) of a tile in the transposed FP8 V copy: lane half
// h of the P.V operand feeds keys {32(e/16) + 8((e%16)/4) + 4h + e%4 : e < 32}
// as bytes 32h + e, so key bits (5, 4:3, 2, 1:0) go to positions (4, 3:2, 5, 1:0).
__device__ __forceinline__ int v8_pos(int r)
{
    return (((r >> 2) & 1) << 5) | (((r >> 5) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3);
}

__device__ __forceinline__ float block_max256(float v, float *red)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Decode of the XCD-aware (tile, head) numbering shared with the bf16 prologue.
__device__ __forceinline__ bool tile_head(int H, int ntiles, int &gt, int &h)
{
    const int b = blockIdx.x;
    gt = 8 * ((b >> 3) / H) + (b & 7);
    h = (b >> 3) % H;
    return gt < ntiles;
}

// ------------------------------------------------------------------ pass 1
// WS (the projection's quantised path): khat and v come from a.k32 / a.v16,
// and qhat was already coded by the projection, so only the K sums and the V
// maxima are formed.
template <bool WS>
__global__ __launch_bounds__(256) void q8_pass1_kernel(Q8Args a)
{
    constexpr int LPR = QD / 8, RPP = 256 / LPR;
    __shared__ float red[4];
    __shared__ float kred[RPP][QD];
    __shared__ float vred[RPP][QD];
    int gt, h;
    if (!tile_head(a.H, a.ntiles, gt, h)) return;
    int s, j, valid;
    tile_seq(a.seq.cu, a.seq.off, a.seq.S, gt, s, j, valid);
    const int t = threadIdx.x, c = t % LPR, rr = t / LPR;
    float ks[8], vm[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ks[i] = vm[i] = 0.f;
    if constexpr (WS) {
#pragma unroll
        for (int pass = 0; pass < kTile / RPP; ++pass) {
            const int r = pass * RPP + rr;
            if (r < valid) {
                const int64_t row = ((int64_t)h * a.Npad + a.seq.off[s] + kTile * j + r) * QD + 8 * c;
                const f32x4_t k0 = *reinterpret_cast<const f32x4_t *>(a.k32 + row);
                const f32x4_t k1 = *reinterpret_cast<const f32x4_t *>(a.k32 + row + 4);
                float x[8];
                unpack8(*reinterpret_cast<const u32x4_t *>(a.v16 + row), x);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ks[i] += k0[i];
                    ks[4 + i] += k1[i];
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) vm[i] = fmaxf(vm[i], fabsf(x[i]));
            }
        }
    } else {
        float wq[8], wk[8], qv[kTile / RPP][8], qa = 0.f;
        load_w8(a.norm_w, h, QD, c, wq);
        load_w8(a.norm_w, a.H + h, QD, c, wk);
#pragma unroll
        for (int pass = 0; pass < kTile / RPP; ++pass) {
            const int r = pass * RPP + rr;
            const bool ok = r < valid;
            const int64_t tok = (int64_t)a.seq.cu[s] + kTile * j + r;
            float cs[8] = {1.f, 0.f, 1.f, 0.f, 1.f, 0.f, 1.f, 0.f};
            if (ok) load_cs8(a.rope, tok, QD, c, cs);
            u32x4_t rq = {0u, 0u, 0u, 0u}, rk = rq, rv = rq;
            if (ok) {
                rq = *reinterpret_cast<const u32x4_t *>(a.q + tok * a.q_stride + h * QD + 8 * c);
                rk = *reinterpret_cast<const u32x4_t *>(a.k + tok * a.k_stride + h * QD + 8 * c);
                rv = *reinterpret_cast<const u32x4_t *>(a.v + tok * a.v_stride + h * QD + 8 * c);
            }
            float x[8], y[8];
            unpack8(rq, x);
            norm_rope8<LPR>(x, wq, cs, 1.0f / QD, a.eps, y);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qv[pass][i] = ok ? y[i] : 0.f;
                qa = fmaxf(qa, fabsf(qv[pass][i]));
            }
            unpack8(rk, x);
            norm_rope8<LPR>(x, wk, cs, 1.0f / QD, a.eps, y);
            if (ok) {
#pragma unroll
                for (int i = 0; i < 8; ++i) ks[i] += y[i];
            }
            unpack8(rv, x);
#pragma unroll
            for (int i = 0; i < 8; ++i) vm[i] = fmaxf(vm[i], fabsf(x[i]));
        }
        const float amax = block_max256(qa, red);
        const float sq = amax > 0.f ? amax / 127.0f : 1.0f;
#pragma unroll
        for (int pass = 0; pass < kTile / RPP; ++pass) {
            const int r = pass * RPP + rr;
            int32_t q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = i8code(qv[pass][i] / sq);
            const u32x2_t w2 = {pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7])};
            *reinterpret_cast<u32x2_t *>(a.q8 + ((int64_t)h * a.Npad + a.seq.off[s] + kTile * j + r) * QD + 8 * c) = w2;
        }
        if (t == 0) a.qscale[(int64_t)h * a.ntiles + gt] = sq;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        kred[rr][8 * c + i] = ks[i];
        vred[rr][8 * c + i] = vm[i];
    }
    __syncthreads();
    if (t < QD) {
        float sum = 0.f, mx = 0.f;
        for (int g = 0; g < RPP; ++g) {
            sum += kred[g][t];
            mx = fmaxf(mx, vred[g][t]);
        }
        const int64_t o = ((int64_t)h * a.ntiles + gt) * QD + t;
        a.ksum[o] = sum;
        a.vmax[o] = mx;
    }
}

// ------------------------------------------------------------------ reduce
// One workgroup per (sequence, head): thread (g, c) folds the per-tile partials
// of channel c for tiles g, g+8, g+16, ...; the 8 groups are then combined in
// LDS in group order, so the result does not depend on timing.
constexpr int kReduceGroups = 8;
__global__ __launch_bounds__(kReduceGroups * QD) void q8_reduce_kernel(Q8Args a)
{
    __shared__ float rs[kReduceGroups][QD], rm[kReduceGroups][QD];
    const int s = blockIdx.x / a.H, h = blockIdx.x % a.H;
    const int c = threadIdx.x % QD, g = threadIdx.x / QD;
    const int n = a.seq.cu[s + 1] - a.seq.cu[s];
    const int t0 = a.seq.off[s] / kTile, nt = (n + kTile - 1) / kTile;
    float sum = 0.f, mx = 0.f;
#pragma unroll 4
    for (int i = g; i < nt; i += kReduceGroups) {
        const int64_t o = ((int64_t)h * a.ntiles + t0 + i) * QD + c;
        sum += a.ksum[o];
        mx = fmaxf(mx, a.vmax[o]);
    }
    rs[g][c] = sum;
    rm[g][c] = mx;
    __syncthreads();
    if (g == 0) {
        for (int k = 1; k < kReduceGroups; ++k) {
            sum += rs[k][c];
            mx = fmaxf(mx, rm[k][c]);
        }
        const int64_t o = ((int64_t)s * a.H + h) * QD + c;
        a.kmean[o] = n > 0 ? sum / (float)n : 0.f;
        a.vscale[o] = mx > 0.f ? mx / 448.0f : 1.0f;
    }
}

// ------------------------------------------------------------------ pass 3
// WS: khat and v read from a.k32 / a.v16 (the projection's quantised path).
template <bool WS>
__global__ __launch_bounds__(256) void q8_pass3_kernel(Q8Args a)
{
    constexpr int LPR = QD / 8, RPP = 256 / LPR;
    __shared__ float red[4];
    __shared__ __attribute__((aligned(16))) uint8_t lv8[QD][kTile + 16];
    int gt, h;
    if (!tile_head(a.H, a.ntiles, gt, h)) return;
    int s, j, valid;
    tile_seq(a.seq.cu, a.seq.off, a.seq.S, gt, s, j, valid);
    const int t = threadIdx.x, c = t % LPR, rr = t / LPR;
    float wk[8], km[8], vsc[8];
    if constexpr (!WS) load_w8(a.norm_w, a.H + h, QD, c, wk);
    load_w8(a.kmean, (int64_t)s * a.H + h, QD, c, km);
    load_w8(a.vscale, (int64_t)s * a.H + h, QD, c, vsc);
    float kv[kTile / RPP][8], ka = 0.f;
#pragma unroll
    for (int pass = 0; pass < kTile / RPP; ++pass) {
        const int r = pass * RPP + rr;
        const bool ok = r < valid;
        const int64_t tok = (int64_t)a.seq.cu[s] + kTile * j + r;
        float x[8], y[8];
        u32x4_t rv = {0u, 0u, 0u, 0u};
        if constexpr (WS) {
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = 0.f;
            if (ok) {
                const int64_t row = ((int64_t)h * a.Npad + a.seq.off[s] + kTile * j + r) * QD + 8 * c;
                const f32x4_t k0 = *reinterpret_cast<const f32x4_t *>(a.k32 + row);
                const f32x4_t k1 = *reinterpret_cast<const f32x4_t *>(a.k32 + row + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    y[i] = k0[i];
                    y[4 + i] = k1[i];
                }
                rv = *reinterpret_cast<const u32x4_t *>(a.v16 + row);
            }
        } else {
            float cs[8] = {1.f, 0.f, 1.f, 0.f, 1.f, 0.f, 1.f, 0.f};
            if (ok) load_cs8(a.rope, tok, QD, c, cs);
            u32x4_t rk = {0u, 0u, 0u, 0u};
            if (ok) {
                rk = *reinterpret_cast<const u32x4_t *>(a.k + tok * a.k_stride + h * QD + 8 * c);
                rv = *reinterpret_cast<const u32x4_t *>(a.v + tok * a.v_stride + h * QD + 8 * c);
            }
            unpack8(rk, x);
            norm_rope8<LPR>(x, wk, cs, 1.0f / QD, a.eps, y);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kv[pass][i] = ok ? y[i] - km[i] : 0.f;
            ka = fmaxf(ka, fabsf(kv[pass][i]));
        }
        unpack8(rv, x);
        float vq[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) vq[i] = ok ? x[i] / vsc[i] : 0.f;
        const uint32_t lo = fp8x4(vq[0], vq[1], vq[2], vq[3]);
        const uint32_t hi = fp8x4(vq[4], vq[5], vq[6], vq[7]);
        const int p = v8_pos(r);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lv8[8 * c + i][p] = (uint8_t)(lo >> (8 * i));
            lv8[8 * c + 4 + i][p] = (uint8_t)(hi >> (8 * i));
        }
    }
    const float amax = block_max256(ka, red);
    const float sk = amax > 0.f ? amax / 127.0f : 1.0f;
#pragma unroll
    for (int pass = 0; pass < kTile / RPP; ++pass) {
        const int r = pass * RPP + rr;
        int32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = i8code(kv[pass][i] / sk);
        const u32x2_t w2 = {pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7])};
        *reinterpret_cast<u32x2_t *>(a.k8 + ((int64_t)h * a.Npad + a.seq.off[s] + kTile * j + r) * QD + 8 * c) = w2;
    }
    if (t == 0) a.kscale[(int64_t)h * a.ntiles + gt] = sk;
    __syncthreads();
    uint8_t *vt = a.v8t + ((int64_t)h * a.ntiles + gt) * (QD * kTile);
#pragma unroll
    for (int g = t; g < QD * kTile / 16; g += 256) {
        const int row = g >> 2, ch = g & 3;
        *reinterpret_cast<u32x4_t *>(vt + row * kTile + 16 * ch) =
            *reinterpret_cast<const u32x4_t *>(&lv8[row][16 * ch]);
    }
}

// -------------------------------------------------------- diagnostic export
__global__ __launch_bounds__(256) void q8_export_kernel(Q8ExportArgs a)
{
    int gt, h;
    if (!tile_head(a.H, a.ntiles, gt, h)) return;
    int s, j, valid;
    tile_seq(a.seq.cu, a.seq.off, a.seq.S, gt, s, j, valid);
    if (valid == 0) return;
    const int t = threadIdx.x, c = t & 15, rr = t >> 4;
    for (int r = rr; r < valid; r += 16) {
        const int64_t tok = (int64_t)a.seq.cu[s] + kTile * j + r;
        const int64_t src = ((int64_t)h * a.Npad + a.seq.off[s] + kTile * j + r) * QD + 8 * c;
        const int64_t dst = (tok * a.H + h) * QD + 8 * c;
        *reinterpret_cast<u32x2_t *>(a.q8_out + dst) = *reinterpret_cast<const u32x2_t *>(a.q8 + src);
        *reinterpret_cast<u32x2_t *>(a.k8_out + dst) = *reinterpret_cast<const u32x2_t *>(a.k8 + src);
        const uint8_t *vt = a.v8t + ((int64_t)h * a.ntiles + gt) * (QD * kTile);
        for (int i = 0; i < 8; ++i) a.v8_out[dst + i] = vt[(8 * c + i) * kTile + v8_pos(r)];
    }
    if (t == 0) {
        int b = 0;
        for (int q = 0; q < s; ++q) b += (a.seq.cu[q + 1] - a.seq.cu[q] + kTile - 1) / kTile;
        a.qscale_out[(int64_t)h * a.nblocks + b + j] = a.qscale[(int64_t)h * a.ntiles + gt];
        a.kscale_out[(int64_t)h * a.nblocks + b + j] = a.kscale[(int64_t)h * a.ntiles + gt];
    }
}

// --------------------------------------------------------------- attention
// One workgroup = 4 waves x 32 query rows of one (sequence, head).  K8 and
// V8^T tiles of 64 keys are filled straight into double-buffered LDS by
// buffer_load ... lds.  The loop is software-pipelined over three tiles so that
// every step of the steady state carries both matrix-core and vector work: step
// j issues the INT8 score MFMAs of tile j+1, the FP8 P.V MFMAs of tile j-1
// (whose P was packed in step j-1; one instruction covers the tile's 64 keys for
// 32 channels) and, beside them, the exp2 and FP8 packing of tile j.  The row
// sum comes from the matrix cores too: one more FP8 MFMA per tile multiplies P
// by a constant row of ones, so l is the sum of the quantised P actually
// applied to V.  It runs on the half-size 16 x 16 x 128 shape (half the
// matrix-core cycles of a 32 x 32 x 64 one, a 4-register accumulator).
__global__ __launch_bounds__(256, 2) void attn_q8_kernel(Q8AttnArgs a)
{
    __shared__ __attribute__((aligned(16))) int8_t lk0[kTile * QD], lk1[kTile * QD];
    __shared__ __attribute__((aligned(16))) uint8_t lv0[QD * kTile], lv1[QD * kTile];

    const int b = blockIdx.x;
    int si = 0;
    while (b >= a.item_pre[si + 1]) ++si;
    const int rem = b - a.item_pre[si];
    const int nqb = a.seq_nqb[si];
    const int head = rem / nqb, qb = rem % nqb;
    const int n = a.seq_n[si];
    const int off = a.seq_off[si];
    const int64_t ntiles = a.Npad / kTile;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, hh = lane >> 5;
    const int q0 = qb * kBlockM + wave * 32;
    H3_CHECK(si < a.nseq && head < a.H && qb < nqb, kCheckItem);
    H3_CHECK(off + q0 + 32 <= a.Npad, kCheckRows);

    i32x4 qf[4];
    {
        const int8_t *qp = a.q8 + ((int64_t)head * a.Npad + off + q0 + m) * QD + 16 * hh;
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const i32x4 *>(qp + 32 * s);
    }
    const float cq = a.qscale[head * ntiles + (off + q0) / kTile] * a.scale_log2;
    const float *ksc = a.kscale + head * ntiles + off / kTile;
    const int nt = (n + kTile - 1) / kTile;

    TileFill<kTile, 8> kfill;       // K8 rows: 128 bytes
    TileFill<QD, 4> vfill;          // V8^T rows: 64 bytes
    kfill.init(wave, lane);
    vfill.init(wave, lane);
    const int tbytes = kTile * QD;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(a.k8 + ((int64_t)head * a.Npad + off) * QD), 0, nt * tbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.v8t + ((int64_t)head * ntiles + off / kTile) * (QD * kTile)), 0, nt * tbytes,
        kBufferFlags);
    auto load_k = [&](int j, void *dst) {
        H3_CHECK(j >= 0 && j < nt, kCheckFillTile);
        H3_JITTER(wave, j, 0);
        kfill.load(krs, (uint32_t)(j * tbytes), dst, wave);
    };
    auto load_v = [&](int j, void *dst) {
        H3_CHECK(j >= 0 && j < nt, kCheckFillTile);
        H3_JITTER(wave, j, 1);
        vfill.load(vrs, (uint32_t)(j * tbytes), dst, wave);
    };

    f32x16 o[4];                    // O^T per 32-channel block
    for (int i = 0; i < 4; ++i) o[i] = (f32x16){};
    // Row sum on the 16 x 16 x 128 FP8 shape.  Its B operand is the P operand
    // as it stands, read as lane L = column L % 16 over keys 32 (L / 16) .. +31
    // (lane L of the 32 x 32 x 64 operand holds query L % 32, key half L / 32),
    // so column j holds queries j and j + 16.  A row 0 is e4m3 1.0 (0x38) in
    // lanes 0 and 32, row 1 in lanes 17 and 49, every other row 0: register 0
    // of lane j < 16 sums query j's P, register 1 query j + 16's, registers
    // 2, 3 and lanes 16..63 stay 0.
    f32x4_t ol = {};
    const uint32_t one4 = (lane == 0 || lane == 32 || lane == 17 || lane == 49) ? 0x38383838u : 0u;
    const i32x8 ones = {(int)one4, (int)one4, (int)one4, (int)one4, (int)one4, (int)one4, (int)one4, (int)one4};
    i32x8 pp = (i32x8){};          // FP8 P of the previous tile, whose P.V is still pending
    float m_run = 0.f;              // running max (log2 units) of the scaled scores
    bool first = true;
    const float lg2p = __builtin_log2f(kPScale);
    // The score accumulators start at the bits of 1.5 * 2^23: integer addition of
    // |S| < 2^22 then leaves the bits of the float 12582912 + S, so no int->float
    // conversion is needed (|S| <= 127 * 127 * 128 < 2^21).
    constexpr int32_t kMagicBits = 0x4B400000;
    constexpr float kMagic = 12582912.0f;
    // Held in VGPRs for the whole kernel (an opaque copy, so the compiler keeps
    // the 16-register block live instead of re-materialising it per tile).
    int32_t magic_v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic_v) : "s"(kMagicBits));
    const i32x16 magic = (i32x16){} + magic_v;

    // K fragment of score chunk c: 32-channel step c/2, key block c%2.
    auto kfrag = [&](const int8_t *kl, int c) -> i32x4 {
        const int ch = (2 * (c >> 1) + hh) ^ swz<8>(m);
        return *reinterpret_cast<const i32x4 *>(kl + (32 * (c & 1) + m) * QD + 16 * ch);
    };
    auto scores = [&](const int8_t *kl, i32x16 &s0, i32x16 &s1) {
        s0 = magic;
        s1 = magic;
#pragma unroll
        for (int c = 0; c < 8; c += 2) {
            s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(kfrag(kl, c), qf[c >> 1], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(kfrag(kl, c + 1), qf[c >> 1], s1, 0, 0, 0);
        }
    };
    // V^T fragment of 32-channel block db: the 64 keys of the tile, in the
    // operand's key order, as two 16-byte pieces.
    auto vfrag = [&](const uint8_t *vl, int db) -> i32x8 {
        const int row = 32 * db + m;
        const int sw = swz<4>(row);
        const i32x4 va = *reinterpret_cast<const i32x4 *>(vl + row * kTile + 16 * ((2 * hh) ^ sw));
        const i32x4 vb = *reinterpret_cast<const i32x4 *>(vl + row * kTile + 16 * ((2 * hh + 1) ^ sw));
        return (i32x8){va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
    };
    auto pv = [&](const uint8_t *vl, const i32x8 &pf) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
            o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vfrag(vl, db), pf, o[db], 0, 0, 0, 0, 0, 0);
        ol = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pf, ol, 0, 0, 0, 0, 0, 0);
    };
    // Key (0..63 within the tile) of element r of the lane's score block kb.
    auto key_of = [&](int kb, int r) { return 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3); };
    // P word w (keys of elements 4(w%4)..4(w%4)+3 of block w/4) as four e4m3
    // bytes: e4m3(2^x), x = raw * cs + c0 (the scaled score relative to m_run,
    // plus log2 224).  This byte order is the FP8 P.V operand's.
    auto pword = [&](const i32x16 &s0, const i32x16 &s1, int w, float cs, float c0) -> int32_t {
        const i32x16 &s = w < 4 ? s0 : s1;
        const int r = 4 * (w & 3);
        return (int32_t)fp8x4(__builtin_amdgcn_exp2f(fmaf(__int_as_float(s[r]), cs, c0)),
                              __builtin_amdgcn_exp2f(fmaf(__int_as_float(s[r + 1]), cs, c0)),
                              __builtin_amdgcn_exp2f(fmaf(__int_as_float(s[r + 2]), cs, c0)),
                              __builtin_amdgcn_exp2f(fmaf(__int_as_float(s[r + 3]), cs, c0)));
    };
    // Row max of tile j's raw scores (monotone in S; keys past the sequence end
    // excluded on the last tile).  When it exceeds m_run by more than kQ8Lazy
    // (always on the first tile) m_run is raised: the pending P.V of the
    // previous tile (V tile in vprev) is applied first, then O and the row sum
    // are rescaled.  Returns c0 for pword.
    auto tile_max = [&](int j, float cs, const i32x16 &s0, const i32x16 &s1, bool mask,
                        const uint8_t *vprev) -> float {
        float e[32];
        const int valid = n - j * kTile;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            e[r] = __int_as_float(s0[r]);
            e[16 + r] = __int_as_float(s1[r]);
            if (mask) {
                if (key_of(0, r) >= valid) e[r] = -INFINITY;
                if (key_of(1, r) >= valid) e[16 + r] = -INFINITY;
            }
        }
        float mx = max3f(e[0], e[1], e[2]);
#pragma unroll
        for (int r = 3; r < 31; r += 2) mx = max3f(mx, e[r], e[r + 1]);
        const float cm = -kMagic * cs;
        mx = fmaf(row_max2(fmaxf(mx, e[31])), cs, cm) - m_run;
        const bool need = first || mx > kQ8Lazy;
        if (__any(need)) {
            const float delta = need ? mx : 0.f;
            if (!first) {
                pv(vprev, pp);
                pp = (i32x8){};
                const float alpha = __builtin_amdgcn_exp2f(-delta);
                ol[0] *= alpha;     // query m of lane m < 16
                // query m + 16: the alpha of lane m + 16
                ol[1] *= __int_as_float(__builtin_amdgcn_ds_bpermute(((lane + 16) & 63) << 2, __float_as_int(alpha)));
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] *= alpha;
            }
            m_run += delta;
            first = false;
        }
        return lg2p - m_run + cm;
    };

    // Steady-state step (hand-scheduled): chunk i issues score MFMA i of the
    // next tile (K in kl), one FP8 MFMA of the pending P.V (row sum at chunk 0,
    // channel block db at chunk 2db+1; V of the previous tile in vprev) and P
    // word i of the current tile (raw scores c0s/c1s).  LDS fragments are read
    // two chunks ahead.  The fills of K tile kj (into kdst) and V tile vj (into
    // vdst) go out one 1 KB piece per chunk in chunks 0-3 (a negative tile
    // index skips them), so their issue overlaps the matrix cores.
    constexpr int KP = decltype(kfill)::PER_WAVE, VP = decltype(vfill)::PER_WAVE;
    static_assert(KP + VP <= 8, "fill pieces must fit in the step's chunks");
    auto body = [&](const int8_t *kl, const uint8_t *vprev, const i32x16 &c0s, const i32x16 &c1s, float cs,
                    float c0, i32x16 &n0, i32x16 &n1, int kj, void *kdst, int vj, void *vdst) {
        H3_CHECK(kj < nt && vj < nt, kCheckFillTile);
        H3_JITTER(wave, kj, 2);
        i32x4 kf[8];
        i32x8 vf[4];
        i32x8 pn;
        kf[0] = kfrag(kl, 0);
        kf[1] = kfrag(kl, 1);
        vf[0] = vfrag(vprev, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i + 2 < 8) kf[i + 2] = kfrag(kl, i + 2);
            if (kj >= 0 && i < KP) kfill.load_piece(krs, (uint32_t)(kj * tbytes), kdst, wave, i);
            else if (vj >= 0 && i >= KP && i < KP + VP)
                vfill.load_piece(vrs, (uint32_t)(vj * tbytes), vdst, wave, i - KP);
            if (i == 1 || i == 3 || i == 5) vf[(i + 1) >> 1] = vfrag(vprev, (i + 1) >> 1);
            const int st = i >> 1;
            if ((i & 1) == 0)
                n0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[i], qf[st], st ? n0 : magic, 0, 0, 0);
            else
                n1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[i], qf[st], st ? n1 : magic, 0, 0, 0);
            if (i == 0)
                ol = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pp, ol, 0, 0, 0, 0, 0, 0);
            else if (i & 1)
                o[i >> 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[i >> 1], pp, o[i >> 1], 0, 0, 0, 0, 0, 0);
            // The empty asm consumes the word here: without it the compiler
            // sinks every exp to the end of the step, where pn is first read.
            int32_t w = pword(c0s, c1s, i, cs, c0);
            asm volatile("" : "+v"(w));
            pn[i] = w;
            __builtin_amdgcn_sched_barrier(0);
        }
        pp = pn;
    };

    // ---- prologue: K0 and K1 resident, scores of tile 0.  V tile 0 also goes
    // to the buffer the first step reads as "previous tile": its pending P is
    // zero, so that P.V adds nothing (and the buffer holds finite values).
    __builtin_amdgcn_sched_barrier(0);
    load_k(0, lk0);
    if (nt > 1) load_k(1, lk1);
    load_v(0, lv1);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    i32x16 sa0, sa1, sb0, sb1;
    scores(lk0, sa0, sa1);
    __syncthreads();

    // Step j: K(j+2) -> kbuf[j%2], V(j) -> vbuf[j%2]; reads K(j+1) from
    // kbuf[(j+1)%2] and V(j-1) from vbuf[(j-1)%2].  The K scale of the next tile
    // is loaded a step ahead so that the wait before each barrier covers it.
    float ks0 = ksc[0];
    int j = 0;
    for (; j + 3 < nt; j += 2) {
        const float ks1 = ksc[j + 1];
        float cs = cq * ks0;
        float c0 = tile_max(j, cs, sa0, sa1, false, lv1);
        body(lk1, lv1, sa0, sa1, cs, c0, sb0, sb1, j + 2, lk0, j, lv0);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        ks0 = ksc[j + 2];
        cs = cq * ks1;
        c0 = tile_max(j + 1, cs, sb0, sb1, false, lv0);
        body(lk0, lv0, sb0, sb1, cs, c0, sa0, sa1, j + 3, lk1, j + 1, lv1);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
    }
    for (; j + 1 < nt; ++j) {
        const uint8_t *vp = ((j - 1) & 1) ? lv1 : lv0;
        if (j + 2 < nt) load_k(j + 2, (j & 1) ? lk1 : lk0);
        load_v(j, (j & 1) ? lv1 : lv0);
        const float cs = cq * ksc[j];
        const float c0 = tile_max(j, cs, sa0, sa1, false, vp);
        body(((j + 1) & 1) ? lk1 : lk0, vp, sa0, sa1, cs, c0, sb0, sb1, -1, nullptr, -1, nullptr);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        sa0 = sb0;
        sa1 = sb1;
    }
    // last tile (keys past the sequence end masked): its V is loaded here
    load_v(j, (j & 1) ? lv1 : lv0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    {
        const uint8_t *vp = ((j - 1) & 1) ? lv1 : lv0, *vl = (j & 1) ? lv1 : lv0;
        const float cs = cq * ksc[j];
        const float c0 = tile_max(j, cs, sa0, sa1, true, vp);
        pv(vp, pp);
        const int valid = n - j * kTile;
        i32x8 pf;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const i32x16 &s = w < 4 ? sa0 : sa1;
            float e[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 4 * (w & 3) + t;
                e[t] = key_of(w >> 2, r) < valid ? __builtin_amdgcn_exp2f(fmaf(__int_as_float(s[r]), cs, c0)) : 0.f;
            }
            pf[w] = (int32_t)fp8x4(e[0], e[1], e[2], e[3]);
        }
        pv(vl, pf);
    }

    // row sum of query m: register m / 16 of lane m % 16
    const float l0 = __shfl(ol[0], m & 15), l1 = __shfl(ol[1], m & 15);
    const float inv = 1.0f / (m < 16 ? l0 : l1);
    const int qrow = q0 + m;
    if (qrow < n) {
        const float *vs = a.vscale + ((int64_t)a.seq_idx[si] * a.H + head) * QD;
        uint16_t *op = a.out + ((int64_t)a.seq_cu[si] + qrow) * a.o_stride + (int64_t)head * QD;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * hh;
                const f32x4_t sc = *reinterpret_cast<const f32x4_t *>(vs + d0);
                const u32x2_t w = {pack2(o[db][4 * i] * sc[0] * inv, o[db][4 * i + 1] * sc[1] * inv),
                                   pack2(o[db][4 * i + 2] * sc[2] * inv, o[db][4 * i + 3] * sc[3] * inv)};
                *reinterpret_cast<u32x2_t *>(op + d0) = w;
            }
        }
    }
}

// Explicit instantiations: the host pass does not emit the launch stub of an
// instantiation that is only named inside the launcher's branches.
template __global__ void q8_pass1_kernel<false>(Q8Args);
template __global__ void q8_pass1_kernel<true>(Q8Args);
template __global__ void q8_pass3_kernel<false>(Q8Args);
template __global__ void q8_pass3_kernel<true>(Q8Args);

// ------------------------------------------------------------------ launch
hipError_t launch_q8_prep(const Q8Args &a, int d, hipStream_t st)
{
    if (d != QD) return hipErrorInvalidValue;
    const int64_t groups = (a.ntiles + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * a.H));
    const bool ws = a.k32 != nullptr;
    if (ws)
        hipLaunchKernelGGL(q8_pass1_kernel<true>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(q8_pass1_kernel<false>, grid, dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(q8_reduce_kernel, dim3((unsigned)(a.seq.S * a.H)), dim3(kReduceGroups * QD), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ws)
        hipLaunchKernelGGL(q8_pass3_kernel<true>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(q8_pass3_kernel<false>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

#ifdef H3ATTN_CHECKED
hipError_t q8_checked(uint32_t *or_into, bool clear, uint32_t jitter_seed)
{
    return checked_state_here(or_into, clear, jitter_seed);
}
#endif

hipError_t launch_attn_q8(const Q8AttnArgs &a, int d, int64_t nitems, hipStream_t st)
{
    if (d != QD) return hipErrorInvalidValue;
    if (nitems <= 0) return hipSuccess;
    hipLaunchKernelGGL(attn_q8_kernel, dim3((unsigned)nitems), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_q8_export(const Q8ExportArgs &a, hipStream_t st)
{
    const int64_t groups = (a.ntiles + 7) / 8;
    hipLaunchKernelGGL(q8_export_kernel, dim3((unsigned)(groups * 8 * a.H)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace h3
