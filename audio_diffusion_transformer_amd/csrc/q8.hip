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
//          v_mfma_f32_32x32x64_f8f6f4; the row sum adds the unquantised p.
//          Finally o_c = O_c * vscale_c / (224 * l).
#include "h3_internal.h"
#include "norm_rope.h"

namespace h3 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int QD = 128;               // head dim of the quantised path
constexpr float kPScale = 224.0f;     // 448 / 2^kQ8Lazy
constexpr float kQ8Lazy = 1.0f;       // running max raised when a tile exceeds it by > 1 (log2 units)

__device__ __forceinline__ int32_t i8code(float r)
{
    return (int32_t)fminf(fmaxf(__builtin_rintf(r), -127.f), 127.f);
}

__device__ __forceinline__ uint32_t pack_i8x4(int32_t a, int32_t b, int32_t c, int32_t d)
{
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// Four fp32 -> four OCP e4m3 bytes (round to nearest even), little-endian.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
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
    float wq[8], wk[8];
    load_w8(a.norm_w, h, QD, c, wq);
    load_w8(a.norm_w, a.H + h, QD, c, wk);
    float qv[kTile / RPP][8], ks[8], vm[8], qa = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ks[i] = vm[i] = 0.f;
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
    if (t == 0) a.qscale[(int64_t)h * a.ntiles + gt] = sq;
}

// ------------------------------------------------------------------ reduce
__global__ __launch_bounds__(128) void q8_reduce_kernel(Q8Args a)
{
    const int s = blockIdx.x / a.H, h = blockIdx.x % a.H, c = threadIdx.x;
    const int n = a.seq.cu[s + 1] - a.seq.cu[s];
    const int t0 = a.seq.off[s] / kTile, nt = (n + kTile - 1) / kTile;
    float sum = 0.f, mx = 0.f;
    for (int i = 0; i < nt; ++i) {
        const int64_t o = ((int64_t)h * a.ntiles + t0 + i) * QD + c;
        sum += a.ksum[o];
        mx = fmaxf(mx, a.vmax[o]);
    }
    const int64_t o = ((int64_t)s * a.H + h) * QD + c;
    a.kmean[o] = n > 0 ? sum / (float)n : 0.f;
    a.vscale[o] = mx > 0.f ? mx / 448.0f : 1.0f;
}

// ------------------------------------------------------------------ pass 3
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
    load_w8(a.norm_w, a.H + h, QD, c, wk);
    load_w8(a.kmean, (int64_t)s * a.H + h, QD, c, km);
    load_w8(a.vscale, (int64_t)s * a.H + h, QD, c, vsc);
    float kv[kTile / RPP][8], ka = 0.f;
#pragma unroll
    for (int pass = 0; pass < kTile / RPP; ++pass) {
        const int r = pass * RPP + rr;
        const bool ok = r < valid;
        const int64_t tok = (int64_t)a.seq.cu[s] + kTile * j + r;
        float cs[8] = {1.f, 0.f, 1.f, 0.f, 1.f, 0.f, 1.f, 0.f};
        if (ok) load_cs8(a.rope, tok, QD, c, cs);
        u32x4_t rk = {0u, 0u, 0u, 0u}, rv = rk;
        if (ok) {
            rk = *reinterpret_cast<const u32x4_t *>(a.k + tok * a.k_stride + h * QD + 8 * c);
            rv = *reinterpret_cast<const u32x4_t *>(a.v + tok * a.v_stride + h * QD + 8 * c);
        }
        float x[8], y[8];
        unpack8(rk, x);
        norm_rope8<LPR>(x, wk, cs, 1.0f / QD, a.eps, y);
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
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(256, 2) void attn_q8_kernel(Q8AttnArgs a)
{
    constexpr int PER = kTile * QD / 16 / 256;      // 16-byte chunks per lane per tile (K and V each)
    __shared__ __attribute__((aligned(16))) int8_t lk[2][kTile * QD];
    __shared__ __attribute__((aligned(16))) uint8_t lv[2][QD * kTile];

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
    const int wave = tid >> 6, lane = tid & 63;
    const int m = lane & 31, hh = lane >> 5;
    const int q0 = qb * kBlockM + wave * 32;

    i32x4 qf[4];
    {
        const int8_t *qp = a.q8 + ((int64_t)head * a.Npad + off + q0 + m) * QD + 16 * hh;
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const i32x4 *>(qp + 32 * s);
    }
    const float cq = a.qscale[head * ntiles + (off + q0) / kTile] * a.scale_log2;
    const float *ksc = a.kscale + head * ntiles + off / kTile;
    const int8_t *kbase = a.k8 + ((int64_t)head * a.Npad + off) * QD;
    const uint8_t *vbase = a.v8t + ((int64_t)head * ntiles + off / kTile) * (QD * kTile);
    const int nt = (n + kTile - 1) / kTile;

    u32x4_t stk[PER], stv[PER];
    auto gload = [&](int j) {
        const u32x4_t *ks = reinterpret_cast<const u32x4_t *>(kbase + (int64_t)j * kTile * QD);
        const u32x4_t *vs = reinterpret_cast<const u32x4_t *>(vbase + (int64_t)j * QD * kTile);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            stk[i] = ks[tid + 256 * i];
            stv[i] = vs[tid + 256 * i];
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int g = tid + 256 * i;
            const int kr = g >> 3, kc = g & 7;
            *reinterpret_cast<u32x4_t *>(&lk[buf][kr * QD + 16 * (kc ^ (kr & 7))]) = stk[i];
            const int vr = g >> 2, vc = g & 3;
            *reinterpret_cast<u32x4_t *>(&lv[buf][vr * kTile + 16 * (vc ^ ((vr >> 1) & 3))]) = stv[i];
        }
    };

    f32x16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (f32x16){};
    float m_used = -INFINITY, l = 0.f;
    const float lg2p = __builtin_log2f(kPScale);

    gload(0);
    lstore(0);
    __syncthreads();

    for (int j = 0; j < nt; ++j) {
        const int buf = j & 1;
        if (j + 1 < nt) gload(j + 1);

        i32x16 s0 = (i32x16){}, s1 = (i32x16){};
        const int8_t *kl = lk[buf];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int ch = (2 * st + hh) ^ (m & 7);
            const i32x4 k0 = *reinterpret_cast<const i32x4 *>(kl + m * QD + 16 * ch);
            const i32x4 k1 = *reinterpret_cast<const i32x4 *>(kl + (32 + m) * QD + 16 * ch);
            s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(k0, qf[st], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(k1, qf[st], s1, 0, 0, 0);
        }
        const float cs = cq * ksc[j];
        float f0[16], f1[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            f0[r] = (float)s0[r] * cs;
            f1[r] = (float)s1[r] * cs;
        }
        const int valid = n - j * kTile;
        if (valid < kTile) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
                if (key >= valid) f0[r] = -INFINITY;
                if (32 + key >= valid) f1[r] = -INFINITY;
            }
        }
        float mx = fmaxf(f0[0], f1[0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(f0[r], f1[r]));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool need = mx - m_used > kQ8Lazy;
        if (__any(need)) {
            const float mn = need ? mx : m_used;
            const float alpha = __builtin_amdgcn_exp2f(m_used - mn);
            m_used = mn;
            l *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] *= alpha;
        }
        const float sub = m_used - lg2p;          // p * 224 = 2^(s - m + log2 224)
        i32x8 pf;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const float *src = w < 4 ? f0 + 4 * w : f1 + 4 * (w - 4);
            const float p0 = __builtin_amdgcn_exp2f(src[0] - sub);
            const float p1 = __builtin_amdgcn_exp2f(src[1] - sub);
            const float p2 = __builtin_amdgcn_exp2f(src[2] - sub);
            const float p3 = __builtin_amdgcn_exp2f(src[3] - sub);
            l += (p0 + p1) + (p2 + p3);
            pf[w] = (int32_t)fp8x4(p0, p1, p2, p3);
        }

        const uint8_t *vl = lv[buf];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int row = 32 * db + m;
            const int sw = (row >> 1) & 3;
            const i32x4 va = *reinterpret_cast<const i32x4 *>(vl + row * kTile + 16 * ((2 * hh) ^ sw));
            const i32x4 vb = *reinterpret_cast<const i32x4 *>(vl + row * kTile + 16 * ((2 * hh + 1) ^ sw));
            const i32x8 vf = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
            o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, o[db], 0, 0, 0, 0, 0, 0);
        }

        if (j + 1 < nt) lstore(buf ^ 1);
        __syncthreads();
    }

    const float lt = l + __shfl_xor(l, 32);
    const float inv = 1.0f / lt;
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
                const u32x2_t w = {pack_bf16(o[db][4 * i] * sc[0] * inv, o[db][4 * i + 1] * sc[1] * inv),
                                   pack_bf16(o[db][4 * i + 2] * sc[2] * inv, o[db][4 * i + 3] * sc[3] * inv)};
                *reinterpret_cast<u32x2_t *>(op + d0) = w;
            }
        }
    }
}

// ------------------------------------------------------------------ launch
hipError_t launch_q8_prep(const Q8Args &a, int d, hipStream_t st)
{
    if (d != QD) return hipErrorInvalidValue;
    const int64_t groups = (a.ntiles + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * a.H));
    hipLaunchKernelGGL(q8_pass1_kernel, grid, dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(q8_reduce_kernel, dim3((unsigned)(a.seq.S * a.H)), dim3(QD), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(q8_pass3_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

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
