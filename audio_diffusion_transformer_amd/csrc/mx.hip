// MXFP4 attention for gfx950: OCP microscaling FP4 (e2m1 codes with one E8M0
// power-of-two scale per 32 elements) on the CDNA4 scaled matrix cores,
// v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation.
//
// Role: the FP4 attention variant.  The FastVideo commit page for
// docs/getting_started notes an FP4 attention switch that is faster, changes
// the output and stays off by default; "H3 Runtime Current State" lists Sage3
// among the approximate backends ("Implemented And Validated") and asks that
// they stay quality-gated ("Quality Work Remaining").  The FP4 kernels named
// there target NVIDIA parts; this path takes the OCP MX format that the CDNA4
// FP4 matrix cores read natively, block scales applied inside the instruction.
//
// Steps (d = 128):
//  pass 1  per 64-token tile and head: RMSNorm + RoPE of q and k in fp32;
//          qhat' = qhat * softmax scale * log2 e -> MXFP4 with blocks of 32
//          channels (the scores of its codes are in log2 units); per-channel
//          partial sums of khat.
//  reduce  per (sequence, head): mean of khat over the sequence, fixed order.
//  pass 3  khat - mean -> MXFP4 along the channels, the tile's rows stored in
//          the key order of the score operand; raw v -> MXFP4 with blocks of
//          32 keys per channel, transposed per tile.
//  attention  S^T = K4 . Q4^T (scaled FP4 MFMA, both block scales in the
//          instruction); online softmax in base 2 with the lazy running max of
//          the quantised path (p <= 2), the max taking the tile maximum's own
//          value when it moves, so that key's p = 2^(s - m) is exactly 1 (the
//          power-of-two scale rule below is discontinuous there); the 32
//          probabilities a lane holds are
//          keys 32h..32h+31 of the tile (that is what the K row order buys) and
//          form one MX block: scale from their largest value, e2m1 codes from
//          the hardware conversion; O^T += V4^T . P4^T; the row sum l from one
//          more MFMA against e2m1 ones, so it sums the quantised P that weight
//          V; o = O / l.
//
// Block scale (OCP MX): X = floor(log2 amax) - 2, limited to [-126, 127], and
// X = 0 for an all-zero block.  Its E8M0 byte X + 127 is, for a normal fp32
// amax, the exponent field minus 2; codes are e2m1(x / 2^X), rounded to
// nearest even and saturated at 6 by v_cvt_scalef32_pk_fp4_f32.
#include <type_traits>

#include "h3_internal.h"
#include "norm_rope.h"
#include "attn_common.h"
#include "h3_checked.h"

namespace h3 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int MD = 128;                      // head dim of the FP4 path
constexpr int kRowBytes = MD / 2;            // FP4 bytes of one token row
constexpr int kTileBytes = kTile * MD / 2;   // FP4 bytes of a K tile or a V^T tile
constexpr int kScaleBytes = 256;             // scale bytes of a K tile or a V^T tile
constexpr float kMxLazy = 1.0f;              // running max raised when a tile exceeds it by > 1 (log2 units)

// E8M0 byte of the scale of an MX block whose largest magnitude is amax.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax)
{
    const int e = (int)(__float_as_uint(amax) >> 23);
    return amax > 0.f ? (uint32_t)max(e - 2, 1) : 127u;
}
__device__ __forceinline__ float mx_scale_value(uint32_t byte) { return __uint_as_float(byte << 23); }

// This lane's index (0..63) from the hardware lane counter, opaque to the
// compiler so that it is computed where it is used rather than kept live (and
// spilled) from the kernel start.
__device__ __forceinline__ int lane_here()
{
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Eight values -> eight e2m1 codes of x / scale (value i in nibble i).  The
// four conversions write the word's four bytes, so its starting value is
// never read; passing a dead input avoids materialising a zero.
__device__ __forceinline__ uint32_t fp4x8(const float *y, float scale)
{
    uint32_t w = __float_as_uint(y[0]);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], scale, 3);
    return w;
}

// Row of key r (0..63) in a stored K tile.  Row 32 kb + i is the score
// operand's A row i of key block kb; it holds key 32 ((i >> 2) & 1) + 16 kb +
// 4 (i >> 3) + (i & 3), so that the accumulator gives lane half h the keys
// 32h..32h+31 (register r of block kb: key 32h + 16 kb + r).
__device__ __forceinline__ int mx_key_row(int r)
{
    return (((r >> 4) & 1) << 5) | (((r >> 2) & 3) << 3) | (((r >> 5) & 1) << 2) | (r & 3);
}
// Byte of a K tile's scales for tile row P and channel block cb: lane
// L = 32 h + m reads word L (consecutive lanes, consecutive words: 4-byte LDS
// reads of a word per lane are conflict-free only that way), whose byte
// 2 kb + st is its A scale in score MFMA (key block kb, channel step st).
__device__ __forceinline__ int mx_kscale_pos(int P, int cb)
{
    return 4 * ((P & 31) + 32 * (cb & 1)) + 2 * (P >> 5) + (cb >> 1);
}
// Byte of a V tile's scales for channel ch and key block b: lane L = 32 h + m
// reads word L, whose byte db is its A scale in the P.V MFMA of channel block
// db.
__device__ __forceinline__ int mx_vscale_pos(int ch, int b)
{
    return 4 * ((ch & 31) + 32 * b) + (ch >> 5);
}

// Decode of the XCD-aware (tile, head) numbering of the prologue launches.
__device__ __forceinline__ bool mx_tile_head(int H, int ntiles, int &gt, int &h)
{
    const int b = blockIdx.x;
    gt = 8 * ((b >> 3) / H) + (b & 7);
    h = (b >> 3) % H;
    return gt < ntiles;
}

// ------------------------------------------------------------------ pass 1
__global__ __launch_bounds__(256) void mx_pass1_kernel(MxArgs a)
{
    constexpr int LPR = MD / 8, RPP = 256 / LPR;
    __shared__ float kred[RPP][MD];
    int gt, h;
    if (!mx_tile_head(a.H, a.ntiles, gt, h)) return;
    int s, j, valid;
    tile_seq(a.seq.cu, a.seq.off, a.seq.S, gt, s, j, valid);
    const int t = threadIdx.x, c = t % LPR, rr = t / LPR;
    float wq[8], wk[8], ks[8];
    load_w8(a.norm_w, h, MD, c, wq);
    load_w8(a.norm_w, a.H + h, MD, c, wk);
#pragma unroll
    for (int i = 0; i < 8; ++i) ks[i] = 0.f;
    const int64_t row0 = (int64_t)h * a.Npad + a.seq.off[s] + kTile * j;
#pragma unroll
    for (int pass = 0; pass < kTile / RPP; ++pass) {
        const int r = pass * RPP + rr;
        const bool ok = r < valid;
        const int64_t tok = (int64_t)a.seq.cu[s] + kTile * j + r;
        float cs[8] = {1.f, 0.f, 1.f, 0.f, 1.f, 0.f, 1.f, 0.f};
        if (ok) load_cs8(a.rope, tok, MD, c, cs);
        u32x4_t rq = {0u, 0u, 0u, 0u}, rk = rq;
        if (ok) {
            rq = *reinterpret_cast<const u32x4_t *>(a.q + tok * a.q_stride + h * MD + 8 * c);
            rk = *reinterpret_cast<const u32x4_t *>(a.k + tok * a.k_stride + h * MD + 8 * c);
        }
        float x[8], y[8];
        unpack8(rq, x);
        norm_rope8<LPR>(x, wq, cs, 1.0f / MD, a.eps, y);
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            y[i] = ok ? y[i] * a.q_mult : 0.f;
            am = fmaxf(am, fabsf(y[i]));
        }
        // the block of 32 channels is spread over the 4 aligned lanes c..c^3
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        const uint32_t byte = mx_scale_byte(am);
        *reinterpret_cast<uint32_t *>(a.qx + (row0 + r) * kRowBytes + 4 * c) = fp4x8(y, mx_scale_value(byte));
        if ((c & 3) == 0) a.qxs[(row0 + r) * (MD / 32) + (c >> 2)] = (uint8_t)byte;
        unpack8(rk, x);
        norm_rope8<LPR>(x, wk, cs, 1.0f / MD, a.eps, y);
        if (ok) {
#pragma unroll
            for (int i = 0; i < 8; ++i) ks[i] += y[i];
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) kred[rr][8 * c + i] = ks[i];
    __syncthreads();
    if (t < MD) {
        float sum = 0.f;
        for (int g = 0; g < RPP; ++g) sum += kred[g][t];
        a.ksum[((int64_t)h * a.ntiles + gt) * MD + t] = sum;
    }
}

// ------------------------------------------------------------------ reduce
// One workgroup per (sequence, head): thread (g, c) sums the per-tile
// partials of channel c for tiles g, g+8, ...; the 8 groups are combined in
// group order, so the result does not depend on timing.
constexpr int kMxReduceGroups = 8;
__global__ __launch_bounds__(kMxReduceGroups * MD) void mx_reduce_kernel(MxArgs a)
{
    __shared__ float rs[kMxReduceGroups][MD];
    const int s = blockIdx.x / a.H, h = blockIdx.x % a.H;
    const int c = threadIdx.x % MD, g = threadIdx.x / MD;
    const int n = a.seq.cu[s + 1] - a.seq.cu[s];
    const int t0 = a.seq.off[s] / kTile, nt = (n + kTile - 1) / kTile;
    float sum = 0.f;
    for (int i = g; i < nt; i += kMxReduceGroups) sum += a.ksum[((int64_t)h * a.ntiles + t0 + i) * MD + c];
    rs[g][c] = sum;
    __syncthreads();
    if (g == 0) {
        for (int k = 1; k < kMxReduceGroups; ++k) sum += rs[k][c];
        a.kmean[((int64_t)s * a.H + h) * MD + c] = n > 0 ? sum / (float)n : 0.f;
    }
}

// ------------------------------------------------------------------ pass 3
__global__ __launch_bounds__(256) void mx_pass3_kernel(MxArgs a)
{
    constexpr int LPR = MD / 8, RPP = 256 / LPR;
    constexpr int VW = MD / 2 + 1;   // LDS words per v row; odd, so rows 32 apart use other banks
    __shared__ uint32_t lv[kTile * VW];
    int gt, h;
    if (!mx_tile_head(a.H, a.ntiles, gt, h)) return;
    int s, j, valid;
    tile_seq(a.seq.cu, a.seq.off, a.seq.S, gt, s, j, valid);
    const int t = threadIdx.x, c = t % LPR, rr = t / LPR;
    float wk[8], km[8];
    load_w8(a.norm_w, a.H + h, MD, c, wk);
    load_w8(a.kmean, (int64_t)s * a.H + h, MD, c, km);
    const int64_t row0 = (int64_t)h * a.Npad + a.seq.off[s] + kTile * j;
    const int64_t tile = (int64_t)h * a.ntiles + gt;
#pragma unroll
    for (int pass = 0; pass < kTile / RPP; ++pass) {
        const int r = pass * RPP + rr;
        const bool ok = r < valid;
        const int64_t tok = (int64_t)a.seq.cu[s] + kTile * j + r;
        float cs[8] = {1.f, 0.f, 1.f, 0.f, 1.f, 0.f, 1.f, 0.f};
        if (ok) load_cs8(a.rope, tok, MD, c, cs);
        u32x4_t rk = {0u, 0u, 0u, 0u}, rv = rk;
        if (ok) {
            rk = *reinterpret_cast<const u32x4_t *>(a.k + tok * a.k_stride + h * MD + 8 * c);
            rv = *reinterpret_cast<const u32x4_t *>(a.v + tok * a.v_stride + h * MD + 8 * c);
        }
        float x[8], y[8];
        unpack8(rk, x);
        norm_rope8<LPR>(x, wk, cs, 1.0f / MD, a.eps, y);
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            y[i] = ok ? y[i] - km[i] : 0.f;
            am = fmaxf(am, fabsf(y[i]));
        }
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        const uint32_t byte = mx_scale_byte(am);
        const int P = mx_key_row(r);
        *reinterpret_cast<uint32_t *>(a.kx + (row0 + P) * kRowBytes + 4 * c) = fp4x8(y, mx_scale_value(byte));
        if ((c & 3) == 0) a.kxs[tile * kScaleBytes + mx_kscale_pos(P, c >> 2)] = (uint8_t)byte;
#pragma unroll
        for (int i = 0; i < 4; ++i) lv[r * VW + 4 * c + i] = rv[i];
    }
    __syncthreads();
    // V: thread t takes channel t/2 and key block t%2 (32 tokens) of the tile
    const int ch = t >> 1, b = t & 1;
    float vv[32], am = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t w = lv[(32 * b + i) * VW + (ch >> 1)];
        vv[i] = (ch & 1) ? bf16hi(w) : bf16lo(w);
        am = fmaxf(am, fabsf(vv[i]));
    }
    const uint32_t byte = mx_scale_byte(am);
    const float sc = mx_scale_value(byte);
    const u32x4_t o = {fp4x8(vv, sc), fp4x8(vv + 8, sc), fp4x8(vv + 16, sc), fp4x8(vv + 24, sc)};
    *reinterpret_cast<u32x4_t *>(a.vxt + (tile * MD + ch) * 32 + 16 * b) = o;
    a.vxs[tile * kScaleBytes + mx_vscale_pos(ch, b)] = (uint8_t)byte;
}

// -------------------------------------------------------- diagnostic export
__device__ __forceinline__ uint8_t nibble(const uint8_t *p, int i) { return (p[i >> 1] >> (4 * (i & 1))) & 15; }

__global__ __launch_bounds__(256) void mx_export_kernel(MxExportArgs a)
{
    int gt, h;
    if (!mx_tile_head(a.H, a.ntiles, gt, h)) return;
    int s, j, valid;
    tile_seq(a.seq.cu, a.seq.off, a.seq.S, gt, s, j, valid);
    if (valid == 0) return;
    const int64_t row0 = (int64_t)h * a.Npad + a.seq.off[s] + kTile * j;
    const int64_t tile = (int64_t)h * a.ntiles + gt;
    const uint8_t *vt = a.vxt + tile * kTileBytes;
    for (int e = threadIdx.x; e < valid * MD; e += 256) {
        const int r = e / MD, c = e % MD;
        const int64_t tok = (int64_t)a.seq.cu[s] + kTile * j + r;
        const int64_t dst = (tok * a.H + h) * MD + c;
        const int P = mx_key_row(r);
        a.q_codes[dst] = nibble(a.qx + (row0 + r) * kRowBytes, c);
        a.k_codes[dst] = nibble(a.kx + (row0 + P) * kRowBytes, c);
        a.v_codes[dst] = nibble(vt + c * 32, r);
        if ((c & 31) == 0) {
            const int64_t xd = (tok * a.H + h) * (MD / 32) + (c >> 5);
            a.q_exp[xd] = a.qxs[(row0 + r) * (MD / 32) + (c >> 5)];
            a.k_exp[xd] = a.kxs[tile * kScaleBytes + mx_kscale_pos(P, c >> 5)];
        }
    }
    for (int e = threadIdx.x; e < 2 * MD; e += 256) {
        const int b = e / MD, ch = e % MD;
        if (32 * b < valid)
            a.v_exp[((int64_t)(a.vblk_pre[s] + 2 * j + b) * a.H + h) * MD + ch] =
                a.vxs[tile * kScaleBytes + mx_vscale_pos(ch, b)];
    }
}

// --------------------------------------------------------------- attention
// One workgroup = 4 waves x 32 query rows of one (sequence, head), three
// workgroups per CU (168 VGPRs): the step's vector work (exp2, FP4 packing) and
// matrix work alternate inside a wave, and the third wave per SIMD fills more of
// the gaps.  The FP4 K tile (64 rows x 64 bytes), the FP4 V^T tile (128 channel
// rows x 32 bytes) and their 256 scale bytes each are filled straight into a
// ring of three LDS buffers by buffer_load ... lds, two tiles ahead: each step
// reads its K fragments, computes the scores and P, then reads its V fragments
// (late, to keep them out of the register peak), issues the fill of the tile
// after next, and at its end waits only for the next tile's fill (three loads
// per wave stay in flight).
__global__ __launch_bounds__(256, 3) void attn_mx_kernel(MxAttnArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t lk0[kTileBytes], lk1[kTileBytes], lk2[kTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lv0[kTileBytes], lv1[kTileBytes], lv2[kTileBytes];
    __shared__ __attribute__((aligned(16))) uint32_t lks0[kScaleBytes / 4], lks1[kScaleBytes / 4],
        lks2[kScaleBytes / 4];
    __shared__ __attribute__((aligned(16))) uint32_t lvs0[kScaleBytes / 4], lvs1[kScaleBytes / 4],
        lvs2[kScaleBytes / 4];

    const int b = blockIdx.x;
    int si = 0;
    while (b >= a.item_pre[si + 1]) ++si;
    const int rem = b - a.item_pre[si];
    const int nqb = a.seq_nqb[si];
    const int head = rem / nqb, qb = rem % nqb;
    const int n = a.seq_n[si];
    const int off = a.seq_off[si];
    const int64_t ntiles = a.Npad / kTile;
    const int nt = (n + kTile - 1) / kTile;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    int m = lane & 31, hh = lane >> 5;    // re-derived before the tail loop
    const int q0 = qb * kBlockM + wave * 32;
    H3_CHECK(si < a.nseq && head < a.H && qb < nqb, kCheckItem);
    H3_CHECK(off + q0 + 32 <= a.Npad, kCheckRows);

    // Q row q0 + m: channels 64 st + 32 hh .. +31 of step st (16 bytes each);
    // the scale word shifted so that bytes 0 and 2 are blocks hh and 2 + hh.
    const int64_t qrow = (int64_t)head * a.Npad + off + q0 + m;
    const i32x4 qf0 = *reinterpret_cast<const i32x4 *>(a.qx + qrow * kRowBytes + 16 * hh);
    const i32x4 qf1 = *reinterpret_cast<const i32x4 *>(a.qx + qrow * kRowBytes + 32 + 16 * hh);
    const uint32_t qsc = *reinterpret_cast<const uint32_t *>(a.qxs + qrow * (MD / 32)) >> (8 * hh);

    TileFill<kTile, 4> kfill;     // K rows: 64 bytes
    TileFill<MD, 2> vfill;        // V^T rows: 32 bytes
    kfill.init(wave, lane);
    vfill.init(wave, lane);
    const int64_t t0 = (int64_t)head * ntiles + off / kTile;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.kx + ((int64_t)head * a.Npad + off) * kRowBytes), 0, nt * kTileBytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.vxt + t0 * kTileBytes), 0, nt * kTileBytes, kBufferFlags);
    // Scale bytes: waves 0 and 2 copy the K tile's, waves 1 and 3 the V tile's
    // (the same bytes land twice), one dword per lane.
    const bool vside = wave & 1;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>((vside ? a.vxs : a.kxs) + t0 * kScaleBytes), 0, nt * kScaleBytes, kBufferFlags);
    auto fill = [&](int jj, void *kd, void *vd, uint32_t *ksd, uint32_t *vsd) {
        H3_CHECK(jj >= 0 && jj < nt, kCheckFillTile);
        H3_JITTER(wave, jj, 0);
        kfill.load(krs, (uint32_t)(jj * kTileBytes), kd, wave);
        vfill.load(vrs, (uint32_t)(jj * kTileBytes), vd, wave);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (__attribute__((address_space(3))) void *)(vside ? vsd : ksd),
                                                 4, 4 * lane, jj * kScaleBytes, 0, 0);
    };

    f32x16 o0 = {}, o1 = {}, o2 = {}, o3 = {};
    // Row sum on the half-size matrix core (16 x 16 x 128, a 4-register
    // accumulator): its B operand is the P operand as it stands, read as lane L
    // = column L % 16, keys 32 (L / 16) .. +31, so column j holds queries j and
    // j + 16.  A row 0 is e2m1 1.0 (code 2) over keys 0-31 and 64-95 (lanes 0
    // and 32), row 1 over keys 32-63 and 96-127 (lanes 17 and 49), the rest 0:
    // register 0 of lane j < 16 sums query j's P, register 1 query j + 16's.
    f32x4 ol = {};
    const int one4 = (lane == 0 || lane == 32 || lane == 17 || lane == 49) ? 0x22222222 : 0;
    const i32x8 ones = {one4, one4, one4, one4, 0, 0, 0, 0};
    float m_run = 0.f;              // running max of the scores (log2 units)
    bool first = true;
    // Every score chain starts from the splat -m_run, so the MFMAs give s - m_run
    // and p = 2^(s - m_run) needs no subtraction.  Rebuilt only when m_run moves;
    // the empty asm keeps the 16 registers live instead of re-materialised.
    f32x16 ninit = {};
    asm volatile("" : "+v"(ninit));

    auto wide = [](i32x4 x) -> i32x8 { return (i32x8){x[0], x[1], x[2], x[3], 0, 0, 0, 0}; };
    // A fragment of the score MFMA for key block kb, channel step st
    auto kfrag = [&](const uint8_t *kl, int kb, int st) -> i32x4 {
        const int row = 32 * kb + m;
        return *reinterpret_cast<const i32x4 *>(kl + row * kRowBytes + 16 * ((2 * st + hh) ^ swz<4>(row)));
    };
    // A fragment of the P.V MFMA for channel block db: keys 32 hh .. +31
    auto vfrag = [&](const uint8_t *vl, int db) -> i32x4 {
        const int row = 32 * db + m;
        return *reinterpret_cast<const i32x4 *>(vl + row * 32 + 16 * (hh ^ swz<2>(row)));
    };

    // One tile: fragments from the current buffers, then the fill of tile
    // jfill (when `more`), scores, the running max, P in FP4, P.V and the row sum.
    auto step = [&](int jj, const uint8_t *kl, const uint8_t *vl, const uint32_t *ksl, const uint32_t *vsl,
                    bool more, void *kn, void *vn, uint32_t *ksn, uint32_t *vsn, bool mask, int jfill) {
        H3_JITTER(wave, jj, 1);
        const i32x4 k00 = kfrag(kl, 0, 0), k10 = kfrag(kl, 1, 0), k01 = kfrag(kl, 0, 1), k11 = kfrag(kl, 1, 1);
        const uint32_t ksw = ksl[lane];

        f32x16 s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wide(k00), wide(qf0), ninit, 4, 4, 0, ksw, 0, qsc);
        f32x16 s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wide(k10), wide(qf0), ninit, 4, 4, 2, ksw, 0, qsc);
        s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wide(k01), wide(qf1), s0, 4, 4, 1, ksw, 2, qsc);
        s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wide(k11), wide(qf1), s1, 4, 4, 3, ksw, 2, qsc);
        if (mask) {
            const int valid = n - jj * kTile;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (32 * hh + r >= valid) s0[r] = -INFINITY;
                if (32 * hh + 16 + r >= valid) s1[r] = -INFINITY;
            }
        }
        // s0, s1 hold s - m_run.  The lane's largest (of its P block) and the row's:
        float lmax = lane_max32(s0, s1);
        const float x = row_max2(lmax);
        const bool need = first || x > kMxLazy;
        // Rare after the first tiles: kept a real branch (the empty asm stops
        // the compiler from if-converting it into 65 multiplies per tile).
        // m_run moves to the tile maximum, m_run + x: the scores lie on the
        // grid of their codes' scales, so x and this sum are exact and the
        // maximum's own p is 2^0 = 1 exactly, which the power-of-two block
        // scale rule needs (it jumps at 1).
        if (__builtin_expect(__any(need), 0)) {
            asm volatile("" ::: "memory");
            const float delta = need ? x : 0.f;
            if (!first) {
                const float alpha = __builtin_amdgcn_exp2f(-delta);
                ol[0] *= alpha;                     // query m of lane m < 16
                // query m + 16 (registers 2, 3 are zero): alpha of lane m + 16
                ol[1] *= __int_as_float(
                    __builtin_amdgcn_ds_bpermute(((lane_here() + 16) & 63) << 2, __float_as_int(alpha)));
                o0 *= alpha;
                o1 *= alpha;
                o2 *= alpha;
                o3 *= alpha;
            }
            m_run += delta;
            s0 -= delta;
            s1 -= delta;
            lmax -= delta;
            ninit = (f32x16){} - m_run;
            asm volatile("" : "+v"(ninit));
            first = false;
        }
        float p[32];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = __builtin_amdgcn_exp2f(s0[r]);
            p[16 + r] = __builtin_amdgcn_exp2f(s1[r]);
        }
        // The block's largest p: v_exp_f32 is non-decreasing (checked on every
        // fp32 input in [-150, 2]; arguments here are <= 1, and below -150 any
        // value gives the same limited scale), so it is exp2 of the largest score.
        const uint32_t pbyte = mx_scale_byte(__builtin_amdgcn_exp2f(lmax));
        const float psc = mx_scale_value(pbyte);
        const i32x8 pf = {(int)fp4x8(p, psc), (int)fp4x8(p + 8, psc), (int)fp4x8(p + 16, psc),
                          (int)fp4x8(p + 24, psc), 0, 0, 0, 0};
        const uint32_t vsw = vsl[lane];
        const i32x4 v0 = vfrag(vl, 0), v1 = vfrag(vl, 1), v2 = vfrag(vl, 2), v3 = vfrag(vl, 3);
        if (more) fill(jfill, kn, vn, ksn, vsn);
        o0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wide(v0), pf, o0, 4, 4, 0, vsw, 0, pbyte);
        o1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wide(v1), pf, o1, 4, 4, 1, vsw, 0, pbyte);
        o2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wide(v2), pf, o2, 4, 4, 2, vsw, 0, pbyte);
        o3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wide(v3), pf, o3, 4, 4, 3, vsw, 0, pbyte);
        ol = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pf, ol, 4, 4, 0, 127u, 0, pbyte);
    };

    // Tile t lives in buffer t % 3.  A fill is three loads per wave (K codes,
    // V codes, one scale block); fills past the last tile repeat the last tile
    // into the free buffer, so every step has the same wait.
    constexpr int kFillLoads = 3;
    // The scheduling fences keep each step's work inside its step (the
    // compiler would otherwise overlap neighbouring steps and spill).
    auto wait_next = [&](auto pending) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(decltype(pending)::value * kFillLoads));
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
    };
    using one_pending = std::integral_constant<int, 1>;
    fill(0, lk0, lv0, lks0, lvs0);
    fill(min(1, nt - 1), lk1, lv1, lks1, lvs1);
    wait_next(one_pending());
    int j = 0;
    for (; j + 3 < nt; j += 3) {
        step(j, lk0, lv0, lks0, lvs0, true, lk2, lv2, lks2, lvs2, false, min(j + 2, nt - 1));
        wait_next(one_pending());
        step(j + 1, lk1, lv1, lks1, lvs1, true, lk0, lv0, lks0, lvs0, false, min(j + 3, nt - 1));
        wait_next(one_pending());
        step(j + 2, lk2, lv2, lks2, lvs2, true, lk1, lv1, lks1, lvs1, false, min(j + 4, nt - 1));
        wait_next(one_pending());
    }
    // The last one to three tiles (buffers 0, 1, 2 in turn; the last tile
    // masked), with the buffer picked at run time: the compiler then waits
    // for every fill before reading LDS, which only costs these few steps,
    // and one copy of the step keeps the code small.
    // The lane's row and half again from the hardware counter: the tail's
    // fragment addresses then need nothing kept live across the main loop.
    {
        const int lr = lane_here();
        m = lr & 31;
        hh = lr >> 5;
    }
    auto kb = [&](int r) -> uint8_t * { return r == 0 ? lk0 : r == 1 ? lk1 : lk2; };
    auto vb = [&](int r) -> uint8_t * { return r == 0 ? lv0 : r == 1 ? lv1 : lv2; };
    auto ksb = [&](int r) -> uint32_t * { return r == 0 ? lks0 : r == 1 ? lks1 : lks2; };
    auto vsb = [&](int r) -> uint32_t * { return r == 0 ? lvs0 : r == 1 ? lvs1 : lvs2; };
    for (int r = 0; j < nt; ++j, ++r) {
        const bool last = j + 1 == nt;
        // a fill only where tile j+2 exists and is not in flight yet (the loop
        // above issued tiles up to j+1)
        const bool more = r == 0 && j + 2 < nt;
        step(j, kb(r), vb(r), ksb(r), vsb(r), more, kb(2), vb(2), ksb(2), vsb(2), last, j + 2);
        if (!last) {
            __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
            barrier_only();
        }
    }
    // no fill may still be writing LDS when the workgroup ends
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));

    // The lane index again: nothing lane-dependent from before the loop has to
    // stay live (or spill) across it.
    const int lane_e = lane_here();
    const int m_e = lane_e & 31, hh_e = lane_e >> 5;
    // row sum of query m: register m / 16 of lane m % 16
    const float l0 = __shfl(ol[0], m_e & 15), l1 = __shfl(ol[1], m_e & 15);
    const float inv = 1.0f / (m_e < 16 ? l0 : l1);
    const int qr = q0 + m_e;
    if (qr < n) {
        uint16_t *op = a.out + ((int64_t)a.seq_cu[si] + qr) * a.o_stride + (int64_t)head * MD;
        const f32x16 *os[4] = {&o0, &o1, &o2, &o3};
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x16 &ov = *os[db];
                const int d0 = 32 * db + 8 * i + 4 * hh_e;
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 w = {pack2(ov[4 * i] * inv, ov[4 * i + 1] * inv),
                                 pack2(ov[4 * i + 2] * inv, ov[4 * i + 3] * inv)};
                *reinterpret_cast<u32x2 *>(op + d0) = w;
            }
        }
    }
}

// ------------------------------------------------------------------ launch
hipError_t launch_mx_prep(const MxArgs &a, int d, hipStream_t st)
{
    if (d != MD) return hipErrorInvalidValue;
    const int64_t groups = (a.ntiles + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * a.H));
    hipLaunchKernelGGL(mx_pass1_kernel, grid, dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mx_reduce_kernel, dim3((unsigned)(a.seq.S * a.H)), dim3(kMxReduceGroups * MD), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(mx_pass3_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

#ifdef H3ATTN_CHECKED
hipError_t mx_checked(uint32_t *or_into, bool clear, uint32_t jitter_seed)
{
    return checked_state_here(or_into, clear, jitter_seed);
}
#endif

hipError_t launch_attn_mx(const MxAttnArgs &a, int d, int64_t nitems, hipStream_t st)
{
    if (d != MD) return hipErrorInvalidValue;
    if (nitems <= 0) return hipSuccess;
    hipLaunchKernelGGL(attn_mx_kernel, dim3((unsigned)nitems), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_mx_export(const MxExportArgs &a, hipStream_t st)
{
    const int64_t groups = (a.ntiles + 7) / 8;
    hipLaunchKernelGGL(mx_export_kernel, dim3((unsigned)(groups * 8 * a.H)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace h3
