// Fused QKV projection + Q/K RMSNorm + RoPE + layout for gfx950.
//
// The GEMMs are the second-largest share of a MiniMax-H3 block after
// attention (about 27% on the page "Buyer Questions: Current Evidence
// Status", question 4), and the page "H3 Runtime Current State" lists the
// attention QKV projection among its tensor-parallel GEMMs and "Fused Q/K
// RMSNorm, RoPE, and layout work" among its owned kernels.  This kernel is
// the projection with that prologue in its epilogue: y = x . W^T on the
// matrix cores, then, still in registers, RMSNorm over each head's d
// features, the norm weight, the RoPE rotation and the head-major store that
// the attention kernel streams.  The projected q and k never go to memory
// unnormalised, and v goes straight into the attention kernel's transposed
// per-tile V layout.
//
// Work decomposition.  One workgroup = 8 waves computes 256 (padded) tokens x
// 2d output features, two consecutive d-feature blocks (heads of q, k or v);
// wave w owns the 64-token tile w%4 of block w/4, i.e. one tile of the
// attention kernel's layout.  Token blocks never straddle sequences (every
// sequence starts at a multiple of 256 padded tokens), rows past a sequence's
// end read as zeros (bounded buffer descriptors) and are stored as zeros.
//
// Matrix-core layout.  C^T = W . X^T on v_mfma_f32_32x32x16_bf16: A = 32
// weight rows (features), B = 32 token rows of x, so the accumulator gives
// lane l token l%32 and 16 features per 32-feature block, in runs of four
// consecutive features.  A head's 128 features of one token are then split
// over lanes l and l^32: the RMSNorm sum of squares is an in-lane sum plus one
// exchange, and every RoPE pair (2j, 2j+1) is inside one lane.
//
// Pipelining.  The model dimension is walked in 32-element slabs through four
// LDS stages (128 KB) filled straight from global memory by
// buffer_load_dwordx4 ... lds, three slabs ahead of the matrix cores; one
// barrier per slab hands a stage back.  Slab rows are 64 bytes, XOR swizzled
// per 16-byte chunk so the fragment reads of 16 lanes cover all 64 banks.
//
// Placement.  Workgroups are dispatched round-robin over the 8 XCDs; each XCD
// takes every 8th token block and walks groups of 2 of its token blocks
// feature-pair by feature-pair, so the ~32 workgroups it runs at a time (one
// per CU) cover 2 token blocks x 16 feature pairs: each x slab is shared by
// 16 of them and each weight slab by 2 through the XCD's L2, and the 1.5 MB x
// block of a token block is reused across 16 feature pairs before it leaves.
//
// What bounds it.  The direct-to-LDS fills: every slab row is a 64-byte
// half cache line of x or W, so the fills issue twice the L2 requests of
// 128-byte rows, and 64-element slabs would leave room for only two 64 KB
// stages (too shallow a prefetch); the LDS fragment reads are not the limit.
#include "h3_internal.h"
#include "attn_common.h"
#include "norm_rope.h"

namespace h3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kProjBM = 256;    // tokens per workgroup
constexpr int kProjBK = 32;     // model-dim elements per pipeline stage (64-byte slab rows)
constexpr int kProjStages = 4;  // LDS stages: fills run 3 slabs ahead (128 KB)
constexpr int kProjNW = 8;      // waves per workgroup
constexpr int kProjGroup = 2;   // token blocks an XCD walks together

// s_waitcnt immediate (gfx9 encoding): vmcnt = n < 64, lgkmcnt = 0, expcnt at its maximum.
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would wait for every direct-to-LDS fill in flight, including those of
// stages that are not read yet.  The caller has already waited for what the
// barrier hands over; the clobber keeps memory accesses on their side of it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Position of token r (0..63) in a transposed V tile (bits 2 and 3 swapped),
// the key order of the attention kernel's P.V operand.
__device__ __forceinline__ int vt_key_pos(int r)
{
    return (r & ~0xC) | ((r >> 1) & 4) | ((r << 1) & 8);
}

// Direct-to-LDS fill of a slab of ROWS rows x CPR 16-byte chunks (CPR * 8
// bf16), the rows `row_bytes` apart in global memory, shared by the
// workgroup's waves.  Wave instruction i writes one 1 KB piece of 64 / CPR
// rows; lane L the 16 bytes at offset 16 L, i.e. row L / CPR of the piece,
// physical chunk L % CPR, which holds logical chunk (L % CPR) ^ swz(row).
template <int ROWS, int CPR, int NW>
struct SlabFill {
    static constexpr int RPK = 64 / CPR;
    static constexpr int PER_WAVE = ROWS / (RPK * NW);
    static_assert(PER_WAVE * RPK * NW == ROWS, "slab rows split evenly over the waves");
    uint32_t voff[PER_WAVE];
    __device__ __forceinline__ void init(int wave, int lane, uint32_t row_bytes)
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int row = (wave * PER_WAVE + i) * RPK + lane / CPR;
            voff[i] = (uint32_t)row * row_bytes + (uint32_t)(((lane % CPR) ^ swz<CPR>(row)) * 16);
        }
    }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, uint32_t soff, uint16_t *lds, int wave) const
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc,
                (__attribute__((address_space(3))) void *)(reinterpret_cast<char *>(lds) +
                                                           (wave * PER_WAVE + i) * 1024),
                16, voff[i], soff, 0, 0);
    }
};

// Byte offset in a slab of logical chunk c of row r.
template <int CPR>
__device__ __forceinline__ uint32_t slab_off(int r, int c) { return (uint32_t)(r * CPR + (c ^ swz<CPR>(r))) * 16u; }

// D: head dim; BK: model-dim elements per slab (32 or 64); ST: LDS stages
// (fills run ST-1 slabs ahead); NW: waves, NW/2 per feature block, each
// owning 256 / (NW/2) tokens of it.
template <int D, int BK, int ST, int NW>
__global__ __launch_bounds__(64 * NW, 1) void qkv_proj_kernel(ProjArgs a)
{
    constexpr int FB = D / 32;                       // 32-feature blocks per head
    constexpr int WROWS = 2 * D;                     // weight rows (features) per workgroup
    constexpr int CPR = BK / 8;
    constexpr int TWG = NW / 2;                      // waves per feature block
    constexpr int TPW = kProjBM / TWG;               // tokens per wave
    constexpr int TB = TPW / 32;                     // 32-token blocks per wave
    constexpr int TILES = TPW / 64;                  // 64-token tiles per wave
    constexpr int FILLS = SlabFill<kProjBM, CPR, NW>::PER_WAVE + SlabFill<WROWS, CPR, NW>::PER_WAVE;
    static_assert(ST >= 2 && ST <= 5, "2 to 5 stages");
    __shared__ __attribute__((aligned(16))) uint16_t lx0[kProjBM * BK], lx1[kProjBM * BK], lx2[kProjBM * BK],
        lx3[kProjBM * BK], lx4[kProjBM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t lw0[WROWS * BK], lw1[WROWS * BK], lw2[WROWS * BK],
        lw3[WROWS * BK], lw4[WROWS * BK];
    auto xs = [&](int j) __attribute__((always_inline)) {
        return j == 0 ? lx0 : j == 1 ? lx1 : j == 2 ? lx2 : j == 3 ? lx3 : lx4;
    };
    auto wsl = [&](int j) __attribute__((always_inline)) {
        return j == 0 ? lw0 : j == 1 ? lw1 : j == 2 ? lw2 : j == 3 ? lw3 : lw4;
    };

    // ---- tile: (token block b, feature pair F2); this wave's feature block
    // F = 2 F2 + wave/4 = which * H + head
    const int H = a.H;
    const int64_t nfb = 3 * (int64_t)H, npair = (nfb + 1) / 2;
    const int x8 = blockIdx.x & 7;
    const int64_t i = blockIdx.x >> 3;
    const int nb_x = (a.nblk - x8 + 7) / 8;          // this XCD's token blocks: x8 + 8k, k < nb_x
    if (i >= (int64_t)nb_x * npair) return;
    const int64_t grp = i / (kProjGroup * npair), r = i % (kProjGroup * npair);
    const int gsz = min(kProjGroup, nb_x - (int)grp * kProjGroup);
    const int F2 = (int)(r / gsz);
    const int b = x8 + 8 * ((int)grp * kProjGroup + (int)(r % gsz));

    int s, j0, valid0;
    tile_seq(a.seq.cu, a.seq.off, a.seq.S, 4 * b, s, j0, valid0);
    const int n_s = a.seq.cu[s + 1] - a.seq.cu[s];
    const int rows_blk = min(n_s - 64 * j0, kProjBM);   // >= 1: blocks exist only where tokens do

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, hh = lane >> 5;
    const int tw = wave % TWG, fw = wave / TWG;      // token group, feature block of this wave
    const int F = 2 * F2 + fw;
    const int which = F / H, head = F % H;
    const int nf_blk = (int)min((int64_t)2, nfb - 2 * F2);   // feature blocks that exist (the last pair may hold one)

    // ---- buffer descriptors: this block's rows of x, this pair's rows of W
    const uint32_t xrow = (uint32_t)(a.x_stride * 2), wrow = (uint32_t)(a.model_dim * 2);
    const uint16_t *xbase = a.x + ((int64_t)a.seq.cu[s] + 64 * j0) * a.x_stride;
    const uint16_t *wbase = a.w + (int64_t)2 * F2 * D * a.model_dim;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(xbase), 0, (int)((uint32_t)(rows_blk - 1) * xrow + wrow), kBufferFlags);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(wbase), 0, (int)((uint32_t)(nf_blk * D) * wrow), kBufferFlags);
    SlabFill<kProjBM, CPR, NW> xfill;
    SlabFill<WROWS, CPR, NW> wfill;
    xfill.init(wave, lane, xrow);
    wfill.init(wave, lane, wrow);

    // per-lane fragment offsets: B = x rows (tokens), A = W rows (features)
    constexpr int KS = BK / 16;                      // matrix-core k-steps per slab
    uint32_t xo[TB][KS], wo[FB][KS];
#pragma unroll
    for (int ss = 0; ss < KS; ++ss) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) xo[tb][ss] = slab_off<CPR>(TPW * tw + 32 * tb + m, 2 * ss + hh);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) wo[fb][ss] = slab_off<CPR>(D * fw + 32 * fb + m, 2 * ss + hh);
    }

    f32x16 acc[TB][FB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) acc[tb][fb] = (f32x16){};

    auto fill = [&](int kk, uint16_t *lx, uint16_t *lw) __attribute__((always_inline)) {
        xfill.load(xrs, (uint32_t)(kk * BK * 2), lx, wave);
        wfill.load(wrs, (uint32_t)(kk * BK * 2), lw, wave);
    };
    auto compute = [&](const uint16_t *lx, const uint16_t *lw) __attribute__((always_inline)) {
#pragma unroll
        for (int ss = 0; ss < KS; ++ss) {
            bf16x8 af[FB], bx[TB];
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
                af[fb] = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(lw) + wo[fb][ss]);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
                bx[tb] = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(lx) + xo[tb][ss]);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int fb = 0; fb < FB; ++fb)
                    acc[tb][fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fb], bx[tb], acc[tb][fb], 0, 0, 0);
        }
    };
    const int nk = a.model_dim / BK;
    // Step kk computes slab kk.  It starts once this wave's fills of slab kk
    // have landed (the ST-2 fill groups issued after them, for the next slabs,
    // may still be in flight) and every wave has passed the barrier; the same
    // barrier guarantees that every wave's fragment reads of slab kk-1 are
    // complete (lgkmcnt 0), so slab kk+ST-1 can go into that stage.  Every step
    // issues a fill, slab 0 again once no slab is left (into a stage nobody
    // reads any more), so the wait count is the same constant at every step and
    // the steady-state loop has no branches: with the stages named at compile
    // time the compiler then sees which stage each fill in flight targets and
    // does not wait for all of them before reading.
    auto step = [&](int j, int knext) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((ST - 2) * FILLS));
        barrier_only();
        fill(knext < nk ? knext : 0, xs((j + ST - 1) % ST), wsl((j + ST - 1) % ST));
        compute(xs(j), wsl(j));
    };
#pragma unroll
    for (int j = 0; j < ST - 1; ++j) fill(j < nk ? j : 0, xs(j), wsl(j));
    int kk = 0;
    for (; kk + ST <= nk; kk += ST) {
#pragma unroll
        for (int j = 0; j < ST; ++j) step(j, kk + j + ST - 1);
    }
#pragma unroll
    for (int j = 0; j < ST - 1; ++j)
        if (kk + j < nk) step(j, kk + j + ST - 1);
    // no fill may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    if (F >= nfb) return;                            // the missing half of the last pair

    // ---- epilogue: this wave's TILES 64-token tiles, two 32-token blocks each
    const float inv_d = 1.0f / (float)D;
#pragma unroll
    for (int q = 0; q < TILES; ++q) {
        const int gt = 4 * b + TILES * tw + q;
        const int jt = j0 + TILES * tw + q;            // tile index inside the sequence
        const int valid = min(max(n_s - 64 * jt, 0), 64);
        float kn2 = 0.f;
#pragma unroll
        for (int tb2 = 0; tb2 < 2; ++tb2) {
            const f32x16 *ac = acc[2 * q + tb2];
            const int t = 32 * tb2 + m;
            const bool ok = t < valid;
            const int64_t tok = (int64_t)a.seq.cu[s] + 64 * jt + t;
            const int64_t prow = (int64_t)a.seq.off[s] + 64 * jt + t;
            if (which < 2) {
                float ss = 0.f;
#pragma unroll
                for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) ss = fmaf(ac[fb][e], ac[fb][e], ss);
                ss = row_sum2(ss);
                const float rs = rsqrtf(fmaf(ss, inv_d, a.eps));
                const float *wn = a.norm_w + (int64_t)(which * H + head) * D;
                uint16_t *dst = (which ? a.khat : a.qhat) + head * a.out_hstride +
                                (a.natural ? tok : prow) * a.out_tstride;
                const float mult = which ? 1.0f : a.q_mult;
                float kss = 0.f;
#pragma unroll
                for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int f0 = 32 * fb + 8 * g + 4 * hh;
                        const f32x4_t w4 = *reinterpret_cast<const f32x4_t *>(wn + f0);
                        f32x4_t cs = {1.f, 0.f, 1.f, 0.f};
                        if (ok) cs = *reinterpret_cast<const f32x4_t *>(a.rope + tok * D + f0);
                        const float x0 = ac[fb][4 * g] * rs * w4[0], x1 = ac[fb][4 * g + 1] * rs * w4[1];
                        const float x2 = ac[fb][4 * g + 2] * rs * w4[2], x3 = ac[fb][4 * g + 3] * rs * w4[3];
                        const float y0 = (x0 * cs[0] - x1 * cs[1]) * mult, y1 = (x0 * cs[1] + x1 * cs[0]) * mult;
                        const float y2 = (x2 * cs[2] - x3 * cs[3]) * mult, y3 = (x2 * cs[3] + x3 * cs[2]) * mult;
                        u32x2 o = {pack2(y0, y1), pack2(y2, y3)};
                        if (!ok) o = (u32x2){0u, 0u};
                        if (which) {
#pragma unroll
                            for (int e = 0; e < 2; ++e) {
                                const float lo = __uint_as_float(o[e] << 16), hi = __uint_as_float(o[e] & 0xffff0000u);
                                kss = fmaf(lo, lo, fmaf(hi, hi, kss));
                            }
                        }
                        if (ok || !a.natural) *reinterpret_cast<u32x2 *>(dst + f0) = o;
                    }
                }
                if (which) kn2 = fmaxf(kn2, row_sum2(kss));
            } else {
                uint16_t *vt = a.vt + ((int64_t)head * a.ntiles + gt) * (D * kTile);
                const int p = vt_key_pos(t);
#pragma unroll
                for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int f0 = 32 * fb + 8 * g + 4 * hh;
                        u32x2 o = {pack2(ac[fb][4 * g], ac[fb][4 * g + 1]), pack2(ac[fb][4 * g + 2], ac[fb][4 * g + 3])};
                        if (!ok) o = (u32x2){0u, 0u};
                        if (a.natural) {
                            if (ok)
                                *reinterpret_cast<u32x2 *>(a.vt + tok * a.out_tstride + head * a.out_hstride + f0) = o;
                        } else {
                            vt[(f0 + 0) * kTile + p] = (uint16_t)(o[0] & 0xffffu);
                            vt[(f0 + 1) * kTile + p] = (uint16_t)(o[0] >> 16);
                            vt[(f0 + 2) * kTile + p] = (uint16_t)(o[1] & 0xffffu);
                            vt[(f0 + 3) * kTile + p] = (uint16_t)(o[1] >> 16);
                        }
                    }
                }
            }
        }
        if (which == 1 && !a.natural) {
#pragma unroll
            for (int msk = 16; msk >= 1; msk >>= 1) kn2 = fmaxf(kn2, __shfl_xor(kn2, msk));
            if (lane == 0) a.knorm[(int64_t)head * a.ntiles + gt] = sqrtf(kn2);
        }
    }
}

// Explicit instantiations: the host pass does not emit the launch stub of an
// instantiation that is only named inside the launcher's branches.
template __global__ void qkv_proj_kernel<64, kProjBK, kProjStages, kProjNW>(ProjArgs);
template __global__ void qkv_proj_kernel<128, kProjBK, kProjStages, kProjNW>(ProjArgs);

hipError_t launch_qkv_proj(const ProjArgs &a, int d, hipStream_t st)
{
    const int64_t per_xcd = (a.nblk + 7) / 8;
    const dim3 grid((unsigned)(8 * per_xcd * ((3 * (int64_t)a.H + 1) / 2)));
    if (d == 128)
        hipLaunchKernelGGL((qkv_proj_kernel<128, kProjBK, kProjStages, kProjNW>), grid, dim3(64 * kProjNW), 0, st, a);
    else
        hipLaunchKernelGGL((qkv_proj_kernel<64, kProjBK, kProjStages, kProjNW>), grid, dim3(64 * kProjNW), 0, st, a);
    return hipGetLastError();
}

}  // namespace h3
