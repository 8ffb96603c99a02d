// Shared main loop of the projection kernels (qkv_proj.hip, out_proj.hip):
// one 8-wave workgroup computes C^T = W . X^T for 256 rows of X (tokens) and
// 2 x D rows of W (output features) over K, on v_mfma_f32_32x32x16_bf16.
//
// Wave w owns the 64 tokens 64*(w%4) .. +63 and the D features D*(w/4) .. +D-1
// of the tile; its accumulator acc[tb][fb] (tb: 32-token block, fb: 32-feature
// block) gives lane l token 32 tb + l%32 and, in register r, feature
// 32 fb + 8 (r/4) + 4 (l/32) + r%4: runs of four consecutive features, every
// feature of a token held by lanes l and l^32.
//
// K is walked in 32-element slabs (64-byte rows) through four LDS stages
// (2 x 16 KB each for D = 128) filled straight from global memory by
// buffer_load_dwordx4 ... lds, three slabs ahead of the matrix cores, with one
// wait and one barrier per slab.  Slab rows are XOR swizzled per 16-byte chunk
// so the fragment reads of 16 lanes cover all 64 LDS banks.
#pragma once

#include "attn_common.h"

namespace h3 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kGemmBM = 256;     // X rows (tokens) per workgroup
constexpr int kGemmBK = 32;      // K elements per slab
constexpr int kGemmStages = 4;
constexpr int kGemmWaves = 8;


// Direct-to-LDS fill of a slab of ROWS rows x 4 16-byte chunks (32 bf16), the
// rows `row_bytes` apart in global memory, shared by the workgroup's waves.
// Wave instruction i writes one 1 KB piece of 16 rows; lane L the 16 bytes at
// offset 16 L, i.e. row L / 4 of the piece, physical chunk L % 4, which holds
// logical chunk (L % 4) ^ swz(row).
template <int ROWS>
struct SlabFill {
    static constexpr int PER_WAVE = ROWS / (16 * kGemmWaves);
    static_assert(PER_WAVE * 16 * kGemmWaves == ROWS, "slab rows split evenly over the waves");
    uint32_t voff[PER_WAVE];
    __device__ __forceinline__ void init(int wave, int lane, uint32_t row_bytes)
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int row = (wave * PER_WAVE + i) * 16 + lane / 4;
            voff[i] = (uint32_t)row * row_bytes + (uint32_t)(((lane % 4) ^ swz<4>(row)) * 16);
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
__device__ __forceinline__ uint32_t slab_off(int r, int c) { return (uint32_t)(r * 4 + (c ^ swz<4>(r))) * 16u; }

// The LDS stages of one workgroup: x slabs of kGemmBM rows, W slabs of 2 D rows.
template <int D>
struct GemmStages {
    uint16_t *x[kGemmStages];
    uint16_t *w[kGemmStages];
};

// acc += (W rows of `wrs`) . (X rows of `xrs`)^T over nk slabs.  xrs / wrs
// cover the workgroup's X rows (xrow bytes apart) and W rows (wrow bytes
// apart); rows past their ranges read as zeros.  Every wave of the workgroup
// calls it with the same nk.  On return no fill is in flight.
template <int D>
__device__ __forceinline__ void gemm_mainloop(f32x16 (&acc)[2][D / 32], const GemmStages<D> &st,
                                              __amdgpu_buffer_rsrc_t xrs, uint32_t xrow,
                                              __amdgpu_buffer_rsrc_t wrs, uint32_t wrow, int nk, int wave, int lane)
{
    constexpr int FB = D / 32;
    constexpr int ST = kGemmStages;
    constexpr int FILLS = SlabFill<kGemmBM>::PER_WAVE + SlabFill<2 * D>::PER_WAVE;   // per wave per slab
    const int m = lane & 31, hh = lane >> 5;
    const int tw = wave & 3, fw = wave >> 2;
    SlabFill<kGemmBM> xfill;
    SlabFill<2 * D> wfill;
    xfill.init(wave, lane, xrow);
    wfill.init(wave, lane, wrow);

    // per-lane fragment offsets: B = x rows (tokens), A = W rows (features)
    uint32_t xo[2][2], wo[FB][2];
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) xo[tb][ss] = slab_off(64 * tw + 32 * tb + m, 2 * ss + hh);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) wo[fb][ss] = slab_off(D * fw + 32 * fb + m, 2 * ss + hh);
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) acc[tb][fb] = (f32x16){};

    auto fill = [&](int kk, int j) __attribute__((always_inline)) {
        xfill.load(xrs, (uint32_t)(kk * kGemmBK * 2), st.x[j], wave);
        wfill.load(wrs, (uint32_t)(kk * kGemmBK * 2), st.w[j], wave);
    };
    auto compute = [&](int j) __attribute__((always_inline)) {
        const char *lx = reinterpret_cast<const char *>(st.x[j]);
        const char *lw = reinterpret_cast<const char *>(st.w[j]);
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            bf16x8_t af[FB], bx[2];
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) af[fb] = *reinterpret_cast<const bf16x8_t *>(lw + wo[fb][ss]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) bx[tb] = *reinterpret_cast<const bf16x8_t *>(lx + xo[tb][ss]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int fb = 0; fb < FB; ++fb)
                    acc[tb][fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fb], bx[tb], acc[tb][fb], 0, 0, 0);
        }
    };
    // Step kk computes slab kk.  It starts once this wave's fills of slab kk
    // have landed (the 2 fill groups issued after them, for the next slabs,
    // may still be in flight) and every wave has passed the barrier; the same
    // barrier guarantees that every wave's fragment reads of slab kk-1 are
    // complete (lgkmcnt 0), so slab kk+3 can go into that stage.  Every step
    // issues a fill, slab 0 again once no slab is left (into a stage nobody
    // reads any more), so the wait count is the same constant at every step and
    // the steady-state loop has no branches: with the stages named at compile
    // time the compiler then sees which stage each fill in flight targets and
    // does not wait for all of them before reading.
    auto step = [&](int j, int knext) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((ST - 2) * FILLS));
        barrier_only();
        fill(knext < nk ? knext : 0, (j + ST - 1) % ST);
        compute(j);
    };
#pragma unroll
    for (int j = 0; j < ST - 1; ++j) fill(j < nk ? j : 0, j);
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
}

// Workgroup -> (token block, feature pair) for nblk token blocks and npair
// feature pairs.  Workgroups are dispatched round-robin over the 8 XCDs; each
// XCD takes every 8th token block and walks groups of G of its token blocks
// pair by pair, so the ~32 workgroups it runs at a time (one per CU) cover G
// token blocks x 32/G feature pairs, which share x and weight slabs through the
// XCD's L2.  A larger G re-reads the weights fewer times (once per group):
// measured on the 125k-token QKV projection (36 feature pairs), G = 8 takes
// 6.94 ms against 7.33 ms for G = 2; the output projection (12 pairs) is
// fastest with G = 2.  Returns false for the padding workgroups of the grid.
template <int G>
__device__ __forceinline__ bool gemm_tile(int64_t nblk, int64_t npair, int &blk, int &pair)
{
    const int x8 = blockIdx.x & 7;
    const int64_t i = blockIdx.x >> 3;
    const int64_t nb_x = (nblk - x8 + 7) / 8;       // this XCD's token blocks: x8 + 8k, k < nb_x
    if (i >= nb_x * npair) return false;
    const int64_t grp = i / (G * npair), r = i % (G * npair);
    const int64_t gsz = min((int64_t)G, nb_x - grp * G);
    pair = (int)(r / gsz);
    blk = x8 + 8 * (int)(grp * G + r % gsz);
    return true;
}

// Grid size for gemm_tile.
inline unsigned gemm_grid(int64_t nblk, int64_t npair) { return (unsigned)(8 * ((nblk + 7) / 8) * npair); }

}  // namespace h3
