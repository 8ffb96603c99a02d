// Flash-style non-causal attention over packed sequences, bf16 MFMA on gfx950.
//
// This is the attention share of a MiniMax-H3 block (about 58% of block time
// on the page "Buyer Questions: Current Evidence Status", question 4), and the
// attention backend tuned to H3's own shapes that the page "H3 Runtime Current
// State" counts as owed ("Owned Performance Kernels").  It consumes the prologue's head-major
// qhat / khat and per-tile transposed V, and computes, for each query row,
// the softmax over the keys of its own sequence tile by tile (an online
// softmax), never materialising the N x N score matrix.
//
// Two kernels.  attn_bf16_pp_kernel runs head_dim 128, dense and block-sparse
// (eight waves, 256 query rows per workgroup, its own notes further down);
// attn_bf16_kernel runs head_dim 64, dense and block-sparse, and the notes
// here describe it.  Both share the matrix-core layout and the softmax below.
//
// Work decomposition.  One workgroup = 4 waves = 128 query rows of one
// (sequence, head); each wave owns 32 query rows.  Workgroups are ordered
// longest sequence first, then head, then query block, so consecutive
// workgroups (which the dispatcher spreads over the 8 XCDs) stream the same
// head's K/V and share it through each XCD's L2.
//
// Matrix-core layout.  Both products use v_mfma_f32_32x32x16_bf16 and are
// arranged so every lane keeps one query row throughout:
//   S^T = K . Q^T   A = K tile rows from LDS (M = key), B = Q^T held in
//                   registers (N = query); the 32x32 accumulator gives lane l
//                   query l%32 and 16 of the 32 keys.
//   O^T = V^T . P^T A = V^T rows from LDS (M = channel), B = P^T straight from
//                   the score registers (N = query); lane l accumulates 16
//                   channels per 32-channel block of query l%32.
// So the softmax row max and row sum are in-lane reductions plus one
// exchange with lane l^32, and the running-max rescale of O is a per-lane
// scalar.  The 8 keys one lane feeds to a P.V step are keys
// {16c + 8(e/4) + 4(l/32) + e%4}; the prologue stores V^T with bits 2 and 3 of
// the in-tile key index swapped so those 8 keys are one contiguous 16-byte LDS
// read.
//
// Pipelining.  K and V^T tiles of 64 keys are double-buffered in LDS and
// filled straight from global memory by buffer_load_dwordx4 ... lds (no
// staging registers; the buffer descriptor bounds every access).  K runs one
// tile ahead of V: iteration j issues the scores of tile j+1 (matrix cores)
// next to the softmax of tile j (vector ALUs), which do not depend on each
// other, then the P.V product of tile j; the loads of K tile j+2 and V tile
// j+1 are in flight meanwhile, and one barrier per tile hands the buffers
// over.  LDS rows are XOR swizzled at 16-byte granularity so the 16-byte
// fragment reads of each group of 16 lanes hit distinct banks.
//
// Softmax in base 2.  The prologue stores qhat * scale * log2(e), and each
// score MFMA chain starts from -m instead of 0 (the splat -m is held in
// registers), so the matrix cores deliver x = s*scale*log2(e) - m directly and
// p = 2^x needs no further VALU work.  m is fixed per row to the bound
// |qhat'| * max|khat| when that bound is at most 48 (softmax does not depend
// on the shift; every p <= 1 and none underflows), which needs neither a
// per-tile row maximum nor a rescale.  Otherwise m is a running maximum raised
// only when a tile exceeds it by more than 8, so O and l are rescaled rarely
// and p stays below 2^8.  P is rounded to bf16 for the P.V product and the
// row sum l adds exactly those rounded values.
#include "h3_internal.h"
#include "attn_common.h"
#include "h3_checked.h"

namespace h3 {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLazyRescale = 8.0f;
// Largest score bound (log2 units) for which the fixed shift is used.
constexpr float kFixedShiftMax = 48.0f;
// Fixed-shift test.  Softmax is unchanged by a per-row shift, and every score
// of the row is at most |q'| * max_k |k| (Cauchy-Schwarz; q' already carries
// scale * log2 e, the norms are those of the stored bf16 rows).  When that
// bound mb is small enough for every row of the wave, m_run = mb for the whole
// row: p = 2^(s - mb) <= 1, and even the row's largest p stays a normal number
// (s_max >= -mb, so p_max >= 2^-2mb), so no running max, no rescale and no
// per-tile row maximum are needed.  Returns whether the whole wave qualifies;
// mb is this lane's row bound.  knorm holds max |k| per 64-key tile.
template <int KSTEPS>
__device__ __forceinline__ bool fixed_shift_bound(const bf16x8 (&qf)[KSTEPS], const float *knorm, int ntiles,
                                                  int lane, float &mb)
{
    float qn2 = 0.f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = (float)qf[s][i];
            qn2 = fmaf(x, x, qn2);
        }
    qn2 = row_sum2(qn2);
    float kmax = 0.f;
    for (int i = lane; i < ntiles; i += 64) kmax = fmaxf(kmax, knorm[i]);
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, mm));
    mb = sqrtf(qn2) * kmax * (1.0f + 1.0f / 1024);
    return __all(mb <= kFixedShiftMax);
}

// Work item of workgroup b of n under the dispatcher's round-robin spread of
// workgroups over the 8 XCDs (b goes to XCD b % 8).  Items are taken in
// windows of W = 512 (the workgroups resident at once, two per CU): a window
// stays on one head, so every XCD streams the same keys through the shared
// last-level cache, and inside it XCD x runs the contiguous items x*64 ..
// x*64 + 63, so the query blocks that share its L2 are neighbours.  The last
// partial window keeps the dispatch order.
__device__ __forceinline__ int xcd_window_item(int b, int n)
{
    constexpr int X = 8, W = 512, C = W / X;
    if (b >= n / W * W) return b;
    const int r = b % W;
    return b - r + (r % X) * C + r / X;
}

// SPARSE: visit only the 64-key tiles listed for this query block's
// kSparseBlockM-row block (block-sparse attention, a.tiles; the two 128-row
// halves of a block read the same list); otherwise every tile of the sequence.
// Sparse work items are numbered by xcd_window_item, so the halves of a block
// and neighbouring blocks run on one XCD and share the tiles its L2 holds.
template <int D, bool SPARSE>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a)
{
    constexpr int KSTEPS = D / 16;          // k-steps of the S^T product
    constexpr int DB = D / 32;              // 32-channel output blocks
    constexpr int KCPR = D / 8;             // 16-byte chunks per K row
    // Separate arrays per buffer: the compiler can then prove that a
    // direct-to-LDS fill of one buffer does not alias fragment reads of the
    // other, and need not wait for the fill before reading.
    __shared__ __attribute__((aligned(16))) uint16_t lk0[kTile * D], lk1[kTile * D];
    __shared__ __attribute__((aligned(16))) uint16_t lv0[D * kTile], lv1[D * kTile];
    __shared__ int32_t ltiles[SPARSE ? kMaxSparseTiles : 1];     // the block's tile list

    // ---- work item: (sequence, head, 128-row query block)
    const int b = SPARSE ? xcd_window_item((int)blockIdx.x, (int)gridDim.x) : (int)blockIdx.x;
    int si = 0;
    while (b >= a.item_pre[si + 1]) ++si;
    const int rem = b - a.item_pre[si];
    const int nqb = a.seq_nqb[si];
    const int head = rem / nqb, qb = rem % nqb;
    const int n = a.seq_n[si];
    const int off = a.seq_off[si];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, hh = lane >> 5;
    const int q0 = qb * kBlockM + wave * 32;
    H3_CHECK(si < a.nseq && head < a.H && qb < nqb, kCheckItem);
    H3_CHECK(off + q0 + 32 <= a.Npad, kCheckRows);

    // ---- Q^T fragments: lane holds query q0+m, channels 16s + 8hh .. +7
    bf16x8 qf[KSTEPS];
    {
        const uint16_t *qp = a.qhat + ((int64_t)head * a.Npad + off + q0 + m) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
    }

    const uint16_t *kbase = a.khat + ((int64_t)head * a.Npad + off) * D;
    const uint16_t *vbase = a.vt + ((int64_t)head * (a.Npad / kTile) + off / kTile) * (D * kTile);
    const int ntk = (n + kTile - 1) / kTile;           // tiles of the sequence
    int nt = ntk;                                     // tiles this block visits
    if constexpr (SPARSE) {
        // the list, clamped to the sequence's tiles, goes to LDS; each visit
        // reads its entry back as a wave-uniform scalar
        constexpr int R = kSparseBlockM / kBlockM;   // work items per list
        nt = min(a.tpb, ntk);
        const int32_t *lst =
            a.tiles + ((int64_t)a.seq_item_base[si] + (int64_t)head * ((nqb + R - 1) / R) + qb / R) * a.tpb;
        for (int i = threadIdx.x; i < nt; i += 256) {
            H3_CHECK(lst[i] >= 0 && lst[i] < ntk, kCheckListEntry);
            ltiles[i] = min(max(lst[i], 0), ntk - 1);
        }
        __syncthreads();
    }
    auto tix = [&](int j) -> int {
        if constexpr (SPARSE)
            return __builtin_amdgcn_readfirstlane(ltiles[j]);
        else
            return j;
    };
    TileFill<kTile, KCPR> kfill;
    TileFill<D, 8> vfill;
    kfill.init(wave, lane);
    vfill.init(wave, lane);
    auto kbuf = [&](int buf) { return buf ? lk1 : lk0; };
    auto vbuf = [&](int buf) { return buf ? lv1 : lv0; };
    // buffer descriptors over this (sequence, head)'s padded K rows and V^T tiles
    const int tbytes = kTile * D * 2;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(kbase), 0, ntk * tbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(vbase), 0, ntk * tbytes, kBufferFlags);
    auto load_k = [&](int j, uint16_t *dst) {
        H3_CHECK(j < nt && tix(j) >= 0 && tix(j) < ntk, kCheckFillTile);
        H3_JITTER(wave, j, 0);
        kfill.load(krs, (uint32_t)(tix(j) * tbytes), dst, wave);
    };
    auto load_v = [&](int j, uint16_t *dst) {
        H3_CHECK(j < nt && tix(j) >= 0 && tix(j) < ntk, kCheckFillTile);
        H3_JITTER(wave, j, 1);
        vfill.load(vrs, (uint32_t)(tix(j) * tbytes), dst, wave);
    };

    f32x16 o[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] = (f32x16){};
    float m_run = 0.f, l = 0.f;         // running max (log2 units), row sum
    // -m_run in all 16 registers: the accumulator start of every score MFMA
    // chain.  It changes only when m_run is raised, and is kept opaque so that
    // the compiler holds it instead of rebuilding the splat for every tile.
    f32x16 ninit = (f32x16){};
    bool first = true;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // Fixed shift when the whole wave qualifies; larger bounds keep the lazily
    // rescaled running max.
    float mb;
    const bool fixed_shift =
        fixed_shift_bound(qf, a.knorm + (int64_t)head * (a.Npad / kTile) + off / kTile, ntk, lane, mb);
    if (fixed_shift) {
        m_run = mb;
        ninit = -m_run;
        asm volatile("" : "+v"(ninit));
        first = false;
    }

    // x^T = K . Q'^T - m_run of one 64-key tile from K buffer kl.
    auto scores = [&](const uint16_t *kl, f32x16 &s0, f32x16 &s1) {
        s0 = ninit;
        s1 = ninit;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
            const int ch = (2 * st + hh) ^ swz<KCPR>(m);
            const bf16x8 k0 = *reinterpret_cast<const bf16x8 *>(kl + m * D + 8 * ch);
            const bf16x8 k1 = *reinterpret_cast<const bf16x8 *>(kl + (32 + m) * D + 8 * ch);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[st], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[st], s1, 0, 0, 0);
        }
    };

    // Tile j's row max (masking keys past the sequence end on the last tile);
    // raise m_run when the tile exceeds it by more than kLazyRescale (always on
    // the first tile), rescaling O and l and shifting the tile's x.
    auto row_max_update = [&](int j, f32x16 &s0, f32x16 &s1, bool mask) {
        // a sparse list may hold the sequence's partial last tile at any position
        const int valid = n - tix(j) * kTile;
        if ((mask || SPARSE) && valid < kTile) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
                if (key >= valid) s0[r] = -INFINITY;
                if (32 + key >= valid) s1[r] = -INFINITY;
            }
        }
        if (fixed_shift) return;
        const float mx = row_max2(lane_max32(s0, s1));
        const bool need = first || mx > kLazyRescale;
        if (__any(need)) {
            const float delta = need ? mx : 0.f;
            if (!first) {
                const float alpha = __builtin_amdgcn_exp2f(-delta);
                l *= alpha;
#pragma unroll
                for (int i = 0; i < DB; ++i) o[i] *= alpha;
            }
            m_run += delta;
            ninit = -m_run;
            asm volatile("" : "+v"(ninit));
            s0 -= delta;
            s1 -= delta;
            first = false;
        }
    };

    // p = 2^x in bf16, l += p, O^T += V^T P^T from V buffer vl (unscheduled form).
    auto exp_pv = [&](const uint16_t *vl, const f32x16 &s0, const f32x16 &s1) {
        uint32_t p0[8], p1[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            p0[r / 2] = pack2(__builtin_amdgcn_exp2f(s0[r]), __builtin_amdgcn_exp2f(s0[r + 1]));
            p1[r / 2] = pack2(__builtin_amdgcn_exp2f(s1[r]), __builtin_amdgcn_exp2f(s1[r + 1]));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p0[i]), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p1[i]), ones, l, false);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const uint32_t *pp = kb ? p1 : p0;
                const u32x4 pw = {pp[4 * cc], pp[4 * cc + 1], pp[4 * cc + 2], pp[4 * cc + 3]};
                const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int row = 32 * db + m;
                    const int ch = (4 * kb + 2 * cc + hh) ^ swz<8>(row);
                    const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(vl + row * kTile + 8 * ch);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
                }
            }
        }
    };

    // Hand-scheduled steady-state body: 2*KSTEPS score MFMAs of tile j+1 then
    // 4*DB P.V MFMAs of tile j, one per chunk; chunk i also issues the LDS
    // fragment read of MFMA i+PD, and each score chunk carries the softmax of
    // element pairs of tile j (exp2, bf16 pack, row-sum dot2).  Scheduling
    // barriers keep the chunks in this order, so every fragment read has PD
    // MFMAs to land and the exps run beside the matrix cores.
    constexpr int PD = 5;
    constexpr int NQK = 2 * KSTEPS, NM = 2 * KSTEPS + 4 * DB;
    auto frag = [&](int i, const uint16_t *kl, const uint16_t *vl) -> bf16x8 {
        if (i < NQK) {
            const int st = i >> 1, blk = i & 1;
            const int ch = (2 * st + hh) ^ swz<KCPR>(m);
            return *reinterpret_cast<const bf16x8 *>(kl + (32 * blk + m) * D + 8 * ch);
        }
        const int k = i - NQK, kb = k / (2 * DB), cc = (k / DB) & 1, db = k % DB;
        const int row = 32 * db + m;
        const int ch = (4 * kb + 2 * cc + hh) ^ swz<8>(row);
        return *reinterpret_cast<const bf16x8 *>(vl + row * kTile + 8 * ch);
    };
    auto body = [&](const uint16_t *kl, const uint16_t *vl, const f32x16 &c0, const f32x16 &c1,
                    f32x16 &n0, f32x16 &n1) {
        bf16x8 fa[NM];
        uint32_t pw[16];
#pragma unroll
        for (int i = 0; i < PD; ++i) fa[i] = frag(i, kl, vl);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if (i + PD < NM) fa[i + PD] = frag(i + PD, kl, vl);
            // the exp-carrying score chunks issue ahead of the other wave on the SIMD
            if (i == 0) __builtin_amdgcn_s_setprio(1);
            if (i == NQK) __builtin_amdgcn_s_setprio(0);
            if (i < NQK) {
                const int st = i >> 1, blk = i & 1;
                if (blk == 0)
                    n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], qf[st], st ? n0 : ninit, 0, 0, 0);
                else
                    n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], qf[st], st ? n1 : ninit, 0, 0, 0);
                constexpr int PIECES = 16 / NQK;        // element pairs of tile j per score chunk
#pragma unroll
                for (int q = 0; q < PIECES; ++q) {
                    const int pi = i * PIECES + q;
                    const int e = 2 * pi, sb = e >> 4, r = e & 15;
                    const f32x16 &sc = sb ? c1 : c0;
                    const uint32_t w = pack2(__builtin_amdgcn_exp2f(sc[r]), __builtin_amdgcn_exp2f(sc[r + 1]));
                    pw[pi] = w;
                    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, l, false);
                }
            } else {
                const int k = i - NQK, kb = k / (2 * DB), cc = (k / DB) & 1, db = k % DB;
                const u32x4 q4 = {pw[8 * kb + 4 * cc], pw[8 * kb + 4 * cc + 1], pw[8 * kb + 4 * cc + 2],
                                  pw[8 * kb + 4 * cc + 3]};
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], __builtin_bit_cast(bf16x8, q4), o[db], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- prologue: K0, V0 (and K1) resident, scores of tile 0
    __builtin_amdgcn_sched_barrier(0);
    load_k(0, lk0);
    load_v(0, lv0);
    if (nt > 1) load_k(1, lk1);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    f32x16 sa0, sa1, sb0, sb1;
    scores(lk0, sa0, sa1);
    __syncthreads();

    // Iteration j: fills K[j+2] -> lk[j&1] and V[j+1] -> lv[(j+1)&1]; scores
    // of tile j+1 from lk[(j+1)&1] beside the softmax of tile j; P.V of tile j
    // from lv[j&1]; then wait for the fills and one barrier.  The steady state
    // runs two iterations per trip with the buffers named at compile time.
    int j = 0;
    for (; j + 3 < nt; j += 2) {
        load_k(j + 2, lk0);
        load_v(j + 1, lv1);
        row_max_update(j, sa0, sa1, false);
        H3_JITTER(wave, j, 2);
        body(lk1, lv0, sa0, sa1, sb0, sb1);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        load_k(j + 3, lk1);
        load_v(j + 2, lv0);
        row_max_update(j + 1, sb0, sb1, false);
        H3_JITTER(wave, j + 1, 2);
        body(lk0, lv1, sb0, sb1, sa0, sa1);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
    }
    for (; j + 1 < nt; ++j) {
        if (j + 2 < nt) load_k(j + 2, kbuf(j & 1));
        load_v(j + 1, vbuf((j + 1) & 1));
        row_max_update(j, sa0, sa1, false);
        H3_JITTER(wave, j, 3);
        scores(kbuf((j + 1) & 1), sb0, sb1);
        exp_pv(vbuf(j & 1), sa0, sa1);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        sa0 = sb0;
        sa1 = sb1;
    }
    row_max_update(j, sa0, sa1, true);
    exp_pv(vbuf(j & 1), sa0, sa1);

    // ---- epilogue: o = O / l, bf16, rows of this sequence only
    const float inv = 1.0f / row_sum2(l);
    const int qrow = q0 + m;
    if (qrow < n) {
        uint16_t *op = a.out + ((int64_t)a.seq_cu[si] + qrow) * a.o_stride + (int64_t)head * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x2 w = {pack2(o[db][4 * i] * inv, o[db][4 * i + 1] * inv),
                                 pack2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv)};
                *reinterpret_cast<u32x2 *>(op + 32 * db + 8 * i + 4 * hh) = w;
            }
        }
    }
}

// Explicit instantiations (the host pass emits launch stubs only for these).
template __global__ void attn_bf16_kernel<64, false>(AttnArgs);
template __global__ void attn_bf16_kernel<64, true>(AttnArgs);

// ---------------------------------------------------------------------------
// Attention at head_dim 128: two groups of four waves per workgroup.  SPARSE
// visits only the tiles of the block's list (block-sparse attention: one list
// per 256-row block, read into LDS at the start; every fill takes its tile
// index from it); otherwise every tile of the sequence.
//
// Work item: (sequence, head, 256-row query block).  Waves 0-3 form group 0
// and waves 4-7 group 1, 32 query rows each; the dispatcher places wave w and
// wave w+4 on the same SIMD.  Per 64-key tile j every wave runs two phases,
// each closed by a workgroup barrier:
//   softmax phase  the score MFMAs of tile j+1, with the softmax of keys 0..31
//                  of tile j (exp2, bf16 pack, row-sum dot2) beside them;
//   P.V phase      the P.V MFMAs of tile j, with the softmax of keys 32..63
//                  beside the first half, which reads keys 0..31 only.
// Group 1 waits one barrier before its first phase and group 0 one after its
// last, so on every SIMD one wave runs its softmax phase while the other runs
// its P.V phase.  Both phases carry 16 MFMAs and 16 exp2.  The mid-tile
// barrier is what keeps the two waves half a tile apart: with one barrier per
// tile they drift back into step and the kernel is slower.  Against two 4-wave
// workgroups per CU, one 256-row workgroup reads each K/V tile from L2 once
// instead of twice; measured, that takes the same cycles per launch at a
// higher engine clock on this power-limited part.
//
// K and V^T tiles rotate through three LDS buffers per operand (96 KB, one
// workgroup per CU).  In its softmax phase of tile j a wave issues its quarter
// of one fill (group 0: K[j+3] into lk[j%3], group 1: V[j+2] into lv[(j+2)%3])
// and waits for it at the end of its following P.V phase.  Every tile is thus
// resident a whole phase before any wave reads it, and each phase's first
// fragments are read at the end of the phase before.  The last tile's softmax
// phase also computes scores of a tile past the end from whatever the buffer
// holds (in bounds, never used), so one loop serves every tile count.
//
// Per row the arithmetic is that of attn_bf16_kernel's main loop: score chains
// from -m, p = 2^x rounded to bf16, l summing the rounded p in key order, and
// the same P.V accumulation order.
static_assert(kBlockM2 == 8 * 32, "eight waves of 32 query rows");

template <int D, bool SPARSE>
__global__ __launch_bounds__(512, 2) void attn_bf16_pp_kernel(AttnArgs a)
{
    static_assert(D == 128, "tile fills assume 16 KB K and V^T tiles");
    constexpr int KSTEPS = D / 16;
    constexpr int DB = D / 32;
    constexpr int KCPR = D / 8;
    constexpr int PD = 5;                              // fragment prefetch distance (MFMAs)
    constexpr int NQK = 2 * KSTEPS, NPV = 4 * DB;      // MFMAs per phase
    static_assert(NQK == 16 && NPV == 16, "one exp2 pair per MFMA slot below");
    __shared__ __attribute__((aligned(16))) uint16_t lk0[kTile * D], lk1[kTile * D], lk2[kTile * D];
    __shared__ __attribute__((aligned(16))) uint16_t lv0[D * kTile], lv1[D * kTile], lv2[D * kTile];
    __shared__ int32_t ltiles[SPARSE ? kMaxSparseTiles : 1];     // the block's tile list

    // ---- work item: (sequence, head, 256-row query block)
    const int b = blockIdx.x;
    int si = 0;
    while (b >= a.item_pre[si + 1]) ++si;
    const int rem = b - a.item_pre[si];
    const int nqb = a.seq_nqb[si];
    const int head = rem / nqb, qb = rem % nqb;
    const int n = a.seq_n[si];
    const int off = a.seq_off[si];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int grp = wave >> 2, gw = wave & 3;
    const int m = lane & 31, hh = lane >> 5;
    const int q0 = qb * kBlockM2 + wave * 32;
    H3_CHECK(si < a.nseq && head < a.H && qb < nqb, kCheckItem);
    H3_CHECK(off + q0 + 32 <= a.Npad, kCheckRows);

    bf16x8 qf[KSTEPS];
    {
        const uint16_t *qp = a.qhat + ((int64_t)head * a.Npad + off + q0 + m) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
    }

    const uint16_t *kbase = a.khat + ((int64_t)head * a.Npad + off) * D;
    const uint16_t *vbase = a.vt + ((int64_t)head * (a.Npad / kTile) + off / kTile) * (D * kTile);
    const int ntk = (n + kTile - 1) / kTile;           // tiles of the sequence
    int nt = ntk;                                     // tiles this block visits
    if constexpr (SPARSE) {
        // the list, clamped to the sequence's tiles, goes to LDS; each visit
        // reads its entry back as a wave-uniform scalar
        nt = min(a.tpb, ntk);
        const int32_t *lst = a.tiles + ((int64_t)a.seq_item_base[si] + (int64_t)head * nqb + qb) * a.tpb;
        for (int i = tid; i < nt; i += 512) {
            H3_CHECK(lst[i] >= 0 && lst[i] < ntk, kCheckListEntry);
            ltiles[i] = min(max(lst[i], 0), ntk - 1);
        }
        __syncthreads();
    }
    // Sequence tile of visit j (j < nt).
    auto tix = [&](int j) -> int {
        if constexpr (SPARSE)
            return __builtin_amdgcn_readfirstlane(ltiles[j]);
        else
            return j;
    };
    const int tbytes = kTile * D * 2;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(kbase), 0, ntk * tbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(vbase), 0, ntk * tbytes, kBufferFlags);
    // group 0 fills K tiles, group 1 V^T tiles: four 1 KB pieces per wave
    uint32_t fgoff[4];
    {
        TileFill<kTile, KCPR> kf;
        TileFill<D, 8> vf;
        static_assert(TileFill<kTile, KCPR>::PER_WAVE == 4 && TileFill<D, 8>::PER_WAVE == 4, "16 KB tiles");
        kf.init(gw, lane);
        vf.init(gw, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) fgoff[i] = grp ? vf.goff[i] : kf.goff[i];
    }
    const __amdgpu_buffer_rsrc_t frs = grp ? vrs : krs;
    // sequence tile t into dst
    auto fill = [&](__amdgpu_buffer_rsrc_t rs, int t, uint16_t *dst) {
        H3_CHECK(t >= 0 && t < ntk, kCheckFillTile);
        const uint32_t toff = (uint32_t)(t * tbytes);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void *)(reinterpret_cast<char *>(dst) + (gw * 4 + i) * 1024),
                16, fgoff[i], toff, 0, 0);
    };

    f32x16 o[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] = (f32x16){};
    float m_run = 0.f, l = 0.f;
    f32x16 ninit = (f32x16){};
    bool first = true;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float mb;
    const bool fixed_shift =
        fixed_shift_bound(qf, a.knorm + (int64_t)head * (a.Npad / kTile) + off / kTile, ntk, lane, mb);
    if (fixed_shift) {
        m_run = mb;
        ninit = -m_run;
        asm volatile("" : "+v"(ninit));
        first = false;
    }

    auto kfrag = [&](int i, const uint16_t *kl) -> bf16x8 {
        const int st = i >> 1, blk = i & 1;
        const int ch = (2 * st + hh) ^ swz<KCPR>(m);
        return *reinterpret_cast<const bf16x8 *>(kl + (32 * blk + m) * D + 8 * ch);
    };
    auto vfrag = [&](int k, const uint16_t *vl) -> bf16x8 {
        const int kb = k / (2 * DB), cc = (k / DB) & 1, db = k % DB;
        const int row = 32 * db + m;
        const int ch = (4 * kb + 2 * cc + hh) ^ swz<8>(row);
        return *reinterpret_cast<const bf16x8 *>(vl + row * kTile + 8 * ch);
    };
    // x^T = K . Q'^T - m_run of one 64-key tile (prologue form)
    auto scores = [&](const uint16_t *kl, f32x16 &s0, f32x16 &s1) {
        s0 = ninit;
        s1 = ninit;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(2 * st, kl), qf[st], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(2 * st + 1, kl), qf[st], s1, 0, 0, 0);
        }
    };
    // Row max of the visit to sequence tile t (masking keys past the sequence
    // end in its partial last tile, which a sparse list may hold at any
    // position); raise m_run when the tile exceeds it by more than kLazyRescale
    // (always on the first visit), rescaling O and l and shifting the tile's x.
    auto row_max_update = [&](int t, f32x16 &s0, f32x16 &s1) {
        const int valid = n - t * kTile;
        if (valid < kTile) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
                if (key >= valid) s0[r] = -INFINITY;
                if (32 + key >= valid) s1[r] = -INFINITY;
            }
        }
        if (fixed_shift) return;
        const float mx = row_max2(lane_max32(s0, s1));
        const bool need = first || mx > kLazyRescale;
        if (__any(need)) {
            const float delta = need ? mx : 0.f;
            if (!first) {
                const float alpha = __builtin_amdgcn_exp2f(-delta);
                l *= alpha;
#pragma unroll
                for (int i = 0; i < DB; ++i) o[i] *= alpha;
            }
            m_run += delta;
            ninit = -m_run;
            asm volatile("" : "+v"(ninit));
            s0 -= delta;
            s1 -= delta;
            first = false;
        }
    };

    uint32_t pw[16];       // P of the current tile in bf16 pairs, key order
    // one element pair of x -> p = 2^x in bf16 -> pw[pi], l += p
    auto soft_pair = [&](int pi, float x0, float x1) {
        const uint32_t w = pack2(__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1));
        pw[pi] = w;
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, l, false);
    };
    // Softmax phase: scores of the next tile (n0, n1) from kl beside the
    // softmax of keys 0..31 of this tile (c0) into pw[0..8).  fa[0..PD) come
    // prefetched in pre; the first PD fragments of the P.V phase (from vl)
    // leave in pre.
    auto phase_s = [&](const uint16_t *kl, const uint16_t *vl, const f32x16 &c0, f32x16 &n0, f32x16 &n1,
                       bf16x8 (&pre)[PD]) {
        bf16x8 fa[NQK];
#pragma unroll
        for (int i = 0; i < PD; ++i) fa[i] = pre[i];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            if (i + PD < NQK)
                fa[i + PD] = kfrag(i + PD, kl);
            else
                pre[i + PD - NQK] = vfrag(i + PD - NQK, vl);
            const int st = i >> 1;
            if ((i & 1) == 0) {
                n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], qf[st], st ? n0 : ninit, 0, 0, 0);
                soft_pair(st, c0[2 * st], c0[2 * st + 1]);
            } else {
                n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], qf[st], st ? n1 : ninit, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // P.V phase: O^T += V^T P^T of this tile from vl, with the softmax of
    // keys 32..63 (c1) into pw[8..16) beside the first eight MFMAs (keys
    // 0..31); fa[0..PD) come prefetched in pre, and the first PD fragments
    // of the next softmax phase (from kl) leave in pre.
    auto phase_p = [&](const uint16_t *vl, const uint16_t *kl, const f32x16 &c1, bf16x8 (&pre)[PD]) {
        bf16x8 fa[NPV];
#pragma unroll
        for (int i = 0; i < PD; ++i) fa[i] = pre[i];
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            if (i + PD < NPV)
                fa[i + PD] = vfrag(i + PD, vl);
            else
                pre[i + PD - NPV] = kfrag(i + PD - NPV, kl);
            const int kb = i / (2 * DB), cc = (i / DB) & 1, db = i % DB;
            const u32x4 q4 = {pw[8 * kb + 4 * cc], pw[8 * kb + 4 * cc + 1], pw[8 * kb + 4 * cc + 2],
                              pw[8 * kb + 4 * cc + 3]};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], __builtin_bit_cast(bf16x8, q4), o[db], 0, 0, 0);
            if (i < 8) soft_pair(8 + i, c1[2 * i], c1[2 * i + 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Phase ends.  The scheduling barriers keep every instruction on its side
    // of the workgroup barrier, so the two phases keep their balance.
    auto end_s = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto end_p = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: K0..K2 (group 0) and V0, V1 (group 1) resident; every
    // wave's scores of tile 0, then a barrier before lk0 is refilled
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0) {
        fill(krs, tix(0), lk0);
        if (nt > 1) fill(krs, tix(1), lk1);
        if (nt > 2) fill(krs, tix(2), lk2);
    } else {
        fill(vrs, tix(0), lv0);
        if (nt > 1) fill(vrs, tix(1), lv1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    f32x16 sa0, sa1, sb0, sb1;
    scores(lk0, sa0, sa1);
    __syncthreads();

    if (grp == 1) barrier_only();
    bf16x8 pre[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) pre[i] = kfrag(i, lk1);
    // Tile j with its buffers named at compile time: kn = lk[(j+1)%3] (scores
    // of tile j+1), vc = lv[j%3], kn2 = lk[(j+2)%3] (prefetch for tile j+1),
    // kf = lk[j%3] and vf = lv[(j+2)%3] (this tile's fills).
    auto tile = [&](int j, const uint16_t *kn, const uint16_t *vc, const uint16_t *kn2, uint16_t *kf, uint16_t *vf,
                    f32x16 &c0, f32x16 &c1, f32x16 &n0, f32x16 &n1) {
        H3_JITTER(wave, j, 0);
        if (j + 3 - grp < nt) fill(frs, tix(j + 3 - grp), grp ? vf : kf);
        row_max_update(tix(j), c0, c1);
        H3_JITTER(wave, j, 1);
        phase_s(kn, vc, c0, n0, n1, pre);
        end_s();
        H3_JITTER(wave, j, 2);
        phase_p(vc, kn2, c1, pre);
        end_p();
    };
    for (int j = 0;; j += 6) {
        tile(j, lk1, lv0, lk2, lk0, lv2, sa0, sa1, sb0, sb1);
        if (j + 1 == nt) break;
        tile(j + 1, lk2, lv1, lk0, lk1, lv0, sb0, sb1, sa0, sa1);
        if (j + 2 == nt) break;
        tile(j + 2, lk0, lv2, lk1, lk2, lv1, sa0, sa1, sb0, sb1);
        if (j + 3 == nt) break;
        tile(j + 3, lk1, lv0, lk2, lk0, lv2, sb0, sb1, sa0, sa1);
        if (j + 4 == nt) break;
        tile(j + 4, lk2, lv1, lk0, lk1, lv0, sa0, sa1, sb0, sb1);
        if (j + 5 == nt) break;
        tile(j + 5, lk0, lv2, lk1, lk2, lv1, sb0, sb1, sa0, sa1);
        if (j + 6 == nt) break;
    }
    if (grp == 0) barrier_only();

    // ---- epilogue: o = O / l, bf16, rows of this sequence only
    const float inv = 1.0f / row_sum2(l);
    const int qrow = q0 + m;
    if (qrow < n) {
        uint16_t *op = a.out + ((int64_t)a.seq_cu[si] + qrow) * a.o_stride + (int64_t)head * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x2 w = {pack2(o[db][4 * i] * inv, o[db][4 * i + 1] * inv),
                                 pack2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv)};
                *reinterpret_cast<u32x2 *>(op + 32 * db + 8 * i + 4 * hh) = w;
            }
        }
    }
}

template __global__ void attn_bf16_pp_kernel<128, false>(AttnArgs);
template __global__ void attn_bf16_pp_kernel<128, true>(AttnArgs);

#ifdef H3ATTN_CHECKED
hipError_t attn_checked(uint32_t *or_into, bool clear, uint32_t jitter_seed)
{
    return checked_state_here(or_into, clear, jitter_seed);
}
#endif

// Head_dim 128 runs attn_bf16_pp_kernel over 256-row query blocks, dense or
// block-sparse (a.tiles); head_dim 64 runs attn_bf16_kernel over 128-row
// blocks (attn_bf16_block_m gives the caller the block size).
hipError_t launch_attn_bf16(const AttnArgs &a, int d, int64_t nitems, hipStream_t st)
{
    if (nitems <= 0) return hipSuccess;
    const dim3 grid((unsigned)nitems);
    if (a.tiles) {
        if (d == 128)
            hipLaunchKernelGGL((attn_bf16_pp_kernel<128, true>), grid, dim3(512), 0, st, a);
        else
            hipLaunchKernelGGL((attn_bf16_kernel<64, true>), grid, dim3(256), 0, st, a);
    } else {
        if (d == 128)
            hipLaunchKernelGGL((attn_bf16_pp_kernel<128, false>), grid, dim3(512), 0, st, a);
        else
            hipLaunchKernelGGL((attn_bf16_kernel<64, false>), grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace h3
