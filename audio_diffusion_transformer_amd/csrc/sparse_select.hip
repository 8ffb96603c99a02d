// Block-sparse tile selection for gfx950: which 64-key tiles each 256-row
// query block (kSparseBlockM rows, one workgroup of the attention kernel)
// attends to.
//
// The page "Open-H3-Regenerate-2K" ("Speed on one B200 (GB200)", per-module
// table) credits a sparse attention backend with most of a refine's speed-up
// over dense attention and calls it lossy; the pages give no algorithm.  The
// selection here is the plain block-level estimate of where the softmax mass
// lies: the query block's mean qhat' row against each key tile's mean khat row
// (the stored bf16 values the attention reads), keeping the tpb tiles with the
// largest pooled score (ties to the lower tile index).
//
// Pass 1 (sparse_pool_kernel): one workgroup per (padded 64-token tile, head)
// sums the tile's khat and qhat' rows column by column (coalesced 256-byte row
// reads; padding rows are zeros) and stores the khat mean (channel-major) and
// the qhat' sum.
// Pass 2 (sparse_select_kernel): one workgroup per (sequence, head, group of 4
// query blocks) forms the 4 query means (each over the block's four tiles),
// scores every tile of the sequence (each kbar value read once for the 4
// blocks), finds each block's L-th largest score by a radix select over
// order-preserving keys (four 8-bit histogram passes in LDS), and writes the
// kept tiles in tile order through a workgroup prefix sum (ties at the
// threshold go to the lower tiles).
#include "h3_internal.h"
#include "norm_rope.h"

namespace h3 {

constexpr int kSelectGroup = 4;     // query blocks per select workgroup

template <int D>
__global__ __launch_bounds__(256) void sparse_pool_kernel(SparseSelectArgs a)
{
    const int gt = blockIdx.x / a.H, h = blockIdx.x % a.H;
    const int c = threadIdx.x % 128, which = threadIdx.x / 128;   // which: 0 khat, 1 qhat'
    int s, j, valid;
    tile_seq(a.seq.cu, a.seq.off, a.seq.S, gt, s, j, valid);
    if (h == 0 && threadIdx.x == 0) a.cnt[gt] = valid;
    if (c >= D) return;
    const uint16_t *src = (which ? a.qhat : a.khat) + ((int64_t)h * a.Npad + (int64_t)gt * kTile) * D + c;
    float sum = 0.f;
#pragma unroll 8
    for (int r = 0; r < kTile; ++r) sum += __uint_as_float((uint32_t)src[(int64_t)r * D] << 16);
    if (which)
        a.qsum[((int64_t)h * a.ntiles + gt) * D + c] = sum;
    else    // channel-major, so the select pass reads consecutive tiles per channel
        a.kbar[((int64_t)h * D + c) * a.ntiles + gt] = valid > 0 ? sum / (float)valid : 0.f;
}

// Order-preserving map of a float to an unsigned key.
__device__ __forceinline__ uint32_t ord_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the 256 threads of the workgroup (4 waves);
// *total receives the sum.  Contains barriers: every thread must call it.
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t *wsum, uint32_t *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    return before + x - v;
}

template <int D>
__global__ __launch_bounds__(256) void sparse_select_kernel(SparseSelectArgs a)
{
    constexpr int PER = kMaxSparseTiles / 256;                  // tiles per thread in the scans
    __shared__ uint32_t ukey[kSelectGroup][kMaxSparseTiles];    // 32 KB
    __shared__ float qv[kSelectGroup][D];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t bc[2];
    __shared__ uint32_t wsum[4];

    // ---- (sequence, head, group of query blocks)
    const int b = blockIdx.x;
    int s = 0;
    while (s + 1 < a.seq.S && b >= a.group_pre[s + 1]) ++s;
    const int n = a.seq.cu[s + 1] - a.seq.cu[s];
    const int nqb = (n + kSparseBlockM - 1) / kSparseBlockM, ntk = (n + kTile - 1) / kTile;
    const int ng = (nqb + kSelectGroup - 1) / kSelectGroup;
    const int rem = b - a.group_pre[s];
    const int h = rem / ng, g = rem % ng;
    const int nq = min(kSelectGroup, nqb - kSelectGroup * g);
    const int t0 = a.seq.off[s] / kTile;                    // the sequence's first padded tile
    const int tid = threadIdx.x;

    // ---- query block means (TPB 64-token tiles each; the padded sequence
    // holds whole blocks, so every one of them exists)
    constexpr int TPB = kSparseBlockM / kTile;
    for (int i = tid; i < kSelectGroup * D; i += 256) {
        const int jq = i / D, c = i % D;
        float v = 0.f;
        if (jq < nq) {
            const int t = t0 + TPB * (kSelectGroup * g + jq);
            const int64_t o = ((int64_t)h * a.ntiles + t) * D + c;
            int cnt = 0;
            float sum = 0.f;
#pragma unroll
            for (int u = 0; u < TPB; ++u) {
                cnt += a.cnt[t + u];
                sum += a.qsum[o + (int64_t)u * D];
            }
            v = sum / (float)max(cnt, 1);
        }
        qv[jq][c] = v;
    }
    __syncthreads();

    // ---- order keys of the pooled scores
    for (int t = tid; t < ntk; t += 256) {
        float sc[kSelectGroup] = {0.f, 0.f, 0.f, 0.f};
        // kbar is channel-major: the lanes of a wave read consecutive tiles of one channel
        const float *kc = a.kbar + (int64_t)h * D * a.ntiles + t0 + t;
#pragma unroll 8
        for (int c = 0; c < D; ++c) {
            const float kv = kc[(int64_t)c * a.ntiles];
#pragma unroll
            for (int jq = 0; jq < kSelectGroup; ++jq) sc[jq] = fmaf(kv, qv[jq][c], sc[jq]);
        }
#pragma unroll
        for (int jq = 0; jq < kSelectGroup; ++jq) ukey[jq][t] = ord_key(sc[jq]);
    }
    __syncthreads();

    const int L = min(a.tpb, ntk);
    for (int jq = 0; jq < nq; ++jq) {
        // ---- radix select of the L-th largest key, 8 bits at a time from the top
        uint32_t prefix = 0, mask = 0;
        uint32_t need = (uint32_t)L;
        for (int shift = 24; shift >= 0; shift -= 8) {
            hist[tid] = 0;
            __syncthreads();
            for (int t = tid; t < ntk; t += 256) {
                const uint32_t k = ukey[jq][t];
                if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                uint32_t cum = 0;
                int bin = 255;
                for (; bin > 0; --bin) {
                    if (cum + hist[bin] >= need) break;
                    cum += hist[bin];
                }
                bc[0] = (uint32_t)bin;
                bc[1] = cum;
            }
            __syncthreads();
            prefix |= bc[0] << shift;
            mask |= 255u << shift;
            need -= bc[1];
            __syncthreads();
        }
        // prefix is the L-th largest key; keep every larger key and the first
        // `need` equal ones in tile order, and place the kept tiles in tile order
        uint32_t k8[PER];
        uint32_t eq_here = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int t = PER * tid + e;
            k8[e] = t < ntk ? ukey[jq][t] : 0u;
            eq_here += (t < ntk && k8[e] == prefix) ? 1u : 0u;
        }
        uint32_t tot;
        uint32_t eq_rank = block_exscan(eq_here, wsum, &tot);
        uint32_t kept_here = 0;
        bool keep[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int t = PER * tid + e;
            const bool valid = t < ntk;
            const bool eq = valid && k8[e] == prefix;
            keep[e] = valid && (k8[e] > prefix || (eq && eq_rank < need));
            eq_rank += eq ? 1u : 0u;
            kept_here += keep[e] ? 1u : 0u;
        }
        uint32_t pos = block_exscan(kept_here, wsum, &tot);
        const int qb = kSelectGroup * g + jq;
        int32_t *dst = a.tiles + ((int64_t)a.item_base[s] + (int64_t)h * nqb + qb) * a.tpb;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            if (keep[e]) dst[pos++] = PER * tid + e;
        for (int i = L + tid; i < a.tpb; i += 256) dst[i] = -1;
        __syncthreads();
    }
}

template __global__ void sparse_pool_kernel<64>(SparseSelectArgs);
template __global__ void sparse_pool_kernel<128>(SparseSelectArgs);
template __global__ void sparse_select_kernel<64>(SparseSelectArgs);
template __global__ void sparse_select_kernel<128>(SparseSelectArgs);

hipError_t launch_sparse_select(const SparseSelectArgs &a, int d, hipStream_t st)
{
    const dim3 pool((unsigned)((int64_t)a.ntiles * a.H)), sel((unsigned)a.group_pre[a.seq.S]);
    if (d == 128) {
        hipLaunchKernelGGL(sparse_pool_kernel<128>, pool, dim3(256), 0, st, a);
        if (a.group_pre[a.seq.S] > 0) hipLaunchKernelGGL(sparse_select_kernel<128>, sel, dim3(256), 0, st, a);
    } else {
        hipLaunchKernelGGL(sparse_pool_kernel<64>, pool, dim3(256), 0, st, a);
        if (a.group_pre[a.seq.S] > 0) hipLaunchKernelGGL(sparse_select_kernel<64>, sel, dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace h3
