// Host side of the C ABI declared in include/h3attn.h: argument checks,
// workspace plan, work ordering and kernel launches.  Every check runs on the
// host before any HIP call, so invalid arguments are reported without a GPU.
#include "h3attn.h"
#include "h3_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>

using namespace h3;

namespace {

thread_local std::string g_last_error;

h3attn_status fail(h3attn_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

h3attn_status ok()
{
    g_last_error.clear();
    return H3ATTN_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Shape, stride and cu_seqlens checks; fills the workspace plan.
h3attn_status make_plan(const h3attn_params *p, const int32_t *cu, Plan *pl)
{
    if (!p) return fail(H3ATTN_ERR_INVALID_ARG, "params is NULL");
    if (!cu) return fail(H3ATTN_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
    if (p->num_heads < 1) return fail(H3ATTN_ERR_INVALID_ARG, "num_heads must be >= 1 (got %d)", p->num_heads);
    if (p->num_heads > 4096) return fail(H3ATTN_ERR_UNSUPPORTED, "num_heads %d > 4096", p->num_heads);
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(H3ATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
    if (p->num_seqs < 1 || p->num_seqs > H3ATTN_MAX_SEQS)
        return fail(H3ATTN_ERR_INVALID_ARG, "num_seqs must be in [1, %d] (got %d)", H3ATTN_MAX_SEQS, p->num_seqs);
    if (p->flags != 0) return fail(H3ATTN_ERR_INVALID_ARG, "flags must be 0");
    const int64_t hd = (int64_t)p->num_heads * p->head_dim;
    const int64_t strides[4] = {p->q_stride, p->k_stride, p->v_stride, p->o_stride};
    const char *names[4] = {"q_stride", "k_stride", "v_stride", "o_stride"};
    for (int i = 0; i < 4; ++i) {
        if (strides[i] < hd)
            return fail(H3ATTN_ERR_INVALID_ARG, "%s %lld < num_heads*head_dim %lld", names[i],
                        (long long)strides[i], (long long)hd);
        if (strides[i] % 8)
            return fail(H3ATTN_ERR_INVALID_ARG, "%s %lld is not a multiple of 8", names[i], (long long)strides[i]);
    }
    if (!(p->eps > 0.f) || !std::isfinite(p->eps))
        return fail(H3ATTN_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (!std::isfinite(p->softmax_scale)) return fail(H3ATTN_ERR_INVALID_ARG, "softmax_scale is not finite");
    if (cu[0] != 0) return fail(H3ATTN_ERR_INVALID_ARG, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
    for (int s = 0; s < p->num_seqs; ++s)
        if (cu[s + 1] < cu[s])
            return fail(H3ATTN_ERR_INVALID_ARG, "cu_seqlens decreases at %d (%d -> %d)", s, cu[s], cu[s + 1]);
    // The attention kernels address one (sequence, head) slice of the K and V
    // copies through a buffer descriptor whose size and offsets are 32-bit
    // signed values: its bf16 slice (whole 64-token tiles) must stay below 2 GiB.
    const int64_t max_seq = (((int64_t)1 << 31) / (2 * (int64_t)p->head_dim)) / kTile * kTile - kTile;
    for (int s = 0; s < p->num_seqs; ++s)
        if ((int64_t)cu[s + 1] - cu[s] > max_seq)
            return fail(H3ATTN_ERR_UNSUPPORTED, "sequence %d has %lld tokens; at head_dim %d at most %lld fit the "
                        "kernels' 2 GiB per-(sequence, head) K/V buffer range", s,
                        (long long)cu[s + 1] - cu[s], p->head_dim, (long long)max_seq);
    std::memset(pl, 0, sizeof *pl);
    pl->S = p->num_seqs;
    pl->H = p->num_heads;
    pl->d = p->head_dim;
    pl->N = cu[p->num_seqs];
    int64_t off = 0;
    for (int s = 0; s <= p->num_seqs; ++s) {
        pl->cu[s] = cu[s];
        pl->off[s] = (int32_t)off;
        if (s < p->num_seqs) off += round_up(cu[s + 1] - cu[s], kSeqPad);
        if (off > INT32_MAX - kSeqPad) return fail(H3ATTN_ERR_UNSUPPORTED, "too many tokens");
    }
    pl->Npad = off;
    const int64_t H = pl->H, d = pl->d, Np = pl->Npad, T = Np / kTile, S = pl->S;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        size_t o = at;
        at = (size_t)round_up((int64_t)(at + bytes), 256);
        return o;
    };
    pl->qhat = take(H * Np * d * 2);
    pl->khat = take(H * Np * d * 2);
    pl->vt = take(H * Np * d * 2);
    pl->knorm = take(H * T * 4);
    pl->bytes_bf16 = std::max<size_t>(at, 256);   // never 0: 0 reports an error
    pl->sp_kbar = take(H * T * d * 4);
    pl->sp_qsum = take(H * T * d * 4);
    pl->sp_cnt = take(T * 4);
    pl->bytes_sparse = std::max<size_t>(at, 256);
    at = 0;
    pl->q8 = take(H * Np * d);
    pl->k8 = take(H * Np * d);
    pl->v8t = take(H * Np * d);
    pl->qscale = take(H * T * 4);
    pl->kscale = take(H * T * 4);
    pl->ksum = take(H * T * d * 4);
    pl->vmax = take(H * T * d * 4);
    pl->kmean = take(S * H * d * 4);
    pl->vscale = take(S * H * d * 4);
    pl->bytes_q8 = std::max<size_t>(at, 256);
    pl->k32 = take(H * Np * d * 4);
    pl->v16 = take(H * Np * d * 2);
    pl->bytes_q8p = std::max<size_t>(at, 256);
    at = 0;
    pl->qx = take(H * Np * d / 2);
    pl->qxs = take(H * Np * d / 32);
    pl->kx = take(H * Np * d / 2);
    pl->kxs = take(H * T * 256);
    pl->vxt = take(H * Np * d / 2);
    pl->vxs = take(H * T * 256);
    pl->mx_ksum = take(H * T * d * 4);
    pl->mx_kmean = take(S * H * d * 4);
    pl->bytes_mx = std::max<size_t>(at, 256);
    return H3ATTN_OK;
}

bool fault_injected();

h3attn_status check_device()
{
    if (fault_injected()) return H3ATTN_OK;   // nothing will be launched
    static std::atomic<int> checked[64];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(H3ATTN_ERR_DEVICE, "no HIP device: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64 && checked[dev].load() == 1) return H3ATTN_OK;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(H3ATTN_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(H3ATTN_ERR_DEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
    if (dev >= 0 && dev < 64) checked[dev].store(1);
    return H3ATTN_OK;
}

h3attn_status check_ptrs(const void *q, const void *k, const void *v, const float *norm_w,
                         const float *rope, const void *out)
{
    const void *ps[6] = {q, k, v, norm_w, rope, out};
    const char *names[6] = {"q", "k", "v", "norm_w", "rope_tables", "out"};
    for (int i = 0; i < 6; ++i) {
        if (!ps[i]) return fail(H3ATTN_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned(ps[i], 16)) return fail(H3ATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    return H3ATTN_OK;
}

SeqTable seq_table(const Plan &pl)
{
    SeqTable t;
    std::memset(&t, 0, sizeof t);
    t.S = pl.S;
    for (int s = 0; s <= pl.S; ++s) {
        t.cu[s] = pl.cu[s];
        t.off[s] = pl.off[s];
    }
    return t;
}

PrologueArgs prologue_args(const h3attn_params *p, const Plan &pl, const void *q, const void *k,
                           const void *v, const float *norm_w, const float *rope)
{
    PrologueArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.q_stride = p->q_stride;
    a.k_stride = p->k_stride;
    a.v_stride = p->v_stride;
    a.norm_w = norm_w;
    a.rope = rope;
    a.H = pl.H;
    a.Npad = pl.Npad;
    a.eps = p->eps;
    a.q_mult = 1.0f;
    a.ntiles = (int32_t)(pl.Npad / kTile);
    a.seq = seq_table(pl);
    return a;
}

float scale_log2(const h3attn_params *p)
{
    const double s = p->softmax_scale > 0.f ? (double)p->softmax_scale : 1.0 / std::sqrt((double)p->head_dim);
    return (float)(s * 1.4426950408889634);
}

// Sequences with work, longest first (stable), and the work-item prefix for
// query blocks of block_m rows.
template <class Args>
int64_t order_work(const Plan &pl, Args &a, int32_t *seq_idx, int block_m = kBlockM)
{
    int order[kMaxSeqs];
    std::iota(order, order + pl.S, 0);
    std::stable_sort(order, order + pl.S, [&](int x, int y) {
        return pl.cu[x + 1] - pl.cu[x] > pl.cu[y + 1] - pl.cu[y];
    });
    int64_t items = 0;
    int k = 0;
    a.item_pre[0] = 0;
    for (int i = 0; i < pl.S; ++i) {
        const int s = order[i];
        const int n = pl.cu[s + 1] - pl.cu[s];
        if (n == 0) continue;
        a.seq_n[k] = n;
        a.seq_cu[k] = pl.cu[s];
        a.seq_off[k] = pl.off[s];
        a.seq_nqb[k] = (n + block_m - 1) / block_m;
        if (seq_idx) seq_idx[k] = s;
        items += (int64_t)pl.H * a.seq_nqb[k];
        a.item_pre[k + 1] = (int32_t)items;
        ++k;
    }
    a.nseq = k;
    for (int i = k + 1; i <= kMaxSeqs; ++i) a.item_pre[i] = (int32_t)items;
    return items;
}

bool env_is(const char *name, const char *value)
{
    const char *e = std::getenv(name);
    return e && std::strcmp(e, value) == 0;
}

// Host-side fault injection for tests of the error path: with the environment
// variable H3ATTN_FAULT=launch, a call that passes every argument check makes no
// HIP call at all (no device check, no launch) and reports its first launch as
// failed.  Read on every call, so a test can switch it in-process.
bool fault_injected() { return env_is("H3ATTN_FAULT", "launch"); }

// Issues one launch (or device copy) and turns its hipError_t into a status.
// With H3ATTN_DEBUG=1 it then waits for the stream and reports an execution
// error as well, naming the launch (this synchronises, so it is not for graph
// capture or timing).
template <class Launch>
h3attn_status launch_status(hipStream_t stream, const char *what, Launch &&launch)
{
    if (fault_injected())
        return fail(H3ATTN_ERR_HIP, "%s: injected failure (H3ATTN_FAULT=launch), nothing was launched", what);
    hipError_t e = launch();
    if (e != hipSuccess) return fail(H3ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    if (env_is("H3ATTN_DEBUG", "1")) {
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess)
            return fail(H3ATTN_ERR_HIP, "%s (checked by H3ATTN_DEBUG=1 after the stream drained): %s", what,
                        hipGetErrorString(e));
    }
    return ok();
}

}  // namespace

extern "C" {

int h3attn_version(void) { return H3ATTN_VERSION; }

const char *h3attn_status_string(h3attn_status s)
{
    switch (s) {
    case H3ATTN_OK: return "H3ATTN_OK";
    case H3ATTN_ERR_INVALID_ARG: return "H3ATTN_ERR_INVALID_ARG";
    case H3ATTN_ERR_UNSUPPORTED: return "H3ATTN_ERR_UNSUPPORTED";
    case H3ATTN_ERR_WORKSPACE: return "H3ATTN_ERR_WORKSPACE";
    case H3ATTN_ERR_DEVICE: return "H3ATTN_ERR_DEVICE";
    case H3ATTN_ERR_HIP: return "H3ATTN_ERR_HIP";
    }
    return "H3ATTN_UNKNOWN_STATUS";
}

const char *h3attn_last_error(void) { return g_last_error.c_str(); }

size_t h3attn_workspace_size(const h3attn_params *p, const int32_t *cu_seqlens_host, int quantized)
{
    Plan pl;
    if (make_plan(p, cu_seqlens_host, &pl) != H3ATTN_OK) return 0;
    if (quantized < 0 || quantized > 4) {
        fail(H3ATTN_ERR_INVALID_ARG, "quantized must be 0, 1, 2, 3 or 4 (got %d)", quantized);
        return 0;
    }
    if ((quantized == 1 || quantized == 3 || quantized == 4) && pl.d != 128) {
        fail(H3ATTN_ERR_UNSUPPORTED, "the quantised paths need head_dim 128");
        return 0;
    }
    ok();
    switch (quantized) {
    case 1: return pl.bytes_q8;
    case 2: return pl.bytes_sparse;
    case 3: return pl.bytes_mx;
    case 4: return pl.bytes_q8p;
    default: return pl.bytes_bf16;
    }
}

h3attn_status h3attn_fwd_stages(const h3attn_params *p, const void *q, const void *k, const void *v,
                                const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                                void *out, void *workspace, size_t workspace_bytes, void *stream, int stages)
{
    Plan pl;
    h3attn_status st = make_plan(p, cu_seqlens_host, &pl);
    if (st != H3ATTN_OK) return st;
    if (stages < 1 || stages > 3) return fail(H3ATTN_ERR_INVALID_ARG, "stages must be 1, 2 or 3 (got %d)", stages);
    if (pl.N == 0) return ok();   // nothing is read or written; pointers may be NULL
    if ((st = check_ptrs(q, k, v, norm_w, rope_tables, out)) != H3ATTN_OK) return st;
    if (!workspace) return fail(H3ATTN_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(H3ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < pl.bytes_bf16)
        return fail(H3ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes_bf16);
    if ((st = check_device()) != H3ATTN_OK) return st;
    if (pl.N == 0) return ok();
    hipStream_t hs = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);

    PrologueArgs pa = prologue_args(p, pl, q, k, v, norm_w, rope_tables);
    pa.qhat = reinterpret_cast<uint16_t *>(ws + pl.qhat);
    pa.khat = reinterpret_cast<uint16_t *>(ws + pl.khat);
    pa.vt = reinterpret_cast<uint16_t *>(ws + pl.vt);
    pa.knorm = reinterpret_cast<float *>(ws + pl.knorm);
    pa.out_hstride = pl.Npad * pl.d;
    pa.out_tstride = pl.d;
    pa.natural = 0;
    pa.q_mult = scale_log2(p);
    if (stages & 1)
        if ((st = launch_status(hs, "prologue launch",
                [&] { return launch_prologue(pa, pl.d, hs); })) != H3ATTN_OK) return st;
    if (!(stages & 2)) return ok();

    AttnArgs aa;
    std::memset(&aa, 0, sizeof aa);
    aa.qhat = pa.qhat;
    aa.khat = pa.khat;
    aa.vt = pa.vt;
    aa.knorm = pa.knorm;
    aa.out = static_cast<uint16_t *>(out);
    aa.o_stride = p->o_stride;
    aa.Npad = pl.Npad;
    aa.H = pl.H;
    const int64_t items = order_work(pl, aa, nullptr, attn_bf16_block_m(pl.d));
    return launch_status(hs, "attention launch", [&] { return launch_attn_bf16(aa, pl.d, items, hs); });
}

h3attn_status h3attn_fwd(const h3attn_params *p, const void *q, const void *k, const void *v,
                         const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                         void *out, void *workspace, size_t workspace_bytes, void *stream)
{
    return h3attn_fwd_stages(p, q, k, v, norm_w, rope_tables, cu_seqlens_host, out, workspace,
                             workspace_bytes, stream, 3);
}

}  // extern "C"

// ---- the static workspace of h3attn_fwd_static (callers that cannot allocate)
//
// A file-scope device array: each device that runs h3attn_fwd_static holds its
// own copy, at its own address, until the process ends.  In host code the name
// `scratch` only identifies the variable for the address lookup; it is not a
// device address and is never passed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[H3ATTN_STATIC_WORKSPACE_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_dev[64];      // device address of `scratch` per device, looked up once

// This device's address of `scratch`, looked up on the first call with the
// device current and kept per device.
h3attn_status scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(H3ATTN_ERR_DEVICE, "no HIP device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(H3ATTN_ERR_DEVICE, "device index %d is outside 0..63", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(H3ATTN_ERR_HIP, "hipGetSymbolAddress of the static workspace on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return H3ATTN_OK;
}

}  // namespace

extern "C" {

h3attn_status h3attn_fwd_static(const h3attn_params *p, const void *q, const void *k, const void *v,
                                const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                                void *out, void *stream)
{
    Plan pl;
    h3attn_status st = make_plan(p, cu_seqlens_host, &pl);
    if (st != H3ATTN_OK) return st;
    if (pl.N == 0) return ok();
    if ((st = check_ptrs(q, k, v, norm_w, rope_tables, out)) != H3ATTN_OK) return st;
    if (pl.bytes_bf16 > H3ATTN_STATIC_WORKSPACE_BYTES)
        return fail(H3ATTN_ERR_WORKSPACE, "this shape needs %zu bytes of workspace; the static workspace holds %zu",
                    pl.bytes_bf16, (size_t)H3ATTN_STATIC_WORKSPACE_BYTES);
    if (fault_injected())
        return launch_status(static_cast<hipStream_t>(stream), "prologue launch", [] { return hipSuccess; });
    if ((st = check_device()) != H3ATTN_OK) return st;
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != H3ATTN_OK) return st;
    return h3attn_fwd_stages(p, q, k, v, norm_w, rope_tables, cu_seqlens_host, out, ws,
                             H3ATTN_STATIC_WORKSPACE_BYTES, stream, 3);
}

h3attn_status h3attn_checked(uint32_t *flags_out, int clear, uint32_t jitter_seed)
{
#ifdef H3ATTN_CHECKED
    h3attn_status st = check_device();
    if (st != H3ATTN_OK) return st;
    uint32_t f[kCheckKinds] = {};
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = attn_checked(f, clear != 0, jitter_seed);
    if (e == hipSuccess) e = q8_checked(f, clear != 0, jitter_seed);
    if (e == hipSuccess) e = mx_checked(f, clear != 0, jitter_seed);
    if (e != hipSuccess) return fail(H3ATTN_ERR_HIP, "checked-build state: %s", hipGetErrorString(e));
    if (flags_out) std::memcpy(flags_out, f, sizeof f);
    return ok();
#else
    (void)flags_out;
    (void)clear;
    (void)jitter_seed;
    return fail(H3ATTN_ERR_UNSUPPORTED, "this library is built without checks (the checked build is "
                "libh3attn_checked.so)");
#endif
}

h3attn_status h3attn_mfma_ceiling(int mix, int workgroups, int iters, float *out, void *stream)
{
    if (mix < 0 || mix > 5) return fail(H3ATTN_ERR_INVALID_ARG, "mix must be in 0..5 (got %d)", mix);
    if (workgroups < 1 || workgroups > (1 << 20))
        return fail(H3ATTN_ERR_INVALID_ARG, "workgroups must be in [1, 2^20] (got %d)", workgroups);
    if (iters < 1 || iters > (1 << 20)) return fail(H3ATTN_ERR_INVALID_ARG, "iters must be in [1, 2^20] (got %d)", iters);
    if (!out) return fail(H3ATTN_ERR_INVALID_ARG, "out is NULL");
    if (!aligned(out, 4)) return fail(H3ATTN_ERR_INVALID_ARG, "out is not 4-byte aligned");
    h3attn_status st;
    if ((st = check_device()) != H3ATTN_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return launch_status(hs, "mfma ceiling launch", [&] { return launch_mfma_ceiling(mix, workgroups, iters, out, hs); });
}

h3attn_status h3attn_prologue(const h3attn_params *p, const void *q, const void *k, const float *norm_w,
                              const float *rope_tables, const int32_t *cu_seqlens_host, void *q_hat,
                              void *k_hat, void *stream)
{
    Plan pl;
    h3attn_status st = make_plan(p, cu_seqlens_host, &pl);
    if (st != H3ATTN_OK) return st;
    if (pl.N == 0) return ok();
    if ((st = check_ptrs(q, k, q, norm_w, rope_tables, q_hat)) != H3ATTN_OK) return st;
    if (!k_hat) return fail(H3ATTN_ERR_INVALID_ARG, "k_hat is NULL");
    if (!aligned(k_hat, 16)) return fail(H3ATTN_ERR_INVALID_ARG, "k_hat is not 16-byte aligned");
    if ((st = check_device()) != H3ATTN_OK) return st;
    if (pl.N == 0) return ok();
    PrologueArgs pa = prologue_args(p, pl, q, k, q, norm_w, rope_tables);
    pa.qhat = static_cast<uint16_t *>(q_hat);
    pa.khat = static_cast<uint16_t *>(k_hat);
    pa.vt = nullptr;
    pa.out_hstride = pl.d;
    pa.out_tstride = (int64_t)pl.H * pl.d;
    pa.natural = 1;
    return launch_status(static_cast<hipStream_t>(stream), "prologue launch",
            [&] { return launch_prologue(pa, pl.d, static_cast<hipStream_t>(stream)); });
}

// Checks of the projection entry points' own arguments; fills the plan.  The
// q/k/v strides of the params are not read by these entry points.
static h3attn_status proj_plan(const h3attn_params *p, int32_t model_dim, int64_t x_stride,
                               const int32_t *cu, Plan &pl)
{
    if (!p) return fail(H3ATTN_ERR_INVALID_ARG, "params is NULL");
    h3attn_params pp = *p;
    pp.q_stride = pp.k_stride = pp.v_stride = (int64_t)p->num_heads * p->head_dim;
    h3attn_status st = make_plan(&pp, cu, &pl);
    if (st != H3ATTN_OK) return st;
    if (model_dim < 32 || model_dim % 32)
        return fail(H3ATTN_ERR_INVALID_ARG, "model_dim must be a positive multiple of 32 (got %d)", model_dim);
    if (x_stride < model_dim || x_stride % 8)
        return fail(H3ATTN_ERR_INVALID_ARG, "x_stride %lld must be >= model_dim %d and a multiple of 8",
                    (long long)x_stride, model_dim);
    // 32-bit buffer offsets: one 256-token block of x, one head's rows of W
    if ((int64_t)255 * x_stride * 2 + (int64_t)model_dim * 2 >= ((int64_t)1 << 31))
        return fail(H3ATTN_ERR_UNSUPPORTED, "x_stride %lld is too large", (long long)x_stride);
    if ((int64_t)pl.d * model_dim * 2 >= ((int64_t)1 << 31))
        return fail(H3ATTN_ERR_UNSUPPORTED, "model_dim %d is too large", model_dim);
    return H3ATTN_OK;
}

static ProjArgs proj_args(const h3attn_params *p, const Plan &pl, int32_t model_dim, const void *x,
                          int64_t x_stride, const void *w_qkv, const float *norm_w, const float *rope)
{
    ProjArgs a;
    std::memset(&a, 0, sizeof a);
    a.x = static_cast<const uint16_t *>(x);
    a.w = static_cast<const uint16_t *>(w_qkv);
    a.x_stride = x_stride;
    a.model_dim = model_dim;
    a.norm_w = norm_w;
    a.rope = rope;
    a.H = pl.H;
    a.Npad = pl.Npad;
    a.ntiles = (int32_t)(pl.Npad / kTile);
    a.nblk = (int32_t)(pl.Npad / kSeqPad);
    a.eps = p->eps;
    a.q_mult = 1.0f;
    a.seq = seq_table(pl);
    return a;
}

h3attn_status h3attn_fwd_proj_stages(const h3attn_params *p, int32_t model_dim, const void *x, int64_t x_stride,
                                     const void *w_qkv, const float *norm_w, const float *rope_tables,
                                     const int32_t *cu_seqlens_host, void *out, void *workspace,
                                     size_t workspace_bytes, void *stream, int stages)
{
    Plan pl;
    h3attn_status st = proj_plan(p, model_dim, x_stride, cu_seqlens_host, pl);
    if (st != H3ATTN_OK) return st;
    if (stages < 1 || stages > 3) return fail(H3ATTN_ERR_INVALID_ARG, "stages must be 1, 2 or 3 (got %d)", stages);
    if (pl.N == 0) return ok();
    if ((st = check_ptrs(x, w_qkv, x, norm_w, rope_tables, out)) != H3ATTN_OK) return st;
    if (!workspace) return fail(H3ATTN_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(H3ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < pl.bytes_bf16)
        return fail(H3ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes_bf16);
    if ((st = check_device()) != H3ATTN_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);

    ProjArgs pa = proj_args(p, pl, model_dim, x, x_stride, w_qkv, norm_w, rope_tables);
    pa.qhat = reinterpret_cast<uint16_t *>(ws + pl.qhat);
    pa.khat = reinterpret_cast<uint16_t *>(ws + pl.khat);
    pa.vt = reinterpret_cast<uint16_t *>(ws + pl.vt);
    pa.knorm = reinterpret_cast<float *>(ws + pl.knorm);
    pa.out_hstride = pl.Npad * pl.d;
    pa.out_tstride = pl.d;
    pa.natural = 0;
    pa.q_mult = scale_log2(p);
    if (stages & 1)
        if ((st = launch_status(hs, "projection launch",
                [&] { return launch_qkv_proj(pa, pl.d, hs); })) != H3ATTN_OK) return st;
    if (!(stages & 2)) return ok();

    AttnArgs aa;
    std::memset(&aa, 0, sizeof aa);
    aa.qhat = pa.qhat;
    aa.khat = pa.khat;
    aa.vt = pa.vt;
    aa.knorm = pa.knorm;
    aa.out = static_cast<uint16_t *>(out);
    aa.o_stride = p->o_stride;
    aa.Npad = pl.Npad;
    aa.H = pl.H;
    const int64_t items = order_work(pl, aa, nullptr, attn_bf16_block_m(pl.d));
    return launch_status(hs, "attention launch", [&] { return launch_attn_bf16(aa, pl.d, items, hs); });
}

h3attn_status h3attn_fwd_proj(const h3attn_params *p, int32_t model_dim, const void *x, int64_t x_stride,
                              const void *w_qkv, const float *norm_w, const float *rope_tables,
                              const int32_t *cu_seqlens_host, void *out, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    return h3attn_fwd_proj_stages(p, model_dim, x, x_stride, w_qkv, norm_w, rope_tables, cu_seqlens_host, out,
                                  workspace, workspace_bytes, stream, 3);
}

h3attn_status h3attn_proj_prologue(const h3attn_params *p, int32_t model_dim, const void *x, int64_t x_stride,
                                   const void *w_qkv, const float *norm_w, const float *rope_tables,
                                   const int32_t *cu_seqlens_host, void *q_hat, void *k_hat, void *v_out,
                                   void *stream)
{
    Plan pl;
    h3attn_status st = proj_plan(p, model_dim, x_stride, cu_seqlens_host, pl);
    if (st != H3ATTN_OK) return st;
    if (pl.N == 0) return ok();
    if ((st = check_ptrs(x, w_qkv, k_hat, norm_w, rope_tables, q_hat)) != H3ATTN_OK) return st;
    if (!v_out) return fail(H3ATTN_ERR_INVALID_ARG, "v_out is NULL");
    if (!aligned(v_out, 16)) return fail(H3ATTN_ERR_INVALID_ARG, "v_out is not 16-byte aligned");
    if ((st = check_device()) != H3ATTN_OK) return st;
    ProjArgs pa = proj_args(p, pl, model_dim, x, x_stride, w_qkv, norm_w, rope_tables);
    pa.qhat = static_cast<uint16_t *>(q_hat);
    pa.khat = static_cast<uint16_t *>(k_hat);
    pa.vt = static_cast<uint16_t *>(v_out);
    pa.out_hstride = pl.d;
    pa.out_tstride = (int64_t)pl.H * pl.d;
    pa.natural = 1;
    return launch_status(static_cast<hipStream_t>(stream), "projection launch",
            [&] { return launch_qkv_proj(pa, pl.d, static_cast<hipStream_t>(stream)); });
}

h3attn_status h3attn_out_proj(int32_t num_heads, int32_t head_dim, int32_t model_dim, int32_t num_seqs,
                              const int32_t *cu_seqlens_host, const void *attn, int64_t attn_stride,
                              const void *w_o, const float *gate, const void *resid, int64_t resid_stride,
                              void *out, int64_t out_stride, void *stream)
{
    if (num_heads < 1) return fail(H3ATTN_ERR_INVALID_ARG, "num_heads must be >= 1 (got %d)", num_heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(H3ATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
    if (num_seqs < 1 || num_seqs > H3ATTN_MAX_SEQS)
        return fail(H3ATTN_ERR_INVALID_ARG, "num_seqs must be in [1, %d] (got %d)", H3ATTN_MAX_SEQS, num_seqs);
    if (!cu_seqlens_host) return fail(H3ATTN_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
    const int32_t *cu = cu_seqlens_host;
    if (cu[0] != 0) return fail(H3ATTN_ERR_INVALID_ARG, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
    for (int s = 0; s < num_seqs; ++s)
        if (cu[s + 1] < cu[s])
            return fail(H3ATTN_ERR_INVALID_ARG, "cu_seqlens decreases at %d (%d -> %d)", s, cu[s], cu[s + 1]);
    if (model_dim < 128 || model_dim % 128)
        return fail(H3ATTN_ERR_INVALID_ARG, "model_dim must be a positive multiple of 128 (got %d)", model_dim);
    const int64_t K = (int64_t)num_heads * head_dim;
    if (attn_stride < K || attn_stride % 8)
        return fail(H3ATTN_ERR_INVALID_ARG, "attn_stride %lld must be >= num_heads*head_dim %lld and a multiple of 8",
                    (long long)attn_stride, (long long)K);
    if (out_stride < model_dim || out_stride % 8)
        return fail(H3ATTN_ERR_INVALID_ARG, "out_stride %lld must be >= model_dim %d and a multiple of 8",
                    (long long)out_stride, model_dim);
    if (resid && (resid_stride < model_dim || resid_stride % 8))
        return fail(H3ATTN_ERR_INVALID_ARG, "resid_stride %lld must be >= model_dim %d and a multiple of 8",
                    (long long)resid_stride, model_dim);
    // 32-bit buffer offsets: one 256-token block of attn, 256 rows of W_o
    if ((int64_t)255 * attn_stride * 2 + K * 2 >= ((int64_t)1 << 31))
        return fail(H3ATTN_ERR_UNSUPPORTED, "attn_stride %lld is too large", (long long)attn_stride);
    if ((int64_t)256 * K * 2 >= ((int64_t)1 << 31))
        return fail(H3ATTN_ERR_UNSUPPORTED, "num_heads * head_dim %lld is too large", (long long)K);
    const int64_t N = cu[num_seqs];
    if (N == 0) return ok();
    const void *ps[3] = {attn, w_o, out};
    const char *names[3] = {"attn", "w_o", "out"};
    for (int i = 0; i < 3; ++i) {
        if (!ps[i]) return fail(H3ATTN_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned(ps[i], 16)) return fail(H3ATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    if (gate && !aligned(gate, 16)) return fail(H3ATTN_ERR_INVALID_ARG, "gate is not 16-byte aligned");
    if (resid && !aligned(resid, 16)) return fail(H3ATTN_ERR_INVALID_ARG, "resid is not 16-byte aligned");
    if (resid && resid != out) {
        // out may be the residual itself (same pointer and stride) but not a partial overlap of it
        const char *r0 = static_cast<const char *>(resid), *o0 = static_cast<const char *>(out);
        const char *r1 = r0 + ((N - 1) * resid_stride + model_dim) * 2, *o1 = o0 + ((N - 1) * out_stride + model_dim) * 2;
        if (r0 < o1 && o0 < r1) return fail(H3ATTN_ERR_INVALID_ARG, "out overlaps resid without being resid");
    }
    if (resid && resid == out && resid_stride != out_stride)
        return fail(H3ATTN_ERR_INVALID_ARG, "out is resid but with another stride");
    h3attn_status st = check_device();
    if (st != H3ATTN_OK) return st;
    OutProjArgs a;
    std::memset(&a, 0, sizeof a);
    a.attn = static_cast<const uint16_t *>(attn);
    a.w = static_cast<const uint16_t *>(w_o);
    a.attn_stride = attn_stride;
    a.K = (int32_t)K;
    a.model_dim = model_dim;
    a.gate = gate;
    a.resid = static_cast<const uint16_t *>(resid);
    a.resid_stride = resid_stride;
    a.out = static_cast<uint16_t *>(out);
    a.out_stride = out_stride;
    a.N = N;
    a.nblk = (int32_t)((N + 255) / 256);
    a.S = num_seqs;
    for (int s = 0; s <= num_seqs; ++s) a.cu[s] = cu[s];
    return launch_status(static_cast<hipStream_t>(stream), "output projection launch",
            [&] { return launch_out_proj(a, static_cast<hipStream_t>(stream)); });
}

// Query blocks (tile lists) of a sequence of n tokens on the block-sparse path.
static int64_t sparse_blocks(int64_t n) { return (n + kSparseBlockM - 1) / kSparseBlockM; }

// Caller-order item bases of the block-sparse lists: items run sequence by
// sequence, then head, then kSparseBlockM-row query block.
static void sparse_item_base(const Plan &pl, int32_t *base, int64_t *total)
{
    int64_t at = 0;
    for (int s = 0; s < pl.S; ++s) {
        base[s] = (int32_t)at;
        at += (int64_t)pl.H * sparse_blocks(pl.cu[s + 1] - pl.cu[s]);
    }
    *total = at;
}

h3attn_status h3attn_fwd_sparse_stages(const h3attn_params *p, const void *q, const void *k, const void *v,
                                       const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                                       int32_t tiles_per_block, int32_t *block_tiles, void *out, void *workspace,
                                       size_t workspace_bytes, void *stream, int stages)
{
    Plan pl;
    h3attn_status st = make_plan(p, cu_seqlens_host, &pl);
    if (st != H3ATTN_OK) return st;
    if (stages < 1 || stages > 7) return fail(H3ATTN_ERR_INVALID_ARG, "stages must be in 1..7 (got %d)", stages);
    if (tiles_per_block < 1 || tiles_per_block > kMaxSparseTiles)
        return fail(H3ATTN_ERR_INVALID_ARG, "tiles_per_block must be in [1, %d] (got %d)", kMaxSparseTiles,
                    tiles_per_block);
    for (int s = 0; s < pl.S; ++s)
        if ((pl.cu[s + 1] - pl.cu[s] + kTile - 1) / kTile > kMaxSparseTiles)
            return fail(H3ATTN_ERR_UNSUPPORTED, "sequence %d has %d tokens; the sparse path takes at most %d", s,
                        pl.cu[s + 1] - pl.cu[s], kMaxSparseTiles * kTile);
    if (pl.N == 0) return ok();
    if ((st = check_ptrs(q, k, v, norm_w, rope_tables, out)) != H3ATTN_OK) return st;
    if (!block_tiles) return fail(H3ATTN_ERR_INVALID_ARG, "block_tiles is NULL");
    if (!aligned(block_tiles, 4)) return fail(H3ATTN_ERR_INVALID_ARG, "block_tiles is not 4-byte aligned");
    if (!workspace) return fail(H3ATTN_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(H3ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    const size_t need = (stages & 2) ? pl.bytes_sparse : pl.bytes_bf16;
    if (workspace_bytes < need)
        return fail(H3ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if ((st = check_device()) != H3ATTN_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    int32_t base[kMaxSeqs];
    int64_t nitems_caller;
    sparse_item_base(pl, base, &nitems_caller);

    PrologueArgs pa = prologue_args(p, pl, q, k, v, norm_w, rope_tables);
    pa.qhat = reinterpret_cast<uint16_t *>(ws + pl.qhat);
    pa.khat = reinterpret_cast<uint16_t *>(ws + pl.khat);
    pa.vt = reinterpret_cast<uint16_t *>(ws + pl.vt);
    pa.knorm = reinterpret_cast<float *>(ws + pl.knorm);
    pa.out_hstride = pl.Npad * pl.d;
    pa.out_tstride = pl.d;
    pa.natural = 0;
    pa.q_mult = scale_log2(p);
    if (stages & 1)
        if ((st = launch_status(hs, "prologue launch",
                [&] { return launch_prologue(pa, pl.d, hs); })) != H3ATTN_OK) return st;

    if (stages & 2) {
        SparseSelectArgs sa;
        std::memset(&sa, 0, sizeof sa);
        sa.qhat = pa.qhat;
        sa.khat = pa.khat;
        sa.kbar = reinterpret_cast<float *>(ws + pl.sp_kbar);
        sa.qsum = reinterpret_cast<float *>(ws + pl.sp_qsum);
        sa.cnt = reinterpret_cast<int32_t *>(ws + pl.sp_cnt);
        sa.tiles = block_tiles;
        sa.tpb = tiles_per_block;
        sa.H = pl.H;
        sa.Npad = pl.Npad;
        sa.ntiles = (int32_t)(pl.Npad / kTile);
        sa.seq = seq_table(pl);
        int64_t g = 0;
        for (int s = 0; s < pl.S; ++s) {
            sa.item_base[s] = base[s];
            sa.group_pre[s] = (int32_t)g;
            g += (int64_t)pl.H * ((sparse_blocks(pl.cu[s + 1] - pl.cu[s]) + 3) / 4);
        }
        sa.group_pre[pl.S] = (int32_t)g;
        if ((st = launch_status(hs, "sparse selection launch",
                [&] { return launch_sparse_select(sa, pl.d, hs); })) != H3ATTN_OK)
            return st;
    }
    if (!(stages & 4)) return ok();

    AttnArgs aa;
    std::memset(&aa, 0, sizeof aa);
    aa.qhat = pa.qhat;
    aa.khat = pa.khat;
    aa.vt = pa.vt;
    aa.knorm = pa.knorm;
    aa.out = static_cast<uint16_t *>(out);
    aa.o_stride = p->o_stride;
    aa.Npad = pl.Npad;
    aa.H = pl.H;
    int32_t seq_idx[kMaxSeqs];
    const int64_t items = order_work(pl, aa, seq_idx, attn_bf16_block_m(pl.d));
    aa.tiles = block_tiles;
    aa.tpb = tiles_per_block;
    for (int i = 0; i < aa.nseq; ++i) aa.seq_item_base[i] = base[seq_idx[i]];
    return launch_status(hs, "sparse attention launch", [&] { return launch_attn_bf16(aa, pl.d, items, hs); });
}

h3attn_status h3attn_fwd_sparse(const h3attn_params *p, const void *q, const void *k, const void *v,
                                const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                                int32_t tiles_per_block, int32_t *block_tiles, void *out, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    return h3attn_fwd_sparse_stages(p, q, k, v, norm_w, rope_tables, cu_seqlens_host, tiles_per_block, block_tiles,
                                    out, workspace, workspace_bytes, stream, 7);
}

static h3attn_status q8_common(const h3attn_params *p, const void *q, const void *k, const void *v,
                               const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                               const void *out, void *workspace, size_t workspace_bytes, Plan &pl, Q8Args &qa)
{
    h3attn_status st = make_plan(p, cu_seqlens_host, &pl);
    if (st != H3ATTN_OK) return st;
    if (pl.d != 128) return fail(H3ATTN_ERR_UNSUPPORTED, "the quantised path needs head_dim 128 (got %d)", pl.d);
    if (pl.N == 0) return H3ATTN_OK;
    if ((st = check_ptrs(q, k, v, norm_w, rope_tables, out)) != H3ATTN_OK) return st;
    if (!workspace) return fail(H3ATTN_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(H3ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < pl.bytes_q8)
        return fail(H3ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes_q8);
    if ((st = check_device()) != H3ATTN_OK) return st;
    char *ws = static_cast<char *>(workspace);
    std::memset(&qa, 0, sizeof qa);
    qa.q = static_cast<const uint16_t *>(q);
    qa.k = static_cast<const uint16_t *>(k);
    qa.v = static_cast<const uint16_t *>(v);
    qa.q_stride = p->q_stride;
    qa.k_stride = p->k_stride;
    qa.v_stride = p->v_stride;
    qa.norm_w = norm_w;
    qa.rope = rope_tables;
    qa.q8 = reinterpret_cast<int8_t *>(ws + pl.q8);
    qa.k8 = reinterpret_cast<int8_t *>(ws + pl.k8);
    qa.v8t = reinterpret_cast<uint8_t *>(ws + pl.v8t);
    qa.qscale = reinterpret_cast<float *>(ws + pl.qscale);
    qa.kscale = reinterpret_cast<float *>(ws + pl.kscale);
    qa.ksum = reinterpret_cast<float *>(ws + pl.ksum);
    qa.vmax = reinterpret_cast<float *>(ws + pl.vmax);
    qa.kmean = reinterpret_cast<float *>(ws + pl.kmean);
    qa.vscale = reinterpret_cast<float *>(ws + pl.vscale);
    qa.H = pl.H;
    qa.Npad = pl.Npad;
    qa.eps = p->eps;
    qa.ntiles = (int32_t)(pl.Npad / kTile);
    qa.seq = seq_table(pl);
    return H3ATTN_OK;
}

h3attn_status h3attn_fwd_q8_stages(const h3attn_params *p, const void *q, const void *k, const void *v,
                                   const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                                   void *out, void *workspace, size_t workspace_bytes, void *stream, int stages)
{
    if (stages < 1 || stages > 3) return fail(H3ATTN_ERR_INVALID_ARG, "stages must be 1, 2 or 3 (got %d)", stages);
    Plan pl;
    Q8Args qa;
    h3attn_status st = q8_common(p, q, k, v, norm_w, rope_tables, cu_seqlens_host, out, workspace,
                                 workspace_bytes, pl, qa);
    if (st != H3ATTN_OK || pl.N == 0) return st == H3ATTN_OK ? ok() : st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (stages & 1)
        if ((st = launch_status(hs, "quantised prologue launch",
                [&] { return launch_q8_prep(qa, pl.d, hs); })) != H3ATTN_OK) return st;
    if (!(stages & 2)) return ok();
    Q8AttnArgs aa;
    std::memset(&aa, 0, sizeof aa);
    aa.q8 = qa.q8;
    aa.k8 = qa.k8;
    aa.v8t = qa.v8t;
    aa.qscale = qa.qscale;
    aa.kscale = qa.kscale;
    aa.vscale = qa.vscale;
    aa.out = static_cast<uint16_t *>(out);
    aa.o_stride = p->o_stride;
    aa.Npad = pl.Npad;
    aa.H = pl.H;
    aa.scale_log2 = scale_log2(p);
    const int64_t items = order_work(pl, aa, aa.seq_idx);
    return launch_status(hs, "quantised attention launch", [&] { return launch_attn_q8(aa, pl.d, items, hs); });
}

h3attn_status h3attn_fwd_q8(const h3attn_params *p, const void *q, const void *k, const void *v,
                            const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                            void *out, void *workspace, size_t workspace_bytes, void *stream)
{
    return h3attn_fwd_q8_stages(p, q, k, v, norm_w, rope_tables, cu_seqlens_host, out, workspace,
                                workspace_bytes, stream, 3);
}

static h3attn_status q8_export(const Plan &pl, const Q8Args &qa, int8_t *q8, int8_t *k8, float *q_scale,
                               float *k_scale, float *k_mean, uint8_t *v8, float *v_scale, hipStream_t hs);

h3attn_status h3attn_q8_prologue(const h3attn_params *p, const void *q, const void *k, const void *v,
                                 const float *norm_w, const float *rope_tables,
                                 const int32_t *cu_seqlens_host, void *workspace, size_t workspace_bytes,
                                 int8_t *q8, int8_t *k8, float *q_scale, float *k_scale, float *k_mean,
                                 uint8_t *v8, float *v_scale, void *stream)
{
    Plan pl;
    Q8Args qa;
    h3attn_status st = q8_common(p, q, k, v, norm_w, rope_tables, cu_seqlens_host, q8, workspace,
                                 workspace_bytes, pl, qa);
    if (st != H3ATTN_OK || pl.N == 0) return st == H3ATTN_OK ? ok() : st;
    const void *outs[6] = {k8, q_scale, k_scale, k_mean, v8, v_scale};
    const char *names[6] = {"k8", "q_scale", "k_scale", "k_mean", "v8", "v_scale"};
    for (int i = 0; i < 6; ++i)
        if (!outs[i]) return fail(H3ATTN_ERR_INVALID_ARG, "%s is NULL", names[i]);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if ((st = launch_status(hs, "quantised prologue launch",
            [&] { return launch_q8_prep(qa, pl.d, hs); })) != H3ATTN_OK) return st;
    return q8_export(pl, qa, q8, k8, q_scale, k_scale, k_mean, v8, v_scale, hs);
}

// The projection's quantised path: argument checks, plan and the arguments
// of its kernels (the projection in its quantised epilogue, the K-mean and
// coding passes reading what it wrote, the quantised attention).
static h3attn_status proj_q8_common(const h3attn_params *p, int32_t model_dim, const void *x, int64_t x_stride,
                                    const void *w_qkv, const float *norm_w, const float *rope_tables,
                                    const int32_t *cu, const void *out, void *workspace, size_t workspace_bytes,
                                    Plan &pl, ProjArgs &pa, Q8Args &qa)
{
    h3attn_status st = proj_plan(p, model_dim, x_stride, cu, pl);
    if (st != H3ATTN_OK) return st;
    if (pl.d != 128) return fail(H3ATTN_ERR_UNSUPPORTED, "the quantised path needs head_dim 128 (got %d)", pl.d);
    if (pl.N == 0) return H3ATTN_OK;
    if ((st = check_ptrs(x, w_qkv, x, norm_w, rope_tables, out)) != H3ATTN_OK) return st;
    if (!workspace) return fail(H3ATTN_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(H3ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < pl.bytes_q8p)
        return fail(H3ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes_q8p);
    if ((st = check_device()) != H3ATTN_OK) return st;
    char *ws = static_cast<char *>(workspace);
    pa = proj_args(p, pl, model_dim, x, x_stride, w_qkv, norm_w, rope_tables);
    pa.q8 = reinterpret_cast<int8_t *>(ws + pl.q8);
    pa.qscale = reinterpret_cast<float *>(ws + pl.qscale);
    pa.k32 = reinterpret_cast<float *>(ws + pl.k32);
    pa.v16 = reinterpret_cast<uint16_t *>(ws + pl.v16);
    std::memset(&qa, 0, sizeof qa);
    qa.norm_w = norm_w;
    qa.rope = rope_tables;
    qa.q8 = pa.q8;
    qa.k8 = reinterpret_cast<int8_t *>(ws + pl.k8);
    qa.v8t = reinterpret_cast<uint8_t *>(ws + pl.v8t);
    qa.qscale = pa.qscale;
    qa.kscale = reinterpret_cast<float *>(ws + pl.kscale);
    qa.ksum = reinterpret_cast<float *>(ws + pl.ksum);
    qa.vmax = reinterpret_cast<float *>(ws + pl.vmax);
    qa.kmean = reinterpret_cast<float *>(ws + pl.kmean);
    qa.vscale = reinterpret_cast<float *>(ws + pl.vscale);
    qa.k32 = pa.k32;
    qa.v16 = pa.v16;
    qa.H = pl.H;
    qa.Npad = pl.Npad;
    qa.eps = p->eps;
    qa.ntiles = (int32_t)(pl.Npad / kTile);
    qa.seq = seq_table(pl);
    return H3ATTN_OK;
}

// Stage 1 of the projection's quantised path: projection with the quantised
// epilogue, then the K means, V scales and the K / V coding.
static h3attn_status proj_q8_stage1(const Plan &pl, const ProjArgs &pa, const Q8Args &qa, hipStream_t hs)
{
    h3attn_status st = launch_status(hs, "projection launch", [&] { return launch_qkv_proj_q8(pa, hs); });
    if (st != H3ATTN_OK) return st;
    return launch_status(hs, "quantised prologue launch", [&] { return launch_q8_prep(qa, pl.d, hs); });
}

h3attn_status h3attn_fwd_proj_q8_stages(const h3attn_params *p, int32_t model_dim, const void *x, int64_t x_stride,
                                        const void *w_qkv, const float *norm_w, const float *rope_tables,
                                        const int32_t *cu_seqlens_host, void *out, void *workspace,
                                        size_t workspace_bytes, void *stream, int stages)
{
    if (stages < 1 || stages > 3) return fail(H3ATTN_ERR_INVALID_ARG, "stages must be 1, 2 or 3 (got %d)", stages);
    Plan pl;
    ProjArgs pa;
    Q8Args qa;
    h3attn_status st = proj_q8_common(p, model_dim, x, x_stride, w_qkv, norm_w, rope_tables, cu_seqlens_host, out,
                                      workspace, workspace_bytes, pl, pa, qa);
    if (st != H3ATTN_OK || pl.N == 0) return st == H3ATTN_OK ? ok() : st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if ((stages & 1) && (st = proj_q8_stage1(pl, pa, qa, hs)) != H3ATTN_OK) return st;
    if (!(stages & 2)) return ok();
    Q8AttnArgs aa;
    std::memset(&aa, 0, sizeof aa);
    aa.q8 = qa.q8;
    aa.k8 = qa.k8;
    aa.v8t = qa.v8t;
    aa.qscale = qa.qscale;
    aa.kscale = qa.kscale;
    aa.vscale = qa.vscale;
    aa.out = static_cast<uint16_t *>(out);
    aa.o_stride = p->o_stride;
    aa.Npad = pl.Npad;
    aa.H = pl.H;
    aa.scale_log2 = scale_log2(p);
    const int64_t items = order_work(pl, aa, aa.seq_idx);
    return launch_status(hs, "quantised attention launch", [&] { return launch_attn_q8(aa, pl.d, items, hs); });
}

h3attn_status h3attn_fwd_proj_q8(const h3attn_params *p, int32_t model_dim, const void *x, int64_t x_stride,
                                 const void *w_qkv, const float *norm_w, const float *rope_tables,
                                 const int32_t *cu_seqlens_host, void *out, void *workspace, size_t workspace_bytes,
                                 void *stream)
{
    return h3attn_fwd_proj_q8_stages(p, model_dim, x, x_stride, w_qkv, norm_w, rope_tables, cu_seqlens_host, out,
                                     workspace, workspace_bytes, stream, 3);
}

// Exports the quantised state in natural layouts (shared by the two
// quantised prologue diagnostics): codes and per-tile scales by the export
// kernel, the K means and V scales by device copies.
static h3attn_status q8_export(const Plan &pl, const Q8Args &qa, int8_t *q8, int8_t *k8, float *q_scale,
                               float *k_scale, float *k_mean, uint8_t *v8, float *v_scale, hipStream_t hs)
{
    Q8ExportArgs ea;
    std::memset(&ea, 0, sizeof ea);
    ea.q8 = qa.q8;
    ea.k8 = qa.k8;
    ea.v8t = qa.v8t;
    ea.qscale = qa.qscale;
    ea.kscale = qa.kscale;
    ea.q8_out = q8;
    ea.k8_out = k8;
    ea.v8_out = v8;
    ea.qscale_out = q_scale;
    ea.kscale_out = k_scale;
    ea.H = pl.H;
    ea.d = pl.d;
    ea.Npad = pl.Npad;
    ea.ntiles = qa.ntiles;
    for (int s = 0; s < pl.S; ++s) ea.nblocks += (pl.cu[s + 1] - pl.cu[s] + kTile - 1) / kTile;
    ea.seq = qa.seq;
    h3attn_status st;
    if ((st = launch_status(hs, "quantised export launch",
            [&] { return launch_q8_export(ea, hs); })) != H3ATTN_OK) return st;
    const size_t sb = (size_t)pl.S * pl.H * pl.d * sizeof(float);
    if ((st = launch_status(hs, "k_mean copy",
            [&] { return hipMemcpyAsync(k_mean, qa.kmean, sb, hipMemcpyDeviceToDevice, hs); })) != H3ATTN_OK)
        return st;
    return launch_status(hs, "v_scale copy",
            [&] { return hipMemcpyAsync(v_scale, qa.vscale, sb, hipMemcpyDeviceToDevice, hs); });
}

h3attn_status h3attn_proj_q8_prologue(const h3attn_params *p, int32_t model_dim, const void *x, int64_t x_stride,
                                      const void *w_qkv, const float *norm_w, const float *rope_tables,
                                      const int32_t *cu_seqlens_host, void *workspace, size_t workspace_bytes,
                                      int8_t *q8, int8_t *k8, float *q_scale, float *k_scale, float *k_mean,
                                      uint8_t *v8, float *v_scale, void *stream)
{
    Plan pl;
    ProjArgs pa;
    Q8Args qa;
    h3attn_status st = proj_plan(p, model_dim, x_stride, cu_seqlens_host, pl);
    if (st != H3ATTN_OK || pl.N == 0) return st == H3ATTN_OK ? ok() : st;
    const void *outs[7] = {q8, k8, q_scale, k_scale, k_mean, v8, v_scale};
    const char *names[7] = {"q8", "k8", "q_scale", "k_scale", "k_mean", "v8", "v_scale"};
    for (int i = 0; i < 7; ++i) {
        if (!outs[i]) return fail(H3ATTN_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned(outs[i], 8)) return fail(H3ATTN_ERR_INVALID_ARG, "%s is not 8-byte aligned", names[i]);
    }
    st = proj_q8_common(p, model_dim, x, x_stride, w_qkv, norm_w, rope_tables, cu_seqlens_host, x, workspace,
                        workspace_bytes, pl, pa, qa);
    if (st != H3ATTN_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if ((st = proj_q8_stage1(pl, pa, qa, hs)) != H3ATTN_OK) return st;
    return q8_export(pl, qa, q8, k8, q_scale, k_scale, k_mean, v8, v_scale, hs);
}

static h3attn_status mx_common(const h3attn_params *p, const void *q, const void *k, const void *v,
                               const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                               const void *out, void *workspace, size_t workspace_bytes, Plan &pl, MxArgs &ma)
{
    h3attn_status st = make_plan(p, cu_seqlens_host, &pl);
    if (st != H3ATTN_OK) return st;
    if (pl.d != 128) return fail(H3ATTN_ERR_UNSUPPORTED, "the FP4 path needs head_dim 128 (got %d)", pl.d);
    if (pl.N == 0) return H3ATTN_OK;
    if ((st = check_ptrs(q, k, v, norm_w, rope_tables, out)) != H3ATTN_OK) return st;
    if (!workspace) return fail(H3ATTN_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(H3ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < pl.bytes_mx)
        return fail(H3ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes_mx);
    if ((st = check_device()) != H3ATTN_OK) return st;
    char *ws = static_cast<char *>(workspace);
    std::memset(&ma, 0, sizeof ma);
    ma.q = static_cast<const uint16_t *>(q);
    ma.k = static_cast<const uint16_t *>(k);
    ma.v = static_cast<const uint16_t *>(v);
    ma.q_stride = p->q_stride;
    ma.k_stride = p->k_stride;
    ma.v_stride = p->v_stride;
    ma.norm_w = norm_w;
    ma.rope = rope_tables;
    ma.qx = reinterpret_cast<uint8_t *>(ws + pl.qx);
    ma.qxs = reinterpret_cast<uint8_t *>(ws + pl.qxs);
    ma.kx = reinterpret_cast<uint8_t *>(ws + pl.kx);
    ma.kxs = reinterpret_cast<uint8_t *>(ws + pl.kxs);
    ma.vxt = reinterpret_cast<uint8_t *>(ws + pl.vxt);
    ma.vxs = reinterpret_cast<uint8_t *>(ws + pl.vxs);
    ma.ksum = reinterpret_cast<float *>(ws + pl.mx_ksum);
    ma.kmean = reinterpret_cast<float *>(ws + pl.mx_kmean);
    ma.H = pl.H;
    ma.Npad = pl.Npad;
    ma.eps = p->eps;
    ma.q_mult = scale_log2(p);
    ma.ntiles = (int32_t)(pl.Npad / kTile);
    ma.seq = seq_table(pl);
    return H3ATTN_OK;
}

h3attn_status h3attn_fwd_mx_stages(const h3attn_params *p, const void *q, const void *k, const void *v,
                                   const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                                   void *out, void *workspace, size_t workspace_bytes, void *stream, int stages)
{
    if (stages < 1 || stages > 3) return fail(H3ATTN_ERR_INVALID_ARG, "stages must be 1, 2 or 3 (got %d)", stages);
    Plan pl;
    MxArgs ma;
    h3attn_status st = mx_common(p, q, k, v, norm_w, rope_tables, cu_seqlens_host, out, workspace,
                                 workspace_bytes, pl, ma);
    if (st != H3ATTN_OK || pl.N == 0) return st == H3ATTN_OK ? ok() : st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (stages & 1)
        if ((st = launch_status(hs, "FP4 prologue launch",
                [&] { return launch_mx_prep(ma, pl.d, hs); })) != H3ATTN_OK) return st;
    if (!(stages & 2)) return ok();
    MxAttnArgs aa;
    std::memset(&aa, 0, sizeof aa);
    aa.qx = ma.qx;
    aa.qxs = ma.qxs;
    aa.kx = ma.kx;
    aa.kxs = ma.kxs;
    aa.vxt = ma.vxt;
    aa.vxs = ma.vxs;
    aa.out = static_cast<uint16_t *>(out);
    aa.o_stride = p->o_stride;
    aa.Npad = pl.Npad;
    aa.H = pl.H;
    const int64_t items = order_work(pl, aa, nullptr);
    return launch_status(hs, "FP4 attention launch", [&] { return launch_attn_mx(aa, pl.d, items, hs); });
}

h3attn_status h3attn_fwd_mx(const h3attn_params *p, const void *q, const void *k, const void *v,
                            const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                            void *out, void *workspace, size_t workspace_bytes, void *stream)
{
    return h3attn_fwd_mx_stages(p, q, k, v, norm_w, rope_tables, cu_seqlens_host, out, workspace,
                                workspace_bytes, stream, 3);
}

h3attn_status h3attn_mx_prologue(const h3attn_params *p, const void *q, const void *k, const void *v,
                                 const float *norm_w, const float *rope_tables,
                                 const int32_t *cu_seqlens_host, void *workspace, size_t workspace_bytes,
                                 uint8_t *q_codes, uint8_t *q_exp, uint8_t *k_codes, uint8_t *k_exp,
                                 float *k_mean, uint8_t *v_codes, uint8_t *v_exp, void *stream)
{
    Plan pl;
    MxArgs ma;
    h3attn_status st = make_plan(p, cu_seqlens_host, &pl);
    if (st != H3ATTN_OK) return st;
    const void *outs[7] = {q_codes, q_exp, k_codes, k_exp, k_mean, v_codes, v_exp};
    const char *names[7] = {"q_codes", "q_exp", "k_codes", "k_exp", "k_mean", "v_codes", "v_exp"};
    for (int i = 0; i < 7 && pl.N > 0; ++i)
        if (!outs[i]) return fail(H3ATTN_ERR_INVALID_ARG, "%s is NULL", names[i]);
    st = mx_common(p, q, k, v, norm_w, rope_tables, cu_seqlens_host, q_codes, workspace, workspace_bytes, pl, ma);
    if (st != H3ATTN_OK || pl.N == 0) return st == H3ATTN_OK ? ok() : st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if ((st = launch_status(hs, "FP4 prologue launch",
            [&] { return launch_mx_prep(ma, pl.d, hs); })) != H3ATTN_OK) return st;
    MxExportArgs ea;
    std::memset(&ea, 0, sizeof ea);
    ea.qx = ma.qx;
    ea.qxs = ma.qxs;
    ea.kx = ma.kx;
    ea.kxs = ma.kxs;
    ea.vxt = ma.vxt;
    ea.vxs = ma.vxs;
    ea.q_codes = q_codes;
    ea.q_exp = q_exp;
    ea.k_codes = k_codes;
    ea.k_exp = k_exp;
    ea.v_codes = v_codes;
    ea.v_exp = v_exp;
    ea.H = pl.H;
    ea.Npad = pl.Npad;
    ea.ntiles = ma.ntiles;
    ea.seq = ma.seq;
    for (int s = 0; s < pl.S; ++s) ea.vblk_pre[s + 1] = ea.vblk_pre[s] + (pl.cu[s + 1] - pl.cu[s] + 31) / 32;
    if ((st = launch_status(hs, "FP4 export launch",
            [&] { return launch_mx_export(ea, hs); })) != H3ATTN_OK) return st;
    const size_t sb = (size_t)pl.S * pl.H * pl.d * sizeof(float);
    return launch_status(hs, "k_mean copy",
            [&] { return hipMemcpyAsync(k_mean, ma.kmean, sb, hipMemcpyDeviceToDevice, hs); });
}

h3attn_status h3attn_rope_fill_video(int32_t T, int32_t Hg, int32_t Wg, int32_t dt, int32_t dh, int32_t dw,
                                     double theta, float *out)
{
    if (T < 0 || Hg < 1 || Wg < 1) return fail(H3ATTN_ERR_INVALID_ARG, "grid must be T >= 0, Hg, Wg >= 1");
    if (dt < 2 || dh < 2 || dw < 2 || (dt | dh | dw) & 1)
        return fail(H3ATTN_ERR_INVALID_ARG, "section sizes must be even and >= 2");
    if (!(theta > 1.0) || !std::isfinite(theta)) return fail(H3ATTN_ERR_INVALID_ARG, "theta must be > 1");
    if (!out && (int64_t)T * Hg * Wg > 0) return fail(H3ATTN_ERR_INVALID_ARG, "out is NULL");
    const int half = (dt + dh + dw) / 2;
    const int64_t HW = (int64_t)Hg * Wg;
    // section `sec` (first pair `p0`) of a row, for position pos
    auto section = [&](float *row, int p0, int sec, int64_t pos) {
        for (int j = 0; j < sec / 2; ++j) {
            const double phi = (double)pos * std::pow(theta, -2.0 * j / sec);
            row[2 * (p0 + j)] = (float)std::cos(phi);
            row[2 * (p0 + j) + 1] = (float)std::sin(phi);
        }
    };
    // Each section depends on one coordinate only, so it is computed on the
    // first row with that coordinate (t: row (t,0,0); y: row (0,y,0); x: row
    // (0,0,x)) and copied from there into every other row: the same values,
    // with T*dt/2 + Hg*dh/2 + Wg*dw/2 angle evaluations in all.
    for (int64_t t = 0; t < T; ++t)
        for (int64_t y = 0; y < Hg; ++y)
            for (int64_t x = 0; x < Wg; ++x) {
                float *row = out + (t * HW + y * Wg + x) * half * 2;
                if (y == 0 && x == 0)
                    section(row, 0, dt, t);
                else
                    std::memcpy(row, out + (t * HW) * half * 2, sizeof(float) * dt);
                if (t == 0 && x == 0)
                    section(row, dt / 2, dh, y);
                else
                    std::memcpy(row + dt, out + (y * Wg) * half * 2 + dt, sizeof(float) * dh);
                if (t == 0 && y == 0)
                    section(row, (dt + dh) / 2, dw, x);
                else
                    std::memcpy(row + dt + dh, out + x * half * 2 + dt + dh, sizeof(float) * dw);
            }
    return ok();
}

h3attn_status h3attn_rope_fill_audio(int32_t n, int32_t pos0, int32_t dim, double theta, float *out)
{
    if (n < 0 || pos0 < 0) return fail(H3ATTN_ERR_INVALID_ARG, "n and pos0 must be >= 0");
    if (dim < 2 || (dim & 1)) return fail(H3ATTN_ERR_INVALID_ARG, "dim must be even and >= 2");
    if (!(theta > 1.0) || !std::isfinite(theta)) return fail(H3ATTN_ERR_INVALID_ARG, "theta must be > 1");
    if (!out && n > 0) return fail(H3ATTN_ERR_INVALID_ARG, "out is NULL");
    for (int64_t i = 0; i < n; ++i) {
        float *row = out + i * dim;
        for (int j = 0; j < dim / 2; ++j) {
            const double phi = (double)(pos0 + i) * std::pow(theta, -2.0 * j / dim);
            row[2 * j] = (float)std::cos(phi);
            row[2 * j + 1] = (float)std::sin(phi);
        }
    }
    return ok();
}

}  // extern "C"
