/*
 * h3attn.h -- C ABI of the MI355X (gfx950) fused Q/K RMSNorm + RoPE +
 * non-causal multi-head attention library.
 *
 * The operation is the self-attention of a joint video+audio diffusion
 * transformer block (MiniMax-H3) over its packed token sequence, with the Q/K
 * RMSNorm and RoPE in front of it: the page "H3 Runtime Current State", section
 * "Owned Performance Kernels", counts a fused norm/RoPE/relayout kernel and an
 * attention backend tuned for H3's shapes among the work still owed.  The page "Buyer
 * Questions: Current Evidence Status", question 4 ("Current answer"), puts
 * attention at about 58% and norm/RoPE at about 4% of a block and credits the
 * removal of the strided-NHD QKV copy with about 3.6%: here q, k and v are
 * read through token strides, so views into a fused QKV buffer need no copy.
 *
 * For every sequence s (packed tokens [cu[s], cu[s+1])), head h and token i:
 *   qhat_i = RoPE_i( q_i / sqrt(mean_c q_ic^2 + eps) * w_q[h] )   (same for k with w_k[h])
 *   o_i    = sum_j softmax_j( scale * qhat_i . khat_j ) v_j       (j in the same sequence)
 * RoPE rotates interleaved pairs (2j, 2j+1) of each section by the per-token
 * angles in `rope_tables` (see h3attn_rope_fill_video / _audio).  Non-causal;
 * sequences do not see each other.
 *
 * Conventions shared by every entry point
 *  - Ownership: every pointer is caller-owned.  The library never allocates,
 *    frees or keeps a pointer after the call returns.
 *  - Asynchrony: device work is enqueued on `stream` (a hipStream_t; NULL is
 *    the null stream) and the call returns without synchronising.  Buffers must
 *    stay alive until the stream reaches that point.  No call allocates or
 *    copies host memory to the device, so the calls may be captured in a HIP
 *    graph (cu_seqlens is read on the host and baked into kernel arguments).
 *  - Errors: every function returns a status; on anything but H3ATTN_OK
 *    nothing was enqueued (except H3ATTN_ERR_HIP after a failed launch) and
 *    h3attn_last_error() gives a message (thread-local).  Argument checks run
 *    on the host before any HIP call.  No C++ exception crosses the ABI.
 *  - Environment switches, read on every call: H3ATTN_DEBUG=1 waits for the
 *    stream after each launch and reports an execution error as
 *    H3ATTN_ERR_HIP naming that launch (it synchronises: not for graph
 *    capture or timing).  H3ATTN_FAULT=launch is for tests of the error path:
 *    a call that passes its argument checks then makes no HIP call at all
 *    (no device check, no launch) and returns H3ATTN_ERR_HIP for its first
 *    launch.
 *  - Device: the current HIP device must be a gfx950 (MI355X); otherwise
 *    H3ATTN_ERR_DEVICE.
 *  - Aliasing: q, k and v may alias one another (e.g. views of a fused
 *    [N, 3, H, d] buffer).  out and the workspace must not overlap any input.
 */
#ifndef H3ATTN_H
#define H3ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3ATTN_VERSION 2   /* 2: block-sparse tile lists per 256-row query block (1: per 128 rows) */
#define H3ATTN_MAX_SEQS 64      /* sequences per call */

typedef enum h3attn_status {
    H3ATTN_OK = 0,
    H3ATTN_ERR_INVALID_ARG = 1,   /* null pointer, bad size, stride or cu_seqlens */
    H3ATTN_ERR_UNSUPPORTED = 2,   /* shape the kernels do not implement */
    H3ATTN_ERR_WORKSPACE = 3,     /* workspace too small or misaligned */
    H3ATTN_ERR_DEVICE = 4,        /* no HIP device, or not a gfx950 */
    H3ATTN_ERR_HIP = 5            /* a HIP runtime call or kernel launch failed */
} h3attn_status;

/* Shape and numerics of one call.  H = num_heads, d = head_dim. */
typedef struct h3attn_params {
    int32_t num_heads;     /* H >= 1 */
    int32_t head_dim;      /* d: 64 or 128 */
    int32_t num_seqs;      /* S in [1, H3ATTN_MAX_SEQS] */
    int32_t flags;         /* reserved, must be 0 */
    int64_t q_stride;      /* elements between consecutive tokens of q: >= H*d, multiple of 8 */
    int64_t k_stride;      /* same for k */
    int64_t v_stride;      /* same for v */
    int64_t o_stride;      /* same for out */
    float eps;             /* RMSNorm epsilon (> 0, e.g. 1e-6) */
    float softmax_scale;   /* scale on q.k; <= 0 selects 1/sqrt(d) */
} h3attn_params;

/*
 * Bytes of device workspace h3attn_fwd (quantized = 0), h3attn_fwd_q8
 * (quantized = 1), h3attn_fwd_sparse with its tile selection (quantized = 2),
 * h3attn_fwd_mx (quantized = 3) or h3attn_fwd_proj_q8 (quantized = 4) needs
 * for this shape.  cu_seqlens_host: HOST int32 [S+1],
 * cu[0] = 0, non-decreasing; N = cu[S] is the packed token count.  Returns 0
 * and sets the last error when the arguments are invalid.
 */
size_t h3attn_workspace_size(const h3attn_params *p, const int32_t *cu_seqlens_host,
                             int quantized);

/*
 * Fused RMSNorm + RoPE + attention in bf16 with fp32 accumulation.
 *   q, k, v     device bf16, token t head h channel c at x[t*stride + h*d + c]
 *   norm_w      device fp32 [2][H][d]: RMSNorm weights of q, then of k
 *   rope_tables device fp32 [N][d/2][2]: (cos, sin) of the angle of pair j of token t
 *   cu_seqlens_host HOST int32 [S+1] (see h3attn_workspace_size)
 *   out         device bf16, token stride o_stride, same channel order as q
 *   workspace   device, 256-byte aligned, >= h3attn_workspace_size(p, cu, 0) bytes;
 *               its contents on entry do not matter and on exit are unspecified
 *   stream      hipStream_t
 * Sequences of length 0 are allowed and produce nothing; when N = 0 nothing is
 * read, written or launched and the pointers may be NULL.
 */
h3attn_status h3attn_fwd(const h3attn_params *p, const void *q, const void *k, const void *v,
                         const float *norm_w, const float *rope_tables,
                         const int32_t *cu_seqlens_host, void *out, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * The two stages of h3attn_fwd as separate launches, for callers that time or
 * schedule them apart: stages = 1 runs the RMSNorm + RoPE + layout prologue
 * (q, k, v -> workspace), stages = 2 the attention (workspace -> out), 3 both.
 * Same arguments and requirements as h3attn_fwd; a stage-2 call must follow a
 * stage-1 call with the same inputs and workspace on the same stream.
 * h3attn_fwd(...) is exactly h3attn_fwd_stages(..., 3).
 */
h3attn_status h3attn_fwd_stages(const h3attn_params *p, const void *q, const void *k,
                                const void *v, const float *norm_w, const float *rope_tables,
                                const int32_t *cu_seqlens_host, void *out, void *workspace,
                                size_t workspace_bytes, void *stream, int stages);

/*
 * h3attn_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * workspace is a static device array of the library, H3ATTN_STATIC_WORKSPACE_BYTES
 * (128 MiB) per device, which each device holds from the first call on it until
 * the process ends.  The other arguments, the result and the errors are those
 * of h3attn_fwd; a shape whose h3attn_workspace_size(p, cu, 0) exceeds the
 * array returns H3ATTN_ERR_WORKSPACE before any HIP call (the limit is
 * H * padded tokens <= about 174,000 at d = 128: e.g. 7,168 tokens at H = 24,
 * 58,112 at H = 3).  No allocation, memset or copy is made: the prologue writes
 * every workspace byte the attention then reads, so nothing carries over from
 * the previous call.  Every call on one device shares the one array: calls
 * that overlap in time on one device (two streams, two threads) race and must
 * be ordered by the caller.  The first call on a device looks up the array's
 * device address (it may load the library's device code), so it should not be
 * the one made under stream capture.
 */
#define H3ATTN_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)
h3attn_status h3attn_fwd_static(const h3attn_params *p, const void *q, const void *k, const void *v,
                                const float *norm_w, const float *rope_tables,
                                const int32_t *cu_seqlens_host, void *out, void *stream);

/*
 * Block-quantised variant with the same arguments and result layout
 * (workspace >= h3attn_workspace_size(p, cu, 1)).  After the same RMSNorm +
 * RoPE: the per-sequence mean of khat over tokens is subtracted (which leaves
 * softmax unchanged); qhat and khat are quantised to symmetric INT8 with one
 * scale per 64-token block (aligned to the sequence start) per head; v to FP8
 * e4m3 with one scale per (sequence, head, channel); scores use INT8 MFMA
 * with i32 accumulation, probabilities are quantised to FP8 e4m3 with a fixed
 * per-row scale and P.V uses FP8 MFMA with fp32 accumulation.  Lossy: the
 * result approximates h3attn_fwd.  The quantised-path design of SageAttention2,
 * the default quality backend on the page "H3 Runtime Current State", is the
 * prior art.
 */
h3attn_status h3attn_fwd_q8(const h3attn_params *p, const void *q, const void *k,
                            const void *v, const float *norm_w, const float *rope_tables,
                            const int32_t *cu_seqlens_host, void *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/* The two stages of h3attn_fwd_q8 (1: quantised prologue, 2: attention, 3: both);
 * same contract as h3attn_fwd_stages. */
h3attn_status h3attn_fwd_q8_stages(const h3attn_params *p, const void *q, const void *k,
                                   const void *v, const float *norm_w, const float *rope_tables,
                                   const int32_t *cu_seqlens_host, void *out, void *workspace,
                                   size_t workspace_bytes, void *stream, int stages);

/*
 * MXFP4 variant with the same arguments and result layout (head_dim 128;
 * workspace >= h3attn_workspace_size(p, cu, 3)).  The FastVideo commit page
 * for docs/getting_started notes an FP4 attention switch (faster, changes the
 * output, off by default) and "H3 Runtime Current State" keeps the approximate
 * backends quality-gated; the pages give no format, so this is OCP MXFP4, the
 * format the CDNA4 FP4 matrix cores take: e2m1 codes (round to nearest even,
 * saturating at 6) with one power-of-two scale 2^X per block of 32 values,
 * X = floor(log2 amax) - 2 limited to [-126, 127] (0 for an all-zero block).
 * After the same RMSNorm + RoPE and the per-sequence K mean of
 * h3attn_fwd_q8: qhat' = qhat * softmax scale * log2 e (so that scores are
 * in log2 units) and khat - mean in blocks of 32 channels, v in blocks
 * of 32 tokens per channel (aligned to the sequence start), scores on the
 * scaled FP4 MFMA with fp32 accumulation, the lazy base-2 running maximum of
 * h3attn_fwd_q8, and each query row's probabilities of every 32-key block
 * (aligned to the sequence start) as one MX block; the row sum is the sum of
 * those quantised probabilities.  Lossy: the result approximates h3attn_fwd
 * more loosely than h3attn_fwd_q8.
 */
h3attn_status h3attn_fwd_mx(const h3attn_params *p, const void *q, const void *k,
                            const void *v, const float *norm_w, const float *rope_tables,
                            const int32_t *cu_seqlens_host, void *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/* The two stages of h3attn_fwd_mx (1: FP4 prologue, 2: attention, 3: both);
 * same contract as h3attn_fwd_stages. */
h3attn_status h3attn_fwd_mx_stages(const h3attn_params *p, const void *q, const void *k,
                                   const void *v, const float *norm_w, const float *rope_tables,
                                   const int32_t *cu_seqlens_host, void *out, void *workspace,
                                   size_t workspace_bytes, void *stream, int stages);

/*
 * Diagnostic: the FP4 prologue of h3attn_fwd_mx, exported in natural layouts,
 * one e2m1 code (0..15: sign bit 8, then exponent and mantissa) per byte and
 * one E8M0 scale byte (X + 127) per block.  Runs the same kernels as
 * h3attn_fwd_mx into `workspace`, then copies out:
 *   q_codes, k_codes  device uint8 [N][H][d]     codes of qhat' (qhat * softmax scale
 *                                                * log2 e) and of khat - mean
 *   q_exp, k_exp      device uint8 [N][H][d/32]  block scale bytes (32 channels)
 *   k_mean            device fp32 [S][H][d]      per-sequence mean of khat
 *   v_codes           device uint8 [N][H][d]     codes of v
 *   v_exp             device uint8 [NB][H][d]    block scale bytes of v: NB = sum
 *                     over sequences of ceil(n_s / 32); block b of sequence s is
 *                     entry (sum_{s'<s} ceil(n_s'/32)) + b
 */
h3attn_status h3attn_mx_prologue(const h3attn_params *p, const void *q, const void *k,
                                 const void *v, const float *norm_w, const float *rope_tables,
                                 const int32_t *cu_seqlens_host, void *workspace,
                                 size_t workspace_bytes, uint8_t *q_codes, uint8_t *q_exp,
                                 uint8_t *k_codes, uint8_t *k_exp, float *k_mean,
                                 uint8_t *v_codes, uint8_t *v_exp, void *stream);

/*
 * Diagnostic: the fused RMSNorm + RoPE prologue alone, written as bf16 qhat and
 * khat in the natural layout (token stride H*d), using the same kernel code as
 * h3attn_fwd.  q_hat and k_hat: device bf16 [N][H][d].
 */
h3attn_status h3attn_prologue(const h3attn_params *p, const void *q, const void *k,
                              const float *norm_w, const float *rope_tables,
                              const int32_t *cu_seqlens_host, void *q_hat, void *k_hat,
                              void *stream);

/*
 * Diagnostic: the quantised prologue of h3attn_fwd_q8, exported in natural
 * layouts.  Runs the same kernels as h3attn_fwd_q8 into `workspace`, then
 * copies out:
 *   q8, k8    device int8 [N][H][d]   INT8 codes of qhat and of khat - mean
 *   q_scale,
 *   k_scale   device fp32 [H][B]      B = sum over sequences of ceil(n_s / 64);
 *                                     block b of sequence s is entry
 *                                     (sum_{s'<s} ceil(n_s'/64)) + b
 *   k_mean    device fp32 [S][H][d]   per-sequence mean of khat
 *   v8        device uint8 [N][H][d]  FP8 e4m3 codes of v
 *   v_scale   device fp32 [S][H][d]   per-(sequence, head, channel) scale of v
 */
h3attn_status h3attn_q8_prologue(const h3attn_params *p, const void *q, const void *k,
                                 const void *v, const float *norm_w, const float *rope_tables,
                                 const int32_t *cu_seqlens_host, void *workspace,
                                 size_t workspace_bytes, int8_t *q8, int8_t *k8,
                                 float *q_scale, float *k_scale, float *k_mean, uint8_t *v8,
                                 float *v_scale, void *stream);

/*
 * QKV projection fused with the same prologue, then the attention: the
 * attention layer from its input hidden states.  The page "H3 Runtime Current
 * State" lists the attention QKV projection among the block's GEMMs (about 27%
 * of a block together, "Buyer Questions: Current Evidence Status", question
 * 4); the pages give no formula, so this is the plain linear map without bias:
 *   [q | k | v]_t = x_t . W^T,  W = w_qkv [3*H*d][model_dim] (nn.Linear layout),
 * output features q first, then k, then v, each head-major (feature h*d + c of
 * its part).  q and k are normalised and rotated in fp32 straight from the
 * fp32 accumulators (they are never rounded before the norm); v is rounded to
 * bf16 once.  Then exactly the attention of h3attn_fwd.
 *   model_dim   D: positive multiple of 32
 *   x           device bf16, token t channel c at x[t*x_stride + c]; x_stride >= D,
 *               multiple of 8
 *   w_qkv       device bf16 [3*H*d][D], rows contiguous
 *   norm_w, rope_tables, cu_seqlens_host, out, workspace, stream: as h3attn_fwd
 *               (workspace >= h3attn_workspace_size(p, cu, 0) bytes)
 * The q_stride, k_stride and v_stride of `p` are not read.  x, w_qkv, norm_w,
 * rope_tables and out must be 16-byte aligned.
 */
h3attn_status h3attn_fwd_proj(const h3attn_params *p, int32_t model_dim, const void *x, int64_t x_stride,
                              const void *w_qkv, const float *norm_w, const float *rope_tables,
                              const int32_t *cu_seqlens_host, void *out, void *workspace,
                              size_t workspace_bytes, void *stream);

/* The two stages of h3attn_fwd_proj (1: projection + prologue into the
 * workspace, 2: attention, 3: both); same contract as h3attn_fwd_stages. */
h3attn_status h3attn_fwd_proj_stages(const h3attn_params *p, int32_t model_dim, const void *x,
                                     int64_t x_stride, const void *w_qkv, const float *norm_w,
                                     const float *rope_tables, const int32_t *cu_seqlens_host,
                                     void *out, void *workspace, size_t workspace_bytes,
                                     void *stream, int stages);

/*
 * Diagnostic: stage 1 of h3attn_fwd_proj exported in natural layouts, by the
 * same kernel: q_hat and k_hat (normalised and rotated, bf16; q_hat without the
 * softmax scale) and the projected v_out (bf16), each device [N][H][d].
 */
h3attn_status h3attn_proj_prologue(const h3attn_params *p, int32_t model_dim, const void *x,
                                   int64_t x_stride, const void *w_qkv, const float *norm_w,
                                   const float *rope_tables, const int32_t *cu_seqlens_host,
                                   void *q_hat, void *k_hat, void *v_out, void *stream);

/*
 * The QKV projection with the quantised prologue of h3attn_fwd_q8 in its
 * epilogue, then the quantised attention.  The page "Buyer Questions: Current
 * Evidence Status" (question 4) counts the block's GEMMs and its scale/pack
 * work beside attention; the pages give no formula, so this is h3attn_fwd_q8
 * applied to the projection of h3attn_fwd_proj, with that entry point's
 * precision: q and k are normalised and rotated in fp32 from the fp32
 * accumulators (never rounded to bf16), v is rounded to bf16 once.  The
 * projection's epilogue codes qhat to INT8 (one scale per 64-token block of a
 * head, amax / 127, as h3attn_fwd_q8), writes khat in fp32 and v in bf16 to
 * the workspace; the K means, V scales and the K / V codes are then formed as
 * in h3attn_fwd_q8, and the attention is that entry point's.
 *   head_dim 128 only (else H3ATTN_ERR_UNSUPPORTED);
 *   workspace >= h3attn_workspace_size(p, cu, 4) bytes;
 *   all other arguments and conventions as h3attn_fwd_proj.
 */
h3attn_status h3attn_fwd_proj_q8(const h3attn_params *p, int32_t model_dim, const void *x, int64_t x_stride,
                                 const void *w_qkv, const float *norm_w, const float *rope_tables,
                                 const int32_t *cu_seqlens_host, void *out, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* The two stages of h3attn_fwd_proj_q8 (1: projection + quantised prologue
 * into the workspace, 2: attention, 3: both); same contract as
 * h3attn_fwd_stages. */
h3attn_status h3attn_fwd_proj_q8_stages(const h3attn_params *p, int32_t model_dim, const void *x,
                                        int64_t x_stride, const void *w_qkv, const float *norm_w,
                                        const float *rope_tables, const int32_t *cu_seqlens_host,
                                        void *out, void *workspace, size_t workspace_bytes,
                                        void *stream, int stages);

/*
 * Diagnostic: stage 1 of h3attn_fwd_proj_q8 exported in natural layouts, with
 * the outputs and layouts of h3attn_q8_prologue (q8, k8, q_scale, k_scale,
 * k_mean, v8, v_scale).  Runs the same kernels into `workspace` (>=
 * h3attn_workspace_size(p, cu, 4) bytes), then copies out.
 */
h3attn_status h3attn_proj_q8_prologue(const h3attn_params *p, int32_t model_dim, const void *x,
                                      int64_t x_stride, const void *w_qkv, const float *norm_w,
                                      const float *rope_tables, const int32_t *cu_seqlens_host,
                                      void *workspace, size_t workspace_bytes, int8_t *q8, int8_t *k8,
                                      float *q_scale, float *k_scale, float *k_mean, uint8_t *v8,
                                      float *v_scale, void *stream);

/*
 * Output projection of the attention output with the gated residual of a
 * DiT-style (adaLN) block.  The page "Buyer Questions: Current Evidence
 * Status", question 4, counts the block's GEMMs (about 27%) and its "gates"
 * (about 2%) beside attention; the pages give no formula, so this is the plain
 * reading:
 *   out[t][c] = resid[t][c] + gate[s(t)][c] * sum_k attn[t][k] * w_o[c][k]
 * with s(t) the sequence of packed token t and k over the H*d attention
 * channels.  fp32 accumulation, gate and residual applied in fp32, one
 * rounding to bf16.
 *   num_heads, head_dim  H >= 1, d in {64, 128}: attn has K = H*d channels
 *   model_dim    D: positive multiple of 128 (output channels)
 *   num_seqs, cu_seqlens_host  as h3attn_workspace_size (HOST int32 [S+1])
 *   attn         device bf16, token t channel k at attn[t*attn_stride + k] (the
 *                [N][H][d] output of h3attn_fwd is this with attn_stride = o_stride)
 *   w_o          device bf16 [D][K], rows contiguous (nn.Linear layout)
 *   gate         device fp32 [S][D], or NULL for a gate of 1
 *   resid        device bf16, token stride resid_stride, or NULL for none
 *   out          device bf16, token stride out_stride; may be resid itself
 *                (same pointer and stride) for an in-place residual update,
 *                must not otherwise overlap any input
 * Strides are in elements: attn_stride >= K, resid_stride and out_stride >= D,
 * all multiples of 8; every non-NULL pointer 16-byte aligned.  No workspace.
 * When N = 0 nothing is read, written or launched.
 */
h3attn_status h3attn_out_proj(int32_t num_heads, int32_t head_dim, int32_t model_dim, int32_t num_seqs,
                              const int32_t *cu_seqlens_host, const void *attn, int64_t attn_stride,
                              const void *w_o, const float *gate, const void *resid, int64_t resid_stride,
                              void *out, int64_t out_stride, void *stream);

/*
 * Block-sparse attention: each 256-row query block attends to a kept subset of
 * its sequence's 64-key tiles, softmax over the kept keys only.  The page
 * "Open-H3-Regenerate-2K" ("Speed on one B200 (GB200)", per-module table)
 * credits a sparse attention backend with most of a refine's speed-up over
 * dense attention and calls it lossy; the pages give no algorithm.  Here:
 *  - block_tiles: device int32 [items][tiles_per_block], items in the order
 *    sequence, then head, then 256-row query block (items = sum over sequences
 *    of H * ceil(n_s / 256)).  Of each row the first
 *    L = min(tiles_per_block, ceil(n_s / 64)) entries are tile indices within
 *    the sequence (tile t = its tokens 64t .. 64t+63), distinct; the rest are
 *    ignored.  Out-of-range entries are clamped to the sequence's tiles.
 *  - stages (bit mask): 1 the RMSNorm + RoPE prologue into the workspace (as
 *    h3attn_fwd_stages stage 1); 2 the tile selection, which writes
 *    block_tiles: for every item the L tiles with the largest dot product of
 *    the query block's mean stored qhat' row and the tile's mean khat row
 *    (ties to the lower index), ascending, -1 after them; 4 the attention over
 *    the listed tiles.  Stage 2 needs workspace_bytes >=
 *    h3attn_workspace_size(p, cu, 2), the others h3attn_workspace_size(p, cu, 0);
 *    a later stage reads what an earlier call left in the same workspace and
 *    stream.  Callers with their own lists use stages 1 | 4.
 *  - tiles_per_block in [1, 2048]; every sequence at most 2048 tiles (131,072
 *    tokens), else H3ATTN_ERR_UNSUPPORTED.
 * Other arguments and conventions as h3attn_fwd.  Keeping every tile
 * (tiles_per_block >= the longest sequence's tile count) gives dense attention.
 */
h3attn_status h3attn_fwd_sparse_stages(const h3attn_params *p, const void *q, const void *k, const void *v,
                                       const float *norm_w, const float *rope_tables,
                                       const int32_t *cu_seqlens_host, int32_t tiles_per_block,
                                       int32_t *block_tiles, void *out, void *workspace, size_t workspace_bytes,
                                       void *stream, int stages);

/* h3attn_fwd_sparse_stages(..., 7): prologue, tile selection into block_tiles,
 * sparse attention. */
h3attn_status h3attn_fwd_sparse(const h3attn_params *p, const void *q, const void *k, const void *v,
                                const float *norm_w, const float *rope_tables, const int32_t *cu_seqlens_host,
                                int32_t tiles_per_block, int32_t *block_tiles, void *out, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Host helpers that fill RoPE tables (fp32 (cos, sin) pairs) on the host.
 * Video: a T x Hg x Wg latent grid in t-major raster order (token n has
 * t = n / (Hg*Wg), y = (n / Wg) % Hg, x = n % Wg, all 0-based); dims [0, dt)
 * rotate with t, [dt, dt+dh) with y, [dt+dh, dt+dh+dw) with x; a section of D
 * dims turns its pair j by pos * theta^(-2j/D).  out: [T*Hg*Wg][(dt+dh+dw)/2][2].
 * Audio: n tokens at positions pos0 .. pos0+n-1, one section over all `dim`
 * dims.  out: [n][dim/2][2].  Section sizes must be even and positive
 * (dt, dh, dw >= 2).  The pages give no formula for the rotation; this is the
 * original interleaved-pair RoPE applied per axis.
 */
h3attn_status h3attn_rope_fill_video(int32_t T, int32_t Hg, int32_t Wg, int32_t dt, int32_t dh,
                                     int32_t dw, double theta, float *out);
h3attn_status h3attn_rope_fill_audio(int32_t n, int32_t pos0, int32_t dim, double theta,
                                     float *out);

/* Static name of a status code. */
const char *h3attn_status_string(h3attn_status s);
/* Detail of the calling thread's last non-OK status ("" if none). */
const char *h3attn_last_error(void);
/*
 * Diagnostic for the checked build of this library (libh3attn_checked.so, the
 * same sources compiled with H3ATTN_CHECKED; the product library returns
 * H3ATTN_ERR_UNSUPPORTED).  Its attention kernels record violated invariants
 * in H3ATTN_CHECK_KINDS device flag words:
 *   0  a work item decoded outside its sequence, head or query block;
 *   1  a workgroup's query rows outside the padded workspace layout;
 *   2  a K/V tile fill outside the sequence's tiles;
 *   3  a block-sparse tile-list entry outside the sequence's tiles (the
 *      kernels clamp it; it breaks the caller contract of h3attn_fwd_sparse).
 * With a nonzero jitter seed every wave of those kernels sleeps a
 * pseudo-random 0..3 x 128 cycles before each tile fill and each phase:
 * synchronisation is unchanged, so outputs must stay bit-identical to the
 * product library for every seed; a difference means a race between the LDS
 * fills and the reads.  The call waits for the device, then
 *   flags_out  HOST uint32 [H3ATTN_CHECK_KINDS] or NULL: the flag words
 *   clear      nonzero: reset the flags to 0 after reading them
 *   jitter_seed  seed for later launches (0: no delays)
 */
#define H3ATTN_CHECK_KINDS 4
h3attn_status h3attn_checked(uint32_t *flags_out, int clear, uint32_t jitter_seed);

/* H3ATTN_VERSION of the built library. */
int h3attn_version(void);

/*
 * Diagnostic, not part of the attention path: the sustained matrix-core rate
 * of the current device, a measured ceiling beside the datasheet peak for
 * the roofline of the attention kernels.  Launches `workgroups` workgroups of
 * 512 threads on `stream`; every wave runs iters x 8 MFMAs on register
 * operands that change from instruction to instruction (hashed values, like a
 * real product, so the part runs at the clock its power limit sets for such
 * work).  mix 0: v_mfma_f32_32x32x16_bf16 alone; mix 1: the same with one
 * v_exp_f32 and one FMA per MFMA (the vector work of the bf16 attention's
 * softmax); mix 2: v_mfma_i32_32x32x32_i8 alone; mix 3: the same with two
 * FMAs, two v_exp_f32, one v_cvt_pk_fp8_f32 and one v_max3_f32 per MFMA (the
 * quantised attention's vector work per 32 matrix-core cycles); mix 4:
 * v_mfma_scale_f32_32x32x64_f8f6f4 on e2m1 operands alone; mix 5: the same
 * with four v_exp_f32, two v_cvt_scalef32_pk_fp4_f32, two v_max3_f32 and one
 * FMA per MFMA (the MXFP4 attention's vector work per 32 matrix-core
 * cycles).  Work: 32768 (mix 0, 1), 65536 (mix 2, 3) or 131072 (mix 4, 5)
 * * 8 * iters * 8 * workgroups operations.  out: device float [512 * workgroups], caller-owned, receives
 * values that only keep the work live.  The caller times the launch (events
 * on the stream).  Errors: H3ATTN_ERR_INVALID_ARG for mix outside 0..5,
 * workgroups or iters outside [1, 2^20], out NULL or not 4-byte aligned;
 * H3ATTN_ERR_DEVICE; H3ATTN_ERR_HIP.
 */
h3attn_status h3attn_mfma_ceiling(int mix, int workgroups, int iters, float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* H3ATTN_H */
