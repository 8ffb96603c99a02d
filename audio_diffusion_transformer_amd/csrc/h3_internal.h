// Internal declarations shared by the host library and the gfx950 kernels.
// Not part of the public ABI (include/h3attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

constexpr int kMaxSeqs = 64;     // == H3ATTN_MAX_SEQS
constexpr int kSeqPad = 256;     // every sequence starts at a multiple of this in the workspace
constexpr int kTile = 64;        // key tile (and quantisation block) in tokens

// Workspace layout of one call.  Head-major copies of the prologue outputs:
//   qhat, khat : bf16 [H][Npad][d]
//   vt         : bf16 [H][Npad/64][d][64]  (V transposed per 64-key tile; the
//                keys inside each 32-key half are stored in the order the
//                P.V matrix-core operand consumes them, see attn_bf16.hip)
//   knorm      : fp32 [H][Npad/64]  largest |khat| (2-norm of the stored bf16
//                row) of each 64-token tile; 0 for padding tiles
// Quantised path:
//   q8, k8     : int8 [H][Npad][d]
//   v8t        : fp8  [H][Npad/64][d][64]  (transposed; key order of the FP8 P.V operand)
//   qscale, kscale : fp32 [H][Npad/64]
//   ksum, vmax : fp32 [H][Npad/64][d]  per-tile partial sums / maxima
//   kmean, vscale : fp32 [S][H][d]
struct Plan {
    int32_t S, H, d;
    int64_t N, Npad;
    int32_t cu[kMaxSeqs + 1];    // packed token starts
    int32_t off[kMaxSeqs + 1];   // padded starts (multiples of kSeqPad)
    size_t qhat, khat, vt, knorm; // byte offsets into the workspace
    size_t q8, k8, v8t, qscale, kscale, ksum, vmax, kmean, vscale;
    size_t sp_kbar, sp_qsum, sp_cnt; // block-sparse selection scratch (after the bf16 regions)
    size_t qx, qxs, kx, kxs, vxt, vxs, mx_ksum, mx_kmean;   // MXFP4 path (mx.hip)
    size_t k32, v16;             // projection's quantised path: fp32 khat, bf16 v (after the q8 regions)
    size_t bytes_bf16, bytes_q8, bytes_sparse, bytes_mx, bytes_q8p;
};

// Which sequence a padded 64-token tile belongs to: tiles of sequence s are
// [off[s]/64, off[s]/64 + ceil(n_s/64)); the remaining tiles up to off[s+1]/64
// are padding.
struct SeqTable {
    int32_t S;
    int32_t cu[kMaxSeqs + 1];
    int32_t off[kMaxSeqs + 1];
};

struct PrologueArgs {
    const uint16_t *q, *k, *v;
    int64_t q_stride, k_stride, v_stride;
    const float *norm_w;
    const float *rope;
    // bf16 outputs.  qhat/khat element (h, padded token t, c) at
    // h*out_hstride + t*out_tstride + c.  When `natural` is set, t is the packed
    // token and padding rows are skipped (diagnostic export).
    uint16_t *qhat, *khat, *vt;
    float *knorm;                // per-tile max |khat| (not written when natural is set)
    int64_t out_hstride, out_tstride;
    int32_t natural;
    int32_t H;
    int64_t Npad;
    float eps;
    float q_mult;                // qhat is stored multiplied by this (softmax scale * log2 e
                                 // for the attention kernel; 1 for the diagnostic export)
    int32_t ntiles;              // Npad / 64
    SeqTable seq;
};

struct AttnArgs {
    const uint16_t *qhat, *khat, *vt;
    const float *knorm;
    uint16_t *out;
    int64_t o_stride;
    int64_t Npad;
    int32_t H;
    int32_t nseq;                // sequences with work, longest first
    int32_t seq_n[kMaxSeqs];
    int32_t seq_cu[kMaxSeqs];
    int32_t seq_off[kMaxSeqs];
    int32_t seq_nqb[kMaxSeqs];        // query blocks of the kernel's block size
    int32_t item_pre[kMaxSeqs + 1];   // prefix sums of H * nqb
    // block-sparse attention (null tiles: dense): tiles is int32
    // [items][tpb] in the caller's item order (sequence, head, 128-row query
    // block); seq_item_base is the caller's first item of each sequence above
    const int32_t *tiles;
    int32_t tpb;
    int32_t seq_item_base[kMaxSeqs];
};

// Longest tile list (and longest sequence, in 64-key tiles) of the
// block-sparse path.
constexpr int kMaxSparseTiles = 2048;
// Query rows sharing one block-sparse tile list: the workgroup of the head_dim
// 128 attention kernel, so each workgroup streams exactly one list.
constexpr int kSparseBlockM = 256;

// Block-sparse tile selection (sparse_select.hip).  From the prologue's qhat'
// and khat in the workspace: per (head, padded 64-token tile) the mean khat row
// (kbar) and the sum of qhat' rows (qsum), and per tile its valid row count;
// then per (sequence, head, kSparseBlockM-row query block) the tpb tiles with the
// largest qbar . kbar, written ascending to tiles [items][tpb] (-1 past
// min(tpb, tiles of the sequence)).
struct SparseSelectArgs {
    const uint16_t *qhat, *khat;     // workspace bf16 [H][Npad][d]
    float *kbar, *qsum;              // fp32 kbar [H][d][ntiles] (channel-major), qsum [H][ntiles][d]
    int32_t *cnt;                    // int32 [ntiles]
    int32_t *tiles;
    int32_t tpb;
    int32_t H;
    int64_t Npad;
    int32_t ntiles;
    SeqTable seq;
    int32_t item_base[kMaxSeqs];     // first item of each sequence (caller order)
    int32_t group_pre[kMaxSeqs + 1]; // prefix of H * ceil(nqb / 4): select workgroups per sequence
};

struct Q8Args {
    const uint16_t *q, *k, *v;
    int64_t q_stride, k_stride, v_stride;
    const float *norm_w, *rope;
    int8_t *q8, *k8;
    uint8_t *v8t;
    float *qscale, *kscale, *ksum, *vmax, *kmean, *vscale;
    // Set for the projection's quantised path: khat (fp32) and v (bf16), both
    // [H][Npad][d], as the projection wrote them; q, k, v are then not read.
    const float *k32;
    const uint16_t *v16;
    int32_t H;
    int64_t Npad;
    float eps;
    int32_t ntiles;
    SeqTable seq;
};

struct Q8AttnArgs {
    const int8_t *q8, *k8;
    const uint8_t *v8t;
    const float *qscale, *kscale, *vscale;
    uint16_t *out;
    int64_t o_stride;
    int64_t Npad;
    int32_t H;
    float scale_log2;
    int32_t nseq;
    int32_t seq_n[kMaxSeqs];
    int32_t seq_cu[kMaxSeqs];
    int32_t seq_off[kMaxSeqs];
    int32_t seq_idx[kMaxSeqs];   // original sequence index (for vscale)
    int32_t seq_nqb[kMaxSeqs];
    int32_t item_pre[kMaxSeqs + 1];
};

struct Q8ExportArgs {
    const int8_t *q8, *k8;
    const uint8_t *v8t;
    const float *qscale, *kscale;
    int8_t *q8_out, *k8_out;
    uint8_t *v8_out;
    float *qscale_out, *kscale_out;
    int32_t H, d;
    int64_t Npad;
    int32_t ntiles;
    int32_t nblocks;             // sum of ceil(n_s / 64)
    SeqTable seq;
};

// MXFP4 attention (mx.hip): OCP microscaling FP4, e2m1 codes with one E8M0
// scale byte (2^(byte - 127)) per 32 elements.  Workspace:
//   qx, kx : fp4 [H][Npad][d/2], two codes per byte (even channel in the low
//            nibble), of qhat' = qhat * q_mult and of khat - mean; the 64 rows of every K tile are stored in the key order
//            of the FP4 score operand (mx_key_row)
//   qxs    : E8M0 [H][Npad][d/32]
//   kxs    : E8M0 [H][ntiles][256], each tile's bytes in the order the
//            attention kernel reads them (mx_kscale_pos)
//   vxt    : fp4 [H][ntiles][d][32], V transposed per tile (a channel row of
//            64 keys, key 2i in the low nibble of byte i)
//   vxs    : E8M0 [H][ntiles][256] (mx_vscale_pos)
//   ksum   : fp32 [H][ntiles][d] per-tile partial sums of khat
//   kmean  : fp32 [S][H][d]
struct MxArgs {
    const uint16_t *q, *k, *v;
    int64_t q_stride, k_stride, v_stride;
    const float *norm_w, *rope;
    uint8_t *qx, *qxs, *kx, *kxs, *vxt, *vxs;
    float *ksum, *kmean;
    int32_t H;
    int64_t Npad;
    float eps;
    float q_mult;                // qhat is quantised times this (softmax scale * log2 e)
    int32_t ntiles;
    SeqTable seq;
};

struct MxAttnArgs {
    const uint8_t *qx, *qxs, *kx, *kxs, *vxt, *vxs;
    uint16_t *out;
    int64_t o_stride;
    int64_t Npad;
    int32_t H;
    int32_t nseq;
    int32_t seq_n[kMaxSeqs];
    int32_t seq_cu[kMaxSeqs];
    int32_t seq_off[kMaxSeqs];
    int32_t seq_nqb[kMaxSeqs];
    int32_t item_pre[kMaxSeqs + 1];
};

// Natural-layout copy of the MXFP4 workspace (diagnostic export), one code
// per byte: q_codes, k_codes, v_codes [N][H][d]; q_exp, k_exp [N][H][d/32]
// and v_exp [NB][H][d] scale bytes, NB = sum over sequences of ceil(n / 32)
// (32-token blocks in sequence order).
struct MxExportArgs {
    const uint8_t *qx, *qxs, *kx, *kxs, *vxt, *vxs;
    uint8_t *q_codes, *q_exp, *k_codes, *k_exp, *v_codes, *v_exp;
    int32_t H;
    int64_t Npad;
    int32_t ntiles;
    SeqTable seq;
    int32_t vblk_pre[kMaxSeqs + 1];   // prefix of ceil(n_s / 32)
};

// Fused QKV projection + RMSNorm + RoPE + layout (qkv_proj.hip).  x is bf16
// [N][D] (token stride x_stride), w is bf16 [3*H*d][D] with the q, k and v
// output features in that order, each head-major.  The outputs are those of
// the prologue: qhat, khat [H][Npad][d] (qhat times q_mult), vt per 64-key
// tile, knorm per tile; with `natural` set they are instead qhat, khat and the
// projected v at packed tokens, [N][H][d], padding skipped.
struct ProjArgs {
    const uint16_t *x, *w;
    int64_t x_stride;            // elements between tokens of x
    int32_t model_dim;           // D, a multiple of 32
    const float *norm_w, *rope;
    uint16_t *qhat, *khat, *vt;
    float *knorm;
    // Quantised epilogue (qkv_proj_q8 launch, d = 128): INT8 qhat codes with one
    // scale per (head, tile), fp32 khat and bf16 v, all [H][Npad][d].
    int8_t *q8;
    float *qscale;
    float *k32;
    uint16_t *v16;
    int64_t out_hstride, out_tstride;
    int32_t natural;
    int32_t H;
    int64_t Npad;
    int32_t ntiles;              // Npad / 64
    int32_t nblk;                // Npad / 256 token blocks
    float eps;
    float q_mult;
    SeqTable seq;
};

// Output projection with the gated residual (out_proj.hip):
//   out[t][c] = resid[t][c] + gate[s(t)][c] * sum_k attn[t][k] * w[c][k]
// attn bf16 [N][K] (K = H*d), w bf16 [D][K], gate fp32 [S][D] (null: 1),
// resid bf16 [N][D] (null: 0), out bf16 [N][D] (may be resid itself).
struct OutProjArgs {
    const uint16_t *attn, *w;
    int64_t attn_stride;
    int32_t K;                   // H * d, a multiple of 32
    int32_t model_dim;           // D, a multiple of 128
    const float *gate;
    const uint16_t *resid;
    int64_t resid_stride;
    uint16_t *out;
    int64_t out_stride;
    int64_t N;
    int32_t nblk;                // ceil(N / 256)
    int32_t S;
    int32_t cu[kMaxSeqs + 1];
};

// Invariants the checked build (H3ATTN_CHECKED) records in the attention
// kernels, one flag word each.
enum CheckKind {
    kCheckItem = 0,        // work item decoded outside its sequence / head / query block
    kCheckRows = 1,        // a workgroup's query rows outside the padded layout
    kCheckFillTile = 2,    // a K/V tile fill outside the sequence's tiles
    kCheckListEntry = 3,   // a block-sparse list entry outside [0, tiles of the sequence) (clamped)
    kCheckKinds = 4
};
#ifdef H3ATTN_CHECKED
// Per translation unit (bf16, quantised, MXFP4 attention): OR the unit's flag
// words into or_into, clear them if asked, set its jitter seed.  The caller
// synchronises the device first.
hipError_t attn_checked(uint32_t *or_into, bool clear, uint32_t jitter_seed);
hipError_t q8_checked(uint32_t *or_into, bool clear, uint32_t jitter_seed);
hipError_t mx_checked(uint32_t *or_into, bool clear, uint32_t jitter_seed);
#endif

// Launchers: return the hipError_t of the launch.
hipError_t launch_prologue(const PrologueArgs &a, int d, hipStream_t st);
hipError_t launch_attn_bf16(const AttnArgs &a, int d, int64_t nitems, hipStream_t st);
hipError_t launch_q8_prep(const Q8Args &a, int d, hipStream_t st);
hipError_t launch_attn_q8(const Q8AttnArgs &a, int d, int64_t nitems, hipStream_t st);
hipError_t launch_q8_export(const Q8ExportArgs &a, hipStream_t st);
hipError_t launch_qkv_proj(const ProjArgs &a, int d, hipStream_t st);
hipError_t launch_qkv_proj_q8(const ProjArgs &a, hipStream_t st);
hipError_t launch_out_proj(const OutProjArgs &a, hipStream_t st);
hipError_t launch_sparse_select(const SparseSelectArgs &a, int d, hipStream_t st);
hipError_t launch_mx_prep(const MxArgs &a, int d, hipStream_t st);
hipError_t launch_attn_mx(const MxAttnArgs &a, int d, int64_t nitems, hipStream_t st);
hipError_t launch_mfma_ceiling(int mix, int workgroups, int iters, float *out, hipStream_t st);
hipError_t launch_mx_export(const MxExportArgs &a, hipStream_t st);

// Queries per workgroup of the attention kernels (work-item granularity).
constexpr int kBlockM = 128;
// Queries per workgroup of the dense bf16 kernel at head_dim 128 (two groups
// of four waves, 32 rows each); every sequence is padded to kSeqPad rows, a
// multiple of it, so its query blocks stay inside the sequence's rows.
constexpr int kBlockM2 = 256;
static_assert(kSeqPad % kBlockM2 == 0, "query blocks stay within a padded sequence");
static_assert(kSparseBlockM == kBlockM2 && kSparseBlockM % kBlockM == 0, "a sparse block is one 8-wave workgroup");
// Rows per work item launch_attn_bf16 expects at head_dim d (dense and
// block-sparse alike: the 8-wave kernel at 128, the 4-wave kernel at 64).
inline int attn_bf16_block_m(int d) { return d == 128 ? kBlockM2 : kBlockM; }

}  // namespace h3
