/*
 * st_attn.h -- C ABI of libstattn: 3D-RoPE full spatiotemporal attention (forward) on MI355X.
 *
 * What is computed.  A video-DiT self-attention layer sees a T' x H' x W' grid of latent tokens
 * ("A video model's architecture: spatiotemporal attention and the 3D VAE", self-test answers 1
 * and 2).  Each head's 128 channels are split into three contiguous ranges rotated by the
 * token's t, h and w coordinate (same page, self-test answer 4 and "Position: RoPE in three
 * dimensions"; "CogVideoX Architecture: ...", section "3. 3D Rotary Position Embeddings (3D RoPE)",
 * the block-diagonal R_3D).  Attention is then non-causal softmax(q~ k~^T / sqrt(d)) v over all
 * tokens together ("full 3D attention"), or, for the factorised variant, spatial attention inside
 * each frame followed by temporal attention at each spatial position (first page, "How attention
 * sees time: factorised or full").
 *
 * Conventions shared by every entry point.
 *   Layout    q, k, v, out, x, y: [N][heads][d] row-major, batch 1, where N = T*H*W + n_text and
 *             token n < T*H*W sits at t = n / (H*W), h = (n / W) % H, w = n % W (t slowest, w
 *             fastest).  Rows n >= T*H*W are text tokens: they attend and are attended like any
 *             token but are not rotated.
 *   RoPE      rope_split = {d_t, d_h, d_w}: even, >= 0, sum d.  Channels [0, d_t) turn with t,
 *             [d_t, d_t + d_h) with h, the rest with w.  Inside a range, pair j is channels
 *             (off + 2j, off + 2j + 1) and turns by pos * theta^(-2j / d_a):
 *             (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).  V is never rotated.
 *   Scale     1 / sqrt(d); no mask, no causality.
 *   dtype     ST_BF16: bfloat16 storage, d == 128; matrix products on MFMA with fp32
 *             accumulation: rotated q/k rounded to fp16 for the scores, softmax weights rounded
 *             to bf16 for the product with v; fp32 softmax; output rounded to bf16.
 *             ST_F32: float32 storage and arithmetic throughout (a checking mode, not a fast
 *             path), even d <= 128.
 *   Memory    Every pointer except rope_split is device memory owned by the caller; the library
 *             allocates nothing, keeps no global state and is re-entrant.  Tensor pointers must
 *             be 16-byte aligned, workspace and table pointers 256-byte aligned.  out must not
 *             overlap q, k or v.
 *   Streams   All work is enqueued on `stream` (0 = the null stream) and returns without
 *             waiting for it.  The caller keeps inputs, workspace and outputs alive until the
 *             stream has run the work.
 *   Errors    Arguments are checked before anything is enqueued; on an error nothing runs and no
 *             output or workspace byte is touched.  A failed launch returns ST_ERR_HIP and
 *             st_last_hip_error() then gives the hipError_t (per calling thread).
 *   Limits    N < 2^24 rows; T, H, W >= 1; heads >= 1; n_text >= 0; theta finite and > 0.
 */
#ifndef ST_ATTN_H
#define ST_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum st_status {
    ST_OK = 0,
    ST_ERR_NULL = 1,        /* a required pointer is NULL */
    ST_ERR_SHAPE = 2,       /* T, H, W, heads, d, n_text or N out of range */
    ST_ERR_SPLIT = 3,       /* rope_split entries odd, negative or not summing to d */
    ST_ERR_UNSUPPORTED = 4, /* valid request this build does not serve (dtype/d combination,
                               text rows on the factorised path, bad theta) */
    ST_ERR_WORKSPACE = 5,   /* workspace or table smaller than the matching *_bytes() size */
    ST_ERR_HIP = 6,         /* a kernel launch failed; see st_last_hip_error() */
    ST_ERR_ALIAS = 7,       /* out overlaps an input */
    ST_ERR_ALIGN = 8        /* a pointer is not aligned as required */
} st_status;

typedef enum st_dtype {
    ST_BF16 = 0,
    ST_F32 = 1
} st_dtype;

/* ---------------------------------------------------------------------------------------------
 * RoPE angle table ("A video model's architecture: spatiotemporal attention and the 3D VAE",
 * "Position: RoPE in three dimensions": each axis range is its own 1D RoPE, so pair j of a range
 * of d_a channels at coordinate p turns by p * theta^(-2j / d_a)).  One (cos, sin) float pair per
 * axis position and pair index, built in fp64 and rounded once to fp32: [T][d_t/2], then
 * [H][d_h/2], then [W][d_w/2], then one identity entry (1, 0) used by text rows.  Depends only on
 * the grid, the split and theta, so a caller that runs many layers on one grid can build it once.
 * The attention entry points build their own copy in their workspace.  The table is written by
 * one launch on `stream`; `table` is caller-owned device memory, 256-byte aligned.
 * ------------------------------------------------------------------------------------------- */

/* Bytes of the table for this grid and split; 0 if the arguments are invalid. */
size_t st_rope3d_table_bytes(int T, int H, int W, const int rope_split[3]);

/* Build the table into `table` (device, >= st_rope3d_table_bytes bytes). */
st_status st_rope3d_table_build(int T, int H, int W, const int rope_split[3], float theta,
                                void* table, size_t table_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Full 3D attention: out = softmax(R q . (R k)^T / sqrt(d)) v over all N rows
 * ("full 3D attention", first page, self-test answer 2 and "How attention sees time").
 *
 * ST_BF16 runs in two steps, both on `stream`:
 *   stage:  the angle table and the rotated K rows as fp16 tiles of 64 keys, written into the
 *           caller's workspace (one pass over K);
 *   attend: the attention kernel; it rotates Q itself and streams the staged K tiles and the
 *           caller's V.  It runs in two launches: the first takes each row's score offset from
 *           its first 64 keys only and flags in the workspace any block of 256 query rows whose
 *           softmax row sums (taken against that offset) reach 2^64, infinity included; the second
 *           redoes only flagged blocks with a running maximum over every 64 keys.  Attention over
 *           fewer than 4096 (block, 64-key tile) pairs runs the second kind alone.  When the
 *           blocks would fill the chip's CUs badly (e.g. 31 blocks x 12 heads on 256 CUs), the
 *           first launch splits every block's keys in two halves, kept apart with their
 *           log-sum-exp in the workspace, and a merge launch combines them before the second.
 * st_attn3d_fwd = st_attn3d_stage + st_attn3d_attend.  The bf16 path rounds rotated q and k to
 * fp16 for the score product (q after its multiplication by log2(e)/sqrt(d)), so every rotated
 * k entry must stay below 65504 in magnitude and every rotated q entry below 65504 * sqrt(128) /
 * log2(e), about 5.1e5 (inputs with |x| < 2^15 are always safe); softmax weights multiply V in
 * bf16.  Past those limits the result is NaN, not a wrong number: the staging step turns a key
 * row with an entry past its limit into NaN, so every output row of that head is NaN, and a
 * query row past its limit gives a NaN output row (its scores are all infinite or NaN).
 * (st_attn3d_fwd_fused, which rotates K in the tile loads, does not make the key check.)
 * ST_F32 runs one fp32 kernel; its workspace is the angle table only.
 * ------------------------------------------------------------------------------------------- */

/* Workspace bytes st_attn3d_fwd (and stage/attend) need; 0 if the arguments are invalid.
 * ST_BF16: table + heads x ceil(N/64) x 64 x d x 2 bytes (K tiles) + heads x ceil(N/256) x 8
 * bytes (block flags), each part 256-byte aligned; with a key split (above) the flags double and
 * N x heads x (8 d + 8) bytes follow them (both halves' fp32 outputs and log-sum-exp).
 * ST_F32: table. */
size_t st_attn3d_workspace_bytes(int T, int H, int W, int n_text, int heads, int d,
                                 const int rope_split[3], st_dtype dtype);

/* q, k, v, out: [N][heads][d] of `dtype`.  The workspace is scratch owned by the caller and may
 * be reused as soon as the stream has run this call. */
st_status st_attn3d_fwd(const void* q, const void* k, const void* v,
                        int T, int H, int W, int n_text, int heads, int d,
                        const int rope_split[3], float theta, st_dtype dtype,
                        void* workspace, size_t ws_bytes, void* out, hipStream_t stream);

/* First step of the ST_BF16 path: fill `workspace` from k.  ST_F32 is not served here
 * (ST_ERR_UNSUPPORTED). */
st_status st_attn3d_stage(const void* k, int T, int H, int W, int n_text, int heads, int d,
                          const int rope_split[3], float theta, st_dtype dtype,
                          void* workspace, size_t ws_bytes, hipStream_t stream);

/* Second step of the ST_BF16 path: attention of q against the K tiles st_attn3d_stage wrote
 * for the same grid, n_text, heads, d and rope_split (read only), with values v.  The block-flag
 * part of the workspace is written (scratch), so calls sharing one workspace must not overlap.
 * Two kernel launches (see above). */
st_status st_attn3d_attend(const void* q, const void* v, int T, int H, int W, int n_text,
                           int heads, int d, const int rope_split[3], st_dtype dtype,
                           void* workspace, size_t ws_bytes, void* out, hipStream_t stream);

/* Workspace bytes of st_attn3d_fwd_fused: the angle table only. */
size_t st_attn3d_fused_workspace_bytes(int T, int H, int W, const int rope_split[3]);

/* The same result with RoPE fused into the attention kernel's tile loads: every K tile is
 * rotated (position decoded from its flat row index) while it is copied into LDS, with no
 * staging pass.  Two launches (table, attention).  ST_F32 runs the
 * fp32 kernel as st_attn3d_fwd does. */
st_status st_attn3d_fwd_fused(const void* q, const void* k, const void* v,
                              int T, int H, int W, int n_text, int heads, int d,
                              const int rope_split[3], float theta, st_dtype dtype,
                              void* workspace, size_t ws_bytes, void* out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Allocation-free full 3D attention, for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The result is st_attn3d_fwd's, bit for bit (same launches); its workspace is a static device
 * array of ST_NOALLOC_SCRATCH_BYTES inside the library, of which each GPU holds one copy from the
 * library's load until the process ends.  The array used is that of the stream's device (the
 * current device for the null stream), which the call makes current while it runs and then
 * restores.  The first call on a device takes the array's device address (hipGetSymbolAddress,
 * with that device current); no call allocates or frees anything.
 *   Limit   st_attn3d_workspace_bytes(...) for the request must not exceed
 *           ST_NOALLOC_SCRATCH_BYTES (128 MiB: e.g. 21x30x52 tokens x 12 heads needs 100.7 MB);
 *           larger requests return ST_ERR_WORKSPACE with nothing enqueued.
 *   Races   Every call on one GPU uses that GPU's single array: calls whose stream work overlaps
 *           on one GPU (other streams, other host threads) race and give wrong results.  Calls
 *           serialised on one stream are safe.
 * Arguments, layout and errors otherwise as st_attn3d_fwd; a failure to obtain the array's
 * address returns ST_ERR_HIP.
 * ------------------------------------------------------------------------------------------- */
#define ST_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

size_t st_attn3d_noalloc_scratch_bytes(void);

st_status st_attn3d_fwd_noalloc(const void* q, const void* k, const void* v,
                                int T, int H, int W, int n_text, int heads, int d,
                                const int rope_split[3], float theta, st_dtype dtype,
                                void* out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Factorised attention (first page, self-test answer 2): stage 1 attends inside each frame
 * (T sequences of H*W rows), stage 2 attends along time at each spatial position (H*W sequences
 * of T rows) with the same rotated q and k and stage 1's output as values.  No text rows
 * (n_text is 0 by construction: N = T*H*W).
 * ------------------------------------------------------------------------------------------- */

/* Workspace bytes: the angle table, for ST_BF16 the staged K tiles of the per-frame sequences
 * and their block flags (as for st_attn3d_fwd), and the stage-1 output [N][heads][d] of `dtype`. */
size_t st_attn_factorized_workspace_bytes(int T, int H, int W, int heads, int d,
                                          const int rope_split[3], st_dtype dtype);

st_status st_attn_factorized_fwd(const void* q, const void* k, const void* v,
                                 int T, int H, int W, int heads, int d,
                                 const int rope_split[3], float theta, st_dtype dtype,
                                 void* workspace, size_t ws_bytes, void* out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Local 3D-window attention (the CogVideoX record page, "Conditions": the W.A.L.T comparison
 * alternates per-frame spatial blocks with local 3D-window blocks).  The T x H x W grid is cut
 * into non-overlapping boxes of window[0] x window[1] x window[2] (t, h, w) tokens; each token
 * attends, non-causally with scale 1/sqrt(d), to the tokens of its own box, with q and k rotated
 * by their own (t, h, w) as in st_attn3d_fwd.  A window equal to the grid is full attention; a
 * window of (1, H, W) is the first stage of st_attn_factorized_fwd.
 *   q, k, v, out  [N][heads][d] in the flat grid order, N = T*H*W (no text rows); out must not
 *                 overlap q, k or v.
 *   window        {wt, wh, ww}, each >= 1 and dividing T, H, W respectively (else ST_ERR_SHAPE).
 * ST_BF16: d == 128, numerics as st_attn3d_fwd, N*heads*d*2 bytes below 2^32 (else
 * ST_ERR_UNSUPPORTED).  ST_F32: even d <= 128, at most 65535 windows.  Workspace (caller-owned,
 * 256-byte aligned, st_attn3d_window_workspace_bytes bytes, 0 for an invalid request): the angle
 * table and, for bf16, the rotated fp16 key tiles and the block flags of every window.  Three or
 * four launches (table, key staging, attention as in st_attn3d_attend) on `stream`.
 * ------------------------------------------------------------------------------------------- */
size_t st_attn3d_window_workspace_bytes(int T, int H, int W, int heads, int d,
                                        const int rope_split[3], const int window[3],
                                        st_dtype dtype);
st_status st_attn3d_window_fwd(const void* q, const void* k, const void* v, int T, int H, int W,
                               int heads, int d, const int rope_split[3], float theta,
                               const int window[3], st_dtype dtype, void* workspace,
                               size_t ws_bytes, void* out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Stand-alone 3D RoPE: y = R_3D(t, h, w) x for every row (text rows copied unchanged): the
 * block-diagonal rotation of "CogVideoX Architecture: ...", section "3. 3D Rotary Position
 * Embeddings (3D RoPE)", with the head cut into t, h and w ranges as in "A video model's
 * architecture: spatiotemporal attention and the 3D VAE", "Position: RoPE in three dimensions".
 * x and y: [N][heads][d]; y == x (in place) is allowed, other overlaps are not.  ST_BF16 needs
 * d % 8 == 0 (each 16-byte chunk holds four whole pairs; d == 128 takes a faster kernel), ST_F32
 * needs d even.  bf16 results are rotated in fp32 and rounded once.  Workspace (caller-owned,
 * 256-byte aligned): st_rope3d_table_bytes bytes; the angle table is rebuilt into it on every
 * call.  Two launches (table, rotation) on `stream`; all arguments are checked first.
 * ------------------------------------------------------------------------------------------- */
st_status st_rope3d_apply(const void* x, void* y, int T, int H, int W, int n_text, int heads,
                          int d, const int rope_split[3], float theta, st_dtype dtype,
                          void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Text cross-attention (the step after the self-attention in a Wan block: "04 · HunyuanVideo 与
 * Wan", section 3.1; queries from the video tokens, keys and values from at most 512 text tokens,
 * the text itself is not updated).  No rotation on either side; non-causal; scale 1/sqrt(d).
 *   q, out  [n_q][heads][d];  k, v  [n_kv][heads][d];  out must not overlap q, k or v.
 *   ST_BF16: d == 128, numerics as st_attn3d_fwd.  ST_F32: even d <= 128.
 *   Workspace (caller-owned, 256-byte aligned): st_attn_cross_workspace_bytes bytes, holding a
 *   table of zero angles (d/2 + 1 entries) and, for bf16, the fp16 key tiles and 8 bytes of flags
 *   per 256-row query block and head (scratch of the attention launches, rewritten every call).
 * ------------------------------------------------------------------------------------------- */
size_t st_attn_cross_workspace_bytes(int n_q, int n_kv, int heads, int d, st_dtype dtype);
st_status st_attn_cross_fwd(const void* q, const void* k, const void* v, int n_q, int n_kv,
                            int heads, int d, st_dtype dtype, void* workspace, size_t ws_bytes,
                            void* out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * QKV projection with the 3D rotation of its q and k outputs (the projections before the
 * attention of a Wan block: "04 · HunyuanVideo 与 Wan", section 3.1; the rotation as in
 * st_attn3d_fwd, "A video model's architecture", "Position: RoPE in three dimensions").
 *   x     [N][C] with N = T*H*W + n_text rows and C = heads * d input features
 *   w     [3C][C] output features by input features (a linear layer's weight layout); output
 *         feature f < C is q channel f % d of head f / d, C <= f < 2C is k, the rest v
 *   bias  [3C] or NULL
 *   q, k, v  [N][heads][d]: q = R(x w_q^T + b_q), k = R(x w_k^T + b_k), v = x w_v^T + b_v, where R
 *         turns each row by its (t, h, w) (text rows unchanged)
 * ST_BF16: d == 128; products on bf16 MFMA with fp32 accumulation, bias and rotation in fp32,
 * results rounded once to bf16; N*C*2 and 3C*C*2 bytes each below 2^31.  ST_F32: even d <= 128,
 * fp32 throughout.  Outputs must not overlap each other or the inputs.  Workspace (256-byte
 * aligned): st_qkv_rope_workspace_bytes bytes (the angle table).
 * ------------------------------------------------------------------------------------------- */
size_t st_qkv_rope_workspace_bytes(int T, int H, int W, const int rope_split[3]);
st_status st_qkv_rope_fwd(const void* x, const void* w, const void* bias, int T, int H, int W,
                          int n_text, int heads, int d, const int rope_split[3], float theta,
                          st_dtype dtype, void* workspace, size_t ws_bytes, void* q, void* k,
                          void* v, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Partial attention over a run of keys, and the merge of such partials (the single-device half
 * of context parallelism: the CogVideoX record page, "Budget for that cost, because it grows",
 * 2D ring and Ulysses; the first page's shard listing under "Position: RoPE in three
 * dimensions": a device holds a contiguous run of tokens whose (t, h, w) are absolute).
 *
 * st_attn3d_partial_fwd: the rows of q are global rows [q_begin, q_begin + q_count) and the rows
 * of k and v are global rows [kv_begin, kv_begin + kv_count) of the T*H*W + n_text sequence;
 * every row is rotated by its own global position.  Writes
 *   out [q_count][heads][d]  softmax over this run of keys times v (normalised, dtype of q)
 *   lse [q_count][heads]     float32 log sum_j exp(q~ . k~_j / sqrt(d)) over the run (natural log)
 * ST_BF16 runs as st_attn3d_attend does (the fast launch and its guard from 4096 (block, key
 * tile) pairs up), except that the keys are never split into halves.  Workspace:
 * st_attn3d_partial_workspace_bytes (0 for invalid arguments): the angle table, the fp16 key
 * tiles of the run and 8 bytes of block flags per 256 query rows and head, sized for a query run
 * of every row.  out, lse and the workspace must not overlap each other or any input.
 *
 * st_attn_merge: combines n_parts (1..16) partial results over disjoint runs of keys for the same
 * query rows into the result over their union: lse = log sum_i exp(lse_i), out = sum_i
 * exp(lse_i - lse) o_i, per (row, head).  o_parts and lse_parts are host arrays of device
 * pointers ([n_rows][heads][d] and [n_rows][heads]); out may be exactly one of the o_parts and
 * lse_out exactly one of the lse_parts (a running in-place merge); other overlaps are rejected.
 * lse_out may be NULL.  ST_BF16 needs d % 8 == 0 (d <= 512), ST_F32 d % 4 == 0 (d <= 256).
 * ------------------------------------------------------------------------------------------- */
size_t st_attn3d_partial_workspace_bytes(int T, int H, int W, int n_text, int heads, int d,
                                         const int rope_split[3], st_dtype dtype, int kv_count);
st_status st_attn3d_partial_fwd(const void* q, const void* k, const void* v, int T, int H, int W,
                                int n_text, int heads, int d, const int rope_split[3], float theta,
                                st_dtype dtype, int q_begin, int q_count, int kv_begin,
                                int kv_count, void* workspace, size_t ws_bytes, void* out,
                                float* lse, hipStream_t stream);
st_status st_attn_merge(int n_parts, const void* const* o_parts, const float* const* lse_parts,
                        int n_rows, int heads, int d, st_dtype dtype, void* out, float* lse_out,
                        hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Diagnostics.
 * ------------------------------------------------------------------------------------------- */

/* Static text naming a status code. */
const char* st_status_str(st_status s);

/* hipError_t of the last ST_ERR_HIP returned on the calling thread (0 if none). */
int st_last_hip_error(void);

/* Library version string, e.g. "0.1.0". */
const char* st_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ST_ATTN_H */
