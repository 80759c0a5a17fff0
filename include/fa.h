/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library libfa.so.
 *
 * The library computes exact scaled dot-product attention
 *     O = softmax(scale * Q K^T) V
 * tile by tile with an online softmax, so the N x N score and probability
 * matrices never reach device memory ("FlashAttention: Mathematical
 * Foundations, IO-Aware Tiling, Online Softmax, and Recomputation Dynamics",
 * sections "The GPU Memory Hierarchy and the Attention Memory Wall" and
 * "IO-Aware Tiling Algorithm"; "The Attention Matrix You Never Write Down",
 * section "The running-statistics trick").  The forward pass stores only O and
 * one per-row statistic, the log-sum-exp; the backward pass recomputes the
 * score and probability tiles on chip from Q, K, V and that statistic (same
 * article, section "Backward Pass and Activation Recomputation").  A
 * block-sparse forward skips the tiles a block mask zeroes ("Attention",
 * learn-kernels.com, paragraph on block-sparse FlashAttention).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Layout: Q, K, V, O, dO, dQ, dK, dV are dense [B][H][N][d] tensors with d
 *    innermost (row stride d elements, no padding).  LSE is dense fp32
 *    [B][H][N].
 *  - LSE is the natural-log log-sum-exp of the row's scaled scores over the
 *    allowed keys: LSE_i = ln(sum_j exp(scale * q_i . k_j)).  A row with no
 *    allowed key gets LSE = -inf and O = 0.
 *  - Masks: causal allows key j for query i iff j <= i.  kv_lens (nullable)
 *    is a device int32[B]; key j of batch entry b is allowed iff
 *    j < kv_lens[b]; every query row is still computed and written.  A block
 *    mask excludes the keys of a zero block from the softmax entirely.
 *  - Pointers: every tensor pointer is a DEVICE pointer owned by the caller;
 *    outputs must not alias inputs.  The library allocates nothing and is
 *    re-entrant.  Its only global state: the fixed device array of
 *    fa_bwd_noalloc (see there), and a per-kernel count of resident
 *    workgroups that the first causal forward call queries and keeps (it
 *    orders the causal work; results do not depend on it).
 *  - Streams: every call only enqueues work on `stream` (NULL = the default
 *    stream) and returns without synchronising; results are valid once the
 *    stream has reached that point.  Calls on different streams that share
 *    output buffers race.
 *  - Errors: return codes only.  Arguments are checked on the host before
 *    anything is enqueued; nothing is launched when a check fails.  The
 *    contents of device buffers (kv_lens values, mask bytes) are not checked:
 *    kv_lens values outside [0, N] are undefined behaviour.
 *  - Supported: d in {64, 128}; dtype BF16 everywhere; dtype FP32 for the
 *    dense forward only.  d = 256 for every bf16 attention entry point: the
 *    large head dimension at which the
 *    tiling loosens ("The Attention Matrix You Never Write Down", section
 *    "What it buys, and where the analysis bites").  bf16 tensors are IEEE
 *    bfloat16, rounded to nearest even on store; all accumulation is fp32.
 *  - Sizes: B, H, N >= 1 and B*H*N*d < 2^31.
 *  - Alignment: tensor pointers 16-byte aligned, LSE and kv_lens 4-byte
 *    aligned, the backward workspace 256-byte aligned (FA_ERR_INVALID_ARG,
 *    resp. FA_ERR_WORKSPACE, otherwise).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t, declared here so that the header needs no
 * HIP include. */
struct ihipStream_t;
typedef struct ihipStream_t *fa_stream_t;

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad scale, bad mask block */
    FA_ERR_UNSUPPORTED = 2, /* d, dtype or tile not built */
    FA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    FA_ERR_LAUNCH = 4       /* the HIP runtime refused the launch */
} fa_status;

typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_FP32 = 1 } fa_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char *fa_status_str(fa_status s);

/*
 * Forward: O and LSE from Q, K, V.
 *   q, k, v   in  [B][H][N][d], dtype
 *   o         out [B][H][N][d], dtype
 *   lse       out [B][H][N] fp32 (natural log)
 *   causal    0 or 1
 *   scale     finite, > 0 (normally 1/sqrt(d))
 *   kv_lens   nullable device int32[B] key-padding lengths
 * Errors: FA_ERR_INVALID_ARG for a null q/k/v/o/lse, B/H/N < 1, a
 * non-finite or non-positive scale, or B*H*N*d >= 2^31; FA_ERR_UNSUPPORTED
 * for d not in {64, 128} (bf16: {64, 128, 256}) or an unknown dtype.
 */
fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int H, int N, int d, int causal, float scale,
                 const int32_t *kv_lens, fa_dtype dtype, fa_stream_t stream);

/*
 * fa_fwd with an explicit key/value tile length tile_n (the B_c of the
 * pages' block-size constraint B_r*d + 2*B_c*d <= M, "FlashAttention:
 * Mathematical Foundations ...", section "IO-Aware Tiling Algorithm").
 * tile_n = 0 picks the default: for bf16 at d = 128 and N >= 2048 the
 * 32-key kernel, otherwise 64 (bf16) or 32 (fp32).  Built: for bf16 at
 * d = 64 and 128, 32 (a workgroup of 256 query rows in two wave groups that
 * alternate between matrix products and the softmax), 64 and 128 (128 query
 * rows, two LDS stages), 256 (one LDS stage: 128 KB of K and V at d = 128,
 * so copies do not overlap work); at d = 256, 32 and 64 (two stages of
 * 128-key tiles would not fit in LDS); 32 for fp32.  Other values give
 * FA_ERR_UNSUPPORTED.
 * Results equal fa_fwd's up to rounding order.
 */
fa_status fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int N, int d, int causal, float scale,
                    const int32_t *kv_lens, fa_dtype dtype, int tile_n,
                    fa_stream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: two fp32
 * [B][H][N] row vectors, each rounded up to 256 B -- the backward's
 * D_i = dO_i . O_i and the stored LSE_i rescaled to log2 units.  Returns 0
 * for invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward: dQ, dK, dV of L = sum(O * dO) from Q, K, V, O, dO and the LSE
 * the forward stored; S and P are recomputed tile by tile ("FlashAttention:
 * Mathematical Foundations ...", section "Backward Pass and Activation
 * Recomputation").  The gradient formulas are the chain rule of the
 * definition: dV = P^T dO, dP = dO V^T, D_i = dO_i . O_i,
 * dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 *   q, k, v, o, dout  in  [B][H][N][d] bf16
 *   lse               in  [B][H][N] fp32, as written by fa_fwd with the same
 *                         q, k, v, causal, scale and kv_lens
 *   dq, dk, dv        out [B][H][N][d] bf16 (dK, dV rows of padded keys are 0)
 *   workspace         device scratch of at least fa_bwd_workspace_bytes()
 *                     bytes, 256-byte aligned; contents on entry ignored
 * Errors: as fa_fwd, plus FA_ERR_WORKSPACE when workspace is NULL or
 * workspace_bytes is too small, and FA_ERR_UNSUPPORTED for dtype FP32.
 */
fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o,
                 const void *dout, const float *lse, void *dq, void *dk, void *dv,
                 int B, int H, int N, int d, int causal, float scale,
                 const int32_t *kv_lens, fa_dtype dtype, void *workspace,
                 size_t workspace_bytes, fa_stream_t stream);

/*
 * fa_bwd with an explicit tile length tile_n for the keys-outer dK/dV
 * kernel: the query rows of each Q and dO tile it streams through LDS past
 * its resident keys (the B_r of the pages' block-size constraint
 * B_r*d + 2*B_c*d <= M, "FlashAttention: Mathematical Foundations ...",
 * section "IO-Aware Tiling Algorithm", on the backward's side).
 * tile_n = 0 picks the default (64); 64 is built at d = 64, 128, 256 and 128
 * at d = 64, 128 (two stages of 128-row Q and dO tiles at d = 256 would need
 * 256 KB of LDS).  Other values give FA_ERR_UNSUPPORTED.  Other arguments and
 * errors as fa_bwd; results equal fa_bwd's up to rounding order.
 */
fa_status fa_bwd_ex(const void *q, const void *k, const void *v, const void *o,
                    const void *dout, const float *lse, void *dq, void *dk, void *dv,
                    int B, int H, int N, int d, int causal, float scale,
                    const int32_t *kv_lens, fa_dtype dtype, int tile_n, void *workspace,
                    size_t workspace_bytes, fa_stream_t stream);

/*
 * fa_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and results, with the backward's scratch (the D and
 * LSE*log2(e) row vectors) in a fixed device array inside the library
 * instead of a caller workspace.  It allocates nothing: no hipMalloc, no
 * hipFree, no allocating library call.
 *   Arguments as fa_bwd, without workspace.  stream must be NULL or a stream
 *   of the current device (whose copy of the array is used).
 *   Limit: B*H*N <= fa_bwd_noalloc_max_rows() (2^20 rows, 8 MiB of scratch
 *   per GPU, held until the process ends); larger sizes give
 *   FA_ERR_WORKSPACE.  A stream of another device gives FA_ERR_INVALID_ARG.
 *   Other errors as fa_bwd.
 * All calls on one GPU share its array: calls that overlap in time on one GPU
 * (other streams, other threads) race and give undefined results; calls
 * ordered on one stream are safe.  Nothing in the array needs clearing
 * between calls (every value read is written first by the same call).
 */
fa_status fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                         const void *dout, const float *lse, void *dq, void *dk, void *dv,
                         int B, int H, int N, int d, int causal, float scale,
                         const int32_t *kv_lens, fa_dtype dtype, fa_stream_t stream);

/* The row limit B*H*N of fa_bwd_noalloc. */
int fa_bwd_noalloc_max_rows(void);

/*
 * The three launches fa_bwd makes, callable one by one on the same stream
 * and in this order (results equal fa_bwd's bit for bit).  Useful to time
 * or overlap the stages separately.  Arguments mean what they mean for
 * fa_bwd; the workspace must be the same buffer for all three calls.
 *   fa_bwd_preprocess: workspace <- D_i = dO_i . O_i and LSE_i * log2(e).
 *   fa_bwd_dkdv:       dK, dV from Q, K, V, dO and the workspace
 *                      (keys-outer kernel).
 *   fa_bwd_dq:         dQ from Q, K, V, dO and the workspace
 *                      (queries-outer kernel).
 * fa_bwd_dkdv and fa_bwd_dq read the LSE only through the workspace; their
 * lse argument is still checked (non-NULL, aligned).
 * Errors: as fa_bwd.
 */
fa_status fa_bwd_preprocess(const void *o, const void *dout, const float *lse, int B, int H,
                            int N, int d, fa_dtype dtype, void *workspace, size_t workspace_bytes,
                            fa_stream_t stream);
fa_status fa_bwd_dkdv(const void *q, const void *k, const void *v, const void *dout,
                      const float *lse, void *dk, void *dv, int B, int H, int N, int d,
                      int causal, float scale, const int32_t *kv_lens, fa_dtype dtype,
                      const void *workspace, size_t workspace_bytes, fa_stream_t stream);
fa_status fa_bwd_dq(const void *q, const void *k, const void *v, const void *dout,
                    const float *lse, void *dq, int B, int H, int N, int d, int causal,
                    float scale, const int32_t *kv_lens, fa_dtype dtype, const void *workspace,
                    size_t workspace_bytes, fa_stream_t stream);

/*
 * Block-sparse forward ("Attention", learn-kernels.com, paragraph on
 * block-sparse FlashAttention): like fa_fwd (non-causal, no padding), but
 * the keys of block (r, c) are visible to the queries of block r only when
 * block_mask[r * (N / mask_block) + c] != 0.  Zero blocks are skipped, not
 * computed.
 *   block_mask  device uint8 [N/mask_block][N/mask_block], row-major,
 *               shared by every (b, h)
 *   mask_block  must be 128; N must be a multiple of it and N <= 65536
 * A query row whose mask row is all zero gets O = 0, LSE = -inf.
 * Errors: as fa_fwd, plus FA_ERR_INVALID_ARG for a null mask, a mask_block
 * other than 128 or N % mask_block != 0; FA_ERR_UNSUPPORTED for dtype FP32
 * or N > 65536.
 */
fa_status fa_fwd_blocksparse(const void *q, const void *k, const void *v, void *o,
                             float *lse, int B, int H, int N, int d, float scale,
                             const uint8_t *block_mask, int mask_block, fa_dtype dtype,
                             fa_stream_t stream);

/*
 * Block-sparse backward: dQ, dK, dV of the block-sparse forward above (same
 * mask, same conventions), with S and P recomputed only on the tiles of
 * nonzero blocks -- the training-side counterpart of the block-sparse
 * paragraph of "Attention" (learn-kernels.com).  The keys of a zero block
 * get no gradient from that block's queries; a key whose mask column is
 * all zero gets dK = dV = 0.
 *   q, k, v, o, dout, lse   as for fa_bwd (lse from fa_fwd_blocksparse with
 *                           the same mask)
 *   block_mask, mask_block  as for fa_fwd_blocksparse
 *   workspace               as for fa_bwd (fa_bwd_workspace_bytes bytes)
 * Errors: as fa_bwd and fa_fwd_blocksparse.
 */
fa_status fa_bwd_blocksparse(const void *q, const void *k, const void *v, const void *o,
                             const void *dout, const float *lse, void *dq, void *dk, void *dv,
                             int B, int H, int N, int d, float scale,
                             const uint8_t *block_mask, int mask_block, fa_dtype dtype,
                             void *workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * Decode-shaped forward with the key range split over workgroups.  The pages
 * single out decoding -- the key/value cache grows by one token per step and
 * each step is a small, frequent product -- as the case that needs its own
 * kernel ("Attention", learn-kernels.com, paragraph on decoding).  Each
 * split computes its keys' normalised output and log-sum-exp, and the splits
 * are combined by the two-block update of "FlashAttention: Mathematical
 * Foundations, IO-Aware Tiling, Online Softmax, and Recomputation Dynamics",
 * section "Incremental Online Updates" (the merge below).  The result is the
 * same exact attention as fa_fwd, over a rectangular score matrix.
 *   q, o     device bf16 [B][H][Nq][d]: the Nq newest query rows of each
 *            sequence, 1 <= Nq <= 8
 *   k, v     device bf16 [B][H][Nk][d]: the key/value cache
 *   lse      device fp32 [B][H][Nq]
 *   kv_lens  nullable device int32[B]: rows 0 .. kv_lens[b]-1 of batch entry
 *            b's cache are filled (all Nk when NULL); values outside [0, Nk]
 *            are clamped to it
 *   causal   0: every query sees every filled key.  1: query t sits at
 *            position kv_len - Nq + t and sees keys j <= kv_len - Nq + t
 *            (for Nq = 1 both are the same)
 *   num_splits  0 chooses the split count from B*H and Nk; otherwise the
 *            requested count, lowered so that each split holds at least 32
 *            keys (fa_splitkv_splits returns the count used)
 *   workspace   device, 256-byte aligned, at least
 *            fa_fwd_splitkv_workspace_bytes(...) bytes (may be NULL when that
 *            is 0, i.e. when one split is used); overwritten
 * A query that sees no key gets O = 0, LSE = -inf.
 * Errors: FA_ERR_INVALID_ARG for null pointers, sizes < 1, num_splits < 0,
 * a non-finite or non-positive scale, misalignment or B*H*max(Nq,Nk)*d >= 2^31;
 * FA_ERR_UNSUPPORTED for d not in {64, 128, 256}, Nq > 8 or dtype other than
 * BF16; FA_ERR_WORKSPACE for a missing, small or misaligned workspace.
 */
int fa_splitkv_splits(int B, int H, int Nk, int num_splits);
size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits);
fa_status fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                         int B, int H, int Nq, int Nk, int d, int causal, float scale,
                         const int32_t *kv_lens, int num_splits, fa_dtype dtype,
                         void *workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * Merge S partial results of the same R rows, each computed over a disjoint
 * set of keys ("FlashAttention: Mathematical Foundations ...", section
 * "Incremental Online Updates", in log-sum-exp form):
 *     LSE = ln(sum_s exp(LSE_s)),   O = sum_s exp(LSE_s - LSE) * O_s.
 * This is the combine step of fa_fwd_splitkv and of any split of one head's
 * keys across calls or devices.
 *   o_parts    device fp32 [S][R][d], each part's normalised output
 *   lse_parts  device fp32 [S][R], natural log; -inf marks an empty part,
 *              whose o_parts rows are ignored
 *   o          device [R][d], dtype BF16 or FP32;  lse  device fp32 [R]
 * Rows whose parts are all empty get O = 0 and LSE = -inf.
 * Errors: FA_ERR_INVALID_ARG for null pointers, S < 1, R < 1, d < 1,
 * d > 1024, R*d >= 2^31 or misaligned pointers (4 bytes; 2 for a bf16 o);
 * FA_ERR_UNSUPPORTED for another dtype.
 */
fa_status fa_merge(const float *o_parts, const float *lse_parts, int S, int R, int d, void *o,
                   float *lse, fa_dtype dtype, fa_stream_t stream);

/*
 * Block-quantised FP8 forward.  The pages describe it as FP8 matrix products
 * on block-quantised operands with dynamic scaling ("FlashAttention:
 * Mathematical Foundations ...", section "FlashAttention-3", item on
 * low-precision FP8 support), made more accurate by incoherent processing
 * ("Attention", learn-kernels.com, paragraph on Hopper).  Format: OCP E4M3
 * ("FN": bias 7, largest finite 448, no infinities), one byte per element.
 * Each block's largest magnitude maps to 448: code = E4M3(x * (448 / amax)),
 * descale = amax / 448 (fp32; an all-zero block gets descale 1).
 *
 * fa_quantize_fp8: bf16 x [B][H][N][d] -> E4M3 codes x8 and descales.
 *   block_rows  128: one scale per 128 consecutive rows of a (b, h), descale
 *               [B][H][ceil(N/128)] (the layout fa_fwd_fp8 takes for Q, K);
 *               0: one scale per (b, h), descale [B][H] (V)
 *   signs       nullable device fp32[d] of +1/-1: before quantising, multiply
 *               every row by R = diag(signs) H_d / sqrt(d) (H_d the Sylvester
 *               Hadamard matrix; fast Walsh-Hadamard butterflies in fp32).
 *               Pass the same signs for Q and K and none for V: R is
 *               orthogonal, so the scores are unchanged
 *   transpose   0: x8 [B][H][N][d]; 1: x8 [B][H][d][N] (the layout fa_fwd_fp8
 *               takes for V); needs N % 16 == 0
 *   workspace   block_rows = 0 only: fa_quantize_fp8_workspace_bytes(...)
 *               bytes, 256-byte aligned (may be NULL when that is 0)
 * Errors: FA_ERR_INVALID_ARG for null pointers, sizes < 1, block_rows not
 * in {0, 128}, B*H*N*d >= 2^31, transpose with N % 16 != 0, misalignment
 * (x, x8: 16 bytes; descale, signs: 4); FA_ERR_UNSUPPORTED for d not in
 * {64, 128}; FA_ERR_WORKSPACE for a missing, small or misaligned workspace.
 *
 * fa_fwd_fp8: O (bf16) and LSE of exact attention on the dequantised
 * inputs, with the probabilities rounded to E4M3 on chip for the P V product
 * (their row sum is taken before rounding).  q8, k8: [B][H][N][d] codes with
 * q_descale, k_descale [B][H][ceil(N/128)]; v8t: [B][H][d][N] codes with
 * v_descale [B][H]; other arguments as fa_fwd.  N must be a multiple of 16.
 * Codes must not be NaN.
 * Errors: FA_ERR_INVALID_ARG for null pointers, sizes < 1, N % 16 != 0, a
 * non-finite or non-positive scale, B*H*N*d >= 2^31, misalignment;
 * FA_ERR_UNSUPPORTED for d not in {64, 128}.
 */
size_t fa_quantize_fp8_workspace_bytes(int B, int H, int N, int d, int block_rows);
fa_status fa_quantize_fp8(const void *x, void *x8, float *descale, int B, int H, int N, int d,
                          int block_rows, const float *signs, int transpose, void *workspace,
                          size_t workspace_bytes, fa_stream_t stream);
fa_status fa_fwd_fp8(const void *q8, const void *k8, const void *v8t, const float *q_descale,
                     const float *k_descale, const float *v_descale, void *o, float *lse, int B,
                     int H, int N, int d, int causal, float scale, const int32_t *kv_lens,
                     fa_stream_t stream);

/*
 * The key/value-outer loop order, kept as an IO ablation of the forward
 * ("FlashAttention: Mathematical Foundations, IO-Aware Tiling, Online
 * Softmax, and Recomputation Dynamics", section "IO-Aware Tiling Algorithm";
 * "01 · FlashAttention", step 5, the HBM accounting).  The outer loop walks
 * 64-key blocks (one launch each) and the inner loop 128-row query blocks, so
 * every query block's fp32 output accumulator and running statistics go
 * through device memory once per key block.  Same results as fa_fwd (exact
 * attention, O bf16 and LSE as in the conventions above; no kv_lens); it is
 * not a fast path.
 *
 * fa_fwd_kvouter_workspace_bytes: bytes of the workspace, or 0 for
 * unsupported sizes: fp32 O accumulator [B][H][N][d] followed by two fp32
 * [B][H][N] statistics, each rounded up to 256 bytes.
 * fa_fwd_kvouter: arguments as fa_fwd (bf16 only), plus the workspace
 * (256-byte aligned, at least the size above; its contents on entry do not
 * matter and are overwritten).
 * Errors: FA_ERR_INVALID_ARG for null pointers, sizes < 1, a non-finite or
 * non-positive scale, B*H*N*d >= 2^31, misalignment; FA_ERR_UNSUPPORTED for
 * d not in {64, 128}; FA_ERR_WORKSPACE for a missing, small or misaligned
 * workspace.
 */
size_t fa_fwd_kvouter_workspace_bytes(int B, int H, int N, int d);
fa_status fa_fwd_kvouter(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                         int H, int N, int d, int causal, float scale, void *workspace,
                         size_t workspace_bytes, fa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
