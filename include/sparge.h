/*
 * sparge.h - C ABI of libsparge, block-sparse self-attention for AMD MI355X (gfx950).
 *
 * The method (SpargeAttention Documentation, the recommended top-k API and
 * "Mask Requirements"; Apply SpargeAttn, opening section) has two parts:
 *
 *   1. Mask prediction. Q is mean-pooled over 128-row blocks and K over 64-row
 *      blocks; pooled blocks are scored with softmax(qbar . kbar^T * scale)
 *      over the key blocks of each query block; each query block keeps the
 *      ceil(topk * n_kblocks) best key blocks, ties going to the lower key-block
 *      index. The result is mask_id of shape (B, H, ceil(N/128), ceil(N/64))
 *      with 0/1 entries.
 *   2. Attention. Softmax attention in which query block i only sees the keys
 *      of the key blocks its mask row selects. Skipped 128x64 tiles are never
 *      read.
 * Causal variant (the top-k API's is_causal flag, same page; its meaning
 * beyond the flag is this library's reading): key c is visible to query row r
 * when c <= r. Query block i ranks only the key blocks 0 .. J(i) =
 * floor(last row of block i / 64), keeps ceil(topk * (J(i) + 1)) of them (the
 * same rounding rule as sparge_topk_count), and within the kept blocks each
 * row sees its visible keys only; a row left with no visible kept key is
 * written as zeros.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Q, K, V and O are bf16, passed as uint16_t bit patterns, with logical
 *    shape (B, H, N, D) as in torch's scaled_dot_product_attention (the
 *    top-k API is a drop-in for it). Their element strides for the B, H and N
 *    axes are passed as int64_t[3]; the D axis must be contiguous. Every
 *    stride must be a non-negative multiple of 8 elements (the token stride of
 *    Q, K and V at most 2^24 elements, and that of K and V at least D, so
 *    that their rows do not overlap) and every base
 *    address 16-byte aligned, so that a row of 8 bf16 is one aligned load.
 *  - D (head dimension) must be 64 or 128. N >= 1, B >= 1, H >= 1; the calls
 *    that run attention also need N <= 2^31 - 128 (the kernel's key and row
 *    arithmetic is 32-bit; four such tensors would not fit in HBM anyway).
 *  - N_QB = ceil(N/128) query blocks and N_KB = ceil(N/64) key blocks.
 *  - scale <= 0 means the default 1/sqrt(D).
 *  - is_causal is 0 (non-causal) or 1 (causal, see above); other values are
 *    rejected with SPARGE_ERR_ARG.
 *  - Pointers are device pointers unless a parameter says otherwise. The
 *    caller owns every buffer. The library allocates no memory and keeps no
 *    state between calls.
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on it and returns without synchronising.
 *  - All arguments are validated on the host before any HIP call is made, so
 *    a rejected call has no side effect. Calls return SPARGE_OK (0) or one of
 *    the negative status codes below; no C++ exception crosses the ABI.
 *  - Calls that race on the same output buffers on different streams are the
 *    caller's responsibility; the library itself uses no global memory other
 *    than the buffers it is given and no atomics on them.
 */
#ifndef SPARGE_H
#define SPARGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARGE_OK 0
#define SPARGE_ERR_NULL -1       /* a required pointer is NULL */
#define SPARGE_ERR_SHAPE -2      /* B, H or N < 1, D not 64/128, N beyond the supported maximum */
#define SPARGE_ERR_TOPK -3       /* topk not in (0, 1] (or NaN) */
#define SPARGE_ERR_STRIDE -4     /* negative / unaligned stride or pointer, or an output layout that overlaps itself */
#define SPARGE_ERR_ALIAS -5      /* an output range overlaps an input range */
#define SPARGE_ERR_WORKSPACE -6  /* workspace NULL or smaller than sparge_workspace_bytes() */
#define SPARGE_ERR_ARG -7        /* another invalid argument (e.g. block_rows not 64/128) */
#define SPARGE_ERR_LAUNCH -8     /* the HIP runtime rejected a kernel launch (or a copy or synchronisation failed) */
#define SPARGE_ERR_MASK_VALUE -9 /* (checking calls only) a mask_id byte is neither 0 nor 1 */
#define SPARGE_ERR_SCRATCH_LIMIT -10 /* (no-allocation call) the shape needs more workspace than its fixed array */

/* Query rows per query block and key rows per key block
 * (SpargeAttention Documentation, "Mask Requirements": fixed 128x64 blocks). */
#define SPARGE_Q_BLOCK 128
#define SPARGE_K_BLOCK 64

/* Largest sequence length the mask-prediction calls accept (one row of
 * N_KB fp32 scores must fit in on-chip LDS). Attention alone has no such limit. */
#define SPARGE_MAX_PREDICT_N 786432

/* Static description of a status code (never NULL). */
const char *sparge_status_string(int status);

/* Host-only helper: the number of key blocks each query block keeps,
 * k = ceil(topk * n_kblocks) evaluated in IEEE double, where a product within
 * 1e-9 of an integer counts as that integer; clamped to [1, n_kblocks].
 * Writes k to *k_out. Errors: SPARGE_ERR_NULL, SPARGE_ERR_ARG (n_kblocks < 1),
 * SPARGE_ERR_TOPK. Makes no HIP call. */
int sparge_topk_count(int64_t n_kblocks, double topk, int64_t *k_out);

/* Bytes of device workspace that sparge_attn_topk (topk in (0,1]) or
 * block_sparse_attn (topk < 0: an arbitrary user mask) needs for this shape.
 * Returns 0 for invalid arguments, and for block_sparse_attn with a NULL mask
 * (dense attention needs no workspace, but the call accepts any workspace). */
size_t sparge_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, double topk);

/* Block-mean pooling, the first step of mask prediction: the "mean" of the
 * top-k API's meansim selection (SpargeAttention Documentation, the paragraph
 * on spas_sage2_attn_meansim_topk_cuda), over the 128-row query blocks and
 * 64-row key blocks of the mask (same page, "Mask Requirements").
 *   x          (B, H, N, D) bf16, strides x_strides (elements, B/H/N axes).
 *   block_rows 128 for Q, 64 for K.
 *   out        (B, H, ceil(N/block_rows), D) fp32, contiguous. Row i is the
 *              mean of x rows [i*block_rows, min(N, (i+1)*block_rows)),
 *              divided by the number of rows actually present.
 * Errors: NULL, SHAPE, STRIDE, ARG, ALIAS (out overlapping x), LAUNCH. */
int sparge_pool_blocks(const uint16_t *x, int64_t B, int64_t H, int64_t N, int64_t D,
                       const int64_t x_strides[3], int block_rows, float *out, void *stream);

/* Pooled-block scoring and per-row top-k selection: the "sim" and "topk" of
 * the same API (SpargeAttention Documentation, the paragraph on
 * spas_sage2_attn_meansim_topk_cuda: topk is the share of key blocks kept,
 * higher favouring accuracy), producing the block mask of "Mask Requirements"
 * (shape (B, H, ceil(N/128), ceil(N/64)), entries 0 or 1).
 *   qbar     (B, H, N_QB, D) fp32 contiguous (sparge_pool_blocks with 128).
 *   kbar     (B, H, N_KB, D) fp32 contiguous (sparge_pool_blocks with 64).
 *   topk     in (0, 1]; each row keeps k = sparge_topk_count(N_KB, topk) blocks
 *            (causal: sparge_topk_count(J(i) + 1, topk) of blocks 0 .. J(i)).
 *   scale    logit scale (<= 0: 1/sqrt(D)); s[i][j] = scale * qbar_i . kbar_j
 *            in fp32. Selection ranks s, which ranks the row softmax the same way.
 *   is_causal  0 or 1.
 *   mask_id  optional (NULL allowed): (B, H, N_QB, N_KB) uint8 contiguous, 1 for
 *            a kept block, 0 otherwise.
 *   kv_idx   (B, H, N_QB, k) int32 contiguous, k = sparge_topk_count(N_KB, topk):
 *            the kept key-block ids of each row in ascending order; entries
 *            past the row's kv_cnt (causal rows keep fewer) are not written.
 *   kv_cnt   (B, H, N_QB) int32: the number kept in each row (k, or the
 *            row's causal count).
 * Ties in s go to the lower key-block index, so the result is deterministic.
 * Errors: NULL, SHAPE (also N > SPARGE_MAX_PREDICT_N), TOPK, ARG, ALIAS, LAUNCH. */
int sparge_predict_mask(const float *qbar, const float *kbar, int64_t B, int64_t H, int64_t N,
                        int64_t D, double topk, float scale, int is_causal, uint8_t *mask_id,
                        int32_t *kv_idx, int32_t *kv_cnt, void *stream);

/* Mask compaction: each mask_id row becomes the ascending list of the key
 * blocks it selects (any nonzero byte counts as selected).
 *   mask_id  (B, H, N_QB, N_KB) uint8 contiguous.
 *   kv_idx   (B, H, N_QB, N_KB) int32 contiguous; entries past kv_cnt are unspecified.
 *   kv_cnt   (B, H, N_QB) int32.
 * Errors: NULL, SHAPE, ALIAS, LAUNCH. */
int sparge_compact_mask(const uint8_t *mask_id, int64_t B, int64_t H, int64_t N,
                        int32_t *kv_idx, int32_t *kv_cnt, void *stream);

/* Block-sparse attention from a compacted block list (the "apply" half of a
 * predict-then-apply split; a list may be reused across calls).
 *   kv_idx   (B, H, N_QB, ld_idx) int32: row r visits key blocks
 *            kv_idx[r][0 .. kv_cnt[r]-1], each in [0, N_KB). NULL means dense
 *            (every row visits all N_KB blocks; kv_cnt and ld_idx are ignored).
 *   kv_cnt   (B, H, N_QB) int32, each in [0, ld_idx].
 *   out      (B, H, N, D) bf16 with strides o_strides; rows with an empty list
 *            are written as zeros.
 * O[r] = sum_c softmax_c(scale * Q[r] . K[c]) V[c] over the keys c of the listed
 * blocks (with is_causal = 1: the listed keys c <= r), with fp32 accumulation,
 * probabilities rounded to bf16 before the PV product and the output rounded
 * to nearest-even bf16.
 * Errors: NULL, SHAPE, STRIDE, ALIAS, ARG (ld_idx < 1), LAUNCH. */
int sparge_attn_from_list(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          const int32_t *kv_idx, const int32_t *kv_cnt, int64_t ld_idx,
                          uint16_t *out, int64_t B, int64_t H, int64_t N, int64_t D,
                          const int64_t q_strides[3], const int64_t k_strides[3],
                          const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                          int is_causal, void *stream);

/* Block-sparse attention with a given block mask
 * (SpargeAttention Documentation, block_sparse_sage2_attn_cuda and "Mask
 * Requirements"). mask_id is (B, H, N_QB, N_KB) uint8 contiguous with 0/1
 * entries (nonzero counts as 1), or NULL for dense attention. The mask is
 * compacted into the workspace, then attention runs over the listed tiles
 * (with is_causal = 1 each row also ignores the keys after it).
 *   workspace   device buffer of at least sparge_workspace_bytes(B,H,N,D,-1).
 * Errors: NULL, SHAPE, STRIDE, ALIAS, ARG, WORKSPACE, LAUNCH. */
int block_sparse_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const uint8_t *mask_id, uint16_t *out, int64_t B, int64_t H, int64_t N,
                      int64_t D, const int64_t q_strides[3], const int64_t k_strides[3],
                      const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                      int is_causal, void *workspace, size_t workspace_bytes, void *stream);

/* Mask value check (SpargeAttention Documentation, "Mask Requirements": the
 * mask consists of 0 and 1 entries). Scans every byte of mask_id
 * ((B, H, N_QB, N_KB) uint8 contiguous) on the device and returns SPARGE_OK if
 * all are 0 or 1, SPARGE_ERR_MASK_VALUE otherwise. Unlike the other calls it
 * SYNCHRONISES `stream` (it reads the result back), so it is for debugging and
 * input validation, not for graph capture.
 *   workspace   device scratch of at least sparge_workspace_bytes(B, H, N, 64, -1)
 *               bytes (it uses 4 bytes per 256 mask bytes, at most 4 KiB).
 * Errors: NULL, SHAPE, WORKSPACE, ALIAS (workspace overlapping the mask), LAUNCH, MASK_VALUE. */
int sparge_check_mask(const uint8_t *mask_id, int64_t B, int64_t H, int64_t N, void *workspace,
                      size_t workspace_bytes, void *stream);

/* block_sparse_attn with its mask checked first: sparge_check_mask, then (only
 * if every byte is 0 or 1) block_sparse_attn with the same arguments. A mask
 * with another value is rejected with SPARGE_ERR_MASK_VALUE and nothing is
 * computed; the fast call instead counts any nonzero byte as 1. Synchronises
 * `stream` when mask_id is not NULL.
 * Errors: those of block_sparse_attn, plus MASK_VALUE. */
int block_sparse_attn_checked(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const uint8_t *mask_id, uint16_t *out, int64_t B, int64_t H, int64_t N,
                              int64_t D, const int64_t q_strides[3], const int64_t k_strides[3],
                              const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                              int is_causal, void *workspace, size_t workspace_bytes, void *stream);

/* Top-k block-sparse attention, a drop-in for scaled dot-product attention
 * (SpargeAttention Documentation, spas_sage2_attn_meansim_topk_cuda: higher
 * topk favours accuracy, lower topk sparsity; is_causal as described above).
 * Runs pooling, prediction and attention back to back on `stream`.
 *   topk        in (0, 1].
 *   scale       used both for the pooled scores and for attention (<= 0: 1/sqrt(D)).
 *   mask_out    optional (NULL allowed): receives the predicted mask_id,
 *               (B, H, N_QB, N_KB) uint8 contiguous.
 *   workspace   device buffer of at least sparge_workspace_bytes(B,H,N,D,topk).
 * Errors: NULL, SHAPE, TOPK, STRIDE, ALIAS, ARG, WORKSPACE, LAUNCH. */
int sparge_attn_topk(const uint16_t *q, const uint16_t *k, const uint16_t *v, double topk,
                     uint16_t *out, int64_t B, int64_t H, int64_t N, int64_t D,
                     const int64_t q_strides[3], const int64_t k_strides[3],
                     const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                     int is_causal, uint8_t *mask_out, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Bytes of the fixed device array that sparge_attn_topk_noalloc uses as its
 * workspace (one array per GPU, held from library load until the process ends). */
#define SPARGE_NOALLOC_SCRATCH_BYTES (128u << 20)

/* sparge_attn_topk for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and arguments, without the workspace arguments. Its
 * workspace is a fixed SPARGE_NOALLOC_SCRATCH_BYTES array in device memory,
 * one per GPU, resolved on the first call on each device; the call itself
 * allocates nothing. The caller still passes inputs and outputs.
 *   A shape whose workspace (sparge_workspace_bytes(B, H, N, D, topk)) exceeds
 *   the array is refused with SPARGE_ERR_SCRATCH_LIMIT before any HIP call
 *   (128 MiB covers, e.g., B=1, H=40, N=75600, D=128 up to topk 0.874).
 *   All calls on one GPU share its array and each call overwrites it: calls
 *   that may overlap on one GPU (different streams, or several host threads)
 *   race and must be serialised by the caller. The stream must belong to the
 *   current device.
 * Errors: those of sparge_attn_topk except WORKSPACE, plus SCRATCH_LIMIT;
 * LAUNCH also if the array's device address cannot be resolved. */
int sparge_attn_topk_noalloc(const uint16_t *q, const uint16_t *k, const uint16_t *v, double topk,
                             uint16_t *out, int64_t B, int64_t H, int64_t N, int64_t D,
                             const int64_t q_strides[3], const int64_t k_strides[3],
                             const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                             int is_causal, uint8_t *mask_out, void *stream);

/* CDF-threshold selection (the inference scripts' "cdfthreshd" mode, SpargeAttention
 * Documentation, output-directory list; the pages give only the name and a
 * value, this is the library's reading): each query block keeps its key blocks
 * in decreasing softmax probability (ties to the lower index) until their
 * cumulative probability reaches tau in (0, 1]; tau = 1 keeps every candidate.
 * The count varies from row to row. Probabilities are fp32 against the row
 * max, summed as exact 31-bit fixed-point weights, so the result is
 * deterministic. Causal candidates as for sparge_predict_mask.
 *   kv_idx   (B, H, N_QB, N_KB) int32 contiguous; row r lists kv_cnt[r] ids ascending.
 *   kv_cnt   (B, H, N_QB) int32.
 * Other arguments as sparge_predict_mask (tau in place of topk; a tau outside
 * (0, 1] is SPARGE_ERR_TOPK).
 * Errors: NULL, SHAPE (also N > SPARGE_MAX_PREDICT_N), TOPK, ARG, ALIAS, LAUNCH. */
int sparge_predict_mask_cdf(const float *qbar, const float *kbar, int64_t B, int64_t H, int64_t N,
                            int64_t D, double tau, float scale, int is_causal, uint8_t *mask_id,
                            int32_t *kv_idx, int32_t *kv_cnt, void *stream);

/* Pool, CDF-threshold selection and attention back to back (as sparge_attn_topk).
 *   workspace   device buffer of at least sparge_workspace_bytes(B, H, N, D, 1.0)
 *               (room for every row to keep every block).
 * Errors: NULL, SHAPE, TOPK (tau), STRIDE, ALIAS, ARG, WORKSPACE, LAUNCH. */
int sparge_attn_cdf(const uint16_t *q, const uint16_t *k, const uint16_t *v, double tau, uint16_t *out,
                    int64_t B, int64_t H, int64_t N, int64_t D, const int64_t q_strides[3],
                    const int64_t k_strides[3], const int64_t v_strides[3], const int64_t o_strides[3],
                    float scale, int is_causal, uint8_t *mask_out, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Token layouts for sparge_token_permutation. */
#define SPARGE_LAYOUT_RASTER 0   /* identity */
#define SPARGE_LAYOUT_CUBE 1     /* video tokens cube by cube */
#define SPARGE_LAYOUT_MORTON 2   /* video tokens along a Morton (Z-order) curve */

/* Host-only helper: a token order that groups video tokens into compact
 * spatiotemporal regions, so that 128-query and 64-key blocks cover nearby
 * tokens (Official repository for AB-Attention, "Optional cube layout": 4x4x4
 * spatiotemporal cubes; Attention Mechanisms (LightX2V), Sol-Attn on Wan2.1,
 * "Tuning and implementation": Morton3D ordering). The sequence is n_text text
 * tokens followed by a T x Hh x Ww video grid in raster order (w fastest).
 *   layout  SPARGE_LAYOUT_RASTER: identity. SPARGE_LAYOUT_CUBE: the text tokens,
 *           then the video tokens cube by cube, cubes of cube[0] x cube[1] x
 *           cube[2] (t, h, w) in raster order of the cube grid (a cube cut by
 *           the grid edge keeps the tokens it has), raster order inside a cube.
 *           SPARGE_LAYOUT_MORTON: the text tokens, then the video tokens by
 *           increasing Morton code (bit b of w, h, t at bits 3b, 3b+1, 3b+2).
 *   cube    int64[3] host array, used by SPARGE_LAYOUT_CUBE only (NULL allowed otherwise).
 *   perm    host array of n_text + T*Hh*Ww int32 the call fills: new position p
 *           holds old token perm[p].
 * Errors: NULL, ARG (negative n_text, empty grid, more than 2^31 - 1 tokens,
 * unknown layout, cube sides < 1, a Morton side beyond 2^21). Makes no HIP call. */
int sparge_token_permutation(int64_t n_text, int64_t T, int64_t Hh, int64_t Ww, int layout,
                             const int64_t cube[3], int32_t *perm);

/* Reorders the token axis of a (B, H, N, D) bf16 tensor by a permutation.
 *   x, x_strides      input, strides as for the attention calls.
 *   perm              device int32[N], a permutation of [0, N) (as from
 *                     sparge_token_permutation); an entry outside [0, N) moves nothing.
 *   out, out_strides  output, must not overlap x or perm.
 *   inverse           0: out[:, :, p] = x[:, :, perm[p]] (into the new order);
 *                     1: out[:, :, perm[p]] = x[:, :, p] (back to the old order).
 * With a perm that is not a permutation, rows of out may be left unwritten or
 * written twice (no out-of-bounds access either way).
 * Errors: NULL, SHAPE, STRIDE, ALIAS, ARG (inverse not 0/1), LAUNCH. */
int sparge_permute_tokens(const uint16_t *x, const int32_t *perm, uint16_t *out, int64_t B, int64_t H,
                          int64_t N, int64_t D, const int64_t x_strides[3],
                          const int64_t out_strides[3], int inverse, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARGE_H */
