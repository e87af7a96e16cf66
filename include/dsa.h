/*
 * dsa.h -- C ABI of libdsa, the gfx950 (MI355X) DeepSeek Sparse Attention
 * (DSA) layer step: lightning-indexer scores, per-query top-k, and sparse
 * MLA attention over only the selected keys, plus the pooled (kpool) NoPE
 * variant.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller (for instance
 *    torch.Tensor.data_ptr()).  Tensors are dense, row-major, with the shape
 *    given next to each argument.  The library never allocates, frees or
 *    keeps device memory; scratch memory comes from a caller-provided
 *    `workspace` of at least the size the matching *_workspace_size() call
 *    returns (NULL is fine when that size is 0).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call is asynchronous on that stream: it only validates arguments
 *    on the host and enqueues kernels.  There is no device synchronisation
 *    and no host<->device copy inside any call.
 *  - Every call returns a dsa_status.  Arguments are checked on the host
 *    before anything is launched; on an error nothing is enqueued and
 *    dsa_last_error() describes the problem.  A fault inside a kernel (for
 *    instance a pointer to too small a buffer) surfaces at the caller's next
 *    synchronisation, as for any HIP kernel.
 *  - Every element of every output is written: INVALID in empty index slots,
 *    -FLT_MAX for invisible scores, 0 / -inf for an empty attention set.
 *  - There is no CPU fallback: a shape outside a kernel's envelope returns
 *    DSA_ERR_UNSUPPORTED.
 *  - Calls are thread-safe; the only state is the per-thread last error.
 *
 * Sources of the definitions (cited per function below):
 *  [fak]    "GLM-5.2: the DSA sparse attention moves onto the pure fak kernel
 *           (2026-06-23)" -- table under "What changed" and the section "The
 *           selection stays host-side BY DESIGN".
 *  [ik]     "Another DSA attempt" (ik_llama.cpp PR #2063) -- the squashed
 *           commit messages of the batch-local indexer and of the decode
 *           indexer-K cache.
 *  [metrale] "Module glm5next_dsa_ref" -- index_scores, visible, topk_pools,
 *           expand_selection, topk_to_mask, pool_states, kept_pools,
 *           mla_masked_attention, INVALID, DsaDims and the invariants list.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The invalid-index sentinel ([metrale] INVALID). */
#define DSA_INVALID (-1)

typedef enum {
    DSA_OK = 0,
    DSA_ERR_ARG = -1,         /* null pointer, non-positive size, bad dtype, ... */
    DSA_ERR_UNSUPPORTED = -2, /* shape or dtype outside every kernel's envelope  */
    DSA_ERR_HIP = -3,         /* a HIP launch failed                              */
    DSA_ERR_WORKSPACE = -4    /* workspace missing or too small                   */
} dsa_status;

typedef enum {
    DSA_F32 = 0,
    DSA_BF16 = 1,
    DSA_FP8_E4M3 = 2 /* OCP FP8 E4M3 ("e4m3fn"): bias 7, max 448, no infinity */
} dsa_dtype;

/* Message of the last failed call on this thread ("" if none). */
const char *dsa_last_error(void);

/* Library version string. */
const char *dsa_version(void);

/* ------------------------------------------------------------------------
 * Visibility ranges.
 *
 * [metrale] visible: a key is visible to a query iff it is causal and not
 * padding.  With left padding `pad[b]` and query position q_pos[b,t] the
 * visible token keys form one range [vis_lo, vis_hi) = [pad, q_pos + 1); the
 * query's own position is visible ([ik] batch-local indexer: base causal
 * mask).  A padded query (q_pos < pad) gets the empty range [0, 0).
 *
 * kpool > 0 gives the ranges over POOLS instead ([metrale] pool_states,
 * invariants list: pooling starts at the first valid token and a pool is
 * valid only if all of its kpool slots are): pool i is a candidate iff all
 * its tokens are visible, so the range is [0, floor((q_pos - pad + 1) /
 * kpool)).
 *
 * pad: [batch] int32; q_pos: [batch, n_q] int32;
 * vis_lo, vis_hi: [batch, n_q] int32 outputs.
 * ------------------------------------------------------------------------ */
int dsa_visibility_ranges(int32_t batch, int32_t n_q, const int32_t *pad,
                          const int32_t *q_pos, int32_t kpool, int32_t *vis_lo,
                          int32_t *vis_hi, void *stream);

/* ------------------------------------------------------------------------
 * Lightning-indexer scores.
 *
 * scores[b,t,s] = sum_h w[b,t,h] * relu(scale * sum_c q[b,t,h,c] * k'[b,s,c])
 * for vis_lo[b,t] <= s < vis_hi[b,t] (clipped to [0, n_k)); every other
 * element is set to -FLT_MAX.  One key head is shared by all indexer heads
 * (MQA).  k' = k, or k * k_scale[b,s] for FP8 keys.
 * ([fak] "The selection stays host-side BY DESIGN"; [ik] batch-local indexer
 * commit: relu(indexer_k . indexer_q), scaled per-head weights, summed over
 * heads; [metrale] index_scores.)
 *
 * q:       [batch, n_q, n_heads, head_dim]  q_dtype (BF16 or F32)
 * k:       [batch, n_k, head_dim]           k_dtype (BF16 or FP8_E4M3 with
 *          BF16 q; F32 with F32 q)
 * k_scale: [batch, n_k] f32 for FP8 keys, else NULL
 * w:       [batch, n_q, n_heads] f32
 * vis_lo, vis_hi: [batch, n_q] int32
 * scores:  [batch, n_q, n_k] f32 output
 *
 * Envelope: BF16 q requires n_heads a multiple of 32 (at most 64) and
 * head_dim 64 or 128, accumulating bf16 products in f32 on MFMA; F32 takes
 * any shape.  Rounding: each product is exact and the sums are f32, so
 * |err| is a few f32 ulps of sum_h |w| |scale| sum_c |q k|.
 * ------------------------------------------------------------------------ */
typedef struct {
    int32_t batch, n_q, n_k, n_heads, head_dim;
    float scale;
} dsa_index_dims; /* no field has a default ([metrale] DsaDims) */

int dsa_index_scores(const dsa_index_dims *d, const void *q, int q_dtype,
                     const void *k, int k_dtype, const float *k_scale,
                     const float *w, const int32_t *vis_lo,
                     const int32_t *vis_hi, float *scores, void *stream);

/* ------------------------------------------------------------------------
 * Per-query top-k.
 *
 * For each row r, the min(top_k, n_visible) visible columns of
 * scores[r, vis_lo[r] .. vis_hi[r]) (clipped to [0, n_cols)), ordered by
 * higher score, then smaller column index; INVALID pads the row to top_k.
 * +0 and -0 are equal scores.  NaN scores are ranked by their bit pattern
 * (a NaN input is outside the method; the oracle rejects it).
 * ([metrale] topk_pools: higher score then smaller index; [ik] batch-local
 * indexer commit: top_k(min(top_k, n_tokens)); [fak] host f64 top-k.)
 * The result is exact: the selection is a pure comparison of the f32 scores.
 *
 * scores:  rows x n_cols f32, row r at scores + r*row_stride
 * vis_lo, vis_hi: [rows] int32
 * out_idx: [rows, top_k] int32 output
 * Envelope: 1 <= top_k <= 2048; n_cols < 2^31.
 * ------------------------------------------------------------------------ */
size_t dsa_topk_workspace_size(int32_t rows, int32_t n_cols, int32_t top_k);

int dsa_topk(const float *scores, int32_t rows, int32_t n_cols,
             int64_t row_stride, const int32_t *vis_lo, const int32_t *vis_hi,
             int32_t top_k, int32_t *out_idx, void *workspace,
             size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Sparse attention over each query's selected keys.
 *
 * For each (b, t, h), over the set J of distinct entries j of idx[b,t,:] with
 * 0 <= j < n_k, j != INVALID and (when vis_lo/vis_hi are given)
 * vis_lo[b,t] <= j < vis_hi[b,t]:
 *   out[b,t,h,:] = sum_{j in J} softmax_j(scale * q[b,t,h,:] . K_j) V_j
 *   lse[b,t,h]   = log sum_{j in J} exp(scale * q[b,t,h,:] . K_j)
 * An empty J gives out = 0 and lse = -inf.
 * ([fak] table under "What changed": per-head softmax(scale*q*k) and the sum
 * of w*V over the selected keys, key width kd = qk_nope + qk_rope different
 * from value width vd; [metrale] topk_to_mask: duplicates collapse,
 * out-of-range and INVALID entries are dropped; mla_masked_attention.)
 *
 * q:   [batch, n_q, n_heads, kd]
 * k:   key row j of sequence b at k + (b*n_k + j)*k_row_stride (elements);
 *      the row holds kv_heads vectors of kd; head h reads vector
 *      h / (n_heads / kv_heads)
 * v:   likewise with vd and v_row_stride; v may alias k (absorbed MLA:
 *      V_j = the first vd columns of the latent row K_j)
 * idx: [batch, n_q, n_sel] int32 (any order; rank order from dsa_topk)
 * vis_lo, vis_hi: [batch, n_q] int32, or both NULL
 * out: [batch, n_q, n_heads, vd] f32 output
 * lse: [batch, n_q, n_heads] f32 output, or NULL
 *
 * dtype (q, k, v): BF16 or F32.  Envelope: n_k <= 524288.  BF16 with
 * kv_heads == 1 runs the gather kernel (MFMA, keys gathered per query and
 * shared by all heads; n_heads == 64, kd == 576, vd == 512, n_k <= 262144).
 * BF16 with kv_heads == n_heads runs the masked-tile kernel (MFMA over key
 * tiles with a per-query selection bitmap; kd == 192, vd == 256).  Other
 * shapes run a plain (non-MFMA) kernel.  The softmax weights enter the
 * value product as a two-term bf16 split (about 16 significant bits); sums
 * are f32.
 * ------------------------------------------------------------------------ */
typedef struct {
    int32_t batch, n_q, n_k, n_heads, kd, vd, kv_heads, n_sel;
    float scale;
} dsa_attn_dims;

size_t dsa_sparse_attend_workspace_size(const dsa_attn_dims *d);

int dsa_sparse_attend(const dsa_attn_dims *d, int dtype, const void *q,
                      const void *k, int64_t k_row_stride, const void *v,
                      int64_t v_row_stride, const int32_t *idx,
                      const int32_t *vis_lo, const int32_t *vis_hi, float *out,
                      float *lse, void *workspace, size_t workspace_bytes,
                      void *stream);

/* ------------------------------------------------------------------------
 * Pooled (kpool) variant.
 *
 * Sequence b has pad[b] left-padding tokens.  Pools start at the first
 * valid token: pool i holds tokens pad + i*kpool + j, j < kpool, and a
 * trailing partial pool is not a pool, so n_pools[b] =
 * floor((seq - pad[b]) / kpool)  ([metrale] pool_states, kept_pools and the
 * invariants list).
 * ------------------------------------------------------------------------ */
typedef struct {
    int32_t batch, seq, n_q, kpool, head_dim, select_k, out_width;
} dsa_pool_dims;

/* Pool keys ([metrale] pool_states; invariants list: the softmax runs over
 * the slot axis separately for each head_dim channel):
 *   pooled[b,i,c] = sum_j softmax_j(gate[b,t_j,c]) * k[b,t_j,c]
 * computed in f32 and rounded once to the storage dtype.
 * k, gate: [batch, seq, head_dim] dtype (BF16 or F32)
 * pad:     [batch] int32
 * pooled:  [batch, seq / kpool, head_dim] dtype output; rows >= n_pools[b]
 *          are zero
 * n_pools: [batch] int32 output */
int dsa_pool_keys(const dsa_pool_dims *d, int dtype, const void *k,
                  const void *gate, const int32_t *pad, void *pooled,
                  int32_t *n_pools, void *stream);

/* Pool select ([metrale] topk_pools followed by expand_selection).  For the
 * query at q_pos = p of sequence b, the candidates are the n_full =
 * floor((p - pad + 1) / kpool) pools whose tokens are all visible (pool
 * visibility extends "a pool is valid only if all kpool slots are valid" to
 * the causal query).  Up to select_k pools are taken in rank order (higher
 * score, then smaller pool index).  The token row lists each taken pool's
 * kpool tokens ascending, pools in rank order, then the visible tail
 * pad + n_full*kpool .. p ascending, then INVALID up to out_width.  A padded
 * query (p < pad) gets an all-INVALID row.
 * pool_scores: [batch, n_q, seq / kpool] f32 (dsa_index_scores over the
 *              pooled keys)
 * pad:        [batch] int32;  q_pos: [batch, n_q] int32
 * out_tok:    [batch, n_q, out_width] int32 output
 * out_pools:  [batch, n_q, select_k] int32 output, or NULL
 * Envelope: 1 <= select_k <= 2048, out_width >= select_k*kpool + kpool - 1,
 * seq / kpool <= 16384. */
size_t dsa_pool_select_workspace_size(const dsa_pool_dims *d);

int dsa_pool_select(const dsa_pool_dims *d, const float *pool_scores,
                    const int32_t *pad, const int32_t *q_pos, int32_t *out_tok,
                    int32_t *out_pools, void *workspace, size_t workspace_bytes,
                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
