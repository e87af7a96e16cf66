/*
 * dsa.h -- C ABI of libdsa, the gfx950 (MI355X) DeepSeek Sparse Attention
 * (DSA) layer step: lightning-indexer scores, per-query top-k, and sparse
 * MLA attention over only the selected keys, plus the pooled (kpool) NoPE
 * variant.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller (for instance
 *    torch.Tensor.data_ptr()).  Tensors are dense, row-major, with the shape
 *    given next to each argument.  The library never allocates or frees
 *    device memory; scratch memory comes from a caller-provided `workspace`
 *    of at least the size the matching *_workspace_size() call returns (NULL
 *    is fine when that size is 0).  The one exception is dsa_topk_noalloc,
 *    whose scratch is a fixed array the library's code object holds on each
 *    GPU.
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
 * Envelope: BF16 q requires n_heads 32 or 64 and head_dim 64 or 128,
 * accumulating the exact bf16 products in f32 on MFMA, so |err| <=
 * (head_dim + n_heads + 4) * 2^-23 * sum_h |w| |scale| sum_c |q k|.  F32
 * takes any shape and sums the exact products in f64, so the score is
 * within a few f32 ulps of its own value unless the sum cancels almost
 * completely.
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
 * Attention sinks (n_sink > 0): the first n_sink columns of each row's
 * visible range -- for token keys, the sequence's first present positions
 * that the query can see -- take ranks 0 .. n_sink-1 in column order, and
 * the row's other visible columns follow in rank order ([ik] decode
 * indexer-K cache commit: the first key(s) get a boost so the sink always
 * survives top-k; per-sequence sink commit: only the query's own sequence's
 * sink; serving-correctness commit: anchored on the first present
 * position).  The pages add 1e20 to the f32 scores of those columns; when
 * every score's magnitude is below 2^42 that addition gives each sink
 * exactly 1e20f and leaves every other score below it, which is the order
 * stated here.  n_sink = 0: no sinks.
 *
 * scores:  rows x n_cols f32, row r at scores + r*row_stride
 * vis_lo, vis_hi: [rows] int32
 * n_sink:  >= 0 (values above top_k act as top_k)
 * out_idx: [rows, top_k] int32 output
 * Envelope: 1 <= top_k <= 2048; n_cols < 2^31; rows x row_stride <= 2^46.
 * dsa_topk_workspace_size returns the bytes dsa_topk needs for these sizes
 * (0 for rows of at most 16384 keys, and 0 for sizes dsa_topk refuses).
 * ------------------------------------------------------------------------ */
size_t dsa_topk_workspace_size(int32_t rows, int32_t n_cols, int32_t top_k);

int dsa_topk(const float *scores, int32_t rows, int32_t n_cols,
             int64_t row_stride, const int32_t *vis_lo, const int32_t *vis_hi,
             int32_t top_k, int32_t n_sink, int32_t *out_idx, void *workspace,
             size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Top-k that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc.
 *
 * Arguments and results are those of dsa_topk without the workspace.  Rows
 * longer than 16384 keys keep their per-block (key, count) pairs and their
 * candidates (up to 262144 keys), or their chunk winners (longer rows), in
 * a scratch array the library holds in each GPU's memory until the process
 * ends (DSA_TOPK_NOALLOC_SCRATCH_BYTES per GPU); its device address is
 * looked up once per device, on the first call made with that device
 * current.  Nothing in it has to start at zero: each call clears the
 * counters it uses in its own first kernel.
 * Limit: dsa_topk_workspace_size(rows, n_cols, top_k) <= 16 MiB (for
 * instance 8 rows of 131072 keys at top_k 2048 need 1.07 MiB); a larger call
 * returns DSA_ERR_UNSUPPORTED and enqueues nothing.  The call itself
 * allocates nothing (no hipMalloc, no library allocation).
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents: calls ordered on one stream are safe, but two calls
 * whose kernels may overlap on one GPU (different streams without ordering)
 * race and give wrong results.  `stream` must belong to the current device
 * (DSA_ERR_ARG otherwise).
 * ------------------------------------------------------------------------ */
#define DSA_TOPK_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int dsa_topk_noalloc(const float *scores, int32_t rows, int32_t n_cols,
                     int64_t row_stride, const int32_t *vis_lo,
                     const int32_t *vis_hi, int32_t top_k, int32_t n_sink,
                     int32_t *out_idx, void *stream);

/* ------------------------------------------------------------------------
 * The indexer front-end: the indexer's q, k and head weights from the
 * layer's activations.
 *
 * [ik] batch-local indexer commit: indexer_q = wq_b(q_lora latent), each
 * head split rope(64) / nope(64), the rope part NEOX-rotated, concatenated
 * back; indexer_k = wk(attention-norm output), then LayerNorm with bias
 * (k_norm), then the same rotation (one key head); the head weights come
 * from weights_proj.  [metrale] layer_norm: subtract the mean, divide by
 * the standard deviation, then w * x + b; linear: y = x w^T.  [ik] CPU
 * crash-fix commit and review: k_norm's eps must be positive (1e-6 in the
 * reference, the model's 1e-5 in one port).
 *
 * For token t at position pos[t]:
 *   q[t,h,:] = rope(q_lora[t,:] wq_b[h*128 .. h*128+128, :]^T)
 *   k[t,:]   = rope(LayerNorm(x[t,:] wk^T; k_norm_w, k_norm_b, norm_eps))
 *   w[t,:]   = x[t,:] w_proj^T
 * where rope rotates entries i and i + rope_dim/2 (i < rope_dim/2) of a
 * 128-vector by the angle pos * rope_theta^(-2i/rope_dim) and leaves
 * entries >= rope_dim unchanged (NEOX pairing).  The variance is the
 * population variance; eps is added inside the square root.
 *
 * q_lora: [tokens, q_lora_rank] bf16;  x: [tokens, hidden] bf16
 * pos:    [tokens] int32 positions
 * wq_b:   [n_heads*128, q_lora_rank] bf16;  wk: [128, hidden] bf16
 * w_proj: [n_heads, hidden] bf16;  k_norm_w, k_norm_b: [128] f32
 * q_out:  [tokens, n_heads, 128] bf16 output (round to nearest even)
 * k_out:  [tokens, 128] bf16 output;  w_out: [tokens, n_heads] f32 output
 * All device pointers; outputs must not overlap inputs; every pointer
 * 16-byte aligned.  Products run on bf16 MFMA with f32 accumulation; the
 * LayerNorm and rotation in f32 with the angle reduced in f64.
 * Envelope: head_dim == 128, n_heads in {32, 64}, rope_dim a multiple of 16
 * in [16, 128], q_lora_rank and hidden multiples of 64, norm_eps > 0.
 * ------------------------------------------------------------------------ */
typedef struct {
    int32_t tokens, q_lora_rank, hidden, n_heads, head_dim, rope_dim;
    float rope_theta, norm_eps;
} dsa_frontend_dims;

int dsa_indexer_frontend(const dsa_frontend_dims *d, const void *q_lora,
                         const void *x, const int32_t *pos, const void *wq_b,
                         const void *wk, const float *k_norm_w,
                         const float *k_norm_b, const void *w_proj,
                         void *q_out, void *k_out, float *w_out, void *stream);

/* ------------------------------------------------------------------------
 * expand_kv: per-head K and V from the compressed latent ([metrale]
 * expand_kv: NoPE only, so K is exactly the no-rope head width kd).
 *
 * y = latent w_kv_b^T, w_kv_b in torch Linear layout with head-major rows,
 * each head's kd key rows followed by its vd value rows:
 *   K[t,h,:] = y[t, h*(kd+vd) .. h*(kd+vd)+kd)
 *   V[t,h,:] = y[t, h*(kd+vd)+kd .. (h+1)*(kd+vd))
 * latent: [tokens, rank] bf16;  w_kv_b: [n_heads*(kd+vd), rank] bf16
 * k_out:  token t's heads at k_out + t*k_row_stride, head h at +h*kd (bf16)
 * v_out:  likewise with v_row_stride and vd (bf16)
 * bf16 MFMA with f32 accumulation, one rounding to bf16 (nearest even).
 * Envelope: rank a multiple of 64; kd, vd multiples of 8; row strides
 * multiples of 8 elements with k_row_stride >= n_heads*kd and
 * v_row_stride >= n_heads*vd; pointers 16-byte aligned.
 * ------------------------------------------------------------------------ */
typedef struct {
    int32_t tokens, rank, n_heads, kd, vd;
} dsa_expand_dims;

int dsa_expand_kv(const dsa_expand_dims *d, const void *latent,
                  const void *w_kv_b, void *k_out, int64_t k_row_stride,
                  void *v_out, int64_t v_row_stride, void *stream);

/* ------------------------------------------------------------------------
 * IndexShare: which layer's selection a layer attends with.
 *
 * [ik] IndexShare commit message and review comments: GLM-5.2 marks 21 of
 * its 78 layers "full" (layers 0, 1, 2, then every 4th up to 74); a full
 * layer computes its own indexer scores and top-k, and each of the other
 * ("shared") layers reuses the selection of the most recent full layer.
 * The rule: layer il is full iff il <= 1 or il % 4 == 2.
 *
 * Returns the layer whose top-k rows layer `layer` uses -- `layer` itself
 * when it is full -- or -1 when layer < 0.  Host function (no GPU work): a
 * caller runs dsa_index_scores and dsa_topk on full layers only and passes
 * the kept rows to dsa_sparse_attend on the shared ones.
 * ------------------------------------------------------------------------ */
int32_t dsa_index_share_source(int32_t layer);

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
 * shapes run a plain (non-MFMA) kernel.  In the gather kernel the softmax
 * weights enter the value product as a two-term bf16 split (about 16
 * significant bits); the masked-tile kernel re-encodes V once per call as
 * fp16 with a power-of-two scale per (sequence, head) and multiplies fp16
 * weights (11 significant bits); sums are f32.
 * dsa_sparse_attend_workspace_size returns the bytes the kernel chosen for
 * these dims needs (assuming, for kv_heads == 1, the absorbed aliasing
 * v == k with one row stride), or 0 when it needs none or the dims are
 * invalid.  Tensors beyond 2^46 elements and more than 2^31 - 1 (query,
 * head) rows return DSA_ERR_UNSUPPORTED.
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
 * Walsh-Hadamard rotation and the indexer-key cache write.
 *
 * "Another DSA attempt" (ik_llama.cpp PR #2063), the commit message of the
 * decode indexer-K cache: the batch's indexer keys are Walsh-Hadamard
 * rotated and written into the per-layer indexer-key cache at kv_head, from
 * where the indexer scores every past key; the queries get the same
 * rotation, which leaves every score unchanged (orthonormal).  The
 * serving-correctness commit: the rotation is the Sylvester construction,
 * symmetric and orthonormal (H*H = I).
 *
 * Rotation: y = H_d x / sqrt(d) per row of d elements, H_d[i][j] =
 * (-1)^popcount(i & j), computed with f64 sums and one f64 multiplication by
 * 1/sqrt(d), then rounded once to f32 (exact rotation, correctly rounded,
 * whenever the f64 sums are exact -- inputs whose magnitudes within a row
 * span less than about 2^29).
 * ------------------------------------------------------------------------ */

/* out[r,:] = H_d in[r,:] / sqrt(d), stored as f32, or as bf16 rounded to
 * nearest even from the f32 value.  in, out: [rows, d] device, F32 or BF16
 * (in == out is allowed: each row is read whole before it is written).
 * Envelope: d in {32, 64, 128, 256}. */
int dsa_hadamard_rotate(int64_t rows, int32_t d, const void *in, int in_dtype,
                        void *out, int out_dtype, void *stream);

typedef struct {
    int32_t batch, n_new, n_cache, head_dim;
} dsa_cache_dims;

/* Rotates the n_new new key rows of each sequence and writes them into the
 * cache at that sequence's kv_head: row i of sequence b goes to cache row
 * kv_head[b] + i.  FP8_E4M3 cache: per row s = max|y| / 448 (f32 division;
 * 1 for an all-zero row), code = e4m3(y / s) (f32 division, OCP e4m3fn,
 * round to nearest even), and k_scale[b, row] = s -- the keys
 * dsa_index_scores reads as FP8 with k_scale.  BF16 cache: y rounded to
 * nearest even.
 * k_new:   [batch, n_new, head_dim] F32 or BF16
 * kv_head: [batch] int32 device array
 * cache:   [batch, n_cache, head_dim] FP8_E4M3 codes or BF16
 * k_scale: [batch, n_cache] f32 for an FP8 cache, else NULL
 * Rows that would land outside [0, n_cache) are not written (kv_head is a
 * device value, so this cannot be checked before the launch); every other
 * cache row and scale is left as it was.  Envelope: head_dim in
 * {32, 64, 128, 256}. */
int dsa_index_cache_write(const dsa_cache_dims *d, const void *k_new,
                          int k_dtype, const int32_t *kv_head, void *cache,
                          int cache_dtype, float *k_scale, void *stream);

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
