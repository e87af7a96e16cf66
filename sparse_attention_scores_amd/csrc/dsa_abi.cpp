// dsa_abi.cpp -- the extern "C" entry points of libdsa (see include/dsa.h):
// host-side argument checks, kernel selection and error reporting.  No
// arithmetic of the method happens here; every step runs in the kernels.
#include "dsa.h"
#include "dsa_internal.hpp"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok()
{
    g_last_error.clear();
    return DSA_OK;
}

int hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(DSA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
    return ok();
}

hipStream_t as_stream(void *s)
{
    return reinterpret_cast<hipStream_t>(s);
}

constexpr int64_t kMaxElems = (int64_t)1 << 46;

// true when the product of the sizes exceeds `limit` (no overflow on the way)
bool too_many(std::initializer_list<int64_t> sizes, int64_t limit = kMaxElems)
{
    return dsa::checked_product(sizes, limit) < 0;
}

} // namespace

extern "C" {

const char *dsa_last_error(void)
{
    return g_last_error.c_str();
}

const char *dsa_version(void)
{
    return "libdsa 0.1 gfx950";
}

int dsa_visibility_ranges(int32_t batch, int32_t n_q, const int32_t *pad, const int32_t *q_pos,
                          int32_t kpool, int32_t *vis_lo, int32_t *vis_hi, void *stream)
{
    if (batch < 0 || n_q < 0 || kpool < 0)
        return fail(DSA_ERR_ARG, "dsa_visibility_ranges: negative size");
    if ((int64_t)batch * n_q > 0x7fffffff)
        return fail(DSA_ERR_UNSUPPORTED, "dsa_visibility_ranges: batch*n_q too large");
    if (batch == 0 || n_q == 0)
        return ok();
    if (!pad || !q_pos || !vis_lo || !vis_hi)
        return fail(DSA_ERR_ARG, "dsa_visibility_ranges: null pointer");
    dsa::RangeArgs a{batch, n_q, kpool, pad, q_pos, vis_lo, vis_hi};
    return hip_status(dsa::launch_visibility_ranges(a, as_stream(stream)),
                      "dsa_visibility_ranges");
}

int dsa_index_scores(const dsa_index_dims *d, const void *q, int q_dtype, const void *k,
                     int k_dtype, const float *k_scale, const float *w, const int32_t *vis_lo,
                     const int32_t *vis_hi, float *scores, void *stream)
{
    if (!d)
        return fail(DSA_ERR_ARG, "dsa_index_scores: dims is NULL");
    if (d->batch < 0 || d->n_q < 0 || d->n_k < 0 || d->n_heads <= 0 || d->head_dim <= 0)
        return fail(DSA_ERR_ARG, "dsa_index_scores: bad dims (batch %d n_q %d n_k %d heads %d dim %d)",
                    d->batch, d->n_q, d->n_k, d->n_heads, d->head_dim);
    if (too_many({d->batch, d->n_q, d->n_k}) ||
        too_many({d->batch, d->n_q, d->n_heads, d->head_dim}) ||
        too_many({d->batch, d->n_k, d->head_dim}))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_index_scores: tensors too large");
    if ((int64_t)d->batch * d->n_q * d->n_k == 0)
        return ok();
    if (!q || !k || !w || !vis_lo || !vis_hi || !scores)
        return fail(DSA_ERR_ARG, "dsa_index_scores: null pointer");
    dsa::IndexArgs a{};
    a.batch = d->batch;
    a.n_q = d->n_q;
    a.n_k = d->n_k;
    a.n_heads = d->n_heads;
    a.head_dim = d->head_dim;
    a.scale = d->scale;
    a.q = q;
    a.k = k;
    a.k_scale = k_scale;
    a.w = w;
    a.vis_lo = vis_lo;
    a.vis_hi = vis_hi;
    a.scores = scores;
    if (q_dtype == DSA_F32 && k_dtype == DSA_F32) {
        if (k_scale)
            return fail(DSA_ERR_ARG, "dsa_index_scores: k_scale is only for FP8 keys");
        a.f32 = true;
    } else if (q_dtype == DSA_BF16 && (k_dtype == DSA_BF16 || k_dtype == DSA_FP8_E4M3)) {
        a.k_fp8 = k_dtype == DSA_FP8_E4M3;
        if (a.k_fp8 && !k_scale)
            return fail(DSA_ERR_ARG, "dsa_index_scores: FP8 keys need k_scale");
        if (!a.k_fp8 && k_scale)
            return fail(DSA_ERR_ARG, "dsa_index_scores: k_scale is only for FP8 keys");
        if (!dsa::index_mfma_supported(d->n_heads, d->head_dim))
            return fail(DSA_ERR_UNSUPPORTED,
                        "dsa_index_scores: bf16 path needs n_heads in {32,64} and head_dim in "
                        "{64,128} (got %d, %d)",
                        d->n_heads, d->head_dim);
    } else {
        return fail(DSA_ERR_ARG, "dsa_index_scores: unsupported dtype pair (q %d, k %d)", q_dtype,
                    k_dtype);
    }
    return hip_status(dsa::launch_index_scores(a, as_stream(stream)), "dsa_index_scores");
}

size_t dsa_topk_workspace_size(int32_t rows, int32_t n_cols, int32_t top_k)
{
    if (rows <= 0 || n_cols <= 0 || top_k <= 0)
        return 0;
    return dsa::topk_workspace_bytes(rows, n_cols, top_k);
}

// Argument checks shared by both top-k entry points: DSA_OK to go on, 1 when
// there is nothing to do, else the error.
static int topk_args(const char *fn, const float *scores, int32_t rows, int32_t n_cols,
                     int64_t row_stride, const int32_t *vis_lo, const int32_t *vis_hi,
                     int32_t top_k, int32_t n_sink, const int32_t *out_idx)
{
    if (rows < 0 || n_cols < 0 || n_sink < 0)
        return fail(DSA_ERR_ARG, "%s: negative size", fn);
    if (top_k < 1 || top_k > 2048)
        return fail(top_k < 1 ? DSA_ERR_ARG : DSA_ERR_UNSUPPORTED,
                    "%s: top_k must be in 1..2048 (got %d)", fn, top_k);
    if (rows == 0)
        return 1;
    if (!out_idx || !vis_lo || !vis_hi || (n_cols > 0 && !scores))
        return fail(DSA_ERR_ARG, "%s: null pointer", fn);
    if (row_stride < n_cols)
        return fail(DSA_ERR_ARG, "%s: row_stride %lld < n_cols %d", fn, (long long)row_stride,
                    n_cols);
    if (too_many({rows, row_stride}))
        return fail(DSA_ERR_UNSUPPORTED, "%s: rows x row_stride too large", fn);
    return DSA_OK;
}

int dsa_topk(const float *scores, int32_t rows, int32_t n_cols, int64_t row_stride,
             const int32_t *vis_lo, const int32_t *vis_hi, int32_t top_k, int32_t n_sink,
             int32_t *out_idx, void *workspace, size_t workspace_bytes, void *stream)
{
    const int rc = topk_args("dsa_topk", scores, rows, n_cols, row_stride, vis_lo, vis_hi, top_k,
                             n_sink, out_idx);
    if (rc == 1)
        return ok();
    if (rc != DSA_OK)
        return rc;
    const size_t need = dsa_topk_workspace_size(rows, n_cols, top_k);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(DSA_ERR_WORKSPACE, "dsa_topk: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    dsa::TopkArgs a{scores, rows,  n_cols,  row_stride, vis_lo,
                    vis_hi, top_k, n_sink, out_idx,    workspace};
    return hip_status(dsa::launch_topk(a, as_stream(stream)), "dsa_topk");
}

int dsa_topk_noalloc(const float *scores, int32_t rows, int32_t n_cols, int64_t row_stride,
                     const int32_t *vis_lo, const int32_t *vis_hi, int32_t top_k,
                     int32_t n_sink, int32_t *out_idx, void *stream)
{
    const int rc = topk_args("dsa_topk_noalloc", scores, rows, n_cols, row_stride, vis_lo,
                             vis_hi, top_k, n_sink, out_idx);
    if (rc == 1)
        return ok();
    if (rc != DSA_OK)
        return rc;
    const size_t need = dsa_topk_workspace_size(rows, n_cols, top_k);
    static_assert(DSA_TOPK_NOALLOC_SCRATCH_BYTES == dsa::kTopkScratchBytes,
                  "the header states the scratch size");
    if (need > dsa::kTopkScratchBytes)
        return fail(DSA_ERR_UNSUPPORTED,
                    "dsa_topk_noalloc: these rows need %zu bytes of scratch, more than the "
                    "library's %zu (use dsa_topk with a workspace)",
                    need, dsa::kTopkScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return hip_status(e, "dsa_topk_noalloc");
        if (hipGetStreamDeviceId(as_stream(stream)) != dev)
            return fail(DSA_ERR_ARG, "dsa_topk_noalloc: the stream is not on the current device");
        e = dsa::topk_scratch(&ws);
        if (e != hipSuccess)
            return hip_status(e, "dsa_topk_noalloc: scratch lookup");
    }
    dsa::TopkArgs a{scores, rows, n_cols, row_stride, vis_lo, vis_hi, top_k, n_sink, out_idx, ws};
    return hip_status(dsa::launch_topk(a, as_stream(stream)), "dsa_topk_noalloc");
}

static bool aligned16(const void *p)
{
    return ((uintptr_t)p & 15u) == 0;
}

int dsa_indexer_frontend(const dsa_frontend_dims *d, const void *q_lora, const void *x,
                         const int32_t *pos, const void *wq_b, const void *wk,
                         const float *k_norm_w, const float *k_norm_b, const void *w_proj,
                         void *q_out, void *k_out, float *w_out, void *stream)
{
    if (!d)
        return fail(DSA_ERR_ARG, "dsa_indexer_frontend: dims is NULL");
    if (d->tokens < 0 || d->q_lora_rank <= 0 || d->hidden <= 0 || d->n_heads <= 0 ||
        d->head_dim <= 0 || d->rope_dim < 0)
        return fail(DSA_ERR_ARG, "dsa_indexer_frontend: bad dims");
    if (!(d->norm_eps > 0.f) || !(d->rope_theta > 0.f))
        return fail(DSA_ERR_ARG, "dsa_indexer_frontend: norm_eps and rope_theta must be positive");
    if (d->head_dim != 128 || (d->n_heads != 32 && d->n_heads != 64) || d->rope_dim < 16 ||
        d->rope_dim > 128 || d->rope_dim % 16 != 0 || d->q_lora_rank % 64 != 0 ||
        d->hidden % 64 != 0)
        return fail(DSA_ERR_UNSUPPORTED,
                    "dsa_indexer_frontend: needs head_dim 128, n_heads 32 or 64, rope_dim a "
                    "multiple of 16 up to 128, q_lora_rank and hidden multiples of 64");
    if (too_many({d->tokens, d->q_lora_rank}) || too_many({d->tokens, d->hidden}) ||
        too_many({d->tokens, d->n_heads, d->head_dim}))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_indexer_frontend: tensors too large");
    if (d->tokens == 0)
        return ok();
    if (!q_lora || !x || !pos || !wq_b || !wk || !k_norm_w || !k_norm_b || !w_proj || !q_out ||
        !k_out || !w_out)
        return fail(DSA_ERR_ARG, "dsa_indexer_frontend: null pointer");
    if (!aligned16(q_lora) || !aligned16(x) || !aligned16(wq_b) || !aligned16(wk) ||
        !aligned16(w_proj) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(w_out))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_indexer_frontend: pointers must be 16-byte aligned");
    dsa::FrontendArgs a{};
    a.tokens = d->tokens;
    a.q_lora_rank = d->q_lora_rank;
    a.hidden = d->hidden;
    a.n_heads = d->n_heads;
    a.rope_dim = d->rope_dim;
    a.rope_theta = d->rope_theta;
    a.norm_eps = d->norm_eps;
    a.q_lora = q_lora;
    a.x = x;
    a.pos = pos;
    a.wq_b = wq_b;
    a.wk = wk;
    a.w_proj = w_proj;
    a.k_norm_w = k_norm_w;
    a.k_norm_b = k_norm_b;
    a.q_out = q_out;
    a.k_out = k_out;
    a.w_out = w_out;
    return hip_status(dsa::launch_indexer_frontend(a, as_stream(stream)), "dsa_indexer_frontend");
}

int dsa_expand_kv(const dsa_expand_dims *d, const void *latent, const void *w_kv_b, void *k_out,
                  int64_t k_row_stride, void *v_out, int64_t v_row_stride, void *stream)
{
    if (!d)
        return fail(DSA_ERR_ARG, "dsa_expand_kv: dims is NULL");
    if (d->tokens < 0 || d->rank <= 0 || d->n_heads <= 0 || d->kd <= 0 || d->vd <= 0)
        return fail(DSA_ERR_ARG, "dsa_expand_kv: bad dims");
    if (k_row_stride < (int64_t)d->n_heads * d->kd || v_row_stride < (int64_t)d->n_heads * d->vd)
        return fail(DSA_ERR_ARG, "dsa_expand_kv: row stride smaller than a token's heads");
    if (d->rank % 64 != 0 || d->kd % 8 != 0 || d->vd % 8 != 0 || k_row_stride % 8 != 0 ||
        v_row_stride % 8 != 0)
        return fail(DSA_ERR_UNSUPPORTED,
                    "dsa_expand_kv: rank must be a multiple of 64; kd, vd and the row strides "
                    "multiples of 8");
    if (too_many({d->n_heads, (int64_t)d->kd + d->vd}, 0x7fffffff) ||
        too_many({d->tokens, d->rank}) || too_many({d->tokens, k_row_stride}) ||
        too_many({d->tokens, v_row_stride}))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_expand_kv: tensors too large");
    if (d->tokens == 0)
        return ok();
    if (!latent || !w_kv_b || !k_out || !v_out)
        return fail(DSA_ERR_ARG, "dsa_expand_kv: null pointer");
    if (!aligned16(latent) || !aligned16(w_kv_b) || !aligned16(k_out) || !aligned16(v_out))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_expand_kv: pointers must be 16-byte aligned");
    dsa::ExpandArgs a{d->tokens, d->rank, d->n_heads, d->kd, d->vd, latent, w_kv_b,
                      k_out,     v_out,   k_row_stride, v_row_stride};
    return hip_status(dsa::launch_expand_kv(a, as_stream(stream)), "dsa_expand_kv");
}

int32_t dsa_index_share_source(int32_t layer)
{
    if (layer < 0)
        return -1;
    // full layers: 0, 1 and every layer congruent to 2 mod 4; any other
    // layer il > 2 reuses the full layer just below it, il - ((il - 2) % 4)
    if (layer <= 1 || layer % 4 == 2)
        return layer;
    return layer - (layer - 2) % 4;
}

static int attend_args(const dsa_attn_dims *d, int dtype, dsa::AttendArgs &a)
{
    if (!d)
        return fail(DSA_ERR_ARG, "dsa_sparse_attend: dims is NULL");
    if (d->batch < 0 || d->n_q < 0 || d->n_k < 0 || d->n_sel < 0 || d->n_heads <= 0 ||
        d->kd <= 0 || d->vd <= 0 || d->kv_heads <= 0)
        return fail(DSA_ERR_ARG, "dsa_sparse_attend: bad dims");
    if (d->n_heads % d->kv_heads != 0)
        return fail(DSA_ERR_ARG, "dsa_sparse_attend: n_heads %d not a multiple of kv_heads %d",
                    d->n_heads, d->kv_heads);
    if (dtype != DSA_F32 && dtype != DSA_BF16)
        return fail(DSA_ERR_ARG, "dsa_sparse_attend: dtype must be F32 or BF16");
    if (d->n_k > 524288)
        return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attend: n_k %d > 524288", d->n_k);
    a = dsa::AttendArgs{};
    a.batch = d->batch;
    a.n_q = d->n_q;
    a.n_k = d->n_k;
    a.n_heads = d->n_heads;
    a.kd = d->kd;
    a.vd = d->vd;
    a.kv_heads = d->kv_heads;
    a.n_sel = d->n_sel;
    a.scale = d->scale;
    a.f32 = dtype == DSA_F32;
    return DSA_OK;
}

size_t dsa_sparse_attend_workspace_size(const dsa_attn_dims *d)
{
    // The kernel choice for the size query assumes the absorbed aliasing
    // (v == k, same stride) when kv_heads == 1; that is the only layout whose
    // kernel uses a workspace.
    dsa::AttendArgs a;
    if (attend_args(d, DSA_BF16, a) != DSA_OK)
        return 0;
    static const char token = 0;
    a.k = a.v = &token;
    a.k_row_stride = a.v_row_stride = (int64_t)d->kv_heads * d->kd;
    return dsa::attend_workspace_bytes(a);
}

int dsa_sparse_attend(const dsa_attn_dims *d, int dtype, const void *q, const void *k,
                      int64_t k_row_stride, const void *v, int64_t v_row_stride,
                      const int32_t *idx, const int32_t *vis_lo, const int32_t *vis_hi,
                      float *out, float *lse, void *workspace, size_t workspace_bytes,
                      void *stream)
{
    dsa::AttendArgs a;
    int rc = attend_args(d, dtype, a);
    if (rc != DSA_OK)
        return rc;
    const int64_t rows = (int64_t)d->batch * d->n_q;
    if (too_many({rows, d->n_heads}, 0x7fffffff) || too_many({rows, d->n_sel}) ||
        too_many({rows, d->n_heads, d->kd}) || too_many({rows, d->n_heads, d->vd}))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attend: too many rows");
    if (rows == 0)
        return ok();
    if (!q || !out || (d->n_k > 0 && (!k || !v)) || (d->n_sel > 0 && !idx))
        return fail(DSA_ERR_ARG, "dsa_sparse_attend: null pointer");
    if ((vis_lo == nullptr) != (vis_hi == nullptr))
        return fail(DSA_ERR_ARG, "dsa_sparse_attend: give both vis_lo and vis_hi or neither");
    if (k_row_stride < (int64_t)d->kv_heads * d->kd || v_row_stride < (int64_t)d->kv_heads * d->vd)
        return fail(DSA_ERR_ARG, "dsa_sparse_attend: row stride smaller than a key row");
    if (too_many({d->batch, d->n_k, k_row_stride}) || too_many({d->batch, d->n_k, v_row_stride}))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attend: key or value rows too large");
    a.q = q;
    a.k = k;
    a.v = v;
    a.k_row_stride = k_row_stride;
    a.v_row_stride = v_row_stride;
    a.idx = idx;
    a.vis_lo = vis_lo;
    a.vis_hi = vis_hi;
    a.out = out;
    a.lse = lse;
    if (!dsa::attend_gather_supported(a) && !dsa::attend_masked_supported(a) &&
        !dsa::attend_plain_supported(a))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attend: vd %d too large", d->vd);
    if (dsa::attend_gather_supported(a) || dsa::attend_masked_supported(a)) {
        // the MFMA kernels move q, K, V and out in 16-byte pieces
        auto al16 = [](const void *p) { return ((uintptr_t)p & 15u) == 0; };
        if (!al16(q) || !al16(k) || !al16(v) || !al16(out) || !al16(workspace))
            return fail(DSA_ERR_UNSUPPORTED,
                        "dsa_sparse_attend: q, k, v, out and workspace must be 16-byte aligned");
    }
    const size_t need = dsa::attend_workspace_bytes(a);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(DSA_ERR_WORKSPACE, "dsa_sparse_attend: workspace of %zu bytes needed, %zu given",
                    need, workspace ? workspace_bytes : (size_t)0);
    a.workspace = workspace;
    return hip_status(dsa::launch_attend(a, as_stream(stream)), "dsa_sparse_attend");
}

int dsa_hadamard_rotate(int64_t rows, int32_t d, const void *in, int in_dtype, void *out,
                        int out_dtype, void *stream)
{
    if (rows < 0)
        return fail(DSA_ERR_ARG, "dsa_hadamard_rotate: negative row count");
    if (!dsa::hadamard_supported(d))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_hadamard_rotate: d must be 32, 64, 128 or 256 (got %d)",
                    d);
    if ((in_dtype != DSA_F32 && in_dtype != DSA_BF16) ||
        (out_dtype != DSA_F32 && out_dtype != DSA_BF16))
        return fail(DSA_ERR_ARG, "dsa_hadamard_rotate: dtypes must be F32 or BF16");
    if (too_many({rows, d}))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_hadamard_rotate: too many rows");
    if (rows == 0)
        return ok();
    if (!in || !out)
        return fail(DSA_ERR_ARG, "dsa_hadamard_rotate: null pointer");
    return hip_status(dsa::launch_hadamard_rotate(in, in_dtype == DSA_F32, out, out_dtype == DSA_F32,
                                                  rows, d, as_stream(stream)),
                      "dsa_hadamard_rotate");
}

int dsa_index_cache_write(const dsa_cache_dims *d, const void *k_new, int k_dtype,
                          const int32_t *kv_head, void *cache, int cache_dtype, float *k_scale,
                          void *stream)
{
    if (!d)
        return fail(DSA_ERR_ARG, "dsa_index_cache_write: dims is NULL");
    if (d->batch < 0 || d->n_new < 0 || d->n_cache < 0)
        return fail(DSA_ERR_ARG, "dsa_index_cache_write: negative size");
    if (!dsa::hadamard_supported(d->head_dim))
        return fail(DSA_ERR_UNSUPPORTED,
                    "dsa_index_cache_write: head_dim must be 32, 64, 128 or 256 (got %d)",
                    d->head_dim);
    if (k_dtype != DSA_F32 && k_dtype != DSA_BF16)
        return fail(DSA_ERR_ARG, "dsa_index_cache_write: k_new must be F32 or BF16");
    if (cache_dtype != DSA_FP8_E4M3 && cache_dtype != DSA_BF16)
        return fail(DSA_ERR_ARG, "dsa_index_cache_write: the cache must be FP8_E4M3 or BF16");
    if ((cache_dtype == DSA_FP8_E4M3) != (k_scale != nullptr))
        return fail(DSA_ERR_ARG, "dsa_index_cache_write: k_scale goes with (only) an FP8 cache");
    if (too_many({d->batch, d->n_cache, d->head_dim}) ||
        too_many({d->batch, d->n_new, d->head_dim}))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_index_cache_write: tensors too large");
    if ((int64_t)d->batch * d->n_new == 0)
        return ok();
    if (!k_new || !kv_head || !cache)
        return fail(DSA_ERR_ARG, "dsa_index_cache_write: null pointer");
    dsa::CacheWriteArgs a{d->batch, d->n_new, d->n_cache, d->head_dim, k_new, k_dtype == DSA_F32,
                          kv_head, cache, cache_dtype == DSA_FP8_E4M3, k_scale};
    return hip_status(dsa::launch_index_cache_write(a, as_stream(stream)), "dsa_index_cache_write");
}

static int pool_dims_ok(const dsa_pool_dims *d, const char *fn)
{
    if (!d)
        return fail(DSA_ERR_ARG, "%s: dims is NULL", fn);
    if (d->batch < 0 || d->seq < 0 || d->n_q < 0 || d->kpool <= 0 || d->head_dim < 0)
        return fail(DSA_ERR_ARG, "%s: bad dims", fn);
    return DSA_OK;
}

int dsa_pool_keys(const dsa_pool_dims *d, int dtype, const void *k, const void *gate,
                  const int32_t *pad, void *pooled, int32_t *n_pools, void *stream)
{
    int rc = pool_dims_ok(d, "dsa_pool_keys");
    if (rc != DSA_OK)
        return rc;
    if (d->head_dim <= 0)
        return fail(DSA_ERR_ARG, "dsa_pool_keys: head_dim must be positive");
    if (dtype != DSA_F32 && dtype != DSA_BF16)
        return fail(DSA_ERR_ARG, "dsa_pool_keys: dtype must be F32 or BF16");
    if (too_many({d->batch, d->seq, d->head_dim}))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_pool_keys: tensors too large");
    if (d->batch == 0)
        return ok();
    if (!pad || !n_pools || (d->seq >= d->kpool && (!k || !gate || !pooled)))
        return fail(DSA_ERR_ARG, "dsa_pool_keys: null pointer");
    dsa::PoolKeysArgs a{d->batch, d->seq, d->kpool, d->head_dim, dtype == DSA_F32,
                        k,        gate,   pad,      pooled,      n_pools};
    return hip_status(dsa::launch_pool_keys(a, as_stream(stream)), "dsa_pool_keys");
}

size_t dsa_pool_select_workspace_size(const dsa_pool_dims *d)
{
    (void)d;
    return 0;
}

int dsa_pool_select(const dsa_pool_dims *d, const float *pool_scores, const int32_t *pad,
                    const int32_t *q_pos, int32_t *out_tok, int32_t *out_pools, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    (void)workspace;
    (void)workspace_bytes;
    int rc = pool_dims_ok(d, "dsa_pool_select");
    if (rc != DSA_OK)
        return rc;
    if (d->select_k < 1 || d->select_k > 2048)
        return fail(d->select_k < 1 ? DSA_ERR_ARG : DSA_ERR_UNSUPPORTED,
                    "dsa_pool_select: select_k must be in 1..2048 (got %d)", d->select_k);
    if ((int64_t)d->out_width < (int64_t)d->select_k * d->kpool + d->kpool - 1)
        return fail(DSA_ERR_ARG, "dsa_pool_select: out_width %d < select_k*kpool + kpool - 1",
                    d->out_width);
    if (d->seq / d->kpool > dsa::kPoolSelectMaxPools)
        return fail(DSA_ERR_UNSUPPORTED, "dsa_pool_select: more than %d pools per row",
                    dsa::kPoolSelectMaxPools);
    const int64_t rows = (int64_t)d->batch * d->n_q;
    if (rows > 0x7fffffff || too_many({rows, d->out_width}) ||
        too_many({rows, d->seq / d->kpool}))
        return fail(DSA_ERR_UNSUPPORTED, "dsa_pool_select: too many rows");
    if (rows == 0)
        return ok();
    if (!pad || !q_pos || !out_tok || (d->seq >= d->kpool && !pool_scores))
        return fail(DSA_ERR_ARG, "dsa_pool_select: null pointer");
    dsa::PoolSelectArgs a{d->batch, d->seq,   d->n_q, d->kpool, d->select_k, d->out_width,
                          pool_scores, pad, q_pos, out_tok, out_pools};
    return hip_status(dsa::launch_pool_select(a, as_stream(stream)), "dsa_pool_select");
}

} // extern "C"
