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
    const int64_t n_scores = (int64_t)d->batch * d->n_q * d->n_k;
    if (n_scores > kMaxElems ||
        (int64_t)d->batch * d->n_q * d->n_heads * d->head_dim > kMaxElems)
        return fail(DSA_ERR_UNSUPPORTED, "dsa_index_scores: tensors too large");
    if (n_scores == 0)
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

int dsa_topk(const float *scores, int32_t rows, int32_t n_cols, int64_t row_stride,
             const int32_t *vis_lo, const int32_t *vis_hi, int32_t top_k, int32_t *out_idx,
             void *workspace, size_t workspace_bytes, void *stream)
{
    if (rows < 0 || n_cols < 0)
        return fail(DSA_ERR_ARG, "dsa_topk: negative size");
    if (top_k < 1 || top_k > 2048)
        return fail(top_k < 1 ? DSA_ERR_ARG : DSA_ERR_UNSUPPORTED,
                    "dsa_topk: top_k must be in 1..2048 (got %d)", top_k);
    if (rows == 0)
        return ok();
    if (!out_idx || !vis_lo || !vis_hi || (n_cols > 0 && !scores))
        return fail(DSA_ERR_ARG, "dsa_topk: null pointer");
    if (row_stride < n_cols)
        return fail(DSA_ERR_ARG, "dsa_topk: row_stride %lld < n_cols %d", (long long)row_stride,
                    n_cols);
    const size_t need = dsa_topk_workspace_size(rows, n_cols, top_k);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(DSA_ERR_WORKSPACE, "dsa_topk: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    dsa::TopkArgs a{scores, rows, n_cols, row_stride, vis_lo, vis_hi, top_k, out_idx, workspace};
    return hip_status(dsa::launch_topk(a, as_stream(stream)), "dsa_topk");
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
    if (rows * d->n_heads > 0x7fffffff || rows * d->n_sel > kMaxElems)
        return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attend: too many rows");
    if (rows == 0)
        return ok();
    if (!q || !out || (d->n_k > 0 && (!k || !v)) || (d->n_sel > 0 && !idx))
        return fail(DSA_ERR_ARG, "dsa_sparse_attend: null pointer");
    if ((vis_lo == nullptr) != (vis_hi == nullptr))
        return fail(DSA_ERR_ARG, "dsa_sparse_attend: give both vis_lo and vis_hi or neither");
    if (k_row_stride < (int64_t)d->kv_heads * d->kd || v_row_stride < (int64_t)d->kv_heads * d->vd)
        return fail(DSA_ERR_ARG, "dsa_sparse_attend: row stride smaller than a key row");
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
    const size_t need = dsa::attend_workspace_bytes(a);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(DSA_ERR_WORKSPACE, "dsa_sparse_attend: workspace of %zu bytes needed, %zu given",
                    need, workspace ? workspace_bytes : (size_t)0);
    a.workspace = workspace;
    return hip_status(dsa::launch_attend(a, as_stream(stream)), "dsa_sparse_attend");
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
    if ((int64_t)d->batch * d->seq * d->head_dim > kMaxElems)
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
    if (rows > 0x7fffffff || rows * d->out_width > kMaxElems)
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
