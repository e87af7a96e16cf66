// dsa_internal.hpp -- host-side launch interface between the C ABI layer
// (dsa_abi.cpp) and the kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct IndexArgs {
    int batch, n_q, n_k, n_heads, head_dim;
    float scale;
    bool f32;     // q and k are f32 (else q is bf16)
    bool k_fp8;   // k is OCP e4m3 with per-row scales
    const void *q;
    const void *k;
    const float *k_scale;
    const float *w;
    const int32_t *vis_lo, *vis_hi;
    float *scores;
};
bool index_mfma_supported(int n_heads, int head_dim);
hipError_t launch_index_scores(const IndexArgs &a, hipStream_t st);

struct TopkArgs {
    const float *scores;
    int rows, n_cols;
    int64_t row_stride;
    const int32_t *vis_lo, *vis_hi;
    int k;
    int32_t *out;
    void *workspace;
};
size_t topk_workspace_bytes(int rows, int n_cols, int k);
hipError_t launch_topk(const TopkArgs &a, hipStream_t st);

struct AttendArgs {
    int batch, n_q, n_k, n_heads, kd, vd, kv_heads, n_sel;
    float scale;
    bool f32;
    const void *q, *k, *v;
    int64_t k_row_stride, v_row_stride;
    const int32_t *idx;
    const int32_t *vis_lo, *vis_hi;
    float *out, *lse;
    void *workspace;
};
bool attend_gather_supported(const AttendArgs &a);
bool attend_masked_supported(const AttendArgs &a);
bool attend_plain_supported(const AttendArgs &a);
size_t attend_workspace_bytes(const AttendArgs &a);
size_t attend_masked_workspace_bytes(const AttendArgs &a);
hipError_t launch_attend_masked(const AttendArgs &a, hipStream_t st);
hipError_t launch_attend(const AttendArgs &a, hipStream_t st);

struct RangeArgs {
    int batch, n_q, kpool;
    const int32_t *pad, *q_pos;
    int32_t *lo, *hi;
};
hipError_t launch_visibility_ranges(const RangeArgs &a, hipStream_t st);

struct PoolKeysArgs {
    int batch, seq, kpool, head_dim;
    bool f32;
    const void *k, *gate;
    const int32_t *pad;
    void *pooled;
    int32_t *n_pools;
};
hipError_t launch_pool_keys(const PoolKeysArgs &a, hipStream_t st);

struct PoolSelectArgs {
    int batch, seq, n_q, kpool, select_k, out_width;
    const float *scores;
    const int32_t *pad, *q_pos;
    int32_t *out_tok, *out_pools;
};
constexpr int kPoolSelectMaxPools = 16384;
hipError_t launch_pool_select(const PoolSelectArgs &a, hipStream_t st);

} // namespace dsa
