// dsa_internal.hpp -- host-side launch interface between the C ABI layer
// (dsa_abi.cpp) and the kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <initializer_list>

namespace dsa {

// Kernel envelopes: the shapes the MFMA kernels are built for.  The kernels
// define their tile constants from these, and the host-side predicates and
// workspace sizes (envelopes.cpp) read them, so both agree by construction.
constexpr int kAbsHeads = 64;         // absorbed gather kernel: heads sharing a latent row,
constexpr int kAbsKd = 576;           //   its key width,
constexpr int kAbsVd = 512;           //   its value width (the row's first vd columns)
constexpr int kAbsMaxKeys = 262144;   //   and its per-row set bitmap's reach
constexpr int kPlainMaxVd = 1024;     // plain attend kernel: value columns per thread block
constexpr int kMaskedKd = 192;        // per-head masked attend: key width,
constexpr int kMaskedVd = 256;        //   value width,
constexpr int kMaskedQBlock = 256;    //   queries per block (the mask's q_pad granule)
constexpr int kMaskedVKeys = 256;     //   keys per block of the V re-encoding passes
constexpr int kTopkChunkKeys = 16384; // top-k: rows longer than this go by chunks
constexpr int kTopkMaxSelect = 2048;  // top-k: largest k

// Product of sizes when it is at most `limit`, else -1, computed without an
// intermediate product overflowing; a negative factor gives -1, a zero
// factor 0.
int64_t checked_product(std::initializer_list<int64_t> factors, int64_t limit);

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
    int n_sink;  // attention sinks: the first n_sink visible columns rank first
    int32_t *out;
    void *workspace;
};
size_t topk_workspace_bytes(int rows, int n_cols, int k);
hipError_t launch_topk(const TopkArgs &a, hipStream_t st);

// Rows of kTopkChunkKeys < n_cols <= kTopkLongKeys * kTopkLongMaxParts keys
// go through a shared threshold: one block per kTopkLongKeys columns reports
// kTopkLongPairs (key, count) pairs, the threshold they imply keeps the
// candidates, and a merge ranks those.  Workspace per row: the candidate
// count, the pairs (keys, then counts) and up to `cap` candidates.
constexpr int kTopkLongKeys = 4096;
constexpr int kTopkLongPairs = 24;
constexpr int kTopkLongMaxParts = 64;
constexpr int kTopkLongMaxCand = 16384;
struct TopkLongLayout {
    int parts, cap;
    int64_t pc_off, cand_off, row_bytes;  // byte offsets inside a row's workspace
};
inline bool topk_long_path(int n_cols)
{
    return n_cols > kTopkChunkKeys && n_cols <= kTopkLongKeys * kTopkLongMaxParts;
}
inline TopkLongLayout topk_long_layout(int n_cols)
{
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    TopkLongLayout l;
    l.parts = (n_cols + kTopkLongKeys - 1) / kTopkLongKeys;
    l.cap = (int)std::min<int64_t>(kTopkLongMaxCand, up(n_cols));
    l.pc_off = 64 + (int64_t)l.parts * kTopkLongPairs * 8;
    l.cand_off = up(l.pc_off + (int64_t)l.parts * kTopkLongPairs * 4);
    l.row_bytes = up(l.cand_off + (int64_t)l.cap * 8);
    return l;
}
// the allocation-free top-k's scratch: its size, and its device address on
// the current device (looked up once per device)
constexpr size_t kTopkScratchBytes = (size_t)16 << 20;
hipError_t topk_scratch(void **ptr);

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
// the masked-tile kernel's shapes with few queries per sequence: a per-head
// gather of each row's selected keys instead (no workspace)
bool attend_heads_gather_supported(const AttendArgs &a);
hipError_t launch_attend_heads(const AttendArgs &a, hipStream_t st);
bool attend_plain_supported(const AttendArgs &a);
// blocks per query row of the gather kernel (split-K over the selected keys)
int attend_gather_splits(const AttendArgs &a);
size_t attend_workspace_bytes(const AttendArgs &a);
size_t attend_masked_workspace_bytes(const AttendArgs &a);
// the per-head attend's workspace: the tile-major selection mask, V as
// fp16, per-run partial maxima of |V| and the per-(sequence, head) scale
// exponents, each region 256-byte aligned
struct MaskedLayout {
    int nw, q_pad, nkb;  // key words (tiles), padded query count, V-pass key runs
    size_t mask_bytes, v16_bytes, part_bytes, vexp_bytes;
    size_t v16_off, part_off, vexp_off, total;
};
MaskedLayout masked_layout(const AttendArgs &a);
hipError_t launch_attend_masked(const AttendArgs &a, hipStream_t st);
hipError_t launch_attend(const AttendArgs &a, hipStream_t st);

struct CacheWriteArgs {
    int batch, n_new, n_cache, head_dim;
    const void *k_new;
    bool k_f32;
    const int32_t *kv_head;
    void *cache;
    bool fp8;
    float *scales;
};
bool hadamard_supported(int d);
hipError_t launch_hadamard_rotate(const void *x, bool x_f32, void *out, bool out_f32, int64_t rows,
                                  int d, hipStream_t st);
hipError_t launch_index_cache_write(const CacheWriteArgs &a, hipStream_t st);

// the indexer front-end: q = rope(q_lora wq_b^T) per head of 128,
// k = rope(LayerNorm(x wk^T)), w = x w_proj^T
struct FrontendArgs {
    int tokens, q_lora_rank, hidden, n_heads, rope_dim;
    float rope_theta, norm_eps;
    const void *q_lora, *x;
    const int32_t *pos;
    const void *wq_b, *wk, *w_proj;
    const float *k_norm_w, *k_norm_b;
    void *q_out, *k_out;
    float *w_out;
};
hipError_t launch_indexer_frontend(const FrontendArgs &a, hipStream_t st);

// expand_kv: per-head K and V from the latent
struct ExpandArgs {
    int tokens, rank, n_heads, kd, vd;
    const void *latent, *w_kv_b;
    void *k_out, *v_out;
    int64_t k_row_stride, v_row_stride;
};
hipError_t launch_expand_kv(const ExpandArgs &a, hipStream_t st);

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
// Blocks per row of the segmented top-k kernels: enough for about 256 blocks
// in all, at most max_parts, segments of at least 64 ranks; 1 = one block
// per row.
int topk_seg_parts(int rows, int k, int max_parts);

} // namespace dsa
