// envelopes.cpp -- host-side kernel selection data: which shapes each kernel
// accepts and how much workspace it needs.  Host code only (no kernels), so
// the C ABI's argument checks and these predicates build and run with any
// host compiler, sanitizers included.  The kernels derive their tile
// constants from the same envelope constants (dsa_internal.hpp).
#include "dsa_internal.hpp"

#include <algorithm>

namespace dsa {

int64_t checked_product(std::initializer_list<int64_t> factors, int64_t limit)
{
    for (int64_t f : factors) {
        if (f < 0)
            return -1;
        if (f == 0)
            return 0;
    }
    int64_t p = 1;
    for (int64_t f : factors) {
        if (p > limit / f)
            return -1;
        p *= f;
    }
    return p;
}

bool index_mfma_supported(int n_heads, int head_dim)
{
    return (n_heads == 32 || n_heads == 64) && (head_dim == 64 || head_dim == 128);
}

size_t topk_workspace_bytes(int rows, int n_cols, int k)
{
    if (rows <= 0 || n_cols <= kTopkChunkKeys || k <= 0)
        return 0;
    // outside the envelope (dsa_topk refuses such k) there is no size
    if (k > kTopkMaxSelect)
        return 0;
    if (topk_long_path(n_cols))
        return (size_t)rows * (size_t)topk_long_layout(n_cols).row_bytes;
    const int64_t n_chunks = ((int64_t)n_cols + kTopkChunkKeys - 1) / kTopkChunkKeys;
    return (size_t)rows * (size_t)n_chunks * (size_t)k * sizeof(uint64_t);
}

bool attend_gather_supported(const AttendArgs &a)
{
    return !a.f32 && a.kv_heads == 1 && a.n_heads == kAbsHeads && a.kd == kAbsKd &&
           a.vd == kAbsVd && a.n_k <= kAbsMaxKeys && a.v == a.k &&
           a.v_row_stride == a.k_row_stride && a.k_row_stride % 8 == 0 &&
           a.k_row_stride >= kAbsKd && a.k_row_stride < (1ll << 30);
}

int attend_gather_splits(const AttendArgs &a)
{
    // blocks = rows x splits; 256 of them fill the CUs
    const int64_t rows = (int64_t)a.batch * a.n_q;
    if (rows <= 0)
        return 1;
    const int by_fill = (int)std::min<int64_t>((256 + rows - 1) / rows, 256);
    const int by_work = std::max(1, std::min(a.n_sel, a.n_k) / 64);
    // the combine kernel keeps one split per lane
    return std::max(1, std::min(std::min(by_fill, by_work), 64));
}

bool attend_plain_supported(const AttendArgs &a)
{
    return a.vd <= kPlainMaxVd;
}

bool attend_masked_supported(const AttendArgs &a)
{
    // V's fp16 copy ([batch, n_k, n_heads, vd]) must stay addressable
    // and the mask ([batch, n_k / 32, q_pad]) as well; the mask builder
    // indexes a group's 32 index rows as one span below 2^24 entries
    return !a.f32 && a.kv_heads == a.n_heads && a.kd == kMaskedKd && a.vd == kMaskedVd &&
           a.n_k > 0 && a.n_q <= (1 << 30) && a.n_sel < (1 << 19) && a.k_row_stride % 8 == 0 &&
           a.v_row_stride % 8 == 0 && (int64_t)a.n_heads * a.vd * 2 < (1ll << 31) &&
           a.k_row_stride < (1ll << 30) &&
           checked_product({a.batch, a.n_k, a.n_heads, a.vd}, (int64_t)1 << 46) >= 0 &&
           checked_product({a.batch, (int64_t)a.n_q + kMaskedQBlock, a.n_k / 32 + 1},
                           (int64_t)1 << 46) >= 0;
}

bool attend_heads_gather_supported(const AttendArgs &a)
{
    // the gathered keys of a sequence (n_q rows x at most n_sel keys) do not
    // exceed what one masked-tile block streams (every key of the range)
    return attend_masked_supported(a) && a.n_sel <= 4096 &&
           (int64_t)a.n_q * std::min(a.n_sel, a.n_k) <= a.n_k;
}

MaskedLayout masked_layout(const AttendArgs &a)
{
    MaskedLayout L{};
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    L.nw = (a.n_k + 31) / 32;
    L.q_pad = (int)(((int64_t)a.n_q + kMaskedQBlock - 1) / kMaskedQBlock * kMaskedQBlock);
    L.nkb = (a.n_k + kMaskedVKeys - 1) / kMaskedVKeys;
    L.mask_bytes = (size_t)a.batch * L.nw * L.q_pad * sizeof(uint32_t);
    L.v16_bytes = (size_t)a.batch * a.n_k * a.n_heads * a.vd * sizeof(uint16_t);
    L.part_bytes = (size_t)a.batch * a.n_heads * L.nkb * sizeof(uint32_t);
    L.vexp_bytes = (size_t)a.batch * a.n_heads * sizeof(float);
    L.v16_off = up(L.mask_bytes);
    L.part_off = L.v16_off + up(L.v16_bytes);
    L.vexp_off = L.part_off + up(L.part_bytes);
    L.total = L.vexp_off + up(L.vexp_bytes);
    return L;
}

size_t attend_masked_workspace_bytes(const AttendArgs &a)
{
    return masked_layout(a).total;
}

size_t attend_workspace_bytes(const AttendArgs &a)
{
    if (attend_heads_gather_supported(a))
        return 0;
    if (attend_masked_supported(a))
        return attend_masked_workspace_bytes(a);
    if (!attend_gather_supported(a))
        return 0;
    const int s = attend_gather_splits(a);
    if (s <= 1)
        return 0;
    const int64_t rows = (int64_t)a.batch * a.n_q;
    // fp16 partials plus one (m, l, e, -) f32 quadruple per (row, split, head)
    return (size_t)rows * s * kAbsHeads * (kAbsVd * sizeof(uint16_t) + 4 * sizeof(float));
}

bool hadamard_supported(int d)
{
    return d == 32 || d == 64 || d == 128 || d == 256;
}

} // namespace dsa
