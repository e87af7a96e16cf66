// attend_set.hpp -- the selected key set of one query row, shared by the
// attention kernels: the row's index entries become a bitmap over the keys
// (set semantics of "Module glm5next_dsa_ref" topk_to_mask: a repeated
// index counts once, INVALID, out-of-range and invisible entries drop),
// and waves read the set back in ascending key order.
#pragma once

#include "dsa_device.hpp"

namespace dsa {

constexpr int kBitmapMaxWords = 16384;  // n_k <= 524288

// Indices base + u*NT + tid (u < U) of a row, -1 past the end.  All U loads
// are issued before any is used.
template <int NT, int U>
__device__ __forceinline__ void load_indices(int (&v)[U], const int32_t *__restrict__ idx_row,
                                             int n_sel, int base)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = base + u * NT + (int)threadIdx.x;
        v[u] = i < n_sel ? idx_row[i] : -1;
    }
}

// Build the selected set of one query row in `bitmap` (words [0, nw)).
// `first` holds the row's first NT*U indices (load_indices at base 0), loaded
// by the caller ahead of other work; the rest are read U per thread at a time.
template <int NT, int U>
__device__ void build_bitmap(uint32_t *bitmap, int nw, const int (&first)[U],
                             const int32_t *__restrict__ idx_row, int n_sel, int lo, int hi)
{
    for (int i = threadIdx.x; i < nw; i += NT)
        bitmap[i] = 0u;
    __syncthreads();
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = first[u];
    for (int base = 0; base < n_sel; base += NT * U) {
        if (base > 0)
            load_indices<NT, U>(v, idx_row, n_sel, base);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = v[u];
            if (j >= lo && j < hi)  // lo >= 0, so INVALID and padding drop here
                atomicOr(&bitmap[j >> 5], 1u << (j & 31));
        }
    }
    __syncthreads();
}

// The bitmap words are read in chunks of 64 (one word per lane, so the
// reads are conflict-free); wave w of NW owns the contiguous chunks
// [c0, c1), so the waves' shares are in key order.
template <int NW>
__device__ __forceinline__ void wave_chunk_range(int nw, int wid, int &c0, int &c1)
{
    const int nch = (nw + 63) >> 6;
    c0 = wid * nch / NW;
    c1 = (wid + 1) * nch / NW;
}

// Number of set bits in this wave's chunks (the same value in every lane).
__device__ __forceinline__ int wave_chunk_count(const uint32_t *bitmap, int nw, int c0, int c1)
{
    const int lane = threadIdx.x & 63;
    int cnt = 0;
    for (int c = c0; c < c1; ++c) {
        const int wd = c * 64 + lane;
        cnt += wd < nw ? __popc(bitmap[wd]) : 0;
    }
    return __builtin_amdgcn_readlane(wave_inclusive_scan(cnt), 63);
}

// Write the set keys of this wave's chunks whose rank (number of set bits
// below them in the whole bitmap) is in [r0, r1) to list[rank - r0]; `run` is
// the number of set bits before chunk c0.
__device__ __forceinline__ void wave_chunk_extract(const uint32_t *bitmap, int nw, int c0, int c1,
                                                   int run, int r0, int r1, int32_t *list)
{
    const int lane = threadIdx.x & 63;
    for (int c = c0; c < c1 && run < r1; ++c) {
        const int wd = c * 64 + lane;
        uint32_t bits = wd < nw ? bitmap[wd] : 0u;
        const int pc = __popc(bits);
        const int incl = wave_inclusive_scan(pc);
        int rank = run + incl - pc;
        if (rank < r1 && rank + pc > r0) {
            while (bits) {
                const int bit = __ffs(bits) - 1;
                bits &= bits - 1;
                if (rank >= r0 && rank < r1)
                    list[rank - r0] = wd * 32 + bit;
                ++rank;
            }
        }
        run += __builtin_amdgcn_readlane(incl, 63);
    }
}

} // namespace dsa
