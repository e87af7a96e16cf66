// topk.hip -- per-row top-k on gfx950, exact.
//
// Rank order: higher score first, then smaller column index ("Module
// glm5next_dsa_ref", topk_pools); at most min(k, n_visible) entries, the
// rest INVALID (ik_llama.cpp PR #2063, batch-local indexer commit:
// top_k(min(top_k, n_tokens))).
//
// A key's place in that order is its composite key
//     (order_key(score) << 32) | (0xffffffff - column)
// (larger = better rank, -0 folded onto +0); all keys of a row are
// distinct, so "the k largest keys" is one well-defined set.
//
// Paths, by shape (every one exact):
//  * up to 16384 keys: value buckets place each winner without sorting the
//    row (topk_seg_kernel), one block per row, or several blocks per row each
//    writing one segment of the ranks when there are few rows; a block whose
//    ranks fall into a crowded bucket sorts the row instead (32-bit radix
//    select, compaction, bucket sort: topk_sort_cached);
//  * longer rows: each 16384-key chunk keeps its own top k (the global top-k
//    is a subset of the union of the chunk top-ks, the order being total),
//    then a merge selects and sorts among those candidates -- segmented over
//    several blocks per row when the candidates fit one block's cache.
#include "dsa_internal.hpp"
#include <algorithm>
#include <mutex>
#include "topk_device.hpp"

namespace dsa {

// First column a row ranks by score: the start of its visible range [lo, hi)
// moved past the `skip` attention-sink columns that lead it (clamped to hi;
// no overflow for any lo).
__device__ __forceinline__ int first_ranked(int lo, int hi, int skip)
{
    lo = max(lo, 0);
    return lo + min(skip, max(hi - lo, 0));
}

// Attention sinks: the first n_s columns of each row's visible range take
// ranks 0 .. n_s - 1 in column order (INVALID past the range's end).
__global__ __launch_bounds__(256) void topk_sink_prefix_kernel(const int32_t *__restrict__ vlo,
                                                               const int32_t *__restrict__ vhi,
                                                               int n_cols, int rows, int n_s,
                                                               int k, int32_t *__restrict__ out)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)rows * n_s)
        return;
    const int row = (int)(e / n_s), j = (int)(e % n_s);
    const int hi = min(vhi[row], n_cols);
    const int lo = max(vlo[row], 0);
    out[(int64_t)row * k + j] = j < hi - lo ? lo + j : -1;
}

// Segmented top-k: `parts` blocks share a row, block `seg` writes output
// positions [seg*seg_len, seg*seg_len + seg_len) of it, so a few rows still
// fill the chip; each places its ranks with value buckets (seg_rank_row).
template <int NT, int CAP>
__global__ __launch_bounds__(NT) void topk_seg_kernel(const float *__restrict__ scores,
                                                      int n_cols, int64_t row_stride,
                                                      const int32_t *__restrict__ vlo,
                                                      const int32_t *__restrict__ vhi, int k,
                                                      int32_t *__restrict__ out,
                                                      int64_t out_stride, int lo_skip, int parts,
                                                      int seg_len)
{
    __shared__ Topk32Smem<NT, CAP> sm;
    const int tid = threadIdx.x;
    const int row = blockIdx.x / parts;
    const int seg = blockIdx.x - row * parts;
    const int hi = min(vhi[row], n_cols);
    const int lo = first_ranked(vlo[row], hi, lo_skip);
    const int n = max(hi - lo, 0);
    const int m = min(k, n);
    int32_t *o = out + (int64_t)row * out_stride;
    const int p0 = seg * seg_len, p1 = min(p0 + seg_len, k);
    const int s0 = p0, s1 = min(p1, m);  // ranks this block writes
    if (s0 < s1)
        seg_rank_row(sm, scores + (int64_t)row * row_stride + lo, lo, n, k, s0, s1,
                     [&](int r, int col) { o[r] = col; });
    for (int i = max(p0, m) + tid; i < p1; i += NT)
        o[i] = -1;
}

constexpr int kMergeCacheKeys = 16384;
template <int NT, bool CACHE>
using MergeSmem = TopkSmem<NT, CACHE ? 2 * kMergeCacheKeys : 1>;

// Sorted top-k of the n candidates cand[0 .. n): m = min(k, real candidates)
// and, on return, v[b] of thread t holds the key of rank t*EPT + b.
template <int NT, int EPT, bool CACHE>
__device__ void merge_sorted(MergeSmem<NT, CACHE> &sm, const uint64_t *__restrict__ cand, int n,
                             int k, uint64_t (&v)[EPT], int &m)
{
    const int tid = threadIdx.x;
    // CACHE: the 64-bit candidates live in sm.ord (two words each)
    uint64_t *cache = reinterpret_cast<uint64_t *>(sm.ord);
    // count the real candidates (and fill the cache)
    if (tid == 0)
        sm.count = 0;
    __syncthreads();
    int local = 0;
    if (CACHE) {
        constexpr int U = 8;
        for (int base = 0; base < n; base += NT * U) {
            uint64_t x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * NT + tid;
                x[u] = i < n ? cand[i] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * NT + tid;
                if (i < n) {
                    cache[i] = x[u];
                    local += x[u] != 0ull;
                }
            }
        }
    } else {
        for (int i = tid; i < n; i += NT)
            local += cand[i] != 0ull;
    }
    atomicAdd(&sm.count, local);
    __syncthreads();
    const int real = sm.count;
    __syncthreads();
    auto key_at = [&](int i) -> uint64_t { return CACHE ? cache[i] : cand[i]; };
    if (real > k) {
        radix_select(sm, n, k, key_at);
        m = k;
    } else {
        if (tid == 0)
            sm.count = 0;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
            const uint64_t key = key_at(i);
            if (key != 0ull) {
                const int pos = atomicAdd(&sm.count, 1);
                sm.sel[pos] = key;
            }
        }
        __syncthreads();
        m = real;
    }
    bitonic_sort_regs<NT, EPT>(sm, m, v);
}

template <int NT, int EPT, bool CACHE>
__global__ __launch_bounds__(NT) void topk_merge_kernel(const uint64_t *__restrict__ ws,
                                                        int n_chunks, int k,
                                                        int32_t *__restrict__ out,
                                                        int64_t out_stride)
{
    __shared__ MergeSmem<NT, CACHE> sm;
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    uint64_t v[EPT];
    int m;
    merge_sorted<NT, EPT, CACHE>(sm, ws + (int64_t)row * n_chunks * k, n_chunks * k, k, v, m);
    int32_t *o = out + (int64_t)row * out_stride;
#pragma unroll
    for (int b = 0; b < EPT; ++b) {
        const int i = tid * EPT + b;
        if (i < k)
            o[i] = i < m ? (int32_t)(0xffffffffu - (uint32_t)v[b]) : -1;
    }
}

// First launch of the long-row path: chunk c of the row keeps its exact top
// min(k, n_c) keys, as composite keys in any order, in ws[row][c][0 .. k),
// zero-padded.  The chunk's keys are counted into value buckets; every key
// of a bucket above the one that holds rank k-1 wins outright, and the
// members of that boundary bucket are ranked among themselves by composite
// key for the remaining places.  Without a finite value range, or with a
// crowded boundary bucket, the 32-bit select and compaction decide instead.
template <int NT, int CAP>
__global__ __launch_bounds__(NT) void topk_chunk_kernel(const float *__restrict__ scores,
                                                        int n_cols, int64_t row_stride,
                                                        const int32_t *__restrict__ vlo,
                                                        const int32_t *__restrict__ vhi, int k,
                                                        uint64_t *__restrict__ ws, int n_chunks,
                                                        int lo_skip)
{
    using S = Topk32Smem<NT, CAP>;
    constexpr int NB = S::NB, NW = S::NW, PB = NB / NT, R = CAP / NT;
    static_assert(PB >= 1 && NB % NT == 0, "every thread owns whole buckets");
    __shared__ S sm;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const uint64_t lt = (1ull << lane) - 1ull;
    const int row = blockIdx.x / n_chunks;
    const int chunk = blockIdx.x - row * n_chunks;
    const int c0 = chunk * CAP;
    const int row_hi = min(vhi[row], n_cols);
    const int lo = max(first_ranked(vlo[row], row_hi, lo_skip), c0);
    const int hi = min(row_hi, c0 + CAP);
    uint32_t omin, omax;
    const int n = load_row32(sm, scores + (int64_t)row * row_stride, lo, hi, omin, omax);
    uint64_t *o = ws + ((int64_t)row * n_chunks + chunk) * k;
    const int m = min(k, n);
    for (int i = m + tid; i < k; i += NT)
        o[i] = 0ull;
    if (n <= k) {
        for (int i = tid; i < n; i += NT)
            o[i] = compose_key(sm.a.ord[i], (uint32_t)(lo + i));
        return;
    }
    ValueBuckets bucket;
    if (omin != omax && bucket.init(omin, omax, NB)) {
        for (int i = tid; i < NB; i += NT)
            sm.bk.fill[i] = 0u;
        if (tid == 0) {
            sm.fill = 0;
            sm.bincnt = 0;
        }
        __syncthreads();
        for (int i = tid; i < n; i += NT)
            atomicAdd(&sm.bk.fill[bucket(sm.a.ord[i])], 1u);
        __syncthreads();
        // the bucket holding rank k-1, the ranks above it and its size
        uint32_t v[PB];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            v[j] = sm.bk.fill[tid * PB + j];
            sum += (int)v[j];
        }
        const int incl = wave_inclusive_scan(sum);
        if (lane == 63)
            sm.tab[0][wid] = incl;
        __syncthreads();
        int run = incl - sum;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            run += w < wid ? sm.tab[0][w] : 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int c = (int)v[j];
            if (run <= k - 1 && k - 1 < run + c) {
                sm.bin = tid * PB + j;
                sm.above = run;
                sm.red[0][0][0] = c;
            }
            run += c;
        }
        __syncthreads();
        const int bb = sm.bin, above = sm.above, cnt_b = sm.red[0][0][0];
        if (cnt_b <= kSegMaxBucket) {
            uint64_t *ck = reinterpret_cast<uint64_t *>(&sm.word[1][0]);
            const int rounds = (n + NT - 1) / NT;
            for (int r = 0; r < rounds; ++r) {  // uniform
                const int i = r * NT + tid;
                const uint32_t ord = i < n ? sm.a.ord[i] : 0u;
                const int b = i < n ? bucket(ord) : NB;
                const uint64_t win = __ballot(b < bb);
                int base = 0;
                if (lane == 0 && win)
                    base = atomicAdd(&sm.fill, __popcll(win));
                base = __builtin_amdgcn_readfirstlane(base);
                if (b < bb)
                    o[base + __popcll(win & lt)] = compose_key(ord, (uint32_t)(lo + i));
                else if (b == bb)
                    ck[atomicAdd(&sm.bincnt, 1)] = compose_key(ord, (uint32_t)(lo + i));
            }
            __syncthreads();
            for (int j = tid; j < cnt_b; j += NT) {
                const uint64_t key = ck[j];
                int r = 0;
                for (int x = 0; x < cnt_b; ++x)
                    r += ck[x] > key;
                if (above + r < k)
                    o[above + r] = key;
            }
            return;
        }
        __syncthreads();  // the bucket arrays are reused below
    }
    uint32_t prefix, mask;
    int need, cand;
    select32(sm, n, k, omin, omax, prefix, mask, need, cand);
    uint32_t wmin, wmax;
    const int mm = cand == need ? compact32_any(sm, n, lo, prefix, mask, wmin, wmax)
                                : compact32(sm, n, lo, prefix, mask, need, cand, wmin, wmax);
    for (int i = tid; i < mm; i += NT)
        o[i] = compose_key(sm.word[0][i], sm.wcol[0][i]);
    (void)R;
}

// LDS of the segmented merge: the candidates' order keys and buckets, or
// the full merge's cache.
template <int NT>
union MergeSegSmem {
    Topk32Smem<NT, kMergeCacheKeys> a;
    MergeSmem<NT, true> b;
};

// Segmented merge of one row's candidates cand[0 .. n) (composite keys,
// zero keys padding; n at most kMergeCacheKeys): the block writes output
// positions [seg*seg_len, seg*seg_len + seg_len) of o, as in
// topk_seg_kernel: value buckets over the real candidates, the buckets that
// hold the block's ranks collected and ranked inside by composite key.
// Crowded buckets or a non-finite range fall back to the full merge of the
// row.
template <int NT>
__device__ void merge_seg_row(MergeSegSmem<NT> &u, const uint64_t *__restrict__ cand, int n,
                              int k, int32_t *__restrict__ o, int seg, int seg_len)
{
    using S = Topk32Smem<NT, kMergeCacheKeys>;
    constexpr int NB = S::NB, NW = S::NW, PB = NB / NT;
    S &sm = u.a;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    // order keys of the candidates (0 = padding: a real key's order part is
    // at least 0x007fffff), their count and range
    int nv = 0;
    uint32_t mn = ~0u, mx = 0u;
    {
        constexpr int U8 = 8;
        for (int base = 0; base < n; base += NT * U8) {
            uint64_t x[U8];
#pragma unroll
            for (int u8 = 0; u8 < U8; ++u8) {
                const int i = base + u8 * NT + tid;
                x[u8] = i < n ? cand[i] : 0ull;
            }
#pragma unroll
            for (int u8 = 0; u8 < U8; ++u8) {
                const int i = base + u8 * NT + tid;
                if (i < n) {
                    const uint32_t ord = (uint32_t)(x[u8] >> 32);
                    sm.a.ord[i] = ord;
                    if (ord) {
                        ++nv;
                        mn = min(mn, ord);
                        mx = max(mx, ord);
                    }
                }
            }
        }
    }
    nv = wave_sum_int(nv);
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        sm.mm[0][wid] = mn;
        sm.mm[1][wid] = mx;
        sm.red[0][0][wid] = nv;
    }
    __syncthreads();
    uint32_t omin = ~0u, omax = 0u;
    int n_valid = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        omin = min(omin, sm.mm[0][w]);
        omax = max(omax, sm.mm[1][w]);
        n_valid += sm.red[0][0][w];
    }
    __syncthreads();
    const int m = min(k, n_valid);
    const int p0 = seg * seg_len, p1 = min(p0 + seg_len, k);
    for (int i = max(p0, m) + tid; i < p1; i += NT)
        o[i] = -1;
    const int s0 = p0, s1 = min(p1, m);  // ranks this block writes
    if (s0 >= s1)
        return;
    ValueBuckets bucket;
    if (omin != omax && bucket.init(omin, omax, NB)) {
        for (int i = tid; i < NB; i += NT)
            sm.bk.fill[i] = 0u;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
            const uint32_t ord = sm.a.ord[i];
            if (ord)
                atomicAdd(&sm.bk.fill[bucket(ord)], 1u);
        }
        __syncthreads();
        uint32_t v[PB];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            v[j] = sm.bk.fill[tid * PB + j];
            sum += (int)v[j];
        }
        const int incl = wave_inclusive_scan(sum);
        if (lane == 63)
            sm.tab[0][wid] = incl;
        __syncthreads();
        int run = incl - sum;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            run += w < wid ? sm.tab[0][w] : 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int b = tid * PB + j, c = (int)v[j];
            sm.bk.off[b] = (uint32_t)run;
            if (run <= s0 && s0 < run + c)
                sm.tab[1][0] = b;
            if (run <= s1 - 1 && s1 - 1 < run + c)
                sm.tab[1][1] = b;
            run += c;
        }
        __syncthreads();
        const int bf = sm.tab[1][0], bl = sm.tab[1][1];
        const int base = (int)sm.bk.off[bf];
        int crowd = 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int b = tid * PB + j;
            if (b >= bf && b <= bl) {
                crowd = max(crowd, (int)v[j]);
                sm.bk.fill[b] = sm.bk.off[b] - (uint32_t)base;
            }
        }
        crowd = (int)wave_max_u32((uint32_t)crowd);
        if (lane == 0)
            sm.red[1][0][wid] = crowd;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w)
            crowd = max(crowd, sm.red[1][0][w]);
        const int total = (bl + 1 < NB ? (int)sm.bk.off[bl + 1] : n_valid) - base;
        if (crowd <= kSegMaxBucket && total <= kTopkMaxK) {
            uint64_t *ck = reinterpret_cast<uint64_t *>(&sm.word[1][0]);
            for (int i = tid; i < n; i += NT) {
                const uint32_t ord = sm.a.ord[i];
                if (ord) {
                    const int b = bucket(ord);
                    if (b >= bf && b <= bl)
                        ck[atomicAdd(&sm.bk.fill[b], 1u)] = cand[i];
                }
            }
            __syncthreads();
            for (int j = tid; j < total; j += NT) {
                const uint64_t key = ck[j];
                const int b = bucket((uint32_t)(key >> 32));
                const int b0 = (int)sm.bk.off[b] - base, b1 = (int)sm.bk.fill[b];
                int r = (int)sm.bk.off[b];
                for (int x = b0; x < b1; ++x)
                    r += ck[x] > key;
                if (r >= s0 && r < s1)
                    o[r] = (int32_t)(0xffffffffu - (uint32_t)key);
            }
            return;
        }
    }
    __syncthreads();  // the segment path's LDS is reused by the full merge
    constexpr int EPT = kTopkMaxK / NT;
    uint64_t v[EPT];
    int mm;
    merge_sorted<NT, EPT, true>(u.b, cand, n, k, v, mm);
#pragma unroll
    for (int b = 0; b < EPT; ++b) {
        const int i = tid * EPT + b;
        if (i >= s0 && i < s1)
            o[i] = (int32_t)(0xffffffffu - (uint32_t)v[b]);
    }
}

// Second launch of the chunked long-row path for few rows: `parts` blocks
// share a row's chunk winners ws[row][0 .. n_chunks * k).
template <int NT>
__global__ __launch_bounds__(NT) void topk_merge_seg_kernel(const uint64_t *__restrict__ ws,
                                                            int n_chunks, int k,
                                                            int32_t *__restrict__ out,
                                                            int64_t out_stride, int parts,
                                                            int seg_len)
{
    __shared__ MergeSegSmem<NT> u;
    const int row = blockIdx.x / parts;
    const int seg = blockIdx.x - row * parts;
    merge_seg_row<NT>(u, ws + (int64_t)row * n_chunks * k, n_chunks * k, k,
                      out + (int64_t)row * out_stride, seg, seg_len);
}

// ------------------------------------------------------ long rows, shared threshold
//
// A row of n keys is cut into blocks of kTopkLongKeys columns.  Block p
// reports pairs (v, c): c is the exact number of its keys whose composite key
// is at least v.  For a threshold t, any pair of block p with v >= t
// guarantees c of its keys at or above t, so
//     G(t) = sum over blocks of the count of the block's last pair with v >= t
// is a lower bound on the row's keys at or above t.  The largest pair value
// t with G(t) >= k is therefore at or below the k-th largest key: every
// winner is at or above it, and the keys at or above it (typically a little
// over k) are the only candidates the merge has to rank.  The pairs sit at
// ranks 0, 1, 2, 3, 5, 7, 10, 15, ... (about sqrt 2 apart) up to
// min(k, n_p) - 1, so the candidates overshoot k by a bounded factor when
// the pairs are exact ranks; a value bucket crowded by outliers makes them
// coarser, and when the candidates exceed the workspace the merge ranks the
// raw row instead (exact, one block, slow).

__device__ __forceinline__ int long_target_rank(int j)
{
    // round(sqrt(2)^(j+1)) - 1, strictly increasing from 0
    constexpr int R[kTopkLongPairs] = {0,   1,   2,   3,   5,    7,    10,   15,
                                       22,  31,  44,  63,  90,   127,  180,  255,
                                       361, 511, 723, 1023, 1447, 2047, 2895, 4095};
    return R[j];
}

// The block's scores at columns c0 + u*NT + t, loaded before the visible
// range is known (it only masks them afterwards, so the loads need not wait
// for it); columns past the row read its last column instead, so every load
// is unconditional and in bounds.
template <int NT>
__device__ __forceinline__ void long_load_block(float (&sv)[kTopkLongKeys / NT],
                                                const float *__restrict__ srow, int c0,
                                                int n_cols)
{
#pragma unroll
    for (int u = 0; u < kTopkLongKeys / NT; ++u)
        sv[u] = srow[min(c0 + u * NT + (int)threadIdx.x, n_cols - 1)];
}

// First launch: the pairs of block p of every row.  Thread t holds columns
// c0 + u*NT + t of the block.  The keys are counted into value buckets
// (linear in the score over the block's [min, max]); each target rank's pair
// is (smallest composite key of the bucket that holds it, keys in that
// bucket and in better ones).  When a target lands in a crowded bucket (an
// outlier stretches the value range, or the range is not finite) the keys
// are counted again into buckets linear in the order key, which follows the
// exponent, and each target keeps the smaller of its two buckets.  Also
// clears the row's candidate count.
template <int NT>
__global__ __launch_bounds__(NT) void topk_long_pairs_kernel(
    const float *__restrict__ scores, int n_cols, int64_t row_stride,
    const int32_t *__restrict__ vlo, const int32_t *__restrict__ vhi, int k, int lo_skip,
    unsigned char *__restrict__ ws, int parts, int64_t pc_off, int64_t row_bytes)
{
    constexpr int KPT = kTopkLongKeys / NT, NB = 1024, PB = NB / NT, NW = NT / 64;
    constexpr int NP = kTopkLongPairs;
    static_assert(KPT * NT == kTopkLongKeys && PB * NT == NB, "whole keys and buckets per thread");
    static_assert(NP <= 64, "one lane per target");
    __shared__ uint32_t hist[2][NB + 1];  // bucket NB counts the invisible keys
    __shared__ int8_t first_target[2][NB + 1];
    __shared__ unsigned long long mink[NP];
    __shared__ int tbin[2][NP], tcnt[2][NP], tsize[2][NP];
    __shared__ uint32_t red[2][NW];
    __shared__ int tab[NW];
    __shared__ int s_crowded;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int row = blockIdx.x / parts, p = blockIdx.x - row * parts;
    unsigned char *w = ws + (int64_t)row * row_bytes;
    uint64_t *pv = reinterpret_cast<uint64_t *>(w + 64) + p * NP;
    uint32_t *pc = reinterpret_cast<uint32_t *>(w + pc_off) + p * NP;
    if (p == 0 && tid == 0)
        *reinterpret_cast<int *>(w) = 0;  // the candidate count, summed by the next launch
    const int c0 = p * kTopkLongKeys;
    float sv[KPT];
    long_load_block<NT>(sv, scores + (int64_t)row * row_stride, c0, n_cols);
    const int row_hi = min(vhi[row], n_cols);
    const int lo = max(first_ranked(vlo[row], row_hi, lo_skip), c0);
    const int hi = min(row_hi, c0 + kTopkLongKeys);
    const int m = min(k, max(hi - lo, 0));  // the pairs cover ranks below m
    uint32_t ord[KPT];
    uint32_t valid = 0u, mn = ~0u, mx = 0u;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int col = c0 + u * NT + tid;
        ord[u] = score_order_key(sv[u]);
        if (col >= lo && col < hi) {
            valid |= 1u << u;
            mn = min(mn, ord[u]);
            mx = max(mx, ord[u]);
        }
    }
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        red[0][wid] = mn;
        red[1][wid] = mx;
    }
    for (int i = tid; i <= NB; i += NT) {
        hist[0][i] = hist[1][i] = 0u;
        first_target[0][i] = first_target[1][i] = -1;
    }
    if (tid < NP)
        mink[tid] = ~0ull;
    if (tid == 0)
        s_crowded = 0;
    __syncthreads();
    uint32_t omin = ~0u, omax = 0u;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        omin = min(omin, red[0][i]);
        omax = max(omax, red[1][i]);
    }
    // target j covers rank min(R_j, m - 1); the pairs after the first that
    // reaches m - 1 are empty (count 0)
    auto past_last = [&](int j) { return j > 0 && long_target_rank(j - 1) >= m - 1; };
    if (m == 0 || omin == omax) {
        // nothing visible, or all keys equal: rank r is column lo + r
        if (tid < NP) {
            const int r = min(long_target_rank(tid), m - 1);
            const bool use = m > 0 && !past_last(tid);
            pv[tid] = use ? compose_key(omin, (uint32_t)(lo + r)) : 0ull;
            pc[tid] = use ? (uint32_t)(r + 1) : 0u;
        }
        return;
    }
    ValueBuckets vb;
    const bool by_value = vb.init(omin, omax, NB);
    // order-key buckets: floor((o - omin) * mul / 2^32), clamped below NB,
    // with mul about NB * 2^32 / span (any mul gives a monotone map; the
    // product stays below 2^43, no 64-bit division)
    const double span = (double)(omax - omin) + 1.0;
    const uint64_t mul = (uint64_t)((double)((uint64_t)NB << 32) / span);
    auto ob = [&](uint32_t o) {
        return NB - 1 - min((int)(((uint64_t)(o - omin) * mul) >> 32), NB - 1);
    };
    // Count scheme sc's buckets b[] and locate each target: thread t owns
    // buckets t*PB .. t*PB + PB - 1 (bucket 0 the best), the keys in better
    // buckets come from a block scan.
    auto count_and_locate = [&](int sc, const int (&b)[KPT]) {
#pragma unroll
        for (int u = 0; u < KPT; ++u)
            atomicAdd(&hist[sc][b[u]], 1u);  // invisible keys carry bucket NB
        __syncthreads();
        uint32_t cv[PB];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            cv[j] = hist[sc][tid * PB + j];
            sum += (int)cv[j];
        }
        const int incl = wave_inclusive_scan(sum);
        if (lane == 63)
            tab[wid] = incl;
        __syncthreads();
        int run0 = incl - sum;
#pragma unroll
        for (int i = 0; i < NW; ++i)
            run0 += i < wid ? tab[i] : 0;
#pragma unroll
        for (int t = 0; t < NP; ++t) {
            const int r = min(long_target_rank(t), m - 1);
            if (run0 <= r && r < run0 + sum) {
                int run = run0;
#pragma unroll
                for (int j = 0; j < PB; ++j) {
                    const int c = (int)cv[j];
                    if (run <= r && r < run + c) {
                        tbin[sc][t] = tid * PB + j;
                        tcnt[sc][t] = run + c;
                        tsize[sc][t] = c;
                    }
                    run += c;
                }
            }
        }
        __syncthreads();
    };
    int bv[KPT], bo[KPT];
    const int first = by_value ? 0 : 1;
#pragma unroll
    for (int u = 0; u < KPT; ++u)
        bv[u] = (valid >> u & 1u) ? (by_value ? vb(ord[u]) : ob(ord[u])) : NB;
    count_and_locate(first, bv);
    // crowded: a target's bucket holds more than twice the keys up to its rank
    if (tid < NP && !past_last(tid)) {
        const int r = min(long_target_rank(tid), m - 1);
        if (tsize[first][tid] > 2 * (r + 1) + 8)
            s_crowded = 1;
    }
    __syncthreads();
    const bool both = by_value && s_crowded;
    if (both) {
#pragma unroll
        for (int u = 0; u < KPT; ++u)
            bo[u] = (valid >> u & 1u) ? ob(ord[u]) : NB;
        count_and_locate(1, bo);
    }
    // each target takes the smaller of its buckets; each chosen bucket is
    // named by its lowest target
    if (tid < NP) {
        const int t = tid;
        const int sc = (both && tsize[1][t] < tsize[0][t]) ? 1 : first;
        bool lowest = true;
        if (!both) {
            // one scheme: a target's bucket is never better than the previous
            // target's, so the targets of a bucket are consecutive
            lowest = t == 0 || tbin[sc][t - 1] != tbin[sc][t];
        } else {
            for (int u = 0; u < t; ++u) {
                const int su = tsize[1][u] < tsize[0][u] ? 1 : 0;
                lowest = lowest && !(su == sc && tbin[su][u] == tbin[sc][t]);
            }
        }
        if (lowest)
            first_target[sc][tbin[sc][t]] = (int8_t)t;
    }
    __syncthreads();
    // the smallest composite key of each chosen bucket
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        // invisible keys sit in bucket NB, which no target names
        const unsigned long long key = compose_key(ord[u], (uint32_t)(c0 + u * NT + tid));
        const int t0 = first_target[first][bv[u]];
        if (t0 >= 0)
            atomicMin(&mink[t0], key);
        if (both) {
            const int t1 = first_target[1][bo[u]];
            if (t1 >= 0)
                atomicMin(&mink[t1], key);
        }
    }
    __syncthreads();
    if (tid < NP) {
        const bool use = !past_last(tid);
        const int sc = (both && tsize[1][tid] < tsize[0][tid]) ? 1 : first;
        pv[tid] = use ? (uint64_t)mink[first_target[sc][tbin[sc][tid]]] : 0ull;
        pc[tid] = use ? (uint32_t)tcnt[sc][tid] : 0u;
    }
}

// Second launch: the row's threshold from all pairs, then block p keeps its
// keys at or above it.  The threshold is found by weight: pair j of a block
// carries the increment c_j - c_(j-1) of its count, so G(v) is the summed
// increments of the pairs at or above v; value buckets over the pairs find
// the bucket where the running sum reaches k, and the pairs inside it are
// summed exactly.
template <int NT>
__global__ __launch_bounds__(NT) void topk_long_filter_kernel(
    const float *__restrict__ scores, int n_cols, int64_t row_stride,
    const int32_t *__restrict__ vlo, const int32_t *__restrict__ vhi, int k, int lo_skip,
    unsigned char *__restrict__ ws, int parts, int64_t pc_off, int64_t cand_off,
    int64_t row_bytes, int cap)
{
    constexpr int KPT = kTopkLongKeys / NT, NW = NT / 64, NP = kTopkLongPairs;
    constexpr int NB = 256;  // pair buckets
    constexpr int MAXP = kTopkLongMaxParts * NP;
    static_assert(KPT * NT == kTopkLongKeys && NT >= NB, "whole keys per thread, a bucket per thread");
    __shared__ uint64_t spv[MAXP];
    __shared__ uint32_t sdelta[MAXP];
    __shared__ uint32_t hist[NB];
    __shared__ uint64_t bin_v[MAXP];
    __shared__ uint32_t bin_d[MAXP];
    __shared__ uint64_t red64[2][NW];
    __shared__ int tab[NW];
    __shared__ int s_bin, s_above, s_nbin, s_base;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int row = blockIdx.x / parts, p = blockIdx.x - row * parts;
    unsigned char *w = ws + (int64_t)row * row_bytes;
    const uint64_t *pv = reinterpret_cast<const uint64_t *>(w + 64);
    const uint32_t *pc = reinterpret_cast<const uint32_t *>(w + pc_off);
    const int np = parts * NP;
    const int c0 = p * kTopkLongKeys;
    float sv[KPT];
    long_load_block<NT>(sv, scores + (int64_t)row * row_stride, c0, n_cols);
    // every pair load in flight before any is used
    constexpr int PPT = (MAXP + NT - 1) / NT;
    uint64_t lv[PPT];
    uint32_t lc[PPT], lcp[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int i = j * NT + tid;
        const bool in = i < np;
        lv[j] = in ? pv[i] : 0ull;
        lc[j] = in ? pc[i] : 0u;
        lcp[j] = (in && i % NP) ? pc[i - 1] : 0u;
    }
    uint64_t vmn = ~0ull, vmx = 0ull;
    int total = 0;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int i = j * NT + tid;
        if (i < np) {
            const uint32_t d = lc[j] > lcp[j] ? lc[j] - lcp[j] : 0u;
            spv[i] = lv[j];
            sdelta[i] = d;
            if (d) {
                vmn = lv[j] < vmn ? lv[j] : vmn;
                vmx = lv[j] > vmx ? lv[j] : vmx;
                total += (int)d;
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t a = shfl_xor_u64(vmn, o), b = shfl_xor_u64(vmx, o);
        vmn = a < vmn ? a : vmn;
        vmx = b > vmx ? b : vmx;
    }
    total = wave_sum_int(total);
    if (lane == 0) {
        red64[0][wid] = vmn;
        red64[1][wid] = vmx;
        tab[wid] = total;
    }
    if (tid < NB)
        hist[tid] = 0u;
    if (tid == 0)
        s_nbin = 0;
    __syncthreads();
    vmn = red64[0][0];
    vmx = red64[1][0];
    total = tab[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
        vmn = red64[0][i] < vmn ? red64[0][i] : vmn;
        vmx = red64[1][i] > vmx ? red64[1][i] : vmx;
        total += tab[i];
    }
    uint64_t t_low = 0ull;  // fewer than k keys guaranteed anywhere: all keys are candidates
    if (total >= k) {
        // bucket of a pair value, linear in the 64-bit key (monotone), 0 the best
        const double scale = vmx > vmn ? (double)(NB - 1) / (double)(vmx - vmn) : 0.0;
        auto pb = [&](uint64_t v) {
            const int b = (int)((double)(v - vmn) * scale);
            return NB - 1 - min(max(b, 0), NB - 1);
        };
        int pbk[PPT];
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int i = j * NT + tid;
            pbk[j] = (i < np && sdelta[i]) ? pb(spv[i]) : -1;
            if (pbk[j] >= 0)
                atomicAdd(&hist[pbk[j]], sdelta[i]);
        }
        __syncthreads();
        if (wid == 0) {
            // lane l owns buckets 4l .. 4l + 3: the bucket where the running
            // weight from the top reaches k
            static_assert(NB == 256, "four pair buckets per lane of one wave");
            uint32_t c4[4];
            int sum = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c4[j] = hist[4 * lane + j];
                sum += (int)c4[j];
            }
            int run = wave_inclusive_scan(sum) - sum;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (run < k && k <= run + (int)c4[j]) {
                    s_bin = 4 * lane + j;
                    s_above = run;
                }
                run += (int)c4[j];
            }
        }
        __syncthreads();
        const int bb = s_bin, ab = s_above;
        // the pairs of that bucket, compacted with one LDS atomic per wave
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const bool in = pbk[j] == bb;
            const uint64_t bal = __ballot(in);
            int base = 0;
            if (lane == 0 && bal)
                base = atomicAdd(&s_nbin, __popcll(bal));
            base = __builtin_amdgcn_readfirstlane(base);
            if (in) {
                const int slot = base + __popcll(bal & ((1ull << lane) - 1ull));
                const int i = j * NT + tid;
                bin_v[slot] = spv[i];
                bin_d[slot] = sdelta[i];
            }
        }
        __syncthreads();
        const int nbin = s_nbin;
        uint64_t best = 0ull;
        for (int i = tid; i < nbin; i += NT) {
            const uint64_t v = bin_v[i];
            int g = ab;
            for (int j = 0; j < nbin; ++j)
                g += bin_v[j] >= v ? (int)bin_d[j] : 0;
            if (g >= k && v > best)
                best = v;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const uint64_t a = shfl_xor_u64(best, o);
            best = a > best ? a : best;
        }
        if (lane == 0)
            red64[0][wid] = best;
        __syncthreads();
        t_low = red64[0][0];
#pragma unroll
        for (int i = 1; i < NW; ++i)
            t_low = red64[0][i] > t_low ? red64[0][i] : t_low;
    }
    // this block's keys at or above the threshold, one atomic per block
    const int row_hi = min(vhi[row], n_cols);
    const int lo = max(first_ranked(vlo[row], row_hi, lo_skip), c0);
    const int hi = min(row_hi, c0 + kTopkLongKeys);
    uint32_t take = 0u;
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int col = c0 + u * NT + tid;
        const bool t = col >= lo && col < hi &&
                       compose_key(score_order_key(sv[u]), (uint32_t)col) >= t_low;
        take |= (uint32_t)t << u;
        cnt += t;
    }
    const int incl = wave_inclusive_scan(cnt);
    __syncthreads();
    if (lane == 63)
        tab[wid] = incl;
    __syncthreads();
    int pos = incl - cnt;
    int block_total = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        pos += i < wid ? tab[i] : 0;
        block_total += tab[i];
    }
    if (block_total == 0)
        return;
    if (tid == 0)
        s_base = atomicAdd(reinterpret_cast<int *>(w), block_total);
    __syncthreads();
    pos += s_base;
    uint64_t *cand = reinterpret_cast<uint64_t *>(w + cand_off);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        if (take >> u & 1u) {
            if (pos < cap)
                cand[pos] = compose_key(score_order_key(sv[u]), (uint32_t)(c0 + u * NT + tid));
            ++pos;
        }
    }
}

// Third launch: `parts` blocks per row rank the row's candidates
// (merge_seg_row).  If the threshold kept more candidates than the
// workspace holds, block 0 of the row ranks the raw row instead: radix
// select of the k largest keys, then a sort.
template <int NT>
__global__ __launch_bounds__(NT) void topk_long_merge_kernel(
    const float *__restrict__ scores, int n_cols, int64_t row_stride,
    const int32_t *__restrict__ vlo, const int32_t *__restrict__ vhi, int k, int lo_skip,
    const unsigned char *__restrict__ ws, int64_t cand_off, int64_t row_bytes, int cap,
    int32_t *__restrict__ out, int64_t out_stride, int parts, int seg_len)
{
    __shared__ MergeSegSmem<NT> u;
    const int row = blockIdx.x / parts;
    const int seg = blockIdx.x - row * parts;
    const unsigned char *w = ws + (int64_t)row * row_bytes;
    const int n = *reinterpret_cast<const int *>(w);
    int32_t *o = out + (int64_t)row * out_stride;
    const uint64_t *cand = reinterpret_cast<const uint64_t *>(w + cand_off);
    if (n <= cap) {
        merge_seg_row<NT>(u, cand, n, k, o, seg, seg_len);
        return;
    }
    if (seg != 0)
        return;
    const int row_hi = min(vhi[row], n_cols);
    const int lo = first_ranked(vlo[row], row_hi, lo_skip);
    const int nv = max(row_hi - lo, 0);  // > cap > k: the threshold kept more than cap keys
    const float *srow = scores + (int64_t)row * row_stride + lo;
    auto key_at = [&](int i) { return compose_key(score_order_key(srow[i]), (uint32_t)(lo + i)); };
    radix_select(u.b, nv, k, key_at);
    constexpr int EPT = kTopkMaxK / NT;
    uint64_t v[EPT];
    bitonic_sort_regs<NT, EPT>(u.b, k, v);
    const int tid = threadIdx.x;
#pragma unroll
    for (int b = 0; b < EPT; ++b) {
        const int i = tid * EPT + b;
        if (i < k)
            o[i] = (int32_t)(0xffffffffu - (uint32_t)v[b]);
    }
}

constexpr int kCapLarge = kTopkChunkKeys;
static_assert(kTopkMaxK == kTopkMaxSelect, "one largest k for the host and the kernels");
constexpr int kCapSmall = 4096;

int topk_seg_parts(int rows, int k, int max_parts)
{
    int parts = (256 + rows - 1) / rows;
    parts = std::min(parts, max_parts);
    parts = std::min(parts, k / 64);
    return std::max(parts, 1);
}

// Scratch of the allocation-free top-k entry point: the threshold path's
// pairs and candidates, or the chunk winners of longer rows, in memory the
// library holds on each GPU for the life of the process.  Host code must not pass `scratch` itself to
// a kernel (in host code the name stands for a host-side shadow, not the
// device address): topk_scratch() looks the device address up once per
// device, with that device current, and every launch takes that pointer.
// Nothing in it has to start at zero: the chunk kernel writes every slot it
// owns (zero keys pad short chunks), and the pairs kernel writes every pair
// and clears the row's candidate count before the filter adds to it.
static __device__ __align__(256) unsigned char scratch[kTopkScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
} // namespace

hipError_t topk_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t st)
{
    // attention sinks take the first n_s ranks of every row; the kernels
    // below rank the rest of the visible range into the remaining k - n_s
    // places (rows keep their stride k)
    const int n_s = std::min(std::max(a.n_sink, 0), a.k);
    if (n_s > 0) {
        const int64_t blocks = ((int64_t)a.rows * n_s + 255) / 256;
        hipLaunchKernelGGL(topk_sink_prefix_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                           a.vis_lo, a.vis_hi, a.n_cols, a.rows, n_s, a.k, a.out);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || n_s == a.k)
            return e;
    }
    const int k = a.k - n_s;
    int32_t *const out = a.out + n_s;
    const int64_t ostride = a.k;
    // sort sizes: NT threads x EPT keys >= k
    if (a.n_cols <= kCapSmall) {
        // value buckets place each winner without sorting the row; several
        // blocks per row when there are few rows
        const int parts = topk_seg_parts(a.rows, k, 16);
        const int seg_len = (k + parts - 1) / parts;
        hipLaunchKernelGGL((topk_seg_kernel<512, kCapSmall>), dim3(a.rows * parts), dim3(512), 0,
                           st, a.scores, a.n_cols, a.row_stride, a.vis_lo, a.vis_hi, k, out,
                           ostride, n_s, parts, seg_len);
        return hipGetLastError();
    }
    constexpr int NT = 1024;
    if (a.n_cols <= kCapLarge) {
        // few rows: several blocks per row, each writing a segment of it
        const int parts = topk_seg_parts(a.rows, k, 16);
        const int seg_len = (k + parts - 1) / parts;
        hipLaunchKernelGGL((topk_seg_kernel<NT, kCapLarge>), dim3(a.rows * parts), dim3(NT), 0,
                           st, a.scores, a.n_cols, a.row_stride, a.vis_lo, a.vis_hi, k, out,
                           ostride, n_s, parts, seg_len);
        return hipGetLastError();
    }
    if (topk_long_path(a.n_cols)) {
        const TopkLongLayout l = topk_long_layout(a.n_cols);
        unsigned char *ws = static_cast<unsigned char *>(a.workspace);
        // 1024 threads, 4 keys each: four waves per SIMD hide each other's latency
        constexpr int LT = 1024;
        const unsigned blocks = (unsigned)(a.rows * l.parts);
        hipLaunchKernelGGL((topk_long_pairs_kernel<LT>), dim3(blocks), dim3(LT), 0, st, a.scores,
                           a.n_cols, a.row_stride, a.vis_lo, a.vis_hi, k, n_s, ws, l.parts,
                           l.pc_off, l.row_bytes);
        hipLaunchKernelGGL((topk_long_filter_kernel<LT>), dim3(blocks), dim3(LT), 0, st, a.scores,
                           a.n_cols, a.row_stride, a.vis_lo, a.vis_hi, k, n_s, ws, l.parts,
                           l.pc_off, l.cand_off, l.row_bytes, l.cap);
        const int mparts = topk_seg_parts(a.rows, k, 32);
        const int seg_len = (k + mparts - 1) / mparts;
        // the merge caches up to kMergeCacheKeys keys: 512 threads (32 per thread)
        hipLaunchKernelGGL((topk_long_merge_kernel<512>), dim3(a.rows * mparts), dim3(512), 0, st,
                           a.scores, a.n_cols, a.row_stride, a.vis_lo, a.vis_hi, k, n_s, ws,
                           l.cand_off, l.row_bytes, l.cap, out, ostride, mparts, seg_len);
        return hipGetLastError();
    }
    const int n_chunks = (a.n_cols + kCapLarge - 1) / kCapLarge;
    hipLaunchKernelGGL((topk_chunk_kernel<NT, kCapLarge>), dim3(a.rows * n_chunks), dim3(NT), 0,
                       st, a.scores, a.n_cols, a.row_stride, a.vis_lo, a.vis_hi, k,
                       static_cast<uint64_t *>(a.workspace), n_chunks, n_s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int mparts = topk_seg_parts(a.rows, k, 32);
    if ((int64_t)n_chunks * k <= kMergeCacheKeys && mparts > 1) {
        const int seg_len = (k + mparts - 1) / mparts;
        hipLaunchKernelGGL((topk_merge_seg_kernel<NT>), dim3(a.rows * mparts), dim3(NT), 0, st,
                           static_cast<const uint64_t *>(a.workspace), n_chunks, k, out, ostride,
                           mparts, seg_len);
        return hipGetLastError();
    }
    if ((int64_t)n_chunks * k <= kMergeCacheKeys)
        hipLaunchKernelGGL((topk_merge_kernel<NT, 2, true>), dim3(a.rows), dim3(NT), 0, st,
                           static_cast<const uint64_t *>(a.workspace), n_chunks, k, out, ostride);
    else
        hipLaunchKernelGGL((topk_merge_kernel<NT, 2, false>), dim3(a.rows), dim3(NT), 0, st,
                           static_cast<const uint64_t *>(a.workspace), n_chunks, k, out, ostride);
    return hipGetLastError();
}

} // namespace dsa
