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
#include "topk_device.hpp"

namespace dsa {

// Sorted top-k of the n order keys cached in sm (column lo + i for key i):
// 32-bit select, compaction, bucket sort (stable radix sort for ties and
// crowded buckets).  Returns m = min(k, n); the winners' columns in rank
// order are sm.wcol[buf][0 .. m).
template <int NT, int CAP>
__device__ int topk_sort_cached(Topk32Smem<NT, CAP> &sm, int n, int lo, int k, uint32_t omin,
                                uint32_t omax, int &buf)
{
    // n <= k: everything wins (mask 0 makes every key a candidate, all taken)
    uint32_t prefix = 0u, mask = 0u;
    int need = n, cand = n;
    if (n > k)
        select32(sm, n, k, omin, omax, prefix, mask, need, cand);
    // The bucket sort places each winner by its composite key (order key,
    // column), so it takes them in any order; when the whole boundary group
    // wins (no tie at the boundary to break by column) the fast unordered
    // compaction feeds it.  Equal order keys everywhere, or a bucket sort
    // that gives up, need the winners in column order (the stable radix
    // sort keeps it for equal keys): then the stable compaction reruns from
    // the key cache, which the bucket sort leaves intact.
    uint32_t wmin, wmax;
    const bool any_order = cand == need;
    int m = any_order ? compact32_any(sm, n, lo, prefix, mask, wmin, wmax)
                      : compact32(sm, n, lo, prefix, mask, need, cand, wmin, wmax);
    bool sorted = (!any_order || wmin != wmax) && bucket_sort32(sm, m, wmin, wmax);
    buf = 0;
    if (!sorted) {
        if (any_order)
            m = compact32(sm, n, lo, prefix, mask, need, cand, wmin, wmax);
        // all keys equal: column order is the rank order already
        buf = wmin == wmax ? 0 : sort32(sm, m, wmin, wmax);
    }
    return m;
}

// Float value of an order key (inverse of score_order_key; -0 comes back
// as +0).
__device__ __forceinline__ float order_key_value(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Segmented top-k: `parts` blocks share a row, block `seg` writes output
// positions [seg*seg_len, seg*seg_len + seg_len) of it, so a few rows still
// fill the chip.  Every block caches the whole row and counts it into NB
// buckets linear in the score value over [min, max] (a monotonic map, so a
// higher bucket never holds a lower-ranked key); the prefix sums give each
// bucket's first rank.  The block then collects only the buckets that hold
// its ranks and places each collected key inside its bucket by counting the
// members with a larger composite key (order key, then smaller column) --
// the exact rank order, ties included.  No block selects, compacts or sorts
// the whole row.  When its ranks fall into crowded buckets (a score range
// stretched by outliers) or the value range is not finite, the block takes
// the full sorted top-k of the row instead and writes its positions from it.
// Value buckets of a row segment (shared by the bucket kernels below): NB
// buckets linear in the score value over [vmin, vmax], numbered from the top
// (bucket 0 holds the largest values).  The map is monotonic, so every key
// of a lower-numbered bucket ranks above every key of a higher-numbered one.
struct ValueBuckets {
    float vmin, scale;
    int nb;
    __device__ bool init(uint32_t omin, uint32_t omax, int nbuckets)
    {
        nb = nbuckets;
        vmin = order_key_value(omin);
        const float vmax = order_key_value(omax);
        scale = (float)nb / (vmax - vmin);
        return __builtin_isfinite(vmin) && __builtin_isfinite(vmax) &&
               __builtin_isfinite(scale) && scale > 0.f;
    }
    __device__ int operator()(uint32_t ord) const
    {
        const int b = (int)((order_key_value(ord) - vmin) * scale);
        return nb - 1 - min(max(b, 0), nb - 1);
    }
};

constexpr int kSegMaxBucket = 256;
template <int NT, int CAP>
__global__ __launch_bounds__(NT) void topk_seg_kernel(const float *__restrict__ scores,
                                                      int n_cols, int64_t row_stride,
                                                      const int32_t *__restrict__ vlo,
                                                      const int32_t *__restrict__ vhi, int k,
                                                      int32_t *__restrict__ out, int parts,
                                                      int seg_len)
{
    using S = Topk32Smem<NT, CAP>;
    constexpr int NB = S::NB, NW = S::NW, PB = NB / NT, R = CAP / NT;
    static_assert(PB >= 1 && NB % NT == 0, "every thread owns whole buckets");
    __shared__ S sm;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int row = blockIdx.x / parts;
    const int seg = blockIdx.x - row * parts;
    const int lo = max(vlo[row], 0), hi = min(vhi[row], n_cols);
    const int n = max(hi - lo, 0);
    const int rounds = (n + NT - 1) / NT;  // uniform, at most R
    // thread t keeps keys r*NT + t (r < rounds) in registers: their order keys
    // and, below, their buckets (all loads issued before any is used)
    const float *rp = scores + (int64_t)row * row_stride + lo;
    uint32_t ord[R];
    {
        float v[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            v[r] = (r < rounds && r * NT + tid < n) ? rp[r * NT + tid] : 0.f;
        uint32_t mn = ~0u, mx = 0u;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            ord[r] = score_order_key(v[r]);
            if (r < rounds && r * NT + tid < n) {
                mn = min(mn, ord[r]);
                mx = max(mx, ord[r]);
            }
        }
        mn = wave_min_u32(mn);
        mx = wave_max_u32(mx);
        if (lane == 0) {
            sm.mm[0][wid] = mn;
            sm.mm[1][wid] = mx;
        }
    }
    for (int i = tid; i < NB; i += NT)
        sm.bk.fill[i] = 0u;
    __syncthreads();
    uint32_t omin = sm.mm[0][0], omax = sm.mm[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        omin = min(omin, sm.mm[0][w]);
        omax = max(omax, sm.mm[1][w]);
    }
    const int m = min(k, n);
    int32_t *o = out + (int64_t)row * k;
    const int p0 = seg * seg_len, p1 = min(p0 + seg_len, k);
    for (int i = max(p0, m) + tid; i < p1; i += NT)
        o[i] = -1;
    const int s0 = p0, s1 = min(p1, m);  // ranks this block writes
    if (s0 >= s1)
        return;
    if (omin == omax) {  // every key equal: column order is the rank order
        for (int i = s0 + tid; i < s1; i += NT)
            o[i] = lo + i;
        return;
    }
    ValueBuckets bucket;
    bool ok = bucket.init(omin, omax, NB);
    if (ok) {
        int bk[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            bk[r] = NB;  // none
            if (r < rounds && r * NT + tid < n) {
                bk[r] = bucket(ord[r]);
                atomicAdd(&sm.bk.fill[bk[r]], 1u);
            }
        }
        __syncthreads();
        // exclusive prefix over the buckets (thread t owns PB consecutive
        // ones); the buckets holding ranks s0 and s1-1
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
        int crowd_lo = 0, crowd_hi = 0;  // sizes of the buckets holding s0 and s1-1
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int b = tid * PB + j, c = (int)v[j];
            sm.bk.off[b] = (uint32_t)run;
            sm.bk.fill[b] = (uint32_t)run;  // fill pointer of the collection below
            if (run <= s0 && s0 < run + c) {
                sm.tab[1][0] = b;
                crowd_lo = c;
            }
            if (run <= s1 - 1 && s1 - 1 < run + c) {
                sm.tab[1][1] = b;
                crowd_hi = c;
            }
            run += c;
        }
        // a bucket strictly between them holds only ranks of this segment
        // (all of which are placed anyway); the two end buckets can hold many
        // keys outside it (ties, or a range stretched by an outlier), and
        // placing a key costs one compare per member of its bucket
        if (crowd_lo)
            sm.red[0][0][0] = crowd_lo;
        if (crowd_hi)
            sm.red[0][0][1] = crowd_hi;
        __syncthreads();
        const int bf = sm.tab[1][0], bl = sm.tab[1][1];
        const int base = (int)sm.bk.off[bf];
        const int crowd = max(sm.red[0][0][0], sm.red[0][0][1]);
        const int total = (bl + 1 < NB ? (int)sm.bk.off[bl + 1] : n) - base;  // keys of bf .. bl
        // the collection buffer holds 3072 keys: k plus the rest of the last bucket
        constexpr int kCollect = (int)((sizeof(sm.word[1]) + sizeof(sm.wcol)) / 8);
        ok = crowd <= kSegMaxBucket && total <= kCollect;
        if (ok) {
            // the collection from registers (key of rank base + i at ck[i])
            uint64_t *ck = reinterpret_cast<uint64_t *>(&sm.word[1][0]);
            static_assert(kCollect >= kTopkMaxK + kSegMaxBucket,
                          "composite key buffer");
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (bk[r] >= bf && bk[r] <= bl)
                    ck[atomicAdd(&sm.bk.fill[bk[r]], 1u) - (uint32_t)base] =
                        ((uint64_t)ord[r] << 32) |
                        (uint64_t)(0xffffffffu - (uint32_t)(lo + r * NT + tid));
            }
            __syncthreads();
            // rank of each collected key: its bucket's first rank plus the
            // members of the bucket above it
            for (int j = tid; j < total; j += NT) {
                const uint64_t key = ck[j];
                const int b = bucket((uint32_t)(key >> 32));
                const int b0 = (int)sm.bk.off[b] - base, b1 = (int)sm.bk.fill[b] - base;
                int r = (int)sm.bk.off[b];
                for (int x = b0; x < b1; ++x)
                    r += ck[x] > key;
                if (r >= s0 && r < s1)
                    o[r] = (int32_t)(0xffffffffu - (uint32_t)key);
            }
            return;
        }
        __syncthreads();  // the bucket arrays are reused below
    }
    // the full sorted top-k of the row, from the key cache
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (r < rounds && r * NT + tid < n)
            sm.a.ord[r * NT + tid] = ord[r];
    __syncthreads();
    int buf;
    topk_sort_cached(sm, n, lo, k, omin, omax, buf);
    for (int i = s0 + tid; i < s1; i += NT)
        o[i] = (int32_t)sm.wcol[buf][i];
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
                                                        int32_t *__restrict__ out)
{
    __shared__ MergeSmem<NT, CACHE> sm;
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    uint64_t v[EPT];
    int m;
    merge_sorted<NT, EPT, CACHE>(sm, ws + (int64_t)row * n_chunks * k, n_chunks * k, k, v, m);
    int32_t *o = out + (int64_t)row * k;
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
                                                        uint64_t *__restrict__ ws, int n_chunks)
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
    const int lo = max(max(vlo[row], 0), c0);
    const int hi = min(min(vhi[row], n_cols), c0 + CAP);
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

// Second launch of the long-row path for few rows: `parts` blocks share a
// row's candidates (the chunk winners ws[row][0 .. n), zero keys padding;
// at most kMergeCacheKeys), block `seg` writes output positions
// [seg*seg_len, seg*seg_len + seg_len), as in topk_seg_kernel: value buckets
// over the real candidates, the buckets that hold the block's ranks
// collected and ranked inside by composite key.  Crowded buckets or a
// non-finite range fall back to the full merge of the row.
template <int NT>
__global__ __launch_bounds__(NT) void topk_merge_seg_kernel(const uint64_t *__restrict__ ws,
                                                            int n_chunks, int k,
                                                            int32_t *__restrict__ out, int parts,
                                                            int seg_len)
{
    using S = Topk32Smem<NT, kMergeCacheKeys>;
    using M = MergeSmem<NT, true>;
    constexpr int NB = S::NB, NW = S::NW, PB = NB / NT;
    union U {
        S a;
        M b;
    };
    __shared__ U u;
    S &sm = u.a;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int row = blockIdx.x / parts;
    const int seg = blockIdx.x - row * parts;
    const uint64_t *cand = ws + (int64_t)row * n_chunks * k;
    const int n = n_chunks * k;
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
    int32_t *o = out + (int64_t)row * k;
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
    constexpr int EPT = 2;
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

constexpr int kCapLarge = 16384;
constexpr int kCapSmall = 4096;

size_t topk_workspace_bytes(int rows, int n_cols, int k)
{
    if (n_cols <= kCapLarge)
        return 0;
    const int64_t n_chunks = (n_cols + kCapLarge - 1) / kCapLarge;
    return (size_t)rows * (size_t)n_chunks * (size_t)k * sizeof(uint64_t);
}

// Blocks per row for the segmented kernels: enough for about 256 blocks in
// all, at most max_parts, and segments of at least 64 ranks; 1 = one block
// per row.
int topk_seg_parts(int rows, int k, int max_parts)
{
    int parts = (256 + rows - 1) / rows;
    parts = std::min(parts, max_parts);
    parts = std::min(parts, k / 64);
    return std::max(parts, 1);
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t st)
{
    // sort sizes: NT threads x EPT keys >= k
    if (a.n_cols <= kCapSmall) {
        // value buckets place each winner without sorting the row; several
        // blocks per row when there are few rows
        const int parts = topk_seg_parts(a.rows, a.k, 16);
        const int seg_len = (a.k + parts - 1) / parts;
        hipLaunchKernelGGL((topk_seg_kernel<512, kCapSmall>), dim3(a.rows * parts), dim3(512), 0,
                           st, a.scores, a.n_cols, a.row_stride, a.vis_lo, a.vis_hi, a.k, a.out,
                           parts, seg_len);
        return hipGetLastError();
    }
    constexpr int NT = 1024;
    if (a.n_cols <= kCapLarge) {
        // few rows: several blocks per row, each writing a segment of it
        const int parts = topk_seg_parts(a.rows, a.k, 16);
        const int seg_len = (a.k + parts - 1) / parts;
        hipLaunchKernelGGL((topk_seg_kernel<NT, kCapLarge>), dim3(a.rows * parts), dim3(NT), 0,
                           st, a.scores, a.n_cols, a.row_stride, a.vis_lo, a.vis_hi, a.k, a.out,
                           parts, seg_len);
        return hipGetLastError();
    }
    const int n_chunks = (a.n_cols + kCapLarge - 1) / kCapLarge;
    hipLaunchKernelGGL((topk_chunk_kernel<NT, kCapLarge>), dim3(a.rows * n_chunks), dim3(NT), 0,
                       st, a.scores, a.n_cols, a.row_stride, a.vis_lo, a.vis_hi, a.k,
                       static_cast<uint64_t *>(a.workspace), n_chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int mparts = topk_seg_parts(a.rows, a.k, 32);
    if ((int64_t)n_chunks * a.k <= kMergeCacheKeys && mparts > 1) {
        const int seg_len = (a.k + mparts - 1) / mparts;
        hipLaunchKernelGGL((topk_merge_seg_kernel<NT>), dim3(a.rows * mparts), dim3(NT), 0, st,
                           static_cast<const uint64_t *>(a.workspace), n_chunks, a.k, a.out,
                           mparts, seg_len);
        return hipGetLastError();
    }
    if ((int64_t)n_chunks * a.k <= kMergeCacheKeys)
        hipLaunchKernelGGL((topk_merge_kernel<NT, 2, true>), dim3(a.rows), dim3(NT), 0, st,
                           static_cast<const uint64_t *>(a.workspace), n_chunks, a.k, a.out);
    else
        hipLaunchKernelGGL((topk_merge_kernel<NT, 2, false>), dim3(a.rows), dim3(NT), 0, st,
                           static_cast<const uint64_t *>(a.workspace), n_chunks, a.k, a.out);
    return hipGetLastError();
}

} // namespace dsa
