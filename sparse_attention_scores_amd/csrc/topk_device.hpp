// topk_device.hpp -- block-wide exact top-k building blocks (gfx950).
//
// Each candidate is one 64-bit composite key
//     (order_key(score) << 32) | (0xffffffff - column)
// whose unsigned order is the rank order "higher score, then smaller index"
// ("Module glm5next_dsa_ref", topk_pools), -0 folded onto +0.  Keys of one
// row are distinct, so "the k largest keys" is a single well-defined set.
#pragma once

#include "dsa_device.hpp"

namespace dsa {

constexpr int kTopkMaxK = 2048;

// Radix histogram copies: waves add into copy (wave % HC) so that LDS
// atomics on a popular bin are spread over HC addresses.
template <int NT, int CAP>
constexpr int topk_hist_copies()
{
    // the 16384-key merge cache leaves room for 4 copies only
    return CAP > 16384 ? 4 : NT / 64;
}

template <int NT, int CAP>
struct __attribute__((aligned(16))) TopkSmem {
    static constexpr int HC = topk_hist_copies<NT, CAP>();
    uint32_t ord[CAP];          // order keys of the row (source = scores)
    uint64_t sel[kTopkMaxK];    // winners
    uint32_t hist[HC][256];
    uint64_t red_min[NT / 64];
    uint64_t red_max[NT / 64];
    int count;
    int bin;
    int above;
    int bincnt;
};

__device__ __forceinline__ uint64_t compose_key(uint32_t ord, uint32_t col)
{
    return ((uint64_t)ord << 32) | (uint64_t)(0xffffffffu - col);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o)
{
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = (uint32_t)__shfl_xor((int)lo, o, kWave);
    hi = (uint32_t)__shfl_xor((int)hi, o, kWave);
    return ((uint64_t)hi << 32) | lo;
}

// x[lane ^ o] for o a power of two below 64, without going through LDS where
// the lane pattern allows: DPP quad permutations for 1 and 2, a quad
// reversal followed by a half-row mirror for 4 (i ^ 3 ^ 7), a row mirror
// followed by a half-row mirror for 8 (i ^ 15 ^ 7), ds_swizzle (xor mask
// within 32 lanes, no memory access) for 16, ds_bpermute for 32.  `o` must
// fold to a constant.
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t x, int o)
{
    switch (o) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
    case 4: {
        const int y = __builtin_amdgcn_update_dpp(0, (int)x, 0x1B, 0xF, 0xF, false);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, y, 0x141, 0xF, 0xF, false);
    }
    case 8: {
        const int y = __builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, y, 0x141, 0xF, 0xF, false);
    }
    case 16: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F);
    default: return (uint32_t)__shfl_xor((int)x, o, kWave);
    }
}

__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v, int o)
{
    const uint32_t lo = lane_xor_u32((uint32_t)v, o), hi = lane_xor_u32((uint32_t)(v >> 32), o);
    return ((uint64_t)hi << 32) | lo;
}

// Select the k largest of n distinct keys (n > k) into sm.sel[0..k).
// key_at(i) returns the i-th key.  Block-wide; all threads call it.
template <int NT, int CAP, typename KeyAt>
__device__ void radix_select(TopkSmem<NT, CAP> &sm, int n, int k, KeyAt key_at)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    // ---- shared high bits: min/max over all keys
    uint64_t mn = ~0ull, mx = 0ull;
    for (int i = tid; i < n; i += NT) {
        uint64_t key = key_at(i);
        mn = key < mn ? key : mn;
        mx = key > mx ? key : mx;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint64_t a = shfl_xor_u64(mn, o), b = shfl_xor_u64(mx, o);
        mn = a < mn ? a : mn;
        mx = b > mx ? b : mx;
    }
    if (lane == 0) {
        sm.red_min[wid] = mn;
        sm.red_max[wid] = mx;
    }
    __syncthreads();
    mn = sm.red_min[0];
    mx = sm.red_max[0];
    for (int i = 1; i < NT / 64; ++i) {
        mn = sm.red_min[i] < mn ? sm.red_min[i] : mn;
        mx = sm.red_max[i] > mx ? sm.red_max[i] : mx;
    }
    // keys are distinct and n > k >= 1, so mn != mx
    const int common = __clzll((long long)(mn ^ mx));
    uint64_t mask = common ? (~0ull << (64 - common)) : 0ull;
    uint64_t prefix = mn & mask;
    int top = 63 - common;  // highest undecided bit
    int need = k;
    while (true) {
        const int shift = top >= 7 ? top - 7 : 0;
        const int width = top - shift + 1;
        const uint32_t dmask = (1u << width) - 1u;
        constexpr int HC = TopkSmem<NT, CAP>::HC;
        for (int i = tid; i < 256 * HC; i += NT)
            (&sm.hist[0][0])[i] = 0;
        __syncthreads();
        uint32_t *hist = sm.hist[wid % HC];
        for (int i = tid; i < n; i += NT) {
            const uint64_t key = key_at(i);
            if ((key & mask) == prefix)
                atomicAdd(&hist[(uint32_t)(key >> shift) & dmask], 1u);
        }
        __syncthreads();
        if (wid == 0) {
            // lane j owns bins 255-4j .. 252-4j (descending)
            int c[4];
            int s = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                int ct = 0;
#pragma unroll
                for (int h = 0; h < HC; ++h)
                    ct += (int)sm.hist[h][255 - 4 * lane - t];
                c[t] = ct;
                s += c[t];
            }
            int above = wave_inclusive_scan(s) - s;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (above < need && need <= above + c[t]) {
                    sm.bin = 255 - 4 * lane - t;
                    sm.above = above;
                    sm.bincnt = c[t];
                }
                above += c[t];
            }
        }
        __syncthreads();
        const int bin = sm.bin;
        need -= sm.above;
        const int bincnt = sm.bincnt;
        prefix |= (uint64_t)bin << shift;
        mask |= (uint64_t)dmask << shift;
        __syncthreads();  // everyone has read sm.bin before the next pass
        if (bincnt == need || shift == 0)
            break;
        top = shift - 1;
    }
    // ---- compaction: exactly k keys satisfy (key & mask) >= prefix.  One
    //      LDS atomic per wave (ballot + prefix count) rather than per key.
    if (tid == 0)
        sm.count = 0;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += NT) {
        const int i = i0 + tid;
        uint64_t key = 0;
        bool take = false;
        if (i < n) {
            key = key_at(i);
            take = (key & mask) >= prefix;
        }
        const uint64_t bal = __ballot(take);
        const int cnt = __popcll(bal);
        int base = 0;
        if (lane == 0 && cnt)
            base = atomicAdd(&sm.count, cnt);
        base = __shfl(base, 0, kWave);
        if (take) {
            const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
            if (pos < kTopkMaxK)
                sm.sel[pos] = key;
        }
    }
    __syncthreads();
}

// Descending bitonic sort of the P = NT*EPT keys sm.sel[0..m) (zero-padded;
// zero is below every real key), held in registers: thread t owns positions
// t*EPT .. t*EPT+EPT-1.  Strides below EPT stay inside a thread, strides up
// to 64*EPT use cross-lane shuffles within the wave, larger strides go
// through LDS.  On return v[b] holds the key of rank t*EPT + b.
template <int NT, int EPT, int CAP>
__device__ void bitonic_sort_regs(TopkSmem<NT, CAP> &sm, int m, uint64_t (&v)[EPT])
{
    constexpr int P = NT * EPT;
    static_assert(P <= kTopkMaxK, "sort size exceeds the LDS staging array");
    const int tid = threadIdx.x;
#pragma unroll
    for (int b = 0; b < EPT; ++b) {
        const int i = tid * EPT + b;
        v[b] = i < m ? sm.sel[i] : 0ull;
    }
#pragma unroll
    for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
        for (int s = size >> 1; s > 0; s >>= 1) {
            if (s < EPT) {
#pragma unroll
                for (int b = 0; b < EPT; ++b) {
                    if ((b & s) == 0) {
                        const int i = tid * EPT + b;
                        const bool desc = (i & size) == 0;
                        const uint64_t x = v[b], y = v[b + s];
                        const bool sw = desc ? (x < y) : (x > y);
                        v[b] = sw ? y : x;
                        v[b + s] = sw ? x : y;
                    }
                }
            } else {
                uint64_t pv[EPT];
                if (s / EPT < 64) {
#pragma unroll
                    for (int b = 0; b < EPT; ++b)
                        pv[b] = lane_xor_u64(v[b], s / EPT);
                } else {
                    __syncthreads();
#pragma unroll
                    for (int b = 0; b < EPT; ++b)
                        sm.sel[tid * EPT + b] = v[b];
                    __syncthreads();
#pragma unroll
                    for (int b = 0; b < EPT; ++b)
                        pv[b] = sm.sel[(tid * EPT + b) ^ s];
                }
#pragma unroll
                for (int b = 0; b < EPT; ++b) {
                    const int i = tid * EPT + b;
                    const bool lower = (i & s) == 0;
                    const bool desc = (i & size) == 0;
                    const uint64_t x = v[b], y = pv[b];
                    const uint64_t hi = x > y ? x : y, lo = x > y ? y : x;
                    v[b] = (lower == desc) ? hi : lo;
                }
            }
        }
    }
    __syncthreads();
}

// Load scores[lo, hi) of one row into sm.ord and return n.  Each thread
// issues all of its loads of a round before it stores any, so a row costs one
// or two memory round trips rather than one per element.
template <int NT, int CAP>
__device__ int load_row(TopkSmem<NT, CAP> &sm, const float *__restrict__ row, int lo, int hi)
{
    constexpr int U = (CAP / NT) < 8 ? (CAP / NT) : 8;
    const int n = max(hi - lo, 0);
    for (int base = 0; base < n; base += NT * U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * NT + (int)threadIdx.x;
            v[u] = i < n ? row[lo + i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * NT + (int)threadIdx.x;
            if (i < n)
                sm.ord[i] = score_order_key(v[u]);
        }
    }
    __syncthreads();
    return n;
}

} // namespace dsa

namespace dsa {

// ---------------------------------------------------------------------------
// Sorted top-k of one row on 32-bit order keys.
//
// The row's order keys sit in LDS in column order.  Rank order is "larger
// order key first, then smaller column", so:
//  1. a radix select over the 32-bit order keys finds the boundary: keys whose
//     masked value is above the boundary prefix all win, and among the keys
//     equal to it the first `need` in column order win;
//  2. a stable compaction (ballots and wave totals, no atomics) writes the
//     winners in column order;
//  3. a stable LSD radix sort on the inverted order key (8-bit digits, only
//     over the bits in which the winners differ) then leaves equal keys in
//     column order, which is exactly the tie rule.
// KM is the largest k the block serves (the winner arrays) and NBK the
// number of value buckets.
template <int NT, int CAP, int KM = kTopkMaxK, int NBK = 2048>
struct __attribute__((aligned(16))) Topk32Smem {
    static constexpr int NW = NT / 64;
    static constexpr int EPT = KM / NT;                  // sort rounds (winners per thread)
    static constexpr int NCNT = 256 * EPT * NW;          // (digit, round, wave) counters
    static constexpr int NB = NBK;                       // bucket-sort buckets
    static constexpr int R = CAP / NT;                   // compaction rounds
    static_assert(KM % NT == 0 && EPT >= 1, "whole sort rounds");
    static_assert(CAP * 4 >= NCNT * 2, "radix-sort counters overlay the key cache");
    static_assert(R <= 32, "round flags are kept in one 32-bit mask");
    union {
        uint32_t ord[CAP];        // order keys of the row, column order
        uint16_t cnt[NCNT];       // radix-sort counters, after the last compaction
    } a;
    int tab[2][R * NW + 1];       // (round, wave) counts -> exclusive prefixes, + total
    uint32_t word[2][KM];         // winners' order keys (sort ping-pong)
    uint32_t wcol[2][KM];         // winners' columns
    union {
        uint32_t hist[NW][256];   // per-wave select histograms
        struct {
            uint32_t off[NB];     // bucket offsets
            uint32_t fill[NB];    // bucket counts, then fill pointers
        } bk;                     // (the bucket sort leaves the key cache intact)
    };
    int red[2][2][NW];            // per-wave totals (two round parities x two counts)
    uint32_t mm[2][NW];           // per-wave min / max
    int bin, above, bincnt, fill;
};

// Load scores[lo, hi) into sm.a.ord (column order) and reduce their min/max.
template <int NT, int CAP, int KM, int NBK>
__device__ int load_row32(Topk32Smem<NT, CAP, KM, NBK> &sm, const float *__restrict__ row, int lo,
                          int hi, uint32_t &omin, uint32_t &omax)
{
    constexpr int U = (CAP / NT) < 8 ? (CAP / NT) : 8;
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int n = max(hi - lo, 0);
    uint32_t mn = ~0u, mx = 0u;
    for (int base = 0; base < n; base += NT * U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * NT + tid;
            v[u] = i < n ? row[lo + i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * NT + tid;
            if (i < n) {
                const uint32_t o = score_order_key(v[u]);
                sm.a.ord[i] = o;
                mn = min(mn, o);
                mx = max(mx, o);
            }
        }
    }
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        sm.mm[0][wid] = mn;
        sm.mm[1][wid] = mx;
    }
    __syncthreads();
    omin = sm.mm[0][0];
    omax = sm.mm[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        omin = min(omin, sm.mm[0][w]);
        omax = max(omax, sm.mm[1][w]);
    }
    __syncthreads();
    return n;
}

// Boundary of the k largest of the n order keys in sm.a.ord (n > k >= 1):
// keys with (ord & mask) > prefix win (k - need of them); of the `cand` keys
// with (ord & mask) == prefix, the first `need` in column order win.
template <int NT, int CAP, int KM, int NBK>
__device__ void select32(Topk32Smem<NT, CAP, KM, NBK> &sm, int n, int k, uint32_t omin,
                         uint32_t omax, uint32_t &prefix, uint32_t &mask, int &need, int &cand)
{
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const uint32_t diff = omin ^ omax;
    int top = diff ? 31 - __clz(diff) : -1;  // highest bit in which keys differ
    mask = top >= 0 ? ~((2u << top) - 1u) : ~0u;
    prefix = omin & mask;
    need = k;
    cand = n;
    while (top >= 0) {
        const int shift = top >= 7 ? top - 7 : 0;
        const int width = top - shift + 1;
        const uint32_t dmask = (1u << width) - 1u;
        for (int i = tid; i < 256 * NW; i += NT)
            (&sm.hist[0][0])[i] = 0u;
        __syncthreads();
        uint32_t *hist = sm.hist[wid];
        for (int i = tid; i < n; i += NT) {
            const uint32_t key = sm.a.ord[i];
            if ((key & mask) == prefix)
                atomicAdd(&hist[(key >> shift) & dmask], 1u);
        }
        __syncthreads();
        if (wid == 0) {
            // lane j owns bins 255-4j .. 252-4j (descending)
            int c[4];
            int s = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                int ct = 0;
#pragma unroll
                for (int h = 0; h < NW; ++h)
                    ct += (int)sm.hist[h][255 - 4 * lane - t];
                c[t] = ct;
                s += ct;
            }
            int above = wave_inclusive_scan(s) - s;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (above < need && need <= above + c[t]) {
                    sm.bin = 255 - 4 * lane - t;
                    sm.above = above;
                    sm.bincnt = c[t];
                }
                above += c[t];
            }
        }
        __syncthreads();
        need -= sm.above;
        cand = sm.bincnt;
        prefix |= (uint32_t)sm.bin << shift;
        mask |= dmask << shift;
        __syncthreads();  // everyone has read sm.bin before the next pass
        if (cand == need)
            break;
        top = shift - 1;
    }
}

// Exclusive scan, in place, of tab[0 .. e) by wave 0 (e <= 256); the total
// goes to tab[e].  Callers synchronise before and after.
__device__ __forceinline__ void wave_scan_table(int *tab, int e)
{
    const int lane = threadIdx.x & 63;
    int v[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = 4 * lane + j < e ? tab[4 * lane + j] : 0;
        s += v[j];
    }
    const int incl = wave_inclusive_scan(s);
    int run = incl - s;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (4 * lane + j < e)
            tab[4 * lane + j] = run;
        run += v[j];
    }
    if (lane == 63)
        tab[e] = incl;
}

// Stable compaction of the winners into sm.word[0] / sm.wcol[0] (column
// order); returns their count (k when n > k, else n) and their min / max.
// Element i = r*NT + tid is held by thread tid in round r, so column order
// is (round, wave, lane): each thread keeps its per-round flags in a bit
// mask, the (round, wave) counts are scanned once by one wave, and the
// positions follow from ballots -- two barriers per counted quantity.
template <int NT, int CAP, int KM, int NBK>
__device__ int compact32(Topk32Smem<NT, CAP, KM, NBK> &sm, int n, int col0, uint32_t prefix,
                         uint32_t mask, int need, int cand, uint32_t &wmin, uint32_t &wmax)
{
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const uint64_t lt = (1ull << lane) - 1ull;
    const int rounds = (n + NT - 1) / NT;
    const int e = rounds * NW;
    uint32_t abv = 0u, eqm = 0u;
    for (int r = 0; r < rounds; ++r) {
        const int i = r * NT + tid;
        if (i < n) {
            const uint32_t key = sm.a.ord[i] & mask;
            abv |= (uint32_t)(key > prefix) << r;
            eqm |= (uint32_t)(key == prefix) << r;
        }
    }
    uint32_t winm = abv;
    if (cand > need) {
        // ties at the boundary: the first `need` candidates in column order win
        for (int r = 0; r < rounds; ++r) {
            const uint64_t cb = __ballot((eqm >> r) & 1u);
            if (lane == 0)
                sm.tab[0][r * NW + wid] = __popcll(cb);
        }
        __syncthreads();
        if (wid == 0)
            wave_scan_table(sm.tab[0], e);
        __syncthreads();
        for (int r = 0; r < rounds; ++r) {
            const uint64_t cb = __ballot((eqm >> r) & 1u);
            const int rank = sm.tab[0][r * NW + wid] + __popcll(cb & lt);
            winm |= (uint32_t)(((eqm >> r) & 1u) && rank < need) << r;
        }
    } else {
        winm |= eqm;  // the whole boundary group wins
    }
    for (int r = 0; r < rounds; ++r) {
        const uint64_t wb = __ballot((winm >> r) & 1u);
        if (lane == 0)
            sm.tab[1][r * NW + wid] = __popcll(wb);
    }
    __syncthreads();
    if (wid == 0)
        wave_scan_table(sm.tab[1], e);
    __syncthreads();
    uint32_t mn = ~0u, mx = 0u;
    for (int r = 0; r < rounds; ++r) {
        const uint64_t wb = __ballot((winm >> r) & 1u);
        if ((winm >> r) & 1u) {
            const int i = r * NT + tid;
            const uint32_t key = sm.a.ord[i];
            const int pos = sm.tab[1][r * NW + wid] + __popcll(wb & lt);
            sm.word[0][pos] = key;
            sm.wcol[0][pos] = (uint32_t)(col0 + i);
            mn = min(mn, key);
            mx = max(mx, key);
        }
    }
    const int total = sm.tab[1][e];
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        sm.mm[0][wid] = mn;
        sm.mm[1][wid] = mx;
    }
    __syncthreads();
    wmin = sm.mm[0][0];
    wmax = sm.mm[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        wmin = min(wmin, sm.mm[0][w]);
        wmax = max(wmax, sm.mm[1][w]);
    }
    return total;
}

// Compaction of the winners into sm.word[0] / sm.wcol[0] in no particular
// order, for the case where the whole boundary group wins (cand == need, or
// n <= k with mask 0): every key with (ord & mask) >= prefix.  Each wave
// counts its winners over all rounds first and claims one range of an LDS
// counter with a single atomic; the positions inside it follow from the
// ballots.  Returns the count and the winners' min / max.
template <int NT, int CAP, int KM, int NBK>
__device__ int compact32_any(Topk32Smem<NT, CAP, KM, NBK> &sm, int n, int col0, uint32_t prefix,
                             uint32_t mask, uint32_t &wmin, uint32_t &wmax)
{
    constexpr int NW = NT / 64, R = CAP / NT;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const uint64_t lt = (1ull << lane) - 1ull;
    if (tid == 0)
        sm.fill = 0;
    __syncthreads();
    const int rounds = (n + NT - 1) / NT;
    uint32_t key[R];
    uint64_t wb[R];
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * NT + tid;
        key[r] = 0u;
        wb[r] = 0ull;
        if (r < rounds) {  // uniform
            key[r] = i < n ? sm.a.ord[i] : 0u;
            wb[r] = __ballot(i < n && (key[r] & mask) >= prefix);
            cnt += __popcll(wb[r]);
        }
    }
    int base = 0;
    if (lane == 0 && cnt)
        base = atomicAdd(&sm.fill, cnt);
    base = __builtin_amdgcn_readfirstlane(base);
    uint32_t mn = ~0u, mx = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if ((wb[r] >> lane) & 1ull) {
            const int pos = base + __popcll(wb[r] & lt);
            sm.word[0][pos] = key[r];
            sm.wcol[0][pos] = (uint32_t)(col0 + r * NT + tid);
            mn = min(mn, key[r]);
            mx = max(mx, key[r]);
        }
        base += __popcll(wb[r]);
    }
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        sm.mm[0][wid] = mn;
        sm.mm[1][wid] = mx;
    }
    __syncthreads();
    wmin = sm.mm[0][0];
    wmax = sm.mm[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        wmin = min(wmin, sm.mm[0][w]);
        wmax = max(wmax, sm.mm[1][w]);
    }
    const int total = sm.fill;
    __syncthreads();  // mm and fill are read before they are reused
    return total;
}

// Bucket sort of the m winners (sm.word / sm.wcol buffer 0, column order) by
// descending order key: buckets on the top (up to) 11 bits in which the
// winners differ, then each winner's place inside its bucket by counting the
// bucket's members that rank above it (larger key, or equal key and smaller
// column).  The result replaces buffer 0.  Returns false, touching nothing
// but the bucket arrays, when a bucket holds more than 64 winners (many
// equal high bits): the caller then sorts with sort32.
template <int NT, int CAP, int KM, int NBK>
__device__ bool bucket_sort32(Topk32Smem<NT, CAP, KM, NBK> &sm, int m, uint32_t wmin, uint32_t wmax)
{
    using S = Topk32Smem<NT, CAP, KM, NBK>;
    constexpr int NB = S::NB, NW = S::NW, PB = NB / NT;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const uint32_t diff = wmin ^ wmax;
    const int bits = diff ? 32 - __clz(diff) : 0;
    if (bits == 0)
        return true;  // all keys equal: column order is rank order
    // about one bucket per winner (at least 64, at most NB)
    int lg = 6;
    while (lg < 11 && (1 << lg) < m)
        ++lg;
    const int dbits = bits < lg ? bits : lg;
    const int shift = bits - dbits;
    const uint32_t dmask = (1u << dbits) - 1u;
    const int nb = 1 << dbits;
    for (int i = tid; i < nb; i += NT)
        sm.bk.fill[i] = 0u;
    __syncthreads();
    for (int i = tid; i < m; i += NT) {
        const int bkt = nb - 1 - (int)((sm.word[0][i] >> shift) & dmask);  // descending
        atomicAdd(&sm.bk.fill[bkt], 1u);
    }
    __syncthreads();
    // exclusive scan of the nb counts (thread t owns PB consecutive buckets)
    // and their maximum
    {
        uint32_t v[PB];
        int s = 0, mx = 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int bkt = tid * PB + j;
            v[j] = bkt < nb ? sm.bk.fill[bkt] : 0u;
            s += (int)v[j];
            mx = max(mx, (int)v[j]);
        }
        const int incl = wave_inclusive_scan(s);
        mx = (int)wave_max_u32((uint32_t)mx);
        if (lane == 63) {
            sm.tab[0][wid] = incl;
            sm.tab[1][wid] = mx;
        }
        __syncthreads();
        int before = incl - s;
        int big = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            before += w < wid ? sm.tab[0][w] : 0;
            big = max(big, sm.tab[1][w]);
        }
        if (big > 64)
            return false;  // uniform: every thread read the same maximum
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int bkt = tid * PB + j;
            if (bkt < nb) {
                sm.bk.off[bkt] = (uint32_t)before;
                sm.bk.fill[bkt] = (uint32_t)before;
            }
            before += (int)v[j];
        }
    }
    __syncthreads();
    // scatter into buffer 1 by bucket (order inside a bucket arbitrary), as
    // composite keys (order key, complemented column): one 64-bit compare
    // then decides the rank order
    uint64_t *ck = reinterpret_cast<uint64_t *>(&sm.word[1][0]);  // word[1], wcol[0..1] region
    static_assert(sizeof(sm.word[1]) + sizeof(sm.wcol) >= KM * 8, "composite key buffer");
    uint64_t mine[S::EPT];
    int mbkt[S::EPT];
#pragma unroll
    for (int r = 0; r < S::EPT; ++r) {
        const int i = r * NT + tid;
        mine[r] = 0ull;
        mbkt[r] = 0;
        if (i < m) {
            const uint32_t key = sm.word[0][i];
            mine[r] = ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - sm.wcol[0][i]);
            mbkt[r] = nb - 1 - (int)((key >> shift) & dmask);
        }
    }
    __syncthreads();  // buffer 0's columns are read before the region is reused
#pragma unroll
    for (int r = 0; r < S::EPT; ++r)
        if (r * NT + tid < m)
            ck[atomicAdd(&sm.bk.fill[mbkt[r]], 1u)] = mine[r];
    __syncthreads();
    // place each winner inside its bucket: rank = members with a larger key
#pragma unroll
    for (int r = 0; r < S::EPT; ++r) {
        if (r * NT + tid < m) {
            const int b0 = (int)sm.bk.off[mbkt[r]], b1 = (int)sm.bk.fill[mbkt[r]];
            int rank = 0;
            for (int j = b0; j < b1; ++j)
                rank += ck[j] > mine[r];
            sm.word[0][b0 + rank] = (uint32_t)(mine[r] >> 32);
            // columns go to buffer 0's column array only after every rank is
            // known (it overlaps the composite keys)
            mbkt[r] = b0 + rank;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < S::EPT; ++r)
        if (r * NT + tid < m)
            sm.wcol[0][mbkt[r]] = 0xffffffffu - (uint32_t)mine[r];
    __syncthreads();
    return true;
}

// Stable LSD radix sort of the m winners (sm.word / sm.wcol buffer 0) by
// descending order key; returns the buffer that holds the result.
template <int NT, int CAP, int KM, int NBK>
__device__ int sort32(Topk32Smem<NT, CAP, KM, NBK> &sm, int m, uint32_t wmin, uint32_t wmax)
{
    using S = Topk32Smem<NT, CAP, KM, NBK>;
    constexpr int NW = S::NW, EPT = S::EPT, NCNT = S::NCNT;
    constexpr int PER = NCNT / NT;  // counters scanned per thread
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const uint64_t lt = (1ull << lane) - 1ull;
    const uint32_t diff = wmin ^ wmax;
    const int bits = diff ? 32 - __clz(diff) : 0;
    int src = 0;
    for (int shift = 0; shift < bits; shift += 8) {
        // zero the counters (as 32-bit words)
        for (int i = tid; i < NCNT / 2; i += NT)
            reinterpret_cast<uint32_t *>(sm.a.cnt)[i] = 0u;
        __syncthreads();
        int dig[EPT], rank[EPT];
#pragma unroll
        for (int r = 0; r < EPT; ++r) {
            const int i = r * NT + tid;
            const bool valid = i < m;
            // inverted digit: larger keys first
            const int d = valid ? 255 - (int)((sm.word[src][i] >> shift) & 255u) : 0;
            uint64_t same = __ballot(valid);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const uint64_t bal = __ballot((d >> b) & 1);
                same &= ((d >> b) & 1) ? bal : ~bal;
            }
            dig[r] = d;
            rank[r] = __popcll(same & lt);
            // the highest lane of each digit group records the group size
            if (valid && (same >> lane) == 1ull)
                sm.a.cnt[(d * EPT + r) * NW + wid] = (uint16_t)__popcll(same);
        }
        __syncthreads();
        // exclusive scan over (digit, round, wave): thread t owns PER
        // consecutive counters
        {
            uint32_t v[PER];
            int s = 0;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                v[j] = sm.a.cnt[tid * PER + j];
                s += (int)v[j];
            }
            const int incl = wave_inclusive_scan(s);
            if (lane == 63)
                sm.red[0][0][wid] = incl;
            __syncthreads();
            int before = incl - s;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                before += w < wid ? sm.red[0][0][w] : 0;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                sm.a.cnt[tid * PER + j] = (uint16_t)before;
                before += (int)v[j];
            }
        }
        __syncthreads();
        // scatter
#pragma unroll
        for (int r = 0; r < EPT; ++r) {
            const int i = r * NT + tid;
            if (i < m) {
                const int pos = (int)sm.a.cnt[(dig[r] * EPT + r) * NW + wid] + rank[r];
                sm.word[src ^ 1][pos] = sm.word[src][i];
                sm.wcol[src ^ 1][pos] = sm.wcol[src][i];
            }
        }
        __syncthreads();
        src ^= 1;
    }
    return src;
}

// Sorted top-k of the n order keys cached in sm (column lo + i for key i):
// 32-bit select, compaction, bucket sort (stable radix sort for ties and
// crowded buckets).  Returns m = min(k, n); the winners' columns in rank
// order are sm.wcol[buf][0 .. m).
template <int NT, int CAP, int KM, int NBK>
__device__ int topk_sort_cached(Topk32Smem<NT, CAP, KM, NBK> &sm, int n, int lo, int k,
                                uint32_t omin, uint32_t omax, int &buf)
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

// Ranks s0 .. s1-1 (0 <= s0 < s1 <= min(k, n)) of the top-k of the row
// rp[0 .. n), whose key i is column lo + i: emit(rank, column) is called once
// for each of them, from whichever thread places it.  Block-wide (all threads
// call it; it returns with the shared memory free for reuse after a barrier).
// The row is counted into NB buckets linear in the score value over
// [min, max] (a monotonic map, so a higher bucket never holds a lower-ranked
// key); the prefix sums give each bucket's first rank.  Only the buckets that
// hold ranks s0 .. s1-1 are collected, and each collected key is placed
// inside its bucket by counting the members with a larger composite key
// (order key, then smaller column) -- the exact rank order, ties included.
// Nothing selects, compacts or sorts the whole row.  When the ranks fall into
// crowded buckets (a score range stretched by outliers) or the value range is
// not finite, the full sorted top-k of the row is taken instead.
template <int NT, int CAP, int KM, int NBK, typename Emit>
__device__ void seg_rank_row(Topk32Smem<NT, CAP, KM, NBK> &sm, const float *__restrict__ rp, int lo,
                             int n, int k, int s0, int s1, Emit emit)
{
    using S = Topk32Smem<NT, CAP, KM, NBK>;
    constexpr int NB = S::NB, NW = S::NW, PB = NB / NT, R = CAP / NT;
    static_assert(PB >= 1 && NB % NT == 0, "every thread owns whole buckets");
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int rounds = (n + NT - 1) / NT;  // uniform, at most R
    // thread t keeps keys r*NT + t (r < rounds) in registers: their order keys
    // and, below, their buckets (all loads issued before any is used)
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
    if (omin == omax) {  // every key equal: column order is the rank order
        for (int i = s0 + tid; i < s1; i += NT)
            emit(i, lo + i);
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
        // a bucket strictly between them holds only ranks s0 .. s1-1 (all of
        // which are placed anyway); the two end buckets can hold many keys
        // outside them (ties, or a range stretched by an outlier), and
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
        // the collection buffer holds k plus the rest of the last bucket
        constexpr int kCollect = (int)((sizeof(sm.word[1]) + sizeof(sm.wcol)) / 8);
        ok = crowd <= kSegMaxBucket && total <= kCollect;
        if (ok) {
            // the collection from registers (key of rank base + i at ck[i])
            uint64_t *ck = reinterpret_cast<uint64_t *>(&sm.word[1][0]);
            static_assert(kCollect >= KM + kSegMaxBucket, "composite key buffer");
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
                    emit(r, (int)(0xffffffffu - (uint32_t)key));
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
        emit(i, (int)sm.wcol[buf][i]);
}

} // namespace dsa
