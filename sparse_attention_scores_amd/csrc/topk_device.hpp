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

template <int NT, int CAP>
struct TopkSmem {
    uint32_t ord[CAP];          // order keys of the row (source = scores)
    uint64_t sel[kTopkMaxK];    // winners
    uint32_t hist[256];
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
        for (int i = tid; i < 256; i += NT)
            sm.hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
            const uint64_t key = key_at(i);
            if ((key & mask) == prefix)
                atomicAdd(&sm.hist[(uint32_t)(key >> shift) & dmask], 1u);
        }
        __syncthreads();
        if (wid == 0) {
            // lane j owns bins 255-4j .. 252-4j (descending)
            int c[4];
            int s = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                c[t] = (int)sm.hist[255 - 4 * lane - t];
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
    // ---- compaction: exactly k keys satisfy (key & mask) >= prefix
    if (tid == 0)
        sm.count = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
        const uint64_t key = key_at(i);
        if ((key & mask) >= prefix) {
            const int pos = atomicAdd(&sm.count, 1);
            if (pos < kTopkMaxK)
                sm.sel[pos] = key;
        }
    }
    __syncthreads();
}

// Descending bitonic sort of sm.sel[0..m), padded with zeros (smaller than
// every real key) to a power of two.
template <int NT, int CAP>
__device__ void bitonic_desc(TopkSmem<NT, CAP> &sm, int m)
{
    const int tid = threadIdx.x;
    int P = 1;
    while (P < m)
        P <<= 1;
    if (P < 2)
        P = 2;
    for (int i = m + tid; i < P; i += NT)
        sm.sel[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < P / 2; t += NT) {
                const int i = 2 * t - (t & (stride - 1));
                const int j = i + stride;
                const uint64_t a = sm.sel[i], b = sm.sel[j];
                const bool desc = (i & size) == 0;
                if (desc ? (a < b) : (a > b)) {
                    sm.sel[i] = b;
                    sm.sel[j] = a;
                }
            }
            __syncthreads();
        }
    }
}

// Load scores[lo, hi) of one row into sm.ord and return n.
template <int NT, int CAP>
__device__ int load_row(TopkSmem<NT, CAP> &sm, const float *__restrict__ row, int lo, int hi)
{
    const int n = max(hi - lo, 0);
    for (int i = threadIdx.x; i < n; i += NT)
        sm.ord[i] = score_order_key(row[lo + i]);
    __syncthreads();
    return n;
}

} // namespace dsa
