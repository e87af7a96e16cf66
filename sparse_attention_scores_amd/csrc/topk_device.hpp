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
