// pool.hip -- visibility ranges, pooled indexer keys and pool selection.
//
// "Module glm5next_dsa_ref": visible (causal and not padding); pool_states
// (pooling starts at the first valid token, softmax over the slot axis for
// each channel, a trailing partial pool is not a pool); kept_pools;
// topk_pools (higher score, then smaller pool index) and expand_selection
// (pools' tokens in rank order, then the visible tail, INVALID up to
// out_width, padded query rows all INVALID).
#include "dsa_internal.hpp"
#include "topk_device.hpp"

#include <math.h>

namespace dsa {

// ------------------------------------------------------------------ ranges
// Token keys: [pad, q_pos + 1).  Pools (kpool > 0): [0, n_full) with
// n_full = floor((q_pos - pad + 1) / kpool), the pools all of whose tokens
// are visible.  A padded query gets [0, 0).
__global__ void visibility_ranges_kernel(const int32_t *__restrict__ pad,
                                         const int32_t *__restrict__ q_pos, int32_t *lo,
                                         int32_t *hi, int n_q, int kpool, int total)
{
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total)
        return;
    const int p = pad[e / n_q];
    const int t = q_pos[e];
    if (t < p) {
        lo[e] = 0;
        hi[e] = 0;
    } else if (kpool > 0) {
        lo[e] = 0;
        hi[e] = (t - p + 1) / kpool;
    } else {
        lo[e] = p;
        hi[e] = t + 1;
    }
}

hipError_t launch_visibility_ranges(const RangeArgs &a, hipStream_t st)
{
    const int total = a.batch * a.n_q;
    hipLaunchKernelGGL(visibility_ranges_kernel, dim3((total + 255) / 256), dim3(256), 0, st,
                       a.pad, a.q_pos, a.lo, a.hi, a.n_q, a.kpool, total);
    return hipGetLastError();
}

// ------------------------------------------------------------------ pool keys
template <typename T>
__device__ __forceinline__ float pk_load(const T *p, int64_t i);
template <>
__device__ __forceinline__ float pk_load<float>(const float *p, int64_t i)
{
    return p[i];
}
template <>
__device__ __forceinline__ float pk_load<uint16_t>(const uint16_t *p, int64_t i)
{
    return bf16_bits_to_f32(p[i]);
}
__device__ __forceinline__ void pk_store(float *p, int64_t i, float v)
{
    p[i] = v;
}
__device__ __forceinline__ void pk_store(uint16_t *p, int64_t i, float v)
{
    p[i] = (uint16_t)f32_to_bf16_bits(v);
}

// One thread per (b, pool, channel); consecutive threads walk channels, so
// each slot's loads are coalesced rows of k and gate.
template <typename T>
__global__ void pool_keys_kernel(const T *__restrict__ k, const T *__restrict__ gate,
                                 const int32_t *__restrict__ pad, T *__restrict__ pooled,
                                 int32_t *__restrict__ n_pools, int seq, int kpool, int D,
                                 int np_max, int64_t total)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total)
        return;
    const int c = (int)(e % D);
    const int64_t bi = e / D;
    const int i = (int)(bi % np_max);
    const int b = (int)(bi / np_max);
    const int p = pad[b];
    const int np = seq > p ? (seq - p) / kpool : 0;
    if (i == 0 && c == 0)
        n_pools[b] = np;
    if (i >= np) {
        pk_store(pooled, e, 0.f);
        return;
    }
    const int64_t base = ((int64_t)b * seq + p + (int64_t)i * kpool) * D + c;
    float m = -INFINITY;
    for (int j = 0; j < kpool; ++j)
        m = fmaxf(m, pk_load(gate, base + (int64_t)j * D));
    float num = 0.f, den = 0.f;
    for (int j = 0; j < kpool; ++j) {
        const float ej = expf(pk_load(gate, base + (int64_t)j * D) - m);
        num = fmaf(ej, pk_load(k, base + (int64_t)j * D), num);
        den += ej;
    }
    pk_store(pooled, e, num / den);
}

// The same per channel, V = 16 / sizeof(T) channels per thread, each slot
// row read as one 16-byte load per thread (D a multiple of V, 16-byte
// aligned rows); the arithmetic per channel is that of pool_keys_kernel.
// With KR > 0 and kpool <= KR the pool's k and gate rows are all loaded
// before any is used and held in registers; otherwise they are read slot by
// slot (the gate rows twice).
template <typename T, int KR>
__global__ void pool_keys_vec_kernel(const T *__restrict__ k, const T *__restrict__ gate,
                                     const int32_t *__restrict__ pad, T *__restrict__ pooled,
                                     int32_t *__restrict__ n_pools, int seq, int kpool, int D,
                                     int np_max, int64_t total)
{
    constexpr int V = 16 / (int)sizeof(T);
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total)
        return;
    const int dv = D / V;
    const int cv = (int)(e % dv);
    const int64_t bi = e / dv;
    const int i = (int)(bi % np_max);
    const int b = (int)(bi / np_max);
    const int p = pad[b];
    const int np = seq > p ? (seq - p) / kpool : 0;
    if (i == 0 && cv == 0)
        n_pools[b] = np;
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(pooled + bi * D) + cv;
    if (i >= np) {
        *dst = u32x4_t{0u, 0u, 0u, 0u};
        return;
    }
    const int64_t base = ((int64_t)b * seq + p + (int64_t)i * kpool) * D + (int64_t)cv * V;
    auto row = [&](const T *src, int j, float (&x)[V]) {
        const u32x4_t r = *reinterpret_cast<const u32x4_t *>(src + base + (int64_t)j * D);
        const T *t = reinterpret_cast<const T *>(&r);
#pragma unroll
        for (int c = 0; c < V; ++c)
            x[c] = pk_load(t, c);
    };
    float m[V], x[V], y[V], num[V], den[V];
#pragma unroll
    for (int c = 0; c < V; ++c) {
        m[c] = -INFINITY;
        num[c] = 0.f;
        den[c] = 0.f;
    }
    if constexpr (KR > 0) {
        u32x4_t gr[KR], kr[KR];
#pragma unroll
        for (int j = 0; j < KR; ++j) {
            if (j < kpool) {
                gr[j] = *reinterpret_cast<const u32x4_t *>(gate + base + (int64_t)j * D);
                kr[j] = *reinterpret_cast<const u32x4_t *>(k + base + (int64_t)j * D);
            }
        }
        auto unpack = [&](const u32x4_t &r, float(&xo)[V]) {
            const T *t = reinterpret_cast<const T *>(&r);
#pragma unroll
            for (int c = 0; c < V; ++c)
                xo[c] = pk_load(t, c);
        };
#pragma unroll
        for (int j = 0; j < KR; ++j) {
            if (j < kpool) {
                unpack(gr[j], x);
#pragma unroll
                for (int c = 0; c < V; ++c)
                    m[c] = fmaxf(m[c], x[c]);
            }
        }
#pragma unroll
        for (int j = 0; j < KR; ++j) {
            if (j < kpool) {
                unpack(gr[j], x);
                unpack(kr[j], y);
#pragma unroll
                for (int c = 0; c < V; ++c) {
                    const float ej = expf(x[c] - m[c]);
                    num[c] = fmaf(ej, y[c], num[c]);
                    den[c] += ej;
                }
            }
        }
    } else {
        for (int j = 0; j < kpool; ++j) {
            row(gate, j, x);
#pragma unroll
            for (int c = 0; c < V; ++c)
                m[c] = fmaxf(m[c], x[c]);
        }
        for (int j = 0; j < kpool; ++j) {
            row(gate, j, x);
            row(k, j, y);
#pragma unroll
            for (int c = 0; c < V; ++c) {
                const float ej = expf(x[c] - m[c]);
                num[c] = fmaf(ej, y[c], num[c]);
                den[c] += ej;
            }
        }
    }
    u32x4_t o;
    T *ot = reinterpret_cast<T *>(&o);
#pragma unroll
    for (int c = 0; c < V; ++c)
        pk_store(ot, c, num[c] / den[c]);
    *dst = o;
}

__global__ void pool_counts_kernel(const int32_t *__restrict__ pad, int32_t *__restrict__ n_pools,
                                   int seq, int kpool, int batch)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < batch)
        n_pools[b] = seq > pad[b] ? (seq - pad[b]) / kpool : 0;
}

hipError_t launch_pool_keys(const PoolKeysArgs &a, hipStream_t st)
{
    const int np_max = a.seq / a.kpool;
    const int64_t total = (int64_t)a.batch * np_max * a.head_dim;
    if (total == 0) {
        // no pool rows at all: only the (zero) counts
        hipLaunchKernelGGL(pool_counts_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, st,
                           a.pad, a.n_pools, a.seq, a.kpool, a.batch);
        return hipGetLastError();
    }
    const int V = a.f32 ? 4 : 8;  // channels per 16-byte load
    const bool vec = a.head_dim % V == 0 &&
                     ((reinterpret_cast<uintptr_t>(a.k) | reinterpret_cast<uintptr_t>(a.gate) |
                       reinterpret_cast<uintptr_t>(a.pooled)) & 15) == 0;
    if (vec) {
        const int64_t tv = total / (int64_t)V;
        const unsigned vb = (unsigned)((tv + 255) / 256);
#define DSA_POOL_KEYS_VEC(T, KR)                                                                   \
    hipLaunchKernelGGL((pool_keys_vec_kernel<T, KR>), dim3(vb), dim3(256), 0, st,                  \
                       static_cast<const T *>(a.k), static_cast<const T *>(a.gate), a.pad,         \
                       static_cast<T *>(a.pooled), a.n_pools, a.seq, a.kpool, a.head_dim, np_max,  \
                       tv)
        // up to 8 slots per pool: every row of the pool in registers at once
        if (a.f32) {
            if (a.kpool <= 8)
                DSA_POOL_KEYS_VEC(float, 8);
            else
                DSA_POOL_KEYS_VEC(float, 0);
        } else {
            if (a.kpool <= 8)
                DSA_POOL_KEYS_VEC(uint16_t, 8);
            else
                DSA_POOL_KEYS_VEC(uint16_t, 0);
        }
#undef DSA_POOL_KEYS_VEC
        return hipGetLastError();
    }
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (a.f32)
        hipLaunchKernelGGL(pool_keys_kernel<float>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const float *>(a.k), static_cast<const float *>(a.gate),
                           a.pad, static_cast<float *>(a.pooled), a.n_pools, a.seq, a.kpool,
                           a.head_dim, np_max, total);
    else
        hipLaunchKernelGGL(pool_keys_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint16_t *>(a.k),
                           static_cast<const uint16_t *>(a.gate), a.pad,
                           static_cast<uint16_t *>(a.pooled), a.n_pools, a.seq, a.kpool,
                           a.head_dim, np_max, total);
    return hipGetLastError();
}

// ------------------------------------------------------------------ pool select
// topk_pools + expand_selection ("Module glm5next_dsa_ref"): the top
// select_k visible pools of each query in rank order (higher pooled score,
// then smaller pool id), each expanded to its kpool token ids ascending, then
// the visible tail, then INVALID to out_width.  `parts` blocks per query row
// (one when there are many rows), block `seg` placing ranks
// [seg*seg_len, seg*seg_len + seg_len); the pools are ranked with value
// buckets (seg_rank_row), and each ranked pool writes its own kpool token
// ids, so the selection is never sorted as a list.
template <int NT, int CAP, int KM, int NBK>
__global__ __launch_bounds__(NT) void pool_select_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ pad,
    const int32_t *__restrict__ q_pos, int32_t *__restrict__ out_tok,
    int32_t *__restrict__ out_pools, int n_q, int np_cols, int kpool, int select_k,
    int out_width, int parts, int seg_len)
{
    __shared__ Topk32Smem<NT, CAP, KM, NBK> sm;
    const int tid = threadIdx.x;
    const int row = blockIdx.x / parts;
    const int seg = blockIdx.x - row * parts;
    const int b = row / n_q;
    const int p = pad[b];
    const int t = q_pos[row];
    const int n_full = t >= p ? min((t - p + 1) / kpool, np_cols) : 0;
    const int m = min(select_k, n_full);
    int32_t *o = out_tok + (int64_t)row * out_width;
    int32_t *op = out_pools ? out_pools + (int64_t)row * select_k : nullptr;
    // four tokens per pool as one 16-byte store where the row allows it
    const bool quad = kpool == 4 && (reinterpret_cast<uintptr_t>(o) & 15) == 0;
    const int p0 = seg * seg_len, p1 = min(p0 + seg_len, select_k);
    if (p0 < min(p1, m))
        seg_rank_row(sm, scores + (int64_t)row * np_cols, 0, n_full, select_k, p0, min(p1, m),
                     [&](int r, int pool) {
                         const int tok = p + pool * kpool;
                         if (quad) {
                             *reinterpret_cast<int4 *>(o + 4 * r) =
                                 make_int4(tok, tok + 1, tok + 2, tok + 3);
                         } else {
                             for (int j = 0; j < kpool; ++j)
                                 o[r * kpool + j] = tok + j;
                         }
                         if (op)
                             op[r] = pool;
                     });
    // the visible tail after the pools' tokens, then INVALID (the row's
    // blocks share these positions)
    const int pool_toks = m * kpool;
    const int tail = t >= p ? (t + 1) - (p + n_full * kpool) : 0;
    for (int i = pool_toks + seg * NT + tid; i < out_width; i += parts * NT)
        o[i] = i < pool_toks + tail ? p + n_full * kpool + (i - pool_toks) : -1;
    if (op)
        for (int i = max(p0, m) + tid; i < p1; i += NT)
            op[i] = -1;
}

hipError_t launch_pool_select(const PoolSelectArgs &a, hipStream_t st)
{
    const int np_cols = a.seq / a.kpool;
    const int rows = a.batch * a.n_q;
    // few rows (decode): several blocks per row, each placing a segment of
    // the ranks, so that the launch still spreads over the chip
    const int parts = topk_seg_parts(rows, a.select_k, 16);
    const int seg_len = (a.select_k + parts - 1) / parts;
    const unsigned blocks = (unsigned)((int64_t)rows * parts);
#define DSA_POOL_SELECT(NT, CAP, KM, NBK)                                                         \
    hipLaunchKernelGGL((pool_select_kernel<NT, CAP, KM, NBK>), dim3(blocks), dim3(NT), 0, st,      \
                       a.scores, a.pad, a.q_pos, a.out_tok, a.out_pools, a.n_q, np_cols, a.kpool,  \
                       a.select_k, a.out_width, parts, seg_len)
    static_assert(kPoolSelectMaxPools <= 16384, "one block caches a row of pools");
    // up to 512 pools selected: winner arrays for 512 and 1024 buckets take
    // 33 KB of LDS, so four blocks share a CU instead of two
    if (np_cols <= 4096 && a.select_k <= 512)
        DSA_POOL_SELECT(512, 4096, 512, 1024);
    else if (np_cols <= 4096)
        DSA_POOL_SELECT(512, 4096, kTopkMaxK, 2048);
    else
        DSA_POOL_SELECT(1024, 16384, kTopkMaxK, 2048);
#undef DSA_POOL_SELECT
    return hipGetLastError();
}

} // namespace dsa
