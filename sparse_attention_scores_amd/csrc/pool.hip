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
// the visible tail, then INVALID to out_width.  The pools' 64-bit composite
// keys are selected by radix passes and ordered by a bitonic sort.
template <int NT, int CAP, int EPT>
__global__ __launch_bounds__(NT) void pool_select_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ pad,
    const int32_t *__restrict__ q_pos, int32_t *__restrict__ out_tok,
    int32_t *__restrict__ out_pools, int n_q, int np_cols, int kpool, int select_k,
    int out_width)
{
    __shared__ TopkSmem<NT, CAP> sm;
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int b = row / n_q;
    const int p = pad[b];
    const int t = q_pos[row];
    const int n_full = t >= p ? min((t - p + 1) / kpool, np_cols) : 0;
    const int n = load_row(sm, scores + (int64_t)row * np_cols, 0, n_full);
    auto key_at = [&](int i) -> uint64_t { return compose_key(sm.ord[i], (uint32_t)i); };
    int m;
    if (n > select_k) {
        radix_select(sm, n, select_k, key_at);
        m = select_k;
    } else {
        for (int i = tid; i < n; i += NT)
            sm.sel[i] = key_at(i);
        __syncthreads();
        m = n;
    }
    {
        uint64_t v[EPT];
        bitonic_sort_regs<NT, EPT>(sm, m, v);
#pragma unroll
        for (int b = 0; b < EPT; ++b)
            sm.sel[tid * EPT + b] = v[b];
        __syncthreads();
    }
    // expand_selection: pools' tokens (rank order), the visible tail, INVALID
    const int pool_toks = m * kpool;
    const int tail = t >= p ? (t + 1) - (p + n_full * kpool) : 0;
    int32_t *o = out_tok + (int64_t)row * out_width;
    for (int i = tid; i < out_width; i += NT) {
        int v = -1;
        if (i < pool_toks) {
            const int pool = (int)(0xffffffffu - (uint32_t)sm.sel[i / kpool]);
            v = p + pool * kpool + i % kpool;
        } else if (i < pool_toks + tail) {
            v = p + n_full * kpool + (i - pool_toks);
        }
        o[i] = v;
    }
    if (out_pools) {
        int32_t *op = out_pools + (int64_t)row * select_k;
        for (int i = tid; i < select_k; i += NT)
            op[i] = i < m ? (int32_t)(0xffffffffu - (uint32_t)sm.sel[i]) : -1;
    }
}

hipError_t launch_pool_select(const PoolSelectArgs &a, hipStream_t st)
{
    const int np_cols = a.seq / a.kpool;
    const unsigned rows = (unsigned)(a.batch * a.n_q);
#define DSA_POOL_SELECT(NT, CAP, EPT)                                                              \
    hipLaunchKernelGGL((pool_select_kernel<NT, CAP, EPT>), dim3(rows), dim3(NT), 0, st, a.scores,  \
                       a.pad, a.q_pos, a.out_tok, a.out_pools, a.n_q, np_cols, a.kpool,            \
                       a.select_k, a.out_width)
    if (np_cols <= 4096) {
        if (a.select_k <= 512)
            DSA_POOL_SELECT(256, 4096, 2);
        else
            DSA_POOL_SELECT(256, 4096, 8);
    } else {
        DSA_POOL_SELECT(1024, 16384, 2);
    }
#undef DSA_POOL_SELECT
    return hipGetLastError();
}

} // namespace dsa
