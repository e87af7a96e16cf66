// cache_write.hip -- Walsh-Hadamard rotation of indexer rows and the
// indexer-key cache write ("Another DSA attempt", ik_llama.cpp PR #2063: the
// commit message of the decode indexer-K cache -- the batch's indexer keys
// are Hadamard-rotated, which leaves the scores unchanged, and written into
// the per-layer key cache at kv_head; the queries get the same rotation --
// and the serving-correctness commit: the Sylvester construction, H
// symmetric and orthonormal).
//
// y = H_d x / sqrt(d) with H_d the Sylvester Hadamard matrix, H[i][j] =
// (-1)^popcount(i & j).  One wave per row: the fast Walsh-Hadamard transform
// in f64 (butterflies (a + b, a - b) at strides 1, 2, ..., d/2; strides
// below 64 pair lanes with a shuffle, larger ones pair a lane's own
// elements), one multiplication by the f64 constant 1/sqrt(d), then one
// rounding to f32.  For bf16 or f32 inputs of moderate range the f64 sums
// are exact, so y_f32 is the correctly rounded rotation.  The cache stores
// e4m3 codes of y / s with s = max|y| / 448 per row (f32 division), or y in
// bf16.
#include "dsa_device.hpp"
#include "dsa_internal.hpp"

#include <math.h>

namespace dsa {

// Row r of x (bf16 bits or f32) rotated: lane l holds elements e*64 + l
// (e < E) of the row; lanes at or past d hold nothing (d = 32).
template <int D>
struct HadamardRow {
    static constexpr int E = D >= 64 ? D / 64 : 1;  // elements per lane
};

template <int D>
__device__ __forceinline__ void hadamard_load_rotate(const void *x, bool x_f32, int64_t row,
                                                     int lane, float (&y)[HadamardRow<D>::E])
{
    constexpr int E = HadamardRow<D>::E;
    double v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int j = e * 64 + lane;
        double t = 0.0;
        if (j < D) {
            if (x_f32)
                t = (double)static_cast<const float *>(x)[row * D + j];
            else
                t = (double)bf16_bits_to_f32(static_cast<const uint16_t *>(x)[row * D + j]);
        }
        v[e] = t;
    }
    // strides inside a lane's own elements (h >= 64)
#pragma unroll
    for (int h = 64; h < D; h *= 2) {
        const int he = h / 64;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if ((e & he) == 0) {
                const double a = v[e], b = v[e + he];
                v[e] = a + b;
                v[e + he] = a - b;
            }
        }
    }
    // strides across lanes (h < 64): the lower lane of a pair keeps a + b,
    // the upper one a - b
#pragma unroll
    for (int h = 1; h < (D < 64 ? D : 64); h *= 2) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const double o = __shfl_xor(v[e], h, kWave);
            v[e] = (lane & h) ? o - v[e] : v[e] + o;
        }
    }
    const double c = 1.0 / sqrt((double)D);
#pragma unroll
    for (int e = 0; e < E; ++e)
        y[e] = (float)(v[e] * c);
}

// Rotation only (queries): out = y as f32 or bf16 (round to nearest even
// from the f32 value).  Four rows per block, one per wave.
template <int D>
__global__ __launch_bounds__(256) void hadamard_rotate_kernel(const void *x, bool x_f32, void *out,
                                                              bool out_f32, int64_t rows)
{
    constexpr int E = HadamardRow<D>::E;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    float y[E];
    hadamard_load_rotate<D>(x, x_f32, row, lane, y);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int j = e * 64 + lane;
        if (j < D) {
            if (out_f32)
                static_cast<float *>(out)[row * D + j] = y[e];
            else
                static_cast<uint16_t *>(out)[row * D + j] = (uint16_t)f32_to_bf16_bits(y[e]);
        }
    }
}

// Cache write: row (b, i) of k_new goes to cache row kv_head[b] + i of
// sequence b when that row is inside [0, n_cache); fp8 codes plus the row's
// scale, or bf16.
template <int D>
__global__ __launch_bounds__(256) void index_cache_write_kernel(
    const void *k_new, bool k_f32, const int32_t *__restrict__ kv_head, int n_new, int n_cache,
    int64_t rows, void *cache, bool fp8, float *__restrict__ scales)
{
    constexpr int E = HadamardRow<D>::E;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int64_t b = row / n_new;
    const int i = (int)(row % n_new);
    const int r = kv_head[b] + i;
    if (r < 0 || r >= n_cache)
        return;
    float y[E];
    hadamard_load_rotate<D>(k_new, k_f32, row, lane, y);
    const int64_t dst = (b * n_cache + r) * D;
    if (!fp8) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = e * 64 + lane;
            if (j < D)
                static_cast<uint16_t *>(cache)[dst + j] = (uint16_t)f32_to_bf16_bits(y[e]);
        }
        return;
    }
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e)
        mx = fmaxf(mx, fabsf(y[e]));  // idle lanes hold 0
    mx = wave_max(mx);
    const float s = mx > 0.f ? mx / 448.0f : 1.0f;
    if (lane == 0)
        scales[b * n_cache + r] = s;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int j = e * 64 + lane;
        if (j < D) {
            const float q = y[e] / s;
            // v_cvt_pk_fp8_f32: OCP e4m3 on gfx950, round to nearest even
            const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false);
            static_cast<uint8_t *>(cache)[dst + j] = (uint8_t)(packed & 0xff);
        }
    }
}

template <int D>
static hipError_t launch_rotate_d(const void *x, bool x_f32, void *out, bool out_f32,
                                  int64_t rows, hipStream_t st)
{
    const int64_t blocks = (rows + 3) / 4;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(hadamard_rotate_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st, x,
                       x_f32, out, out_f32, rows);
    return hipGetLastError();
}

hipError_t launch_hadamard_rotate(const void *x, bool x_f32, void *out, bool out_f32, int64_t rows,
                                  int d, hipStream_t st)
{
    switch (d) {
    case 32: return launch_rotate_d<32>(x, x_f32, out, out_f32, rows, st);
    case 64: return launch_rotate_d<64>(x, x_f32, out, out_f32, rows, st);
    case 128: return launch_rotate_d<128>(x, x_f32, out, out_f32, rows, st);
    case 256: return launch_rotate_d<256>(x, x_f32, out, out_f32, rows, st);
    default: return hipErrorInvalidValue;
    }
}

template <int D>
static hipError_t launch_cache_d(const CacheWriteArgs &a, hipStream_t st)
{
    const int64_t rows = (int64_t)a.batch * a.n_new;
    const int64_t blocks = (rows + 3) / 4;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(index_cache_write_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st,
                       a.k_new, a.k_f32, a.kv_head, a.n_new, a.n_cache, rows, a.cache, a.fp8,
                       a.scales);
    return hipGetLastError();
}

hipError_t launch_index_cache_write(const CacheWriteArgs &a, hipStream_t st)
{
    switch (a.head_dim) {
    case 32: return launch_cache_d<32>(a, st);
    case 64: return launch_cache_d<64>(a, st);
    case 128: return launch_cache_d<128>(a, st);
    case 256: return launch_cache_d<256>(a, st);
    default: return hipErrorInvalidValue;
    }
}

} // namespace dsa
