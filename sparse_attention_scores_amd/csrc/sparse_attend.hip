// sparse_attend.hip -- sparse attention over each query's selected keys.
//
// out[h] = sum_{j in J} softmax_j(scale * q_h . K_j) V_j over the set J of
// distinct, in-range, non-INVALID, visible indices of the query's row
// ("GLM-5.2: the DSA sparse attention moves onto the pure fak kernel",
// table under "What changed"; "Module glm5next_dsa_ref", topk_to_mask and
// mla_masked_attention).
//
// Set semantics without a separate pass: each block inserts the row's valid
// indices into an LDS bitmap over the n_k keys (duplicates collapse there),
// takes a popcount prefix sum, and reads its share of the set bits back in
// ascending key order.  The keys are therefore processed in a fixed order
// (deterministic results) and the gathers walk memory upwards.
//
// Gather kernel (absorbed MLA: one 576-wide latent row per key, shared by
// all 64 heads, V = its first 512 columns):
//  * block = 4 waves x 16 heads of one query, over a contiguous share of the
//    query's selected keys (split-K across blocks when there are few
//    queries, merged by a combine kernel);
//  * per tile of 32 keys the rows are gathered once into LDS (row-major for
//    Q.K^T, transposed for P.V) with 16-byte coalesced loads, and reused by
//    all 4 waves (64 heads);
//  * S^T = K Q^T on 16x16x32 bf16 MFMA with Q held in registers; online
//    softmax in f32 (exp2, log2e folded into the scale);
//  * O^T += V^T P^T on MFMA, with P entering as a two-term bf16 split
//    (hi + lo, about 16 significant bits) so the rounding of the weights
//    stays far below the tolerance; each lane's accumulators all belong to
//    one head, so the softmax rescale needs no cross-lane traffic.
#include "dsa_device.hpp"
#include "dsa_internal.hpp"

#include <float.h>
#include <math.h>

namespace dsa {

// ------------------------------------------------------------------ shared
constexpr int kBitmapMaxWords = 16384;  // n_k <= 524288

// Block-wide exclusive scan of one int per thread (blockDim.x == NT).
template <int NT>
__device__ int block_exclusive_scan(int v, int *wave_tot, int &total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63)
        wave_tot[wid] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        const int t = wave_tot[i];
        before += i < wid ? t : 0;
        tot += t;
    }
    total = tot;
    __syncthreads();
    return before + incl - v;
}

// Build the selected set of one query row in `bitmap` (words [0, nw)).
template <int NT>
__device__ void build_bitmap(uint32_t *bitmap, int nw, const int32_t *__restrict__ idx_row,
                             int n_sel, int lo, int hi)
{
    for (int i = threadIdx.x; i < nw; i += NT)
        bitmap[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n_sel; i += NT) {
        const int j = idx_row[i];
        if (j >= lo && j < hi)
            atomicOr(&bitmap[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
}

// Write the set keys with rank in [r0, r1) to list[0 .. r1-r0), ascending.
// Each thread owns a contiguous run of words; `before` is the number of set
// bits in earlier runs.
__device__ __forceinline__ void extract_keys(const uint32_t *bitmap, int w0, int w1, int before,
                                             int r0, int r1, int32_t *list)
{
    int rank = before;
    for (int wd = w0; wd < w1 && rank < r1; ++wd) {
        uint32_t bits = bitmap[wd];
        const int pc = __popc(bits);
        if (rank + pc <= r0) {
            rank += pc;
            continue;
        }
        while (bits) {
            const int bit = __ffs(bits) - 1;
            bits &= bits - 1;
            if (rank >= r0 && rank < r1)
                list[rank - r0] = wd * 32 + bit;
            ++rank;
        }
    }
}

// ------------------------------------------------------------------ gather kernel
constexpr int AB_H = 64;
constexpr int AB_KD = 576;
constexpr int AB_VD = 512;
constexpr int AB_TILE = 32;
constexpr int AB_KS = AB_KD / 32;             // 18 k-steps of the 16x16x32 MFMA
constexpr int AB_NC = AB_VD / 16;             // 32 output column tiles per wave
constexpr int AB_ROWB = AB_KD * 2;            // 1152 bytes per latent row
constexpr int AB_TILEB = AB_TILE * AB_ROWB;   // 36 KB per tile (36 DMA instructions)
constexpr int AB_LIST = 1024;                 // keys per batch of a block
constexpr int AB_NT = 256;

// LDS tile: 32 latent rows, 1152 bytes apart, with the 16-byte chunks of row
// r stored XOR-swizzled (chunk_swz) so that both the row-wise Q.K^T operand
// reads and the transposing P.V operand reads spread over all banks.  V is
// the first 512 columns of the same rows.
struct __attribute__((aligned(16))) AbsSmem {
    union {
        unsigned char tile[2][AB_TILEB];
        uint32_t bitmap[kBitmapMaxWords];
    } u;
    int32_t list[AB_LIST];
    int wave_tot[AB_NT / 64];
};

__device__ __forceinline__ int ab_chunk(int row, int logical)
{
    return row * (AB_ROWB / 16) + (logical ^ chunk_swz(row));
}

__global__ __launch_bounds__(AB_NT) void attend_gather_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv, int64_t row_stride,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ vlo,
    const int32_t *__restrict__ vhi, float *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ ws_o, float *__restrict__ ws_ml, int n_q, int n_k, int n_sel,
    int splits, float scale_log2)
{
    __shared__ AbsSmem sm;
    DSA_LDS_ESCAPE(sm);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int g = lane >> 4, col = lane & 15;
    const int row = blockIdx.x / splits;
    const int split = blockIdx.x % splits;
    const int64_t b = row / n_q;

    int lo = 0, hi = n_k;
    if (vlo) {
        lo = max(vlo[row], 0);
        hi = min(vhi[row], n_k);
    }
    const int nw = (n_k + 31) >> 5;
    const int wpt = (nw + AB_NT - 1) / AB_NT;
    const int w0 = min(tid * wpt, nw), w1 = min(w0 + wpt, nw);

    // Q^T fragments (B operand): lane holds head wid*16+col, dims ks*32+g*8..+8
    const int head = wid * 16 + col;
    u32x4_t qf[AB_KS];
    {
        const uint16_t *qp = q + ((int64_t)row * AB_H + head) * AB_KD + g * 8;
#pragma unroll
        for (int ks = 0; ks < AB_KS; ++ks)
            qf[ks] = *reinterpret_cast<const u32x4_t *>(qp + ks * 32);
    }
    f32x4_t oacc[AB_NC];
#pragma unroll
    for (int n = 0; n < AB_NC; ++n)
        oacc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_part = 0.f;

    const unsigned char *kvb =
        reinterpret_cast<const unsigned char *>(kv) + b * (int64_t)n_k * row_stride * 2;

    // DMA one tile: 36 wave instructions of 1 KB; lane slot p of instruction
    // s is LDS byte s*1024 + 16*lane = (row, physical chunk) -> its logical
    // chunk of that row's key.
    auto dma_tile = [&](unsigned char *dst, int t0, int nvalid) {
        for (int s = wid; s < AB_TILEB / 1024; s += AB_NT / 64) {
            const int c = s * 64 + lane;            // physical chunk index in the tile
            const int r = c / (AB_ROWB / 16);
            const int logical = (c % (AB_ROWB / 16)) ^ chunk_swz(r);
            const int key = sm.list[t0 + min(r, nvalid - 1)];
            lds_dma16(kvb + (int64_t)key * row_stride * 2 + logical * 16, dst + s * 1024);
        }
    };

    // The block's share of the selected set is ranks [r0, r1) in ascending
    // key order, read out in batches of AB_LIST keys.  The bitmap shares LDS
    // with the tile buffers, so each batch rebuilds it (one pass over the
    // row's n_sel indices).
    for (int batch = 0;; ++batch) {
        build_bitmap<AB_NT>(sm.u.bitmap, nw, idx + (int64_t)row * n_sel, n_sel, lo, hi);
        int cnt = 0;
        for (int wd = w0; wd < w1; ++wd)
            cnt += __popc(sm.u.bitmap[wd]);
        int total;
        const int before = block_exclusive_scan<AB_NT>(cnt, sm.wave_tot, total);
        const int r0 = (int)(((int64_t)total * split) / splits);
        const int r1 = (int)(((int64_t)total * (split + 1)) / splits);
        const int rb = r0 + batch * AB_LIST;
        if (rb >= r1)
            break;
        const int re = min(rb + AB_LIST, r1);
        extract_keys(sm.u.bitmap, w0, w1, before, rb, re, sm.list);
        __syncthreads();
        const int n_my = re - rb;
        const int ntiles = (n_my + AB_TILE - 1) / AB_TILE;

        dma_tile(sm.u.tile[0], 0, min(AB_TILE, n_my));
        for (int t = 0; t < ntiles; ++t) {
            const int t0 = t * AB_TILE;
            const int nvalid = min(AB_TILE, n_my - t0);
            // tile t has landed (own DMA) and is visible to all waves
            lds_dma_wait();
            __syncthreads();
            if (t + 1 < ntiles)
                dma_tile(sm.u.tile[(t + 1) & 1], t0 + AB_TILE, min(AB_TILE, n_my - t0 - AB_TILE));
            const unsigned char *T = sm.u.tile[t & 1];
            const u32x4_t *T16 = reinterpret_cast<const u32x4_t *>(T);

            // ---- S^T[key][head]: keys 0-15 (s0) and 16-31 (s1), two chains each
            f32x4_t s0a = {0.f, 0.f, 0.f, 0.f}, s0b = s0a, s1a = s0a, s1b = s0a;
#pragma unroll
            for (int ks = 0; ks < AB_KS; ks += 2) {
                const u32x4_t a0 = T16[ab_chunk(col, 4 * ks + g)];
                const u32x4_t a1 = T16[ab_chunk(16 + col, 4 * ks + g)];
                const u32x4_t a2 = T16[ab_chunk(col, 4 * (ks + 1) + g)];
                const u32x4_t a3 = T16[ab_chunk(16 + col, 4 * (ks + 1) + g)];
                s0a = mfma_16x16x32(a0, qf[ks], s0a);
                s1a = mfma_16x16x32(a1, qf[ks], s1a);
                s0b = mfma_16x16x32(a2, qf[ks + 1], s0b);
                s1b = mfma_16x16x32(a3, qf[ks + 1], s1b);
            }
            const f32x4_t s0 = s0a + s0b, s1 = s1a + s1b;

            // ---- online softmax (log2 domain); lane's keys: 4g+i and 16+4g+i
            float x0[4], x1[4];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x0[i] = (4 * g + i < nvalid) ? s0[i] * scale_log2 : -INFINITY;
                x1[i] = (16 + 4 * g + i < nvalid) ? s1[i] * scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, fmaxf(x0[i], x1[i]));
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
            // Lazy rescale: the reference max only moves when the tile max
            // exceeds it by more than kRescaleLog2, so p <= 2^kRescaleLog2
            // and the O accumulators are rarely touched.  Exact: l and O
            // always share the same reference.
            const bool grow = tmax > m_run + kRescaleLog2;
            if (__any(grow)) {
                const float m_new = grow ? tmax : m_run;
                // lanes that do not grow keep alpha = 1 (m_run may still be -inf
                // there, and -inf - -inf would be NaN); a growing lane with
                // m_run = -inf gets 0
                const float alpha = grow ? exp2f(m_run - m_new) : 1.f;
                if (__any(grow && m_run != -INFINITY)) {
#pragma unroll
                    for (int n = 0; n < AB_NC; ++n)
                        oacc[n] *= alpha;
                }
                l_part *= alpha;
                m_run = m_new;
            }
            // m_run is -inf only while every key seen so far (this tile
            // included) is masked; then all x are -inf and p must be 0.
            const float m_ref = (m_run == -INFINITY) ? 0.f : m_run;
            float p0[4], p1[4];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p0[i] = exp2f(x0[i] - m_ref);
                p1[i] = exp2f(x1[i] - m_ref);
                psum += p0[i] + p1[i];
            }
            l_part += psum;
            // ---- P^T fragments (B operand): element j <-> key 4g+j (j < 4),
            //      16+4g+(j-4) (j >= 4); two-term bf16 split
            u32x4_t bhi, blo;
            {
                float h0[4], h1[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h0[i] = bf16_bits_to_f32(f32_to_bf16_bits(p0[i]));
                    h1[i] = bf16_bits_to_f32(f32_to_bf16_bits(p1[i]));
                }
                bhi = u32x4_t{pack_bf16x2(h0[0], h0[1]), pack_bf16x2(h0[2], h0[3]),
                              pack_bf16x2(h1[0], h1[1]), pack_bf16x2(h1[2], h1[3])};
                blo = u32x4_t{pack_bf16x2(p0[0] - h0[0], p0[1] - h0[1]),
                              pack_bf16x2(p0[2] - h0[2], p0[3] - h0[3]),
                              pack_bf16x2(p1[0] - h1[0], p1[1] - h1[1]),
                              pack_bf16x2(p1[2] - h1[2], p1[3] - h1[3])};
            }
            // ---- O^T[c][head] += V^T[c][keys] P^T[keys][head]; the V^T
            //      fragment of column c = n*16+col is read transposed from the
            //      row-major tile: source lane col = a + 4j points at row
            //      4g + j (then 16 + 4g + j), columns n*16 + 4a .. + 3.
            {
                const int ra = 4 * g + (col >> 2);
                const int a8 = (col & 3) * 8;            // byte offset of 4 columns
#pragma unroll
                for (int n = 0; n < AB_NC; ++n) {
                    const int lc = 2 * n + (a8 >> 4);    // logical 16-byte chunk
                    const u32x2_t va = lds_read_tr16x4(T + ab_chunk(ra, lc) * 16 + (a8 & 8));
                    const u32x2_t vb =
                        lds_read_tr16x4(T + ab_chunk(16 + ra, lc) * 16 + (a8 & 8));
                    const u32x4_t av = u32x4_t{va[0], va[1], vb[0], vb[1]};
                    oacc[n] = mfma_16x16x32(av, bhi, oacc[n]);
                    oacc[n] = mfma_16x16x32(av, blo, oacc[n]);
                }
            }
        }
        __syncthreads();  // last tile consumed before the bitmap reuses LDS
    }

    // ---- epilogue: l over the 4 lane groups of the head
    float l_tot = l_part + __shfl_xor(l_part, 16, kWave);
    l_tot += __shfl_xor(l_tot, 32, kWave);
    if (splits == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *op = out + ((int64_t)row * AB_H + head) * AB_VD + 4 * g;
#pragma unroll
        for (int n = 0; n < AB_NC; ++n)
            *reinterpret_cast<f32x4_t *>(op + n * 16) = oacc[n] * inv;
        if (lse && g == 0)
            lse[(int64_t)row * AB_H + head] =
                l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
        const int64_t pr_ = ((int64_t)row * splits + split) * AB_H + head;
        float *op = ws_o + pr_ * AB_VD + 4 * g;
#pragma unroll
        for (int n = 0; n < AB_NC; ++n)
            *reinterpret_cast<f32x4_t *>(op + n * 16) = oacc[n];
        if (g == 0) {
            ws_ml[pr_ * 2] = l_tot > 0.f ? m_run : -INFINITY;
            ws_ml[pr_ * 2 + 1] = l_tot;
        }
    }
}

// Merge the split partials of each (row, head): O = sum_s 2^(m_s - m) O_s / L.
// One block per (row, head); each thread owns 4 consecutive columns.
__global__ __launch_bounds__(128) void attend_combine_kernel(const float *__restrict__ ws_o,
                                                             const float *__restrict__ ws_ml,
                                                             float *__restrict__ out,
                                                             float *__restrict__ lse, int H,
                                                             int vd, int splits)
{
    const int row = blockIdx.x / H;
    const int h = blockIdx.x % H;
    float m = -INFINITY;
    for (int s = 0; s < splits; ++s)
        m = fmaxf(m, ws_ml[(((int64_t)row * splits + s) * H + h) * 2]);
    float L = 0.f;
    for (int s = 0; s < splits; ++s) {
        const int64_t pr = ((int64_t)row * splits + s) * H + h;
        const float ms = ws_ml[pr * 2];
        L += (m == -INFINITY || ms == -INFINITY) ? 0.f : exp2f(ms - m) * ws_ml[pr * 2 + 1];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    for (int c = threadIdx.x * 4; c < vd; c += blockDim.x * 4) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < splits; ++s) {
            const int64_t pr = ((int64_t)row * splits + s) * H + h;
            const float ms = ws_ml[pr * 2];
            if (ms != -INFINITY)
                acc += exp2f(ms - m) * *reinterpret_cast<const f32x4_t *>(ws_o + pr * vd + c);
        }
        *reinterpret_cast<f32x4_t *>(out + ((int64_t)row * H + h) * vd + c) = acc * inv;
    }
    if (lse && threadIdx.x == 0)
        lse[(int64_t)row * H + h] = L > 0.f ? (m + log2f(L)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ plain kernel
// Any shape, f32 or bf16 storage, f32 arithmetic.  One block per (row, head);
// the keys are visited in ascending order, one block-wide dot product each.
template <typename T>
__device__ __forceinline__ float ld_elem(const T *p, int64_t i);
template <>
__device__ __forceinline__ float ld_elem<float>(const float *p, int64_t i)
{
    return p[i];
}
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t *p, int64_t i)
{
    return bf16_bits_to_f32(p[i]);
}

constexpr int PL_NT = 128;
constexpr int PL_MAXVD = 1024;

struct PlainSmem {
    uint32_t bitmap[kBitmapMaxWords];
    float red[PL_NT / 64];
};

template <typename T>
__global__ __launch_bounds__(PL_NT) void attend_plain_kernel(
    const T *__restrict__ q, const T *__restrict__ k, int64_t ksr, const T *__restrict__ v,
    int64_t vsr, const int32_t *__restrict__ idx, const int32_t *__restrict__ vlo,
    const int32_t *__restrict__ vhi, float *__restrict__ out, float *__restrict__ lse, int n_q,
    int n_k, int H, int kd, int vd, int kv_heads, int n_sel, float scale_log2)
{
    __shared__ PlainSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int row = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int64_t b = row / n_q;
    const int kvh = h / (H / kv_heads);
    int lo = 0, hi = n_k;
    if (vlo) {
        lo = max(vlo[row], 0);
        hi = min(vhi[row], n_k);
    }
    const int nw = (n_k + 31) >> 5;
    build_bitmap<PL_NT>(sm.bitmap, nw, idx + (int64_t)row * n_sel, n_sel, lo, hi);
    const T *qp = q + ((int64_t)row * H + h) * kd;
    float o[PL_MAXVD / PL_NT];
#pragma unroll
    for (int i = 0; i < PL_MAXVD / PL_NT; ++i)
        o[i] = 0.f;
    float m = -INFINITY, l = 0.f;
    for (int wd = 0; wd < nw; ++wd) {
        uint32_t bits = sm.bitmap[wd];
        while (bits) {
            const int j = wd * 32 + __ffs(bits) - 1;
            bits &= bits - 1;
            const T *kr = k + (b * n_k + j) * ksr + (int64_t)kvh * kd;
            float part = 0.f;
            for (int c = tid; c < kd; c += PL_NT)
                part = fmaf(ld_elem(qp, c), ld_elem(kr, c), part);
            part = wave_sum(part);
            __syncthreads();
            if (lane == 0)
                sm.red[wid] = part;
            __syncthreads();
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < PL_NT / 64; ++i)
                dot += sm.red[i];
            const float x = dot * scale_log2;
            const float m_new = fmaxf(m, x);
            const float alpha = exp2f(m - m_new);
            const float p = exp2f(x - m_new);
            l = l * alpha + p;
            m = m_new;
            const T *vr = v + (b * n_k + j) * vsr + (int64_t)kvh * vd;
#pragma unroll
            for (int i = 0; i < PL_MAXVD / PL_NT; ++i) {
                const int c = tid + i * PL_NT;
                if (c < vd)
                    o[i] = o[i] * alpha + p * ld_elem(vr, c);
            }
        }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *op = out + ((int64_t)row * H + h) * vd;
#pragma unroll
    for (int i = 0; i < PL_MAXVD / PL_NT; ++i) {
        const int c = tid + i * PL_NT;
        if (c < vd)
            op[c] = o[i] * inv;
    }
    if (lse && tid == 0)
        lse[(int64_t)row * H + h] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ host side
bool attend_gather_supported(const AttendArgs &a)
{
    return !a.f32 && a.kv_heads == 1 && a.n_heads == AB_H && a.kd == AB_KD && a.vd == AB_VD &&
           a.v == a.k && a.v_row_stride == a.k_row_stride && a.k_row_stride % 8 == 0;
}

int attend_gather_splits(const AttendArgs &a)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    int by_fill = (int)((256 + rows - 1) / rows);
    int by_work = max(1, min(a.n_sel, a.n_k) / 64);
    return max(1, min(by_fill, by_work));
}

size_t attend_workspace_bytes(const AttendArgs &a)
{
    if (attend_masked_supported(a))
        return attend_masked_workspace_bytes(a);
    if (!attend_gather_supported(a))
        return 0;
    const int s = attend_gather_splits(a);
    if (s <= 1)
        return 0;
    const int64_t rows = (int64_t)a.batch * a.n_q;
    return (size_t)rows * s * AB_H * (AB_VD + 2) * sizeof(float);
}

bool attend_plain_supported(const AttendArgs &a)
{
    return a.vd <= PL_MAXVD;
}

hipError_t launch_attend(const AttendArgs &a, hipStream_t st)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    const float scale_log2 = a.scale * kLog2e;
    if (attend_gather_supported(a)) {
        const int splits = attend_gather_splits(a);
        float *ws_o = static_cast<float *>(a.workspace);
        float *ws_ml = ws_o ? ws_o + rows * splits * AB_H * AB_VD : nullptr;
        hipLaunchKernelGGL(attend_gather_kernel, dim3((unsigned)(rows * splits)), dim3(AB_NT), 0,
                           st, static_cast<const uint16_t *>(a.q),
                           static_cast<const uint16_t *>(a.k), a.k_row_stride, a.idx, a.vis_lo,
                           a.vis_hi, a.out, a.lse, ws_o, ws_ml, a.n_q, a.n_k, a.n_sel, splits,
                           scale_log2);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || splits == 1)
            return e;
        hipLaunchKernelGGL(attend_combine_kernel, dim3((unsigned)(rows * AB_H)), dim3(128), 0, st,
                           ws_o, ws_ml, a.out, a.lse, AB_H, AB_VD, splits);
        return hipGetLastError();
    }
    if (attend_masked_supported(a))
        return launch_attend_masked(a, st);
    const unsigned blocks = (unsigned)(rows * a.n_heads);
    if (a.f32)
        hipLaunchKernelGGL(attend_plain_kernel<float>, dim3(blocks), dim3(PL_NT), 0, st,
                           static_cast<const float *>(a.q), static_cast<const float *>(a.k),
                           a.k_row_stride, static_cast<const float *>(a.v), a.v_row_stride, a.idx,
                           a.vis_lo, a.vis_hi, a.out, a.lse, a.n_q, a.n_k, a.n_heads, a.kd, a.vd,
                           a.kv_heads, a.n_sel, scale_log2);
    else
        hipLaunchKernelGGL(attend_plain_kernel<uint16_t>, dim3(blocks), dim3(PL_NT), 0, st,
                           static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
                           a.k_row_stride, static_cast<const uint16_t *>(a.v), a.v_row_stride,
                           a.idx, a.vis_lo, a.vis_hi, a.out, a.lse, a.n_q, a.n_k, a.n_heads, a.kd,
                           a.vd, a.kv_heads, a.n_sel, scale_log2);
    return hipGetLastError();
}

} // namespace dsa
