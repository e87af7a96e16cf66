// masked_attend.hip -- per-head (non-absorbed) sparse attention over each
// query's selected tokens, as in the pooled NoPE variant ("Module
// glm5next_dsa_ref": topk_to_mask turns an index row into the visibility
// mask the attention reads -- duplicates collapse, out-of-range and INVALID
// entries are dropped -- and mla_masked_attention attends over it).
//
// With per-head K and V nothing is shared across heads, so gathering each
// query's ~2k selected rows per head would move ~100 MB per query.  Instead:
//  1. topk_to_mask_kernel writes one bit per (query, key): the query's
//     selected set, intersected with its visible range;
//  2. attend_masked_kernel is a flash-style pass per (head, block of 128
//     queries) over the key tiles the block's causal range covers; each tile
//     is staged once in LDS and used by all 128 queries, non-selected keys
//     are masked out of the online softmax, and tiles no query selects are
//     skipped.
// MFMA layout (32x32x16 bf16): S^T[key][query] = K_tile * Q^T with the
// queries of a wave in the B operand (held in registers), and
// O^T[c][query] += V^T * P^T, where each lane's accumulators all belong to
// one query, so the softmax rescale needs no cross-lane traffic.  V^T keeps
// the keys of each 16-key half in the order the S^T accumulators hold them,
// so P^T comes straight from the softmax registers.
#include "dsa_device.hpp"
#include "dsa_internal.hpp"

#include <float.h>
#include <math.h>

namespace dsa {

constexpr int MK_MAXWORDS = 16384;  // n_k <= 524288

// One block per query row: the row's selected set as bits over n_k keys.
__global__ __launch_bounds__(256) void topk_to_mask_kernel(const int32_t *__restrict__ idx,
                                                           const int32_t *__restrict__ vlo,
                                                           const int32_t *__restrict__ vhi,
                                                           uint32_t *__restrict__ mask, int n_k,
                                                           int n_sel, int nw)
{
    __shared__ uint32_t bits[MK_MAXWORDS];
    const int row = blockIdx.x;
    int lo = 0, hi = n_k;
    if (vlo) {
        lo = max(vlo[row], 0);
        hi = min(vhi[row], n_k);
    }
    for (int i = threadIdx.x; i < nw; i += 256)
        bits[i] = 0u;
    __syncthreads();
    const int32_t *ir = idx + (int64_t)row * n_sel;
    for (int i = threadIdx.x; i < n_sel; i += 256) {
        const int j = ir[i];
        if (j >= lo && j < hi)
            atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    uint32_t *mr = mask + (int64_t)row * nw;
    for (int i = threadIdx.x; i < nw; i += 256)
        mr[i] = bits[i];
}

template <int KD, int VD>
struct __attribute__((aligned(16))) MaskedSmem {
    static constexpr int KB = 32 * KD * 2;  // K tile bytes (32 keys, row-major, swizzled)
    static constexpr int VB = 32 * VD * 2;  // V tile bytes
    unsigned char k[2][KB];
    unsigned char v[2][VB];
    int red[8];
};

template <int KD, int VD>
__global__ __launch_bounds__(256) void attend_masked_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, int64_t ksr,
    const uint16_t *__restrict__ v, int64_t vsr, const uint32_t *__restrict__ mask,
    const int32_t *__restrict__ vlo, const int32_t *__restrict__ vhi, float *__restrict__ out,
    float *__restrict__ lse, int n_q, int n_k, int H, int kv_heads, int nw, int n_qblocks,
    int BH, float scale_log2)
{
    constexpr int KS = KD / 16;      // k-steps of the 32x32x16 MFMA over kd
    constexpr int NCT = VD / 32;     // output column tiles of 32
    constexpr int KCH = KD / 8;      // 16-byte chunks of a K row
    constexpr int VCH = VD / 8;      // 16-byte chunks of a V row
    static_assert(KCH % 8 == 0 && VCH % 8 == 0, "rows must hold a multiple of 8 chunks");
    using Sm = MaskedSmem<KD, VD>;
    static_assert(Sm::KB % 1024 == 0 && Sm::VB % 1024 == 0, "tiles are whole DMA instructions");
    __shared__ Sm sm;
    DSA_LDS_ESCAPE(sm);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int g = lane >> 5, col = lane & 31;
    // Head-major order: the query blocks of one (sequence, head) run together
    // and stream the same K/V tiles (served from L2/MALL after the first
    // read); within a head the heaviest (latest) query blocks go first.
    const int qblk = n_qblocks - 1 - (int)(blockIdx.x % n_qblocks);
    const int bh = blockIdx.x / n_qblocks;
    const int b = bh / H, h = bh % H;
    const int kvh = h / (H / kv_heads);
    const int q0 = qblk * 128;
    const int qi = q0 + wid * 32 + col;  // this lane's query
    const bool q_ok = qi < n_q;
    const int64_t row = (int64_t)b * n_q + (q_ok ? qi : 0);

    // key range of the block: union of the visible ranges
    int lo = 0, hi = n_k;
    if (vlo) {
        lo = q_ok ? max(vlo[row], 0) : n_k;
        hi = q_ok ? min(vhi[row], n_k) : 0;
    }
    {
        int mn = lo, mx = hi;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            mn = min(mn, __shfl_xor(mn, o, kWave));
            mx = max(mx, __shfl_xor(mx, o, kWave));
        }
        if (lane == 0) {
            sm.red[wid] = mn;
            sm.red[4 + wid] = mx;
        }
        __syncthreads();
        lo = min(min(sm.red[0], sm.red[1]), min(sm.red[2], sm.red[3]));
        hi = max(max(sm.red[4], sm.red[5]), max(sm.red[6], sm.red[7]));
    }
    const int t_begin = lo / 32;
    const int t_end = hi > lo ? (hi + 31) / 32 : t_begin;

    // Q^T fragments (B operand): query qi, dims ks*16 + g*8 .. +8
    u32x4_t qf[KS];
    {
        const uint16_t *qp = q + (row * H + h) * KD + g * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = q_ok ? *reinterpret_cast<const u32x4_t *>(qp + ks * 16)
                          : u32x4_t{0u, 0u, 0u, 0u};
    }
    f32x16_t oacc[NCT];
#pragma unroll
    for (int n = 0; n < NCT; ++n)
        oacc[n] = f32x16_t{};
    float m_run = -INFINITY, l_part = 0.f;

    const unsigned char *kb =
        reinterpret_cast<const unsigned char *>(k + (int64_t)b * n_k * ksr + (int64_t)kvh * KD);
    const unsigned char *vb =
        reinterpret_cast<const unsigned char *>(v + (int64_t)b * n_k * vsr + (int64_t)kvh * VD);
    const uint32_t *mrow = mask + row * nw;

    // DMA the 32 K rows and 32 V rows of tile t (rows past n_k repeat the
    // last key; they are masked out).
    auto dma_tile = [&](int t, int par) {
        const int k0 = t * 32;
        for (int s = wid; s < (Sm::KB + Sm::VB) / 1024; s += 4) {
            if (s < Sm::KB / 1024) {
                const int c = s * 64 + lane;
                const int r = c / KCH;
                const int logical = (c % KCH) ^ chunk_swz(r);
                const int key = min(k0 + r, n_k - 1);
                lds_dma16(kb + ((int64_t)key * ksr) * 2 + logical * 16, sm.k[par] + s * 1024);
            } else {
                const int sv = s - Sm::KB / 1024;
                const int c = sv * 64 + lane;
                const int r = c / VCH;
                const int logical = (c % VCH) ^ chunk_swz(r);
                const int key = min(k0 + r, n_k - 1);
                lds_dma16(vb + ((int64_t)key * vsr) * 2 + logical * 16, sm.v[par] + sv * 1024);
            }
        }
    };

    if (t_begin < t_end)
        dma_tile(t_begin, 0);
    for (int t = t_begin; t < t_end; ++t) {
        const int par = (t - t_begin) & 1;
        const uint32_t word = q_ok ? mrow[t] : 0u;
        lds_dma_wait();
        const bool any = __syncthreads_or(word != 0u);  // also: tile t visible to all
        if (t + 1 < t_end)
            dma_tile(t + 1, par ^ 1);
        if (any) {
            const u32x4_t *K16 = reinterpret_cast<const u32x4_t *>(sm.k[par]);
            const unsigned char *Vt = sm.v[par];
            // ---- S^T[key][query] for the 32 keys of the tile
            f32x16_t sa = {}, sb = {};
#pragma unroll
            for (int ks = 0; ks < KS; ks += 2) {
                sa = mfma_32x32x16(K16[col * KCH + ((2 * ks + g) ^ chunk_swz(col))], qf[ks], sa);
                if (ks + 1 < KS)
                    sb = mfma_32x32x16(K16[col * KCH + ((2 * ks + 2 + g) ^ chunk_swz(col))],
                                       qf[ks + 1], sb);
            }
            const f32x16_t s = sa + sb;
            // lane holds keys 8*(i/4) + 4g + i%4 of the tile for query qi
            float x[16];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kk = 8 * (i / 4) + 4 * g + (i % 4);
                x[i] = ((word >> kk) & 1u) ? s[i] * scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, x[i]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
            // lazy rescale (see the gather kernel): p <= 2^kRescaleLog2
            const bool grow = tmax > m_run + kRescaleLog2;
            if (__any(grow)) {
                const float m_new = grow ? tmax : m_run;
                // lanes that do not grow keep alpha = 1 (m_run may still be -inf
                // there, and -inf - -inf would be NaN); a growing lane with
                // m_run = -inf gets 0
                const float alpha = grow ? exp2f(m_run - m_new) : 1.f;
                if (__any(grow && m_run != -INFINITY)) {
#pragma unroll
                    for (int n = 0; n < NCT; ++n)
                        oacc[n] *= alpha;
                }
                l_part *= alpha;
                m_run = m_new;
            }
            // m_run is -inf only while every key seen so far (this tile
            // included) is masked; then all x are -inf and p must be 0.
            const float m_ref = (m_run == -INFINITY) ? 0.f : m_run;
            float p[16];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                p[i] = exp2f(x[i] - m_ref);
                psum += p[i];
            }
            l_part += psum;
            // ---- O^T[c][query] += V^T[c][keys] P^T[keys][query], per 16-key half.
            //      V^T fragments are read transposed from the row-major V tile:
            //      16-lane group G = (g, column half ch); source lane i = a + 4j
            //      points at row kh*16 + 4g + j (then + 8), columns
            //      n*32 + ch*16 + 4a .. + 3.
            const int grp = lane >> 4, gg = grp >> 1, ch = grp & 1;
            const int li = lane & 15, la = li & 3, lj = li >> 2;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                float hv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    hv[j] = bf16_bits_to_f32(f32_to_bf16_bits(p[kh * 8 + j]));
                const u32x4_t bhi = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]),
                                     pack_bf16x2(hv[4], hv[5]), pack_bf16x2(hv[6], hv[7])};
                const u32x4_t blo = {
                    pack_bf16x2(p[kh * 8 + 0] - hv[0], p[kh * 8 + 1] - hv[1]),
                    pack_bf16x2(p[kh * 8 + 2] - hv[2], p[kh * 8 + 3] - hv[3]),
                    pack_bf16x2(p[kh * 8 + 4] - hv[4], p[kh * 8 + 5] - hv[5]),
                    pack_bf16x2(p[kh * 8 + 6] - hv[6], p[kh * 8 + 7] - hv[7])};
                const int ra = kh * 16 + 4 * gg + lj, rb2 = ra + 8;
#pragma unroll
                for (int n = 0; n < NCT; ++n) {
                    const int lc = 4 * n + 2 * ch + (la >> 1);  // logical 16-byte chunk
                    const int off = 8 * (la & 1);
                    const u32x2_t va =
                        lds_read_tr16x4(Vt + (ra * VCH + (lc ^ chunk_swz(ra))) * 16 + off);
                    const u32x2_t vbb =
                        lds_read_tr16x4(Vt + (rb2 * VCH + (lc ^ chunk_swz(rb2))) * 16 + off);
                    const u32x4_t a = u32x4_t{va[0], va[1], vbb[0], vbb[1]};
                    oacc[n] = mfma_32x32x16(a, bhi, oacc[n]);
                    oacc[n] = mfma_32x32x16(a, blo, oacc[n]);
                }
            }
        }
    }

    // ---- epilogue
    const float l_tot = l_part + __shfl_xor(l_part, 32, kWave);
    if (q_ok) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *op = out + (row * H + h) * VD;
#pragma unroll
        for (int n = 0; n < NCT; ++n) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int c = n * 32 + 8 * r4 + 4 * g;
                const f32x4_t v4 = {oacc[n][4 * r4] * inv, oacc[n][4 * r4 + 1] * inv,
                                    oacc[n][4 * r4 + 2] * inv, oacc[n][4 * r4 + 3] * inv};
                *reinterpret_cast<f32x4_t *>(op + c) = v4;
            }
        }
        if (lse && g == 0)
            lse[row * H + h] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

bool attend_masked_supported(const AttendArgs &a)
{
    return !a.f32 && a.kv_heads == a.n_heads && a.kd == 192 && a.vd == 256 &&
           a.k_row_stride % 8 == 0 && a.v_row_stride % 8 == 0;
}

size_t attend_masked_workspace_bytes(const AttendArgs &a)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    const int64_t nw = (a.n_k + 31) / 32;
    return (size_t)(rows * nw) * sizeof(uint32_t);
}

hipError_t launch_attend_masked(const AttendArgs &a, hipStream_t st)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    const int nw = (a.n_k + 31) / 32;
    uint32_t *mask = static_cast<uint32_t *>(a.workspace);
    hipLaunchKernelGGL(topk_to_mask_kernel, dim3((unsigned)rows), dim3(256), 0, st, a.idx,
                       a.vis_lo, a.vis_hi, mask, a.n_k, a.n_sel, nw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int n_qblocks = (a.n_q + 127) / 128;
    const int BH = a.batch * a.n_heads;
    const int64_t blocks = (int64_t)n_qblocks * BH;
    hipLaunchKernelGGL((attend_masked_kernel<192, 256>), dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
                       a.k_row_stride, static_cast<const uint16_t *>(a.v), a.v_row_stride, mask,
                       a.vis_lo, a.vis_hi, a.out, a.lse, a.n_q, a.n_k, a.n_heads, a.kv_heads, nw,
                       n_qblocks, BH, a.scale * kLog2e);
    return hipGetLastError();
}

} // namespace dsa
