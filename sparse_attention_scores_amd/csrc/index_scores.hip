// index_scores.hip -- lightning-indexer scores on gfx950.
//
// score[b,t,s] = sum_h w[b,t,h] * relu(scale * q[b,t,h,:] . k'[b,s,:])
// ("GLM-5.2: the DSA sparse attention moves onto the pure fak kernel",
// section "The selection stays host-side BY DESIGN"; "Module
// glm5next_dsa_ref", index_scores), over the visible range [lo, hi) of each
// query; every other score is -FLT_MAX.
//
// MFMA kernel: one 32x32x16 bf16 MFMA tile holds 32 heads x 32 keys of one
// query; the heads x dims contraction runs on the matrix core and the
// epilogue (scale, relu, x w, sum over heads) stays in registers: each lane
// owns one key and 16 heads of it, sums them, and one cross-half shuffle
// finishes the head sum.  The key tile is the B operand, loaded straight
// from HBM in the operand layout (each lane reads contiguous 16-byte pieces
// of its key row), so the scores never exist per head.
#include "dsa_device.hpp"
#include "dsa_internal.hpp"

#include <float.h>

namespace dsa {

// D: head_dim; MT: 32-head groups (n_heads = 32*MT); QPW: queries per wave;
// WQ: waves along queries in a block (4/WQ waves split the key tiles);
// FP8: keys are OCP e4m3 codes with a per-row f32 scale.
template <int D, int MT, int QPW, int WQ, bool FP8>
__global__ __launch_bounds__(256) void index_scores_mfma_kernel(
    const uint16_t *__restrict__ q, const void *__restrict__ kv, const float *__restrict__ kscale,
    const float *__restrict__ w, const int32_t *__restrict__ vlo, const int32_t *__restrict__ vhi,
    float *__restrict__ scores, int n_q, int n_k, float scale, int n_qblocks, int n_chunks,
    int chunk)
{
    constexpr int H = 32 * MT;
    constexpr int KS = D / 16;  // MFMA k-steps of 16 dims
    constexpr int QB = WQ * QPW;
    constexpr int WK = 4 / WQ;
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int wq = wid % WQ, wk = wid / WQ;
    const int g = lane >> 5;      // half-wave: which 8-dim group of a k-step
    const int col = lane & 31;    // key (B column) / head (A row) within the tile

    int bid = blockIdx.x;
    const int kc = bid % n_chunks;
    bid /= n_chunks;
    const int qblk = bid % n_qblocks;
    const int b = bid / n_qblocks;

    // ---- the wave's queries: q fragments, weights and visible ranges
    u32x4_t qf[QPW][MT][KS];
    float wr[QPW][MT][16];
    int lo[QPW], hi[QPW];
    int64_t qrow[QPW];
    bool qok[QPW];
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
        const int t = qblk * QB + wq * QPW + qi;
        qok[qi] = t < n_q;
        const int tt = qok[qi] ? t : 0;
        qrow[qi] = (int64_t)b * n_q + tt;
        int l0 = vlo[qrow[qi]], h0 = vhi[qrow[qi]];
        l0 = max(l0, 0);
        h0 = min(h0, n_k);
        lo[qi] = qok[qi] ? l0 : 0;
        hi[qi] = qok[qi] ? h0 : 0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int head = mt * 32 + col;
            const uint16_t *qp = q + (qrow[qi] * H + head) * D;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                // dims of (g, ks): bf16 keys use ks*16 + g*8; fp8 keys use
                // g*(D/2) + ks*8 so that a lane's fp8 bytes are contiguous.
                const int d0 = FP8 ? g * (D / 2) + ks * 8 : ks * 16 + g * 8;
                qf[qi][mt][ks] = *reinterpret_cast<const u32x4_t *>(qp + d0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int h = mt * 32 + 8 * (i / 4) + 4 * g + (i % 4);
                wr[qi][mt][i] = w[qrow[qi] * H + h];
            }
        }
    }

    const int c0 = kc * chunk;
    const int c1 = min(c0 + chunk, n_k);
    const int ntiles = (c1 - c0 + 31) / 32;

    // A tile is "active" if any of the wave's queries sees a key in it.
    auto tile_active = [&](int s0) {
        bool act = false;
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi)
            act |= (lo[qi] < s0 + 32) && (hi[qi] > s0) && (lo[qi] < hi[qi]);
        return act;
    };
    // B-operand fragments of the tile's keys (lane = key s0 + col), and the
    // per-key factor scale * k_scale.
    auto load_tile = [&](int s0, u32x4_t (&kf)[KS], float &gsc) {
        const int kl = min(s0 + col, n_k - 1);
        gsc = scale;
        if constexpr (FP8) {
            const uint8_t *kp = reinterpret_cast<const uint8_t *>(kv) +
                                ((int64_t)b * n_k + kl) * D + g * (D / 2);
#pragma unroll
            for (int p = 0; p < KS / 2; ++p)
                kf[2 * p] = *reinterpret_cast<const u32x4_t *>(kp + p * 16);
            gsc = scale * kscale[(int64_t)b * n_k + kl];
        } else {
            const uint16_t *kp = reinterpret_cast<const uint16_t *>(kv) +
                                 ((int64_t)b * n_k + kl) * D + g * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[ks] = *reinterpret_cast<const u32x4_t *>(kp + ks * 16);
        }
    };
    auto compute_tile = [&](int s0, bool act, u32x4_t (&kf)[KS], float gsc) {
        const int key = s0 + col;
        if (!act) {
            if (lane < 32 && key < c1) {
#pragma unroll
                for (int qi = 0; qi < QPW; ++qi)
                    if (qok[qi])
                        scores[qrow[qi] * n_k + key] = -FLT_MAX;
            }
            return;
        }
        if constexpr (FP8) {
            // 16 raw e4m3 codes per 16-byte load -> two k-steps of 8 bf16
#pragma unroll
            for (int p = KS / 2 - 1; p >= 0; --p) {
                const u32x4_t c = kf[2 * p];
                const u32x2_t a0 = e4m3x4_to_bf16x4(c[0]);
                const u32x2_t a1 = e4m3x4_to_bf16x4(c[1]);
                const u32x2_t a2 = e4m3x4_to_bf16x4(c[2]);
                const u32x2_t a3 = e4m3x4_to_bf16x4(c[3]);
                kf[2 * p] = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
                kf[2 * p + 1] = u32x4_t{a2[0], a2[1], a3[0], a3[1]};
            }
        }
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) {
            float part = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x16_t acc = {};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = mfma_32x32x16(qf[qi][mt][ks], kf[ks], acc);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    part += wr[qi][mt][i] * fmaxf(acc[i] * gsc, 0.f);
            }
            part += __shfl_xor(part, 32, kWave);
            if (lane < 32 && key < c1 && qok[qi])
                scores[qrow[qi] * n_k + key] = (key >= lo[qi] && key < hi[qi]) ? part : -FLT_MAX;
        }
    };

    // Two tiles in flight per wave: the next tile's loads are issued before
    // the current tile's MFMA work.
    u32x4_t kfa[KS], kfb[KS];
    float ga = scale, gb = scale;
    int tile = wk;
    bool act_a = false;
    if (tile < ntiles) {
        act_a = tile_active(c0 + tile * 32);
        if (act_a)
            load_tile(c0 + tile * 32, kfa, ga);
    }
    while (tile < ntiles) {
        const int nxt = tile + WK;
        bool act_b = false;
        if (nxt < ntiles) {
            act_b = tile_active(c0 + nxt * 32);
            if (act_b)
                load_tile(c0 + nxt * 32, kfb, gb);
        }
        compute_tile(c0 + tile * 32, act_a, kfa, ga);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kfa[ks] = kfb[ks];
        ga = gb;
        act_a = act_b;
        tile = nxt;
    }
}

// Plain f32 kernel: one thread per (query row, key).
__global__ void index_scores_f32_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                        const float *__restrict__ w,
                                        const int32_t *__restrict__ vlo,
                                        const int32_t *__restrict__ vhi,
                                        float *__restrict__ scores, int n_q, int n_k, int H,
                                        int D, float scale, int64_t total)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total)
        return;
    const int64_t row = e / n_k;
    const int s = (int)(e % n_k);
    const int64_t b = row / n_q;
    const int l0 = max(vlo[row], 0), h0 = min(vhi[row], n_k);
    if (s < l0 || s >= h0) {
        scores[e] = -FLT_MAX;
        return;
    }
    const float *kr = k + (b * n_k + s) * D;
    float total_s = 0.f;
    for (int h = 0; h < H; ++h) {
        const float *qr = q + (row * H + h) * D;
        float dot = 0.f;
        for (int c = 0; c < D; ++c)
            dot = fmaf(qr[c], kr[c], dot);
        total_s += w[row * H + h] * fmaxf(scale * dot, 0.f);
    }
    scores[e] = total_s;
}

template <int D, int MT, int QPW, int WQ, bool FP8>
static hipError_t launch_mfma(const IndexArgs &a, hipStream_t st)
{
    constexpr int QB = QPW * WQ;
    const int chunk = WQ == 1 ? 512 : 256;
    const int n_qblocks = (a.n_q + QB - 1) / QB;
    const int n_chunks = (a.n_k + chunk - 1) / chunk;
    const int64_t blocks = (int64_t)a.batch * n_qblocks * n_chunks;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((index_scores_mfma_kernel<D, MT, QPW, WQ, FP8>), dim3((unsigned)blocks),
                       dim3(256), 0, st, static_cast<const uint16_t *>(a.q), a.k, a.k_scale, a.w,
                       a.vis_lo, a.vis_hi, a.scores, a.n_q, a.n_k, a.scale, n_qblocks, n_chunks,
                       chunk);
    return hipGetLastError();
}

template <int D, int MT, bool FP8>
static hipError_t launch_mfma_mode(const IndexArgs &a, hipStream_t st)
{
    if (a.n_q >= 8)
        return launch_mfma<D, MT, 2, 4, FP8>(a, st);
    return launch_mfma<D, MT, 1, 1, FP8>(a, st);
}

template <int D, int MT>
static hipError_t launch_mfma_keys(const IndexArgs &a, hipStream_t st)
{
    return a.k_fp8 ? launch_mfma_mode<D, MT, true>(a, st) : launch_mfma_mode<D, MT, false>(a, st);
}

bool index_mfma_supported(int n_heads, int head_dim)
{
    return (n_heads == 32 || n_heads == 64) && (head_dim == 64 || head_dim == 128);
}

hipError_t launch_index_scores(const IndexArgs &a, hipStream_t st)
{
    if (a.f32) {
        const int64_t total = (int64_t)a.batch * a.n_q * a.n_k;
        const int64_t blocks = (total + 255) / 256;
        if (blocks > 0x7fffffff)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(index_scores_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                           static_cast<const float *>(a.q), static_cast<const float *>(a.k), a.w,
                           a.vis_lo, a.vis_hi, a.scores, a.n_q, a.n_k, a.n_heads, a.head_dim,
                           a.scale, total);
        return hipGetLastError();
    }
    if (a.head_dim == 128)
        return a.n_heads == 32 ? launch_mfma_keys<128, 1>(a, st) : launch_mfma_keys<128, 2>(a, st);
    return a.n_heads == 32 ? launch_mfma_keys<64, 1>(a, st) : launch_mfma_keys<64, 2>(a, st);
}

} // namespace dsa
