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

#include <algorithm>

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

// Decode kernel (one query per block): the same MFMA tile and epilogue, but
// each wave streams its key tiles through an LDS ring of its own.  A tile's
// rows arrive by direct-to-LDS 16-byte loads, every load instruction one
// contiguous 1 KB of key rows (whole cache lines), with the 16-byte chunks of
// row r stored at chunk ^ (r & (chunks per row - 1)); the B operands are then
// read from LDS, where 32 rows at one chunk hit different banks.  (Loaded
// straight in the operand layout, one instruction touches 32 rows in 32-byte
// pieces, and the key stream ran about an eighth slower, measured.)  The
// fp8 keys' per-row scales ride along as one 4-byte-per-lane load per tile.
// No barrier: a wave reads only the tiles it loaded, after waiting for them.
constexpr int ID_STAGES = 2;
template <int D, int MT, bool FP8>
__global__ __launch_bounds__(256) void index_scores_decode_kernel(
    const uint16_t *__restrict__ q, const void *__restrict__ kv, const float *__restrict__ kscale,
    const float *__restrict__ w, const int32_t *__restrict__ vlo, const int32_t *__restrict__ vhi,
    float *__restrict__ scores, int n_q, int n_k, float scale, int n_chunks, int chunk)
{
    constexpr int H = 32 * MT;
    constexpr int KS = D / 16;                      // MFMA k-steps of 16 dims
    constexpr int RB = D * (FP8 ? 1 : 2);           // bytes per key row
    constexpr int CPR = RB / 16;                    // 16-byte chunks per row
    constexpr int TB = 32 * RB;                     // tile bytes
    constexpr int DPT = TB / 1024;                  // load instructions per tile
    constexpr int VPT = DPT + (FP8 ? 1 : 0);        // vector-memory ops per tile
    constexpr int NCH = FP8 ? KS / 2 : KS;          // 16-byte operand chunks per lane
    constexpr int SB = TB + (FP8 ? 256 : 0);        // stage bytes (tile, k-scales)
    static_assert(TB % 1024 == 0 && (NCH == 4 || NCH == 8), "tile shape");
    __shared__ __attribute__((aligned(16))) unsigned char ring[4][ID_STAGES][SB];
    DSA_LDS_ESCAPE(ring);
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, col = lane & 31;

    int bid = blockIdx.x;
    const int kc = bid % n_chunks;
    bid /= n_chunks;
    const int64_t qrow = bid;                       // (batch, query) row
    const int64_t b = qrow / n_q;
    const int lo = max(vlo[qrow], 0), hi = min(vhi[qrow], n_k);

    // q fragments and head weights (as in the tile kernel above)
    u32x4_t qf[MT][KS];
    float wr[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int head = mt * 32 + col;
        const uint16_t *qp = q + (qrow * H + head) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = FP8 ? g * (D / 2) + ks * 8 : ks * 16 + g * 8;
            qf[mt][ks] = *reinterpret_cast<const u32x4_t *>(qp + d0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            wr[mt][i] = w[qrow * H + mt * 32 + 8 * (i / 4) + 4 * g + (i % 4)];
    }

    // this wave's tiles of the chunk, and the ones that see a key
    const int c0 = kc * chunk, c1 = min(c0 + chunk, n_k);
    const int ntc = (c1 - c0 + 31) / 32;
    const int wt0 = wid * ntc / 4, wt1 = (wid + 1) * ntc / 4;
    int at0 = wt1, at1 = wt1;
    if (lo < hi) {
        at0 = min(max(wt0, (lo - c0) / 32), wt1);
        at1 = max(min(wt1, (hi - c0 + 31) / 32), at0);
    }
    float *srow = scores + qrow * n_k;
    // keys of the wave's tiles outside [at0, at1) see nothing
    for (int s = c0 + wt0 * 32 + lane; s < min(c1, c0 + at0 * 32); s += 64)
        srow[s] = -FLT_MAX;
    for (int s = c0 + at1 * 32 + lane; s < min(c1, c0 + wt1 * 32); s += 64)
        srow[s] = -FLT_MAX;

    // load slot of this lane in instruction i: (row, byte offset of the
    // logical chunk it fetches), fixed over tiles
    uint32_t dslot[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
        const int off = i * 1024 + lane * 16, r = off / RB, pc = (off % RB) / 16;
        dslot[i] = ((uint32_t)r << 16) | (uint32_t)((pc ^ (r & (CPR - 1))) * 16);
    }
    // operand chunk offsets inside a stage: key col, logical chunk lc
    uint32_t rofs[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int lc = FP8 ? g * (CPR / 2) + j : 2 * j + g;
        rofs[j] = (uint32_t)(col * RB + (lc ^ (col & (CPR - 1))) * 16);
    }
    const unsigned char *kbase =
        reinterpret_cast<const unsigned char *>(kv) + b * (int64_t)n_k * RB;
    auto load_tile = [&](int t, int st) {
        const int s0 = c0 + t * 32;
        unsigned char *dst = ring[wid][st];
#pragma unroll
        for (int i = 0; i < DPT; ++i) {
            const int r = min(s0 + (int)(dslot[i] >> 16), n_k - 1);
            lds_dma16(kbase + (int64_t)r * RB + (dslot[i] & 0xffffu), dst + i * 1024);
        }
        if constexpr (FP8)
            lds_dma4(kscale + b * n_k + min(s0 + col, n_k - 1), dst + TB);
    };

    vm_wait<0>();  // q and w are in registers: the ring's waits count tiles only
    const int nt = at1 - at0;
    for (int j = 0; j < ID_STAGES - 1 && j < nt; ++j)
        load_tile(at0 + j, j);
    for (int t = 0; t < nt; ++t) {
        vm_wait_tiles<VPT>(min(nt - 1, t + ID_STAGES - 2) - t);  // tile t is in
        if (t + ID_STAGES - 1 < nt)  // refill the stage read in the last iteration
            load_tile(at0 + t + ID_STAGES - 1, (t + ID_STAGES - 1) % ID_STAGES);
        const uint32_t sb = lds_addr(ring[wid][t % ID_STAGES]);
        uint32_t ad[NCH];
#pragma unroll
        for (int j = 0; j < NCH; ++j)
            ad[j] = sb + rofs[j];
        u32x4_t kf[KS];
        float gsc = scale;
        if constexpr (NCH == 8) {
            u32x4_t v[8];
            lds_read_b128_a8(v, ad);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                kf[FP8 ? 2 * j : j] = v[j];
        } else {
            u32x4_t v[4];
            lds_read_b128_a4(v, ad);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                kf[FP8 ? 2 * j : j] = v[j];
        }
        if constexpr (FP8) {
            gsc = scale * __uint_as_float(lds_read_u32_wait(sb + TB + 4 * col));
            // 16 raw e4m3 codes per chunk -> two k-steps of 8 bf16
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
        float part = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x16_t acc = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = mfma_32x32x16(qf[mt][ks], kf[ks], acc);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                part += wr[mt][i] * fmaxf(acc[i] * gsc, 0.f);
        }
        part += __shfl_xor(part, 32, kWave);
        const int key = c0 + (at0 + t) * 32 + col;
        if (lane < 32 && key < c1)
            srow[key] = (key >= lo && key < hi) ? part : -FLT_MAX;
    }
}

// Prefill kernel (bf16 keys, 32 heads x 128 dims, many queries): a block of
// 8 waves x 2 queries shares each key tile.  Tiles of 32 keys (8 KB) stream
// into a 3-stage LDS ring by direct-to-LDS loads (one 1-KB instruction per
// wave per tile) and every wave reads its B operands from there, so a key
// row crosses L2 once per 16 queries instead of once per 2.  The 16-byte
// chunks of key row r sit at chunk ^ (r & 15), which keeps the operand reads
// (32 rows at two adjacent chunks) at the full LDS rate on gfx950, measured.
constexpr int IP_D = 128, IP_H = 32, IP_QPW = 2, IP_NW = 8, IP_QB = IP_QPW * IP_NW;
constexpr int IP_TILEB = 32 * IP_D * 2, IP_STAGES = 3;
static_assert(IP_TILEB == 1024 * IP_NW, "one DMA instruction per wave per tile");

// Balance: under a causal mask the number of key tiles a query block sees
// grows with its position, and with about one block per CU the kernel would
// last as long as the latest block.  Query blocks are therefore paired (the
// i-th earliest with the i-th latest) and each pair's visible tiles, the
// later block's first, are split evenly between two workgroups; a
// workgroup reloads the queries when its share moves on to the earlier
// block.  With many query blocks per CU (`paired` false) each workgroup
// takes one query block whole, the latest first, and loads its queries
// once.
__global__ __launch_bounds__(64 * IP_NW) void index_scores_prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv, const float *__restrict__ w,
    const int32_t *__restrict__ vlo, const int32_t *__restrict__ vhi, float *__restrict__ scores,
    int n_q, int n_k, float scale, int n_qblocks, int n_chunks, int chunk, bool paired)
{
    constexpr int KS = IP_D / 16;
    __shared__ __attribute__((aligned(16))) unsigned char tiles[IP_STAGES][IP_TILEB];
    DSA_LDS_ESCAPE(tiles);
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int g = lane >> 5, col = lane & 31;
    const int n_units = paired ? (n_qblocks + 1) / 2 : n_qblocks;
    int bid = blockIdx.x;
    const int half = paired ? bid & 1 : 0;
    if (paired)
        bid >>= 1;
    const int kc = bid % n_chunks;
    bid /= n_chunks;
    const int unit = bid % n_units;
    const int b = bid / n_units;
    // a pair (equal for a middle block), or one block
    const int qb_late = n_qblocks - 1 - unit, qb_early = paired ? unit : qb_late;

    const int c0 = kc * chunk;
    const int c1 = min(c0 + chunk, n_k);
    const int nt = (c1 - c0 + 31) / 32;
    const bool neg_scale = scale < 0.f;
    const unsigned char *kb = reinterpret_cast<const unsigned char *>(kv) + (int64_t)b * n_k * IP_D * 2;

    // tiles [ta, tb) of the chunk hold a key some query of block qb sees
    auto visible_tiles = [&](int qb, int &ta, int &tb) {
        int ulo = n_k, uhi = 0;
        const int t = qb * IP_QB + (lane & (IP_QB - 1));
        if (t < n_q) {
            const int64_t r = (int64_t)b * n_q + t;
            ulo = max(vlo[r], 0);
            uhi = min(vhi[r], n_k);
            if (ulo >= uhi) {
                ulo = n_k;
                uhi = 0;
            }
        }
        ulo = (int)wave_min_u32((uint32_t)ulo);
        uhi = (int)wave_max_u32((uint32_t)uhi);
        ta = ulo < uhi ? min(nt, max(0, (ulo - c0) / 32)) : nt;
        tb = ulo < uhi ? max(ta, min(nt, (uhi - c0 + 31) / 32)) : nt;
    };
    int la, lb, ea = 0, eb = 0;
    visible_tiles(qb_late, la, lb);
    if (qb_early != qb_late)
        visible_tiles(qb_early, ea, eb);
    // the pair's visible tiles, the later block's first, split in two halves
    const int n_late = lb - la, n_all = n_late + (eb - ea);
    const int cut = paired ? (n_all + 1) / 2 : n_all;
    const int w0 = half ? cut : 0, w1 = half ? n_all : cut;

    // DMA: wave w fills LDS bytes w*1024 + 16*lane of the tile = row r, physical
    // chunk p <- logical chunk p ^ (r & 15) of key c0 + 32*tile + r
    const int dr = (wid * 64 + lane) / 16;
    const uint32_t doff = (uint32_t)((((wid * 64 + lane) % 16) ^ (dr & 15)) * 16);
    auto dma_tile = [&](int tt, int st) {
        const int key = min(c0 + tt * 32 + dr, n_k - 1);
        lds_dma16(kb + (int64_t)key * (IP_D * 2) + doff, tiles[st] + wid * 1024);
    };
    // B operand of k-step ks: row col, logical chunk 2ks + g
    uint32_t kaddr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        kaddr[ks] = (uint32_t)((col * 16 + ((2 * ks + g) ^ (col & 15))) * 16);
    const uint32_t lds0 = lds_addr(tiles[0]);

    // -FLT_MAX over the keys of the chunk before tile ta and from tile tb on
    // (the invisible tiles of block qb) for the wave's queries, in 16-byte
    // stores, the two halves taking half of each range: 8x fewer store
    // instructions than one 4-byte score per lane.  Issued after the block's
    // tiles, so no wait for the query loads or tile DMAs waits for them.
    auto fill_invisible = [&](int qb, int ta, int tb) {
#pragma unroll
        for (int qi = 0; qi < IP_QPW; ++qi) {
            const int t = qb * IP_QB + wid * IP_QPW + qi;
            if (t >= n_q)
                continue;
            float *rp = scores + ((int64_t)b * n_q + t) * n_k;
            const int g0 = (int)((reinterpret_cast<uintptr_t>(rp) >> 2) & 3);  // row start mod 4 floats
            const int ra[2] = {c0, min(c1, c0 + 32 * tb)};
            const int rb[2] = {min(c1, c0 + 32 * ta), c1};
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int mid = paired ? ra[r] + ((rb[r] - ra[r]) / 2 & ~3) : rb[r];
                const int a = half ? mid : ra[r], e = half ? rb[r] : mid;
                if (a >= e)
                    continue;
                // scalar head up to a 16-byte boundary, vector body, scalar tail
                const int ha = min(e, a + (int)((4 - ((g0 + a) & 3)) & 3));
                const int tb4 = max(ha, e - (int)((g0 + e) & 3));
                if (a + lane < ha)
                    rp[a + lane] = -FLT_MAX;
                for (int j = ha + 4 * lane; j < tb4; j += 256)
                    *reinterpret_cast<f32x4_t *>(rp + j) =
                        f32x4_t{-FLT_MAX, -FLT_MAX, -FLT_MAX, -FLT_MAX};
                if (tb4 + lane < e)
                    rp[tb4 + lane] = -FLT_MAX;
            }
        }
    };

    // Tiles [t0, t1) (chunk tile indices, all visible to block qb) for the
    // wave's queries of block qb.
    auto run = [&](int qb, int t0, int t1) {
        u32x4_t qf[IP_QPW][KS];
        float wr[IP_QPW][16];
        int lo[IP_QPW], hi[IP_QPW];
        int64_t qrow[IP_QPW];
        bool qok[IP_QPW];
#pragma unroll
        for (int qi = 0; qi < IP_QPW; ++qi) {
            const int t = qb * IP_QB + wid * IP_QPW + qi;
            qok[qi] = t < n_q;
            qrow[qi] = (int64_t)b * n_q + (qok[qi] ? t : 0);
            lo[qi] = qok[qi] ? max(vlo[qrow[qi]], 0) : 0;
            hi[qi] = qok[qi] ? min(vhi[qrow[qi]], n_k) : 0;
            // the sign of the scale goes into q (bf16 sign bits), so the
            // epilogue is relu(s) * (w * |scale|) whatever the sign
            const uint16_t *qp = q + (qrow[qi] * IP_H + col) * IP_D + g * 8;
            const uint32_t qsign = neg_scale ? 0x80008000u : 0u;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[qi][ks] = *reinterpret_cast<const u32x4_t *>(qp + ks * 16) ^ qsign;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                wr[qi][i] = w[qrow[qi] * IP_H + 8 * (i / 4) + 4 * g + (i % 4)] * fabsf(scale);
        }
        if (t0 >= t1)
            return;
        // epilogue of one tile: w * relu(scale * s) = (w * |scale|) * relu(sign(scale) * s),
        // summed over the lane's 16 heads and the other half-wave's 16; relu
        // is a signed-integer max on the bits (negative floats, -0 included,
        // are negative integers), one instruction per element
        auto finish = [&](const f32x16_t(&acc)[IP_QPW], int tt) {
            const int key = c0 + tt * 32 + col;
#pragma unroll
            for (int qi = 0; qi < IP_QPW; ++qi) {
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    part += wr[qi][i] * __int_as_float(max(__float_as_int(acc[qi][i]), 0));
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                                 __float_as_uint(part), false, false);
                part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                if (lane < 32 && key < c1 && qok[qi])
                    scores[qrow[qi] * n_k + key] =
                        (key >= lo[qi] && key < hi[qi]) ? part : -FLT_MAX;
            }
        };
        // the query data are in registers before the first tile DMA
        vm_wait<0>();
        for (int j = 0; j < IP_STAGES - 1 && t0 + j < t1; ++j)
            dma_tile(t0 + j, j);
        // Tile tt's MFMAs into acc (after the ring barrier that releases it),
        // interleaved with the epilogue sums of the previous tile (prev, if
        // `fin`): a wave issues in order, and a run of MFMAs would hold it at
        // each one until the matrix core takes it, so the VALU work goes in
        // between -- two relu-weighted terms after each MFMA, pinned by
        // scheduling-group barriers -- and the two streams overlap.
        auto step = [&](int tt, f32x16_t(&acc)[IP_QPW], const f32x16_t(&prev)[IP_QPW],
                        float (&part)[IP_QPW], bool fin) {
            static_assert(IP_QPW == 2, "the sums are pinned for two queries");
            const int st = (tt - t0) % IP_STAGES;
            // tile tt has landed once at most the later tiles' DMAs are
            // outstanding (loads complete in order; the score stores between
            // them only make the wait stricter)
            vm_wait_tiles<1>(min(t1 - 1, tt + IP_STAGES - 2) - tt);
            lds_barrier();
            if (tt + IP_STAGES - 1 < t1)
                dma_tile(tt + IP_STAGES - 1, (tt - t0 + IP_STAGES - 1) % IP_STAGES);
            const uint32_t base = lds0 + st * IP_TILEB;
            // operand reads run two k-steps ahead of the MFMAs that use them,
            // so the tile's LDS reads (all 8 waves read all of it) overlap
            // the matrix work instead of preceding it
            u32x4_t kf[KS];
            lds_read_b128_nowait(kf[0], base + kaddr[0]);
            lds_read_b128_nowait(kf[1], base + kaddr[1]);
#pragma unroll
            for (int qi = 0; qi < IP_QPW; ++qi) {
                acc[qi] = f32x16_t{};
                part[qi] = 0.f;
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 2 < KS) {
                    lds_read_b128_nowait(kf[ks + 2], base + kaddr[ks + 2]);
                    lds_operand_wait<2>(kf[ks]);
                } else if (ks + 1 < KS) {
                    lds_operand_wait<1>(kf[ks]);
                } else {
                    lds_operand_wait<0>(kf[ks]);
                }
#pragma unroll
                for (int qi = 0; qi < IP_QPW; ++qi) {
                    acc[qi] = mfma_32x32x16(qf[qi][ks], kf[ks], acc[qi]);
                    if (fin) {
                        // MFMA number j = 2ks + qi takes terms 2(j%8), 2(j%8)+1 of
                        // query j/8
                        const int j = 2 * ks + qi, pq = j / 8, i0 = 2 * (j % 8);
#pragma unroll
                        for (int i = i0; i < i0 + 2; ++i)
                            part[pq] += wr[pq][i] * __int_as_float(max(__float_as_int(prev[pq][i]), 0));
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // then VALU
                }
            }
            // the sums are complete here (kept from sinking past the MFMAs)
            asm volatile("" : "+v"(part[0]), "+v"(part[1]));
        };
        // the head sum's second half and the stores of tile tt
        // (one store for both queries: lanes 0-31 write query 0's row,
        // lanes 32-63 query 1's; after the swap both halves hold each sum)
        auto store = [&](float (&part)[IP_QPW], int tt) {
            const int key = c0 + tt * 32 + col;
            float v[IP_QPW];
#pragma unroll
            for (int qi = 0; qi < IP_QPW; ++qi) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[qi]),
                                                                 __float_as_uint(part[qi]), false,
                                                                 false);
                v[qi] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
            static_assert(IP_QPW == 2, "one query per half-wave");
            const float val = g ? v[1] : v[0];
            const bool ok = g ? qok[1] : qok[0];
            const int klo = g ? lo[1] : lo[0], khi = g ? hi[1] : hi[0];
            const int64_t rowoff = (g ? qrow[1] : qrow[0]) * n_k;
            if (key < c1 && ok)
                scores[rowoff + key] = (key >= klo && key < khi) ? val : -FLT_MAX;
        };
        f32x16_t acc_a[IP_QPW], acc_b[IP_QPW];
        float part[IP_QPW];
        step(t0, acc_a, acc_b, part, false);
        int tt = t0 + 1;
        for (; tt + 1 < t1; tt += 2) {
            step(tt, acc_b, acc_a, part, true);
            store(part, tt - 1);
            step(tt + 1, acc_a, acc_b, part, true);
            store(part, tt);
        }
        if (tt < t1) {
            step(tt, acc_b, acc_a, part, true);
            store(part, tt - 1);
            finish(acc_b, tt);
        } else {
            finish(acc_a, tt - 1);
        }
        lds_barrier();  // every wave is done with the ring before it is refilled
    };
    // this half's share of the pair's list, then the invisible keys of both
    // blocks
    run(qb_late, la + min(w0, n_late), la + min(w1, n_late));
    if (qb_early != qb_late)
        run(qb_early, ea + max(w0 - n_late, 0), ea + max(w1 - n_late, 0));
    fill_invisible(qb_late, la, lb);
    if (qb_early != qb_late)
        fill_invisible(qb_early, ea, eb);
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
    // f64 sums: a product of two f32 values is exact in f64, so the score
    // carries one f32 rounding at the end and the f64 sums' error (a few
    // 2^-53 of sum_h |w| |scale| sum_c |q k|) on top -- relative accuracy far
    // below 1e-5 wherever the sum does not cancel almost completely
    const float *kr = k + (b * n_k + s) * D;
    double total_s = 0.0;
    for (int h = 0; h < H; ++h) {
        const float *qr = q + (row * H + h) * D;
        double dot = 0.0;
        for (int c = 0; c < D; ++c)
            dot = fma((double)qr[c], (double)kr[c], dot);
        total_s += (double)w[row * H + h] * fmax((double)scale * dot, 0.0);
    }
    scores[e] = (float)total_s;
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

// Decode launch: chunks sized for about two blocks per CU (at least 128 keys,
// a multiple of 128 so each of the 4 waves has whole tiles).
template <int D, int MT, bool FP8>
static hipError_t launch_decode(const IndexArgs &a, hipStream_t st)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    int64_t chunk = ((int64_t)a.n_k * rows + 511) / 512;
    chunk = std::max<int64_t>(128, (chunk + 127) / 128 * 128);
    const int n_chunks = (int)((a.n_k + chunk - 1) / chunk);
    const int64_t blocks = rows * n_chunks;
    if (blocks > 0x7fffffff || chunk > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((index_scores_decode_kernel<D, MT, FP8>), dim3((unsigned)blocks), dim3(256),
                       0, st, static_cast<const uint16_t *>(a.q), a.k, a.k_scale, a.w, a.vis_lo,
                       a.vis_hi, a.scores, a.n_q, a.n_k, a.scale, n_chunks, (int)chunk);
    return hipGetLastError();
}

template <int D, int MT, bool FP8>
static hipError_t launch_mfma_mode(const IndexArgs &a, hipStream_t st)
{
    if (!FP8 && D == IP_D && MT * 32 == IP_H && a.n_q >= IP_QB) {
        // long key chunks: a block's 16 queries are loaded once per chunk
        const int n_qblocks = (a.n_q + IP_QB - 1) / IP_QB;
        const int chunk = 4096;
        const int n_chunks = (a.n_k + chunk - 1) / chunk;
        // two workgroups per pair of query blocks, or one per query block
        // when there are at least eight per CU (see the kernel)
        const bool paired = (int64_t)a.batch * n_qblocks * n_chunks < 8 * 256;
        const int64_t blocks = paired ? (int64_t)a.batch * ((n_qblocks + 1) / 2) * n_chunks * 2
                                      : (int64_t)a.batch * n_qblocks * n_chunks;
        if (blocks > 0x7fffffff)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(index_scores_prefill_kernel, dim3((unsigned)blocks), dim3(64 * IP_NW), 0,
                           st, static_cast<const uint16_t *>(a.q),
                           static_cast<const uint16_t *>(a.k), a.w, a.vis_lo, a.vis_hi, a.scores,
                           a.n_q, a.n_k, a.scale, n_qblocks, n_chunks, chunk, paired);
        return hipGetLastError();
    }
    if (a.n_q >= 8)
        return launch_mfma<D, MT, 2, 4, FP8>(a, st);
    if constexpr (FP8 && D == 64)  // 64-byte rows: too few chunks for the ring's swizzle
        return launch_mfma<D, MT, 1, 1, FP8>(a, st);
    else
        return launch_decode<D, MT, FP8>(a, st);
}

template <int D, int MT>
static hipError_t launch_mfma_keys(const IndexArgs &a, hipStream_t st)
{
    return a.k_fp8 ? launch_mfma_mode<D, MT, true>(a, st) : launch_mfma_mode<D, MT, false>(a, st);
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
