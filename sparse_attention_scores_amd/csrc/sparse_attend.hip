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

#include <type_traits>

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
constexpr int AB_ROWB = AB_KD * 2;            // 1152 bytes per latent row
constexpr int AB_CPR = AB_ROWB / 16;          // 72 16-byte chunks per row
constexpr int AB_TILEB = AB_TILE * AB_ROWB;   // 36 KB per tile
constexpr int AB_DMA = AB_TILEB / 1024;       // 36 one-KB wave DMA instructions per tile
constexpr int AB_LIST = 1024;                 // keys per batch of a block
constexpr int AB_NT = 512;                    // 8 waves: 4 head groups x 2 halves
constexpr int AB_NW = AB_NT / 64;
constexpr int AB_NC = AB_VD / 2 / 16;         // 16 output column tiles per wave
constexpr int AB_STAGES = 3;                  // tiles resident in LDS (ring)
// wave w issues the tile's DMA instructions w, w + 8, ...: 5 for waves 0-3,
// 4 for waves 4-7
constexpr int AB_DMA_HI = (AB_DMA + AB_NW - 1) / AB_NW;
constexpr int AB_DMA_LO = AB_DMA / AB_NW;
static_assert(AB_DMA % AB_NW == AB_NW / 2, "waves 0-3 issue one DMA more than waves 4-7");

// LDS tile: 32 latent rows, 1152 bytes apart, with the 16-byte chunks of row
// r stored XOR-swizzled (chunk_swz_odd) so that both the row-wise Q.K^T operand
// reads and the transposing P.V operand reads spread over all banks.  V is
// the first 512 columns of the same rows.
// The tiles are the only LDS object the direct-to-LDS loads write, and they
// are only read through asm; the other LDS data live in objects of their own,
// so the compiler can tell them apart and puts no wait for the tile loads in
// front of their accesses.
struct __attribute__((aligned(16))) AbsTiles {
    union {
        unsigned char tile[AB_STAGES][AB_TILEB];
        uint32_t bitmap[kBitmapMaxWords];
    } u;
};

// Wave w of a block owns heads 16*(w&3) .. +15 and half h = w>>2 of the work
// on them: the k-steps ks = 2m + h of Q.K^T (the partner wave w^4 does the
// others; the two partial score tiles are exchanged through LDS, so both
// hold the same S) and output columns 256h .. 256h + 255 of P.V.  Partners
// share a SIMD, so one's LDS waits overlap the other's MFMAs.
__global__ __launch_bounds__(AB_NT) void attend_gather_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv, int64_t row_stride,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ vlo,
    const int32_t *__restrict__ vhi, float *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ ws_o, float *__restrict__ ws_ml, int n_q, int n_k, int n_sel,
    int splits, float scale_log2)
{
    __shared__ AbsTiles sm;
    __shared__ f32x4_t sm_xs[AB_NW][2][64];  // partial S^T of each wave, for its partner
    __shared__ int32_t sm_list[AB_LIST];
    __shared__ int sm_wave_tot[AB_NW];
    DSA_LDS_ESCAPE(sm);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, col = lane & 15;
    const int hg = wid & 3, half = wid >> 2;
    // the splits of one row run on one XCD (shared q, idx and partials);
    // without splits the rows keep launch order, which spreads the uneven
    // causal rows evenly over the XCDs
    const int lb = splits > 1 ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;
    const int row = lb / splits;
    const int split = lb % splits;
    const int64_t b = row / n_q;

    int lo = 0, hi = n_k;
    if (vlo) {
        lo = max(vlo[row], 0);
        hi = min(vhi[row], n_k);
    }
    const int nw = (n_k + 31) >> 5;
    const int wpt = (nw + AB_NT - 1) / AB_NT;
    const int w0 = min(tid * wpt, nw), w1 = min(w0 + wpt, nw);

    // Q^T fragments (B operand) of this wave's k-steps ks = 2m + half: lane
    // holds head hg*16+col, dims ks*32 + g*8 .. +8
    const int head = hg * 16 + col;
    u32x4_t qf[AB_KS / 2];
    {
        const uint16_t *qp = q + ((int64_t)row * AB_H + head) * AB_KD + half * 32 + g * 8;
#pragma unroll
        for (int m = 0; m < AB_KS / 2; ++m)
            qf[m] = *reinterpret_cast<const u32x4_t *>(qp + m * 64);
    }
    f32x4_t oacc[AB_NC];
#pragma unroll
    for (int n = 0; n < AB_NC; ++n)
        oacc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_part = 0.f;

    const unsigned char *kvb =
        reinterpret_cast<const unsigned char *>(kv) + b * (int64_t)n_k * row_stride * 2;

    // DMA one tile: wave instruction s (1 KB) fills LDS bytes s*1024 + 16*lane
    // = (row, physical chunk) from the logical chunk of that row's key.  Wave
    // w issues instructions w + 8i for i < 4, and waves 0-3 also w + 32.  The
    // (row, byte offset) of each of this lane's slots is fixed and packed in
    // one register; the keys are looked up first so the list reads overlap.
    // Offsets are 32-bit (the host keeps 2*row_stride below 2^31).
    uint32_t dma_slot[AB_DMA_HI];
#pragma unroll
    for (int i = 0; i < AB_DMA_HI; ++i) {
        const int c = min(wid + i * AB_NW, AB_DMA - 1) * 64 + lane;
        dma_slot[i] = ((uint32_t)(c / AB_CPR) << 16) |
                      (uint32_t)(((c % AB_CPR) ^ chunk_swz_odd(c / AB_CPR)) * 16);
    }
    const uint32_t rs2 = (uint32_t)(row_stride * 2);
    const bool dma_extra = wid < AB_DMA - AB_DMA_LO * AB_NW;
    auto dma_tile = [&](unsigned char *dst, int t0, int nvalid) {
        const int32_t *lst = sm_list + t0;
        int key[AB_DMA_HI];
#pragma unroll
        for (int i = 0; i < AB_DMA_HI; ++i)
            key[i] = lst[min((int)(dma_slot[i] >> 16), nvalid - 1)];
#pragma unroll
        for (int i = 0; i < AB_DMA_LO; ++i)
            lds_dma16(kvb + (uint64_t)(uint32_t)key[i] * rs2 + (dma_slot[i] & 0xffffu),
                      dst + (wid + i * AB_NW) * 1024);
        if (dma_extra)
            lds_dma16(kvb + (uint64_t)(uint32_t)key[AB_DMA_LO] * rs2 +
                          (dma_slot[AB_DMA_LO] & 0xffffu),
                      dst + (wid + AB_DMA_LO * AB_NW) * 1024);
    };

    // Per-lane LDS byte offsets inside a tile (constant over tiles).
    //  Q.K^T: lane reads rows col and 16+col at logical chunk 4*ks + g =
    //  8m + 4*half + g; the swizzle only touches the low 3 bits, so that is
    //  physical chunk 8m + ((4*half + g) ^ swz(col)): one base, immediates.
    const uint32_t qk_base = (col * AB_CPR + ((4 * half + g) ^ chunk_swz_odd(col))) * 16;
    //  P.V: the V^T fragment of output column tile n = 16*half + 8M + r is
    //  read transposed from rows ra and 16+ra at logical chunk 2n + hb, i.e.
    //  physical chunk 32*half + 16M + 8(r>>2) + ((2(r&3) + hb) ^ swz(ra)):
    //  four bases (r & 3) plus immediates; byte (col&1)*8 inside the chunk.
    const int ra = 4 * g + (col >> 2);
    const int hb = (col & 3) >> 1;
    const int swr = chunk_swz_odd(ra);
    uint32_t pv_base[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        pv_base[r] = (ra * AB_CPR + ((2 * r + hb) ^ swr)) * 16 + (col & 1) * 8 + half * 512;
    const uint32_t lds_tiles = lds_addr(sm.u.tile[0]);

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
        const int before = block_exclusive_scan<AB_NT>(cnt, sm_wave_tot, total);
        const int r0 = (int)(((int64_t)total * split) / splits);
        const int r1 = (int)(((int64_t)total * (split + 1)) / splits);
        const int rb = r0 + batch * AB_LIST;
        if (rb >= r1)
            break;
        const int re = min(rb + AB_LIST, r1);
        extract_keys(sm.u.bitmap, w0, w1, before, rb, re, sm_list);
        __syncthreads();
        const int n_my = re - rb;
        const int ntiles = (n_my + AB_TILE - 1) / AB_TILE;
        // the Q fragments (and anything else loaded so far) are in registers
        // before the first tile DMA, so no later wait is needed for them
        vm_wait<0>();

        // ring of AB_STAGES tiles: tiles t+1 .. t+AB_STAGES-1 are in flight
        // while tile t is consumed
        for (int s = 0; s < AB_STAGES - 1 && s < ntiles; ++s)
            dma_tile(sm.u.tile[s], s * AB_TILE, min(AB_TILE, n_my - s * AB_TILE));
        for (int t = 0; t < ntiles; ++t) {
            const int t0 = t * AB_TILE;
            const int nvalid = min(AB_TILE, n_my - t0);
            // tile t has landed (this wave's DMA; the later tiles may still fly)
            const int after = min(ntiles - 1, t + AB_STAGES - 2) - t;
            if (wid < AB_NW / 2)
                vm_wait_tiles<AB_DMA_HI>(after);
            else
                vm_wait_tiles<AB_DMA_LO>(after);
            lds_barrier();  // ... for every wave, and tile t-1's buffer is free
            const int tn = t + AB_STAGES - 1;
            if (tn < ntiles)
                dma_tile(sm.u.tile[tn % AB_STAGES], tn * AB_TILE,
                         min(AB_TILE, n_my - tn * AB_TILE));
            const int toff = (t % AB_STAGES) * AB_TILEB;

            // ---- partial S^T[key][head] over this wave's 9 k-steps: keys
            //      0-15 (s0) and 16-31 (s1), two chains each; operands read in
            //      groups of 3 k-steps
            f32x4_t s0a = {0.f, 0.f, 0.f, 0.f}, s0b = s0a, s1a = s0a, s1b = s0a;
            {
                const uint32_t kb = lds_tiles + toff + qk_base;
                constexpr int R16 = 16 * AB_ROWB;  // rows 16..31
                auto qk_group = [&](auto J, const u32x4_t(&a)[6]) {
                    constexpr int j = decltype(J)::value;
#pragma unroll
                    for (int u = 0; u < 3; ++u) {
                        const int m = 3 * j + u;
                        if (m & 1) {
                            s0b = mfma_16x16x32(a[2 * u], qf[m], s0b);
                            s1b = mfma_16x16x32(a[2 * u + 1], qf[m], s1b);
                        } else {
                            s0a = mfma_16x16x32(a[2 * u], qf[m], s0a);
                            s1a = mfma_16x16x32(a[2 * u + 1], qf[m], s1a);
                        }
                    }
                };
                u32x4_t a[6];
                lds_read_b128_x6<0, R16>(a, kb);
                qk_group(std::integral_constant<int, 0>{}, a);
                lds_read_b128_x6<384, R16>(a, kb);
                qk_group(std::integral_constant<int, 1>{}, a);
                lds_read_b128_x6<768, R16>(a, kb);
                qk_group(std::integral_constant<int, 2>{}, a);
            }
            f32x4_t s0 = s0a + s0b, s1 = s1a + s1b;
            // ---- add the partner's partial (same lane layout); a + b == b + a,
            //      so both waves hold bit-identical scores
            sm_xs[wid][0][lane] = s0;
            sm_xs[wid][1][lane] = s1;
            lds_barrier();
            s0 += sm_xs[wid ^ (AB_NW / 2)][0][lane];
            s1 += sm_xs[wid ^ (AB_NW / 2)][1][lane];

            // ---- online softmax (log2 domain); lane's keys: 4g+i and 16+4g+i
            float x0[4], x1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x0[i] = s0[i] * scale_log2;
                x1[i] = s1[i] * scale_log2;
            }
            if (nvalid < AB_TILE) {  // ragged last tile: rows past the end are padding
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x0[i] = (4 * g + i < nvalid) ? x0[i] : -INFINITY;
                    x1[i] = (16 + 4 * g + i < nvalid) ? x1[i] : -INFINITY;
                }
            }
            float tmax = fmaxf(fmaxf(fmaxf(x0[0], x0[1]), fmaxf(x0[2], x0[3])),
                               fmaxf(fmaxf(x1[0], x1[1]), fmaxf(x1[2], x1[3])));
            tmax = max_across_rows(tmax);
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
            // x - m_ref <= kRescaleLog2, so the hardware exp2 (no denormal
            // results) is all that is needed.
            const float m_ref = (m_run == -INFINITY) ? 0.f : m_run;
            float p[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = __builtin_amdgcn_exp2f(x0[i] - m_ref);
                p[4 + i] = __builtin_amdgcn_exp2f(x1[i] - m_ref);
            }
            l_part += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            // ---- P^T fragments (B operand): element j <-> key 4g+j (j < 4),
            //      16+4g+(j-4) (j >= 4); two-term bf16 split
            u32x4_t bhi, blo;
            {
                uint32_t h[4], l[4];
                split_bf16x8(p, h, l);
                bhi = u32x4_t{h[0], h[1], h[2], h[3]};
                blo = u32x4_t{l[0], l[1], l[2], l[3]};
            }
            // ---- O^T[c][head] += V^T[c][keys] P^T[keys][head], 8 column tiles
            //      per group: 16 transposing reads, then the hi terms of all 8
            //      tiles and the lo terms, so no MFMA waits on its predecessor.
            {
                const uint32_t tb = lds_tiles + toff;
                const uint32_t b0 = tb + pv_base[0], b1 = tb + pv_base[1];
                const uint32_t b2 = tb + pv_base[2], b3 = tb + pv_base[3];
                auto pv_group = [&](auto M, const u32x2_t(&va)[8], const u32x2_t(&vb)[8]) {
                    constexpr int m = decltype(M)::value;
                    u32x4_t av[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        av[r] = u32x4_t{va[r][0], va[r][1], vb[r][0], vb[r][1]};
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        oacc[8 * m + r] = mfma_16x16x32(av[r], bhi, oacc[8 * m + r]);
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        oacc[8 * m + r] = mfma_16x16x32(av[r], blo, oacc[8 * m + r]);
                };
                constexpr int ROW16 = 16 * AB_ROWB;
                u32x2_t va[8], vb[8];
                lds_read_tr16x4_x16<0, 128, ROW16>(va, vb, b0, b1, b2, b3);
                pv_group(std::integral_constant<int, 0>{}, va, vb);
                lds_read_tr16x4_x16<256, 384, ROW16>(va, vb, b0, b1, b2, b3);
                pv_group(std::integral_constant<int, 1>{}, va, vb);
            }
        }
        __syncthreads();  // last tile consumed before the bitmap reuses LDS
    }

    // ---- epilogue: l over the 4 lane groups of the head
    const float l_tot = sum_across_rows(l_part);
    if (splits == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *op = out + ((int64_t)row * AB_H + head) * AB_VD + half * (AB_VD / 2) + 4 * g;
#pragma unroll
        for (int n = 0; n < AB_NC; ++n)
            *reinterpret_cast<f32x4_t *>(op + n * 16) = oacc[n] * inv;
        if (lse && half == 0 && g == 0)
            lse[(int64_t)row * AB_H + head] =
                l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
        const int64_t pr_ = ((int64_t)row * splits + split) * AB_H + head;
        float *op = ws_o + pr_ * AB_VD + half * (AB_VD / 2) + 4 * g;
#pragma unroll
        for (int n = 0; n < AB_NC; ++n)
            *reinterpret_cast<f32x4_t *>(op + n * 16) = oacc[n];
        if (half == 0 && g == 0) {
            ws_ml[pr_ * 2] = l_tot > 0.f ? m_run : -INFINITY;
            ws_ml[pr_ * 2 + 1] = l_tot;
        }
    }
}

// Merge the split partials of each (row, head):
//   O = sum_s 2^(m_s - m) O_s / L,  L = sum_s 2^(m_s - m) l_s,  m = max_s m_s.
// One block per (row, 4 heads), one wave per head; lane j owns columns
// 8j .. 8j+7 of the 512, so every split's partial row is one coalesced 2 KB
// read.  Blocks follow the gather kernel's XCD order, so a row's partials are
// read back from the L2 they were written to.
constexpr int CB_HEADS = 4;
__global__ __launch_bounds__(64 * CB_HEADS) void attend_combine_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_ml, float *__restrict__ out,
    float *__restrict__ lse, int splits)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int row = lb / (AB_H / CB_HEADS);
    const int h = (lb % (AB_H / CB_HEADS)) * CB_HEADS + wid;
    // lane s < splits holds split s's (m, l)
    float ms = -INFINITY, ls = 0.f;
    if (lane < splits) {
        const int64_t pr = ((int64_t)row * splits + lane) * AB_H + h;
        ms = ws_ml[pr * 2];
        ls = ws_ml[pr * 2 + 1];
    }
    const float m = wave_max(ms);
    const float wgt = (ms == -INFINITY) ? 0.f : exp2f(ms - m);
    const float L = wave_sum(wgt * ls);
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
    for (int s = 0; s < splits; ++s) {
        const float ws_ = __shfl(wgt, s, kWave);
        if (ws_ != 0.f) {
            const f32x4_t *src = reinterpret_cast<const f32x4_t *>(
                ws_o + (((int64_t)row * splits + s) * AB_H + h) * AB_VD + 8 * lane);
            a0 += ws_ * src[0];
            a1 += ws_ * src[1];
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    f32x4_t *dst = reinterpret_cast<f32x4_t *>(out + ((int64_t)row * AB_H + h) * AB_VD + 8 * lane);
    dst[0] = a0 * inv;
    dst[1] = a1 * inv;
    if (lse && lane == 0)
        lse[(int64_t)row * AB_H + h] = L > 0.f ? (m + log2f(L)) * kLn2 : -INFINITY;
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
           a.v == a.k && a.v_row_stride == a.k_row_stride && a.k_row_stride % 8 == 0 &&
           a.k_row_stride >= AB_KD && a.k_row_stride < (1ll << 30);
}

int attend_gather_splits(const AttendArgs &a)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    int by_fill = (int)((256 + rows - 1) / rows);
    int by_work = max(1, min(a.n_sel, a.n_k) / 64);
    // the merge kernel keeps one split per lane
    return max(1, min(min(by_fill, by_work), 64));
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
        hipLaunchKernelGGL(attend_combine_kernel, dim3((unsigned)(rows * (AB_H / CB_HEADS))),
                           dim3(64 * CB_HEADS), 0, st, ws_o, ws_ml, a.out, a.lse, splits);
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
