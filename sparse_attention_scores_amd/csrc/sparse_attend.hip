// sparse_attend.hip -- sparse attention over each query's selected keys.
//
// out[h] = sum_{j in J} softmax_j(scale * q_h . K_j) V_j over the set J of
// distinct, in-range, non-INVALID, visible indices of the query's row
// ("GLM-5.2: the DSA sparse attention moves onto the pure fak kernel",
// table under "What changed"; "Module glm5next_dsa_ref", topk_to_mask and
// mla_masked_attention).
//
// Set semantics: a row's selected set has each valid key once.  The gather
// kernel first takes the valid entries in index order (rows without a
// repeated key, the case of every top-k output) and checks behind the first
// tiles, with an LDS bitmap over the n_k keys, that no key repeats; a row
// that has one is redone from the bitmap, whose popcount prefix sums give
// each block its share of the set bits in ascending key order (duplicates
// collapse there).  The other kernels always use the bitmap.  Either way a
// row's keys are processed in a fixed order, so results are deterministic.
//
// Gather kernel (absorbed MLA: one 576-wide latent row per key, shared by
// all 64 heads, V = its first 512 columns):
//  * block = 4 waves (one per SIMD) x 16 heads of one query, over a
//    contiguous share of the query's selected keys (split-K across blocks
//    when there are few queries, merged by a combine kernel);
//  * per tile of 32 keys the rows are gathered once into LDS with
//    direct-to-LDS loads (16 bytes per lane) through a three-stage ring, and
//    read by all 4 waves (64 heads): row-major for Q.K^T, transposed for P.V;
//  * S^T = K Q^T on 16x16x32 bf16 MFMA with Q held in registers; online
//    softmax in f32 (exp2, log2e folded into the scale);
//  * O^T += V^T P^T on MFMA, with P entering as a two-term bf16 split
//    (hi + lo, about 16 significant bits) so the rounding of the weights
//    stays far below the tolerance; each lane's accumulators all belong to
//    one head, so the softmax rescale needs no cross-lane traffic.
#include "attend_set.hpp"
#include "dsa_device.hpp"
#include "dsa_internal.hpp"

#include <float.h>
#include <math.h>

#include <type_traits>

namespace dsa {

// ------------------------------------------------------------------ gather kernel
constexpr int AB_H = kAbsHeads;                    // heads of the absorbed attention
constexpr int AB_KD = kAbsKd;
constexpr int AB_VD = kAbsVd;
constexpr int AB_TILE = 32;                   // keys per LDS tile
constexpr int AB_KS = AB_KD / 32;             // 18 k-steps of the 16x16x32 MFMA
constexpr int AB_ROWB = AB_KD * 2;            // 1152 bytes per latent row
constexpr int AB_CPR = AB_ROWB / 16;          // 72 16-byte chunks per row
constexpr int AB_TILEB = AB_TILE * AB_ROWB;   // 36 KB per tile
constexpr int AB_DMA = AB_TILEB / 1024;       // 36 one-KB wave DMA instructions per tile
constexpr int AB_CW = 4;                      // compute waves, one per SIMD: 16 heads each
constexpr int AB_CT = 64 * AB_CW;             // compute threads
constexpr int AB_NL = 2;                      // loader waves
constexpr int AB_NT = AB_CT + 64 * AB_NL;     // plus the loader waves
constexpr int AB_NC = AB_VD / 16;             // 32 output column tiles per wave
constexpr int AB_STAGES = 3;                  // tiles resident in LDS (ring)
constexpr int AB_DMA_L = AB_DMA / AB_NL;      // 18 of them per loader wave
constexpr int AB_EARLY = 6;                   // loader's DMAs of tile j issued before tile j-1 is released
constexpr int AB_KB = 6;                      // loader key reads per LDS batch
constexpr int AB_LIST = 2048;                 // keys per batch of a block
constexpr int AB_IDX_U = 8;                   // fast path: row entries per thread (n_sel <= 2048)
constexpr int AB_SET_WORDS = kAbsMaxKeys / 32;           // set bitmap of the row: n_k <= 262144
static_assert(AB_DMA % AB_NL == 0 && AB_DMA_L % AB_KB == 0 && AB_EARLY % AB_KB == 0 &&
                  AB_EARLY < AB_DMA_L,
              "each loader issues whole key batches");
static_assert(AB_LIST == AB_CT * AB_IDX_U, "the fast path lists a whole row");

// LDS tile: 32 latent rows, 1152 bytes apart, with the 16-byte chunks of row
// r stored XOR-swizzled (chunk_swz_odd) so that both the row-wise Q.K^T operand
// reads and the transposing P.V operand reads spread over all banks.  V is
// the first 512 columns of the same rows.
// The tiles are the only LDS object the direct-to-LDS loads write, and they
// are only read through asm; the other LDS data live in objects of their own,
// so the compiler can tell them apart and puts no wait for the tile loads in
// front of their accesses.
struct __attribute__((aligned(16))) AbsTiles {
    unsigned char tile[AB_STAGES][AB_TILEB];
};

// Block = (query row, key split): 4 compute waves (one per SIMD) and two
// loader waves.  Compute wave w owns heads 16w .. 16w+15 with Q for all 576
// dims and O for all 512 columns in registers, and every key of every tile;
// each tile (loaded once, 36 KB) feeds all 64 heads.  The loader waves issue
// every direct-to-LDS load of the tiles (half each), so the compute waves
// never stall on a full memory queue: a wave that issues loads waits at each
// one until the queue takes it, and while the kernel streams rows the queue
// is full.  Two loaders keep more loads in flight than one, which alone
// held a CU near 10 bytes per cycle.  Tile j's first AB_EARLY loads (per
// loader) are issued before the loaders wait for tile j-1, so the queue
// stays fed across the barrier that releases tile j-1.
//
// Which keys: the selected set of the row (distinct, in range, visible) is
// split into `splits` contiguous shares.  Fast path (n_sel <= 2048): the
// valid entries are listed in index order and the shares taken from that
// list, so the tiles start streaming at once; the loader waves build the
// row's set bitmap from the list while the last tile is computed, and if it
// holds fewer keys than there were valid entries (a key repeats) the block
// starts over from the bitmap (keys in ascending order, duplicates
// collapsed).  Rows with n_sel > 2048 go to the bitmap directly.
// The two roles are separate instantiations, so the registers of one (Q and
// O of the compute waves, the load slots of the loaders) are not live in the
// other; they share only LDS and the barriers, which both pass in the same
// sequence.
struct AbsShared {
    AbsTiles sm;
    int32_t list[AB_LIST];
    uint32_t set[AB_SET_WORDS];
    int wave_tot[AB_CW];
};

template <bool LOADER>
__device__ __forceinline__ void attend_gather_role(
    AbsShared &shm, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    int64_t row_stride, const int32_t *__restrict__ idx, const int32_t *__restrict__ vlo,
    const int32_t *__restrict__ vhi, float *__restrict__ out, float *__restrict__ lse,
    uint16_t *__restrict__ ws_o, f32x4_t *__restrict__ ws_ml, int n_q, int n_k, int n_sel,
    int splits, float scale_log2)
{
    AbsTiles &sm = shm.sm;
    int32_t *sm_list = shm.list;
    uint32_t *sm_set = shm.set;
    int *sm_wave_tot = shm.wave_tot;
    constexpr bool loader = LOADER;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lw = LOADER ? wid - AB_CW : 0;  // loader wave index
    const int g = lane >> 4, col = lane & 15;
    // the splits of one row run on one XCD (shared q, idx and partials);
    // without splits the rows keep launch order, which spreads the uneven
    // causal rows evenly over the XCDs
    const int lb = splits > 1 ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;
    const int row = lb / splits;
    const int split = lb - row * splits;
    const int64_t bseq = row / n_q;
    const int32_t *idx_row = idx + (int64_t)row * n_sel;
    const int nw = (n_k + 31) >> 5;
    bool fast = n_sel <= AB_LIST;

    // compute threads request the row's indices first (thread t: entries
    // 8t .. 8t+7), then Q; the validity scan below waits for the indices alone
    int ent[AB_IDX_U];
    if (fast && !loader) {
#pragma unroll
        for (int u = 0; u < AB_IDX_U; ++u) {
            const int i = AB_IDX_U * tid + u;
            ent[u] = i < n_sel ? idx_row[i] : -1;
        }
    }

    // Q^T fragments (B operand) of all 18 k-steps: lane holds head
    // 16w + col, dims 32ks + 8g .. +8
    const int head = min(wid, AB_CW - 1) * 16 + col;
    u32x4_t qf[AB_KS];
    if (!loader) {
        const uint16_t *qp = q + ((int64_t)row * AB_H + head) * AB_KD + g * 8;
#pragma unroll
        for (int ks = 0; ks < AB_KS; ++ks)
            qf[ks] = *reinterpret_cast<const u32x4_t *>(qp + ks * 32);
    }
    int lo = 0, hi = n_k;
    if (vlo) {
        lo = max(vlo[row], 0);
        hi = min(vhi[row], n_k);
    }
    for (int i = tid; i < nw; i += AB_NT)
        sm_set[i] = 0u;

    f32x4_t oacc[AB_NC];
    float m_run, l_part;
    auto reset_acc = [&]() {
#pragma unroll
        for (int n = 0; n < AB_NC; ++n)
            oacc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_part = 0.f;
    };
    reset_acc();

    const unsigned char *kvb =
        reinterpret_cast<const unsigned char *>(kv) + bseq * (int64_t)n_k * row_stride * 2;
    const uint32_t rs2 = (uint32_t)(row_stride * 2);
    const uint32_t lds_tiles = lds_addr(sm.tile[0]);
    const uint32_t lds_list = lds_addr(sm_list);
    const uint32_t lds_set = lds_addr(sm_set);

    // Loaders: wave instruction s (1 KB) of a tile fills LDS bytes s*1024 +
    // 16*lane = (row, physical chunk) from the logical chunk of that row's
    // key; loader lw issues instructions 18lw .. 18lw+17.  The (row, byte
    // offset) of this lane's slot is fixed and packed in one register.
    // Offsets are 32-bit (the host keeps 2*row_stride below 2^31).
    uint32_t slot[AB_DMA_L];
    if (loader) {
#pragma unroll
        for (int s = 0; s < AB_DMA_L; ++s) {
            const int c = (lw * AB_DMA_L + s) * 64 + lane;
            slot[s] = ((uint32_t)(c / AB_CPR) << 16) |
                      (uint32_t)(((c % AB_CPR) ^ chunk_swz_odd(c / AB_CPR)) * 16);
        }
    }
    // loads [S0, S1) of the tile whose keys start at LDS byte lkeys (nvalid
    // of them; the padding rows repeat the last key)
    auto issue = [&](auto S0c, auto S1c, unsigned char *dst, uint32_t lkeys, int nvalid) {
        constexpr int S0 = decltype(S0c)::value, S1 = decltype(S1c)::value;
#pragma unroll
        for (int s = S0; s < S1; s += AB_KB) {
            uint32_t ka[AB_KB], key[AB_KB];
#pragma unroll
            for (int b = 0; b < AB_KB; ++b)
                ka[b] = lkeys + 4u * (uint32_t)min((int)(slot[s + b] >> 16), nvalid - 1);
            lds_read_u32_x6(key, ka);
#pragma unroll
            for (int b = 0; b < AB_KB; ++b)
                lds_dma16(kvb + (uint64_t)key[b] * rs2 + (slot[s + b] & 0xffffu),
                          dst + (lw * AB_DMA_L + s + b) * 1024);
        }
    };

    // Per-lane LDS byte offsets inside a tile (constant over tiles).
    //  Q.K^T: lane reads rows col and 16+col (same swizzle) at logical chunk
    //  4ks + g, i.e. physical chunk 8(ks>>1) + ((4(ks&1) + g) ^ swz(col)): an
    //  even and an odd base plus immediates.
    constexpr int R16 = 16 * AB_ROWB;
    const uint32_t qk_e = (col * AB_CPR + (g ^ chunk_swz_odd(col))) * 16;
    const uint32_t qk_o = (col * AB_CPR + ((4 + g) ^ chunk_swz_odd(col))) * 16;
    //  P.V: the V^T fragment of column tile n is read transposed from rows
    //  ra = 4g + (col>>2) and 16+ra at logical chunk 2n + hb, i.e. physical
    //  chunk 8(n>>2) + ((2(n&3) + hb) ^ swz(ra)): four bases (n & 3) plus
    //  immediates; byte (col&1)*8 inside the chunk.  Lane (col, g) receives
    //  V[4g + j][16n + col] and V[16 + 4g + j][16n + col], j < 4.
    const int ra = 4 * g + (col >> 2);
    const int hb = (col & 3) >> 1;
    const int swr = chunk_swz_odd(ra);
    uint32_t pv_base[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        pv_base[r] = (ra * AB_CPR + ((2 * r + hb) ^ swr)) * 16 + (col & 1) * 8;

    // One tile of a compute wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
    auto compute_tile = [&](uint32_t tb, int nvalid) {
        // ---- S^T[key][head]: keys 0-15 (s0) and 16-31 (s1).  Operand read
        //      i = 2ks + r (k-step ks, row block r) is issued three reads ahead
        //      of its MFMA: with the registers this wave has left, the
        //      compiler would otherwise issue each read right before its MFMA
        //      and wait out the whole LDS latency 36 times per tile.
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
        {
            const uint32_t be = tb + qk_e, bo = tb + qk_o;
            u32x4_t a[2 * AB_KS];
            auto rd = [&](auto Ic) {
                constexpr int i = decltype(Ic)::value, ks = i >> 1, r = i & 1;
                lds_read_b128_nowait<128 * (ks >> 1) + r * R16>(a[i], (ks & 1) ? bo : be);
            };
            auto step = [&](auto Ic) {
                constexpr int i = decltype(Ic)::value, ks = i >> 1;
                constexpr int n = 2 * AB_KS;
                if constexpr (i + 3 < n) {
                    rd(std::integral_constant<int, i + 3>{});
                    lds_operand_wait<3>(a[i]);
                } else {
                    lds_operand_wait<n - 1 - i>(a[i]);
                }
                // the empty asm keeps each MFMA between its wait and the next
                // read (the scheduler would otherwise sink them all, and keep
                // every operand live)
                if constexpr ((i & 1) == 0) {
                    s0 = mfma_16x16x32(a[i], qf[ks], s0);
                    asm volatile("" : "+v"(s0));
                } else {
                    s1 = mfma_16x16x32(a[i], qf[ks], s1);
                    asm volatile("" : "+v"(s1));
                }
            };
            rd(std::integral_constant<int, 0>{});
            rd(std::integral_constant<int, 1>{});
            rd(std::integral_constant<int, 2>{});
            static_assert(2 * AB_KS == 36, "36 operand reads");
#define AB_QK_STEP(I) step(std::integral_constant<int, I>{});
            AB_QK_STEP(0) AB_QK_STEP(1) AB_QK_STEP(2) AB_QK_STEP(3) AB_QK_STEP(4) AB_QK_STEP(5)
            AB_QK_STEP(6) AB_QK_STEP(7) AB_QK_STEP(8) AB_QK_STEP(9) AB_QK_STEP(10) AB_QK_STEP(11)
            AB_QK_STEP(12) AB_QK_STEP(13) AB_QK_STEP(14) AB_QK_STEP(15) AB_QK_STEP(16)
            AB_QK_STEP(17) AB_QK_STEP(18) AB_QK_STEP(19) AB_QK_STEP(20) AB_QK_STEP(21)
            AB_QK_STEP(22) AB_QK_STEP(23) AB_QK_STEP(24) AB_QK_STEP(25) AB_QK_STEP(26)
            AB_QK_STEP(27) AB_QK_STEP(28) AB_QK_STEP(29) AB_QK_STEP(30) AB_QK_STEP(31)
            AB_QK_STEP(32) AB_QK_STEP(33) AB_QK_STEP(34) AB_QK_STEP(35)
#undef AB_QK_STEP
        }

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
        // ---- O^T[c][head] += V^T[c][keys] P^T[keys][head], one column tile n
        //      per step: its two transposing reads are issued three tiles
        //      ahead, and step n runs the hi term of tile n and the lo term of
        //      tile n-1, so no MFMA waits on its predecessor
        {
            const uint32_t b0 = tb + pv_base[0], b1 = tb + pv_base[1];
            const uint32_t b2 = tb + pv_base[2], b3 = tb + pv_base[3];
            u32x2_t va[AB_NC], vb[AB_NC];
            auto rd = [&](auto Nc) {
                constexpr int n = decltype(Nc)::value, r = n & 3, o = 128 * (n >> 2);
                const uint32_t bb = r == 0 ? b0 : r == 1 ? b1 : r == 2 ? b2 : b3;
                lds_read_tr16_nowait<o>(va[n], bb);
                lds_read_tr16_nowait<o + R16>(vb[n], bb);
            };
            auto av = [&](int n) { return u32x4_t{va[n][0], va[n][1], vb[n][0], vb[n][1]}; };
            auto step = [&](auto Nc) {
                constexpr int n = decltype(Nc)::value;
                if constexpr (n + 3 < AB_NC) {
                    rd(std::integral_constant<int, n + 3>{});
                    lds_operand_wait<6>(va[n], vb[n]);
                } else {
                    lds_operand_wait<2 * (AB_NC - 1 - n)>(va[n], vb[n]);
                }
                oacc[n] = mfma_16x16x32(av(n), bhi, oacc[n]);
                if constexpr (n > 0)
                    oacc[n - 1] = mfma_16x16x32(av(n - 1), blo, oacc[n - 1]);
            };
            rd(std::integral_constant<int, 0>{});
            rd(std::integral_constant<int, 1>{});
            rd(std::integral_constant<int, 2>{});
            static_assert(AB_NC == 32, "32 column tiles");
#define AB_PV_STEP(N) step(std::integral_constant<int, N>{});
            AB_PV_STEP(0) AB_PV_STEP(1) AB_PV_STEP(2) AB_PV_STEP(3) AB_PV_STEP(4) AB_PV_STEP(5)
            AB_PV_STEP(6) AB_PV_STEP(7) AB_PV_STEP(8) AB_PV_STEP(9) AB_PV_STEP(10) AB_PV_STEP(11)
            AB_PV_STEP(12) AB_PV_STEP(13) AB_PV_STEP(14) AB_PV_STEP(15) AB_PV_STEP(16)
            AB_PV_STEP(17) AB_PV_STEP(18) AB_PV_STEP(19) AB_PV_STEP(20) AB_PV_STEP(21)
            AB_PV_STEP(22) AB_PV_STEP(23) AB_PV_STEP(24) AB_PV_STEP(25) AB_PV_STEP(26)
            AB_PV_STEP(27) AB_PV_STEP(28) AB_PV_STEP(29) AB_PV_STEP(30) AB_PV_STEP(31)
#undef AB_PV_STEP
            oacc[AB_NC - 1] = mfma_16x16x32(av(AB_NC - 1), blo, oacc[AB_NC - 1]);
        }
    };

    // The tiles of the key list sm_list[first .. first + n_my) through a ring
    // of AB_STAGES buffers.  Barrier B_t releases tile t to the compute
    // waves; they reach it after finishing tile t-1, so once past B_t the
    // loader may refill tile t-1's buffer with tile t+2.  Both roles pass
    // the same ntiles barriers, then one more after the last tile.
    auto run_tiles = [&](int first, int n_my) {
        const int ntiles = (n_my + AB_TILE - 1) / AB_TILE;
        const uint32_t lkeys = lds_list + 4u * (uint32_t)first;
        auto tile_buf = [&](int t) { return lds_tiles + (uint32_t)((t % AB_STAGES) * AB_TILEB); };
        auto tile_ptr = [&](int t) { return sm.tile[t % AB_STAGES]; };
        auto tile_n = [&](int t) { return min(AB_TILE, n_my - t * AB_TILE); };
        if (loader) {
            if (ntiles > 0)
                issue(std::integral_constant<int, 0>{}, std::integral_constant<int, AB_DMA_L>{},
                      tile_ptr(0), lkeys, tile_n(0));
            for (int j = 1; j <= ntiles; ++j) {
                // tile j's first loads, then tile j-1 has landed: release it
                if (j < ntiles) {
                    issue(std::integral_constant<int, 0>{},
                          std::integral_constant<int, AB_EARLY>{}, tile_ptr(j),
                          lkeys + 4u * (uint32_t)(j * AB_TILE), tile_n(j));
                    vm_wait<AB_EARLY>();
                } else {
                    vm_wait<0>();
                }
                lds_barrier();  // B_{j-1}
                if (j < ntiles)
                    issue(std::integral_constant<int, AB_EARLY>{},
                          std::integral_constant<int, AB_DMA_L>{}, tile_ptr(j),
                          lkeys + 4u * (uint32_t)(j * AB_TILE), tile_n(j));
            }
        } else {
            // the Q fragments (and anything else loaded) are in registers
            vm_wait<0>();
            for (int t = 0; t < ntiles; ++t) {
                lds_barrier();  // B_t
                compute_tile(tile_buf(t), tile_n(t));
            }
        }
    };

    int n_valid = 0;
    if (fast) {
        // valid entries, their ranks in index order (entry order = position);
        // the whole list goes to sm_list
        uint32_t vm = 0;
        int c = 0, incl = 0;
        if (!loader) {
#pragma unroll
            for (int u = 0; u < AB_IDX_U; ++u)
                vm |= (ent[u] >= lo && ent[u] < hi) ? 1u << u : 0u;  // lo >= 0: INVALID drops
            c = __popc(vm);
            incl = wave_inclusive_scan(c);
            if (lane == 63)
                sm_wave_tot[wid] = incl;
        }
        __syncthreads();  // also orders the set-bitmap clear before the inserts
        int before = 0;
#pragma unroll
        for (int i = 0; i < AB_CW; ++i) {
            const int t = sm_wave_tot[i];
            before += i < wid ? t : 0;
            n_valid += t;
        }
        if (!loader) {
            int rank = before + incl - c;
#pragma unroll
            for (int u = 0; u < AB_IDX_U; ++u) {
                if (vm & (1u << u))
                    sm_list[rank++] = ent[u];
            }
        }
        __syncthreads();
    } else {
        // the set bitmap of the whole row, in one pass
        int first[8];
        if (!loader)
            load_indices<AB_CT, 8>(first, idx_row, n_sel, 0);
        __syncthreads();  // the clear above is complete
        if (!loader) {
            for (int base = 0; base < n_sel; base += AB_CT * 8) {
                if (base > 0)
                    load_indices<AB_CT, 8>(first, idx_row, n_sel, base);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = first[u];
                    if (j >= lo && j < hi)
                        atomicOr(&sm_set[j >> 5], 1u << (j & 31));
                }
            }
        }
        __syncthreads();
    }

    int c0, c1;
    wave_chunk_range<AB_CW>(nw, min(wid, AB_CW - 1), c0, c1);
    // balanced contiguous shares of `total` keys: the first total % splits
    // get one more
    auto share = [&](int total, int &r0, int &r1) {
        const int per = total / splits, extra = total % splits;
        r0 = split * per + min(split, extra);
        r1 = r0 + per + (split < extra ? 1 : 0);
    };
    bool restart = false;
    for (int batch = fast ? -1 : 0;; ++batch) {
        if (restart) {  // a key repeats: start over on the bitmap
            reset_acc();
            restart = false;
        }
        // this batch: list entries [first, first + n_my); the fast path's
        // list is the whole row, the slow path's one batch of its share
        int first = 0, n_my = 0, re = 0, r1 = 0;
        if (batch < 0) {
            share(n_valid, first, r1);
            n_my = r1 - first;
        } else {
            // Slow path: the block's share is ranks [r0, r1) of the selected
            // set in ascending key order, in batches of AB_LIST keys.
            int before = 0, total = 0;
            if (!loader) {
                const int wcnt = wave_chunk_count(sm_set, nw, c0, c1);
                if (lane == 0)
                    sm_wave_tot[wid] = wcnt;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < AB_CW; ++i) {
                const int t = sm_wave_tot[i];
                before += i < wid ? t : 0;
                total += t;
            }
            int r0;
            share(total, r0, r1);
            const int rb = r0 + batch * AB_LIST;
            if (rb >= r1)
                break;
            re = min(rb + AB_LIST, r1);
            if (!loader)
                wave_chunk_extract(sm_set, nw, c0, c1, before, rb, re, sm_list);
            __syncthreads();
            n_my = re - rb;
        }
        run_tiles(first, n_my);
        if (batch < 0 && loader) {
            // the loaders put the listed entries into the set bitmap while
            // the compute waves finish the last tile
            for (int i0 = lw * 64 * AB_KB; i0 < n_valid; i0 += 64 * AB_KB * AB_NL) {
                uint32_t ka[AB_KB], key[AB_KB];
#pragma unroll
                for (int b = 0; b < AB_KB; ++b)
                    ka[b] = lds_list + 4u * (uint32_t)min(i0 + 64 * b + lane, n_valid - 1);
                lds_read_u32_x6(key, ka);
#pragma unroll
                for (int b = 0; b < AB_KB; ++b)
                    lds_or_async(lds_set + (key[b] >> 5) * 4u, 1u << (key[b] & 31));
            }
        }
        lds_barrier();  // every insert is in, every wave is done with the tiles and the list
        if (batch < 0) {
            // fewer set bits than valid entries means a key repeats in the row
            if (!loader) {
                const int wcnt = wave_chunk_count(sm_set, nw, c0, c1);
                if (lane == 0)
                    sm_wave_tot[wid] = wcnt;
            }
            __syncthreads();
            int bits = 0;
#pragma unroll
            for (int i = 0; i < AB_CW; ++i)
                bits += sm_wave_tot[i];
            if (bits == n_valid)
                break;
            restart = true;
            __syncthreads();  // sm_wave_tot is rewritten by the first batch
            continue;
        }
        if (re >= r1)
            break;
    }
    if (loader)
        return;

    // ---- epilogue: l over the 4 lane groups of the head
    const float l_tot = sum_across_rows(l_part);
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
        // Split partial: O in fp16 with a power-of-two scale per (row, split,
        // head) that puts the head's largest |O| in [2^14, 2^15), so every
        // element keeps fp16's 11 significant bits (more than the bf16
        // operands carry) whatever the magnitude of V; O = stored * 2^e.
        float amax = 0.f;
#pragma unroll
        for (int n = 0; n < AB_NC; ++n)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(oacc[n][0]), fabsf(oacc[n][1])),
                                     fmaxf(fabsf(oacc[n][2]), fabsf(oacc[n][3]))));
        amax = max_across_rows(amax);
        const int e = __builtin_amdgcn_frexp_expf(amax) - 15;
        const int64_t pr_ = ((int64_t)row * splits + split) * AB_H + head;
        // The wave's 16 x 512 fp16 block goes through LDS (the tile ring is
        // free now; each wave has a region of its own) so that every store
        // instruction writes one whole 1 KB head row: the accumulator layout
        // would scatter each store over 16 rows in 32-byte pieces.  Rows are
        // padded by 16 bytes to spread the transposing writes over the banks.
        constexpr int SROW = AB_VD + 8;  // fp16 per staged row
        static_assert(AB_CW * 16 * SROW * 2 <= (int)sizeof(AbsTiles), "staging fits the tiles");
        uint16_t *stg = reinterpret_cast<uint16_t *>(sm.tile[0]) + wid * 16 * SROW;
#pragma unroll
        for (int n = 0; n < AB_NC; ++n) {
            typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
            const f32x4_t sc = {ldexpf(oacc[n][0], -e), ldexpf(oacc[n][1], -e),
                                ldexpf(oacc[n][2], -e), ldexpf(oacc[n][3], -e)};
            *reinterpret_cast<u32x2_t *>(stg + col * SROW + 16 * n + 4 * g) =
                __builtin_bit_cast(u32x2_t, __builtin_convertvector(sc, h4_t));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint16_t *op = ws_o + (pr_ - col) * AB_VD + 8 * lane;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            *reinterpret_cast<u32x4_t *>(op + r * AB_VD) =
                *reinterpret_cast<const u32x4_t *>(stg + r * SROW + 8 * lane);
        if (g == 0)
            ws_ml[pr_] = f32x4_t{l_tot > 0.f ? m_run : -INFINITY, l_tot, (float)e, 0.f};
    }
}

__global__ __launch_bounds__(AB_NT) void attend_gather_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv, int64_t row_stride,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ vlo,
    const int32_t *__restrict__ vhi, float *__restrict__ out, float *__restrict__ lse,
    uint16_t *__restrict__ ws_o, f32x4_t *__restrict__ ws_ml, int n_q, int n_k, int n_sel,
    int splits, float scale_log2)
{
    __shared__ AbsShared shm;
    DSA_LDS_ESCAPE(shm);
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= AB_CW)
        attend_gather_role<true>(shm, q, kv, row_stride, idx, vlo, vhi, out, lse, ws_o, ws_ml,
                                 n_q, n_k, n_sel, splits, scale_log2);
    else
        attend_gather_role<false>(shm, q, kv, row_stride, idx, vlo, vhi, out, lse, ws_o, ws_ml,
                                  n_q, n_k, n_sel, splits, scale_log2);
}

// Merge the split partials of each (row, head):
//   O = sum_s 2^(m_s - m) O_s / L,  L = sum_s 2^(m_s - m) l_s,  m = max_s m_s,
// with O_s = stored_s * 2^(e_s) (fp16 partials, see the gather epilogue), so
// the weight of the stored values is 2^(m_s - m + e_s).  One block per (row,
// 4 heads), one wave per head; lane j owns columns 8j .. 8j+7 of the 512, so
// every split's partial row is one coalesced 1 KB read.  Blocks follow the
// gather kernel's XCD order, so a row's partials are read back from the L2
// they were written to.
constexpr int CB_HEADS = 4;
constexpr int CB_U = 8;
__global__ __launch_bounds__(64 * CB_HEADS) void attend_combine_kernel(
    const uint16_t *__restrict__ ws_o, const f32x4_t *__restrict__ ws_ml,
    float *__restrict__ out, float *__restrict__ lse, int splits)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int row = lb / (AB_H / CB_HEADS);
    const int h = (lb % (AB_H / CB_HEADS)) * CB_HEADS + wid;
    // lane s < splits holds split s's (m, l, e)
    float ms = -INFINITY, ls = 0.f, es = 0.f;
    if (lane < splits) {
        const f32x4_t ml = ws_ml[((int64_t)row * splits + lane) * AB_H + h];
        ms = ml[0];
        ls = ml[1];
        es = ml[2];
    }
    const float m = wave_max(ms);
    const float wgt = (ms == -INFINITY) ? 0.f : exp2f(ms - m);
    const float L = wave_sum(wgt * ls);
    const float wo = ldexpf(wgt, (int)es);  // weight of the stored fp16 values
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
    // CB_U splits per round, all loads issued before the first is used
    const uint16_t *base = ws_o + ((int64_t)row * splits * AB_H + h) * AB_VD + 8 * lane;
    const int64_t sstride = (int64_t)AB_H * AB_VD;
    typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
    for (int s0 = 0; s0 < splits; s0 += CB_U) {
        u32x4_t v[CB_U];
#pragma unroll
        for (int u = 0; u < CB_U; ++u) {
            const int s = min(s0 + u, splits - 1);
            v[u] = *reinterpret_cast<const u32x4_t *>(base + s * sstride);
        }
#pragma unroll
        for (int u = 0; u < CB_U; ++u) {
            // an empty split has weight 0 and zero partials; splits past the
            // end re-read the last one with weight 0
            const float w_ = s0 + u < splits ? __shfl(wo, s0 + u, kWave) : 0.f;
            const f32x4_t lo4 = __builtin_convertvector(
                __builtin_bit_cast(h4_t, u32x2_t{v[u][0], v[u][1]}), f32x4_t);
            const f32x4_t hi4 = __builtin_convertvector(
                __builtin_bit_cast(h4_t, u32x2_t{v[u][2], v[u][3]}), f32x4_t);
            a0 += w_ * lo4;
            a1 += w_ * hi4;
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
constexpr int PL_MAXVD = kPlainMaxVd;

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
    {
        const int32_t *idx_row = idx + (int64_t)row * n_sel;
        int first[8];
        load_indices<PL_NT, 8>(first, idx_row, n_sel, 0);
        build_bitmap<PL_NT, 8>(sm.bitmap, nw, first, idx_row, n_sel, lo, hi);
    }
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
hipError_t launch_attend(const AttendArgs &a, hipStream_t st)
{
    const int64_t rows = (int64_t)a.batch * a.n_q;
    const float scale_log2 = a.scale * kLog2e;
    if (attend_gather_supported(a)) {
        const int splits = attend_gather_splits(a);
        uint16_t *ws_o = static_cast<uint16_t *>(a.workspace);
        f32x4_t *ws_ml =
            ws_o ? reinterpret_cast<f32x4_t *>(ws_o + rows * splits * AB_H * AB_VD) : nullptr;
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
    if (attend_heads_gather_supported(a))
        return launch_attend_heads(a, st);
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
