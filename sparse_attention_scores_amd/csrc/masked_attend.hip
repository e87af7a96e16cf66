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
    extern __shared__ uint32_t bits[];  // nw words (launch size), at most MK_MAXWORDS
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

// LDS row swizzles of the per-head tiles, chosen by measurement on gfx950
// (both keep their access pattern at the full LDS rate):
//  K rows (192 bf16 = 384 bytes = 24 chunks): physical chunk = logical ^
//  ((row >> 1) & 7) -- the 32x32x16 operand reads (32 rows at one chunk);
//  V rows (256 bf16 = 512 bytes = 32 chunks, so every row starts on bank 0):
//  physical chunk = logical ^ (((row & 3) << 2) | ((row >> 2) & 3)) -- the
//  transposing reads (4 rows x 2 chunks per 16 lanes).
__device__ __forceinline__ int mk_swz_k(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int mk_swz_v(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Three 4-byte LDS reads and the wait (asm: the words arrive by direct-to-LDS
// loads, and the compiler would otherwise wait for every such load in flight).
__device__ __forceinline__ void lds_read_b32_3(uint32_t &x, uint32_t &y, uint32_t &z,
                                               uint32_t ax, uint32_t ay, uint32_t az)
{
    asm volatile(
        "ds_read_b32 %0, %3\n\t"
        "ds_read_b32 %1, %4\n\t"
        "ds_read_b32 %2, %5\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x), "=&v"(y), "=&v"(z)
        : "v"(ax), "v"(ay), "v"(az)
        : "memory");
}

constexpr int MK_STAGES = 2;  // tiles resident in LDS (ring)

template <int KD, int VD>
struct __attribute__((aligned(16))) MaskedSmem {
    static constexpr int KB = 32 * KD * 2;  // K tile bytes (32 keys, row-major, swizzled)
    static constexpr int VB = 32 * VD * 2;  // V tile bytes
    unsigned char k[MK_STAGES][KB];
    unsigned char v[MK_STAGES][VB];
    uint32_t mw[MK_STAGES][4][64];          // mask words of the tile: [wave][lane & 31]
};

// Per (sequence, head, block of 128 queries); wave w owns queries
// q0 + 32w .. +31 (lane col = query, half g = lane >> 5).  Tiles of 32 keys
// stream through a ring of MK_STAGES LDS tiles by direct-to-LDS loads, with the
// queries' mask words for the tile riding along (one 4-byte load per lane);
// each wave issues the same number of loads per tile (7 of the 28 K/V
// instructions plus its mask words), so a counted wait finds its tile.
template <int KD, int VD>
__global__ __launch_bounds__(256, 2) void attend_masked_kernel(
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
    static_assert(KD == 192 && VD == 256, "the swizzles and read groups are laid out for 192/256");
    using Sm = MaskedSmem<KD, VD>;
    constexpr int NKV = (Sm::KB + Sm::VB) / 1024;  // 28 K/V DMA instructions per tile
    constexpr int PER = NKV / 4;                   // 7 per wave
    static_assert(NKV % 4 == 0, "K/V DMA splits evenly over the waves");
    __shared__ Sm sm;
    __shared__ int sm_red[8];
    DSA_LDS_ESCAPE(sm);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
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
            sm_red[wid] = mn;
            sm_red[4 + wid] = mx;
        }
        __syncthreads();
        lo = min(min(sm_red[0], sm_red[1]), min(sm_red[2], sm_red[3]));
        hi = max(max(sm_red[4], sm_red[5]), max(sm_red[6], sm_red[7]));
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
    // mask words of this lane's query (lanes 32..63 repeat lanes 0..31; an
    // invalid query reads a valid row of the batch and is never used)
    const uint32_t *mrow =
        mask + ((int64_t)b * n_q + min(q0 + wid * 32 + col, n_q - 1)) * nw;

    // DMA: this wave issues instructions s = wid + 4i (i < 7) of the tile's 28
    // (12 for K, then 16 for V); lane l of instruction s fills LDS bytes
    // 16l of that KB = (row, physical chunk), fetching the row's logical chunk
    // (recomputed per tile: a few VALU instead of seven live registers)
    const uint32_t ksr2 = (uint32_t)(ksr * 2), vsr2 = (uint32_t)(vsr * 2);
    auto dma_tile = [&](int t, int st) {
        const int k0 = t * 32;
        // an opaque copy of the lane index keeps the compiler from hoisting the
        // seven 64-bit addresses out of the tile loop (as live registers)
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int s_ = wid + 4 * i;
            if (s_ < Sm::KB / 1024) {
                const int c = s_ * 64 + ln, r = c / KCH;
                const int key = min(k0 + r, n_k - 1);  // rows past n_k are masked
                lds_dma16(kb + (uint64_t)(uint32_t)key * ksr2 +
                              (uint32_t)(((c % KCH) ^ mk_swz_k(r)) * 16),
                          sm.k[st] + s_ * 1024);
            } else {
                const int c = (s_ - Sm::KB / 1024) * 64 + ln, r = c / VCH;
                const int key = min(k0 + r, n_k - 1);
                lds_dma16(vb + (uint64_t)(uint32_t)key * vsr2 +
                              (uint32_t)(((c % VCH) ^ mk_swz_v(r)) * 16),
                          sm.v[st] + (s_ - Sm::KB / 1024) * 1024);
            }
        }
        lds_dma4(mrow + t, sm.mw[st][wid]);
    };

    // per-lane LDS byte offsets inside a stage (constant over tiles)
    //  Q.K^T: row col, logical chunk 2ks + g = 8(ks>>2) + (2(ks&3) + g):
    //  one base per ks & 3, immediates 128 * (ks >> 2)
    const int swk = mk_swz_k(col);
    uint32_t kq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        kq[j] = (col * KCH + ((2 * j + g) ^ swk)) * 16;
    //  P.V: 16-lane group (gg, ch), lane i = a + 4j reads row kh*16 + 4gg + j
    //  (ra) and ra + 8 (rb), logical chunk 4n + c' with c' = 2ch + (a >> 1),
    //  byte 8(a & 1): 16(n >> 2) + ((4(n & 3) + c') ^ swz) -- one base per
    //  (row, n & 3), immediates 256 * (n >> 2) and 16 rows * 512 for kh
    const int grp = lane >> 4, gg = grp >> 1, ch = grp & 1;
    const int li = lane & 15, la = li & 3, lj = li >> 2;
    const int ra = 4 * gg + lj, rb = ra + 8;
    const int cp = 2 * ch + (la >> 1);
    uint32_t va_[4], vb_[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        va_[j] = (ra * VCH + ((4 * j + cp) ^ mk_swz_v(ra))) * 16 + 8 * (la & 1);
        vb_[j] = (rb * VCH + ((4 * j + cp) ^ mk_swz_v(rb))) * 16 + 8 * (la & 1);
    }
    const uint32_t lds_k = lds_addr(sm.k[0]), lds_v = lds_addr(sm.v[0]);

    // the Q fragments and ranges are in registers before the first tile DMA
    vm_wait<0>();
    for (int j = 0; j < MK_STAGES - 1 && t_begin + j < t_end; ++j)
        dma_tile(t_begin + j, j);
    for (int t = t_begin; t < t_end; ++t) {
        const int st = (t - t_begin) % MK_STAGES;
        // this wave's part of tile t has landed (later tiles may still fly)
        vm_wait_tiles<PER + 1>(min(t_end - 1, t + MK_STAGES - 2) - t);
        lds_barrier();  // ... every wave's, and tile t-1's stage is free
        if (t + MK_STAGES - 1 < t_end)
            dma_tile(t + MK_STAGES - 1, (t - t_begin + MK_STAGES - 1) % MK_STAGES);
        uint32_t word, w0, w1;
        {
            const uint32_t mb = lds_addr(&sm.mw[st][0][0]) + 4 * col;
            lds_read_b32_3(word, w0, w1, mb + 256 * wid, mb + 256 * g, mb + 256 * (2 + g));
        }
        // skip the tile when none of the block's 128 queries selects a key in it
        if (!__any((w0 | w1) != 0u))
            continue;
        // ---- S^T[key][query] for the 32 keys of the tile
        f32x16_t s = {};
        {
            const uint32_t kt = lds_k + st * Sm::KB;
            // k-step ks reads base kq[ks & 3] + 128 * (ks >> 2); the reads run
            // two k-steps ahead of the MFMAs that use them
            u32x4_t a[KS];
            lds_read_b128_nowait<0>(a[0], kt + kq[0]);
            lds_read_b128_nowait<0>(a[1], kt + kq[1]);
            auto qk = [&](auto KSc) {
                constexpr int ks = decltype(KSc)::value;
                if constexpr (ks + 2 < KS) {
                    lds_read_b128_nowait<128 * ((ks + 2) >> 2)>(a[ks + 2], kt + kq[(ks + 2) & 3]);
                    lds_operand_wait<2>(a[ks]);
                } else if constexpr (ks + 1 < KS) {
                    lds_operand_wait<1>(a[ks]);
                } else {
                    lds_operand_wait<0>(a[ks]);
                }
                s = mfma_32x32x16(a[ks], qf[ks], s);
            };
            static_assert(KS == 12, "twelve k-steps");
            qk(std::integral_constant<int, 0>{});
            qk(std::integral_constant<int, 1>{});
            qk(std::integral_constant<int, 2>{});
            qk(std::integral_constant<int, 3>{});
            qk(std::integral_constant<int, 4>{});
            qk(std::integral_constant<int, 5>{});
            qk(std::integral_constant<int, 6>{});
            qk(std::integral_constant<int, 7>{});
            qk(std::integral_constant<int, 8>{});
            qk(std::integral_constant<int, 9>{});
            qk(std::integral_constant<int, 10>{});
            qk(std::integral_constant<int, 11>{});
        }
        // lane holds keys 8*(i/4) + 4g + i%4 of the tile for query qi
        float x[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kk = 8 * (i / 4) + 4 * g + (i % 4);
            x[i] = ((word >> kk) & 1u) ? s[i] * scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, x[i]);
        }
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                             __float_as_uint(tmax), false, false);
            tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
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
            p[i] = __builtin_amdgcn_exp2f(x[i] - m_ref);
            psum += p[i];
        }
        l_part += psum;
        // ---- O^T[c][query] += V^T[c][keys] P^T[keys][query], per 16-key half
        // step T (kh = T >> 3, column tile n = T & 7) reads V^T rows ra / rb
        // of key half kh at column tile n: bases va_/vb_[n & 3], immediate
        // 256 * (n >> 2) + 16 rows * kh; the reads run two steps ahead of
        // the MFMAs that use them
        const uint32_t vt = lds_v + st * Sm::VB;
        u32x2_t ra2[2 * NCT], rb2[2 * NCT];
        auto rd = [&](auto Tc) {
            constexpr int T = decltype(Tc)::value, n = T & 7, kh = T >> 3;
            constexpr int o = 256 * (n >> 2) + kh * 16 * VD * 2;
            lds_read_tr16_nowait<o>(ra2[T], vt + va_[n & 3]);
            lds_read_tr16_nowait<o>(rb2[T], vt + vb_[n & 3]);
        };
        u32x4_t bhi, blo;
        auto step = [&](auto Tc) {
            constexpr int T = decltype(Tc)::value, n = T & 7;
            constexpr int NS = 2 * NCT;
            if constexpr (T + 2 < NS) {
                rd(std::integral_constant<int, T + 2>{});
                lds_operand_wait<4>(ra2[T], rb2[T]);
            } else {
                lds_operand_wait<2 * (NS - 1 - T)>(ra2[T], rb2[T]);
            }
            if constexpr (n == 0) {
                uint32_t hi4[4], lo4[4];
                float ph[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    ph[j] = p[(T >> 3) * 8 + j];
                split_bf16x8(ph, hi4, lo4);
                bhi = u32x4_t{hi4[0], hi4[1], hi4[2], hi4[3]};
                blo = u32x4_t{lo4[0], lo4[1], lo4[2], lo4[3]};
            }
            const u32x4_t av = {ra2[T][0], ra2[T][1], rb2[T][0], rb2[T][1]};
            oacc[n] = mfma_32x32x16(av, bhi, oacc[n]);
            oacc[n] = mfma_32x32x16(av, blo, oacc[n]);
        };
        static_assert(NCT == 8, "eight column tiles");
        rd(std::integral_constant<int, 0>{});
        rd(std::integral_constant<int, 1>{});
#define MK_PV_STEP(T) step(std::integral_constant<int, T>{});
        MK_PV_STEP(0) MK_PV_STEP(1) MK_PV_STEP(2) MK_PV_STEP(3) MK_PV_STEP(4) MK_PV_STEP(5)
        MK_PV_STEP(6) MK_PV_STEP(7) MK_PV_STEP(8) MK_PV_STEP(9) MK_PV_STEP(10) MK_PV_STEP(11)
        MK_PV_STEP(12) MK_PV_STEP(13) MK_PV_STEP(14) MK_PV_STEP(15)
#undef MK_PV_STEP
    }

    // ---- epilogue
    float l_tot;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part),
                                                         __float_as_uint(l_part), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
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
    if (nw > MK_MAXWORDS)  // the ABI rejects such rows before this
        return hipErrorInvalidValue;
    // LDS sized to the row (2 KB for 16384 keys) so that many rows share a CU
    hipLaunchKernelGGL(topk_to_mask_kernel, dim3((unsigned)rows), dim3(256),
                       (unsigned)(nw * sizeof(uint32_t)), st, a.idx,
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
