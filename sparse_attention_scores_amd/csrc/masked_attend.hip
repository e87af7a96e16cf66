// masked_attend.hip -- per-head (non-absorbed) sparse attention over each
// query's selected tokens, as in the pooled NoPE variant ("Module
// glm5next_dsa_ref": topk_to_mask turns an index row into the visibility
// mask the attention reads -- duplicates collapse, out-of-range and INVALID
// entries are dropped -- and mla_masked_attention attends over it).
//
// With per-head K and V nothing is shared across heads, so gathering each
// query's ~2k selected rows per head would move ~100 MB per query.  Instead
// the selection becomes a bitmap and the attention runs over key tiles:
//  1. topk_to_mask_kernel writes one bit per (query, key) -- the query's
//     selected set intersected with its visible range -- tile-major, so the
//     words of one key tile for a block of consecutive queries are one
//     contiguous run;
//  2. v_scale_max_kernel / v_to_f16_kernel re-encode V once as fp16 with a
//     power-of-two scale per (sequence, head) that puts the largest |V| in
//     [2^14, 2^15): every bf16 value whose magnitude is above 2^-29 of that
//     maximum is exact in fp16, so the softmax weights can enter the P.V
//     product as fp16 (11 significant bits) in one MFMA instead of a
//     two-term bf16 split;
//  3. attend_masked_kernel is a flash-style pass per (sequence, head, block
//     of 256 queries) over the key tiles the block's causal range covers:
//     each K/V tile is staged once in LDS and used by all 256 queries,
//     non-selected keys are masked out of the online softmax, and a wave
//     skips the tiles in which none of its 32 queries selects a key.
// MFMA layout (32x32x16): S^T[key][query] = K_tile * Q^T (bf16) with the
// queries of a wave in the B operand (held in registers), and
// O^T[c][query] += V^T * P^T (fp16), where each lane's accumulators all
// belong to one query, so the softmax rescale needs no cross-lane traffic.
// V^T keeps the keys of each 16-key half in the order the S^T accumulators
// hold them, so P^T comes straight from the softmax registers.
#include "attend_set.hpp"
#include "dsa_device.hpp"
#include "dsa_internal.hpp"

#include <float.h>
#include <math.h>

namespace dsa {

constexpr int MK_QB = kMaskedQBlock; // queries per attention block (8 waves x 32)
constexpr int MK_TILE = 32;         // keys per tile
constexpr int MK_ROWS = 32;         // query rows per mask-building block
constexpr int MK_WCHUNK = 512;      // mask words per row held in LDS at once
constexpr int MK_VKEYS = kMaskedVKeys; // keys per block of the V passes

// ------------------------------------------------------------------ mask

// Block (b, group of 32 queries): the rows' selected sets as bits, written
// tile-major: mask[(b * nw + w) * q_pad + q] holds keys 32w .. 32w+31 of
// query q.  Rows past n_q (up to q_pad) get zero words, so every word of the
// mask is written.  The group's index rows are one contiguous span of
// 32 x n_sel entries, read flat (eight coalesced loads in flight per
// thread, of four entries each when n_sel is a multiple of 4 and the base
// is 16-byte aligned: the four then share one row); keys are processed
// MK_WCHUNK words at a time.
__global__ __launch_bounds__(256) void topk_to_mask_kernel(const int32_t *__restrict__ idx,
                                                           const int32_t *__restrict__ vlo,
                                                           const int32_t *__restrict__ vhi,
                                                           uint32_t *__restrict__ mask, int n_q,
                                                           int n_k, int n_sel, int nw, int q_pad)
{
    constexpr int U = 8;
    __shared__ uint32_t bits[MK_ROWS][MK_WCHUNK + 1];
    __shared__ int rlo[MK_ROWS], rhi[MK_ROWS];
    const int groups = q_pad / MK_ROWS;
    const int b = blockIdx.x / groups;
    const int q0 = (blockIdx.x % groups) * MK_ROWS;
    const int tid = threadIdx.x;
    const int nrows = max(min(MK_ROWS, n_q - q0), 0);
    if (tid < MK_ROWS) {
        int lo = 0, hi = 0;
        if (tid < nrows) {
            const int64_t row = (int64_t)b * n_q + q0 + tid;
            lo = 0;
            hi = n_k;
            if (vlo) {
                lo = max(vlo[row], 0);
                hi = min(vhi[row], n_k);
            }
        }
        rlo[tid] = lo;
        rhi[tid] = hi;
    }
    const int32_t *span = idx + ((int64_t)b * n_q + q0) * n_sel;
    const int total = nrows * n_sel;  // < 2^31: checked on the host
    const float inv_sel = 1.0f / (float)max(n_sel, 1);
    const bool quad = (n_sel & 3) == 0 && (reinterpret_cast<uintptr_t>(idx) & 15) == 0;
    // row of entry e: a float estimate, corrected by one step
    auto row_of = [&](int e) {
        int r = (int)((float)e * inv_sel);
        r -= r * n_sel > e;
        r += (r + 1) * n_sel <= e;
        return r;
    };
    for (int w0 = 0; w0 < nw; w0 += MK_WCHUNK) {
        const int wn = min(MK_WCHUNK, nw - w0);
        for (int i = tid; i < MK_ROWS * (MK_WCHUNK + 1); i += 256)
            (&bits[0][0])[i] = 0u;
        __syncthreads();
        const int c_lo = w0 * 32, c_hi = (w0 + wn) * 32;
        auto set = [&](int r, int j, int jl, int jh) {
            if (j >= jl && j < jh)
                atomicOr(&bits[r][(j >> 5) - w0], 1u << (j & 31));
        };
        if (quad) {
            const int4 *span4 = reinterpret_cast<const int4 *>(span);
            const int total4 = total >> 2;
            for (int e0 = 0; e0 < total4; e0 += 256 * U) {
                int4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int e = e0 + u * 256 + tid;
                    v[u] = e < total4 ? span4[e] : make_int4(-1, -1, -1, -1);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int e = e0 + u * 256 + tid;
                    if (e >= total4)
                        continue;
                    const int r = row_of(4 * e);
                    const int jl = max(rlo[r], c_lo), jh = min(rhi[r], c_hi);
                    set(r, v[u].x, jl, jh);
                    set(r, v[u].y, jl, jh);
                    set(r, v[u].z, jl, jh);
                    set(r, v[u].w, jl, jh);
                }
            }
        }
        for (int e0 = 0; !quad && e0 < total; e0 += 256 * U) {
            int v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = e0 + u * 256 + tid;
                v[u] = e < total ? span[e] : -1;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = e0 + u * 256 + tid;
                if (e >= total)
                    continue;
                const int r = row_of(e);
                set(r, v[u], max(rlo[r], c_lo), min(rhi[r], c_hi));
            }
        }
        __syncthreads();
        uint32_t *mb = mask + ((int64_t)b * nw + w0) * q_pad + q0;
        for (int i = tid; i < wn * MK_ROWS; i += 256) {
            const int w = i / MK_ROWS, r = i % MK_ROWS;
            mb[(int64_t)w * q_pad + r] = bits[r][w];
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ V as fp16

// Exponent e of the power-of-two scale 2^-e that puts the largest |V| of a
// (sequence, head) in [2^14, 2^15) -- well inside fp16's finite range -- from
// the f32 bits of that largest magnitude; 0 when V is all zero.
__device__ __forceinline__ int v16_exponent(uint32_t maxbits)
{
    if (maxbits == 0u)
        return 0;
    const int ex = (int)((maxbits >> 23) & 0xffu) - 127;
    return min(max(ex - 14, -120), 120);
}

// Block (b, h, run of MK_VKEYS keys): largest |V| of the run, one partial
// per block (no atomics, nothing to clear first).
__global__ __launch_bounds__(256) void v_scale_max_kernel(const uint16_t *__restrict__ v,
                                                          int64_t vsr, int n_k, int H, int vd,
                                                          int nkb, uint32_t *__restrict__ part)
{
    __shared__ uint32_t red[4];
    const int bh = blockIdx.x / nkb, kb = blockIdx.x % nkb;
    const int b = bh / H, h = bh % H;
    const int cpr = vd / 8;  // 16-byte chunks per head row
    const int tid = threadIdx.x;
    uint32_t mx = 0u;
    const int k0 = kb * MK_VKEYS, k1 = min(k0 + MK_VKEYS, n_k);
    for (int c = tid; c < (k1 - k0) * cpr; c += 256) {
        const int key = k0 + c / cpr, ch = c % cpr;
        const u32x4_t x = *reinterpret_cast<const u32x4_t *>(
            v + ((int64_t)b * n_k + key) * vsr + (int64_t)h * vd + ch * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // |bf16| as f32 bits: the sign cleared, compared as integers
            mx = max(mx, (x[j] << 16) & 0x7fffffffu);
            mx = max(mx, x[j] & 0x7fff0000u);
        }
    }
    mx = wave_max_u32(mx);
    if ((tid & 63) == 0)
        red[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0)
        part[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// Same blocks: V * 2^-e(b,h) as fp16 (round to nearest even) into the dense
// workspace copy v16[b][key][h][vd]; every block also writes its head's
// 2^e (the same value from each block of the head).
__global__ __launch_bounds__(256) void v_to_f16_kernel(const uint16_t *__restrict__ v, int64_t vsr,
                                                       int n_k, int H, int vd, int nkb,
                                                       const uint32_t *__restrict__ part,
                                                       uint16_t *__restrict__ v16,
                                                       float *__restrict__ vexp)
{
    const int bh = blockIdx.x / nkb, kb = blockIdx.x % nkb;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x;
    uint32_t mx = 0u;
    for (int i = tid & 63; i < nkb; i += 64)
        mx = max(mx, part[(int64_t)bh * nkb + i]);
    mx = wave_max_u32(mx);
    const int e = v16_exponent(mx);
    const float down = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
    if (tid == 0 && kb == 0)
        vexp[bh] = __uint_as_float((uint32_t)(127 + e) << 23);      // 2^e
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    const int cpr = vd / 8;
    const int k0 = kb * MK_VKEYS, k1 = min(k0 + MK_VKEYS, n_k);
    for (int c = tid; c < (k1 - k0) * cpr; c += 256) {
        const int key = k0 + c / cpr, ch = c % cpr;
        const u32x4_t x = *reinterpret_cast<const u32x4_t *>(
            v + ((int64_t)b * n_k + key) * vsr + (int64_t)h * vd + ch * 8);
        u32x4_t y;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float lo = __uint_as_float(x[j] << 16) * down;
            const float hi = __uint_as_float(x[j] & 0xffff0000u) * down;
            y[j] = __builtin_bit_cast(uint32_t,
                                      __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
        }
        *reinterpret_cast<u32x4_t *>(v16 + (((int64_t)b * n_k + key) * H + h) * vd + ch * 8) = y;
    }
}

// ------------------------------------------------------------------ attention

// LDS row swizzles of the per-head tiles, chosen by measurement on gfx950
// (both keep their access pattern at the full LDS rate):
//  K rows (192 bf16 = 384 bytes = 24 chunks): physical chunk = logical ^
//  ((row >> 1) & 7) -- the 32x32x16 operand reads (32 rows at one chunk);
//  V rows (256 fp16 = 512 bytes = 32 chunks, so every row starts on bank 0):
//  physical chunk = logical ^ (((row & 3) << 2) | ((row >> 2) & 3)) -- the
//  transposing reads (4 rows x 2 chunks per 16 lanes).
__device__ __forceinline__ int mk_swz_k(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int mk_swz_v(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

constexpr int MK_STAGES = 4;  // tiles resident in LDS (ring)
constexpr int MK_AHEAD = 5;   // MFMAs between an operand read and its use

// The matrix phase's stream of NP P.V steps and NQ Q.K^T k-steps: op j is a
// P.V step while P.V is behind its share of the ops issued so far.
template <int NP, int NQ>
constexpr bool mk_is_pv(int j)
{
    int np = 0, nq = 0;
    for (int x = 0; x <= j; ++x) {
        const bool pv = nq >= NQ || (np < NP && np * NQ <= nq * NP);
        if (x == j)
            return pv;
        if (pv)
            ++np;
        else
            ++nq;
    }
    return false;
}
// index of op j among the ops of its own kind
template <int NP, int NQ>
constexpr int mk_index_of(int j)
{
    int c = 0;
    for (int x = 0; x < j; ++x)
        c += mk_is_pv<NP, NQ>(x) == mk_is_pv<NP, NQ>(j);
    return c;
}
// LDS read instructions of ops j0 .. j1 (a P.V step reads twice, a Q.K^T
// k-step once)
template <int NP, int NQ>
constexpr int mk_reads_between(int j0, int j1)
{
    int c = 0;
    for (int y = j0; y <= j1 && y < NP + NQ; ++y)
        c += mk_is_pv<NP, NQ>(y) ? 2 : 1;
    return c;
}
template <int N, int I = 0, class F>
__device__ __forceinline__ void mk_unroll(F &f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        mk_unroll<N, I + 1>(f);
    }
}

template <int KD, int VD>
struct __attribute__((aligned(16))) MaskedSmem {
    static constexpr int KB = MK_TILE * KD * 2;  // K tile bytes (row-major, swizzled)
    static constexpr int VB = MK_TILE * VD * 2;  // V tile bytes (fp16)
    unsigned char k[MK_STAGES][KB];
    unsigned char v[MK_STAGES][VB];
    uint32_t mw[MK_STAGES][MK_QB];              // the block's mask words of the tile
};

// Direct-to-LDS 16-byte load per lane from a scalar base plus a 32-bit lane
// offset (global_load_lds_dwordx4, saddr form) into LDS bytes lds_dst + 16 *
// lane.  Written as asm so the compiler neither hoists base + offset out of
// the tile loop as 64-bit registers nor merges the K, V and mask loads into
// one load with selected operands; M0 carries the LDS address (one wait
// state after writing it).  Completion is tracked with vm_wait.
// (The compiler keeps M0 reserved and warns that the clobber is not
// honoured; no other code of these kernels uses M0.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16_s(const void *sbase, uint32_t voff, uint32_t lds_dst)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_dst)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ f32x16_t mfma_32x32x16_f16(const u32x4_t &a, const u32x4_t &b,
                                                      f32x16_t c)
{
    typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t cvt_pk_f16(float a, float b)
{
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}

// One LDS read of a 4-byte word and the wait (asm: the word arrives by a
// direct-to-LDS load, and the compiler would otherwise wait for every such
// load in flight).
__device__ __forceinline__ uint32_t mk_read_word(uint32_t a)
{
    uint32_t x;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(a) : "memory");
    return x;
}

// Per (sequence, head, block of 256 queries), 8 waves: wave w owns queries
// q0 + 32w .. +31 (lane col = query, half g = lane >> 5).  Key tiles of 32
// stream through a ring of MK_STAGES LDS stages by direct-to-LDS loads (12
// one-KB instructions for K, 16 for V, one for the block's mask words: 29,
// four per wave for waves 0-6 and the mask for wave 7).
//
// Ping-pong: the waves of one SIMD (w and w + 4) alternate between a matrix
// phase (P.V of the previous tile, then Q.K^T of this one) and a vector
// phase (this tile's softmax).  Waves 4-7 run half an iteration behind waves
// 0-3, held there by one workgroup barrier at each phase boundary, so while
// one wave of a SIMD issues its MFMAs the other runs its exponentials.
template <int KD, int VD>
__global__ __launch_bounds__(512, 1) void attend_masked_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, int64_t ksr,
    const uint16_t *__restrict__ v16, const float *__restrict__ vexp,
    const uint32_t *__restrict__ mask, const int32_t *__restrict__ vlo,
    const int32_t *__restrict__ vhi, float *__restrict__ out, float *__restrict__ lse, int n_q,
    int n_k, int H, int nw, int q_pad, int n_qblocks, float c_log2, float thr, bool neg_q)
{
    constexpr int KS = KD / 16;      // k-steps of the 32x32x16 MFMA over kd
    constexpr int NCT = VD / 32;     // output column tiles of 32
    constexpr int KCH = KD / 8;      // 16-byte chunks of a K row
    constexpr int VCH = VD / 8;      // 16-byte chunks of a V row
    static_assert(KD == kMaskedKd && VD == kMaskedVd && KD == 192 && VD == 256,
                  "the swizzles and read groups are laid out for 192/256");
    using Sm = MaskedSmem<KD, VD>;
    constexpr int NK_DMA = Sm::KB / 1024;            // 12
    constexpr int NV_DMA = Sm::VB / 1024;            // 16
    constexpr int NSLOT = NK_DMA + NV_DMA + 1;       // 29 one-KB loads per tile
    static_assert(NSLOT <= 32, "four load slots per wave");
    __shared__ Sm sm;
    __shared__ int sm_red[16];
    DSA_LDS_ESCAPE(sm);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool grp_b = wid >= 4;
    const int g = lane >> 5, col = lane & 31;
    // Each XCD takes a contiguous range of blocks: the query blocks of one
    // (sequence, head) run together on one XCD and stream the same K/V tiles
    // through its L2; within a head the heaviest (latest) blocks go first.
    // The later half of a head's blocks starts together and walks its tiles
    // upward; each block of the earlier half starts when one of those ends,
    // the shortest first, and walks its tiles downward, so that all of the
    // earlier half read the same tile at the same time (L2 keeps it for
    // all of them) and end together.
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int qblk = n_qblocks - 1 - lb % n_qblocks;
    const bool desc = qblk < n_qblocks / 2;
    const int bh = lb / n_qblocks;
    const int b = bh / H, h = bh % H;
    const int q0 = qblk * MK_QB;
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
            sm_red[8 + wid] = mx;
        }
        __syncthreads();
        lo = sm_red[0];
        hi = sm_red[8];
#pragma unroll
        for (int w = 1; w < 8; ++w) {
            lo = min(lo, sm_red[w]);
            hi = max(hi, sm_red[8 + w]);
        }
    }
    const int T0 = lo / MK_TILE;
    const int T1 = hi > lo ? (hi + MK_TILE - 1) / MK_TILE : T0;

    // Q^T fragments (B operand): query qi, dims ks*16 + g*8 .. +8; negated
    // (exactly) when the scale is negative, so the softmax runs on |scale|
    u32x4_t qf[KS];
    {
        const uint16_t *qp = q + (row * H + h) * KD + g * 8;
        const uint32_t flip = neg_q ? 0x80008000u : 0u;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = q_ok ? *reinterpret_cast<const u32x4_t *>(qp + ks * 16)
                          : u32x4_t{0u, 0u, 0u, 0u};
            qf[ks] ^= u32x4_t{flip, flip, flip, flip};
        }
    }
    f32x16_t oacc[NCT];
#pragma unroll
    for (int n = 0; n < NCT; ++n)
        oacc[n] = f32x16_t{};
    float m_run = -INFINITY, l_part = 0.f;

    const unsigned char *kb =
        reinterpret_cast<const unsigned char *>(k + (int64_t)b * n_k * ksr + (int64_t)h * KD);
    const unsigned char *vb =
        reinterpret_cast<const unsigned char *>(v16 + ((int64_t)b * n_k * H + h) * VD);
    const unsigned char *mb = reinterpret_cast<const unsigned char *>(
        mask + (int64_t)b * nw * q_pad + q0);
    const uint32_t ksr2 = (uint32_t)(ksr * 2), vsr2 = (uint32_t)(H * VD * 2);
    const uint64_t q_pad4 = (uint64_t)q_pad * 4u;
    // this wave's load slots: 4w .. 4w+3 of the tile's 29
    const int n_mine = min(4, NSLOT - 4 * wid);

    // Load slot s of a tile: s < 12 fills K bytes 1 KB * s, 12..27 V bytes
    // 1 KB * (s - 12), 28 the block's mask words.  Lane l of a slot fills LDS
    // bytes 16l of that KB = (row, physical chunk) and fetches the row's
    // logical chunk; its byte offset from the tile's first key row is the
    // same for every tile, so each load is a scalar tile base plus this
    // per-lane constant.
    uint32_t voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int s_ = 4 * wid + j;
        if (s_ < NK_DMA) {
            const int c = s_ * 64 + lane, r = c / KCH;
            voff[j] = (uint32_t)r * ksr2 + (uint32_t)(((c % KCH) ^ mk_swz_k(r)) * 16);
        } else if (s_ < NK_DMA + NV_DMA) {
            const int c = (s_ - NK_DMA) * 64 + lane, r = c / VCH;
            voff[j] = (uint32_t)r * vsr2 + (uint32_t)(((c % VCH) ^ mk_swz_v(r)) * 16);
        } else {
            voff[j] = 16u * (uint32_t)lane;
        }
    }
    const uint32_t lds_k0 = __builtin_amdgcn_readfirstlane(lds_addr(sm.k[0])),
                   lds_v0 = __builtin_amdgcn_readfirstlane(lds_addr(sm.v[0])),
                   lds_m0 = __builtin_amdgcn_readfirstlane(lds_addr(&sm.mw[0][0]));
    // DMA of tile t into stage st; the last tile of a row whose length is
    // not a multiple of 32 clamps its rows past n_k to the last key (those
    // keys are masked) with addresses computed per lane
    // tile u of the walk (T0 <= u < T1) is key tile u, or T0 + T1 - 1 - u
    // downward
    const int t_flip = T0 + T1 - 1;
    auto dma_tile = [&](int u, auto STc) {
        constexpr int st = decltype(STc)::value;
        const int t = desc ? t_flip - u : u;
        const int k0 = t * MK_TILE;
        const bool full = k0 + MK_TILE <= n_k;
        const unsigned char *ks_ = kb + (uint64_t)(uint32_t)k0 * ksr2;
        const unsigned char *vs_ = vb + (uint64_t)(uint32_t)k0 * vsr2;
        const unsigned char *ms_ = mb + (uint64_t)(uint32_t)t * q_pad4;
        const uint32_t lk = lds_k0 + st * Sm::KB, lv = lds_v0 + st * Sm::VB,
                       lm = lds_m0 + st * (MK_QB * 4);
        // the clamped addresses of a partial tile derive from an opaque copy
        // of the lane index, so none of them is hoisted out of the loop
        int ln = lane;
        if (!full)
            asm volatile("" : "+v"(ln));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s_ = 4 * wid + j;
            if (s_ < NK_DMA) {
                uint32_t o = voff[j];
                if (!full) {
                    const int c = s_ * 64 + ln, r = c / KCH;
                    o = (uint32_t)(min(k0 + r, n_k - 1) - k0) * ksr2 +
                        (uint32_t)(((c % KCH) ^ mk_swz_k(r)) * 16);
                }
                lds_dma16_s(ks_, o, lk + s_ * 1024);
            } else if (s_ < NK_DMA + NV_DMA) {
                uint32_t o = voff[j];
                if (!full) {
                    const int c = (s_ - NK_DMA) * 64 + ln, r = c / VCH;
                    o = (uint32_t)(min(k0 + r, n_k - 1) - k0) * vsr2 +
                        (uint32_t)(((c % VCH) ^ mk_swz_v(r)) * 16);
                }
                lds_dma16_s(vs_, o, lv + (s_ - NK_DMA) * 1024);
            } else if (s_ < NSLOT) {
                lds_dma16_s(ms_, voff[j], lm);
            }
        }
    };
    // wait until this wave's loads of the tile `after` tiles before the
    // newest one issued have landed
    auto wait_tile = [&](int after) {
        if (n_mine == 4)
            vm_wait_tiles<4>(after);
        else
            vm_wait_tiles<1>(after);
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
    const uint32_t lds_mw = lds_addr(&sm.mw[0][0]) + 4u * (uint32_t)(wid * 32 + col);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kq[j] += lds_k;
        va_[j] += lds_v;
        vb_[j] += lds_v;
    }

    f32x16_t s = {};
    u32x4_t p0 = {}, p1 = {};  // P^T of the previous tile (fp16, both key halves)

    // Matrix phase: P.V of the tile in stage sv and Q.K^T of the tile in
    // stage sk as one stream of MFMAs, P.V steps and
    // Q.K^T k-steps interleaved, every operand read issued MK_AHEAD MFMAs
    // before the MFMA that uses it (the two read kinds share the LDS counter,
    // so each wait counts the reads issued after its own).
    //  P.V step T: column tile n = T & 7 of key half T >> 3, two transposing
    //  reads of V^T rows ra / rb (bases va_/vb_[n & 3], immediate
    //  256 * (n >> 2) + 16 rows * 512 for the key half).
    //  Q.K^T k-step ks: one read of K rows at base kq[ks & 3], immediate
    //  128 * (ks >> 2).
    auto m_phase = [&](auto SVc, auto SKc) {
        constexpr int SV = decltype(SVc)::value, SK = decltype(SKc)::value;
        constexpr int NP = 2 * NCT, NQ = KS, N = NP + NQ;
        // every LDS address is a per-lane register plus an immediate (the
        // stage is a compile-time constant of the unrolled loop)
        u32x2_t ra2[2 * NCT], rb2[2 * NCT];
        u32x4_t a[KS];
        auto issue = [&](auto Jc) {
            constexpr int J = decltype(Jc)::value;
            if constexpr (J < N) {
                constexpr int x = mk_index_of<NP, NQ>(J);
                if constexpr (mk_is_pv<NP, NQ>(J)) {
                    constexpr int n = x & 7, kh = x >> 3;
                    constexpr int o = SV * Sm::VB + 256 * (n >> 2) + kh * 16 * VD * 2;
                    lds_read_tr16_nowait<o>(ra2[x], va_[n & 3]);
                    lds_read_tr16_nowait<o>(rb2[x], vb_[n & 3]);
                } else {
                    lds_read_b128_nowait<SK * Sm::KB + 128 * (x >> 2)>(a[x], kq[x & 3]);
                }
            }
        };
        auto op = [&](auto Jc) {
            constexpr int J = decltype(Jc)::value;
            issue(std::integral_constant<int, J + MK_AHEAD>{});
            constexpr int after = mk_reads_between<NP, NQ>(J + 1, J + MK_AHEAD);
            constexpr int x = mk_index_of<NP, NQ>(J);
            if constexpr (mk_is_pv<NP, NQ>(J)) {
                lds_operand_wait<after>(ra2[x], rb2[x]);
                const u32x4_t av = {ra2[x][0], ra2[x][1], rb2[x][0], rb2[x][1]};
                oacc[x & 7] = mfma_32x32x16_f16(av, (x >> 3) ? p1 : p0, oacc[x & 7]);
            } else {
                lds_operand_wait<after>(a[x]);
                s = mfma_32x32x16(a[x], qf[x], s);
            }
        };
        s = f32x16_t{};
        mk_unroll<MK_AHEAD>(issue);
        mk_unroll<N>(op);
    };

    // the first matrix phase runs P.V with zero weights over the last stage,
    // which no tile has filled yet: clear its V so that 0 * V stays 0
    for (int i = tid; i < Sm::VB / 16; i += 512)
        reinterpret_cast<u32x4_t *>(sm.v[MK_STAGES - 1])[i] = u32x4_t{0u, 0u, 0u, 0u};
    // the Q fragments and ranges are in registers before the first tile DMA
    vm_wait<0>();
    {
        auto pro = [&](auto Jc) {
            constexpr int j = decltype(Jc)::value;
            if (T0 + j < T1)
                dma_tile(T0 + j, Jc);
        };
        mk_unroll<MK_STAGES - 1>(pro);
    }
    if (T1 > T0)
        wait_tile(min(T1 - 1, T0 + MK_STAGES - 2) - T0);
    lds_barrier();  // tile T0 is in LDS for every wave
    if (grp_b)
        lds_barrier();  // waves 4-7 start half an iteration behind

    // this wave's tiles: the union of its 32 queries' visible ranges (the
    // mask words are zero outside it; inside it a tile none of the queries
    // selects skips its softmax)
    int tw_begin, tw_end;
    {
        int wl = q_ok ? (vlo ? max(vlo[row], 0) : 0) : n_k;
        int wh = q_ok ? (vhi ? min(vhi[row], n_k) : n_k) : 0;
        wl = (int)wave_min_u32((uint32_t)wl);
        wh = (int)wave_max_u32((uint32_t)wh);
        tw_begin = wl / MK_TILE;
        tw_end = wh > wl ? (wh + MK_TILE - 1) / MK_TILE : tw_begin;
    }

    bool act_prev = false;
    // One ping-pong iteration for tile t held in stage ST, a compile-time
    // constant (the loop is unrolled over the ring); false after the final
    // matrix phase.
    auto iteration = [&](auto STc, int t) -> bool {
        constexpr int ST = decltype(STc)::value;
        constexpr int SP = (ST + MK_STAGES - 1) % MK_STAGES;
        // ---------------- matrix phase: P.V of tile t-1, Q.K^T of tile t
        // (the mask word is read now and waited for after the phase)
        uint32_t word = 0u;
        if (t < T1)
            lds_read_b32_nowait<ST * MK_QB * 4>(word, lds_mw);
        const int tp = desc ? t_flip - t : t;
        const bool act = t < T1 && tp >= tw_begin && tp < tw_end;
        // one instruction stream for both products keeps the register
        // allocation within 256: an inactive previous tile contributes zero
        // weights (P = 0 against finite V), and the scores of an inactive
        // tile are not used
        if (act_prev || act)
            m_phase(std::integral_constant<int, SP>{}, std::integral_constant<int, ST>{});
        if (grp_b && t + 1 < T1)
            wait_tile(min(T1 - 1, t + MK_STAGES - 2) - (t + 1));
        lds_barrier();
        if (t == T1)
            return false;
        lds_operand_wait<0>(word);
        // ---------------- vector phase: tile loads, then the softmax of tile t
        // (waves 0-3 refill the stage that held tile t-2, waves 4-7 the one
        // that held tile t-1: both are done with it by now)
        if (!grp_b && t > T0 && t + MK_STAGES - 2 < T1)
            dma_tile(t + MK_STAGES - 2, std::integral_constant<int, (ST + MK_STAGES - 2) % MK_STAGES>{});
        if (grp_b && t + MK_STAGES - 1 < T1)
            dma_tile(t + MK_STAGES - 1, std::integral_constant<int, (ST + MK_STAGES - 1) % MK_STAGES>{});
        const bool soft = act && __any(word != 0u);
        if (soft) {            // lane holds keys 8*(i/4) + 4g + i%4 of the tile for query qi;
            // unselected keys become -inf (sign-extended bit as a bit mask)
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kk = 8 * (i / 4) + 4 * g + (i % 4);
                const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)word, kk, 1);
                x[i] = __uint_as_float((__float_as_uint(s[i]) & m) | (~m & 0xff800000u));
            }
            float tmax = fmaxf(fmaxf(x[0], x[1]), x[2]);
            tmax = fmaxf(fmaxf(tmax, x[3]), x[4]);
            tmax = fmaxf(fmaxf(tmax, x[5]), x[6]);
            tmax = fmaxf(fmaxf(tmax, x[7]), x[8]);
            tmax = fmaxf(fmaxf(tmax, x[9]), x[10]);
            tmax = fmaxf(fmaxf(tmax, x[11]), x[12]);
            tmax = fmaxf(fmaxf(tmax, x[13]), x[14]);
            tmax = fmaxf(tmax, x[15]);
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(
                    __float_as_uint(tmax), __float_as_uint(tmax), false, false);
                tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            // lazy rescale (raw score units; thr = 8 / c): p <= 2^8
            const bool grow = tmax > m_run + thr;
            if (__any(grow)) {
                const float m_new = grow ? tmax : m_run;
                // lanes that do not grow keep alpha = 1 (m_run may still be
                // -inf there, and -inf - -inf would be NaN); a growing lane
                // with m_run = -inf gets 0
                const float alpha = grow ? exp2f((m_run - m_new) * c_log2) : 1.f;
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
            const float mc = (m_run == -INFINITY) ? 0.f : m_run * c_log2;
            float p[16];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c_log2, -mc));
                psum += p[i];
            }
#pragma unroll
            for (int i = 8; i < 16; ++i) {
                p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c_log2, -mc));
                psum += p[i];
            }
            l_part += psum;
            p0 = u32x4_t{cvt_pk_f16(p[0], p[1]), cvt_pk_f16(p[2], p[3]),
                         cvt_pk_f16(p[4], p[5]), cvt_pk_f16(p[6], p[7])};
            p1 = u32x4_t{cvt_pk_f16(p[8], p[9]), cvt_pk_f16(p[10], p[11]),
                         cvt_pk_f16(p[12], p[13]), cvt_pk_f16(p[14], p[15])};
        } else {
            p0 = u32x4_t{0u, 0u, 0u, 0u};
            p1 = p0;
        }
        act_prev = act;
        if (!grp_b && t + 1 < T1)
            wait_tile(min(T1 - 1, t + MK_STAGES - 2) - (t + 1));
        lds_barrier();
        return true;
    };
    for (int t = T0;; t += MK_STAGES) {
        bool go = true;
        auto step = [&](auto STc) {
            if (go)
                go = iteration(STc, t + decltype(STc)::value);
        };
        mk_unroll<MK_STAGES>(step);
        if (!go)
            break;
    }
    if (!grp_b)
        lds_barrier();  // the barrier count of waves 0-3 matches waves 4-7

    // ---- epilogue
    float l_tot;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part),
                                                         __float_as_uint(l_part), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (q_ok) {
        const float inv = l_tot > 0.f ? vexp[(int64_t)b * H + h] / l_tot : 0.f;
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
            lse[row * H + h] = l_tot > 0.f ? (m_run * c_log2 + log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

// ------------------------------------------------------------------ few queries

// Per-head attention for a few queries per sequence (decode): one block per
// (query row, head) gathers only the row's selected keys, K and V of that
// head -- what one block of the masked-tile kernel would stream over the
// whole key range for one useful query.  Two passes over the selected set,
// in ascending key order: scores (eight lanes per key, 24 bf16 of K each),
// then the max and the softmax weights in LDS, then the weighted sum of V
// (a half-wave per key, eight columns per lane).  f32 arithmetic
// throughout; many keys' loads are in flight per lane in both passes.
constexpr int HG_NT = 256;       // 4 waves
constexpr int HG_LIST = 4096;    // largest selected set the block holds
constexpr int HG_KU = 4;         // keys per lane group per score round
constexpr int HG_VU = 8;         // key pairs per wave per value round

struct HeadsGatherSmem {
    uint32_t bitmap[kBitmapMaxWords];
    int32_t list[HG_LIST];
    float p[HG_LIST];
    float o[HG_NT / 64][256];
    float red[HG_NT / 64];
    int cnt[HG_NT / 64];
};

__device__ __forceinline__ void bf16x8_to_f32(const u32x4_t &r, float (&f)[8])
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(r[j] << 16);
        f[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
    }
}

template <int KD, int VD>
__global__ __launch_bounds__(HG_NT) void attend_heads_gather_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, int64_t ksr,
    const uint16_t *__restrict__ v, int64_t vsr, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ vlo, const int32_t *__restrict__ vhi, float *__restrict__ out,
    float *__restrict__ lse, int n_q, int n_k, int H, int n_sel, float scale_log2)
{
    constexpr int KC = KD / 64;  // 16-byte chunks of a K row per lane (8 lanes per key)
    static_assert(KD % 64 == 0 && VD == HG_NT && VD / 8 == 32, "K in 8 lanes, V in a half-wave");
    constexpr int NW = HG_NT / 64;
    __shared__ HeadsGatherSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    // a row's heads are consecutive blocks on one XCD: its index row comes
    // from that L2
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int row = lb / H, h = lb % H;
    const int64_t b = row / n_q;
    int lo = 0, hi = n_k;
    if (vlo) {
        lo = max(vlo[row], 0);
        hi = min(vhi[row], n_k);
    }
    const int nw = (n_k + 31) >> 5;
    const int32_t *idx_row = idx + (int64_t)row * n_sel;
    int first[8];
    load_indices<HG_NT, 8>(first, idx_row, n_sel, 0);
    // this lane's share of q (chunks sub, sub + 8, ...), scaled to log2 units
    const int sub = lane & 7, grp = lane >> 3;
    float qf[KC][8];
    {
        const uint16_t *qp = q + ((int64_t)row * H + h) * KD;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            bf16x8_to_f32(*reinterpret_cast<const u32x4_t *>(qp + (c * 8 + sub) * 8), qf[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                qf[c][e] *= scale_log2;
        }
    }
    build_bitmap<HG_NT, 8>(sm.bitmap, nw, first, idx_row, n_sel, lo, hi);
    int c0, c1;
    wave_chunk_range<NW>(nw, wid, c0, c1);
    const int cnt = wave_chunk_count(sm.bitmap, nw, c0, c1);
    if (lane == 0)
        sm.cnt[wid] = cnt;
    __syncthreads();
    int run = 0, n = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        run += w < wid ? sm.cnt[w] : 0;
        n += sm.cnt[w];
    }
    wave_chunk_extract(sm.bitmap, nw, c0, c1, run, 0, HG_LIST, sm.list);
    n = min(n, HG_LIST);
    __syncthreads();
    float *orow = out + ((int64_t)row * H + h) * VD;
    if (n == 0) {  // empty set: zero output, lse = -inf
        orow[tid] = 0.f;
        if (lse && tid == 0)
            lse[(int64_t)row * H + h] = -INFINITY;
        return;
    }

    // pass 1: scores of the selected keys, in log2 units
    const uint16_t *kb = k + (int64_t)b * n_k * ksr + (int64_t)h * KD + sub * 8;
    float mloc = -INFINITY;
    for (int base = wid * (8 * HG_KU); base < n; base += NW * 8 * HG_KU) {
        u32x4_t kr[HG_KU][KC];
#pragma unroll
        for (int u = 0; u < HG_KU; ++u) {
            const int i = min(base + u * 8 + grp, n - 1);
            const uint16_t *p = kb + (int64_t)sm.list[i] * ksr;
#pragma unroll
            for (int c = 0; c < KC; ++c)
                kr[u][c] = *reinterpret_cast<const u32x4_t *>(p + c * 64);
        }
#pragma unroll
        for (int u = 0; u < HG_KU; ++u) {
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                float kf[8];
                bf16x8_to_f32(kr[u][c], kf);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    dot = fmaf(qf[c][e], kf[e], dot);
            }
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            dot += __shfl_xor(dot, 4);
            const int i = base + u * 8 + grp;
            if (i < n) {
                mloc = fmaxf(mloc, dot);
                if (sub == 0)
                    sm.p[i] = dot;
            }
        }
    }
    mloc = wave_max(mloc);
    if (lane == 0)
        sm.red[wid] = mloc;
    __syncthreads();
    float m = sm.red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        m = fmaxf(m, sm.red[w]);
    float lloc = 0.f;
    for (int i = tid; i < n; i += HG_NT) {
        const float pw = exp2f(sm.p[i] - m);
        sm.p[i] = pw;
        lloc += pw;
    }
    lloc = wave_sum(lloc);
    __syncthreads();  // every max is read before red is reused; the weights are written
    if (lane == 0)
        sm.red[wid] = lloc;
    __syncthreads();
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        l += sm.red[w];

    // pass 2: sum of p_j V_j, a half-wave per key
    const int half = lane >> 5, col = (lane & 31) * 8;
    const uint16_t *vb = v + (int64_t)b * n_k * vsr + (int64_t)h * VD + col;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        o[e] = 0.f;
    for (int base = wid * (2 * HG_VU); base < n; base += NW * 2 * HG_VU) {
        u32x4_t vr[HG_VU];
        float pw[HG_VU];
#pragma unroll
        for (int u = 0; u < HG_VU; ++u) {
            const int i = base + 2 * u + half;
            const int ii = min(i, n - 1);
            vr[u] = *reinterpret_cast<const u32x4_t *>(vb + (int64_t)sm.list[ii] * vsr);
            pw[u] = i < n ? sm.p[ii] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < HG_VU; ++u) {
            float vf[8];
            bf16x8_to_f32(vr[u], vf);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] = fmaf(pw[u], vf[e], o[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        o[e] += __shfl_xor(o[e], 32);
    if (half == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sm.o[wid][col + e] = o[e];
    }
    __syncthreads();
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        acc += sm.o[w][tid];
    orow[tid] = acc / l;
    if (lse && tid == 0)
        lse[(int64_t)row * H + h] = (m + log2f(l)) * kLn2;
}

// ------------------------------------------------------------------ host side

hipError_t launch_attend_heads(const AttendArgs &a, hipStream_t st)
{
    const int64_t blocks = (int64_t)a.batch * a.n_q * a.n_heads;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attend_heads_gather_kernel<192, 256>), dim3((unsigned)blocks),
                       dim3(HG_NT), 0, st, static_cast<const uint16_t *>(a.q),
                       static_cast<const uint16_t *>(a.k), a.k_row_stride,
                       static_cast<const uint16_t *>(a.v), a.v_row_stride, a.idx, a.vis_lo,
                       a.vis_hi, a.out, a.lse, a.n_q, a.n_k, a.n_heads, a.n_sel,
                       a.scale * kLog2e);
    return hipGetLastError();
}

hipError_t launch_attend_masked(const AttendArgs &a, hipStream_t st)
{
    const MaskedLayout L = masked_layout(a);
    unsigned char *ws = static_cast<unsigned char *>(a.workspace);
    uint32_t *mask = reinterpret_cast<uint32_t *>(ws);
    uint16_t *v16 = reinterpret_cast<uint16_t *>(ws + L.v16_off);
    uint32_t *part = reinterpret_cast<uint32_t *>(ws + L.part_off);
    float *vexp = reinterpret_cast<float *>(ws + L.vexp_off);
    const int64_t mblocks = (int64_t)a.batch * (L.q_pad / MK_ROWS);
    const int64_t vblocks = (int64_t)a.batch * a.n_heads * L.nkb;
    const int n_qblocks = L.q_pad / MK_QB;
    const int64_t blocks = (int64_t)n_qblocks * a.batch * a.n_heads;
    if (mblocks > 0x7fffffff || vblocks > 0x7fffffff || blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(topk_to_mask_kernel, dim3((unsigned)mblocks), dim3(256), 0, st, a.idx,
                       a.vis_lo, a.vis_hi, mask, a.n_q, a.n_k, a.n_sel, L.nw, L.q_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const uint16_t *v = static_cast<const uint16_t *>(a.v);
    hipLaunchKernelGGL(v_scale_max_kernel, dim3((unsigned)vblocks), dim3(256), 0, st, v,
                       a.v_row_stride, a.n_k, a.n_heads, a.vd, L.nkb, part);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(v_to_f16_kernel, dim3((unsigned)vblocks), dim3(256), 0, st, v,
                       a.v_row_stride, a.n_k, a.n_heads, a.vd, L.nkb, part, v16, vexp);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // softmax in base 2 on |scale| (the queries are negated for a negative
    // scale); a zero scale keeps a tiny positive factor so that masked keys
    // still come out as -inf rather than NaN
    const float c = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
    hipLaunchKernelGGL((attend_masked_kernel<192, 256>), dim3((unsigned)blocks), dim3(512), 0, st,
                       static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
                       a.k_row_stride, v16, vexp, mask, a.vis_lo, a.vis_hi, a.out, a.lse, a.n_q,
                       a.n_k, a.n_heads, L.nw, L.q_pad, n_qblocks, c, kRescaleLog2 / c,
                       a.scale < 0.f);
    return hipGetLastError();
}

} // namespace dsa
