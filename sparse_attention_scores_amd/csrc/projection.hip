// projection.hip -- dense projections ahead of the path, on the matrix cores:
//  * the lightning indexer's front-end ("Another DSA attempt", the
//    batch-local indexer commit): q = wq_b(q_lora) split per head with the
//    leading rope_dim entries NEOX-rotated; k = wk(x) through LayerNorm with
//    bias (k_norm) and the same rotation; w = weights_proj(x) ("Module
//    glm5next_dsa_ref": linear, layer_norm and the k_norm invariant; the
//    pages' CPU crash-fix commit and review: k_norm's eps must be positive,
//    1e-6 in the reference);
//  * expand_kv ("Module glm5next_dsa_ref"): per-head K and V from the
//    compressed latent, NoPE, each head's kd key rows then vd value rows.
//
// One GEMM body, C[m][n] = sum_k A[m][k] B[n][k] (both operands K-major,
// the torch Linear layout), bf16 on v_mfma_f32_32x32x16_bf16 with f32
// accumulation: a block owns a BM x BN tile, its waves a (BM/WM) x (BN/WN)
// sub-tile; K streams through an LDS ring in steps of 64 by
// direct-to-LDS loads (each one-KB load is eight 128-byte row segments, the
// 16-byte chunks of row r stored at chunk ^ pj_swz(r)).
// After the last step the f32 tile is staged in LDS and an epilogue policy
// finishes the rows: the K/V split store, the rotary q store, or LayerNorm +
// rotary k plus the f32 head weights.
#include "dsa_device.hpp"
#include "dsa_internal.hpp"

#include <math.h>

namespace dsa {

constexpr int PJ_BK = 64;     // K elements per stage: 128 bytes of each row

template <int BM, int BN, int WM, int WN, int ST, int CR = BM>
struct PjCfg {
    static constexpr int NW = WM * WN;
    static constexpr int NT = 64 * NW;
    static constexpr int TM = BM / WM / 32;   // 32x32 tiles per wave along M
    static constexpr int TN = BN / WN / 32;   // and along N
    static constexpr int AB = BM * PJ_BK * 2; // stage bytes of A
    static constexpr int SB = AB + BN * PJ_BK * 2;
    static constexpr int DMA = SB / 1024;     // one-KB loads per stage
    static constexpr int LPW = DMA / NW;      // of them per wave
    static constexpr int CP = BN + 4;         // staged C row pitch in floats
    static constexpr int RING = ST * SB;
    static constexpr int CTILE = CR * CP * 4;  // staged C rows (CR of them at a time)
    static constexpr int LDS = RING > CTILE ? RING : CTILE;
    static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "whole MFMA tiles per wave");
    static_assert(DMA * 1024 == SB && DMA % NW == 0, "equal one-KB loads per wave");
    static_assert(LPW * 3 <= 63 && ST >= 2 && ST <= 4, "vmcnt range, ring depth");
    static_assert(BM % CR == 0 && CR % 32 == 0, "row chunks of whole 32-row tiles");
};

// Operand sources: rows [0, n_split) of B come from b0, the rest from b1
// (the fused k / head-weight projection reads two weight matrices).
struct PjOperands {
    const uint16_t *a;
    int64_t lda;
    const uint16_t *b0, *b1;
    int64_t ldb;
    int M, N, K, n_split;
};

// ---------------------------------------------------------------- epilogues

// Rotary frequencies inv[i] = theta^(-2i / rope_dim), i < rope_dim / 2,
// computed on the host in f64 and passed by value.
struct RopeArgs {
    double inv[64];
    int rope_dim;
};

// Rotate the pair (x, y) by the angle pos * inv: the angle is formed and
// reduced to [-pi, pi] in f64 (exact enough at any position below 2^31),
// then its sine and cosine are taken in f32.
__device__ __forceinline__ void rope_pair(float &x, float &y, int pos, double inv)
{
    const double two_pi = 6.283185307179586476925286766559;
    const double a = (double)pos * inv;
    const double r = fma(-rint(a * (1.0 / two_pi)), two_pi, a);
    float s, c;
    sincosf((float)r, &s, &c);
    const float x2 = x * c - y * s;
    const float y2 = y * c + x * s;
    x = x2;
    y = y2;
}

__device__ __forceinline__ void store_bf16x8(uint16_t *dst, const float (&v)[8])
{
    u32x4_t p;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        p[j] = cvt_pk_bf16(v[2 * j], v[2 * j + 1]);
    *reinterpret_cast<u32x4_t *>(dst) = p;
}

__device__ __forceinline__ void load_f32x8(float (&v)[8], const float *c)
{
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = c[j];
}

// Rows of one 128-wide head vector in the staged tile: chunk c < R/16 of the
// rope part is rotated with its partner chunk c + R/16 (entries i and
// i + R/2 pair up), the other chunks are copied; bf16 out.  `row` points at
// the head's first staged column, `dst` at its first output element.
__device__ __forceinline__ void head_item(const float *row, uint16_t *dst, int item, int pos,
                                          const RopeArgs &rp)
{
    const int nr = rp.rope_dim / 16;  // rotated chunk pairs
    if (item < nr) {
        const int c0 = item, c1 = item + nr;
        float x[8], y[8];
        load_f32x8(x, row + c0 * 8);
        load_f32x8(y, row + c1 * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            rope_pair(x[j], y[j], pos, rp.inv[c0 * 8 + j]);
        store_bf16x8(dst + c0 * 8, x);
        store_bf16x8(dst + c1 * 8, y);
    } else {
        const int c = item - nr + 2 * nr;  // chunks 2nr .. 15 pass through
        float x[8];
        load_f32x8(x, row + c * 8);
        store_bf16x8(dst + c * 8, x);
    }
}

// q: the tile holds whole heads of 128: out[m][head][0..128).
struct EpiRopeQ {
    uint16_t *out;
    int64_t out_row;  // elements per token (n_heads * 128)
    const int32_t *pos;
    RopeArgs rope;

    template <int BM, int BN, int NT>
    __device__ void run(const float *C, int m0, int n0, int M, int tid) const
    {
        static_assert(BN % 128 == 0, "whole heads of 128 per tile");
        constexpr int HT = BN / 128;
        const int ipr = rope.rope_dim / 16 + (128 - rope.rope_dim) / 8;
        for (int it = tid; it < BM * HT * ipr; it += NT) {
            const int r = it / (HT * ipr), rem = it % (HT * ipr);
            const int hh = rem / ipr, item = rem % ipr;
            const int m = m0 + r;
            if (m >= M)
                continue;
            head_item(C + r * (BN + 4) + hh * 128,
                      out + (int64_t)m * out_row + n0 + hh * 128, item, pos[m], rope);
        }
    }
};

// k and the head weights (BN = 128 + n_heads): LayerNorm over the 128 k
// columns (two threads per row, two-pass mean and variance in f32), weight
// and bias, then the rotation; the head weights go out as f32.
struct EpiNormRopeK {
    uint16_t *k_out;    // [T, 128]
    float *w_out;       // [T, n_heads]
    const float *gamma, *beta;
    float eps;
    int n_heads;
    const int32_t *pos;
    RopeArgs rope;

    template <int BM, int BN, int NT>
    __device__ void run(float *C, int m0, int n0, int M, int tid) const
    {
        static_assert(NT == 2 * BM, "two threads per row");
        constexpr int CP = BN + 4;
        {
            const int r = tid >> 1, h = tid & 1;
            float *row = C + r * CP + 64 * h;
            float s = 0.f;
            for (int j = 0; j < 64; ++j)
                s += row[j];
            s += __shfl_xor(s, 1);
            const float mu = s * (1.0f / 128.0f);
            float v = 0.f;
            for (int j = 0; j < 64; ++j) {
                const float d = row[j] - mu;
                v = fmaf(d, d, v);
            }
            v += __shfl_xor(v, 1);
            const float inv_sd = 1.0f / sqrtf(v * (1.0f / 128.0f) + eps);
            for (int j = 0; j < 64; ++j)
                row[j] = fmaf((row[j] - mu) * inv_sd, gamma[64 * h + j], beta[64 * h + j]);
        }
        __syncthreads();
        const int ipk = rope.rope_dim / 16 + (128 - rope.rope_dim) / 8;
        const int ipr = ipk + n_heads / 4;
        for (int it = tid; it < BM * ipr; it += NT) {
            const int r = it / ipr, item = it % ipr;
            const int m = m0 + r;
            if (m >= M)
                continue;
            const float *row = C + r * CP;
            if (item < ipk) {
                head_item(row, k_out + (int64_t)m * 128, item, pos[m], rope);
            } else {
                const int c = item - ipk;  // four head weights per item
                f32x4_t w;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w[j] = row[128 + 4 * c + j];
                *reinterpret_cast<f32x4_t *>(w_out + (int64_t)m * n_heads + 4 * c) = w;
            }
        }
        (void)n0;
    }
};

// expand_kv: column n = head * (kd + vd) + j goes to K[m][head][j] for
// j < kd, else V[m][head][j - kd]; eight columns per 16-byte store (kd, vd
// and the row strides are multiples of 8).
struct EpiSplitKV {
    uint16_t *k, *v;
    int64_t ksr, vsr;  // elements per token
    int kd, vd;

    template <int BM, int BN, int NT>
    __device__ void run(const float *C, int m0, int n0, int M, int N, int tid) const
    {
        constexpr int CPR = BN / 8;
        const int hw = kd + vd;
        for (int it = tid; it < BM * CPR; it += NT) {
            const int r = it / CPR, c = it % CPR;
            const int m = m0 + r, n = n0 + 8 * c;
            if (m >= M || n >= N)
                continue;
            const int head = n / hw, j = n - head * hw;
            uint16_t *dst = j < kd ? k + (int64_t)m * ksr + (int64_t)head * kd + j
                                   : v + (int64_t)m * vsr + (int64_t)head * vd + (j - kd);
            float x[8];
            load_f32x8(x, C + r * (BN + 4) + 8 * c);
            store_bf16x8(dst, x);
        }
    }
};

// ---------------------------------------------------------------- GEMM body

// Tile of logical block b on a grid of mb x nb tiles: each XCD takes a
// contiguous run of b (xcd_remap), and a run walks groups of GM tile rows
// column by column, so the tiles an XCD holds at once share GM row blocks of
// A and a few column blocks of B in its L2.
template <int GM>
__device__ __forceinline__ void pj_tile_of(int b, int mb, int nb, int &tm, int &tn)
{
    const int per_group = GM * nb;
    const int grp = b / per_group, in = b % per_group;
    const int first = grp * GM;
    const int gm = min(mb - first, GM);
    tm = first + in % gm;
    tn = in / gm;
}

constexpr int PJ_GROUP_M = 8;

// Chunk swizzle of the 128-byte operand rows: physical chunk = logical chunk
// ^ ((r >> 1) & 7).  A ds_read_b128 serves 16 lanes per pass (64 banks x 4
// bytes); the operand reads give 16 consecutive rows at one logical chunk to
// those lanes.  Row r starts at bank 32 (r & 1), so the even rows and the odd
// rows each need eight distinct chunk slots, which (r >> 1) & 7 gives.
__device__ __forceinline__ int pj_swz(int r)
{
    return (r >> 1) & 7;
}

// wait until at most W LDS reads are outstanding, tied to every register
// of one operand buffer
template <int W, int N>
__device__ __forceinline__ void wait_operands(u32x4_t (&v)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        lds_operand_wait<W>(v[i]);
}

// The block's f32 tile C = A[m0 .. m0+BM) B[n0 .. n0+BN)^T in the waves'
// accumulators (wave (wm, wn) holds rows wm * BM/WM .., columns wn * BN/WN ..),
// each 32 x 32 block transposed: the MFMA takes the B fragment as its first
// operand, so lane l holds row l % 32 and four consecutive columns per
// group of four accumulators (8 (e / 4) + 4 (l / 32) + e % 4).
// Rows past M (and past N) load the last valid row instead, so every load
// stays inside the operands; the epilogues skip them.
template <int BM, int BN, int WM, int WN, int ST>
__device__ __forceinline__ void pj_tile(const PjOperands &op, int m0, int n0, unsigned char *smem,
                                        f32x16_t (&acc)[BM / WM / 32][BN / WN / 32])
{
    using Cfg = PjCfg<BM, BN, WM, WN, ST>;
    constexpr int TM = Cfg::TM, TN = Cfg::TN, LPW = Cfg::LPW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid % WM, wn = wid / WM;
    const uint32_t lds0 = lds_addr(smem);

    // this lane's source row segment for each of its loads
    const uint16_t *src[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int j = wid + Cfg::NW * i;        // the load: rows 8j .. 8j+7
        const int r = 8 * j + (lane >> 3);      // row of the stage (A rows, then B rows)
        const int chunk = (lane & 7) ^ pj_swz(r);
        if (r < BM) {
            const int m = min(m0 + r, op.M - 1);
            src[i] = op.a + (int64_t)m * op.lda + chunk * 8;
        } else {
            const int n = min(n0 + r - BM, op.N - 1);
            src[i] = (n < op.n_split ? op.b0 + (int64_t)n * op.ldb
                                     : op.b1 + (int64_t)(n - op.n_split) * op.ldb) +
                     chunk * 8;
        }
    }
    auto issue = [&](int kt, int st) {
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            lds_dma16(src[i] + kt * PJ_BK, smem + st * Cfg::SB + (wid + Cfg::NW * i) * 1024);
    };

    // operand read addresses in stage 0 (k-step s adds 32 bytes: chunks 2s, 2s+1)
    uint32_t a_addr[TM], b_addr[TN];
    const int g = lane >> 5;
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const int r = wm * (BM / WM) + t * 32 + (lane & 31);
        a_addr[t] = lds0 + r * 128 + ((g ^ pj_swz(r)) << 4);
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int r = BM + wn * (BN / WN) + t * 32 + (lane & 31);
        b_addr[t] = lds0 + r * 128 + ((g ^ pj_swz(r)) << 4);
    }

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.f;

    const int nk = op.K / PJ_BK;
    int issued = 0;
    for (; issued < ST - 1 && issued < nk; ++issued)
        issue(issued, issued);
    for (int kt = 0; kt < nk; ++kt) {
        vm_wait_tiles<LPW>(issued - kt - 1);
        lds_barrier();  // stage kt landed for every wave; stage kt-1 is free
        if (issued < nk) {
            issue(issued, issued % ST);
            ++issued;
        }
        const uint32_t so = (uint32_t)((kt % ST) * Cfg::SB);
        // the chunk pair of k-step s: logical chunks 2s + g; the swizzle XORs
        // the low three bits, and 2s only touches bits 1-2, so the physical
        // chunk is (g ^ swz) ^ 2s.  The operands of k-step s+1 are read while
        // the MFMAs of k-step s run (two register buffers).
        u32x4_t av[2][TM], bv[2][TN];
        auto read = [&](int s, int buf) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
                lds_read_b128_nowait(av[buf][t], (a_addr[t] + so) ^ (uint32_t)(s << 5));
#pragma unroll
            for (int t = 0; t < TN; ++t)
                lds_read_b128_nowait(bv[buf][t], (b_addr[t] + so) ^ (uint32_t)(s << 5));
        };
        read(0, 0);
#pragma unroll
        for (int s = 0; s < PJ_BK / 16; ++s) {
            const int cur = s & 1;
            if (s + 1 < PJ_BK / 16) {
                read(s + 1, cur ^ 1);
                wait_operands<TM + TN>(av[cur]);
                wait_operands<TM + TN>(bv[cur]);
            } else {
                wait_operands<0>(av[cur]);
                wait_operands<0>(bv[cur]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = mfma_32x32x16(bv[cur][j], av[cur][i], acc[i][j]);
        }
    }
    lds_barrier();  // every wave is done with the ring before it is reused
}

// Stage the tile in LDS CR rows at a time and hand each chunk to
// finish(C, r0) on every thread.  A lane writes its row's four consecutive
// columns as one 16-byte store; the row pitch of BN + 4 floats starts each
// of 16 consecutive rows on a different group of four banks.
template <int BM, int BN, int WM, int WN, int CR, class F>
__device__ __forceinline__ void pj_stage(const f32x16_t (&acc)[BM / WM / 32][BN / WN / 32],
                                         unsigned char *smem, F &&finish)
{
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32, CP = BN + 4;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid % WM, wn = wid / WM;
    const int g = lane >> 5;
    float *C = reinterpret_cast<float *>(smem);
    for (int r0 = 0; r0 < BM; r0 += CR) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int rt = wm * (BM / WM) + i * 32;  // the 32-row tile's first row
            if (rt < r0 || rt >= r0 + CR)
                continue;
            const int row = rt - r0 + (lane & 31);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = wn * (BN / WN) + j * 32 + 8 * q + 4 * g;
                    *reinterpret_cast<f32x4_t *>(C + row * CP + col) =
                        f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                acc[i][j][4 * q + 3]};
                }
            }
        }
        lds_barrier();  // LDS only: the chunk's global stores stay in flight
        finish(C, r0);
        lds_barrier();
    }
}

template <int BM, int BN, int WM, int WN, int ST, int CR>
__global__ __launch_bounds__(64 * WM *WN) void pj_rope_q_kernel(PjOperands op, EpiRopeQ epi)
{
    using Cfg = PjCfg<BM, BN, WM, WN, ST, CR>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg::LDS];
    DSA_LDS_ESCAPE(smem);
    const int nb = (op.N + BN - 1) / BN, mb = (op.M + BM - 1) / BM;
    int tm, tn;
    pj_tile_of<PJ_GROUP_M>(xcd_remap(blockIdx.x, gridDim.x), mb, nb, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    f32x16_t acc[Cfg::TM][Cfg::TN];
    pj_tile<BM, BN, WM, WN, ST>(op, m0, n0, smem, acc);
    pj_stage<BM, BN, WM, WN, CR>(acc, smem, [&](const float *C, int r0) {
        epi.template run<CR, BN, Cfg::NT>(C, m0 + r0, n0, op.M, threadIdx.x);
    });
}

template <int BM, int BN, int WM, int WN, int ST>
__global__ __launch_bounds__(64 * WM *WN) void pj_norm_k_kernel(PjOperands op, EpiNormRopeK epi)
{
    using Cfg = PjCfg<BM, BN, WM, WN, ST>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg::LDS];
    DSA_LDS_ESCAPE(smem);
    const int m0 = blockIdx.x * BM;
    f32x16_t acc[Cfg::TM][Cfg::TN];
    pj_tile<BM, BN, WM, WN, ST>(op, m0, 0, smem, acc);
    pj_stage<BM, BN, WM, WN, BM>(acc, smem, [&](float *C, int r0) {
        epi.template run<BM, BN, Cfg::NT>(C, m0 + r0, 0, op.M, threadIdx.x);
    });
}

template <int BM, int BN, int WM, int WN, int ST, int CR>
__global__ __launch_bounds__(64 * WM *WN) void pj_expand_kv_kernel(PjOperands op, EpiSplitKV epi)
{
    using Cfg = PjCfg<BM, BN, WM, WN, ST, CR>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg::LDS];
    DSA_LDS_ESCAPE(smem);
    const int nb = (op.N + BN - 1) / BN, mb = (op.M + BM - 1) / BM;
    int tm, tn;
    pj_tile_of<PJ_GROUP_M>(xcd_remap(blockIdx.x, gridDim.x), mb, nb, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    f32x16_t acc[Cfg::TM][Cfg::TN];
    pj_tile<BM, BN, WM, WN, ST>(op, m0, n0, smem, acc);
    pj_stage<BM, BN, WM, WN, CR>(acc, smem, [&](const float *C, int r0) {
        epi.template run<CR, BN, Cfg::NT>(C, m0 + r0, n0, op.M, op.N, threadIdx.x);
    });
}

// ---------------------------------------------------------------- host side

static RopeArgs rope_args(int rope_dim, float theta)
{
    RopeArgs r{};
    r.rope_dim = rope_dim;
    for (int i = 0; i < rope_dim / 2; ++i)
        r.inv[i] = pow((double)theta, -2.0 * i / rope_dim);
    return r;
}

// q and expand_kv: 256 x 256 tiles of 8 waves, each 64 x 128 (8 MFMAs per
// 6 operand reads), a two-stage ring of 64 KB stages; the tile is staged
// 64 rows at a time for the epilogue.  k and the head weights: the whole
// 128 + n_heads columns in one tile (LayerNorm needs the full row).
constexpr int PJ_Q_BM = 256, PJ_Q_BN = 256;
constexpr int PJ_K_BM = 128;
constexpr int PJ_E_BM = 256, PJ_E_BN = 256;
constexpr int PJ_CR = 64;

hipError_t launch_indexer_frontend(const FrontendArgs &a, hipStream_t st)
{
    const RopeArgs rp = rope_args(a.rope_dim, a.rope_theta);
    {
        PjOperands op{static_cast<const uint16_t *>(a.q_lora), a.q_lora_rank,
                      static_cast<const uint16_t *>(a.wq_b), nullptr, a.q_lora_rank,
                      a.tokens, a.n_heads * 128, a.q_lora_rank, a.n_heads * 128};
        EpiRopeQ epi{static_cast<uint16_t *>(a.q_out), (int64_t)a.n_heads * 128, a.pos, rp};
        const int64_t blocks =
            (int64_t)((a.tokens + PJ_Q_BM - 1) / PJ_Q_BM) * ((op.N + PJ_Q_BN - 1) / PJ_Q_BN);
        if (blocks > 0x7fffffff)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((pj_rope_q_kernel<PJ_Q_BM, PJ_Q_BN, 4, 2, 2, PJ_CR>),
                           dim3((unsigned)blocks), dim3(512), 0, st, op, epi);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    PjOperands op{static_cast<const uint16_t *>(a.x), a.hidden,
                  static_cast<const uint16_t *>(a.wk), static_cast<const uint16_t *>(a.w_proj),
                  a.hidden, a.tokens, 128 + a.n_heads, a.hidden, 128};
    EpiNormRopeK epi{static_cast<uint16_t *>(a.k_out), a.w_out, a.k_norm_w, a.k_norm_b,
                     a.norm_eps, a.n_heads, a.pos, rp};
    const unsigned blocks = (unsigned)((a.tokens + PJ_K_BM - 1) / PJ_K_BM);
    if (a.n_heads == 32)
        hipLaunchKernelGGL((pj_norm_k_kernel<PJ_K_BM, 160, 4, 1, 3>), dim3(blocks), dim3(256), 0,
                           st, op, epi);
    else
        hipLaunchKernelGGL((pj_norm_k_kernel<PJ_K_BM, 192, 4, 1, 3>), dim3(blocks), dim3(256), 0,
                           st, op, epi);
    return hipGetLastError();
}

hipError_t launch_expand_kv(const ExpandArgs &a, hipStream_t st)
{
    const int N = a.n_heads * (a.kd + a.vd);
    PjOperands op{static_cast<const uint16_t *>(a.latent), a.rank,
                  static_cast<const uint16_t *>(a.w_kv_b), nullptr, a.rank, a.tokens, N, a.rank,
                  N};
    EpiSplitKV epi{static_cast<uint16_t *>(a.k_out), static_cast<uint16_t *>(a.v_out),
                   a.k_row_stride, a.v_row_stride, a.kd, a.vd};
    const int64_t blocks =
        (int64_t)((a.tokens + PJ_E_BM - 1) / PJ_E_BM) * ((N + PJ_E_BN - 1) / PJ_E_BN);
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((pj_expand_kv_kernel<PJ_E_BM, PJ_E_BN, 4, 2, 2, PJ_CR>),
                       dim3((unsigned)blocks), dim3(512), 0, st, op, epi);
    return hipGetLastError();
}

} // namespace dsa
