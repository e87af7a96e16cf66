// dsa_device.hpp -- device-side helpers shared by the libdsa kernels (gfx950).
//
// MFMA operand layouts used throughout (CDNA3/CDNA4 wave64 conventions):
//  v_mfma_f32_32x32x16_bf16: lane l supplies A[l%32][g*8 .. g*8+7] and
//    B[g*8 .. g*8+7][l%32] with g = l/32; it receives
//    C[8*(i/4) + 4*g + i%4][l%32] in accumulator i (i < 16).
//  v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][g*8 .. g*8+7] and
//    B[g*8 .. g*8+7][l%16] with g = l/16; it receives C[4*g + i][l%16] in
//    accumulator i (i < 4).
// The contraction index k = g*8 + j is only a label: any bijection between
// (g, j) and the physical reduction index gives the same product as long as
// A and B use the same one.  The kernels use that freedom to make each
// lane's loads contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Online softmax: the running reference max is only raised when a tile's max
// exceeds it by more than this (log2 units), bounding p = 2^(x - m) by 2^8.
constexpr float kRescaleLog2 = 8.f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16)
{
    return __uint_as_float(b16 << 16);
}

// Round-to-nearest-even float -> bf16 bits (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats -> packed bf16x2 (low half = a), one v_cvt_pk_bf16_f32 (RNE).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Two-term bf16 split of 8 f32 weights, packed as MFMA operands:
// hi = bf16(p), lo = bf16(p - hi).  p - hi is exact in f32, so hi + lo
// carries about 16 significant bits of p.
__device__ __forceinline__ void split_bf16x8(const float (&p)[8], uint32_t (&hi)[4],
                                             uint32_t (&lo)[4])
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t h = cvt_pk_bf16(p[2 * k], p[2 * k + 1]);
        hi[k] = h;
        lo[k] = cvt_pk_bf16(p[2 * k] - __uint_as_float(h << 16),
                            p[2 * k + 1] - __uint_as_float(h & 0xffff0000u));
    }
}

__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t &a, const u32x4_t &b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_32x32x16(const u32x4_t &a, const u32x4_t &b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Four OCP e4m3 codes (one dword) -> four bf16 (two dwords).  Every e4m3
// value is exactly representable in bf16 (4 significant bits, exponent range
// inside bf16's), so truncating the exact f32 to its upper half is exact.
__device__ __forceinline__ u32x2_t e4m3x4_to_bf16x4(uint32_t codes)
{
    f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, false);
    f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, true);
    u32x2_t r;
    r[0] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xffff0000u);
    r[1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u);
    return r;
}

// LDS pointers for the gfx950 LDS builtins.
typedef short lds_v4i16_t __attribute__((ext_vector_type(4)));
#define DSA_LDS_PTR(T, p) ((T __attribute__((address_space(3))) *)(p))

// Direct global -> LDS copy (global_load_lds_dwordx4): each lane copies 16
// bytes from its own `src`; lane l's bytes land at lds_base + 16*l, so one
// wave instruction fills 1 KB of LDS.  lds_base must be wave-uniform.
// Completion is tracked by vmcnt (wait with s_waitcnt before reading).
__device__ __forceinline__ void lds_dma16(const void *src, void *lds_base)
{
    __builtin_amdgcn_global_load_lds(src, DSA_LDS_PTR(void, lds_base), 16, 0, 0);
}

// Make an LDS object's address visible to an opaque asm.  An LDS array that
// only lds_dma16 ever fills is otherwise seen by the optimizer as never
// stored to (its initial value is undefined), and reads of it may be folded.
#define DSA_LDS_ESCAPE(obj) asm volatile("" ::"s"((const void *)&(obj)) : "memory")

// Wait until at most N of this wave's vector-memory operations (LDS DMA
// included; they complete in issue order) are outstanding.  gfx9 s_waitcnt
// immediate: vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15)
// left at "no wait".
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}

// An LDS operand read issued now and waited for later, so that reads run a
// few MFMAs ahead of their use.  lds_operand_wait<N> waits until at most N
// LDS operations are outstanding (LDS reads complete in issue order, and an
// SMEM load in flight only makes the wait stricter) and ties the register to
// that wait, so the compiler cannot use it earlier.  Nothing may read or
// copy the destination between the two calls; users check the generated
// code for that.
__device__ __forceinline__ void lds_read_b128_nowait(u32x4_t &v, uint32_t a)
{
    asm volatile("ds_read_b128 %0, %1" : "=&v"(v) : "v"(a) : "memory");
}
template <int N>
__device__ __forceinline__ void lds_operand_wait(u32x4_t &v)
{
    static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N) : "memory");
}
template <int O>
__device__ __forceinline__ void lds_read_b128_nowait(u32x4_t &v, uint32_t a)
{
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(v) : "v"(a), "i"(O) : "memory");
}
template <int O>
__device__ __forceinline__ void lds_read_b32_nowait(uint32_t &v, uint32_t a)
{
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=&v"(v) : "v"(a), "i"(O) : "memory");
}
template <int N>
__device__ __forceinline__ void lds_operand_wait(uint32_t &v)
{
    static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N) : "memory");
}
// Transposing 4 x 16-bit read (ds_read_b64_tr_b16) issued now, waited for
// by lds_operand_wait on the pair it belongs to.
template <int O>
__device__ __forceinline__ void lds_read_tr16_nowait(u32x2_t &v, uint32_t a)
{
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=&v"(v) : "v"(a), "i"(O) : "memory");
}
template <int N>
__device__ __forceinline__ void lds_operand_wait(u32x2_t &v0, u32x2_t &v1)
{
    static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(v0), "+v"(v1) : "n"(N) : "memory");
}

// vm_wait<N * per_tile> for a runtime N in [0, 3] (the tiles still in flight
// behind the one needed).
template <int PER_TILE>
__device__ __forceinline__ void vm_wait_tiles(int tiles_after)
{
    switch (tiles_after) {
    case 0: vm_wait<0>(); break;
    case 1: vm_wait<PER_TILE>(); break;
    case 2: vm_wait<2 * PER_TILE>(); break;
    default: vm_wait<3 * PER_TILE>(); break;
    }
}

// Workgroup barrier that orders LDS only: this wave's LDS reads and writes
// are complete before it arrives.  __syncthreads() also makes the compiler
// wait for every direct-to-LDS load still in flight (it counts them as
// pending LDS writes), which would drain the tiles being prefetched; callers
// of this barrier wait for the tiles they need themselves (vm_wait).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 4 bytes per lane, global -> LDS at lds_base + 4*lane.
__device__ __forceinline__ void lds_dma4(const void *src, void *lds_base)
{
    __builtin_amdgcn_global_load_lds(src, DSA_LDS_PTR(void, lds_base), 4, 0, 0);
}

// Plain LDS reads at a 32-bit LDS byte address, for waves that issue no
// direct-to-LDS loads themselves (the compiler then has no such loads to wait
// for in front of them, and schedules and allocates them freely).
__device__ __forceinline__ u32x4_t lds_ld128(uint32_t a)
{
    return *(const u32x4_t __attribute__((address_space(3))) *)(uintptr_t)a;
}
__device__ __forceinline__ u32x2_t lds_ld_tr16(uint32_t a)
{
    const lds_v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t __attribute__((address_space(3))) *)(uintptr_t)a);
    return __builtin_bit_cast(u32x2_t, r);
}

// LDS atomic OR without return (ds_or_b32) at a byte address.  Written as asm
// so that the compiler does not order it behind the direct-to-LDS loads in
// flight (it would wait for them before any LDS store); the next
// lds_barrier (s_waitcnt lgkmcnt(0)) covers its completion.
__device__ __forceinline__ void lds_or_async(uint32_t lds_byte_addr, uint32_t bits)
{
    asm volatile("ds_or_b32 %0, %1" ::"v"(lds_byte_addr), "v"(bits) : "memory");
}

// Six 4-byte LDS reads from per-lane byte addresses and the wait for them, in
// one asm statement (the destinations are complete when the compiler first
// sees them; no wait for direct-to-LDS loads in flight is implied).
__device__ __forceinline__ void lds_read_u32_x6(uint32_t (&v)[6], const uint32_t (&a)[6])
{
    asm volatile(
        "ds_read_b32 %0, %6\n\t"
        "ds_read_b32 %1, %7\n\t"
        "ds_read_b32 %2, %8\n\t"
        "ds_read_b32 %3, %9\n\t"
        "ds_read_b32 %4, %10\n\t"
        "ds_read_b32 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
        : "memory");
}

// N 16-byte LDS reads from per-lane byte addresses and the wait for them, in
// one asm statement (N = 4 or 8).
__device__ __forceinline__ void lds_read_b128_a4(u32x4_t (&v)[4], const uint32_t (&a)[4])
{
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
}
__device__ __forceinline__ void lds_read_b128_a8(u32x4_t (&v)[8], const uint32_t (&a)[8])
{
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7])
        : "memory");
}
// One 4-byte LDS read and the wait for it.
__device__ __forceinline__ uint32_t lds_read_u32_wait(uint32_t a)
{
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
    return v;
}

// 32-bit LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)DSA_LDS_PTR(const char, p);
}

// XOR swizzle of the 16-byte chunks of row r of an LDS tile whose rows are a
// multiple of 128 bytes apart and hold a multiple of 8 chunks: physical chunk
// = logical chunk ^ chunk_swz(r).  Eight consecutive rows read at the same
// logical chunk (ds_read_b128 operand fetches) hit 8 different chunk slots,
// and the 4 rows x 2 adjacent chunks of a transposing read do too.
__device__ __forceinline__ int chunk_swz(int row)
{
    return ((row & 3) << 1) | ((row >> 2) & 1);
}

// Swizzle for tiles whose rows are an odd multiple of 128 bytes apart (the
// 1152-byte latent rows): physical chunk = logical chunk ^ (row & 7).  On
// gfx950 (64 banks of 4 bytes) this keeps both access patterns of the
// absorbed attention at full LDS rate, measured: the Q.K^T operand reads
// (ds_read_b128, 16 rows x 4 chunk columns per instruction) and the
// transposing P.V reads (ds_read_b64_tr_b16, 16 rows x 2 chunks); the
// swizzles built for 32 lanes per cycle halve the ds_read_b128 rate.
__device__ __forceinline__ int chunk_swz_odd(int row)
{
    return row & 7;
}

// XCD-aware block order.  The dispatcher deals consecutive workgroup ids
// round-robin over the 8 XCDs (each with its own L2), so id b runs on XCD
// b % 8.  This maps b to a logical index such that each XCD receives one
// contiguous range of logical indices: blocks that share data (the splits
// of one query row, and later the merge of that row) then share an L2.  A
// bijection on [0, total) for any total.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int b, int total)
{
    const int per = total / kXcds, rem = total % kXcds;
    const int x = b % kXcds, j = b / kXcds;
    return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + j;
}

// Order-preserving map of an f32 score to u32: larger score <=> larger key.
// -0 is first folded onto +0 so that the two compare equal.
__device__ __forceinline__ uint32_t score_order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide reductions (wave64), every lane gets the result, without LDS:
// DPP quad_perm [1,0,3,2] and [2,3,0,1] reduce each quad, row_half_mirror
// pairs the two quads of each half-row, row_mirror the two halves of each
// 16-lane row, then the gfx950 row swaps v_permlane16_swap / v_permlane32_swap
// pair the rows (each returns both values of the pair).
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_bits(uint32_t v, Op op)
{
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return op(b[0], b[1]);
}

__device__ __forceinline__ float wave_max(float v)
{
    return __uint_as_float(wave_reduce_bits(__float_as_uint(v), [](uint32_t x, uint32_t y) {
        return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
    }));
}

__device__ __forceinline__ float wave_sum(float v)
{
    return __uint_as_float(wave_reduce_bits(__float_as_uint(v), [](uint32_t x, uint32_t y) {
        return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
    }));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    return wave_reduce_bits(v, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    return wave_reduce_bits(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}

__device__ __forceinline__ int wave_sum_int(int v)
{
    return (int)wave_reduce_bits((uint32_t)v, [](uint32_t x, uint32_t y) { return x + y; });
}

// max / sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows)
// with the gfx950 row-swap instructions: v_permlane16_swap pairs each lane
// with its partner one row away, v_permlane32_swap with the partner half a
// wave away; each returns both values of the pair, so a symmetric op of the
// two is the reduction over the pair (no LDS round trip).
__device__ __forceinline__ float max_across_rows(float v)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_across_rows(float v)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), with
// DPP moves: shifts by 1, 2, 4 and 8 lanes inside each 16-lane row give the
// row prefixes, then row_bcast:15 adds row r-1's total into rows 1 and 3 and
// row_bcast:31 adds the total of rows 0-1 into rows 2 and 3.  A lane whose
// source is outside its row, or whose row is masked off, reads the "old"
// operand 0.
__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

} // namespace dsa
