// peaks.hip -- two calibration kernels for the measurement harness (not
// part of libdsa): a plain streaming copy, whose rate is the HBM bandwidth
// a simple kernel reaches on this GPU, and a loop of bf16 MFMAs with no
// memory traffic, whose rate is the matrix cores' reachable dense bf16
// throughput at the clock the chip actually runs under that load.  Both are
// reported next to the published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte loads and stores.  Each workgroup copies one contiguous span,
// four 4 KB rows of it per round with all four loads issued before the
// stores, so every wave keeps whole cache lines of one DRAM page in flight.
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4_t *__restrict__ src,
                                                         u32x4_t *__restrict__ dst, int64_t n16)
{
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    int64_t i = b0 + threadIdx.x;
    for (; i + 768 < b1; i += 1024) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        const u32x4_t b = __builtin_nontemporal_load(src + i + 256);
        const u32x4_t c = __builtin_nontemporal_load(src + i + 512);
        const u32x4_t d = __builtin_nontemporal_load(src + i + 768);
        __builtin_nontemporal_store(a, dst + i);
        __builtin_nontemporal_store(b, dst + i + 256);
        __builtin_nontemporal_store(c, dst + i + 512);
        __builtin_nontemporal_store(d, dst + i + 768);
    }
    for (; i < b1; i += 256)
        dst[i] = src[i];
}

// Each wave keeps four independent accumulation chains of
// v_mfma_f32_32x32x16_bf16 (32768 flops each) busy for `iters` rounds; the
// operands come from the lane index so nothing folds, and one value per
// lane is stored so nothing is dropped.
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float *__restrict__ out)
{
    const uint32_t l = threadIdx.x;
    const u32x4_t a = {0x3f803f80u ^ l, 0x3f003f00u, 0x3e803e80u, 0x3f403f40u ^ (l << 1)};
    const u32x4_t b = {0x3f803f80u, 0x3f003f00u ^ l, 0x3f403f40u, 0x3e803e80u};
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a), bv = __builtin_bit_cast(bf16x8_t, b);
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, av, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, av, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, bv, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        s += c0[j] + c1[j] + c2[j] + c3[j];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Direct-to-LDS streaming of 32 KB tiles, the way the attention kernels
// stage theirs: one workgroup of 8 waves per CU, 29 one-KB
// global_load_lds_dwordx4 per tile (four per wave; waves 0-6 take four
// slots, wave 7 one), a ring of four LDS stages, two tiles in flight, one
// workgroup barrier per tile.  Workgroup b reads tile (7b + i) mod n_tiles at
// step i, so a small n_tiles is served by L2 and a large one by HBM.
__global__ __launch_bounds__(512, 1) void probe_lds_stream_kernel(const unsigned char *__restrict__ src,
                                                                 int n_tiles, int steps,
                                                                 uint32_t *__restrict__ sink)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds[4][32768];
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    uint32_t acc = 0;
    for (int i = 0; i < steps; ++i) {
        const unsigned char *s = src + (size_t)((blockIdx.x * 7 + i) % n_tiles) * 32768;
        const int st = i & 3;
        for (int j = 0; j < 4; ++j) {
            const int slot = wid * 4 + j;
            if (slot < 29)
                __builtin_amdgcn_global_load_lds(
                    s + slot * 1024 + lane * 16,
                    (__attribute__((address_space(3))) void *)&lds[st][slot * 1024], 16, 0, 0);
        }
        // the tile issued two steps ago has landed (at most the last two
        // tiles' loads outstanding), then every wave's share is visible
        if (i >= 2)
            __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));  // vmcnt(8)
        else
            __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // vmcnt(0)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        acc += *reinterpret_cast<const uint32_t *>(&lds[(i + 2) & 3][lane * 4]);
    }
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));
    asm volatile("s_barrier" ::: "memory");
    if (acc == 0x12345678u)
        sink[0] = acc;
}

extern "C" {

// Copies `bytes` (a multiple of 16) from src to dst on `stream`.
int probe_copy(const void *src, void *dst, int64_t bytes, int blocks, void *stream)
{
    if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || blocks <= 0)
        return -1;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream),
                       static_cast<const u32x4_t *>(src), static_cast<u32x4_t *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// `blocks` workgroups of 4 waves, each wave 4 * iters MFMAs of 32x32x16;
// `out` holds blocks * 256 floats.  Flops = blocks * 4 * iters * 4 * 32768.
int probe_mfma_bf16(int blocks, int iters, float *out, void *stream)
{
    if (!out || blocks <= 0 || iters <= 0)
        return -1;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// 256 workgroups stream `steps` tiles each from src (n_tiles tiles of
// 32 KB); bytes moved = 256 * steps * 29 KB.  sink: 4 bytes, never written
// unless the data sum is one particular value.
int probe_lds_stream(const void *src, int n_tiles, int steps, uint32_t *sink, void *stream)
{
    if (!src || !sink || n_tiles <= 0 || steps <= 0)
        return -1;
    hipLaunchKernelGGL(probe_lds_stream_kernel, dim3(256), dim3(512), 0,
                       reinterpret_cast<hipStream_t>(stream),
                       static_cast<const unsigned char *>(src), n_tiles, steps, sink);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

} // extern "C"
