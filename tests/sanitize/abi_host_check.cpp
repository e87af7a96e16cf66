// abi_host_check.cpp -- the C ABI's host-side argument checks and kernel
// selection, built with the host compiler under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py).
//
// The kernel launches and the three HIP runtime calls the ABI layer makes
// are replaced here by stubs that record what they were given, so the
// checks run without a GPU and no kernel is ever launched: every entry point
// is called with valid, invalid and extreme arguments (sizes near 2^31 and
// 2^63, where an unchecked product would overflow), and the test asserts the
// status, that refused calls launch nothing, and which kernel family valid
// calls select.  Device pointers are fake addresses that nothing
// dereferences.
#include "dsa.h"
#include "dsa_internal.hpp"

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

// ---------------------------------------------------------------- stubs

namespace {
std::string g_launched;   // name of the last stubbed launch ("" = none)
dsa::TopkArgs g_topk{};
dsa::AttendArgs g_attend{};
dsa::IndexArgs g_index{};
char g_scratch_token;
} // namespace

extern "C" {
hipError_t hipGetDevice(int *dev)
{
    *dev = 0;
    return hipSuccess;
}
int hipGetStreamDeviceId(hipStream_t)
{
    return 0;
}
const char *hipGetErrorString(hipError_t)
{
    return "stubbed HIP error";
}
}

namespace dsa {
hipError_t launch_index_scores(const IndexArgs &a, hipStream_t)
{
    g_launched = "index";
    g_index = a;
    return hipSuccess;
}
hipError_t launch_topk(const TopkArgs &a, hipStream_t)
{
    g_launched = "topk";
    g_topk = a;
    return hipSuccess;
}
hipError_t topk_scratch(void **p)
{
    *p = &g_scratch_token;
    return hipSuccess;
}
hipError_t launch_attend_masked(const AttendArgs &a, hipStream_t)
{
    g_launched = "attend_masked";
    g_attend = a;
    return hipSuccess;
}
hipError_t launch_attend(const AttendArgs &a, hipStream_t)
{
    // the library's own launch_attend dispatches on the same predicates
    g_launched = attend_gather_supported(a)         ? "attend_gather"
                 : attend_heads_gather_supported(a) ? "attend_heads"
                 : attend_masked_supported(a)       ? "attend_masked"
                                                    : "attend_plain";
    g_attend = a;
    return hipSuccess;
}
hipError_t launch_hadamard_rotate(const void *, bool, void *, bool, int64_t, int, hipStream_t)
{
    g_launched = "rotate";
    return hipSuccess;
}
hipError_t launch_index_cache_write(const CacheWriteArgs &, hipStream_t)
{
    g_launched = "cache_write";
    return hipSuccess;
}
hipError_t launch_visibility_ranges(const RangeArgs &, hipStream_t)
{
    g_launched = "ranges";
    return hipSuccess;
}
hipError_t launch_pool_keys(const PoolKeysArgs &, hipStream_t)
{
    g_launched = "pool_keys";
    return hipSuccess;
}
hipError_t launch_pool_select(const PoolSelectArgs &, hipStream_t)
{
    g_launched = "pool_select";
    return hipSuccess;
}
hipError_t launch_indexer_frontend(const FrontendArgs &, hipStream_t)
{
    g_launched = "frontend";
    return hipSuccess;
}
hipError_t launch_expand_kv(const ExpandArgs &, hipStream_t)
{
    g_launched = "expand_kv";
    return hipSuccess;
}
} // namespace dsa

// ---------------------------------------------------------------- checks

namespace {
int g_failures = 0;
int g_checks = 0;

// a fake, 256-byte aligned device address (never dereferenced)
template <class T = void>
T *dev(uintptr_t slot)
{
    return reinterpret_cast<T *>((uintptr_t)0x7f0000000000ull + slot * 0x100000ull);
}

void expect(int got, int want, const char *want_launch, const char *what, int line)
{
    ++g_checks;
    const bool launch_ok =
        want_launch ? g_launched == want_launch : g_launched.empty();
    if (got != want || !launch_ok) {
        ++g_failures;
        std::fprintf(stderr, "FAIL line %d (%s): status %d (want %d), launched '%s' (want '%s'); %s\n",
                     line, what, got, want, g_launched.c_str(), want_launch ? want_launch : "",
                     dsa_last_error());
    }
    if (got != DSA_OK && std::strlen(dsa_last_error()) == 0) {
        ++g_failures;
        std::fprintf(stderr, "FAIL line %d (%s): error without a message\n", line, what);
    }
    g_launched.clear();
}
#define EXPECT(call, want, launch) \
    do {                           \
        g_launched.clear();        \
        const int rc_ = (call);    \
        expect(rc_, want, launch, #call, __LINE__); \
    } while (0)
#define CHECK(cond)                                                              \
    do {                                                                         \
        ++g_checks;                                                              \
        if (!(cond)) {                                                           \
            ++g_failures;                                                        \
            std::fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #cond);        \
        }                                                                        \
    } while (0)

void *const kStream = nullptr;
const int32_t *const kLo = dev<const int32_t>(1);
const int32_t *const kHi = dev<const int32_t>(2);

void ranges()
{
    EXPECT(dsa_visibility_ranges(-1, 1, kLo, kLo, 0, dev<int32_t>(3), dev<int32_t>(4), kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_visibility_ranges(INT32_MAX, INT32_MAX, kLo, kLo, 0, dev<int32_t>(3),
                                 dev<int32_t>(4), kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    EXPECT(dsa_visibility_ranges(0, 5, nullptr, nullptr, 0, nullptr, nullptr, kStream), DSA_OK,
           nullptr);
    EXPECT(dsa_visibility_ranges(2, 5, kLo, nullptr, 0, dev<int32_t>(3), dev<int32_t>(4),
                                 kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_visibility_ranges(2, 5, kLo, kHi, 4, dev<int32_t>(3), dev<int32_t>(4), kStream),
           DSA_OK, "ranges");
}

void index_scores()
{
    dsa_index_dims d{32, 1, 8192, 32, 128, 0.088f};
    const void *q = dev(10), *k = dev(11);
    const float *w = dev<const float>(12), *ks = dev<const float>(13);
    float *S = dev<float>(14);
    EXPECT(dsa_index_scores(nullptr, q, DSA_BF16, k, DSA_BF16, nullptr, w, kLo, kHi, S, kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_index_scores(&d, q, DSA_BF16, k, DSA_BF16, nullptr, w, kLo, kHi, S, kStream),
           DSA_OK, "index");
    CHECK(!g_index.f32 && !g_index.k_fp8 && g_index.n_k == 8192);
    EXPECT(dsa_index_scores(&d, q, DSA_BF16, k, DSA_FP8_E4M3, ks, w, kLo, kHi, S, kStream),
           DSA_OK, "index");
    CHECK(g_index.k_fp8 && g_index.k_scale == ks);
    EXPECT(dsa_index_scores(&d, q, DSA_BF16, k, DSA_FP8_E4M3, nullptr, w, kLo, kHi, S, kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_index_scores(&d, q, DSA_BF16, k, DSA_BF16, ks, w, kLo, kHi, S, kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_index_scores(&d, q, DSA_F32, k, DSA_F32, ks, w, kLo, kHi, S, kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_index_scores(&d, q, DSA_F32, k, DSA_BF16, nullptr, w, kLo, kHi, S, kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_index_scores(&d, q, DSA_BF16, k, DSA_BF16, nullptr, w, kLo, kHi, nullptr, kStream),
           DSA_ERR_ARG, nullptr);
    dsa_index_dims f{1, 64, 64, 4, 32, 0.17f};
    EXPECT(dsa_index_scores(&f, q, DSA_F32, k, DSA_F32, nullptr, w, kLo, kHi, S, kStream), DSA_OK,
           "index");
    CHECK(g_index.f32);
    dsa_index_dims odd{1, 64, 64, 4, 32, 0.17f};   // bf16 needs 32/64 heads of 64/128
    EXPECT(dsa_index_scores(&odd, q, DSA_BF16, k, DSA_BF16, nullptr, w, kLo, kHi, S, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_index_dims big{INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, 1.f};
    EXPECT(dsa_index_scores(&big, q, DSA_BF16, k, DSA_BF16, nullptr, w, kLo, kHi, S, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_index_dims keys{1, 1, 1 << 30, 32, 1 << 20, 1.f};   // only the key tensor is too large
    EXPECT(dsa_index_scores(&keys, q, DSA_BF16, k, DSA_BF16, nullptr, w, kLo, kHi, S, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_index_dims neg{1, -1, 5, 32, 128, 1.f};
    EXPECT(dsa_index_scores(&neg, q, DSA_BF16, k, DSA_BF16, nullptr, w, kLo, kHi, S, kStream),
           DSA_ERR_ARG, nullptr);
    dsa_index_dims empty{4, 0, 100, 32, 128, 1.f};
    EXPECT(dsa_index_scores(&empty, nullptr, DSA_BF16, nullptr, DSA_BF16, nullptr, nullptr,
                            nullptr, nullptr, nullptr, kStream),
           DSA_OK, nullptr);
}

void topk()
{
    const float *S = dev<const float>(20);
    int32_t *out = dev<int32_t>(21);
    void *ws = dev(22);
    CHECK(dsa_topk_workspace_size(32, 8192, 2048) == 0);
    // rows of 131072 keys (threshold path): per row a 64-byte header, 32
    // blocks x 24 pairs of (8-byte key, 4-byte count) and 16384 candidates,
    // each part starting on a 256-byte boundary
    const size_t need = dsa_topk_workspace_size(8, 131072, 2048);
    CHECK(need == (size_t)8 * (9472 + 131072));
    CHECK(9472 == ((64 + 32 * 24 * 12) + 255) / 256 * 256);
    // rows of 300000 keys (chunked path): 19 chunks of 2048 winners
    CHECK(dsa_topk_workspace_size(2, 300000, 2048) == (size_t)2 * 19 * 2048 * 8);
    CHECK(dsa_topk_workspace_size(8, 131072, 4096) == 0);
    CHECK(dsa_topk_workspace_size(INT32_MAX, INT32_MAX, 2048) ==
          (size_t)INT32_MAX * 131072 * 2048 * 8);
    CHECK(dsa_topk_workspace_size(INT32_MAX, INT32_MAX, INT32_MAX) == 0);
    CHECK(dsa_topk_workspace_size(-3, 100000, 16) == 0);
    EXPECT(dsa_topk(S, 32, 8192, 8192, kLo, kHi, 2048, 0, out, nullptr, 0, kStream), DSA_OK, "topk");
    CHECK(g_topk.workspace == nullptr && g_topk.k == 2048);
    EXPECT(dsa_topk(S, 8, 131072, 131072, kLo, kHi, 2048, 0, out, ws, need - 1, kStream),
           DSA_ERR_WORKSPACE, nullptr);
    EXPECT(dsa_topk(S, 8, 131072, 131072, kLo, kHi, 2048, 0, out, nullptr, need, kStream),
           DSA_ERR_WORKSPACE, nullptr);
    EXPECT(dsa_topk(S, 8, 131072, 131072, kLo, kHi, 2048, 0, out, ws, need, kStream), DSA_OK,
           "topk");
    CHECK(g_topk.workspace == ws);
    EXPECT(dsa_topk(S, 8, 100, 99, kLo, kHi, 16, 0, out, nullptr, 0, kStream), DSA_ERR_ARG, nullptr);
    EXPECT(dsa_topk(S, 8, 100, 100, kLo, kHi, 0, 0, out, nullptr, 0, kStream), DSA_ERR_ARG, nullptr);
    EXPECT(dsa_topk(S, 8, 100, 100, kLo, kHi, 2049, 0, out, nullptr, 0, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    EXPECT(dsa_topk(S, 0, 100, 100, kLo, kHi, 16, 0, out, nullptr, 0, kStream), DSA_OK, nullptr);
    EXPECT(dsa_topk(S, 8, 100, 100, nullptr, kHi, 16, 0, out, nullptr, 0, kStream), DSA_ERR_ARG,
           nullptr);
    EXPECT(dsa_topk(S, INT32_MAX, 100, INT64_MAX, kLo, kHi, 16, 0, out, nullptr, 0, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    EXPECT(dsa_topk(S, 8, -1, 100, kLo, kHi, 16, 0, out, nullptr, 0, kStream), DSA_ERR_ARG, nullptr);
    // attention sinks: passed through; a negative count is refused
    EXPECT(dsa_topk(S, 32, 8192, 8192, kLo, kHi, 2048, 3, out, nullptr, 0, kStream), DSA_OK,
           "topk");
    CHECK(g_topk.n_sink == 3 && g_topk.k == 2048);
    EXPECT(dsa_topk(S, 32, 8192, 8192, kLo, kHi, 2048, -1, out, nullptr, 0, kStream), DSA_ERR_ARG,
           nullptr);
    EXPECT(dsa_topk_noalloc(S, 8, 131072, 131072, kLo, kHi, 2048, 1, out, kStream), DSA_OK,
           "topk");
    CHECK(g_topk.n_sink == 1);
    // the allocation-free variant: the scratch array in place of a workspace
    EXPECT(dsa_topk_noalloc(S, 8, 131072, 131072, kLo, kHi, 2048, 0, out, kStream), DSA_OK, "topk");
    CHECK(g_topk.workspace == &g_scratch_token);
    EXPECT(dsa_topk_noalloc(S, 32, 8192, 8192, kLo, kHi, 2048, 0, out, kStream), DSA_OK, "topk");
    CHECK(g_topk.workspace == nullptr);
    // 16 MiB of scratch: 1024 rows of 32768 keys at k = 2048 need 32 MiB
    EXPECT(dsa_topk_noalloc(S, 1024, 32768, 32768, kLo, kHi, 2048, 0, out, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    EXPECT(dsa_topk_noalloc(S, 8, 100, 100, kLo, kHi, 4096, 0, out, kStream), DSA_ERR_UNSUPPORTED,
           nullptr);
}

void attend()
{
    const void *q = dev(30), *kv = dev(31), *v = dev(32);
    const int32_t *idx = dev<const int32_t>(33);
    float *out = dev<float>(34), *lse = dev<float>(35);
    void *ws = dev(36);
    // decode, absorbed: 32 rows, 2048 selected -> split-K partials
    dsa_attn_dims dec{32, 1, 8192, 64, 576, 512, 1, 2048, 0.04f};
    const size_t need = dsa_sparse_attend_workspace_size(&dec);
    CHECK(need > 0);
    EXPECT(dsa_sparse_attend(&dec, DSA_BF16, q, kv, 576, kv, 576, idx, kLo, kHi, out, lse, ws,
                             need, kStream),
           DSA_OK, "attend_gather");
    EXPECT(dsa_sparse_attend(&dec, DSA_BF16, q, kv, 576, kv, 576, idx, kLo, kHi, out, lse, ws,
                             need - 1, kStream),
           DSA_ERR_WORKSPACE, nullptr);
    EXPECT(dsa_sparse_attend(&dec, DSA_BF16, q, kv, 576, kv, 576, idx, kLo, nullptr, out, lse, ws,
                             need, kStream),
           DSA_ERR_ARG, nullptr);
    // misaligned operand of an MFMA kernel
    EXPECT(dsa_sparse_attend(&dec, DSA_BF16, (const char *)q + 2, kv, 576, kv, 576, idx, kLo, kHi,
                             out, lse, ws, need, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    // no rows: the size query must not divide by the row count
    dsa_attn_dims none{0, 1, 8192, 64, 576, 512, 1, 2048, 0.04f};
    CHECK(dsa_sparse_attend_workspace_size(&none) == 0);
    dsa_attn_dims none_q{4, 0, 8192, 64, 576, 512, 1, 2048, 0.04f};
    CHECK(dsa_sparse_attend_workspace_size(&none_q) == 0);
    EXPECT(dsa_sparse_attend(&none_q, DSA_BF16, nullptr, nullptr, 576, nullptr, 576, nullptr,
                             nullptr, nullptr, nullptr, nullptr, nullptr, 0, kStream),
           DSA_OK, nullptr);
    // pooled per-head: masked-tile kernel
    dsa_attn_dims ph{4, 16384, 16384, 64, 192, 256, 64, 2052, 0.072f};
    const size_t need_ph = dsa_sparse_attend_workspace_size(&ph);
    CHECK(need_ph >= (size_t)4 * 16384 * 64 * 256 * 2);
    EXPECT(dsa_sparse_attend(&ph, DSA_BF16, q, kv, 64 * 192, v, 64 * 256, idx, kLo, kHi, out,
                             lse, ws, need_ph, kStream),
           DSA_OK, "attend_masked");
    // pooled decode (one query per sequence): the per-head gather, no workspace
    dsa_attn_dims pd{4, 1, 16384, 64, 192, 256, 64, 2052, 0.072f};
    CHECK(dsa_sparse_attend_workspace_size(&pd) == 0);
    EXPECT(dsa_sparse_attend(&pd, DSA_BF16, q, kv, 64 * 192, v, 64 * 256, idx, kLo, kHi, out,
                             lse, nullptr, 0, kStream),
           DSA_OK, "attend_heads");
    dsa_attn_dims pd_big{4, 1, 16384, 64, 192, 256, 64, 4097, 0.072f};   // beyond its set size
    CHECK(dsa_sparse_attend_workspace_size(&pd_big) > 0);
    // f32 per-head: the plain kernel, no workspace
    dsa_attn_dims tiny{1, 64, 64, 4, 48, 32, 4, 8, 0.14f};
    CHECK(dsa_sparse_attend_workspace_size(&tiny) == 0);
    EXPECT(dsa_sparse_attend(&tiny, DSA_F32, q, kv, 4 * 48, v, 4 * 32, idx, kLo, kHi, out, lse,
                             nullptr, 0, kStream),
           DSA_OK, "attend_plain");
    dsa_attn_dims gqa{1, 64, 64, 4, 48, 32, 3, 8, 0.14f};
    EXPECT(dsa_sparse_attend(&gqa, DSA_F32, q, kv, 3 * 48, v, 3 * 32, idx, kLo, kHi, out, lse,
                             nullptr, 0, kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_sparse_attend(&tiny, DSA_F32, q, kv, 4 * 48 - 1, v, 4 * 32, idx, kLo, kHi, out, lse,
                             nullptr, 0, kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_sparse_attend(&tiny, DSA_FP8_E4M3, q, kv, 4 * 48, v, 4 * 32, idx, kLo, kHi, out,
                             lse, nullptr, 0, kStream),
           DSA_ERR_ARG, nullptr);
    dsa_attn_dims wide{1, 64, 64, 4, 48, 2048, 4, 8, 0.14f};
    EXPECT(dsa_sparse_attend(&wide, DSA_F32, q, kv, 4 * 48, v, 4 * 2048, idx, kLo, kHi, out, lse,
                             nullptr, 0, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    // extreme sizes: refused, and the size query neither overflows nor traps
    dsa_attn_dims big{INT32_MAX, INT32_MAX, 524288, INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX,
                      INT32_MAX, 1.f};
    (void)dsa_sparse_attend_workspace_size(&big);
    EXPECT(dsa_sparse_attend(&big, DSA_BF16, q, kv, INT64_MAX, v, INT64_MAX, idx, kLo, kHi, out,
                             lse, ws, SIZE_MAX, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_attn_dims big_ph{INT32_MAX, INT32_MAX, 524288, 64, 192, 256, 64, 2052, 1.f};
    (void)dsa_sparse_attend_workspace_size(&big_ph);
    dsa_attn_dims rows_ok{1, 1024, 524288, 64, 192, 256, 64, 2052, 1.f};
    EXPECT(dsa_sparse_attend(&rows_ok, DSA_BF16, q, kv, INT64_MAX / 2, v, 64 * 256, idx, kLo, kHi,
                             out, lse, ws, SIZE_MAX, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_attn_dims too_long{1, 1, 524289, 64, 576, 512, 1, 2048, 1.f};
    EXPECT(dsa_sparse_attend(&too_long, DSA_BF16, q, kv, 576, kv, 576, idx, kLo, kHi, out, lse, ws,
                             need, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    EXPECT(dsa_sparse_attend(nullptr, DSA_BF16, q, kv, 576, kv, 576, idx, kLo, kHi, out, lse, ws,
                             need, kStream),
           DSA_ERR_ARG, nullptr);
}

void cache_write()
{
    const void *x = dev(40);
    void *y = dev(41);
    const int32_t *head = dev<const int32_t>(42);
    float *sc = dev<float>(43);
    EXPECT(dsa_hadamard_rotate(256, 128, x, DSA_BF16, y, DSA_BF16, kStream), DSA_OK, "rotate");
    EXPECT(dsa_hadamard_rotate(256, 96, x, DSA_BF16, y, DSA_BF16, kStream), DSA_ERR_UNSUPPORTED,
           nullptr);
    EXPECT(dsa_hadamard_rotate(-1, 128, x, DSA_BF16, y, DSA_BF16, kStream), DSA_ERR_ARG, nullptr);
    EXPECT(dsa_hadamard_rotate(INT64_MAX, 256, x, DSA_BF16, y, DSA_BF16, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    EXPECT(dsa_hadamard_rotate(4, 128, x, DSA_FP8_E4M3, y, DSA_BF16, kStream), DSA_ERR_ARG,
           nullptr);
    EXPECT(dsa_hadamard_rotate(0, 128, nullptr, DSA_BF16, nullptr, DSA_BF16, kStream), DSA_OK,
           nullptr);
    dsa_cache_dims d{8, 1, 131072, 128};
    EXPECT(dsa_index_cache_write(&d, x, DSA_BF16, head, y, DSA_FP8_E4M3, sc, kStream), DSA_OK,
           "cache_write");
    EXPECT(dsa_index_cache_write(&d, x, DSA_BF16, head, y, DSA_FP8_E4M3, nullptr, kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_index_cache_write(&d, x, DSA_BF16, head, y, DSA_BF16, sc, kStream), DSA_ERR_ARG,
           nullptr);
    EXPECT(dsa_index_cache_write(&d, x, DSA_FP8_E4M3, head, y, DSA_BF16, nullptr, kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_index_cache_write(&d, x, DSA_BF16, nullptr, y, DSA_BF16, nullptr, kStream),
           DSA_ERR_ARG, nullptr);
    dsa_cache_dims big{INT32_MAX, INT32_MAX, INT32_MAX, 256};
    EXPECT(dsa_index_cache_write(&big, x, DSA_BF16, head, y, DSA_BF16, nullptr, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_cache_dims odd{8, 1, 100, 48};
    EXPECT(dsa_index_cache_write(&odd, x, DSA_BF16, head, y, DSA_BF16, nullptr, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_cache_dims empty{8, 0, 100, 64};
    EXPECT(dsa_index_cache_write(&empty, nullptr, DSA_BF16, nullptr, nullptr, DSA_BF16, nullptr,
                                 kStream),
           DSA_OK, nullptr);
    EXPECT(dsa_index_cache_write(nullptr, x, DSA_BF16, head, y, DSA_BF16, nullptr, kStream),
           DSA_ERR_ARG, nullptr);
}

void pools()
{
    const void *k = dev(50), *g = dev(51);
    void *pooled = dev(52);
    int32_t *np = dev<int32_t>(53), *tok = dev<int32_t>(54);
    const int32_t *pad = dev<const int32_t>(55), *qpos = dev<const int32_t>(56);
    const float *S = dev<const float>(57);
    dsa_pool_dims d{4, 16384, 16384, 4, 128, 512, 2052};
    EXPECT(dsa_pool_keys(&d, DSA_BF16, k, g, pad, pooled, np, kStream), DSA_OK, "pool_keys");
    EXPECT(dsa_pool_keys(&d, DSA_FP8_E4M3, k, g, pad, pooled, np, kStream), DSA_ERR_ARG, nullptr);
    EXPECT(dsa_pool_keys(&d, DSA_BF16, k, nullptr, pad, pooled, np, kStream), DSA_ERR_ARG,
           nullptr);
    dsa_pool_dims zero_kpool{4, 16384, 16384, 0, 128, 512, 2052};
    EXPECT(dsa_pool_keys(&zero_kpool, DSA_BF16, k, g, pad, pooled, np, kStream), DSA_ERR_ARG,
           nullptr);
    dsa_pool_dims big{INT32_MAX, INT32_MAX, INT32_MAX, 1, INT32_MAX, 2048, INT32_MAX};
    EXPECT(dsa_pool_keys(&big, DSA_BF16, k, g, pad, pooled, np, kStream), DSA_ERR_UNSUPPORTED,
           nullptr);
    EXPECT(dsa_pool_select(&big, S, pad, qpos, tok, nullptr, nullptr, 0, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    CHECK(dsa_pool_select_workspace_size(&d) == 0);
    EXPECT(dsa_pool_select(&d, S, pad, qpos, tok, nullptr, nullptr, 0, kStream), DSA_OK,
           "pool_select");
    dsa_pool_dims narrow{4, 16384, 16384, 4, 128, 512, 2050};
    EXPECT(dsa_pool_select(&narrow, S, pad, qpos, tok, nullptr, nullptr, 0, kStream), DSA_ERR_ARG,
           nullptr);
    dsa_pool_dims many{1, 4 * 16385, 1, 4, 128, 512, 2052};
    EXPECT(dsa_pool_select(&many, S, pad, qpos, tok, nullptr, nullptr, 0, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_pool_dims sel0{4, 16384, 16384, 4, 128, 0, 2052};
    EXPECT(dsa_pool_select(&sel0, S, pad, qpos, tok, nullptr, nullptr, 0, kStream), DSA_ERR_ARG,
           nullptr);
    EXPECT(dsa_pool_select(&d, S, pad, nullptr, tok, nullptr, nullptr, 0, kStream), DSA_ERR_ARG,
           nullptr);
    dsa_pool_dims no_rows{4, 16384, 0, 4, 128, 512, 2052};
    EXPECT(dsa_pool_select(&no_rows, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                           kStream),
           DSA_OK, nullptr);
}
} // namespace

void index_share()
{
    // the pages' enumeration: full layers 0, 1, 2, then every 4th up to 74
    int n_full = 0, last_full = -1;
    for (int il = 0; il < 78; ++il) {
        const bool full = il <= 2 || (il >= 6 && (il - 2) % 4 == 0);
        if (full) {
            ++n_full;
            last_full = il;
        }
        CHECK(dsa_index_share_source(il) == last_full);
    }
    CHECK(n_full == 21);
    CHECK(dsa_index_share_source(-1) == -1);
    CHECK(dsa_index_share_source(INT32_MIN) == -1);
    CHECK(dsa_index_share_source(INT32_MAX) == INT32_MAX - (INT32_MAX - 2) % 4);
}

void projections()
{
    const void *ql = dev(60), *x = dev(61), *wq = dev(62), *wk = dev(63), *wp = dev(64);
    const int32_t *pos = dev<const int32_t>(65);
    const float *g = dev<const float>(66), *b = dev<const float>(67);
    void *qo = dev(68), *ko = dev(69);
    float *wo = dev<float>(70);
    dsa_frontend_dims d{4096, 2048, 6144, 32, 128, 64, 10000.f, 1e-6f};
    EXPECT(dsa_indexer_frontend(&d, ql, x, pos, wq, wk, g, b, wp, qo, ko, wo, kStream), DSA_OK,
           "frontend");
    dsa_frontend_dims e0 = d;
    e0.norm_eps = 0.f;  // the pages' CPU crash: LayerNorm with eps 0
    EXPECT(dsa_indexer_frontend(&e0, ql, x, pos, wq, wk, g, b, wp, qo, ko, wo, kStream),
           DSA_ERR_ARG, nullptr);
    dsa_frontend_dims hd = d;
    hd.head_dim = 64;
    EXPECT(dsa_indexer_frontend(&hd, ql, x, pos, wq, wk, g, b, wp, qo, ko, wo, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_frontend_dims rd = d;
    rd.rope_dim = 40;
    EXPECT(dsa_indexer_frontend(&rd, ql, x, pos, wq, wk, g, b, wp, qo, ko, wo, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_frontend_dims big{INT32_MAX, 1 << 30, 1 << 30, 32, 128, 64, 10000.f, 1e-6f};
    EXPECT(dsa_indexer_frontend(&big, ql, x, pos, wq, wk, g, b, wp, qo, ko, wo, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    EXPECT(dsa_indexer_frontend(&d, ql, x, nullptr, wq, wk, g, b, wp, qo, ko, wo, kStream),
           DSA_ERR_ARG, nullptr);
    EXPECT(dsa_indexer_frontend(&d, (const char *)ql + 8, x, pos, wq, wk, g, b, wp, qo, ko, wo,
                                kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_expand_dims xd{65536, 512, 64, 192, 256};
    EXPECT(dsa_expand_kv(&xd, x, wq, ko, 64 * 192, qo, 64 * 256, kStream), DSA_OK, "expand_kv");
    EXPECT(dsa_expand_kv(&xd, x, wq, ko, 64 * 192 - 8, qo, 64 * 256, kStream), DSA_ERR_ARG,
           nullptr);
    EXPECT(dsa_expand_kv(&xd, x, wq, ko, 64 * 192 + 4, qo, 64 * 256, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_expand_dims xbig{INT32_MAX, 512, INT32_MAX, INT32_MAX, 8};
    EXPECT(dsa_expand_kv(&xbig, x, wq, ko, INT64_MAX, qo, INT64_MAX, kStream),
           DSA_ERR_UNSUPPORTED, nullptr);
    dsa_expand_dims xr{16, 100, 4, 8, 8};
    EXPECT(dsa_expand_kv(&xr, x, wq, ko, 32, qo, 32, kStream), DSA_ERR_UNSUPPORTED, nullptr);
    dsa_expand_dims x0{0, 512, 64, 192, 256};
    EXPECT(dsa_expand_kv(&x0, nullptr, nullptr, nullptr, 64 * 192, nullptr, 64 * 256, kStream),
           DSA_OK, nullptr);
}

int main()
{
    projections();
    CHECK(std::strlen(dsa_version()) > 0);
    index_share();
    ranges();
    index_scores();
    topk();
    attend();
    cache_write();
    pools();
    std::printf("%d checks, %d failures\n", g_checks, g_failures);
    return g_failures == 0 ? 0 : 1;
}
