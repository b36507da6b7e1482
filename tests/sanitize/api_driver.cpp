// api_driver.cpp -- drives every entry point of the C ABI (include/gdn.h) through its
// host-side validation, built together with gdn_api.cpp and stub_launchers.cpp under
// AddressSanitizer and UndefinedBehaviorSanitizer on a CPU.  Host memory stands in for
// device memory: the validation layer only looks at pointer values, sizes and (in the debug
// check) cu_seqlens and the workspace status word, which the stubs copy with memcpy.
// Exits non-zero on the first unexpected status.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gdn.h"

extern int g_launches;

static int failures = 0;

#define EXPECT(expr, want)                                                                     \
    do {                                                                                       \
        const int got_ = (expr);                                                               \
        if (got_ != (want)) {                                                                  \
            std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #expr,  \
                         got_, (int)(want));                                                   \
            ++failures;                                                                        \
        }                                                                                      \
    } while (0)

int main() {
    // 1 GiB of address space in 16 MiB slots; nothing is read except where noted
    const size_t slot = (size_t)16 << 20;
    std::vector<char> mem(64 * slot + 4096);
    char *base = mem.data() + (256 - ((uintptr_t)mem.data() & 255));
    auto P = [&](int i, size_t off = 0) { return (void *)(base + (size_t)i * slot + off); };

    for (int s = -1; s <= 10; ++s) EXPECT(gdn_status_string(s) != nullptr, 1);
    EXPECT(gdn_abi_version(), GDN_ABI_VERSION);

    // ---- conv prep
    const int T = 200, Hk = 2, Hv = 4, d = 64, C = 2 * Hk * d + Hv * d;
    g_launches = 0;
    EXPECT(gdn_conv_qk_prep(P(0), P(1), nullptr, 1, nullptr, nullptr, (float *)P(2), (float *)P(3), (float *)P(4),
                            T, Hk, Hv, d, d, GDN_BF16, 1e-6f, nullptr), GDN_OK);
    EXPECT(g_launches, 1);
    EXPECT(gdn_conv_qk_prep(nullptr, P(1), nullptr, 1, nullptr, nullptr, (float *)P(2), (float *)P(3),
                            (float *)P(4), T, Hk, Hv, d, d, GDN_BF16, 1e-6f, nullptr), GDN_ERR_NULL_POINTER);
    EXPECT(gdn_conv_qk_prep(P(0, 2), P(1), nullptr, 1, nullptr, nullptr, (float *)P(2), (float *)P(3),
                            (float *)P(4), T, Hk, Hv, d, d, GDN_BF16, 1e-6f, nullptr), GDN_ERR_ALIGN);
    EXPECT(gdn_conv_qk_prep(P(0), P(1), nullptr, 1, nullptr, nullptr, (float *)P(0, 256), (float *)P(3),
                            (float *)P(4), T, Hk, Hv, d, d, GDN_BF16, 1e-6f, nullptr), GDN_ERR_ALIAS);
    EXPECT(gdn_conv_qk_prep(P(0), P(1), nullptr, 1, nullptr, nullptr, (float *)P(2), (float *)P(3), (float *)P(4),
                            INT_MAX, Hk, Hv, d, d, GDN_BF16, 1e-6f, nullptr), GDN_ERR_ALIAS);   // spans overlap
    EXPECT(gdn_conv_qk_prep(P(0), P(1), nullptr, 1, nullptr, nullptr, (float *)P(2), (float *)P(3), (float *)P(4),
                            -1, Hk, Hv, d, d, GDN_BF16, 1e-6f, nullptr), GDN_ERR_BAD_SHAPE);

    // ---- chunked prefill: MFMA, fp32 token recurrence, fp32 chunked form
    const size_t need = gdn_chunk_prefill_workspace_size(T, 1, Hk, Hv, d, d, GDN_MATH_MFMA);
    EXPECT(need > 0, 1);
    EXPECT((int)gdn_chunk_prefill_workspace_size(T, 1, Hk, Hv, d, d, GDN_MATH_F32_CHUNKED), 0);
    for (int math : {GDN_MATH_MFMA, GDN_MATH_F32, GDN_MATH_F32_CHUNKED}) {
        g_launches = 0;
        EXPECT(gdn_chunk_prefill((float *)P(2), (float *)P(3), (float *)P(4), (float *)P(5), (float *)P(6), nullptr,
                                 1, nullptr, (float *)P(7), (float *)P(8), 0.5f, T, Hk, Hv, d, d, math, 0, P(20),
                                 need, nullptr), GDN_OK);
        EXPECT(g_launches, 1);
    }
    EXPECT(gdn_chunk_prefill((float *)P(2), (float *)P(3), (float *)P(4), (float *)P(5), (float *)P(6), nullptr, 1,
                             nullptr, (float *)P(7), (float *)P(8), 0.5f, T, Hk, Hv, d, d, GDN_MATH_MFMA, 0, P(20),
                             need - 1, nullptr), GDN_ERR_WORKSPACE);
    EXPECT(gdn_chunk_prefill((float *)P(2), (float *)P(3), (float *)P(4), (float *)P(5), (float *)P(6), nullptr, 1,
                             nullptr, (float *)P(7), (float *)P(8), 0.5f, T, Hk, Hv, 128, 128, GDN_MATH_F32_CHUNKED,
                             0, nullptr, 0, nullptr), GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_chunk_prefill((float *)P(2), (float *)P(3), (float *)P(4), (float *)P(5), (float *)P(6), nullptr, 1,
                             nullptr, (float *)P(7), (float *)P(8), 0.5f, T, Hk, Hv, d, d, 7, 0, P(20), need,
                             nullptr), GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_chunk_prefill_local((float *)P(2), (float *)P(3), (float *)P(4), (float *)P(5), (float *)P(6),
                                   nullptr, 1, 1.f, T, Hk, Hv, d, d, 0, P(20), need, nullptr), GDN_OK);
    EXPECT(gdn_chunk_prefill_state(nullptr, 1, nullptr, (float *)P(7), (float *)P(8), T, Hk, Hv, d, d, P(20), need,
                                   nullptr), GDN_OK);

    // ---- fused prefill with cu_seqlens (read only by the debug check)
    int32_t *cu = (int32_t *)P(30);
    cu[0] = 0; cu[1] = 80; cu[2] = 80; cu[3] = T;
    const size_t need3 = gdn_chunk_prefill_workspace_size(T, 3, Hk, Hv, d, d, GDN_MATH_MFMA);
    EXPECT(gdn_prefill(P(0), P(1), cu, 3, P(9), P(9), (float *)P(5), (float *)P(6), (float *)P(10), (float *)P(10),
                       (float *)P(8), 1.f, 1e-6f, T, Hk, Hv, d, d, GDN_BF16, 1, P(20), need3, nullptr), GDN_OK);
    EXPECT(gdn_prefill(P(0), P(1), cu, 3, P(9), P(9, 16), (float *)P(5), (float *)P(6), nullptr, nullptr,
                       (float *)P(8), 1.f, 1e-6f, T, Hk, Hv, d, d, GDN_BF16, 0, P(20), need3, nullptr),
           GDN_ERR_ALIAS);
    EXPECT(gdn_prefill_local(P(0), P(1), cu, 3, nullptr, nullptr, (float *)P(5), (float *)P(6), 1.f, 1e-6f, T, Hk,
                             Hv, d, d, GDN_F32, 0, P(20), need3, nullptr), GDN_OK);
    // with GDN_DEBUG_CHECK set, a decreasing cu_seqlens is refused before any launch
    const char *dbg = std::getenv("GDN_DEBUG_CHECK");
    if (dbg && std::strcmp(dbg, "0") != 0) {
        cu[1] = 120; cu[2] = 90;
        g_launches = 0;
        EXPECT(gdn_prefill(P(0), P(1), cu, 3, nullptr, nullptr, (float *)P(5), (float *)P(6), nullptr, nullptr,
                           (float *)P(8), 1.f, 1e-6f, T, Hk, Hv, d, d, GDN_BF16, 0, P(20), need3, nullptr),
               GDN_ERR_BAD_SHAPE);
        EXPECT(gdn_chunk_prefill((float *)P(2), (float *)P(3), (float *)P(4), (float *)P(5), (float *)P(6), cu, 3,
                                 nullptr, nullptr, (float *)P(8), 1.f, T, Hk, Hv, d, d, GDN_MATH_F32, 0, nullptr, 0,
                                 nullptr), GDN_ERR_BAD_SHAPE);
        cu[3] = T + 1;
        cu[1] = 80; cu[2] = 80;
        EXPECT(gdn_chunk_prefill((float *)P(2), (float *)P(3), (float *)P(4), (float *)P(5), (float *)P(6), cu, 3,
                                 nullptr, nullptr, (float *)P(8), 1.f, T, Hk, Hv, d, d, GDN_MATH_F32, 0, nullptr, 0,
                                 nullptr), GDN_ERR_BAD_SHAPE);   // cu[N] != T
        EXPECT(g_launches, 0);
        cu[3] = T;
        // a clear status word after the (stubbed) kernels: the call returns GDN_OK
        EXPECT(gdn_prefill(P(0), P(1), cu, 3, nullptr, nullptr, (float *)P(5), (float *)P(6), nullptr, nullptr,
                           (float *)P(8), 1.f, 1e-6f, T, Hk, Hv, d, d, GDN_BF16, 0, P(20), need3, nullptr), GDN_OK);
        std::printf("debug checks exercised\n");
    }

    // ---- the workspace status word (the stub reads host memory)
    unsigned long long *hdr = (unsigned long long *)P(20);
    *hdr = 0;
    EXPECT(gdn_prefill_workspace_status(P(20), need, nullptr), GDN_OK);
    *hdr = (0x67646e73ull << 32) | GDN_ERR_NONFINITE;
    EXPECT(gdn_prefill_workspace_status(P(20), need, nullptr), GDN_ERR_NONFINITE);
    EXPECT(gdn_prefill_workspace_status(P(20), need, nullptr), GDN_OK);   // cleared by the read
    *hdr = 0x1234567812345678ull;                                           // a word no kernel wrote
    EXPECT(gdn_prefill_workspace_status(P(20), need, nullptr), GDN_OK);
    EXPECT(gdn_prefill_workspace_status(P(20), 8, nullptr), GDN_ERR_WORKSPACE);
    EXPECT(gdn_prefill_workspace_status(nullptr, need, nullptr), GDN_ERR_NULL_POINTER);

    // ---- decode, gated decode, gated RMSNorm
    const int B = 7;
    EXPECT(gdn_decode_step(P(0), P(1), P(9), (float *)P(5), (float *)P(6), (float *)P(10), (float *)P(8), 1.f, 1e-6f,
                           B, Hk, Hv, d, d, GDN_BF16, 0, nullptr), GDN_OK);
    EXPECT(gdn_decode_step(P(0), P(1), P(9), (float *)P(5), (float *)P(6), (float *)P(9, 64), (float *)P(8), 1.f,
                           1e-6f, B, Hk, Hv, d, d, GDN_BF16, 0, nullptr), GDN_ERR_ALIAS);
    EXPECT(gdn_decode_step_gated(P(0), P(1), P(9), (float *)P(5), (float *)P(6), (float *)P(10), P(11), P(12), P(13),
                                 1.f, 1e-6f, 1e-6f, B, Hk, Hv, d, d, GDN_BF16, 1, nullptr), GDN_OK);
    EXPECT(gdn_gated_rmsnorm((float *)P(8), P(11), P(12), P(13), 1000, d, 1e-6f, GDN_BF16, nullptr), GDN_OK);
    EXPECT(gdn_gated_rmsnorm((float *)P(8), P(11), P(12), P(13), LONG_MAX / 8, d, 1e-6f, GDN_BF16, nullptr),
           GDN_ERR_BAD_SHAPE);   // a row count whose byte sizes would not fit 64 bits
    EXPECT(gdn_decode_step(P(0), P(1), P(9), (float *)P(5), (float *)P(6), (float *)P(10), (float *)P(8), 1.f, 1e-6f,
                           B, 1 << 20, 1 << 20, d, d, GDN_BF16, 0, nullptr), GDN_ERR_BAD_SHAPE);   // too many heads
    EXPECT(gdn_gated_rmsnorm((float *)P(8), P(11), P(12), P(13), 10, 48, 1e-6f, GDN_BF16, nullptr),
           GDN_ERR_UNSUPPORTED);

    // ---- projections and the layer
    const int E = 256;
    EXPECT(gdn_linear(P(0), P(1), P(2), 100, 260, 192, nullptr), GDN_OK);
    EXPECT(gdn_linear(P(0), P(1), P(2), 100, 260, 100, nullptr), GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_in_proj(P(0), P(1), P(2), P(3), (float *)P(4), (float *)P(5), T, E, Hk, Hv, d, d, nullptr), GDN_OK);
    const size_t lws = gdn_layer_prefill_workspace_size(T, 3, Hk, Hv, d, d);
    EXPECT(lws > 0, 1);
    EXPECT(gdn_layer_prefill(P(0), P(1), P(2), P(3), P(4), cu, 3, P(5), P(5), (float *)P(6), (float *)P(6), P(7),
                             1.f, 1e-6f, 1e-6f, T, E, Hk, Hv, d, d, 0, P(40), lws, nullptr), GDN_OK);
    EXPECT(gdn_layer_prefill(P(0), P(1), P(2), P(3), P(4), cu, 3, P(5), P(5), (float *)P(6), (float *)P(6), P(7),
                             1.f, 1e-6f, 1e-6f, T, E, Hk, Hv, d, d, 0, P(40), lws - 1, nullptr), GDN_ERR_WORKSPACE);
    const size_t dws = gdn_layer_decode_workspace_size(B, E, Hk, Hv, d, d);
    EXPECT(gdn_layer_decode(P(0), P(1), P(2), P(3), P(4), P(5), (float *)P(6), P(7), 1.f, 1e-6f, 1e-6f, B, E, Hk, Hv,
                            d, d, 0, P(40), dws, nullptr), GDN_OK);
    EXPECT((int)gdn_layer_decode_workspace_size(-1, E, Hk, Hv, d, d), 0);
    EXPECT((int)gdn_layer_prefill_workspace_size(T, 3, 2, 3, d, d), 0);   // Hv % Hk != 0

    if (failures) {
        std::fprintf(stderr, "%d unexpected statuses\n", failures);
        return 1;
    }
    std::printf("api driver ok\n");
    return 0;
}
