// Host-side driver for the sanitizer test (tests/test_host_sanitizers.py):
// calls every entry point of include/slim.h with arguments the boundary must
// reject (NULL or misaligned pointers, bad and extreme shapes, negative
// strides, overlapping outputs) and every size query with extreme values,
// and checks the status or size each returns.  Built with host-only
// AddressSanitizer and UndefinedBehaviorSanitizer over the library's C++
// code; it makes no device call that could reach a kernel (every call here
// is rejected before one), so it runs without a GPU.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "slim.h"

static int g_fail = 0;

#define EXPECT_STATUS(expr, want)                                                                  \
    do {                                                                                         \
        const slim_status got_ = (expr);                                                         \
        if (got_ != (want)) {                                                                    \
            fprintf(stderr, "FAIL %s:%d: %s -> %d (%s), want %d\n", __FILE__, __LINE__, #expr, (int)got_, \
                    slim_last_error(), (int)(want));                                             \
            ++g_fail;                                                                            \
        } else if (got_ != SLIM_OK && strlen(slim_last_error()) == 0) {                          \
            fprintf(stderr, "FAIL %s:%d: %s: no error message\n", __FILE__, __LINE__, #expr);    \
            ++g_fail;                                                                            \
        }                                                                                        \
    } while (0)

#define EXPECT_SIZE(expr, want)                                                                    \
    do {                                                                                         \
        const size_t got_ = (expr);                                                              \
        if (got_ != (size_t)(want)) {                                                            \
            fprintf(stderr, "FAIL %s:%d: %s -> %zu, want %zu\n", __FILE__, __LINE__, #expr, got_, (size_t)(want)); \
            ++g_fail;                                                                            \
        }                                                                                        \
    } while (0)

int main() {
    // 16-byte aligned host buffers stand in for device pointers: every call
    // below is rejected before anything dereferences or launches them.
    alignas(16) static unsigned char buf[1 << 12];
    void* P = buf;
    void* Q = buf + 1;                                   // misaligned
    const int64_t BIG = INT64_MAX, HUGE40 = (int64_t)1 << 40, NEG = -1;
    const slim_status INVAL = SLIM_EINVAL, UNSUP = SLIM_EUNSUPPORTED;
    const uint16_t* X = (const uint16_t*)P;
    const uint8_t* V = (const uint8_t*)P;
    const uint16_t* S = (const uint16_t*)P;
    uint16_t* Y = (uint16_t*)P;

    // Status strings and the version.
    for (int s = -1; s < 8; ++s)
        if (!slim_status_string(s)) { fprintf(stderr, "FAIL status string %d\n", s); ++g_fail; }
    if (slim_version() != 1) { fprintf(stderr, "FAIL version\n"); ++g_fail; }

    // Size queries: documented values, and 0 for shapes no call accepts.
    EXPECT_SIZE(slim_values_bytes(4096, 4096), 4096 * 4096 / 4);
    EXPECT_SIZE(slim_meta_bytes(4096, 11008), 4096 * 11008 / 8);
    EXPECT_SIZE(slim_scales_bytes(11008, 4096, 128), 11008 * 32 * 2);
    EXPECT_SIZE(slim_values_bytes(NEG, 128), 0);
    EXPECT_SIZE(slim_values_bytes(16, 100), 0);
    EXPECT_SIZE(slim_values_bytes(BIG, BIG - 127), 0);
    EXPECT_SIZE(slim_meta_bytes(HUGE40, HUGE40), 0);
    EXPECT_SIZE(slim_scales_bytes(BIG, 128, 128), 0);
    EXPECT_SIZE(slim_scales_bytes(16, 128, 64), 0);
    EXPECT_SIZE(slim_adapter_codes_bytes(BIG, BIG - 7), 0);
    EXPECT_SIZE(slim_adapter_scales_bytes(BIG, 128, 128), 0);
    EXPECT_SIZE(slim_transposed_values_bytes(BIG - 15, BIG - 127), 0);
    EXPECT_SIZE(slim_transposed_meta_bytes(HUGE40, HUGE40), 0);
    EXPECT_SIZE(slim_linear_workspace_bytes(BIG, 4096, 4096, 416), 0);
    EXPECT_SIZE(slim_linear_workspace_bytes(16, BIG, 4096, 416), 0);
    EXPECT_SIZE(slim_linear_workspace_bytes(16, 4096, BIG, 416), 0);
    EXPECT_SIZE(slim_linear_workspace_bytes(16, 4096, 4096, BIG), 0);
    EXPECT_SIZE(slim_linear_workspace_bytes(16, 4096, 4096, 33), 0);
    EXPECT_SIZE(slim_linear_qa_workspace_bytes(HUGE40, HUGE40, HUGE40, 416), 0);
    EXPECT_SIZE(slim_linear_a8_workspace_bytes(HUGE40, 16, 128, 32), 0);
    if (slim_linear_workspace_bytes(2048, 4096, 11008, 416) == 0) { fprintf(stderr, "FAIL ws size\n"); ++g_fail; }

    // slim_pack
    EXPECT_STATUS(slim_pack((const float*)P, 16, 128, 64, (uint8_t*)P, (uint8_t*)P, (uint16_t*)P, 0), UNSUP);
    EXPECT_STATUS(slim_pack(nullptr, 16, 128, 128, (uint8_t*)P, (uint8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_pack((const float*)Q, 16, 128, 128, (uint8_t*)P, (uint8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_pack((const float*)P, 0, 128, 128, (uint8_t*)P, (uint8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_pack((const float*)P, 16, 100, 128, (uint8_t*)P, (uint8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_pack((const float*)P, BIG, BIG - 127, 128, (uint8_t*)P, (uint8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_pack((const float*)P, HUGE40, HUGE40, 128, (uint8_t*)P, (uint8_t*)P, (uint16_t*)P, 0), INVAL);

    // slim_linear / slim_linear_noalloc / slim_linear_batched
    EXPECT_STATUS(slim_linear(X, 16, 512, 512, V, V, S, 64, X, X, 32, Y, P, 1 << 30, 0), UNSUP);
    EXPECT_STATUS(slim_linear(X, NEG, 512, 512, V, V, S, 128, X, X, 32, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear(X, 16, 100, 512, V, V, S, 128, X, X, 32, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear(X, 16, 512, 500, V, V, S, 128, X, X, 32, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear(X, 16, 512, 512, V, V, S, 128, X, X, 33, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear(X, BIG, BIG - 15, BIG - 127, V, V, S, 128, X, X, 32, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear(X, 16, 512, 512, V, V, S, 128, X, X, BIG - 31, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear(nullptr, 16, 512, 512, V, V, S, 128, X, X, 32, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear(X, 16, 512, 512, V, V, S, 128, nullptr, X, 32, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear((const uint16_t*)Q, 16, 512, 512, V, V, S, 128, X, X, 32, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear(X, 16, 512, 512, V, V, S, 128, X, X, 32, Y, nullptr, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear(X, 16, 512, 512, V, V, S, 128, X, X, 32, Y, P, 16, 0), INVAL);
    EXPECT_STATUS(slim_linear(X, 0, 512, 512, nullptr, nullptr, nullptr, 128, nullptr, nullptr, 32, nullptr,
                              nullptr, 0, 0), SLIM_OK);      // M == 0: nothing to do
    EXPECT_STATUS(slim_linear_noalloc(X, 16, 512, 512, V, V, S, 128, X, X, 33, Y, 0), INVAL);
    EXPECT_STATUS(slim_linear_noalloc(X, 1 << 20, 1 << 14, 4096, V, V, S, 128, X, X, 416, Y, 0), INVAL);
    EXPECT_STATUS(slim_linear_batched(NEG, 16, 512, 512, 32, 128, X, 0, V, 0, V, 0, S, 0, X, 0, X, 0, Y, 0, P,
                                      1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear_batched(1 << 20, 16, 512, 512, 32, 128, X, 0, V, 0, V, 0, S, 0, X, 0, X, 0, Y, 0, P,
                                      1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear_batched(2, 16, 512, 512, 32, 128, X, NEG, V, 0, V, 0, S, 0, X, 0, X, 0, Y, 8192, P,
                                      1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear_batched(2, 16, 512, 512, 32, 128, X, 3, V, 0, V, 0, S, 0, X, 0, X, 0, Y, 8192, P,
                                      1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear_batched(2, 16, 512, 512, 32, 128, X, 0, V, 0, V, 0, S, 0, X, 0, X, 0, Y, 100, P,
                                      1 << 30, 0), INVAL);       // outputs overlap
    EXPECT_STATUS(slim_linear_batched(2, 16, 512, 512, 32, 128, X, 0, V, 0, V, 0, S, 0, X, 0, X, 0, Y, BIG, P,
                                      1 << 30, 0), INVAL);       // problem offsets past the address space
    EXPECT_STATUS(slim_linear_batched(0, 16, 512, 512, 32, 128, nullptr, 0, nullptr, 0, nullptr, 0, nullptr, 0,
                                      nullptr, 0, nullptr, 0, nullptr, 0, nullptr, 0, 0), SLIM_OK);

    // Quantised adapters
    EXPECT_STATUS(slim_pack_adapter((const float*)P, 16, 128, 64, (uint8_t*)P, (uint16_t*)P, 0), UNSUP);
    EXPECT_STATUS(slim_pack_adapter(nullptr, 16, 128, 128, (uint8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_pack_adapter((const float*)P, 16, 100, 32, (uint8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_pack_adapter((const float*)P, BIG, BIG - 127, 128, (uint8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_linear_qa(X, 16, 512, 512, V, V, S, 128, V, S, V, S, 0, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear_qa(X, 16, 512, 512, V, V, S, 128, nullptr, S, V, S, 32, Y, P, 1 << 30, 0), INVAL);
    EXPECT_STATUS(slim_linear_qa(X, 16, 512, 512, V, V, S, 128, V, S, V, S, 32, Y, P, 16, 0), INVAL);

    // 8-bit input
    EXPECT_STATUS(slim_quantize_input(nullptr, 16, 512, (int8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_quantize_input(X, NEG, 512, (int8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_quantize_input(X, BIG, BIG, (int8_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_linear_a8((const int8_t*)P, nullptr, 16, 512, 512, V, V, S, 128, X, X, 32, Y, P, 1 << 30, 0),
                  INVAL);
    EXPECT_STATUS(slim_linear_a8((const int8_t*)P, S, 16, 512, 512, V, V, S, 128, X, X, 32, Y, P, 16, 0), INVAL);

    // Hybrid tiles
    EXPECT_STATUS(slim_pack_hybrid((const float*)P, 16, 128, 128, nullptr, (uint8_t*)P, (uint8_t*)P,
                                   (uint16_t*)P, (uint8_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_pack_hybrid((const float*)P, BIG, BIG - 127, 128, (const int32_t*)P, (uint8_t*)P,
                                   (uint8_t*)P, (uint16_t*)P, (uint8_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_linear_hybrid(X, 16, 512, 512, V, V, S, nullptr, (const int32_t*)P, 128, X, X, 32, Y, P,
                                     1 << 30, 0), INVAL);

    // Double-pruned transpose
    EXPECT_STATUS(slim_pack_transposed(V, V, S, 16, 128, 64, (uint16_t*)P, (uint16_t*)P, 0), UNSUP);
    EXPECT_STATUS(slim_pack_transposed(V, V, S, 15, 128, 128, (uint16_t*)P, (uint16_t*)P, 0), INVAL);
    EXPECT_STATUS(slim_pack_transposed(V, V, S, BIG - 15, BIG - 127, 128, (uint16_t*)P, (uint16_t*)P, 0), INVAL);

    // Give-up count and wait limit
    uint64_t count = 0;
    EXPECT_STATUS(slim_linear_giveups(nullptr, 0, &count, 0), INVAL);
    EXPECT_STATUS(slim_linear_giveups(P, 0, nullptr, 0), INVAL);
    EXPECT_STATUS(slim_linear_giveups(Q, 0, &count, 0), INVAL);
    const int64_t old = slim_set_wait_limit(BIG);
    slim_set_wait_limit(NEG);
    slim_set_wait_limit(old);

    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("abi sanitize driver: all checks passed\n");
    return 0;
}
