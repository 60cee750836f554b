// Drives the C ABI's host-side code under ASan/UBSan, without a GPU: status
// strings, every workspace-size query over ordinary and extreme shapes (the
// size arithmetic must neither overflow nor read out of bounds), and every
// entry point's argument checks with placeholder device pointers (each case
// returns before any device work).  Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "vwl.h"

static int failures = 0;
#define EXPECT(cond)                                                                                                   \
    do {                                                                                                               \
        if (!(cond)) {                                                                                                 \
            std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);                                             \
            ++failures;                                                                                                \
        }                                                                                                              \
    } while (0)

static void *P(uintptr_t off) { return reinterpret_cast<void *>(uintptr_t(1) << 40 | off); }

int main() {
    for (int s = -2; s <= 9; ++s)
        EXPECT(vwl_status_string(s) != nullptr);
    EXPECT(vwl_status_string(77) != nullptr);

    // size queries: ordinary, edge and absurd shapes
    const int Bs[] = {1, 2, 64, 256, 4096, 1 << 20, 0, -1};
    const int Ks[] = {0, 1, 2, 4, 63, 64, -1};
    const int Vs[] = {1, 2, 7, 1024, 151936, 1 << 21, (1 << 21) + 1, 0, -5, 1 << 30};
    for (int B : Bs)
        for (int K : Ks)
            for (int V : Vs)
                for (int dt = -1; dt <= 2; ++dt) {
                    const size_t a = vwl_asym_workspace_bytes(B, K, V, (vwl_dtype)dt);
                    const size_t r = vwl_rapid_workspace_bytes(B, K, V, (vwl_dtype)dt);
                    const size_t e = vwl_e2sci_workspace_bytes(B, K + 1, V, (vwl_dtype)dt);
                    const size_t x = vwl_asym_xfam_workspace_bytes(B, K, V, V > 1 ? V - 1 : V, (vwl_dtype)dt);
                    const bool ok = B >= 1 && K >= 0 && K <= VWL_MAX_K && V >= 1 && (dt == 0 || dt == 1);
                    if (!ok) {
                        EXPECT(a == 0);
                        EXPECT(e == 0);
                    }
                    (void)r;
                    (void)x;
                }
    for (int H : {0, 64, 100, 2560, 5120})
        (void)vwl_asym_lmhead_workspace_bytes(64, 2, 151936, H, 2 * H);

    // argument checks (every case returns before any device work)
    const size_t need = vwl_asym_workspace_bytes(2, 2, 100, VWL_F32);
    EXPECT(need > 0);
    EXPECT(vwl_asym_check(P(0), P(0x1000), P(0x2000), (const int32_t *)P(0x3000), 2, 2, 100, 0, 1.0f, 0.5f, P(0x4000),
                          P(0x5000), P(0x6000), P(0x7000), P(0x8000), P(0x9000), P(0xA000), need, need) == VWL_OK);
    EXPECT(vwl_asym_check(nullptr, P(0x1000), P(0x2000), (const int32_t *)P(0x3000), 2, 2, 100, 0, 1.0f, 0.5f,
                          P(0x4000), P(0x5000), P(0x6000), P(0x7000), P(0x8000), P(0x9000), P(0xA000), need,
                          need) == VWL_ERR_NULL);
    EXPECT(vwl_asym_check(P(0), P(0x1000), P(0x2000), (const int32_t *)P(0x3000), 2, 64, 100, 0, 1.0f, 0.5f, P(0x4000),
                          P(0x5000), P(0x6000), P(0x7000), P(0x8000), P(0x9000), P(0xA000), need, need) ==
           VWL_ERR_SHAPE);
    EXPECT(vwl_asym_check(P(4), P(0x1000), P(0x2000), (const int32_t *)P(0x3000), 2, 2, 100, 0, 1.0f, 0.5f, P(0x4000),
                          P(0x5000), P(0x6000), P(0x7000), P(0x8000), P(0x9000), P(0xA000), need, need) ==
           VWL_ERR_ALIGN);
    EXPECT(vwl_asym_check(P(0), P(0x1000), P(0x2000), (const int32_t *)P(0x3000), 2, 2, 100, 0, 1.0f / 0.0f, 0.5f,
                          P(0x4000), P(0x5000), P(0x6000), P(0x7000), P(0x8000), P(0x9000), P(0xA000), need,
                          need) == VWL_ERR_PARAM);
    const size_t rneed = vwl_rapid_workspace_bytes(2, 3, 100, VWL_F32);
    EXPECT(vwl_rapid_check(P(0), P(0x1000), (const int32_t *)P(0x2000), (const float *)P(0x3000),
                           (const float *)P(0x4000), 2, 3, 100, 0, 10.0f, 1.0f, P(0x5000), P(0x6000), P(0x7000),
                           P(0x8000), rneed, rneed) == VWL_OK);
    EXPECT(vwl_rapid_check(P(0), P(0x1000), (const int32_t *)P(0x2000), (const float *)P(0x3000),
                           (const float *)P(0x4000), 2, 3, 100, 0, 10.0f, 0.0f, P(0x5000), P(0x6000), P(0x7000),
                           P(0x8000), rneed, rneed) == VWL_ERR_PARAM);
    // full entry points: a missing workspace or a bad shape returns first
    float D, g;
    EXPECT(asym_verify(P(0), P(0x1000), P(0x2000), (const int32_t *)P(0x3000), 2, 2, 100, VWL_F32, 1.0f, 0.5f, &D, &g,
                       (uint8_t *)P(0x4000), (int32_t *)P(0x5000), (int32_t *)P(0x6000), (int32_t *)P(0x7000),
                       nullptr, nullptr, 0, nullptr) == VWL_ERR_WORKSPACE);
    EXPECT(asym_verify(P(0), P(0x1000), P(0x2000), (const int32_t *)P(0x3000), 0, 2, 100, VWL_F32, 1.0f, 0.5f, &D, &g,
                       (uint8_t *)P(0x4000), (int32_t *)P(0x5000), (int32_t *)P(0x6000), (int32_t *)P(0x7000),
                       nullptr, nullptr, 0, nullptr) == VWL_ERR_SHAPE);
    vwl_e2sci_params prm = {1.0f, 0.5f, 0.1f, 0.01f, 0.3f, 0.3f, 0.0f, 1, 0.0f, 0.0f};
    EXPECT(e2sci_verify(P(0), P(0x1000), 2, 4, 100, VWL_F32, (const float *)P(0x2000), (const float *)P(0x3000),
                        (float *)P(0x4000), nullptr, &prm, (float *)P(0x5000), (uint8_t *)P(0x6000),
                        (int32_t *)P(0x7000), (float *)P(0x8000), nullptr, nullptr, 0, nullptr) ==
           VWL_ERR_WORKSPACE);
    prm.min_refresh = 3;
    EXPECT(e2sci_verify(P(0), P(0x1000), 2, 4, 100, VWL_F32, (const float *)P(0x2000), (const float *)P(0x3000),
                        (float *)P(0x4000), nullptr, &prm, (float *)P(0x5000), (uint8_t *)P(0x6000),
                        (int32_t *)P(0x7000), (float *)P(0x8000), nullptr, nullptr, 0, nullptr) == VWL_ERR_NULL);
    EXPECT(vwl_set_plan_override(0, 3, 0) == VWL_ERR_PARAM);
    EXPECT(vwl_set_plan_override(0, 0, 0) == VWL_OK);
    EXPECT(vwl_set_xfam_override(2, 0) == VWL_ERR_PARAM);
    EXPECT(vwl_set_xfam_override(0, 0) == VWL_OK);
    if (failures)
        std::fprintf(stderr, "%d check(s) failed\n", failures);
    else
        std::printf("host harness: all checks passed\n");
    return failures ? 1 : 0;
}
