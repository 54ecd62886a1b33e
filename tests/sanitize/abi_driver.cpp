// Host-only driver for the address/undefined-behaviour sanitizer build of the
// library's host code (the C-ABI argument checks, workspace planning, the
// segment-table checker and the mixed-adapter batching helpers).  No call here
// reaches a kernel launch: every layer call fails validation first (the
// pointers are fake but aligned).  Exits non-zero on an unexpected status.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "lora_fused.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        const lora_status _s = (call);                                                  \
        if (_s != (want)) {                                                             \
            std::fprintf(stderr, "%s:%d: %s -> %d, want %d (%s)\n", __FILE__, __LINE__, \
                         #call, (int)_s, (int)(want), lora_last_error_message());       \
            ++failures;                                                                 \
        }                                                                               \
    } while (0)

int main() {
    void *F = (void *)(uintptr_t)0x10000;  // aligned, never dereferenced
    float *Ff = (float *)F;
    uint32_t *Fu = (uint32_t *)F;
    const lora_status OK = LORA_OK, INV = LORA_ERR_INVALID_ARG, UNS = LORA_ERR_UNSUPPORTED,
                      WS = LORA_ERR_WORKSPACE;
    for (int s = -5; s <= 1; ++s)
        if (lora_status_string((lora_status)s) == nullptr) ++failures;

    // workspace queries over many shapes, including degenerate ones
    const int64_t ms[] = {0, 1, 63, 64, 257, 8192, 1 << 20};
    const int64_t ks[] = {0, 8, 136, 4096, 28672};
    const int32_t rs[] = {0, 1, 8, 17, 33, 64, 128, 200, 256};
    for (int64_t m : ms)
        for (int64_t k : ks)
            for (int32_t r : rs) {
                (void)lora_linear_fwd_workspace_size(m, k, 4096, r);
                (void)lora_linear_bwd_workspace_size(m, k, 4096, r);
                (void)multi_lora_fwd_workspace_size(m, k, 4096, r, 8, 8);
                (void)multi_lora_bwd_workspace_size(m, k, 4096, r, 8, 8);
                (void)multi_lora_bwd_workspace_size(m, k, 4096, r, 0, 0);
            }

    // single-adapter layer calls: every invalid argument class
    EXPECT(lora_linear_fwd(F, F, F, F, 64, 60, 64, 8, 1.f, 0.1f, 0, 0, F, Ff, Fu, F, 1 << 30, nullptr), INV);
    EXPECT(lora_linear_fwd(F, F, F, F, 64, 64, 64, 0, 1.f, 0.1f, 0, 0, F, Ff, Fu, F, 1 << 30, nullptr), INV);
    EXPECT(lora_linear_fwd(F, F, F, F, 64, 64, 64, 257, 1.f, 0.1f, 0, 0, F, Ff, Fu, F, 1 << 30, nullptr), INV);
    EXPECT(lora_linear_fwd(F, F, F, F, 64, 64, 64, 8, 1.f, 1.0f, 0, 0, F, Ff, Fu, F, 1 << 30, nullptr), INV);
    EXPECT(lora_linear_fwd(F, F, F, F, 64, 64, 64, 8, 1.f, -0.5f, 0, 0, F, Ff, Fu, F, 1 << 30, nullptr), INV);
    EXPECT(lora_linear_fwd(F, F, F, F, 64, 64, 64, 8, 1.f, 0.1f, 0, 3, F, Ff, Fu, F, 1 << 30, nullptr), INV);
    EXPECT(lora_linear_fwd(F, F, F, F, 64, 64, 64, 8, 1.f, 0.1f, 0, 0, F, Ff, nullptr, F, 1 << 30, nullptr), INV);
    EXPECT(lora_linear_fwd(F, F, F, F, 64, 4096, 4096, 128, 1.f, 0.1f, 0, 0, F, Ff, Fu, F, 0, nullptr), WS);
    EXPECT(lora_linear_fwd(F, F, F, F, 64, 64, 1 << 22, 256, 1.f, 0.1f, 0, 0, F, Ff, Fu, F, 1 << 30, nullptr), UNS);
    EXPECT(lora_linear_fwd(nullptr, F, F, F, 0, 64, 64, 8, 1.f, 0.1f, 0, 0, nullptr, nullptr, nullptr, nullptr, 0,
                           nullptr), OK);
    EXPECT(lora_linear_bwd(F, F, F, F, F, Ff, Fu, 64, 64, 64, 8, 1.f, 0.1f, F, F, F, F, 0, nullptr), WS);
    EXPECT(lora_linear_bwd(F, F, F, F, F, Ff, Fu, 64, 64, 1 << 22, 256, 1.f, 0.1f, F, F, F, F, 1 << 30, nullptr),
           UNS);
    EXPECT(lora_linear_bwd(F, F, F, F, F, Ff, nullptr, 64, 64, 64, 8, 1.f, 0.1f, F, F, F, F, 1 << 30, nullptr),
           INV);
    EXPECT(lora_linear_bwd_noalloc(F, F, F, F, F, Ff, Fu, 8192, 4096, 4096, 256, 1.f, 0.1f, F, F, F, nullptr),
           UNS);
    EXPECT(lora_linear_fwd_concat(F, F, F, F, 64, 64, 64, 32, 1.f, F, Ff, nullptr), UNS);
    EXPECT(lora_linear_fwd_concat(F, F, (char *)F + 2, F, 64, 64, 64, 16, 1.f, F, Ff, nullptr), UNS);
    EXPECT(lora_dropout_mask(0, 3, 4, 64, 0.1f, Fu, nullptr), INV);
    EXPECT(lora_frozen_fwd(F, F, 64, 60, 64, F, nullptr), INV);
    EXPECT(lora_dora_norm(F, F, F, 64, 64, 0, 1.f, Ff, F, 1 << 30, nullptr), INV);

    // mixed-adapter calls and the host segment checker
    const lora_adapter *tab = (const lora_adapter *)F;
    const int64_t *so = (const int64_t *)F;
    const int32_t *sa = (const int32_t *)F;
    EXPECT(multi_lora_linear_fwd(F, F, tab, 0, so, sa, 1, 64, 64, 64, 16, 0, 0, F, Ff, Fu, F, 1 << 30, nullptr),
           INV);
    EXPECT(multi_lora_linear_bwd(F, F, F, tab, 2, so, sa, 2, Ff, Fu, 64, 64, 64, 300, F, F, 1 << 30, nullptr),
           INV);
    const int64_t off_ok[] = {0, 10, 10, 64};
    const int32_t ad_ok[] = {1, 0, 1};
    const int32_t ranks[] = {8, 16};
    EXPECT(multi_lora_check_segments(off_ok, ad_ok, 3, 64, ranks, 2, 16), OK);
    const int64_t off_bad[] = {0, 40, 30, 64};
    EXPECT(multi_lora_check_segments(off_bad, ad_ok, 3, 64, ranks, 2, 16), INV);
    const int32_t ad_bad[] = {1, 2, 0};
    EXPECT(multi_lora_check_segments(off_ok, ad_bad, 3, 64, ranks, 2, 16), INV);
    EXPECT(multi_lora_check_segments(off_ok, ad_ok, 3, 64, ranks, 2, 8), INV);

    // batching helpers on seeded random global batches
    std::mt19937 rng(7);
    for (int trial = 0; trial < 50; ++trial) {
        const int ns = 1 + (int)(rng() % 400), na = 1 + (int)(rng() % 6);
        const int64_t cap = 256 + (int64_t)(rng() % 4096);
        std::vector<int32_t> len(ns), ad(ns), batch(ns), mb(ns);
        for (int i = 0; i < ns; ++i) {
            len[i] = 1 + (int32_t)(rng() % cap);
            ad[i] = (int32_t)(rng() % na);
            batch[i] = (int32_t)(rng() % 3);
        }
        int32_t nmb = -1;
        EXPECT(lora_pack_greedy(len.data(), ns, cap, mb.data(), &nmb), OK);
        for (int32_t q = 0; q < nmb; ++q) {
            std::vector<int32_t> order(ns), seg_ad(na);
            std::vector<int64_t> seg_off(na + 1);
            int32_t nmem = 0, nseg = 0;
            EXPECT(lora_microbatch_segments(len.data(), ad.data(), mb.data(), ns, na, q, order.data(), &nmem,
                                            seg_off.data(), seg_ad.data(), &nseg), OK);
        }
        int64_t viol = -1;
        EXPECT(lora_check_bubble_lemma(mb.data(), ad.data(), batch.data(), ns, na, 1 + (int)(rng() % 4), &viol), OK);
    }
    const int32_t too_long[] = {5, 5000};
    int32_t mb2[2], n2 = 0;
    EXPECT(lora_pack_greedy(too_long, 2, 4096, mb2, &n2), INV);
    EXPECT(lora_pack_greedy(nullptr, 2, 4096, mb2, &n2), INV);

    if (failures) {
        std::fprintf(stderr, "%d unexpected statuses\n", failures);
        return 1;
    }
    std::printf("abi driver: all checks passed\n");
    return 0;
}
