// host_driver.cpp -- runs the host side of the C ABI (argument validation,
// the varlen planner, the split arithmetic) under AddressSanitizer and
// UndefinedBehaviorSanitizer, on the CPU.  The kernel launchers are stubs
// that must never be reached: without a GPU every valid call stops at the
// device check.  Test infrastructure, built and run by
// tests/test_host_sanitizers.py.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "attn_fwd.h"
#include "attn_params.h"

namespace attn {
hipError_t launch_fwd(const FwdParams&, int, int, bool, bool, bool, hipStream_t) { abort(); }
hipError_t launch_bwd(const BwdParams&, int, int, bool, bool, hipStream_t) { abort(); }
hipError_t launch_merge(const float*, const float*, uint16_t*, float*, int, long long, int,
                        hipStream_t) {
    abort();
}
hipError_t launch_decode(const DecParams&, int, int, bool, hipStream_t) { abort(); }
hipError_t bwd_scratch_rows(float**) { abort(); }
}  // namespace attn

static int failures = 0;
static void expect(bool ok, const char* what, int line) {
    if (!ok) {
        fprintf(stderr, "host_driver.cpp:%d: %s\n", line, what);
        ++failures;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// deterministic pseudo-random lengths (a fixed linear congruential sequence)
static uint32_t lcg(uint32_t& s) {
    s = s * 1664525u + 1013904223u;
    return s >> 8;
}

int main() {
    // the planner on many length mixes, with empty sequences and Lq != Lk
    uint32_t s = 12345;
    for (int trial = 0; trial < 200; ++trial) {
        const int n_seq = 1 + (int)(lcg(s) % 12);
        std::vector<int> cq(n_seq + 1, 0), ck(n_seq + 1, 0);
        for (int i = 0; i < n_seq; ++i) {
            cq[i + 1] = cq[i] + (int)(lcg(s) % 700) * ((lcg(s) % 5) != 0);
            ck[i + 1] = ck[i] + (int)(lcg(s) % 700) * ((lcg(s) % 7) != 0);
        }
        const int G = 1 << (lcg(s) % 4), Hkv = 1 + (int)(lcg(s) % 4), causal = (int)(lcg(s) & 1);
        int n = -1;
        EXPECT(attn_varlen_plan(cq.data(), ck.data(), n_seq, G * Hkv, Hkv, causal, nullptr, 0,
                                &n) == ATTN_OK);
        EXPECT(n >= 0 && n % 8 == 0);
        std::vector<int> plan((size_t)n * ATTN_VARLEN_RECORD_INTS + 1, -7);
        int m = -1;
        EXPECT(attn_varlen_plan(cq.data(), ck.data(), n_seq, G * Hkv, Hkv, causal, plan.data(), n,
                                &m) == ATTN_OK);
        EXPECT(m == n);
        EXPECT(plan[(size_t)n * ATTN_VARLEN_RECORD_INTS] == -7);  // nothing written past the end
        for (int r = 0; r < n; ++r) {
            const int* rec = &plan[(size_t)r * ATTN_VARLEN_RECORD_INTS];
            if (rec[1] == 0) continue;  // padding
            EXPECT(rec[0] >= 0 && rec[0] + rec[1] <= cq[n_seq]);
            EXPECT(rec[2] >= 0 && rec[2] + rec[3] <= ck[n_seq]);
        }
        if (n > 0)
            EXPECT(attn_varlen_plan(cq.data(), ck.data(), n_seq, G * Hkv, Hkv, causal, plan.data(),
                                    n - 1, &m) == ATTN_ERR_BAD_ARGUMENT);
    }
    int n = 0;
    const int bad[3] = {0, 5, 4};
    EXPECT(attn_varlen_plan(bad, bad, 2, 2, 1, 0, nullptr, 0, &n) == ATTN_ERR_BAD_SHAPE);

    // split widths
    for (int lk = 1; lk < 3000; lk += 37)
        for (int ns = 1; ns < 70; ns += 7) {
            const int w = attn_split_keys(lk, ns);
            EXPECT(w > 0 && w % 64 == 0 && (long long)w * ns >= lk);
        }
    EXPECT(attn_split_keys(0, 4) < 0 && attn_split_keys(100, 0) < 0);

    // every entry point: bad arguments first, valid ones stop at the device check
    char* base = static_cast<char*>(aligned_alloc(256, 1 << 12));
    void *q = base, *k = base + 256, *v = base + 512, *o = base + 768;
    float* lse = reinterpret_cast<float*>(base + 1024);
    const int no_dev[2] = {ATTN_ERR_NO_DEVICE, ATTN_ERR_UNSUPPORTED_ARCH};
    auto is_no_dev = [&](int rc) { return rc == no_dev[0] || rc == no_dev[1]; };
    EXPECT(attn_fwd(nullptr, k, v, o, lse, 1, 2, 1, 64, 64, 128, 128, 0, 0.1f, nullptr) ==
           ATTN_ERR_NULL_PTR);
    EXPECT(attn_fwd(q, k, v, o, lse, 1, 3, 2, 64, 64, 128, 128, 0, 0.1f, nullptr) ==
           ATTN_ERR_GQA_RATIO);
    EXPECT(is_no_dev(attn_fwd(q, k, v, o, lse, 2, 8, 2, 300, 500, 128, 128, 1, 0.1f, nullptr)));
    EXPECT(is_no_dev(attn_fwd(q, k, v, o, lse, 1, 16, 16, 32768, 32768, 192, 128, 1, 0.07f,
                              nullptr)));
    // the allocation-free backward: its row limit is checked before any device call
    EXPECT(attn_bwd_noalloc(q, k, v, o, o, lse, o, o, o, 1, 64, 64, 65537, 64, 128, 128, 0, 0.1f,
                            nullptr) == ATTN_ERR_SCRATCH);
    EXPECT(is_no_dev(attn_bwd_noalloc(q, k, v, o, o, lse, o, o, o, 1, 64, 64, 65536, 64, 128,
                                      128, 0, 0.1f, nullptr)));
    EXPECT(attn_bwd_noalloc(q, k, v, o, o, nullptr, o, o, o, 1, 2, 2, 64, 64, 128, 128, 0, 0.1f,
                            nullptr) == ATTN_ERR_NULL_PTR);
    // the backward of every head shape and element type validates, then stops at the device
    EXPECT(is_no_dev(attn_bwd(q, k, v, o, o, lse, o, o, o, lse, 1, 16, 16, 2048, 2048, 192, 128,
                              1, 0.07f, nullptr)));
    EXPECT(is_no_dev(attn_bwd_ex(q, k, v, o, o, lse, o, o, o, lse, 1, 8, 2, 300, 200, 64, 64, 1,
                                 0, 0.125f, nullptr)));
    EXPECT(attn_bwd_ex(q, k, v, o, o, lse, o, o, o, lse, 1, 8, 2, 300, 200, 64, 64, 2, 0, 0.125f,
                       nullptr) == ATTN_ERR_BAD_ARGUMENT);
    EXPECT(attn_bwd(q, k, v, o, o, lse, o, o, o, lse, 1, 8, 2, 300, 200, 192, 192, 0, 0.1f,
                    nullptr) == ATTN_ERR_UNSUPPORTED_HEAD_DIM);
    EXPECT(attn_bwd(q, k, v, o, o, lse, o, o, o, lse, 1, 1, 1, 6000000, 64, 192, 128, 0, 0.1f,
                    nullptr) == ATTN_ERR_TOO_LARGE);
    unsigned long long cnt = 0;
    EXPECT(is_no_dev(attn_fwd_dbg(q, k, v, o, lse, 1, 1, 1, 256, 256, 64, 64, 0, 0.125f, nullptr,
                                  0.0f, 0, &cnt)));
    EXPECT(attn_fwd_dbg(q, k, v, o, lse, 1, 1, 1, 256, 256, 64, 64, 0, 0.125f, nullptr, 0.0f, 1,
                        &cnt) == ATTN_ERR_BAD_ARGUMENT);
    attn_strides sq = {3LL * 100 * 4 * 128, 128, 3 * 4 * 128}, so = {100LL * 4 * 128, 128, 512};
    EXPECT(is_no_dev(attn_fwd_ex(q, k, v, o, lse, 1, 4, 4, 100, 100, 128, 128, sq, sq, sq, so, 1,
                                 0, 0.1f, nullptr)));
    float* op = reinterpret_cast<float*>(base + 2048);
    EXPECT(is_no_dev(attn_fwd_split(q, k, v, op, lse, 2, 8, 2, 1, 4096, 128, 128, 0, 0.1f, 4,
                                    nullptr)));
    EXPECT(is_no_dev(attn_fwd_split(q, k, v, op, lse, 2, 8, 2, 200, 4096, 128, 128, 1, 0.1f, 4,
                                    nullptr)));
    EXPECT(attn_fwd_decode(q, k, v, op, lse, 2, 8, 2, 5, 4096, 128, 128, 0, 0.1f, 4, nullptr) ==
           ATTN_ERR_BAD_ARGUMENT);
    EXPECT(is_no_dev(attn_merge(op, lse, o, lse, 4, 64, 128, nullptr)));
    EXPECT(is_no_dev(attn_bwd(q, k, v, o, o, lse, q, k, v, lse, 1, 4, 2, 100, 100, 64, 64, 1,
                              0.1f, nullptr)));
    const int* plan_dev = reinterpret_cast<const int*>(base + 3072);
    EXPECT(is_no_dev(attn_fwd_varlen(q, k, v, o, lse, plan_dev, 8, 100, 100, 4, 4, 128, 128, 1,
                                     0.1f, nullptr)));
    EXPECT(attn_fwd_varlen(q, k, v, o, lse, nullptr, 8, 100, 100, 4, 4, 128, 128, 1, 0.1f,
                           nullptr) == ATTN_ERR_NULL_PTR);
    for (int st = -1; st < 14; ++st) EXPECT(attn_status_string(st) != nullptr);
    free(base);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("host driver: all checks passed\n");
    return 0;
}
