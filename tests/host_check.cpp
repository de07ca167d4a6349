// Host-side checks of libdeepselect's C ABI, for a build with the address and
// undefined-behaviour sanitizers on the host code (tests/test_sanitizers.py).
// Only entry points that return before touching a GPU are called: argument
// validation, the split planner, layout sizes, status strings, and
// deepselect_topk(_ex) calls rejected by their argument checks. Exits 0 when
// every expectation holds (the sanitizers abort the process on a finding).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "deepselect.h"

static int failures = 0;
#define EXPECT(c)                                                  \
    do {                                                           \
        if (!(c)) {                                                \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                            \
        }                                                          \
    } while (0)

int main() {
    const int64_t ns[] = {1, 2, 7, 1000, 4096, 131072, 1048576, ((int64_t)1 << 31) - 1, (int64_t)1 << 31,
                          INT64_MAX};
    const int32_t ks[] = {1, 2, 64, 512, 2048, 65536, INT32_MAX};
    const int32_t bs[] = {1, 3, 256, 1024, 2048, 4096, 1 << 20, INT32_MAX};
    const int64_t batches[] = {0, 1, 64, 128, 1 << 20, INT64_MAX};
    int checked = 0;
    for (int dtype = -1; dtype <= 2; ++dtype)
        for (int64_t n : ns)
            for (int32_t k : ks)
                for (int32_t b : bs)
                    for (int64_t batch : batches) {
                        const int v = deepselect_validate(dtype, batch, n, n, k, b, b);
                        EXPECT(v <= 0);
                        if (dtype != DS_F32 && dtype != DS_BF16) EXPECT(v == DS_ERR_DTYPE);
                        if ((dtype == DS_F32 || dtype == DS_BF16) && batch >= 0 && n < ((int64_t)1 << 31) && k > n)
                            EXPECT(v == DS_ERR_K);
                        for (int32_t cus : {1, 64, 256, 4096}) {
                            const int s = deepselect_plan_split(dtype, batch, n, k, b, b, cus);
                            if (v == DS_OK && batch > 0) EXPECT(s >= 1 || s == DS_ERR_UNSUPPORTED);
                            if (s >= 1) {
                                EXPECT(s <= 1024);
                                (void)deepselect_workspace_bytes(dtype, batch, n, k, b, b, s);
                                EXPECT(deepselect_lds_bytes(dtype, n, k, b, b, s) <= ((size_t)1 << 32));
                            }
                        }
                        for (int32_t split : {0, 1, 2, 64, 1024, INT32_MAX})
                            (void)deepselect_workspace_bytes(dtype, batch, n, k, b, b, split);
                        ++checked;
                    }
    // status strings: every code has a static, non-empty description
    for (int st = -20; st <= 5; ++st) {
        const char* m = deepselect_status_string(st);
        EXPECT(m != nullptr && strlen(m) > 0);
    }
    // calls rejected before any HIP call
    float dummy[16];
    int32_t idx[16];
    EXPECT(deepselect_topk(nullptr, DS_F32, 1, 16, 16, 4, 8, 8, 0, dummy, idx, nullptr) == DS_ERR_NULL);
    EXPECT(deepselect_topk(dummy, 9, 1, 16, 16, 4, 8, 8, 0, dummy, idx, nullptr) == DS_ERR_DTYPE);
    EXPECT(deepselect_topk(dummy, DS_F32, 1, 16, 16, 17, 8, 8, 0, dummy, idx, nullptr) == DS_ERR_K);
    EXPECT(deepselect_topk(dummy, DS_F32, 1, 16, 15, 4, 8, 8, 0, dummy, idx, nullptr) == DS_ERR_SHAPE);
    EXPECT(deepselect_topk(dummy, DS_F32, 0, 16, 16, 4, 8, 8, 0, nullptr, nullptr, nullptr) == DS_OK);
    ds_options_t opt;
    memset(&opt, 0, sizeof(opt));
    opt.waves = 5;
    EXPECT(deepselect_topk_ex(dummy, DS_F32, 1, 16, 16, 4, 8, 8, 0, dummy, idx, nullptr, &opt) == DS_ERR_BLOCK);
    opt.waves = 0;
    opt.kernel = 9;
    EXPECT(deepselect_topk_ex(dummy, DS_F32, 1, 16, 16, 4, 8, 8, 0, dummy, idx, nullptr, &opt) == DS_ERR_BLOCK);
    opt.kernel = 0;
    opt.sorted = 2;
    EXPECT(deepselect_topk_ex(dummy, DS_F32, 1, 16, 16, 4, 8, 8, 0, dummy, idx, nullptr, &opt) == DS_ERR_BLOCK);
    opt.sorted = 0;
    opt.workspace = dummy;
    EXPECT(deepselect_topk_noalloc(dummy, DS_F32, 1, 16, 16, 4, 8, 8, 0, dummy, idx, nullptr, &opt) ==
           DS_ERR_SCRATCH);
    EXPECT(deepselect_scratch_bytes() >= ((size_t)1 << 20));
    printf("host checks: %d shapes, %d failures\n", checked, failures);
    return failures == 0 ? 0 : 1;
}
