/* The C oracle (oracle/topk_sort.c) under the address and undefined-behaviour
 * sanitizers (tests/test_sanitizers.py): random rows of both widths, with
 * strides and ties, one and four threads, each result checked by brute force
 * (k entries, distinct columns, and no unselected key above a selected one). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_topk(const void *x, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                void *out_vals, int32_t *out_idx, int nthreads);
uint32_t oracle_key(int dtype, uint32_t raw);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 16);
}

int main(void) {
    int failures = 0;
    for (int trial = 0; trial < 200; ++trial) {
        const int dtype = trial % 2;
        const int64_t batch = 1 + next_u32() % 4, n = 1 + next_u32() % 300, stride = n + next_u32() % 5;
        const int32_t k = 1 + (int32_t)(next_u32() % (uint32_t)n);
        const int es = dtype == 0 ? 4 : 2;
        unsigned char *x = malloc((size_t)(batch * stride) * es);
        void *vals = malloc((size_t)(batch * k) * es);
        int32_t *idx = malloc((size_t)(batch * k) * sizeof(int32_t));
        const uint32_t alphabet = trial % 3 == 0 ? 5 : 0;  /* heavy ties in a third of the trials */
        for (int64_t i = 0; i < batch * stride; ++i) {
            const uint32_t r = alphabet ? next_u32() % alphabet : next_u32();
            if (dtype == 0)
                ((uint32_t *)x)[i] = alphabet ? 0x3F800000u + (r << 20) : r;
            else
                ((uint16_t *)x)[i] = (uint16_t)(alphabet ? 0x3F80u + (r << 4) : r);
        }
        if (oracle_topk(x, dtype, batch, n, stride, k, vals, idx, 1 + trial % 4) != 0) ++failures;
        for (int64_t r = 0; r < batch; ++r) {
            char *sel = calloc((size_t)n, 1);
            uint32_t minsel = 0xFFFFFFFFu;
            for (int32_t j = 0; j < k; ++j) {
                const int32_t c = idx[r * k + j];
                if (c < 0 || c >= n || sel[c]) {
                    ++failures;
                    continue;
                }
                sel[c] = 1;
                const uint32_t raw = dtype == 0 ? ((uint32_t *)x)[r * stride + c] : ((uint16_t *)x)[r * stride + c];
                const uint32_t key = oracle_key(dtype, raw);
                if (key < minsel) minsel = key;
            }
            for (int64_t c = 0; c < n; ++c) {
                const uint32_t raw = dtype == 0 ? ((uint32_t *)x)[r * stride + c] : ((uint16_t *)x)[r * stride + c];
                if (!sel[c] && oracle_key(dtype, raw) > minsel) ++failures;
            }
            free(sel);
        }
        free(x);
        free(vals);
        free(idx);
    }
    /* rejected arguments */
    uint32_t one = 0;
    int32_t i1 = 0;
    if (oracle_topk(NULL, 0, 1, 1, 1, 1, &one, &i1, 1) != -1) ++failures;
    if (oracle_topk(&one, 0, 1, 1, 1, 2, &one, &i1, 1) != -1) ++failures;
    printf("oracle checks: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
