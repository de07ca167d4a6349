/*
 * TEST INFRASTRUCTURE ONLY. Plain, slow, obviously correct CPU oracle for
 * batched row-wise top-k. Only tests, the smoke check and the benchmark's CPU
 * baseline may load it; the GPU library never does, and the two share no code.
 *
 * What it computes (the plain definition of the result):
 *   "CUDA 算子笔记 4" (milkfeng.top), section "Top K Selection": the k largest
 *   values of an array. The DeepSelect deep-dive (PFCCLab/DeepSelect,
 *   section "算法") returns the same set: DeepSelect is exact, it only drops
 *   elements that cannot enter the top-k.
 *
 * Value order: the order-preserving unsigned key of "CUDA 算子笔记 4",
 * section "改造 Radix Sort" (float_to_key): flip every bit of a pattern whose
 * sign bit is set, else flip only the sign bit. The same rule is applied to
 * 16-bit bfloat16 patterns. Under this key -0 < +0, a positive NaN lies above
 * +inf and a negative NaN below -inf; on every other pair it is float order.
 *
 * Result per row: sort all positions i by (key descending, index ascending)
 * and keep the first k. Implementation: pack ((KEYMAX - key) << 32) | i into a
 * 64-bit integer, sort ascending with qsort, unpack. out_vals receives the raw
 * bit pattern of x[i] and out_idx the column i.
 */
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

static uint32_t key32(uint32_t u) { return (u & 0x80000000u) ? ~u : (u | 0x80000000u); }

static uint32_t key16(uint32_t u) {
    u &= 0xFFFFu;
    return (u & 0x8000u) ? (~u & 0xFFFFu) : (u | 0x8000u);
}

static int cmp_u64(const void *a, const void *b) {
    uint64_t x = *(const uint64_t *)a, y = *(const uint64_t *)b;
    return (x > y) - (x < y);
}

/* Key of one raw pattern (exported so tests can compare it with float order). */
uint32_t oracle_key(int dtype, uint32_t raw) { return dtype == ORACLE_F32 ? key32(raw) : key16(raw); }

/*
 * x: host array of raw patterns (uint32 for f32, uint16 for bf16), row r at
 * x + r*row_stride elements. out_vals: batch*k raw patterns of the same width.
 * out_idx: batch*k int32. Returns 0, or -1 for bad arguments, -2 when out of
 * memory.
 */
int oracle_topk(const void *x, int dtype, int64_t batch, int64_t n, int64_t row_stride,
                int32_t k, void *out_vals, int32_t *out_idx, int nthreads) {
    if (!x || !out_vals || !out_idx) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    if (batch < 0 || n < 1 || row_stride < n || k < 1 || k > n || n >= ((int64_t)1 << 31)) return -1;
    if (nthreads < 1) nthreads = 1;
    int failed = 0;
    const uint64_t keymax = dtype == ORACLE_F32 ? 0xFFFFFFFFull : 0xFFFFull;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) reduction(| : failed)
    for (int64_t r = 0; r < batch; ++r) {
        uint64_t *a = (uint64_t *)malloc((size_t)n * sizeof(uint64_t));
        if (!a) {
            failed |= 1;
            continue;
        }
        for (int64_t i = 0; i < n; ++i) {
            uint32_t raw = dtype == ORACLE_F32 ? ((const uint32_t *)x)[r * row_stride + i]
                                               : ((const uint16_t *)x)[r * row_stride + i];
            uint64_t key = oracle_key(dtype, raw);
            a[i] = ((keymax - key) << 32) | (uint64_t)i;
        }
        qsort(a, (size_t)n, sizeof(uint64_t), cmp_u64);
        for (int32_t j = 0; j < k; ++j) {
            int64_t i = (int64_t)(a[j] & 0xFFFFFFFFull);
            out_idx[r * k + j] = (int32_t)i;
            if (dtype == ORACLE_F32)
                ((uint32_t *)out_vals)[r * k + j] = ((const uint32_t *)x)[r * row_stride + i];
            else
                ((uint16_t *)out_vals)[r * k + j] = ((const uint16_t *)x)[r * row_stride + i];
        }
        free(a);
    }
    return failed ? -2 : 0;
}
