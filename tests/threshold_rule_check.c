/* Exhaustive check of the bfloat16 threshold test on raw bits against the key
 * order (tests/test_threshold_rule.py builds and runs it).
 *
 * argv[1] names a file of 65536 little-endian uint32 keys, key[p] for the
 * 16-bit pattern p, written from the oracle's key transform. For every
 * threshold pattern t and every value pattern h, the test below must equal
 * key[h] > key[t]:
 *   - T >= +0 (key[t] >= 0x8000): (int32)(h << 16 | low) > (int32)(t << 16 | 0xFFFF)
 *   - T <  0:                     (uint32)(h << 16 | low) < (uint32)(t << 16)
 * for low = 0, 0xFFFF and a pseudo-random low half; and the 16-bit form with
 * a saturating subtract: sat(t - h) < 0 (T >= +0), or
 * sat((h ^ 0x8000) - (t ^ 0x8000)) < 0 (T < 0), on signed halves.
 * Prints the first mismatch and exits 1 on any; exits 0 otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

static uint32_t key[65536];

static int32_t sat16(int32_t a, int32_t b) {
    int32_t d = a - b;
    return d > 32767 ? 32767 : (d < -32768 ? -32768 : d);
}

int main(int argc, char** argv) {
    if (argc != 2) return 2;
    FILE* f = fopen(argv[1], "rb");
    if (!f || fread(key, 4, 65536, f) != 65536) return 2;
    fclose(f);
    static uint32_t lowr[65536];
    uint32_t s = 0x9E3779B9u;
    for (int h = 0; h < 65536; ++h) {
        s ^= s << 13;
        s ^= s >> 17;
        s ^= s << 5;
        lowr[h] = s & 0xFFFFu;
    }
    uint64_t bad = 0;
    for (uint32_t t = 0; t < 65536; ++t) {
        const uint32_t kt = key[t];
        const int neg = kt < 0x8000u;
        const uint32_t thr = neg ? (t << 16) : ((t << 16) | 0xFFFFu);
        const int32_t ts = (int16_t)t, tx = (int16_t)(t ^ 0x8000u);
        uint64_t miss = 0;
        for (uint32_t h = 0; h < 65536; ++h) {
            const int want = key[h] > kt;
            const uint32_t w0 = h << 16, w1 = (h << 16) | 0xFFFFu, w2 = (h << 16) | lowr[h];
            int r0, r1, r2, rp;
            if (neg) {
                r0 = w0 < thr;
                r1 = w1 < thr;
                r2 = w2 < thr;
                rp = sat16((int16_t)(h ^ 0x8000u), tx) < 0;
            } else {
                r0 = (int32_t)w0 > (int32_t)thr;
                r1 = (int32_t)w1 > (int32_t)thr;
                r2 = (int32_t)w2 > (int32_t)thr;
                rp = sat16(ts, (int16_t)h) < 0;
            }
            miss += (uint64_t)((r0 != want) + (r1 != want) + (r2 != want) + (rp != want));
        }
        if (miss && !bad) {
            for (uint32_t h = 0; h < 65536; ++h) {
                const int want = key[h] > kt;
                const int r = neg ? ((h << 16) < thr) : ((int32_t)(h << 16) > (int32_t)thr);
                if (r != want) {
                    fprintf(stderr, "threshold %#06x value %#06x: rule %d, key order %d\n", t, h, r, want);
                    break;
                }
            }
        }
        bad += miss;
    }
    printf("bfloat16 threshold rule: %llu mismatches over 2^32 pairs x 4 forms\n", (unsigned long long)bad);
    return bad ? 1 : 0;
}
