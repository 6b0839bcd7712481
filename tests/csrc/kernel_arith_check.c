/*
 * Exhaustive CPU checks of two arithmetic shortcuts the quantize kernel takes
 * (restated here from their definitions, not shared with the kernel):
 *
 * 1. Division. For bf16 weights w and a block absmax c1 in [2^-60, 2^60] with
 *    |w| <= c1, the kernel forms x = w / c1 as rc = RN(1/c1), x0 = RN(w*rc),
 *    e = RN(w - x0*c1) (one FMA), x = RN(x0 + e*rc) (one FMA). check_division
 *    compares that against the IEEE quotient for every such bf16 pair: the
 *    NF4 code must always agree, and the value itself whenever |w/c1| >= 2^-10.
 * 2. Code search. The kernel maps x in [-1,1] to bucket floor(32x + 32),
 *    computed as the byte offset (int)fmaf(x, 256, 256) & 0x3F8 = 8 * bucket
 *    (one FMA, one AND), and takes code = (#thresholds below the bucket) +
 *    (x > the one threshold inside the bucket). check_buckets checks the
 *    offset against 8 floor(32x + 32) and the code against #{i : x > T[i]}
 *    for every fp32 x in [-1, 1].
 * 3. Code from the weight (the bf16 path). The kernel forms no quotient:
 *    with rc = RN(1/c1), f = RN(w * (256 rc) + 2^23 + 264) (one FMA) has ulp
 *    1, so (bits(f) & 0x3F8) / 8 = round(256x + 264) / 8 rounded down is
 *    bucket + 1, an entry of a table that holds each bucket's quotient
 *    threshold t' and threshold count; code = count + (RN(w - t' c1) > 0)
 *    (one FMA). check_quotient_codes compares that against the code of the
 *    IEEE quotient for every bf16 pair with c1 in [2^-60, 2^60], |w| <= c1.
 * IEEE binary32 arithmetic, round to nearest even, no flush to zero; fmaf is
 * the fused multiply-add of the C library.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static uint32_t count_above(float x, const float thr[15]) {
    uint32_t c = 0;
    for (int i = 0; i < 15; ++i) c += x > thr[i];
    return c;
}

/* Over every bf16 pair: returns the number of pairs whose NF4 code differs
 * between the shortcut and the IEEE quotient; *value_bad counts pairs with
 * |w/c1| >= 2^-10 whose quotient differs at all (tiny quotients may differ in
 * low bits once intermediate terms underflow; they all sit far below every
 * threshold). */
int64_t check_division(const float thr[15], int64_t* checked, int64_t* value_bad) {
    int64_t bad = 0, n = 0, vbad = 0;
    for (uint32_t cb = 0; cb < 0x8000u; ++cb) {          /* positive bf16 c1 */
        float c1 = f_of(cb << 16);
        if (!(c1 >= 0x1p-60f && c1 <= 0x1p60f)) continue;
        volatile float one = 1.0f;
        float rc = one / c1;
        for (uint32_t wb = 0; wb < 0x10000u; ++wb) {     /* every bf16 w */
            float w = f_of(wb << 16);
            if (!(fabsf(w) <= c1)) continue;
            float x0 = w * rc;
            float e = fmaf(-x0, c1, w);
            float x = fmaf(e, rc, x0);
            float ref = w / c1;
            n++;
            if (x != ref && fabsf(ref) >= 0x1p-10f) vbad++;
            if (count_above(x, thr) != count_above(ref, thr)) bad++;
        }
    }
    *checked = n;
    *value_bad = vbad;
    return bad;
}

int64_t check_buckets(const float thr[15], int64_t* checked) {
    uint32_t lut_thr[65];
    uint32_t lut_below[65];
    for (int b = 0; b < 65; ++b) {
        float lo = -1.0f + (float)b * 0.03125f, hi = lo + 0.03125f;
        uint32_t below = 0;
        float inside = 2.0f;
        for (int i = 0; i < 15; ++i) {
            below += thr[i] < lo;
            if (thr[i] >= lo && thr[i] < hi) inside = thr[i];
        }
        lut_thr[b] = u_of(inside);
        lut_below[b] = below;
    }
    int64_t bad = 0, n = 0;
    /* all fp32 in [-1, 1]: non-negative patterns 0..0x3F800000 and their negatives */
    for (uint32_t u = 0; u <= 0x3F800000u; ++u) {
        for (int sgn = 0; sgn < 2; ++sgn) {
            float x = f_of(u | (sgn ? 0x80000000u : 0u));
            int b = ((int)fmaf(x, 32.0f, 32.0f)) & 127;
            /* the kernel's form: byte offset of the 8-byte entry */
            int off = (int)((uint32_t)(int)fmaf(x, 256.0f, 256.0f) & 0x3F8u);
            if (b > 64 || off != 8 * b) { bad++; continue; }
            uint32_t code = lut_below[b] + (x > f_of(lut_thr[b]) ? 1u : 0u);
            uint32_t ref = 0;
            for (int i = 0; i < 15; ++i) ref += x > thr[i];
            n++;
            if (code != ref) bad++;
        }
    }
    *checked = n;
    return bad;
}

int64_t check_quotient_codes(const float thr[15], const float thr_q[15], int64_t* checked) {
    uint32_t lut_thr[128];
    uint32_t lut_below[128];
    for (int j = 0; j < 128; ++j) {
        int b = j - 1 < 0 ? 0 : (j - 1 > 64 ? 64 : j - 1);
        float lo = -1.0f + (float)b * 0.03125f, hi = lo + 0.03125f;
        uint32_t below = 0;
        float inside = 2.0f;
        for (int i = 0; i < 15; ++i) {
            below += thr[i] < lo;
            if (thr[i] >= lo && thr[i] < hi) inside = thr_q[i];
        }
        lut_thr[j] = u_of(inside);
        lut_below[j] = below;
    }
    int64_t bad = 0, n = 0;
    for (uint32_t cb = 0; cb < 0x8000u; ++cb) {          /* positive bf16 c1 */
        float c1 = f_of(cb << 16);
        if (!(c1 >= 0x1p-60f && c1 <= 0x1p60f)) continue;
        volatile float one = 1.0f;
        float rc256 = (one / c1) * 256.0f;
        for (uint32_t wb = 0; wb < 0x10000u; ++wb) {     /* every bf16 w */
            float w = f_of(wb << 16);
            if (!(fabsf(w) <= c1)) continue;
            float f = fmaf(w, rc256, 8388872.0f);
            uint32_t j = (u_of(f) & 0x3F8u) >> 3;
            float d = fmaf(-f_of(lut_thr[j]), c1, w);
            uint32_t code = lut_below[j] + (d > 0.0f ? 1u : 0u);
            n++;
            if (code != count_above(w / c1, thr)) bad++;
        }
    }
    *checked = n;
    return bad;
}
