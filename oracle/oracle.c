/*
 * CPU oracle for the FP4 paged-MQA prefill indexer with exact TopK.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow reference that the
 * HIP path is checked against. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it. It shares no code, table or
 * header with the GPU library, and the GPU library never calls it.
 *
 * Sources (the pages):
 *  [P1] "[FlyDSL] Add FP4 LiteTopK prefill operator" (ROCm/aiter PR 5309):
 *       Summary (model table: H=64, D=128, K in {512,1024}, C4 context);
 *       Implementation (fused FP4 paged-MQA scoring, stable exact TopK,
 *       page mapping; supported-K contract; fail closed on invalid
 *       metadata/pages).
 *  [P2] "[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK" (ROCm/aiter PR 5282):
 *       Changes (score radix then logical-index radix = total order with score
 *       descending and index ascending; NaN below numbers; +0 above -0; raw C4
 *       positions mapped through the page table; short-row contract: length <=
 *       topk returns every logical position in order, padded with -1);
 *       Scope (FP4 E2M1 payload with UE8M0 scales, page size 64, H=64, D=128).
 *  The score itself is the DeepSeek-V4 indexer score that these operators
 *  compute: score[q,s] = sum_h w[q,h] * ReLU(q_h . k_s), one key vector per
 *  C4 position shared by all 64 heads (multi-query attention).
 *
 * Everything is computed in float64. Each 32-element block sum is exact (every
 * E2M1 product is a multiple of 1/4, |block| <= 1152), and every UE8M0 scale
 * is a power of two, so a per-head dot product is exact whenever the four
 * block scale products span less than 2^38 (the generator's exponents, in
 * [-2, 2] per operand, span 2^8). Wider spreads round once per block add.
 *
 * Readings where the pages are silent:
 *  - element 2j of a packed vector is the low nibble of byte j;
 *  - a UE8M0 byte e scales by 2^(e-127); the byte 0xFF decodes to NaN
 *    (out of contract, parity unpinned);
 *  - ReLU(x) = x if x > 0 else +0, and the head sum starts at +0 and runs over
 *    h = 0..63 in order;
 *  - raw indices are absolute logical C4 positions; a window [start, end) is
 *    invalid if start < 0, end < start or end > 64 * P_log (code -1), and a row
 *    fails with code -2 if any page its window touches maps outside
 *    [0, P_phys);
 *  - the K selected positions of a long row are reported in ascending order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_H 64
#define ORACLE_D 128
#define ORACLE_PAGE 64
#define ORACLE_VEC_BYTES 64   /* 128 E2M1 codes */
#define ORACLE_VEC_SCALES 4   /* one UE8M0 byte per 32 elements */

/* E2M1 value of each 4-bit code (OCP MX E2M1: 1 sign, 2 exponent, 1 mantissa
 * bit; codes 8..15 are the negatives of codes 0..7, code 8 is -0). */
static const double E2M1_VALUE[16] = {
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
};

double oracle_e2m1_value(int code) { return E2M1_VALUE[code & 15]; }

/* UE8M0 scale byte -> 2^(e - 127); 0xFF is NaN. */
double oracle_ue8m0_value(int e) {
    if ((e & 255) == 255) return NAN;
    return ldexp(1.0, (e & 255) - 127);
}

/* Code of element i of a packed 64-byte vector (element 2j = low nibble of byte j). */
static int element_code(const uint8_t* v, int i) {
    const uint8_t b = v[i >> 1];
    return (i & 1) ? (b >> 4) : (b & 15);
}

/* Dot product of one query head with one key: sum over the four 32-element
 * blocks of (query block scale) * (key block scale) * sum_j q_j * k_j. */
double oracle_head_dot(const uint8_t* q_head, const uint8_t* q_scale_head,
                       const uint8_t* k_vec, const uint8_t* k_scale_vec) {
    double d = 0.0;
    for (int b = 0; b < ORACLE_D / 32; ++b) {
        double block = 0.0;
        for (int j = 0; j < 32; ++j) {
            const int i = 32 * b + j;
            block += E2M1_VALUE[element_code(q_head, i)] * E2M1_VALUE[element_code(k_vec, i)];
        }
        d += block * oracle_ue8m0_value(q_scale_head[b]) * oracle_ue8m0_value(k_scale_vec[b]);
    }
    return d;
}

/* Indexer score of one query row against one key:
 *   score = sum_h w[h] * ReLU(d_h), starting from +0, h = 0..63.
 * *mag receives sum_h |w[h]| * ReLU(d_h) (used for error bounds). */
double oracle_score(const uint8_t* q_row, const uint8_t* q_scale_row, const float* w_row,
                    const uint8_t* k_vec, const uint8_t* k_scale_vec, double* mag) {
    double acc = 0.0, m = 0.0;
    for (int h = 0; h < ORACLE_H; ++h) {
        const double d = oracle_head_dot(q_row + (size_t)h * ORACLE_VEC_BYTES,
                                         q_scale_row + (size_t)h * ORACLE_VEC_SCALES,
                                         k_vec, k_scale_vec);
        const double r = d > 0.0 ? d : 0.0;
        acc += (double)w_row[h] * r;
        m += fabs((double)w_row[h]) * r;
    }
    if (mag) *mag = m;
    return acc;
}

/* Physical page of logical page p, or -1 if p or its entry is out of range. */
static int64_t physical_page(const int32_t* page_table, int64_t P_log, int64_t P_phys, int64_t p) {
    if (p < 0 || p >= P_log) return -1;
    const int64_t e = page_table[p];
    return (e >= 0 && e < P_phys) ? e : -1;
}

/* Validate a row window (fail-closed contract, [P1] Implementation):
 * 0 = valid, -1 = invalid window, -2 = a touched page maps out of range. */
int oracle_validate_row(int64_t start, int64_t end, const int32_t* page_table,
                        int64_t P_log, int64_t P_phys) {
    if (start < 0 || end < start || end > ORACLE_PAGE * P_log) return -1;
    if (end > start) {
        for (int64_t p = start / ORACLE_PAGE; p <= (end - 1) / ORACLE_PAGE; ++p)
            if (physical_page(page_table, P_log, P_phys, p) < 0) return -2;
    }
    return 0;
}

/* Scores of one row over logical positions [p0, p1) through the page table.
 * Returns 0, or -2 if a page of the range is invalid (nothing is written then). */
int oracle_row_scores(const uint8_t* q_row, const uint8_t* q_scale_row, const float* w_row,
                      const uint8_t* k_pages, const uint8_t* k_scale, int64_t P_phys,
                      const int32_t* page_table, int64_t P_log, int64_t p0, int64_t p1,
                      double* out_score, double* out_mag, int nthreads) {
    for (int64_t s = p0; s < p1; s += ORACLE_PAGE - (s % ORACLE_PAGE))
        if (physical_page(page_table, P_log, P_phys, s / ORACLE_PAGE) < 0) return -2;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t s = p0; s < p1; ++s) {
        const int64_t phys = physical_page(page_table, P_log, P_phys, s / ORACLE_PAGE);
        const size_t slot = (size_t)phys * ORACLE_PAGE + (size_t)(s % ORACLE_PAGE);
        double m = 0.0;
        out_score[s - p0] = oracle_score(q_row, q_scale_row, w_row,
                                         k_pages + slot * ORACLE_VEC_BYTES,
                                         k_scale + slot * ORACLE_VEC_SCALES, &m);
        if (out_mag) out_mag[s - p0] = m;
    }
    (void)nthreads;
    return 0;
}

/* Total order of [P2] Changes: a ranks before b iff
 * a's score is larger, NaN being below every number and +0 above -0, and equal
 * scores (all NaNs are equal) rank by smaller logical index first. */
int oracle_ranks_before(double sa, int64_t ia, double sb, int64_t ib) {
    const int na = isnan(sa) != 0, nb = isnan(sb) != 0;
    if (na != nb) return nb;             /* the number ranks before the NaN */
    if (!na) {
        if (sa > sb) return 1;
        if (sa < sb) return 0;
        if (sa == 0.0 && signbit(sa) != signbit(sb)) return signbit(sb) ? 1 : 0;
    }
    return ia < ib;
}

typedef struct {
    double score;
    int64_t index;
} scored_pos;

static int cmp_rank(const void* pa, const void* pb) {
    const scored_pos* a = (const scored_pos*)pa;
    const scored_pos* b = (const scored_pos*)pb;
    if (oracle_ranks_before(a->score, a->index, b->score, b->index)) return -1;
    if (oracle_ranks_before(b->score, b->index, a->score, a->index)) return 1;
    return 0;
}

static int cmp_i32(const void* pa, const void* pb) {
    const int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/* Exact TopK of a window whose n scores belong to positions start..start+n-1.
 * Short rows (n <= K) return every position in order; long rows return the
 * first K positions of the total order, reported in ascending order. Unused
 * entries of out_raw[K] are -1. Returns the valid count min(n, K). */
int64_t oracle_select_topk(const double* scores, int64_t n, int64_t start, int64_t K,
                           int32_t* out_raw) {
    for (int64_t i = 0; i < K; ++i) out_raw[i] = -1;
    if (n <= K) {
        for (int64_t i = 0; i < n; ++i) out_raw[i] = (int32_t)(start + i);
        return n;
    }
    scored_pos* v = (scored_pos*)malloc((size_t)n * sizeof(scored_pos));
    if (!v) return -100;
    for (int64_t i = 0; i < n; ++i) {
        v[i].score = scores[i];
        v[i].index = start + i;
    }
    qsort(v, (size_t)n, sizeof(scored_pos), cmp_rank);
    for (int64_t i = 0; i < K; ++i) out_raw[i] = (int32_t)v[i].index;
    free(v);
    qsort(out_raw, (size_t)K, sizeof(int32_t), cmp_i32);
    return K;
}

/* Physical slot of a raw logical position: page_table[raw / 64] * 64 + raw % 64;
 * -1 stays -1 ([P2] Changes: logical positions are translated into physical slots by the
 * page table). */
int64_t oracle_slot(int64_t raw, const int32_t* page_table) {
    if (raw < 0) return -1;
    return (int64_t)page_table[raw / ORACLE_PAGE] * ORACLE_PAGE + raw % ORACLE_PAGE;
}

/* The whole operator for one row. Writes out_raw[K], out_slot[K] and, if given,
 * out_sel_score[K] (the float64 scores of the selected positions, NaN where
 * unused) and returns the count, or -1/-2 for an invalid row (outputs all -1). */
int64_t oracle_topk_row(const uint8_t* q, const uint8_t* q_scale, const float* weights,
                        const uint8_t* k_pages, const uint8_t* k_scale, int64_t P_phys,
                        const int32_t* page_table, int64_t P_log,
                        const int32_t* row_start, const int32_t* row_end, int64_t row,
                        int64_t K, int32_t* out_raw, int32_t* out_slot, double* out_sel_score,
                        int nthreads) {
    const int64_t start = row_start[row], end = row_end[row];
    for (int64_t i = 0; i < K; ++i) {
        out_raw[i] = -1;
        out_slot[i] = -1;
        if (out_sel_score) out_sel_score[i] = NAN;
    }
    const int v = oracle_validate_row(start, end, page_table, P_log, P_phys);
    if (v < 0) return v;
    const int64_t n = end - start;
    int64_t count;
    if (n <= K) {
        count = oracle_select_topk(NULL, n, start, K, out_raw);
    } else {
        double* s = (double*)malloc((size_t)n * sizeof(double));
        if (!s) return -100;
        oracle_row_scores(q + (size_t)row * ORACLE_H * ORACLE_VEC_BYTES,
                          q_scale + (size_t)row * ORACLE_H * ORACLE_VEC_SCALES,
                          weights + (size_t)row * ORACLE_H, k_pages, k_scale, P_phys,
                          page_table, P_log, start, end, s, NULL, nthreads);
        count = oracle_select_topk(s, n, start, K, out_raw);
        if (out_sel_score)
            for (int64_t i = 0; i < count; ++i) out_sel_score[i] = s[out_raw[i] - start];
        free(s);
    }
    for (int64_t i = 0; i < count; ++i) out_slot[i] = (int32_t)oracle_slot(out_raw[i], page_table);
    return count;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- MXFP4 quantisation: the producer of the path's FP4 inputs ------------
 *
 * The pages name the payload only ("FP4 E2M1 payload with UE8M0 scales", [P2]
 * Scope); the rule that turns real values into it is the OCP Microscaling
 * Formats (MX) v1.0 conversion of a vector of scalars into one MX block, read
 * for E2M1 elements (largest element exponent emax = 2, largest magnitude 6)
 * and a UE8M0 shared scale:
 *   1. the shared exponent is floor(log2(max_i |V_i|)) - emax;
 *   2. the scale is X = 2^(shared exponent);
 *   3. every element is V_i / X rounded to the nearest E2M1 value, a tie going
 *      to the code whose mantissa bit is 0, magnitudes beyond 6 saturating to 6,
 *      and the sign kept (a negative value that rounds to zero is -0, code 8).
 * Readings where that rule leaves the encoding open:
 *   - the scale byte is shared + 127, clamped to [0, 254];
 *   - a block whose elements are all zero gets scale byte 0 and the zero codes
 *     of their signs;
 *   - a block holding a NaN or an infinity gets scale byte 0xFF (the UE8M0 NaN)
 *     and all-zero codes;
 *   - element 2j of a block is the low nibble of byte j (as everywhere here).
 * The division by X is exact (a power of two; a result below the float64
 * normal range would be far below the first rounding boundary, 0.25).
 */

/* E2M1 code (0..15) of a real value already divided by the block scale. */
int oracle_e2m1_encode(double v) {
    const int neg = signbit(v) ? 1 : 0;
    const double a = fabs(v);
    int best = 0;
    for (int m = 1; m < 8; ++m) {
        const double dm = fabs(a - E2M1_VALUE[m]), db = fabs(a - E2M1_VALUE[best]);
        if (dm < db || (dm == db && (m & 1) == 0)) best = m;
    }
    return best | (neg << 3);
}

/* Scale byte of one 32-element block (see the readings above). */
int oracle_mx_scale_byte(const float* x) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        if (!isfinite(x[i])) return 0xFF;
        if (fabs((double)x[i]) > amax) amax = fabs((double)x[i]);
    }
    if (amax == 0.0) return 0;
    int e2;
    (void)frexp(amax, &e2);            /* amax = f * 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
    int byte = (e2 - 1) - 2 + 127;
    if (byte < 0) byte = 0;
    if (byte > 254) byte = 254;
    return byte;
}

/* n_blocks blocks of 32 floats -> 16 code bytes and one scale byte each. */
void oracle_mx_quantize(const float* x, int64_t n_blocks, uint8_t* codes, uint8_t* scales) {
    for (int64_t b = 0; b < n_blocks; ++b) {
        const float* xb = x + 32 * b;
        const int sb = oracle_mx_scale_byte(xb);
        scales[b] = (uint8_t)sb;
        for (int j = 0; j < 16; ++j) {
            int lo = 0, hi = 0;
            if (sb != 0xFF) {
                const double X = ldexp(1.0, sb - 127);
                lo = oracle_e2m1_encode((double)xb[2 * j] / X);
                hi = oracle_e2m1_encode((double)xb[2 * j + 1] / X);
            }
            codes[16 * b + j] = (uint8_t)(lo | (hi << 4));
        }
    }
}
