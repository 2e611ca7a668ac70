/*
 * Exercise of the CPU oracle (oracle/vts_oracle.c) for a sanitizer build
 * (AddressSanitizer + UndefinedBehaviorSanitizer): rows of every dtype with
 * ties, signed zeros, infinities, NaNs of both signs, empty and short rows,
 * every top_k from 1 to past the row, several threads, odd windows and page
 * tables with entries outside the table.  Checks the properties the oracle
 * promises (distinct in-window indices, -1 suffix, descending order) and exits
 * non-zero on the first violation; memory and UB errors abort the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t vts_oracle_valid_len(int32_t, int32_t, int32_t, int32_t, int64_t);
void vts_oracle_varlen_rows(const int32_t*, int64_t, int32_t, int32_t, int64_t, int64_t*, int64_t*);
void vts_oracle_window_rows(const int32_t*, const int32_t*, int64_t, int64_t, int64_t*, int64_t*);
int vts_oracle_select(const void*, int, int64_t, int64_t, const int64_t*, const int64_t*, int32_t,
                      int32_t*, void*, int);
int vts_oracle_page_translate(const int32_t*, int64_t, int32_t, const int32_t*, int64_t, int64_t,
                              const int32_t*, const int64_t*, int32_t, int32_t*);

static uint64_t rng = 88172645463325252ull;
static uint32_t next32(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}

static const uint32_t F32_POOL[] = {0x00000000u, 0x80000000u, 0x3F800000u, 0xBF800000u, 0x40000000u,
                                    0x7F800000u, 0xFF800000u, 0x00000001u, 0x80000001u, 0x7FC00000u,
                                    0xFFC00000u, 0x7F7FFFFFu, 0x3F000000u};
static const uint16_t H16_POOL[] = {0x0000u, 0x8000u, 0x3C00u, 0xBC00u, 0x4000u, 0x7C00u, 0xFC00u,
                                    0x0001u, 0x7E00u, 0xFE00u, 0x3F80u, 0x7F80u, 0x7FC0u};

static double val(const void* x, int dt, int64_t i) {
    if (dt == 0) {
        uint32_t b;
        memcpy(&b, (const char*)x + i * 4, 4);
        float f;
        memcpy(&f, &b, 4);
        return f;
    }
    uint16_t b;
    memcpy(&b, (const char*)x + i * 2, 2);
    if (dt == 1) {
        uint32_t w = (uint32_t)b << 16;
        float f;
        memcpy(&f, &w, 4);
        return f;
    }
    int s = b >> 15, e = (b >> 10) & 31, m = b & 1023;
    double v = e == 0 ? ldexp(m, -24) : e == 31 ? (m ? NAN : INFINITY) : ldexp(m + 1024, e - 25);
    return s ? -v : v;
}

static int fail(const char* what, int dt, int64_t r, int32_t k) {
    fprintf(stderr, "violation: %s (dtype %d, row %lld, k %d)\n", what, dt, (long long)r, k);
    return 1;
}

int main(void) {
    for (int trial = 0; trial < 60; ++trial) {
        const int dt = trial % 3;
        const int64_t R = 1 + next32() % 6, S = 1 + next32() % 300;
        const size_t isz = dt == 0 ? 4 : 2;
        char* x = malloc((size_t)(R * S) * isz);
        for (int64_t i = 0; i < R * S; ++i) {
            if (dt == 0) {
                uint32_t b = (next32() & 3) ? F32_POOL[next32() % 13] : next32();
                memcpy(x + i * 4, &b, 4);
            } else {
                uint16_t b = (next32() & 3) ? H16_POOL[next32() % 13] : (uint16_t)next32();
                memcpy(x + i * 2, &b, 2);
            }
        }
        int32_t* lengths = malloc(R * sizeof(int32_t));
        int32_t* starts = malloc(R * sizeof(int32_t));
        for (int64_t r = 0; r < R; ++r) {
            lengths[r] = (int32_t)(next32() % (S + 20)) - 5;
            starts[r] = (int32_t)(next32() % (S + 4)) - 2;
        }
        int64_t* base = malloc(R * sizeof(int64_t));
        int64_t* n = malloc(R * sizeof(int64_t));
        vts_oracle_window_rows(lengths, (trial & 1) ? starts : NULL, R, S, base, n);
        for (int32_t k = 1; k <= S + 3; k += 1 + (int32_t)(next32() % 7)) {
            int32_t* idx = malloc((size_t)(R * k) * sizeof(int32_t));
            void* vals = malloc((size_t)(R * k) * isz);
            if (vts_oracle_select(x, dt, R, S, base, n, k, idx, vals, 1 + trial % 4) != 0)
                return fail("select failed", dt, -1, k);
            for (int64_t r = 0; r < R; ++r) {
                const int64_t m = n[r] < k ? n[r] : k;
                for (int64_t j = 0; j < k; ++j) {
                    const int32_t c = idx[r * k + j];
                    if (j >= m) {
                        if (c != -1) return fail("suffix not -1", dt, r, k);
                        continue;
                    }
                    if (c < 0 || c >= n[r]) return fail("index outside the window", dt, r, k);
                    for (int64_t q = 0; q < j; ++q)
                        if (idx[r * k + q] == c) return fail("duplicate index", dt, r, k);
                    if (n[r] > k && j > 0) {
                        const double a = val(x, dt, r * S + base[r] + idx[r * k + j - 1]);
                        const double b = val(x, dt, r * S + base[r] + c);
                        if (!isnan(a) && !isnan(b) && a < b) return fail("not descending", dt, r, k);
                    }
                }
            }
            /* page translation of the selection, with a narrow table */
            const int32_t P = 1 + (int32_t)(next32() % 16), ps = 1 + (int32_t)(next32() % 8);
            int32_t* pt = malloc((size_t)(R * P) * sizeof(int32_t));
            int32_t* ptrs = malloc(R * sizeof(int32_t));
            for (int64_t i = 0; i < R * P; ++i) pt[i] = (int32_t)(next32() % 100000);
            for (int64_t r = 0; r < R; ++r) ptrs[r] = (int32_t)(next32() % 5) - 1;
            int32_t* out = malloc((size_t)(R * k) * sizeof(int32_t));
            vts_oracle_page_translate(idx, R, k, pt, P, P, (trial & 2) ? ptrs : NULL, base, ps, out);
            for (int64_t i = 0; i < R * k; ++i)
                if (idx[i] < 0 && out[i] != -1) return fail("translated -1", dt, i / k, k);
            free(pt);
            free(ptrs);
            free(out);
            free(idx);
            free(vals);
        }
        /* the valid-length rule over extreme lengths */
        int32_t seq[4] = {INT32_MIN, -1, INT32_MAX, (int32_t)(next32() % 1000)};
        int64_t b2[8], n2[8];
        vts_oracle_varlen_rows(seq, 8, 2, 1 + trial % 4, S, b2, n2);
        for (int i = 0; i < 8; ++i)
            if (n2[i] < 0 || n2[i] > S) return fail("valid length out of range", dt, i, 0);
        free(x);
        free(lengths);
        free(starts);
        free(base);
        free(n);
    }
    printf("oracle battery clean\n");
    return 0;
}
