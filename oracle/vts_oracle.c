/*
 * vts_oracle.c -- CPU oracle for exact batched variable-length top-K selection.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the HIP path is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It shares
 * no code, header, table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * What it computes, and where that is defined:
 *
 *   valid length   FlashInfer "flashinfer.top_k_varlen" documentation, the
 *                  `seq_lens` and `compress_ratio` parameters: row t of request
 *                  i ranks its first max(0, (seq_lens[i] - next_n + t + 1) //
 *                  compress_ratio) columns, clamped to the logits width; a row
 *                  with no valid column is all -1.
 *   selection      same page, the `gvr_2` backend text and the `returns`
 *                  section: exact top-k of each row, ties interchangeable.
 *                  Done here by a full sort of the row (descending value, then
 *                  ascending column), keeping the first k.  That is the plain
 *                  definition; the sort is a library primitive (qsort).
 *   short rows     TensorRT-LLM PR #17821 (self-sampling GVR V2), the commit
 *                  on the short-row pad convention: n <= k gives the identity
 *                  indices then -1; the commit adding the optional `values`
 *                  output: the short path copies the head and pads with
 *                  -FLT_MAX.
 *   transform      FlashInfer page-table-transform PR body quoted on the
 *                  SGLang PR #33237 page, "Description" section:
 *                    physical_page = src_page_table[b, page_table_row_start + idx / page_size]
 *                    output        = physical_page * page_size + idx % page_size
 *                  with `row_starts` in score elements, `page_table_row_starts`
 *                  in page-table entries, and -1 in every unused suffix slot of
 *                  both outputs.  `lengths`/`row_starts` follow the SGLang
 *                  TopK_Ops page, I/O contract of fast_topk_v2.
 *
 * Readings taken where the pages are silent:
 *   - equal values (including -0 and +0) are ties; the oracle breaks them by
 *     ascending column so its own output is deterministic;
 *   - NaN: the pages call its order implementation specific.  The oracle puts a
 *     NaN with the sign bit clear above +inf and one with the sign bit set
 *     below -inf, so its comparison is a total order; no parity case holds NaN
 *     and this order is parity unpinned (rows with NaN are checked for valid,
 *     distinct indices only);
 *   - value padding: -FLT_MAX for fp32; for bf16/fp16 the lowest finite value
 *     of that type (0xFF7F, 0xFBFF);
 *   - transform row window: n = clamp(length, 0, width - row_start); a row
 *     start outside [0, width] gives an empty row;
 *   - a page-table read outside [0, page_table_width) yields -1 in `out`.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -pthread vts_oracle.c -o liboracle.so
 */
#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2 };

/* ------------------------------------------------------------------ */
/* element decoding: raw bits -> double (exact for all three formats)  */
/* ------------------------------------------------------------------ */

static double decode_f32(uint32_t bits) {
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double decode_bf16(uint16_t bits) { return decode_f32((uint32_t)bits << 16); }

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits. */
static double decode_f16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1F;
    int m = bits & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal (or zero): m * 2^-24 */
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double load_elem(const void *x, int dtype, int64_t off, int *sign_out) {
    if (dtype == ORC_F32) {
        uint32_t b;
        memcpy(&b, (const char *)x + off * 4, 4);
        *sign_out = (int)(b >> 31);
        return decode_f32(b);
    } else {
        uint16_t b;
        memcpy(&b, (const char *)x + off * 2, 2);
        *sign_out = (int)(b >> 15);
        return dtype == ORC_BF16 ? decode_bf16(b) : decode_f16(b);
    }
}

static void copy_elem(const void *x, int dtype, int64_t off, void *dst, int64_t dst_off) {
    size_t sz = dtype == ORC_F32 ? 4 : 2;
    memcpy((char *)dst + dst_off * sz, (const char *)x + off * sz, sz);
}

static void store_pad(int dtype, void *dst, int64_t dst_off) {
    if (dtype == ORC_F32) {
        uint32_t b = 0xFF7FFFFFu; /* -FLT_MAX */
        memcpy((char *)dst + dst_off * 4, &b, 4);
    } else {
        uint16_t b = dtype == ORC_BF16 ? 0xFF7Fu : 0xFBFFu; /* lowest finite */
        memcpy((char *)dst + dst_off * 2, &b, 2);
    }
}

/* ------------------------------------------------------------------ */
/* valid lengths                                                       */
/* ------------------------------------------------------------------ */

/* FlashInfer top_k_varlen doc, `seq_lens`: row t of request i ranks its first
 * max(0, (seq_lens[i] - next_n + t + 1) // compress_ratio) columns, clamped to
 * the width.  Evaluated in 64-bit so no seq_len can overflow. */
int64_t vts_oracle_valid_len(int32_t seq_len, int32_t next_n, int32_t t, int32_t compress_ratio,
                             int64_t width) {
    int64_t num = (int64_t)seq_len - (int64_t)next_n + (int64_t)t + 1;
    int64_t n = num <= 0 ? 0 : num / compress_ratio;
    return n < width ? n : width;
}

/* One entry per row: base = 0, n from the formula above, request i = r / next_n. */
void vts_oracle_varlen_rows(const int32_t *seq_lens, int64_t num_rows, int32_t next_n,
                            int32_t compress_ratio, int64_t width, int64_t *base_out,
                            int64_t *n_out) {
    for (int64_t r = 0; r < num_rows; ++r) {
        base_out[r] = 0;
        n_out[r] = vts_oracle_valid_len(seq_lens[r / next_n], next_n, (int32_t)(r % next_n),
                                        compress_ratio, width);
    }
}

/* SGLang TopK_Ops page, fast_topk_v2: `lengths` is the valid length of each
 * row and `row_starts` the start of each row's window in the score row.
 * Reading: the window is clamped to the row width; an out-of-range start gives
 * an empty row. */
void vts_oracle_window_rows(const int32_t *lengths, const int32_t *row_starts, int64_t num_rows,
                            int64_t width, int64_t *base_out, int64_t *n_out) {
    for (int64_t r = 0; r < num_rows; ++r) {
        int64_t base = row_starts ? (int64_t)row_starts[r] : 0;
        int64_t len = lengths[r];
        int64_t n;
        if (base < 0 || base > width) {
            base = 0;
            n = 0;
        } else {
            int64_t room = width - base;
            n = len < 0 ? 0 : (len > room ? room : len);
        }
        base_out[r] = base;
        n_out[r] = n;
    }
}

/* ------------------------------------------------------------------ */
/* per-row selection by full sort                                      */
/* ------------------------------------------------------------------ */

typedef struct {
    double v;
    int nan_class; /* 0 = not NaN, +1 = NaN with sign clear, -1 = NaN with sign set */
    int64_t col;
} item_t;

/* Descending by value; -0 and +0 compare equal as doubles; ties by ascending
 * column.  NaN classes sit above +inf (+1) or below -inf (-1). */
static int cmp_desc(const void *pa, const void *pb) {
    const item_t *a = (const item_t *)pa, *b = (const item_t *)pb;
    if (a->nan_class != b->nan_class) return a->nan_class > b->nan_class ? -1 : 1;
    if (a->nan_class == 0) {
        if (a->v > b->v) return -1;
        if (a->v < b->v) return 1;
    }
    if (a->col < b->col) return -1;
    if (a->col > b->col) return 1;
    return 0;
}

typedef struct {
    const void *x;
    int dtype;
    int64_t num_rows;
    int64_t row_stride;
    const int64_t *base;
    const int64_t *n;
    int32_t k;
    int32_t *out_idx;
    void *out_vals;
    atomic_llong next_row;
    atomic_int failed;
} job_t;

static void select_row(job_t *J, int64_t r, item_t *buf) {
    const int64_t k = J->k, n = J->n[r];
    int32_t *oi = J->out_idx + r * k;
    const int64_t row_off = r * J->row_stride + J->base[r];
    if (n <= k) {
        /* every valid column is selected: identity, then -1 */
        for (int64_t j = 0; j < k; ++j) {
            oi[j] = j < n ? (int32_t)j : -1;
            if (J->out_vals) {
                if (j < n)
                    copy_elem(J->x, J->dtype, row_off + j, J->out_vals, r * k + j);
                else
                    store_pad(J->dtype, J->out_vals, r * k + j);
            }
        }
        return;
    }
    for (int64_t j = 0; j < n; ++j) {
        int sign;
        double v = load_elem(J->x, J->dtype, row_off + j, &sign);
        buf[j].v = v;
        buf[j].nan_class = isnan(v) ? (sign ? -1 : 1) : 0;
        buf[j].col = j;
    }
    qsort(buf, (size_t)n, sizeof(item_t), cmp_desc);
    for (int64_t j = 0; j < k; ++j) {
        oi[j] = (int32_t)buf[j].col;
        if (J->out_vals) copy_elem(J->x, J->dtype, row_off + buf[j].col, J->out_vals, r * k + j);
    }
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    int64_t cap = 0;
    for (int64_t r = 0; r < J->num_rows; ++r)
        if (J->n[r] > cap) cap = J->n[r];
    item_t *buf = (item_t *)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(item_t));
    if (!buf) {
        atomic_store(&J->failed, 1);
        return NULL;
    }
    for (;;) {
        int64_t r = atomic_fetch_add(&J->next_row, 1);
        if (r >= J->num_rows) break;
        select_row(J, r, buf);
    }
    free(buf);
    return NULL;
}

/* Exact top-k of each row window x[r, base[r] : base[r] + n[r]).
 * out_idx: int32[num_rows, k], window-relative columns, the k largest in
 * descending order (ties by ascending column), -1 for slots beyond n.
 * out_vals (nullable): bit copies of the selected elements, padding after n.
 * Rows are spread over nthreads POSIX threads.  Returns 0, or -1 when memory
 * could not be allocated. */
int vts_oracle_select(const void *x, int dtype, int64_t num_rows, int64_t row_stride,
                      const int64_t *base, const int64_t *n, int32_t k, int32_t *out_idx,
                      void *out_vals, int nthreads) {
    job_t J;
    J.x = x;
    J.dtype = dtype;
    J.num_rows = num_rows;
    J.row_stride = row_stride;
    J.base = base;
    J.n = n;
    J.k = k;
    J.out_idx = out_idx;
    J.out_vals = out_vals;
    atomic_init(&J.next_row, 0);
    atomic_init(&J.failed, 0);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[started], NULL, worker, &J) != 0) break;
        ++started;
    }
    worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    return atomic_load(&J.failed) ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* page-table transform                                                */
/* ------------------------------------------------------------------ */

/* Page-table transform of the FlashInfer PR body ("Description"), applied to
 * window-relative indices `raw`:
 *   out = src_page_table[r * pt_stride + pt_start + raw / page_size] * page_size
 *         + raw % page_size,
 * pt_start = page_table_row_starts[r] when given, else base[r] (the shared
 * start).  raw < 0 gives -1.  A page-table column outside [0, pt_width) gives
 * -1 (reading).  Computed in 64-bit; a result outside int32 is reported by a
 * return value of 1 (the entry is still stored, truncated). */
int vts_oracle_page_translate(const int32_t *raw, int64_t num_rows, int32_t k,
                              const int32_t *src_page_table, int64_t pt_stride, int64_t pt_width,
                              const int32_t *page_table_row_starts, const int64_t *base,
                              int32_t page_size, int32_t *out) {
    int overflow = 0;
    for (int64_t r = 0; r < num_rows; ++r) {
        int64_t pt_start = page_table_row_starts ? (int64_t)page_table_row_starts[r] : base[r];
        for (int64_t j = 0; j < k; ++j) {
            int64_t idx = raw[r * k + j];
            int64_t res = -1;
            if (idx >= 0) {
                int64_t col = pt_start + idx / page_size;
                if (col >= 0 && col < pt_width) {
                    int64_t page = src_page_table[r * pt_stride + col];
                    res = page * page_size + idx % page_size;
                    if (res > INT32_MAX || res < INT32_MIN) overflow = 1;
                }
            }
            out[r * k + j] = (int32_t)res;
        }
    }
    return overflow;
}
