/*
 * oracle.c -- CPU oracle for the stable merge of two sorted arrays.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no code, header, table or constant with
 * the HIP path.  It is deliberately plain and slow: one host thread, no
 * blocking, no vectorisation, no allocation (the caller owns every buffer).
 *
 * What it computes (all pinned; nothing here is "parity unpinned"):
 *
 *   oracle_merge_i32   The two-pointer merge: walk A and B once, and at each
 *                      output take A[i] when B is exhausted, or when A is not
 *                      exhausted and A[i] <= B[j] (signed 32-bit compare).
 *                      This is the sequential merge of "merge_path.cu"
 *                      (gpu-preview.ayushworks.com, the host reference
 *                      routine), and the "<=" is the rule "equal keys: the
 *                      element of A goes first" stated in the overview table
 *                      of "Co-rank Function ... Basic Parallel Merge Kernel"
 *                      (pmpp.huatsai.dev, 12-merge/02).
 *   oracle_merge_kv    The same walk on (key, payload) pairs.  Only keys are
 *                      compared; the payload travels with its key.  The pages
 *                      merge keys only; this is the plainest extension, and
 *                      the result is the unique stable merge of the pairs.
 *   oracle_co_rank_all For every output rank k = 0..m+n, the number of A
 *                      elements among the first k outputs of that same walk.
 *                      That is the definition of the co-rank i(k) in the
 *                      section "Co-rank function definition and the i+j=k
 *                      invariant" of the 12-merge/02 page: A[0..i) and
 *                      B[0..k-i) are exactly the first k merged outputs.
 *                      It is found by counting, not by any search.
 *
 *   oracle_merge_keys / oracle_merge_pairs / oracle_key_le
 *                      The same walk for other key types (32- and 64-bit
 *                      integers, signed or not, binary32 and binary64) and
 *                      payload widths (4 or 8 bytes), and for descending
 *                      order; only the comparison and the widths change.
 *                      merge_path.cu merges float keys with "<=" and the
 *                      12-merge pages int keys; neither fixes an order for
 *                      -0.0 against +0.0 or for NaN, so float keys here use
 *                      IEEE 754-2008 totalOrder (clause 5.10), written from
 *                      that definition with float compares: numeric order
 *                      first; among equal numbers -0 precedes +0; a NaN with
 *                      the sign bit set precedes every non-NaN and one without
 *                      follows every non-NaN; two NaNs of one sign order by
 *                      their fraction field (for a negative sign, larger
 *                      fields first).  For keys with no NaN and no pair of
 *                      zeros of opposite sign this is exactly the pages'
 *                      float "<=".  binary64 keys follow the same clause.
 *                      Descending order "x before-or-equal y" is ascending
 *                      "y before-or-equal x"; ties still take A.
 *   oracle_merge_batched  Independent merges of consecutive ranges of A and
 *                      B, each by the walk above, outputs one after another.
 *   oracle_sort        Stable sort by key: bottom-up merge sort with the
 *                      walk above (left run as A).  Its result is the unique
 *                      stable order, which is what it is pinned against.
 *   oracle_merge_runs  One pass of a k-way merge sort: every group of `ways`
 *                      consecutive sorted runs of `run` elements (the last
 *                      group, and its last run, may be short) becomes one
 *                      sorted run.  At each output the smallest head of the
 *                      group's runs is taken; among equal heads, the run that
 *                      comes first in the input.  That is the stable merge of
 *                      the group (its equal keys keep their input order), the
 *                      merge-sort stage of the 13-sorting practice page with
 *                      `ways` runs merged at once instead of two.
 *
 * int32 keys are compared signed.  Lengths are int64, matching the size_t
 * lengths of merge_path.cu.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Take-from-A decision of the two-pointer walk. */
static int take_a(const int32_t *A, int64_t m, int64_t i,
                  const int32_t *B, int64_t n, int64_t j)
{
    if (j >= n)
        return 1;
    if (i < m && A[i] <= B[j])
        return 1;
    return 0;
}

void oracle_merge_i32(const int32_t *A, int64_t m, const int32_t *B,
                      int64_t n, int32_t *C)
{
    int64_t i = 0, j = 0, k;
    for (k = 0; k < m + n; ++k) {
        if (take_a(A, m, i, B, n, j)) {
            C[k] = A[i];
            ++i;
        } else {
            C[k] = B[j];
            ++j;
        }
    }
}

void oracle_merge_kv(const int32_t *Ak, const uint32_t *Av, int64_t m,
                     const int32_t *Bk, const uint32_t *Bv, int64_t n,
                     int32_t *Ck, uint32_t *Cv)
{
    int64_t i = 0, j = 0, k;
    for (k = 0; k < m + n; ++k) {
        if (take_a(Ak, m, i, Bk, n, j)) {
            Ck[k] = Ak[i];
            Cv[k] = Av[i];
            ++i;
        } else {
            Ck[k] = Bk[j];
            Cv[k] = Bv[j];
            ++j;
        }
    }
}

/* I must hold m+n+1 entries.  I[k] = number of A elements among the first k
 * outputs; the matching B count is k - I[k]. */
void oracle_co_rank_all(const int32_t *A, int64_t m, const int32_t *B,
                        int64_t n, int64_t *I)
{
    int64_t i = 0, j = 0, k;
    I[0] = 0;
    for (k = 0; k < m + n; ++k) {
        if (take_a(A, m, i, B, n, j))
            ++i;
        else
            ++j;
        I[k + 1] = i;
    }
}

/* Key kinds and the descending flag, as the typed routines take them. */
enum {
    KIND_I32 = 0, KIND_U32 = 1, KIND_F32 = 2,
    KIND_I64 = 3, KIND_U64 = 4, KIND_F64 = 5,
    ORDER_DESCENDING = 8
};

static int key_size(int kind)
{
    return kind >= KIND_I64 ? 8 : 4;
}

static float as_float(uint32_t bits)
{
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

static double as_double(uint64_t bits)
{
    double d;
    memcpy(&d, &bits, sizeof d);
    return d;
}

/* IEEE 754 totalOrder(x, y): does x come before y, or are they the same
 * datum?  x and y are binary32 bit patterns.  The quiet bit is the top
 * fraction bit, so "signaling before quiet, then by payload" (for a positive
 * sign; reversed for a negative one) is one compare of the fraction fields. */
static int total_order_f32(uint32_t xb, uint32_t yb)
{
    float x = as_float(xb), y = as_float(yb);
    int x_nan = isnan(x), y_nan = isnan(y);
    int x_neg = signbit(x) != 0, y_neg = signbit(y) != 0;
    uint32_t x_frac = xb & 0x7FFFFFu, y_frac = yb & 0x7FFFFFu;
    if (!x_nan && !y_nan) {
        if (x < y)
            return 1;
        if (x > y)
            return 0;
        if (x == 0.0f)            /* both zeros: -0 first */
            return x_neg >= y_neg;
        return 1;                 /* the same number */
    }
    if (x_nan && y_nan) {
        if (x_neg != y_neg)
            return x_neg;         /* -NaN before +NaN */
        return x_neg ? x_frac >= y_frac : x_frac <= y_frac;
    }
    if (x_nan)
        return x_neg;             /* -NaN before anything, +NaN after */
    return !y_neg;                /* y is the NaN */
}

/* The same definition for binary64 bit patterns. */
static int total_order_f64(uint64_t xb, uint64_t yb)
{
    double x = as_double(xb), y = as_double(yb);
    int x_nan = isnan(x), y_nan = isnan(y);
    int x_neg = signbit(x) != 0, y_neg = signbit(y) != 0;
    uint64_t x_frac = xb & 0xFFFFFFFFFFFFFull, y_frac = yb & 0xFFFFFFFFFFFFFull;
    if (!x_nan && !y_nan) {
        if (x < y)
            return 1;
        if (x > y)
            return 0;
        if (x == 0.0)
            return x_neg >= y_neg;
        return 1;
    }
    if (x_nan && y_nan) {
        if (x_neg != y_neg)
            return x_neg;
        return x_neg ? x_frac >= y_frac : x_frac <= y_frac;
    }
    if (x_nan)
        return x_neg;
    return !y_neg;
}

/* Ascending order relation "x before-or-equal y" of one key kind; 32-bit
 * keys are the low 32 bits of x and y. */
static int le_ascending(int kind, uint64_t x, uint64_t y)
{
    switch (kind) {
    case KIND_U32:
        return (uint32_t)x <= (uint32_t)y;
    case KIND_F32:
        return total_order_f32((uint32_t)x, (uint32_t)y);
    case KIND_I64:
        return (int64_t)x <= (int64_t)y;
    case KIND_U64:
        return x <= y;
    case KIND_F64:
        return total_order_f64(x, y);
    default:
        return (int32_t)(uint32_t)x <= (int32_t)(uint32_t)y;
    }
}

int oracle_key_le(int order, uint64_t x, uint64_t y)
{
    int kind = order & 7;
    if (order & ORDER_DESCENDING)
        return le_ascending(kind, y, x);
    return le_ascending(kind, x, y);
}

/* Key i of an array of `size`-byte keys, as a 64-bit pattern. */
static uint64_t key_at(const unsigned char *keys, int size, int64_t i)
{
    uint32_t k32;
    uint64_t k64;
    if (size == 8) {
        memcpy(&k64, keys + 8 * i, 8);
        return k64;
    }
    memcpy(&k32, keys + 4 * i, 4);
    return k32;
}

/* Take-from-A decision of the walk for keys of `order`. */
static int take_a_typed(int order, const unsigned char *A, int64_t m, int64_t i,
                        const unsigned char *B, int64_t n, int64_t j)
{
    int size = key_size(order & 7);
    if (j >= n)
        return 1;
    if (i < m && oracle_key_le(order, key_at(A, size, i), key_at(B, size, j)))
        return 1;
    return 0;
}

/* Keys are 4- or 8-byte patterns per the kind; `order` is a key kind, plus
 * ORDER_DESCENDING for descending inputs and output. */
void oracle_merge_keys(int order, const void *A, int64_t m, const void *B,
                       int64_t n, void *C)
{
    const unsigned char *a = A, *b = B;
    unsigned char *c = C;
    int ks = key_size(order & 7);
    int64_t i = 0, j = 0, k;
    for (k = 0; k < m + n; ++k) {
        if (take_a_typed(order, a, m, i, b, n, j)) {
            memcpy(c + ks * k, a + ks * i, ks);
            ++i;
        } else {
            memcpy(c + ks * k, b + ks * j, ks);
            ++j;
        }
    }
}

/* (key, payload) pairs; payloads are val_bytes (4 or 8) wide and are copied
 * with their keys, never compared. */
void oracle_merge_pairs(int order, int val_bytes, const void *Ak,
                        const void *Av, int64_t m, const void *Bk,
                        const void *Bv, int64_t n, void *Ck, void *Cv)
{
    const unsigned char *ak = Ak, *av = Av, *bk = Bk, *bv = Bv;
    unsigned char *ck = Ck, *cv = Cv;
    int ks = key_size(order & 7), vs = val_bytes;
    int64_t i = 0, j = 0, k;
    for (k = 0; k < m + n; ++k) {
        if (take_a_typed(order, ak, m, i, bk, n, j)) {
            memcpy(ck + ks * k, ak + ks * i, ks);
            memcpy(cv + vs * k, av + vs * i, vs);
            ++i;
        } else {
            memcpy(ck + ks * k, bk + ks * j, ks);
            memcpy(cv + vs * k, bv + vs * j, vs);
            ++j;
        }
    }
}

/* One typed merge of keys, with payloads when val_bytes > 0. */
static void merge_range(int order, int val_bytes, const void *Ak,
                        const void *Av, int64_t m, const void *Bk,
                        const void *Bv, int64_t n, void *Ck, void *Cv)
{
    if (val_bytes > 0)
        oracle_merge_pairs(order, val_bytes, Ak, Av, m, Bk, Bv, n, Ck, Cv);
    else
        oracle_merge_keys(order, Ak, m, Bk, n, Ck);
}

/* A batch of independent merges (the merge-sort stages of page "Practice -
 * Sorting Foundations and Parallel Radix Sort", 13-sorting): merge p takes
 * A[a_off[p], a_off[p+1]) and B[b_off[p], b_off[p+1]) and writes its output
 * at C[a_off[p] + b_off[p] ...).  Each is the walk above. */
void oracle_merge_batched(int order, int val_bytes, const void *Ak,
                          const void *Av, const int64_t *a_off,
                          const void *Bk, const void *Bv,
                          const int64_t *b_off, int64_t pairs, void *Ck,
                          void *Cv)
{
    int ks = key_size(order & 7), vs = val_bytes;
    int64_t p;
    for (p = 0; p < pairs; ++p) {
        int64_t a0 = a_off[p], b0 = b_off[p];
        int64_t c0 = a0 + b0;
        merge_range(order, vs, (const unsigned char *)Ak + ks * a0,
                    vs ? (const unsigned char *)Av + vs * a0 : 0,
                    a_off[p + 1] - a0, (const unsigned char *)Bk + ks * b0,
                    vs ? (const unsigned char *)Bv + vs * b0 : 0,
                    b_off[p + 1] - b0, (unsigned char *)Ck + ks * c0,
                    vs ? (unsigned char *)Cv + vs * c0 : 0);
    }
}

/* Stable sort by key (same page: a stable sort keeps the input order of
 * equal keys), as the page's merge sort: sorted runs of width 1, 2, 4, ...
 * merged pairwise with the walk above (the left run is A, so equal keys keep
 * their input order), until one run remains.  tmp_keys / tmp_vals hold n
 * keys / payloads of scratch; out and in may be the same arrays. */
void oracle_sort(int order, int val_bytes, const void *in_keys,
                 const void *in_vals, int64_t n, void *out_keys,
                 void *out_vals, void *tmp_keys, void *tmp_vals)
{
    int ks = key_size(order & 7), vs = val_bytes;
    unsigned char *src_k = out_keys, *src_v = out_vals;
    unsigned char *dst_k = tmp_keys, *dst_v = tmp_vals;
    int64_t width, i;
    if (out_keys != in_keys)
        memcpy(out_keys, in_keys, (size_t)(n * ks));
    if (vs > 0 && out_vals != in_vals)
        memcpy(out_vals, in_vals, (size_t)(n * vs));
    for (width = 1; width < n; width *= 2) {
        for (i = 0; i < n; i += 2 * width) {
            int64_t la = width < n - i ? width : n - i;
            int64_t lb = n - i - la < width ? n - i - la : width;
            merge_range(order, vs, src_k + ks * i, vs ? src_v + vs * i : 0,
                        la, src_k + ks * (i + la),
                        vs ? src_v + vs * (i + la) : 0, lb, dst_k + ks * i,
                        vs ? dst_v + vs * i : 0);
        }
        {
            unsigned char *t = src_k;
            src_k = dst_k;
            dst_k = t;
            t = src_v;
            src_v = dst_v;
            dst_v = t;
        }
    }
    if (src_k != (unsigned char *)out_keys) {
        memcpy(out_keys, src_k, (size_t)(n * ks));
        if (vs > 0)
            memcpy(out_vals, src_v, (size_t)(n * vs));
    }
}

/* One pass of a k-way merge sort (see the header): each group of `ways`
 * runs of `run` elements of keys[0, n) (and vals) is merged into the same
 * positions of out_keys (out_vals) by repeatedly taking the smallest head,
 * ties to the run that comes first.  out must not overlap the input. */
void oracle_merge_runs(int order, int val_bytes, const void *keys,
                       const void *vals, int64_t n, int64_t run, int ways,
                       void *out_keys, void *out_vals)
{
    int ks = key_size(order & 7), vs = val_bytes;
    const unsigned char *k8 = keys, *v8 = vals;
    unsigned char *ok = out_keys, *ov = out_vals;
    int64_t g0, pos[64], end[64];
    int r;
    if (ways < 1 || ways > 64 || run < 1)
        return;
    for (g0 = 0; g0 < n; g0 += run * ways) {
        int64_t out = g0;
        for (r = 0; r < ways; ++r) {
            int64_t s = g0 + run * r;
            pos[r] = s < n ? s : n;
            end[r] = s + run < n ? s + run : n;
        }
        for (;;) {
            int best = -1;
            for (r = 0; r < ways; ++r) {
                if (pos[r] >= end[r])
                    continue;
                /* a later run takes over only with a strictly smaller key */
                if (best < 0 || !oracle_key_le(order, key_at(k8, ks, pos[best]),
                                               key_at(k8, ks, pos[r])))
                    best = r;
            }
            if (best < 0)
                break;
            memcpy(ok + ks * out, k8 + ks * pos[best], ks);
            if (vs > 0)
                memcpy(ov + vs * out, v8 + vs * pos[best], vs);
            ++pos[best];
            ++out;
        }
    }
}
