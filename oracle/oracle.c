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
