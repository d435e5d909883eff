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
 *                      The same walk for other 32-bit key types and for
 *                      descending order; only the comparison changes.
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
 *                      float "<=".  Descending order "x before-or-equal y" is
 *                      ascending "y before-or-equal x"; ties still take A.
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
enum { KIND_I32 = 0, KIND_U32 = 1, KIND_F32 = 2, ORDER_DESCENDING = 4 };

static float as_float(uint32_t bits)
{
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* IEEE 754 totalOrder(x, y): does x come before y, or are they the same
 * datum?  x and y are binary32 bit patterns. */
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

/* Ascending order relation "x before-or-equal y" of one key kind. */
static int le_ascending(int kind, uint32_t x, uint32_t y)
{
    if (kind == KIND_U32)
        return x <= y;
    if (kind == KIND_F32)
        return total_order_f32(x, y);
    return (int32_t)x <= (int32_t)y;
}

int oracle_key_le(int order, uint32_t x, uint32_t y)
{
    int kind = order & 3;
    if (order & ORDER_DESCENDING)
        return le_ascending(kind, y, x);
    return le_ascending(kind, x, y);
}

/* Take-from-A decision of the walk for keys of `order`. */
static int take_a_typed(int order, const uint32_t *A, int64_t m, int64_t i,
                        const uint32_t *B, int64_t n, int64_t j)
{
    if (j >= n)
        return 1;
    if (i < m && oracle_key_le(order, A[i], B[j]))
        return 1;
    return 0;
}

/* Keys are passed as their 32-bit patterns; `order` is a key kind, plus
 * ORDER_DESCENDING for descending inputs and output. */
void oracle_merge_keys(int order, const uint32_t *A, int64_t m,
                       const uint32_t *B, int64_t n, uint32_t *C)
{
    int64_t i = 0, j = 0, k;
    for (k = 0; k < m + n; ++k) {
        if (take_a_typed(order, A, m, i, B, n, j))
            C[k] = A[i++];
        else
            C[k] = B[j++];
    }
}

void oracle_merge_pairs(int order, const uint32_t *Ak, const uint32_t *Av,
                        int64_t m, const uint32_t *Bk, const uint32_t *Bv,
                        int64_t n, uint32_t *Ck, uint32_t *Cv)
{
    int64_t i = 0, j = 0, k;
    for (k = 0; k < m + n; ++k) {
        if (take_a_typed(order, Ak, m, i, Bk, n, j)) {
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
