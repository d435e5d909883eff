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
 * Keys are signed int32 throughout.  Lengths are int64, matching the size_t
 * lengths of merge_path.cu.
 */
#include <stdint.h>

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
