// corank.hpp -- device co-rank search for gfx950.
//
// The co-rank of output rank k is the i for which A[0..i) and B[0..k-i) are
// exactly the first k outputs of the stable merge (page "Co-rank Function ...
// and Basic Parallel Merge Kernel", pmpp.huatsai.dev/12-merge/02, section
// "Co-rank function definition and the i+j=k invariant").
//
// The search is the one that page describes under "Binary-Search
// Implementation" and in its formula table: start from the upper bound
// i = min(k, m), j = k - i, with lower bounds i_low = max(0, k - n) and
// j_low = max(0, k - m).  A split with A[i-1] > B[j] holds too many A
// elements: i moves down and j up by ceil((i - i_low)/2), and j_low rises to
// the old j.  A split with B[j-1] >= A[i] holds too many B elements: j moves
// down and i up by ceil((j - j_low)/2), and i_low rises to the old i.  Any
// other split is the answer.  The strict '>' against '>=' is what puts equal
// A keys first; the half-step must round up or an interval of width one never
// shrinks (page "merge_path.cu", comment on its co-rank routine).
//
// The same logic serves global memory (the partition kernel) and the LDS ring
// of the merge kernel: only the element accessors differ, which is the
// "simplified model" of page "Tiled and Circular Buffer Merge Kernel"
// (12-merge/03): user code sees a contiguous window, accessors translate.
//
// MI355X specifics: each step issues its four neighbour loads together (the
// indices are clamped into range, so none is conditional), which costs one
// memory round trip per step instead of two.  The step count is capped: for
// sorted input the search makes at most bitlen(min(m, n)) adjustments, so the
// cap is never reached; it only bounds the loop when the caller breaks the
// sortedness precondition.  Every adjustment keeps
// max(0, k-n) <= i <= min(k, m), so the result is always in range.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <limits>
#include <type_traits>

namespace omerge {

// Key orders.  Every supported key type and direction is merged as a signed
// integer of the key's width after an order-preserving bijection of its bits,
// applied when a key is read from HBM and undone when it is written back, so
// the output keeps the input's exact bits:
//   int32 / int64 ascending      identity
//   uint32 / uint64 ascending    flip the sign bit
//   float32 / float64 ascending  IEEE 754 totalOrder (-NaN < -inf < ... < -0 <
//                                +0 < ... < +inf < +NaN): flip every bit but
//                                the sign of negative values, so larger
//                                magnitudes sort lower
//   descending                   bitwise NOT of the ascending image
//                                (~y = -y-1 reverses signed order)
// Ties (equal images) still take A first.  Each ascending map is its own
// inverse; from_ord undoes the final NOT first.
enum KeyKind : int {
    kKeyI32 = 0,
    kKeyU32 = 1,
    kKeyF32 = 2,
    kKeyI64 = 3,
    kKeyU64 = 4,
    kKeyF64 = 5
};
constexpr int kKeyDescending = 8;  // OR-ed into a kind: descending order

template <int ORDER>  // ORDER = KeyKind | kKeyDescending (optional)
struct KeyOrder {
    static constexpr int kKind = ORDER & 7;
    static constexpr bool kDescending = (ORDER & kKeyDescending) != 0;
    static constexpr bool kWide = kKind >= kKeyI64;
    // The key's bits as a signed integer of its width.
    using T = typename std::conditional<kWide, long long, int>::type;
    static constexpr int kWords = kWide ? 2 : 1;  // 32-bit words per key
    static constexpr T kMax = kWide ? T(INT64_MAX) : T(INT32_MAX);
    __host__ __device__ static __forceinline__ T asc(T x) {
        constexpr int kTop = 8 * sizeof(T) - 1;
        constexpr T kSign = std::numeric_limits<T>::min();  // the sign bit alone
        if (kKind == kKeyU32 || kKind == kKeyU64) return x ^ kSign;
        if (kKind == kKeyF32 || kKind == kKeyF64) return x ^ ((x >> kTop) & ~kSign);
        return x;
    }
    __host__ __device__ static __forceinline__ T to_ord(T x) {
        return kDescending ? ~asc(x) : asc(x);
    }
    __host__ __device__ static __forceinline__ T from_ord(T y) {
        return asc(kDescending ? ~y : y);
    }
};

// Adjustment cap for 64-bit searches over global memory and for 32-bit
// searches inside one LDS tile (windows of at most 2^16 elements).
constexpr int kMaxStepsGlobal = 2 * 64 + 2;
constexpr int kMaxStepsTile = 2 * 17 + 2;

template <typename Idx, typename LoadA, typename LoadB>
__device__ __forceinline__ Idx co_rank(Idx k, Idx m, Idx n, LoadA load_a,
                                       LoadB load_b, int max_steps) {
    Idx i = k < m ? k : m;
    Idx j = k - i;
    if (m == 0 || n == 0) return i;  // one side empty: the bound is the answer
    Idx i_low = k > n ? k - n : Idx(0);
    Idx j_low = k > m ? k - m : Idx(0);
    for (int step = 0; step < max_steps; ++step) {
        const auto a_prev = load_a(i > 0 ? i - 1 : Idx(0));
        const auto a_here = load_a(i < m ? i : m - 1);
        const auto b_prev = load_b(j > 0 ? j - 1 : Idx(0));
        const auto b_here = load_b(j < n ? j : n - 1);
        const bool too_many_a = i > 0 && j < n && a_prev > b_here;
        const bool too_many_b = j > 0 && i < m && b_prev >= a_here;
        if (too_many_a) {
            const Idx d = (i - i_low + 1) >> 1;
            j_low = j;
            i -= d;
            j += d;
        } else if (too_many_b) {
            const Idx d = (j - j_low + 1) >> 1;
            i_low = i;
            i += d;
            j -= d;
        } else {
            break;
        }
    }
    return i;
}

// Co-rank over two arrays in global memory, 64-bit indices, keys compared
// in the order ORDER (KeyOrder).
template <int ORDER = 0>
__device__ __forceinline__ int64_t co_rank_global(
    int64_t k, const typename KeyOrder<ORDER>::T* __restrict__ A, int64_t m,
    const typename KeyOrder<ORDER>::T* __restrict__ B, int64_t n) {
    using K = KeyOrder<ORDER>;
    return co_rank<int64_t>(
        k, m, n, [=](int64_t x) { return K::to_ord(A[x]); },
        [=](int64_t x) { return K::to_ord(B[x]); }, kMaxStepsGlobal);
}

}  // namespace omerge
