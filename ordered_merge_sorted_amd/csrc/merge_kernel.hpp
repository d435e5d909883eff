// merge_kernel.hpp -- partition kernel and LDS-ring segment merge kernel.
//
// Decomposition (page "Tiled and Circular Buffer Merge Kernel",
// pmpp.huatsai.dev/12-merge/03):
//   * The output rank space 0..m+n is cut into segments of seg_len outputs.
//     The partition kernel writes the co-rank of every segment boundary
//     ("Block-Level Co-Rank": one search per block, not per thread).
//   * One workgroup merges one segment.  It walks the segment in tiles of
//     TILE = THREADS*ITEMS outputs.  A and B stream through two circular
//     buffers in LDS; after each tile only the consumed part of each buffer
//     is refilled ("Circular Buffer Merge Kernel"), so every input element
//     is read from HBM once (the non-circular tiled kernel reloads half of
//     what it loads: section "The Half-Bandwidth Deficiency").
//   * Inside a tile each lane finds its split by a co-rank search in LDS,
//     merges ITEMS outputs in registers (the sequential two-pointer merge),
//     and the tile goes back to HBM as coalesced 16-byte stores, from
//     registers or through an LDS stage.
//
// Elements.  Keys are 32- or 64-bit (KW = 1 or 2 words) and payloads 0, 1 or
// 2 words (VW).  Rings, refills, stages and stores move 32-bit words;
// searches and merges read whole elements.  Keys are held in LDS as their
// order images (KeyOrder, corank.hpp), so every key type and direction is a
// signed-integer merge; payloads are opaque words.
//
// gfx950 choices (none of these is on the pages):
//   * Ring slot of a word = its absolute word address (address/4) modulo the
//     power-of-two ring capacity.  A 16-byte-aligned vector in HBM then lands
//     on a 16-byte-aligned slot quad, so refills are global_load_dwordx4 +
//     ds_write_b128 with no wrap inside a vector, and 8-byte-aligned 64-bit
//     elements land on even slots.  Partial vectors at the two ends of a
//     refill are loaded one element at a time (never past the range, so
//     never past the array).
//   * The refill for tile t+1 is issued into registers as soon as tile t's
//     split is known, before tile t is merged, and written to LDS only after
//     every lane has read its candidates and before the tile's stores; the
//     HBM latency hides behind the merge.
//   * Each lane searches the END of its slice; its start is the previous
//     slice's end, read from a small LDS array, and the last slice's end is
//     the tile's split.  One search per lane per tile.  Inside a tile the
//     search is a fixed-trip, branchless bisection of the merge diagonal
//     (one probe pair per step) within the same bounds as the pages' search;
//     it returns the same unique co-rank with about a third of the
//     instructions of the two-test loop.
//   * Key-only merges order a lane's ITEMS outputs with a min/max bitonic
//     network instead of the serial two-pointer loop.  The co-ranks already
//     fix which elements belong to each lane (A first on ties); inside a lane
//     equal keys are indistinguishable in a key-only output, so any exact
//     ordering of the lane's keys is bit-identical to the stable merge.  The
//     network has no LDS round trip per output and no branches.  Key+payload
//     merges keep the serial loop, where the tie order is visible.
//   * Tiles whose outputs all come from one side are stored straight from
//     that side's ring window: no search, no network, no stage.
//   * Each key ring has a guard zone that mirrors its first ITEMS elements
//     past its end, so a lane reads its ITEMS candidates at one base address
//     with immediate offsets and no wrap arithmetic.
//   * Merges and sort passes of 4-byte keys (alone or with 4-byte payloads)
//     into 16-byte-aligned outputs store from registers: the lanes of a
//     wavefront take its 64 slices in the order 0,32,1,33,..., so one DPP
//     swap inside each lane pair gives every lane two 16-byte pieces of two
//     1 KB runs of the output (store_direct8).  With no stage a 4-byte-key
//     workgroup needs 17 KB of LDS instead of 26 KB, and 8 workgroups share
//     a CU instead of 6: a third more refill loads in flight.  8-byte keys
//     alone do the same with a transpose inside each lane quad
//     (store_direct16).
//   * The other shapes, unaligned outputs and batches go through an LDS stage
//     padded by 4 words every 32, which makes the 16-byte stage writes
//     (lane-contiguous) and 16-byte stage reads (for the coalesced stores)
//     free of bank conflicts.
//   * The partition kernel can search each boundary with a group of G lanes:
//     G points of the diagonal are tested at once and a ballot narrows the
//     interval to one of the G+1 gaps per round (the pages note the search
//     may be higher-radix).  After the first round the points are placed by
//     interpolation on the keys at the interval's ends (co_rank_group), so
//     evenly spread keys need about 5 rounds instead of 12.  G is a tuning
//     choice of the launcher.
//   * A descriptor mode lets the same kernel merge any list of (A, B, C)
//     ranges: the pieces of a batch of merges or of a merge-sort pass
//     (batch_kernel.hpp).
//   * All arithmetic is integer compares and index arithmetic; no MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "corank.hpp"

namespace omerge {

typedef int int4v __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Number of bits of x: the steps a bisection of x+1 candidates needs.
__host__ __device__ constexpr int bit_length(int x) {
    int b = 0;
    while (x > 0) {
        x >>= 1;
        ++b;
    }
    return b;
}

template <typename T>
__device__ __forceinline__ T clamp_to(T x, T lo, T hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

// Element-address phase: (address / 4) of p, as an int (only low bits used).
__device__ __forceinline__ int word_phase(const void* p) {
    return static_cast<int>(reinterpret_cast<uintptr_t>(p) >> 2);
}

// Tile geometry and LDS layout.  Elements are KW 32-bit words of key (1 or
// 2) and VW words of payload (0 = keys only, 1 or 2); rings, stages and
// refills work in 32-bit words, searches and merges in elements.
template <int THREADS, int ITEMS, int KW, int VW, bool STAGE = true>
struct MergeCfg {
    static_assert(THREADS % 64 == 0, "whole 64-lane wavefronts");
    static_assert(ITEMS >= 4 && (ITEMS & (ITEMS - 1)) == 0,
                  "ITEMS: a power of two, at least one 16-byte vector");
    static_assert(KW == 1 || KW == 2, "32- or 64-bit keys");
    static_assert(VW >= 0 && VW <= 2, "no payload, or a 32- or 64-bit one");
    static_assert(ITEMS * KW <= 32 || (ITEMS * KW) % 32 == 0, "lane-contiguous stage rows");
    static_assert(VW == 0 || ITEMS * VW <= 32 || (ITEMS * VW) % 32 == 0,
                  "lane-contiguous stage rows");
    static constexpr bool kKV = VW > 0;
    static constexpr int kTile = THREADS * ITEMS;       // outputs per tile
    static constexpr int kCap = next_pow2(kTile * KW);  // key ring words per side
    static constexpr int kMask = kCap - 1;
    static constexpr int kGuard = ITEMS * KW;           // mirrored words past the end
    static constexpr int kSide = kCap + kGuard;         // words per key side ring
    static constexpr int kVCap = VW ? next_pow2(kTile * VW) : 1;  // payload ring words
    static constexpr int kVMask = kVCap - 1;
    static constexpr int kVSide = VW ? kVCap : 0;       // payload rings need no guard
    // Output stage (none when the lanes store their outputs from registers).
    static constexpr int kStageWords = STAGE ? kTile * KW + kTile * KW / 8 : 0;
    static constexpr int kVStageWords = STAGE ? kTile * VW + kTile * VW / 8 : 0;
    // LDS layout in 32-bit words.
    static constexpr int kRing = 0;  // keys: A ring [0,kSide), B ring [kSide,2kSide)
    static constexpr int kValRing = kRing + 2 * kSide;  // payload rings
    static constexpr int kStage = kValRing + 2 * kVSide;
    static constexpr int kValStage = kStage + kStageWords;
    static constexpr int kSplit = kValStage + kVStageWords;
    static constexpr int kWords = kSplit + THREADS;
    static constexpr int kLdsBytes = kWords * 4;
};

// Global 16-byte accesses for streaming data.  By default they carry the
// nontemporal hint: every input is read once and every output written once,
// and on MI355X the hint raises a plain 16-byte copy from ~5.7 to ~6.2 TB/s
// and the merge by ~4%.  Building with OMERGE_NT_LOADS=0 / OMERGE_NT_STORES=0
// gives plain accesses.
#ifndef OMERGE_NT_LOADS
#define OMERGE_NT_LOADS 1
#endif
#ifndef OMERGE_NT_STORES
#define OMERGE_NT_STORES 1
#endif
__device__ __forceinline__ int4v load_stream4(const int32_t* p) {
    const int4v* q = reinterpret_cast<const int4v*>(p);
    return OMERGE_NT_LOADS ? __builtin_nontemporal_load(q) : *q;
}
__device__ __forceinline__ void store_stream4(int32_t* p, int4v x) {
    int4v* q = reinterpret_cast<int4v*>(p);
    if (OMERGE_NT_STORES)
        __builtin_nontemporal_store(x, q);
    else
        *q = x;
}

// Stage word of tile output p: 4 spare words after every 32.
__host__ __device__ constexpr int stage_word(int p) { return p + ((p >> 5) << 2); }

// ---------------------------------------------------------------------------
// Partition and co-rank query kernels.

// Co-rank of k over global memory by a group of G lanes (G divides 64;
// `g_lane` = 0..G-1 within the group, `g_shift` = the group's first lane in
// the wavefront).  Each round tests G points of [lo, hi) on the diagonal.  A
// point i passes when A[i] <= B[k-1-i], i.e. A[i] is among the first k
// outputs; the passing points form a prefix, so the answer lies just after
// the last passing point and at or before the first failing one.  Every
// round keeps max(0,k-n) <= lo <= hi <= min(k,m) and shrinks the interval,
// whatever the data, so the loop ends even on unsorted input.  All lanes of
// the wavefront must call this together (the votes and shuffles are
// wavefront-wide).
//
// Where the points go.  The first round splits [lo, hi) evenly.  After that
// the group knows g = image(A[i]) - image(B[k-1-i]) at both ends of the
// interval (g <= 0 at the last passing point, g >= 1 at the first failing
// one; g rises with i), and places the points around the linear
// interpolation of where g crosses 1/2, spread by the larger of
// 0.7*sqrt(width) (how far the crossing of evenly spread keys strays from
// the line) and half the width of one unit of key image.  On keys spread
// evenly over their range this takes about 5 rounds instead of 12 for
// 2^28+2^28 elements.  An interpolated round that narrows the interval less
// than an even split would (G+1 times) turns interpolation off for the rest
// of the search, so clustered or heavily tied keys cost at most about one
// round more than even splits.  Only the points change: the interval update
// is the same, so the result is the co-rank whatever the placement.
#ifndef OMERGE_PART_INTERP
#define OMERGE_PART_INTERP 1
#endif
//
// A caller that knows more may pass a narrower interval [lo_in, hi_in] that
// holds the answer (it is intersected with the bounds above) and a guess of
// the answer inside it; the first round then places its points around the
// guess, spread by 0.7*sqrt(width), unless that would cover more than half
// the interval.  A first round that misses does not turn interpolation off.
template <int G, int ORDER>
__device__ __forceinline__ int64_t co_rank_group(int64_t k,
                                                 const typename KeyOrder<ORDER>::T* __restrict__ A,
                                                 int64_t m,
                                                 const typename KeyOrder<ORDER>::T* __restrict__ B,
                                                 int64_t n, int g_lane, int g_shift,
                                                 int64_t lo_in = 0, int64_t hi_in = INT64_MAX,
                                                 double guess = -1.0) {
    static_assert(G >= 2 && G <= 64 && (64 % G) == 0, "group size");
    constexpr int kLog = bit_length(G) - 1;
    int64_t lo = k > n ? k - n : 0;
    int64_t hi = k < m ? k : m;
    lo = lo_in > lo ? (lo_in < hi ? lo_in : hi) : lo;
    hi = hi_in < hi ? (hi_in > lo ? hi_in : lo) : hi;
    // g at the interval's ends once known: at lo - 1 (last passing point)
    // and at hi (first failing point).
    double g_lo = 0.0, g_hi = 0.0;
    bool have_lo = false, have_hi = false;
    bool even_only = !OMERGE_PART_INTERP;
    for (int round = 0; round < 64; ++round) {
        if (__ballot(lo < hi) == 0) break;  // every group of the wavefront is done
        const int64_t span = hi - lo;
        double centre = 0.0, spread = 0.0;
        bool interp = false;
        if (round == 0 && guess >= 0.0 && OMERGE_PART_INTERP) {
            centre = guess;
            spread = fmax(1.0, 0.7 * sqrt(static_cast<double>(span)));
            interp = (G - 1) * spread < 0.5 * static_cast<double>(span);
        } else if (!even_only && have_lo && have_hi && g_hi > g_lo) {
            const double w = static_cast<double>(span + 1);  // from lo - 1 to hi
            const double unit = w / (g_hi - g_lo);           // outputs per unit of image
            centre = static_cast<double>(lo - 1) + (0.5 - g_lo) * unit;
            spread = fmax(1.0, fmax(0.7 * sqrt(w), 0.5 * unit));
            interp = (G - 1) * spread < 0.5 * static_cast<double>(span);
        }
        const int64_t q = span >> kLog, r = span & (G - 1);
        const int live = interp || span >= G ? G : static_cast<int>(span);
        // l-th point: lo + floor(span*l/G) for long intervals, lo + l for
        // short; or centre + spread*(l - (G-1)/2), clamped into [lo, hi-1]
        // (in double first, so that the conversion stays in range; then
        // exactly, against rounding).
        const double dlo = static_cast<double>(lo), dhi = static_cast<double>(hi - 1);
        auto point = [=](int l) -> int64_t {
            if (interp) {
                const double p = rint(centre + spread * (0.5 * (2 * l - (G - 1))));
                const int64_t i = static_cast<int64_t>(fmin(fmax(p, dlo), dhi));
                return i < lo ? lo : (i > hi - 1 ? hi - 1 : i);
            }
            return span < G ? lo + l : lo + q * l + ((r * l) >> kLog);
        };
        const int64_t p = point(g_lane);
        bool pass = false;
        double g = 0.0;
        if (g_lane < live) {
            const auto a = KeyOrder<ORDER>::to_ord(A[p]);
            const auto b = KeyOrder<ORDER>::to_ord(B[k - 1 - p]);
            pass = a <= b;
            g = static_cast<double>(a) - static_cast<double>(b);
        }
        const unsigned long long votes = __ballot(pass);
        const unsigned long long mine =
            G == 64 ? votes : (votes >> g_shift) & ((1ull << (G == 64 ? 0 : G)) - 1);
        const int c = __popcll(mine);
        const double g_left = __shfl(g, g_shift + (c > 0 ? c - 1 : 0));
        const double g_right = __shfl(g, g_shift + (c < live ? c : 0));
        if (lo < hi) {
            const int64_t new_lo = c > 0 ? point(c - 1) + 1 : lo;
            const int64_t new_hi = c < live ? point(c) : hi;
            if (c > 0) {
                g_lo = g_left;
                have_lo = true;
            }
            if (c < live) {
                g_hi = g_right;
                have_hi = true;
            }
            if (interp && round > 0 && (new_hi - new_lo) * (G + 1) > span) even_only = true;
            lo = new_lo;
            hi = new_hi;
        }
    }
    return lo;
}

// part[s] = co-rank of k_s = min(s*seg_len, m+n).  G = 1: one lane per
// boundary running the pages' two-test search.  G > 1: a workgroup of 256
// lanes holds 256/G consecutive boundaries, one G-lane group each, in two
// phases.  Phase 1 searches every kStride-th boundary (and the first of the
// next workgroup) over the whole diagonal.  Phase 2 searches the others
// inside the interval their two searched neighbours c0 < s < c1 allow: the
// co-rank never falls as k grows and grows by at most one per output, so
// max(i(c0), i(c1) - (k_c1 - k)) <= i(k) <= min(i(c1), i(c0) + (k - k_c0)),
// with the first probes around the straight line between the neighbours.
// Boundaries close together share their expensive first rounds this way.
// STRIDE is kStride (capped at 256/G); phase 2 may use G2 <= G lanes per
// boundary.  Fewer phase-1 searches fetch fewer random lines, while wider
// phase-2 gaps take more rounds: on 4,096-output segments a stride of 16
// measured marginally fastest (2^28+2^28 uniform keys: 40.0 us and 210 MB
// of reads against 40.7 us and 215 MB at 8; no gain at 32 or 64), and
// 2-lane phase-2 groups were slower.
template <int G, int ORDER, int G2 = G, int STRIDE = 8>
__global__ __launch_bounds__(256) void partition_kernel(
    const typename KeyOrder<ORDER>::T* __restrict__ A, int64_t m,
    const typename KeyOrder<ORDER>::T* __restrict__ B, int64_t n, int64_t seg_len, int64_t count,
    int64_t* __restrict__ part) {
    if constexpr (G == 1) {
        const int64_t gid = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
        if (gid >= count) return;
        const int64_t k = gid < count - 1 ? gid * seg_len : m + n;
        part[gid] = co_rank_global<ORDER>(k, A, m, B, n);
    } else {
        constexpr int kGroups = 256 / G;  // boundaries per workgroup
        constexpr int kStride = kGroups >= STRIDE ? STRIDE : kGroups;
        // Phase 2 searches each boundary with G2 lanes (G2 <= G), so its
        // groups fill the first kGroups*G2 lanes: whole wavefronts.
        static_assert(G2 >= 2 && G2 <= G && (kGroups * G2) % 64 == 0, "phase-2 group size");
        constexpr int kCoarse = kGroups / kStride + 1;
        constexpr int kPhase1Lanes = (kCoarse * G + 63) / 64 * 64;  // whole wavefronts
        __shared__ int64_t coarse[kCoarse];
        const int tid = threadIdx.x;
        const int grp = tid / G;
        const int g_lane = tid % G;
        const int g_shift = (tid & 63) - g_lane;
        const int64_t s0 = blockIdx.x * static_cast<int64_t>(kGroups);
        auto k_of = [&](int64_t s) { return s < count - 1 ? s * seg_len : m + n; };
        auto coarse_index = [&](int j) {
            const int64_t s = s0 + static_cast<int64_t>(kStride) * j;
            return s < count - 1 ? s : count - 1;
        };
        // Phase 1.  Groups past kCoarse (or of a wavefront past the whole
        // grid) vote with empty ranges.
        if (tid < kPhase1Lanes) {
            const bool act = grp < kCoarse;
            const int64_t kc = act ? k_of(coarse_index(grp)) : 0;
            const int64_t ic = co_rank_group<G, ORDER>(kc, A, act ? m : 0, B, act ? n : 0, g_lane,
                                                       g_shift);
            if (act && g_lane == 0) coarse[grp] = ic;
        }
        __syncthreads();
        // Phase 2.  Wavefronts past the phase-2 lanes, and a wavefront whose
        // groups are all past the end, leave together; groups past the end
        // inside a live wavefront, and the boundaries phase 1 has found,
        // vote with empty ranges.
        if (tid >= kGroups * G2) return;
        const int grp2 = tid / G2;
        const int g_lane2 = tid % G2;
        const int g_shift2 = (tid & 63) - g_lane2;
        const int64_t s = s0 + grp2;
        if (s0 + (tid & ~63) / G2 >= count) return;
        const bool live = s < count;
        const int j = grp2 / kStride;
        const bool known = grp2 % kStride == 0;
        int64_t i;
        if (live && !known) {
            const int64_t c0 = coarse_index(j), c1 = coarse_index(j + 1);
            const int64_t k = k_of(s), k0 = k_of(c0), k1 = k_of(c1);
            const int64_t i0 = coarse[j], i1 = coarse[j + 1];
            const int64_t lo = i1 - (k1 - k) > i0 ? i1 - (k1 - k) : i0;
            const int64_t hi = i0 + (k - k0) < i1 ? i0 + (k - k0) : i1;
            const double guess =
                k1 > k0 ? static_cast<double>(i0) + static_cast<double>(i1 - i0) *
                                                        static_cast<double>(k - k0) /
                                                        static_cast<double>(k1 - k0)
                        : -1.0;
            i = co_rank_group<G2, ORDER>(k, A, m, B, n, g_lane2, g_shift2, lo, hi,
                                         guess >= static_cast<double>(lo) ? guess : -1.0);
        } else {
            i = co_rank_group<G2, ORDER>(0, A, 0, B, 0, g_lane2, g_shift2);
            if (live) i = coarse[j];
        }
        if (live && g_lane2 == 0) part[s] = i;
    }
}

// Co-rank at arbitrary ranks, one lane per query, with the pages' two-test
// search (corank.hpp).
template <int ORDER>
__global__ void co_rank_kernel(const typename KeyOrder<ORDER>::T* __restrict__ A, int64_t m,
                               const typename KeyOrder<ORDER>::T* __restrict__ B, int64_t n,
                               const int64_t* __restrict__ ks, int64_t count,
                               int64_t* __restrict__ out) {
    const int64_t s = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
    if (s >= count) return;
    const int64_t k = clamp_to<int64_t>(ks[s], 0, m + n);
    out[s] = co_rank_global<ORDER>(k, A, m, B, n);
}

// Global-memory merge, no LDS: one lane per slice of `per` outputs
// [k0, k1).  With two_searches the lane finds the co-ranks of both ends and
// merges exactly its two sub-arrays (the basic kernel of page "Co-rank
// Function ... and Basic Parallel Merge Kernel"); otherwise it finds the
// co-rank of k0 only and walks k1-k0 steps of the two-pointer merge with the
// whole arrays' bounds (the co-rank kernel of page "merge_path.cu").  Every
// read and write goes to HBM directly, lane-strided: this is the pattern the
// pages' coalescing critique describes, kept as a measured ablation.
__global__ __launch_bounds__(256) void direct_merge_kernel(const int32_t* __restrict__ A, int64_t m,
                                                           const int32_t* __restrict__ B, int64_t n,
                                                           int32_t* __restrict__ C, int64_t per,
                                                           int two_searches) {
    const int64_t t = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
    const int64_t total = m + n;
    const int64_t k0 = t * per;
    if (k0 >= total) return;
    const int64_t k1 = k0 + per < total ? k0 + per : total;
    int64_t a = co_rank_global(k0, A, m, B, n);
    int64_t b = k0 - a;
    int64_t a_end = m, b_end = n;
    if (two_searches) {
        a_end = co_rank_global(k1, A, m, B, n);
        b_end = k1 - a_end;
    }
    for (int64_t k = k0; k < k1; ++k) {
        const bool take_a = a < a_end && (b >= b_end || A[a] <= B[b]);
        if (take_a) {
            C[k] = A[a];
            ++a;
        } else {
            C[k] = B[b];
            ++b;
        }
    }
}

// Bandwidth reference: each lane copies UNROLL 16-byte vectors, all loads
// issued before the stores; single words at the two ends.
template <int UNROLL>
__global__ __launch_bounds__(256) void stream_copy_kernel(const int32_t* __restrict__ src,
                                                          int64_t n, int32_t* __restrict__ dst) {
    const int64_t lane = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
    const int head0 = (4 - (word_phase(dst) & 3)) & 3;
    const int64_t head = head0 < n ? head0 : n;
    const bool same_phase = ((word_phase(src) - word_phase(dst)) & 3) == 0;
    if (same_phase) {
        const int64_t nvec = (n - head) >> 2;
        const int64_t first = blockIdx.x * static_cast<int64_t>(blockDim.x) * UNROLL + threadIdx.x;
        int4v v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t q = first + u * static_cast<int64_t>(blockDim.x);
            if (q < nvec) v[u] = load_stream4(src + head + 4 * q);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t q = first + u * static_cast<int64_t>(blockDim.x);
            if (q < nvec) store_stream4(dst + head + 4 * q, v[u]);
        }
        if (lane < head) dst[lane] = src[lane];
        const int64_t done = head + 4 * nvec;
        if (lane < n - done) dst[done + lane] = src[done + lane];
    } else {
        for (int u = 0; u < 4 * UNROLL; ++u) {
            const int64_t p = (lane / 64) * 64 * 4 * UNROLL + u * 64 + (lane & 63);
            if (p < n) dst[p] = src[p];
        }
    }
}

// ---------------------------------------------------------------------------
// Element maps.  Keys enter the rings as their order images
// (KeyOrder<ORDER>::to_ord) and leave through from_ord; payloads use an
// identity order of their width.  A 16-byte vector holds 4/W elements of W
// words: arrays of 64-bit elements are 8-byte aligned, so a 16-byte-aligned
// vector (and every ring or stage quad) starts on an element.

__device__ __forceinline__ long long join_words(int lo, int hi) {
    return static_cast<long long>((static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) |
                                  static_cast<unsigned>(lo));
}
__device__ __forceinline__ int low_word(long long x) { return static_cast<int>(x); }
__device__ __forceinline__ int high_word(long long x) { return static_cast<int>(x >> 32); }

template <int ORDER, bool TO>
__device__ __forceinline__ typename KeyOrder<ORDER>::T map_elem(typename KeyOrder<ORDER>::T x) {
    return TO ? KeyOrder<ORDER>::to_ord(x) : KeyOrder<ORDER>::from_ord(x);
}

template <int ORDER, bool TO>
__device__ __forceinline__ int4v map_vec(int4v x) {
    if constexpr (KeyOrder<ORDER>::kWords == 1) {
        x.x = map_elem<ORDER, TO>(x.x);
        x.y = map_elem<ORDER, TO>(x.y);
        x.z = map_elem<ORDER, TO>(x.z);
        x.w = map_elem<ORDER, TO>(x.w);
    } else {
        const long long e0 = map_elem<ORDER, TO>(join_words(x.x, x.y));
        const long long e1 = map_elem<ORDER, TO>(join_words(x.z, x.w));
        x.x = low_word(e0);
        x.y = high_word(e0);
        x.z = low_word(e1);
        x.w = high_word(e1);
    }
    return x;
}

// One element of type T at word `w` of an LDS or global word array.
template <typename T>
__device__ __forceinline__ T ld_elem(const int* base, int w) {
    return *reinterpret_cast<const T*>(base + w);
}
template <typename T>
__device__ __forceinline__ void st_elem(int* base, int w, T x) {
    *reinterpret_cast<T*>(base + w) = x;
}

// ---------------------------------------------------------------------------
// Ring refill: copies a segment-relative word range [r0, r1) of one side
// into its ring.  Issue and commit are split so the loads can be in flight
// while the current tile is merged.  The NL loading lanes share one
// assignment of the body vectors of side A then side B, so a refill of at
// most TILE elements needs V = TILE*W/(4*NL) vectors per lane.  The partial
// vectors at the two ends of a side (up to 3 words each: 3 elements of one
// word, or 1 element of two) are loaded one element at a time by loading
// lanes 0..11.  Slots below the guard size are also written to their mirror
// past the ring's end.

struct SideRange {
    const int32_t* src;  // segment base of this array in global memory (words)
    int base;            // ring slot of segment-relative word 0
    int r0;              // first segment-relative word to load
    int head;            // words before the first 16-byte boundary
    int nvec;            // whole 16-byte vectors
    int tail;            // words after the last whole vector

    __device__ __forceinline__ void set(const int32_t* s, int b, int lo, int hi) {
        src = s;
        base = b;
        r0 = lo;
        const int len = hi > lo ? hi - lo : 0;
        const int h = (4 - ((word_phase(s) + lo) & 3)) & 3;
        head = h < len ? h : len;
        nvec = (len - head) >> 2;
        tail = (len - head) & 3;
    }
};

template <int NL, int V, int CAP, int SIDE, int ORDER>
struct Refill {
    using T = typename KeyOrder<ORDER>::T;  // one element (W words)
    static constexpr int W = KeyOrder<ORDER>::kWords;
    static constexpr int kVec = V;
    static constexpr int kMask = CAP - 1;
    static constexpr int kGuard = SIDE - CAP;
    int4v body[kVec];
    T loose;          // one head/tail element (lanes 0..11)
    int loose_slot;   // its first ring word, or -1
    int loose_side;   // 0 = A ring, 1 = B ring
    SideRange sa, sb;

    __device__ __forceinline__ void issue(const SideRange& a, const SideRange& b, int tid) {
        sa = a;
        sb = b;
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
            const int q = tid + v * NL;
            if (q < sa.nvec) {
                body[v] = load_stream4(sa.src + sa.r0 + sa.head + 4 * q);
            } else if (q - sa.nvec < sb.nvec) {
                const int qb = q - sa.nvec;
                body[v] = load_stream4(sb.src + sb.r0 + sb.head + 4 * qb);
            }
        }
        loose_slot = -1;
        if (tid < 12) {
            const SideRange& s = tid < 6 ? sa : sb;
            const int w = tid < 6 ? tid : tid - 6;
            int r = -1;  // first word of this lane's element
            if (w < 3) {
                if (W * (w + 1) <= s.head) r = s.r0 + W * w;
            } else if (W * (w - 2) <= s.tail) {
                r = s.r0 + s.head + 4 * s.nvec + W * (w - 3);
            }
            if (r >= 0) {
                loose = ld_elem<T>(s.src, r);
                loose_slot = (s.base + r) & kMask;
                loose_side = tid < 6 ? 0 : 1;
            }
        }
    }

    __device__ __forceinline__ static void put4(int* side, int slot, int4v x) {
        *reinterpret_cast<int4v*>(side + slot) = x;
        if (slot < kGuard) *reinterpret_cast<int4v*>(side + CAP + slot) = x;
    }

    // ring points at the A ring; the B ring starts SIDE words later.
    __device__ __forceinline__ void commit(int* ring, int tid) const {
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
            const int q = tid + v * NL;
            const int4v x = map_vec<ORDER, true>(body[v]);
            if (q < sa.nvec) {
                put4(ring, (sa.base + sa.r0 + sa.head + 4 * q) & kMask, x);
            } else if (q - sa.nvec < sb.nvec) {
                const int qb = q - sa.nvec;
                put4(ring + SIDE, (sb.base + sb.r0 + sb.head + 4 * qb) & kMask, x);
            }
        }
        if (loose_slot >= 0) {
            int* side = ring + (loose_side ? SIDE : 0);
            const T y = map_elem<ORDER, true>(loose);
            st_elem<T>(side, loose_slot, y);
            if (loose_slot < kGuard) st_elem<T>(side, CAP + loose_slot, y);
        }
    }
};

// Co-rank of diagonal k inside one tile: A window of wa elements starting at
// ring word sa, B window of wb elements at word sb, W words per key.  Bisects
// [max(0,k-wb), min(k,wa)] for the first i at which A[i] is not among the
// first k outputs (A[i] <= B[k-1-i] fails).  STEPS = bit_length of a bound
// on the interval's width covers it; finished lanes idle through the
// remaining steps, so the loop has no data-dependent exit.  (Binary lifting,
// with fewer instructions per step, measured slower here: its first probes
// sit at the lanes' interval ends, eight words apart, and conflict in the
// LDS banks.)
template <int STEPS, int MASK, typename T>
__device__ __forceinline__ int co_rank_tile(int k, int wa, int wb, const int* ring_a, int sa,
                                            const int* ring_b, int sb) {
    constexpr int W = sizeof(T) / 4;
    int lo = k > wb ? k - wb : 0;
    int hi = k < wa ? k : wa;
#pragma unroll
    for (int step = 0; step < STEPS; ++step) {
        const int mid = (lo + hi) >> 1;
        const T av = ld_elem<T>(ring_a, (sa + W * mid) & MASK);
        const T bv = ld_elem<T>(ring_b, (sb + W * (k - 1 - mid)) & MASK);
        const bool live = lo < hi;
        const bool a_first = av <= bv;
        lo = (live && a_first) ? mid + 1 : lo;
        hi = (live && !a_first) ? mid : hi;
    }
    return lo;
}

// Orders x[0..N) ascending when x is bitonic (min/max network).
template <int N, typename T>
__device__ __forceinline__ void bitonic_clean(T (&x)[N]) {
#pragma unroll
    for (int d = N / 2; d >= 1; d >>= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if ((i & d) == 0) {
                const T lo = min(x[i], x[i + d]);
                const T hi = max(x[i], x[i + d]);
                x[i] = lo;
                x[i + d] = hi;
            }
        }
    }
}

// Stores tile output words [0, len) from the padded LDS stage to dst[0, len)
// with NS storing lanes (`tid` = 0..NS-1), V 16-byte vectors per lane at
// most: 16-byte stores on the aligned body, single elements at the ends.
// Elements leave through KeyOrder<ORDER>::from_ord.
template <int NS, int V, int ORDER>
__device__ __forceinline__ void store_tile(int32_t* __restrict__ dst, int len,
                                           const int* stage, int tid) {
    using T = typename KeyOrder<ORDER>::T;
    constexpr int W = KeyOrder<ORDER>::kWords;
    const int head0 = (4 - (word_phase(dst) & 3)) & 3;
    const int head = head0 < len ? head0 : len;
    const int nvec = (len - head) >> 2;
    const int tail = (len - head) & 3;
    if (head == 0) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int q = tid + v * NS;
            if (q < nvec) {
                const int p = 4 * q;
                const int4v x = *reinterpret_cast<const int4v*>(stage + stage_word(p));
                store_stream4(dst + p, map_vec<ORDER, false>(x));
            }
        }
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int q = tid + v * NS;
            if (q < nvec) {
                const int p = head + 4 * q;
                int4v x;
                x.x = stage[stage_word(p)];
                x.y = stage[stage_word(p + 1)];
                x.z = stage[stage_word(p + 2)];
                x.w = stage[stage_word(p + 3)];
                store_stream4(dst + p, map_vec<ORDER, false>(x));
            }
        }
        if (W * tid < head) {
            int* const d = reinterpret_cast<int*>(dst);
            st_elem<T>(d, W * tid, map_elem<ORDER, false>(ld_elem<T>(stage, stage_word(W * tid))));
        }
    }
    if (tid >= 4 && W * (tid - 3) <= tail) {
        const int p = head + 4 * nvec + W * (tid - 4);
        int* const d = reinterpret_cast<int*>(dst);
        st_elem<T>(d, p, map_elem<ORDER, false>(ld_elem<T>(stage, stage_word(p))));
    }
}

// Stores a one-sided tile straight from a ring window: output word p is the
// window's word p, at ring slot (start + p) & MASK.  Consecutive lanes read
// consecutive slots (no bank conflicts); 16-byte reads when the ring quads
// line up with the output's 16-byte vectors, single words otherwise.
template <int THREADS, int V, int MASK, int ORDER>
__device__ __forceinline__ void store_from_ring(int32_t* __restrict__ dst, int len,
                                                const int* side, int start, int tid) {
    using T = typename KeyOrder<ORDER>::T;
    constexpr int W = KeyOrder<ORDER>::kWords;
    const int head0 = (4 - (word_phase(dst) & 3)) & 3;
    const int head = head0 < len ? head0 : len;
    const int nvec = (len - head) >> 2;
    const int tail = (len - head) & 3;
    const bool quads = ((start + head) & 3) == 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int q = tid + v * THREADS;
        if (q < nvec) {
            const int p = head + 4 * q;
            int4v x;
            if (quads) {
                x = *reinterpret_cast<const int4v*>(side + ((start + p) & MASK));
            } else {
                x.x = side[(start + p) & MASK];
                x.y = side[(start + p + 1) & MASK];
                x.z = side[(start + p + 2) & MASK];
                x.w = side[(start + p + 3) & MASK];
            }
            store_stream4(dst + p, map_vec<ORDER, false>(x));
        }
    }
    int* const d = reinterpret_cast<int*>(dst);
    if (W * tid < head)
        st_elem<T>(d, W * tid, map_elem<ORDER, false>(ld_elem<T>(side, (start + W * tid) & MASK)));
    if (tid >= 4 && W * (tid - 3) <= tail) {
        const int p = head + 4 * nvec + W * (tid - 4);
        st_elem<T>(d, p, map_elem<ORDER, false>(ld_elem<T>(side, (start + p) & MASK)));
    }
}

// Stores a tile from registers, for one word per output and 8 outputs per
// lane.  The lanes of a wavefront own its 64 slices of 8 outputs in the
// order lane 2i -> slice i, lane 2i+1 -> slice 32+i (direct_slice).  One swap
// inside each lane pair (DPP) then gives every lane the 4 outputs
// [4l, 4l+4) and [256+4l, 256+4l+4) of the wavefront's 512: two 16-byte
// stores per lane, each wavefront instruction writing 1 KB contiguous.  x
// holds the lane's outputs (order images for keys, mapped back here);
// `base` is the wavefront's first output word in dst, `len` how many of the
// tile's words exist past dst.  16-byte stores need dst 16-byte aligned
// (`aligned`); otherwise, and at the tile's ragged end, single words.
__device__ __forceinline__ int direct_slice(int tid) {
    return (tid & ~63) + ((tid & 63) >> 1) + ((tid & 1) << 5);
}

__device__ __forceinline__ int swap_pair_lanes(int x) {
    return __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
}

template <int ORDER>
__device__ __forceinline__ void store_direct8(int32_t* __restrict__ dst, int base, int len,
                                              bool aligned, const int (&x)[8], int tid) {
    const bool odd = (tid & 1) != 0;
    int z[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) z[t] = swap_pair_lanes(odd ? x[t] : x[4 + t]);
    int4v v[2];
    v[0].x = odd ? z[0] : x[0];
    v[0].y = odd ? z[1] : x[1];
    v[0].z = odd ? z[2] : x[2];
    v[0].w = odd ? z[3] : x[3];
    v[1].x = odd ? x[4] : z[0];
    v[1].y = odd ? x[5] : z[1];
    v[1].z = odd ? x[6] : z[2];
    v[1].w = odd ? x[7] : z[3];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int p = base + 256 * h + 4 * (tid & 63);
        const int4v y = map_vec<ORDER, false>(v[h]);
        if (aligned && p + 4 <= len) {
            store_stream4(dst + p, y);
        } else {
            const int ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (p + u < len) dst[p + u] = ys[u];
        }
    }
}

// The same for two words per output (8-byte keys): a lane's slice is 64
// bytes and the wavefront's output four 1 KB runs.  Lane 4Q+r merges slice
// 16r+Q (direct_slice_wide), so store u (run u) needs the four 16-byte
// quarters of the slice lane 4Q+u holds, one per lane of quad Q: a 4x4
// transpose of 16-byte blocks inside each quad, done as two exchange stages
// (lane pairs 1 apart, then 2 apart) in which each lane sends by DPP the two
// blocks it replaces.  w holds the lane's 8 outputs as 16 words.
__device__ __forceinline__ int direct_slice_wide(int tid) {
    return (tid & ~63) + ((tid & 3) << 4) + ((tid & 63) >> 2);
}

template <int XOR>
__device__ __forceinline__ int swap_quad_lanes(int x) {
    static_assert(XOR == 1 || XOR == 2, "quad exchange");
    return __builtin_amdgcn_update_dpp(x, x, XOR == 1 ? 0xB1 : 0x4E, 0xF, 0xF, false);
}

// One exchange stage: blocks j with (j ^ r) & XOR set (r = lane in quad) go
// to the partner r ^ XOR, which sends back its blocks j ^ XOR into them.
template <int XOR>
__device__ __forceinline__ void quad_exchange(int (&w)[16], int r) {
    const bool hi = (r & XOR) != 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        // The two blocks of this pair of positions: lo has bit XOR clear.
        const int lo = XOR == 1 ? 2 * k : k;
        const int hib = lo + XOR;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int a = w[4 * lo + u];
            const int b = w[4 * hib + u];
            const int recv = swap_quad_lanes<XOR>(hi ? a : b);
            w[4 * lo + u] = hi ? recv : a;
            w[4 * hib + u] = hi ? b : recv;
        }
    }
}

template <int ORDER>
__device__ __forceinline__ void store_direct16(int32_t* __restrict__ dst, int base, int len,
                                               bool aligned, int (&w)[16], int tid) {
    const int r = tid & 3;
    quad_exchange<1>(w, r);
    quad_exchange<2>(w, r);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int p = base + 256 * h + 4 * (tid & 63);
        int4v v;
        v.x = w[4 * h];
        v.y = w[4 * h + 1];
        v.z = w[4 * h + 2];
        v.w = w[4 * h + 3];
        const int4v y = map_vec<ORDER, false>(v);
        if (aligned && p + 4 <= len) {
            store_stream4(dst + p, y);
        } else {
            if (p < len) dst[p] = y.x;
            if (p + 1 < len) dst[p + 1] = y.y;
            if (p + 2 < len) dst[p + 2] = y.z;
            if (p + 3 < len) dst[p + 3] = y.w;
        }
    }
}

// ---------------------------------------------------------------------------
// Segment merge kernel: one workgroup per segment of the output.
//
// Keys are typed by ORDER (KeyOrder<ORDER>::T, 1 or 2 words); payloads are
// VW words per element (0 = keys only), passed as word arrays.

// DESC = false: segment s is outputs [s*seg_len, (s+1)*seg_len) of one merge
// of A and B, its A range given by the partition (part[s], part[s+1]).
// DESC = true: segment s is described by desc[s] (any ranges of A, B and C,
// e.g. one piece of one merge of a batch, or of one merge-sort pass in which
// A and B are the same array); seg_len bounds its length and C holds c_total
// elements.
struct SegDesc {
    int64_t a0, b0, c0;  // first A, B and C element
    int64_t a1, b1;      // one past the last A and B element
};

// REG = true: tiles leave from registers (store_direct8, store_direct16)
// instead of through the LDS stage; 4-byte keys with no or 4-byte payloads,
// or 8-byte keys alone, and 8 outputs per lane only.  Any output works, but only 16-byte-aligned segment outputs
// get 16-byte stores, so the launcher picks it when they are.
//
// SELF = true (with DESC = false): part is not read; the workgroup finds the
// co-ranks of its own two boundaries first (the pages' block-level co-rank
// done by the block itself), with two 4-lane group searches in its first
// wavefront.  The search's dependent rounds then lengthen every
// workgroup's life, which costs more than a partition kernel once the
// workgroups run in several waves; a grid that fits the device in one wave
// saves the partition's launch and its array instead.
template <int THREADS, int ITEMS, int VW, int ORDER, bool DESC = false, bool REG = false,
          bool SELF = false>
__global__ __launch_bounds__(THREADS) void merge_segments_kernel(
    const typename KeyOrder<ORDER>::T* __restrict__ A, const uint32_t* __restrict__ Av, int64_t m,
    const typename KeyOrder<ORDER>::T* __restrict__ B, const uint32_t* __restrict__ Bv, int64_t n,
    const int64_t* __restrict__ part, int64_t seg_len,
    typename KeyOrder<ORDER>::T* __restrict__ C, uint32_t* __restrict__ Cv,
    const SegDesc* __restrict__ desc, int64_t c_total) {
    static_assert(!(SELF && DESC), "a workgroup searches its boundaries only in partition mode");
    using Key = typename KeyOrder<ORDER>::T;
    constexpr int KW = KeyOrder<ORDER>::kWords;
    constexpr bool KV = VW > 0;
    // Payloads move through rings and stage as opaque words: an identity
    // order of the payload's width.
    constexpr int VORDER = VW == 2 ? kKeyI64 : kKeyI32;
    // With REG each tile is stored from registers (store_direct8) and there
    // is no LDS stage: the LDS saved lets more workgroups, and so more refill
    // loads, share a CU.
    static_assert(!REG || (((KW == 1 && VW <= 1) || (KW == 2 && VW == 0)) && ITEMS == 8),
                  "register stores: 4-byte keys with no or 4-byte payloads, or 8-byte keys");
    constexpr bool kDirect = REG;
    using Cfg = MergeCfg<THREADS, ITEMS, KW, VW, !kDirect>;
    constexpr int kTile = Cfg::kTile;
    constexpr int kCap = Cfg::kCap;
    constexpr int kMask = Cfg::kMask;
    constexpr int kSide = Cfg::kSide;
    constexpr int kVCap = Cfg::kVCap;
    constexpr int kVMask = Cfg::kVMask;
    constexpr int kVSide = Cfg::kVSide;
    // Every lane takes part in the refill loads (kLoadVec 16-byte vectors
    // each) and in the tile stores.  (Giving the loads and the stores to
    // separate wavefronts, so that no wavefront's wait on the vector-memory
    // counter ever covers a store, measured 1% slower.)
    constexpr int kLoadVec = kTile * KW / 4 / THREADS;
    constexpr int kStoreVec = kLoadVec;
    constexpr int kVLoadVec = KV ? kTile * VW / 4 / THREADS : 1;
    using RefillT = Refill<THREADS, kLoadVec, kCap, kSide, ORDER>;
    using VRefillT = Refill<THREADS, kVLoadVec, kVCap, kVSide, VORDER>;
    __shared__ __attribute__((aligned(16))) int lds[Cfg::kWords];
    int* const ring = lds + Cfg::kRing;      // A ring; B ring at ring + kSide
    int* const vring = lds + Cfg::kValRing;  // payload rings: A, then B at + kVSide
    int* const stage = lds + Cfg::kStage;
    int* const vstage = lds + Cfg::kValStage;
    int* const split = lds + Cfg::kSplit;

    const int tid = threadIdx.x;
    // The slice of the tile this lane merges: ITEMS outputs from slice*ITEMS.
    const int slice = !kDirect ? tid : (KW == 1 ? direct_slice(tid) : direct_slice_wide(tid));
    const int64_t seg = blockIdx.x;
    int64_t k0, i0, j0;  // first output, first A and first B element of the segment
    int c_len, a_len, b_len;
    if constexpr (!DESC) {
        const int64_t total = m + n;
        k0 = seg * seg_len;
        const int64_t k1 = k0 + seg_len < total ? k0 + seg_len : total;
        c_len = static_cast<int>(k1 - k0);
        int64_t p0, p1;  // co-ranks of k0 and k1
        if constexpr (SELF) {
            // Lanes 0-3 search k0, lanes 4-7 k1; the rest of the first
            // wavefront votes with empty ranges.  The results pass through
            // the split words, which the tiles use only after the barriers.
            if (tid < 64) {
                const int grp = tid >> 2;
                const int g_lane = tid & 3;
                const bool act = grp < 2;
                const int64_t i = co_rank_group<4, ORDER>(act ? (grp == 0 ? k0 : k1) : 0, A,
                                                          act ? m : 0, B, act ? n : 0, g_lane,
                                                          tid - g_lane);
                if (act && g_lane == 0) {
                    split[2 * grp] = static_cast<int>(static_cast<uint32_t>(i));
                    split[2 * grp + 1] = static_cast<int>(static_cast<uint64_t>(i) >> 32);
                }
            }
            __syncthreads();
            p0 = static_cast<int64_t>(
                (static_cast<uint64_t>(static_cast<uint32_t>(split[1])) << 32) |
                static_cast<uint32_t>(split[0]));
            p1 = static_cast<int64_t>(
                (static_cast<uint64_t>(static_cast<uint32_t>(split[3])) << 32) |
                static_cast<uint32_t>(split[2]));
            __syncthreads();  // every lane has read them before the tiles reuse the words
        } else {
            p0 = part[seg];
            p1 = part[seg + 1];
        }
        // Segment windows from the partition, clamped so that any partition
        // (even one made from unsorted input) keeps every access in range.
        i0 = clamp_to<int64_t>(p0, k0 > n ? k0 - n : 0, k0 < m ? k0 : m);
        const int64_t i1 = clamp_to<int64_t>(p1, k1 > n ? k1 - n : 0, k1 < m ? k1 : m);
        a_len = static_cast<int>(clamp_to<int64_t>(i1 - i0, 0, c_len));
        b_len = c_len - a_len;
        j0 = k0 - i0;
    } else {
        // A segment descriptor names its ranges of A, B and C directly.  They
        // are clamped into the arrays (m, n and c_total elements) and to
        // seg_len outputs, and a segment whose output would leave C is
        // skipped, so any descriptor keeps every access in range.
        const SegDesc d = desc[seg];
        i0 = clamp_to<int64_t>(d.a0, 0, m);
        const int64_t i1 = clamp_to<int64_t>(d.a1, i0, m);
        j0 = clamp_to<int64_t>(d.b0, 0, n);
        const int64_t j1 = clamp_to<int64_t>(d.b1, j0, n);
        a_len = static_cast<int>(i1 - i0 < seg_len ? i1 - i0 : seg_len);
        b_len = static_cast<int>(j1 - j0 < seg_len - a_len ? j1 - j0 : seg_len - a_len);
        c_len = a_len + b_len;
        k0 = d.c0;
        if (k0 < 0 || k0 > c_total - c_len) {
            k0 = 0;
            a_len = b_len = c_len = 0;
        }
    }

    // Word pointers to the segment's first element of each array.
    const int32_t* const As = reinterpret_cast<const int32_t*>(A + i0);
    const int32_t* const Bs = reinterpret_cast<const int32_t*>(B + j0);
    int32_t* const Cs = reinterpret_cast<int32_t*>(C + k0);
    const int a_base = word_phase(As) & kMask;
    const int b_base = word_phase(Bs) & kMask;
    // Payload rings use their own arrays' phases.
    const int32_t* const Avs = KV ? reinterpret_cast<const int32_t*>(Av) + VW * i0 : nullptr;
    const int32_t* const Bvs = KV ? reinterpret_cast<const int32_t*>(Bv) + VW * j0 : nullptr;
    int32_t* const Cvs = KV ? reinterpret_cast<int32_t*>(Cv) + VW * k0 : nullptr;
    const int va_base = KV ? (word_phase(Avs) & kVMask) : 0;
    const int vb_base = KV ? (word_phase(Bvs) & kVMask) : 0;
    // 16-byte stores from registers need a 16-byte-aligned output.
    [[maybe_unused]] const bool c_aligned = (word_phase(Cs) & 3) == 0;
    [[maybe_unused]] const bool cv_aligned = KV && (word_phase(Cvs) & 3) == 0;

    int a_cons = 0, b_cons = 0;  // elements consumed so far (segment-relative)
    int a_loaded = a_len < kTile ? a_len : kTile;
    int b_loaded = b_len < kTile ? b_len : kTile;

    // Initial fill: up to one tile of each side.
    {
        SideRange ra, rb, none;
        none.set(As, a_base, 0, 0);
        RefillT fa, fb;
        ra.set(As, a_base, 0, KW * a_loaded);
        rb.set(Bs, b_base, 0, KW * b_loaded);
        fa.issue(ra, none, tid);
        fb.issue(none, rb, tid);
        fa.commit(ring, tid);
        fb.commit(ring, tid);
        if constexpr (KV) {
            SideRange va, vb, vnone;
            vnone.set(Avs, va_base, 0, 0);
            va.set(Avs, va_base, 0, VW * a_loaded);
            vb.set(Bvs, vb_base, 0, VW * b_loaded);
            VRefillT ga, gb;
            ga.issue(va, vnone, tid);
            gb.issue(vnone, vb, tid);
            ga.commit(vring, tid);
            gb.commit(vring, tid);
        }
    }
    __syncthreads();

    bool probe_one_sided = true;  // test the first tile up front
    for (int c_done = 0; c_done < c_len;) {
        const int c_tile = c_len - c_done < kTile ? c_len - c_done : kTile;
        const int wa = a_loaded - a_cons;  // A window in the ring: min(TILE, left)
        const int wb = b_loaded - b_cons;
        const int sa = (a_base + KW * a_cons) & kMask;  // word of the window's first A
        const int sb = (b_base + KW * b_cons) & kMask;
        const int vsa = (va_base + VW * a_cons) & kVMask;  // same for the payloads
        const int vsb = (vb_base + VW * b_cons) & kVMask;
        const int* const ring_a = ring;
        const int* const ring_b = ring + kSide;

        // One-sided tile: every output comes from one side when the tile's
        // last A precedes the first B (A wins ties), or the tile's last B
        // precedes the first A.  Then the tile is a copy of that side's window:
        // no sort and no stage.  Such tiles come in runs (skewed inputs, long
        // runs of equal keys), so the check is made up front -- skipping the
        // searches too -- only after a one-sided tile; otherwise the searches'
        // own result (x_t = 0 or c_tile) detects it at no extra cost.
        int side = 0;  // 0: general tile, 1: all from A, 2: all from B
        if (probe_one_sided) {
            const bool all_a =
                wa >= c_tile && (wb == 0 || ld_elem<Key>(ring_a, (sa + KW * (c_tile - 1)) & kMask) <=
                                                ld_elem<Key>(ring_b, sb));
            const bool all_b =
                !all_a && wb >= c_tile &&
                (wa == 0 ||
                 ld_elem<Key>(ring_b, (sb + KW * (c_tile - 1)) & kMask) < ld_elem<Key>(ring_a, sa));
            side = __builtin_amdgcn_readfirstlane(all_a ? 1 : (all_b ? 2 : 0));
        }

        // Co-rank of the end of this lane's slice, searched in the ring; the
        // lane's start is its left neighbour's end.
        const int c_end = (slice + 1) * ITEMS < c_tile ? (slice + 1) * ITEMS : c_tile;
        int e = 0;
        int x_t;  // A elements this tile consumes
        if (side == 0) {
            // A lane's diagonal is at most (lane + 1) * ITEMS, so the lower
            // wavefronts' searches take fewer steps (10, 11, 11 and 12 for
            // 256 lanes of 8).
            const int wave_k = __builtin_amdgcn_readfirstlane(((tid >> 6) + 1) * 64 * ITEMS);
            if (wave_k <= kTile / 4)
                e = co_rank_tile<bit_length(kTile / 4), kMask, Key>(c_end, wa, wb, ring_a, sa,
                                                                    ring_b, sb);
            else if (wave_k <= kTile / 2)
                e = co_rank_tile<bit_length(kTile / 2), kMask, Key>(c_end, wa, wb, ring_a, sa,
                                                                    ring_b, sb);
            else if (wave_k < kTile)
                e = co_rank_tile<bit_length(kTile - 1), kMask, Key>(c_end, wa, wb, ring_a, sa,
                                                                    ring_b, sb);
            else
                e = co_rank_tile<bit_length(kTile), kMask, Key>(c_end, wa, wb, ring_a, sa, ring_b,
                                                                sb);
            split[slice] = e;
            __syncthreads();
            // The same for every lane, so it is moved to a scalar register and
            // the refill bookkeeping stays scalar.
            x_t = __builtin_amdgcn_readfirstlane(split[THREADS - 1]);
            side = x_t == c_tile ? 1 : (x_t == 0 ? 2 : 0);
        } else {
            x_t = side == 1 ? c_tile : 0;
        }
        probe_one_sided = side != 0;

        // Prefetch the next refill: exactly what this tile consumes, clamped
        // to what is left of the segment.  It is in flight while this tile
        // is merged and stored.
        const int a_cons2 = a_cons + x_t;
        const int b_cons2 = b_cons + (c_tile - x_t);
        const int a_loaded2 = a_cons2 + kTile < a_len ? a_cons2 + kTile : a_len;
        const int b_loaded2 = b_cons2 + kTile < b_len ? b_cons2 + kTile : b_len;
        RefillT rf;
        VRefillT rv;
        {
            SideRange ra, rb;
            ra.set(As, a_base, KW * a_loaded, KW * a_loaded2);
            rb.set(Bs, b_base, KW * b_loaded, KW * b_loaded2);
            rf.issue(ra, rb, tid);
            if constexpr (KV) {
                SideRange va, vb;
                va.set(Avs, va_base, VW * a_loaded, VW * a_loaded2);
                vb.set(Bvs, vb_base, VW * b_loaded, VW * b_loaded2);
                rv.issue(va, vb, tid);
            }
        }

        if (side != 0) {
            const int* const win = side == 1 ? ring_a : ring_b;
            const int start = side == 1 ? sa : sb;
            store_from_ring<THREADS, kStoreVec, kMask, ORDER>(Cs + KW * c_done, KW * c_tile, win,
                                                              start, tid);
            if constexpr (KV) {
                const int* const vwin = side == 1 ? vring : vring + kVSide;
                const int vstart = side == 1 ? vsa : vsb;
                store_from_ring<THREADS, kVLoadVec, kVMask, VORDER>(Cvs + VW * c_done,
                                                                    VW * c_tile, vwin, vstart, tid);
            }
            __syncthreads();  // every read of the consumed slots is done
            rf.commit(ring, tid);
            if constexpr (KV) rv.commit(vring, tid);
        } else {
            const int c_beg = slice * ITEMS < c_tile ? slice * ITEMS : c_tile;
            const int s = slice > 0 ? split[slice - 1] : 0;

            // This lane's row of the stage: ITEMS contiguous elements.
            int* const row = stage + stage_word(tid * ITEMS * KW);
            // Outputs kept in registers for store_direct8 (keys, payloads).
            int kout[kDirect ? ITEMS * KW : 1];
            int vout[kDirect && KV ? ITEMS : 1];
            if constexpr (!KV) {
                // Candidates: the next ITEMS keys of each side from the lane's
                // split.  The lane's outputs are the ITEMS smallest of them; any
                // candidate past the lane's own range is >= all of its outputs
                // (it comes later in the merge), so only candidates past the
                // window need replacing, by the largest key image.
                const int bs = c_beg - s;
                const int* const pa = ring_a + ((sa + KW * s) & kMask);
                const int* const pb = ring_b + ((sb + KW * bs) & kMask);
                Key a[ITEMS], b[ITEMS], x[ITEMS];
#pragma unroll
                for (int t = 0; t < ITEMS; ++t) {
                    a[t] = ld_elem<Key>(pa, KW * t);
                    b[t] = ld_elem<Key>(pb, KW * t);
                }
                if (s + ITEMS > wa || bs + ITEMS > wb) {
#pragma unroll
                    for (int t = 0; t < ITEMS; ++t) {
                        a[t] = s + t < wa ? a[t] : KeyOrder<ORDER>::kMax;
                        b[t] = bs + t < wb ? b[t] : KeyOrder<ORDER>::kMax;
                    }
                }
                // a ascending followed by b descending is bitonic; the pairwise
                // minima hold its ITEMS smallest, themselves bitonic.
#pragma unroll
                for (int t = 0; t < ITEMS; ++t) x[t] = min(a[t], b[ITEMS - 1 - t]);
                bitonic_clean<ITEMS>(x);
                if constexpr (kDirect) {
#pragma unroll
                    for (int t = 0; t < ITEMS; ++t) {
                        if constexpr (KW == 1) {
                            kout[t] = static_cast<int>(x[t]);
                        } else {
                            kout[2 * t] = low_word(x[t]);
                            kout[2 * t + 1] = high_word(x[t]);
                        }
                    }
                } else {
#pragma unroll
                for (int v = 0; v < ITEMS * KW / 4; ++v) {
                    int4v q;
                    if constexpr (KW == 1) {
                        q.x = x[4 * v];
                        q.y = x[4 * v + 1];
                        q.z = x[4 * v + 2];
                        q.w = x[4 * v + 3];
                    } else {
                        q.x = low_word(x[2 * v]);
                        q.y = high_word(x[2 * v]);
                        q.z = low_word(x[2 * v + 1]);
                        q.w = high_word(x[2 * v + 1]);
                    }
                    *reinterpret_cast<int4v*>(row + 4 * v) = q;
                }
                }
            } else {
                // Key+payload: the serial two-pointer merge of the lane's exact
                // ranges, so equal keys keep A's payloads first.
                Key out[ITEMS];
                int src[ITEMS];  // payload ring word of each output
                int a = s;
                int b = c_beg - s;
                const int a_end = e;
                const int b_end = c_end - e;
                Key ka = ld_elem<Key>(ring_a, (sa + KW * a) & kMask);
                Key kb = ld_elem<Key>(ring_b, (sb + KW * b) & kMask);
#pragma unroll
                for (int t = 0; t < ITEMS; ++t) {
                    const bool take_a = a < a_end && (b >= b_end || ka <= kb);
                    out[t] = take_a ? ka : kb;
                    src[t] = take_a ? ((vsa + VW * a) & kVMask) : kVSide + ((vsb + VW * b) & kVMask);
                    a += take_a ? 1 : 0;
                    b += take_a ? 0 : 1;
                    if (t + 1 < ITEMS) {
                        const int w = take_a ? ((sa + KW * a) & kMask) : kSide + ((sb + KW * b) & kMask);
                        const Key nxt = ld_elem<Key>(ring, w);
                        ka = take_a ? nxt : ka;
                        kb = take_a ? kb : nxt;
                    }
                }
                if constexpr (kDirect) {
                    // Payloads leave the ring before the refill lands there.
#pragma unroll
                    for (int t = 0; t < ITEMS; ++t) {
                        kout[t] = static_cast<int>(out[t]);
                        vout[t] = vring[src[t]];
                    }
                } else {
                int* const vrow = vstage + stage_word(tid * ITEMS * VW);
#pragma unroll
                for (int t = 0; t < ITEMS; ++t) {
                    st_elem<Key>(row, KW * t, out[t]);
                    if constexpr (VW == 1) {
                        vrow[t] = vring[src[t]];
                    } else {
                        st_elem<long long>(vrow, 2 * t, ld_elem<long long>(vring, src[t]));
                    }
                }
                }
            }
            __syncthreads();

            // Commit the refill before this tile's stores go out: the wait on
            // the vector-memory counter (which counts loads and stores alike)
            // then covers the refill loads and only stores issued a whole tile
            // earlier.  The refill lands in the slots this tile consumed.
            rf.commit(ring, tid);
            if constexpr (KV) rv.commit(vring, tid);

            if constexpr (kDirect) {
                // From registers: each wavefront stores its 512 outputs as two
                // 1 KB runs (store_direct8).
                const int wbase = (tid >> 6) * 64 * ITEMS * KW;
                if constexpr (KW == 1)
                    store_direct8<ORDER>(Cs + c_done, wbase, c_tile, c_aligned, kout, tid);
                else
                    store_direct16<ORDER>(Cs + KW * c_done, wbase, KW * c_tile, c_aligned, kout,
                                          tid);
                if constexpr (KV)
                    store_direct8<VORDER>(Cvs + c_done, wbase, c_tile, cv_aligned, vout, tid);
            } else {
                // Coalesced 16-byte stores of the whole tile from the stage.
                // (Storing each lane's ITEMS contiguous outputs straight from
                // registers, as two 16-byte stores per lane, measured 10%
                // slower, and 2.3x slower with nontemporal stores: each store
                // instruction then covers every other 16 bytes, and the pieces
                // of a line reach HBM apart.  store_direct8 avoids that.)
                store_tile<THREADS, kStoreVec, ORDER>(Cs + KW * c_done, KW * c_tile, stage, tid);
                if constexpr (KV) {
                    store_tile<THREADS, kVLoadVec, VORDER>(Cvs + VW * c_done, VW * c_tile,
                                                           vstage, tid);
                }
            }
        }  // general tile

        a_cons = a_cons2;
        b_cons = b_cons2;
        a_loaded = a_loaded2;
        b_loaded = b_loaded2;
        c_done += c_tile;
        __syncthreads();
    }
}

}  // namespace omerge
