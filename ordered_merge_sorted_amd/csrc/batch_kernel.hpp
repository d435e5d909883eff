// batch_kernel.hpp -- many merges in one launch, and the merge-sort stages.
//
// Page "Practice - Sorting Foundations and Parallel Radix Sort"
// (pmpp.huatsai.dev/13-sorting/practice-sorting), its merge-sort item: in
// the early stages of a merge sort there are many independent merges of few
// keys each, and the parallelism is across merges (one merge per block);
// in the late stages there are few, large merges, and each one is cut into
// independent pieces with the co-rank function of the merge chapter.  The
// same page notes that sorting networks, although asymptotically worse, are
// often the fastest way to sort short sequences.
//
// Both regimes run through one segment merge kernel here (merge_kernel.hpp,
// descriptor mode): a plan kernel cuts every merge of a batch, or of one
// merge-sort pass, into segments of at most seg_len outputs, each lying
// inside one merge, and writes one descriptor per segment (its A, B and C
// ranges).  Small merges become one segment each (parallel across merges);
// a large merge becomes many (parallel inside the merge).  The boundary
// co-ranks are found with the group search of the partition kernel, inside
// the one merge that holds the boundary.
//
// The first stage of the merge sort is block_sort_kernel: each workgroup
// sorts one tile in registers and LDS (a bitonic network per lane, then
// in-LDS merges of the lanes' runs by co-rank), producing sorted runs of
// one tile for the merge passes.
#pragma once

#include "merge_kernel.hpp"

namespace omerge {

// ---------------------------------------------------------------------------
// Plans.  A plan has segs segments and segs + 1 boundaries; boundary w is
// the start of segment w and the end of segment w-1.  One group of G lanes
// handles one boundary: it finds the co-rank there (if the boundary is inside
// a merge) and writes the start of desc[w] and the end of desc[w-1].

// Merge-sort pass: src (total elements) holds sorted runs of `run` elements;
// runs 2p (as A) and 2p+1 (as B) merge into the same positions of the output.
// A full pair is cut into per_pair segments of seg_len outputs; a short last
// pair (total not a multiple of 2*run) into as many as it needs.
template <int G, int ORDER>
__global__ __launch_bounds__(256) void plan_runs_kernel(
    const typename KeyOrder<ORDER>::T* __restrict__ src, int64_t total, int64_t run,
    int64_t seg_len, int64_t per_pair, int64_t segs, SegDesc* __restrict__ desc) {
    static_assert(G >= 2, "group search");
    const int64_t gid = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
    if ((gid & ~int64_t(63)) / G > segs) return;  // the whole wavefront is past the end
    const int64_t w = gid / G;
    const bool live = w <= segs;
    const int g_lane = static_cast<int>(gid % G);
    const int g_shift = static_cast<int>(threadIdx.x & 63) - g_lane;

    const int64_t full_pairs = total / (2 * run);
    int64_t p, g;  // pair, and segment within the pair
    if (w < full_pairs * per_pair) {
        p = w / per_pair;
        g = w % per_pair;
    } else {
        p = full_pairs;
        g = w - full_pairs * per_pair;
    }
    const int64_t base = p * 2 * run;
    const int64_t rem = total > base ? total - base : 0;
    const int64_t la = rem < run ? rem : run;
    const int64_t lb = rem - la < run ? rem - la : run;
    const int64_t k = g * seg_len < la + lb ? g * seg_len : la + lb;
    const int64_t i = co_rank_group<G, ORDER>(live ? k : 0, src + base, live ? la : 0,
                                              src + base + la, live ? lb : 0, g_lane, g_shift);
    if (!live || g_lane != 0) return;
    if (w < segs) {
        desc[w].a0 = base + i;
        desc[w].b0 = base + la + (k - i);
        desc[w].c0 = base + k;
    }
    if (w > 0) {
        if (g > 0) {  // inside a pair: the previous segment ends here
            desc[w - 1].a1 = base + i;
            desc[w - 1].b1 = base + la + (k - i);
        } else {      // first segment of pair p: the previous one ends pair p-1
            desc[w - 1].a1 = base - run;
            desc[w - 1].b1 = base;
        }
    }
}

// The first x in [0, pairs] whose merge start start(x) lies past c, or
// pairs + 1 if none does: the points with start(x) <= c form a prefix, as
// merge starts never fall.  G lanes per search (G < 64), all lanes of the
// wavefront together.  Each round tests G points of [lo, hi); the answer
// lies after the last passing point and at or before the first failing one.
// The first round tests G consecutive points around `guess`, where the
// answer sits when the merges have equal lengths (then one round finds it);
// later rounds split the interval evenly.  Every round shrinks the interval,
// whatever the starts hold, so the search ends.
template <int G, typename Start>
__device__ __forceinline__ int64_t first_start_after(int64_t c, int64_t pairs, double guess,
                                                     bool live, Start start, int g_lane,
                                                     int g_shift) {
    static_assert(G >= 2 && G < 64 && (64 % G) == 0, "group size");
    constexpr int kLog = bit_length(G) - 1;
    int64_t lo = 0, hi = live ? pairs + 1 : 0;
    for (int round = 0; round < 64; ++round) {
        if (__ballot(lo < hi) == 0) break;  // every group of the wavefront is done
        const int64_t span = hi - lo;
        const bool near = round == 0 && span > G;
        int64_t first = 0;
        if (near) {
            const double f = floor(guess) - (G / 2 - 1);
            const double top = static_cast<double>(hi - G);
            first = static_cast<int64_t>(fmin(fmax(f, static_cast<double>(lo)), top));
        }
        const int64_t q = span >> kLog, r = span & (G - 1);
        const int npts = near || span >= G ? G : static_cast<int>(span);
        auto point = [=](int l) -> int64_t {
            if (near) return first + l;
            return span < G ? lo + l : lo + q * l + ((r * l) >> kLog);
        };
        const bool pass = lo < hi && g_lane < npts && start(point(g_lane)) <= c;
        const unsigned long long mine = (__ballot(pass) >> g_shift) & ((1ull << G) - 1);
        const int cnt = __popcll(mine);
        if (lo < hi) {
            const int64_t new_lo = cnt > 0 ? point(cnt - 1) + 1 : lo;
            const int64_t new_hi = cnt < npts ? point(cnt) : hi;
            lo = new_lo;
            hi = new_hi;
        }
    }
    return lo;
}

// Batch of merges: merge p takes A[a_off[p], a_off[p+1]) and B[b_off[p],
// b_off[p+1]) to C[a_off[p]+b_off[p], a_off[p+1]+b_off[p+1]), p = 0..pairs-1
// (a_off[0] = b_off[0] = 0, a_off[pairs] = m, b_off[pairs] = n).  The
// boundaries are every merge's start and every multiple of seg_len inside
// (0, m+n), in order, a merge start first where the two coincide: merge
// start p is boundary p + ceil(c_p/seg_len) - 1 (c_p its first output), and
// the multiple g*seg_len is boundary (g-1) + #{p : c_p <= g*seg_len} (moved
// to halfway to the next boundary when it falls on a merge start, below).
// In these concatenated coordinates the end of one segment is the start of
// the next even across merges.  Offsets are clamped into [0, m] / [0, n], so
// even invalid offsets keep every access in range.
template <int G, int ORDER>
__global__ __launch_bounds__(256) void plan_batched_kernel(
    const typename KeyOrder<ORDER>::T* __restrict__ A, const int64_t* __restrict__ a_off,
    int64_t m, const typename KeyOrder<ORDER>::T* __restrict__ B,
    const int64_t* __restrict__ b_off, int64_t n, int64_t pairs, int64_t seg_len,
    int64_t segs, SegDesc* __restrict__ desc) {
    static_assert(G >= 2, "group search");
    const int64_t gid = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
    if ((gid & ~int64_t(63)) / G > segs) return;
    const int64_t w = gid / G;
    const bool live = w <= segs;
    const int g_lane = static_cast<int>(gid % G);
    const int g_shift = static_cast<int>(threadIdx.x & 63) - g_lane;
    auto ao = [&](int64_t p) { return clamp_to<int64_t>(a_off[p], 0, m); };
    auto bo = [&](int64_t p) { return clamp_to<int64_t>(b_off[p], 0, n); };

    int64_t p = 0, k = 0, idx = 0, c = 0;
    bool search = false;
    // Multiples g*seg_len look up the number of merge starts <= c (guessed
    // from an even share of the outputs per merge); merge starts need none.
    const bool multiple = live && w > pairs;
    const int64_t total = m + n;
    const int64_t cm = multiple ? (w - pairs) * seg_len : 0;
    const double guess =
        total > 0 ? static_cast<double>(cm) * static_cast<double>(pairs) / static_cast<double>(total)
                  : 0.0;
    const int64_t lo = first_start_after<G>(
        cm, pairs, guess, multiple, [&](int64_t x) { return ao(x) + bo(x); }, g_lane, g_shift);
    if (live && w <= pairs) {  // start of merge w
        p = w;
        c = ao(p) + bo(p);
        idx = p + (c > 0 ? (c - 1) / seg_len : 0);
    } else if (live) {         // multiple g*seg_len inside some merge
        const int64_t g = w - pairs;
        c = cm;
        idx = (g - 1) + lo;
        p = lo > 0 ? (lo - 1 < pairs ? lo - 1 : pairs - 1) : 0;
        k = c - (ao(p) + bo(p));
        search = true;
        // A multiple that falls on a merge start leaves an empty segment
        // between the two boundaries.  Merges whose lengths are multiples of
        // seg_len do that after every merge, and the half-empty grid ran at
        // 60% of the speed (2^14 merges of 8192 + 8192 keys: 0.66 ms against
        // 0.39 ms).  When the merge starting there is at least seg_len long,
        // such a multiple moves to the middle of the merge's first seg_len
        // outputs: same boundary count and order, no empty segment.  (With
        // shorter merges an empty segment comes at most every other merge,
        // which measured no slower than splitting their merges.)
        if (k == 0 && p < pairs && ao(p + 1) + bo(p + 1) - c >= seg_len) {
            c += seg_len / 2;
            k = seg_len / 2;
        }
    }
    int64_t la = 0, lb = 0;
    if (search && p < pairs) {
        const int64_t a1 = ao(p + 1), b1 = bo(p + 1);
        la = a1 > ao(p) ? a1 - ao(p) : 0;
        lb = b1 > bo(p) ? b1 - bo(p) : 0;
        k = clamp_to<int64_t>(k, 0, la + lb);
    } else {
        k = 0;
    }
    const int64_t a_base = search ? ao(p) : 0, b_base = search ? bo(p) : 0;
    const int64_t i = co_rank_group<G, ORDER>(k, A + a_base, la, B + b_base, lb, g_lane, g_shift);
    if (!live || g_lane != 0 || idx < 0 || idx > segs) return;
    const int64_t a = search ? a_base + i : ao(p);
    const int64_t b = search ? b_base + (k - i) : bo(p);
    if (idx < segs) {
        desc[idx].a0 = a;
        desc[idx].b0 = b;
        desc[idx].c0 = c;
    }
    if (idx > 0) {
        desc[idx - 1].a1 = a;
        desc[idx - 1].b1 = b;
    }
}

// ---------------------------------------------------------------------------
// Block sort: workgroup t sorts elements [t*TILE, min((t+1)*TILE, total)) of
// src into the same positions of dst (dst may be src: a tile is read whole
// before it is written).  Keys are sorted as their order images; with
// payloads (VW words each) the sort is stable: every element carries its
// position in the tile, and (key, position) pairs are all distinct, so
// ordering them exactly is the stable order.  The tile's missing tail is
// padded with the largest image and positions past the end, which sort
// last and are never stored.

// Sorts x[0..N) (with positions pos when POS) ascending by a bitonic network.
template <int N, bool POS, typename T>
__device__ __forceinline__ void bitonic_sort(T (&x)[N], int (&pos)[N]) {
#pragma unroll
    for (int kk = 2; kk <= N; kk <<= 1) {
#pragma unroll
        for (int j = kk >> 1; j > 0; j >>= 1) {
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int l = i ^ j;
                if (l > i && !POS) {
                    // Keys alone: the compare-exchange as min and max (the
                    // swap form below compiles to a compare and two selects).
                    const T lo = min(x[i], x[l]), hi = max(x[i], x[l]);
                    const bool up = (i & kk) == 0;
                    x[i] = up ? lo : hi;
                    x[l] = up ? hi : lo;
                } else if (l > i) {
                    const bool up = (i & kk) == 0;
                    const bool gt = POS ? (x[i] > x[l] || (x[i] == x[l] && pos[i] > pos[l]))
                                        : x[i] > x[l];
                    if (gt == up) {
                        const T t = x[i];
                        x[i] = x[l];
                        x[l] = t;
                        if (POS) {
                            const int q = pos[i];
                            pos[i] = pos[l];
                            pos[l] = q;
                        }
                    }
                }
            }
        }
    }
}

// Sorts x[0..N) ascending by Batcher's odd-even merge sort (N a power of
// two): merges of sorted halves at distances p = 1, 2, 4, ..., each a
// cascade of compare-exchanges at strides k = p, p/2, ..., 1 between
// elements of the same 2p block.  Every exchange keeps the smaller first,
// so keys alone take one min and one max each; for N = 32 the network has
// 191 exchanges against the bitonic network's 240.
template <int N, typename T>
__device__ __forceinline__ void odd_even_sort(T (&x)[N]) {
#pragma unroll
    for (int p = 1; p < N; p <<= 1) {
#pragma unroll
        for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
            for (int j = k % p; j + k < N; j += 2 * k) {
#pragma unroll
                for (int i = 0; i < k; ++i) {
                    const int a = i + j, b = i + j + k;
                    if (b < N && a / (2 * p) == b / (2 * p)) {
                        const T lo = min(x[a], x[b]), hi = max(x[a], x[b]);
                        x[a] = lo;
                        x[b] = hi;
                    }
                }
            }
        }
    }
}

// A lane's row of ITEMS elements (keys or int positions) to / from the
// padded LDS layout of the merge stage (4 spare words after every 32), as
// 16-byte accesses, which that padding keeps free of bank conflicts.
template <int ITEMS, typename T>
__device__ __forceinline__ void put_row(int* buf, int tid, const T (&x)[ITEMS]) {
    constexpr int W = sizeof(T) / 4;
    int* const row = buf + stage_word(tid * ITEMS * W);
#pragma unroll
    for (int v = 0; v < ITEMS * W / 4; ++v) {
        int4v q;
        if constexpr (W == 1) {
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

template <int ITEMS, typename T>
__device__ __forceinline__ void get_row(const int* buf, int tid, T (&x)[ITEMS]) {
    constexpr int W = sizeof(T) / 4;
    const int* const row = buf + stage_word(tid * ITEMS * W);
#pragma unroll
    for (int v = 0; v < ITEMS * W / 4; ++v) {
        const int4v q = *reinterpret_cast<const int4v*>(row + 4 * v);
        if constexpr (W == 1) {
            x[4 * v] = q.x;
            x[4 * v + 1] = q.y;
            x[4 * v + 2] = q.z;
            x[4 * v + 3] = q.w;
        } else {
            x[2 * v] = join_words(q.x, q.y);
            x[2 * v + 1] = join_words(q.z, q.w);
        }
    }
}

// A 32-bit word as held by lane (lane ^ MASK) of the wavefront; every lane
// takes part (every DPP pattern below reads a lane of the same row, so all
// lanes are written and the old value of the destination never shows; the
// mov form leaves it undefined, which spares a copy of x per exchange).  The route depends on the mask: DPP inside each row of 16
// lanes where a row pattern is the xor (quad_perm for 1, 2 and 3; half-row
// mirror for 7; rotate by 8 for 8; row mirror for 15), ds_swizzle in bit
// mode (and 0x1f, xor MASK) inside each half of the wavefront for the other
// masks below 32, and a full shuffle across the halves.
template <int MASK>
__device__ __forceinline__ int lane_xor_word(int x) {
    static_assert(MASK > 0 && MASK < 64, "a lane mask of the wavefront");
    if constexpr (MASK == 1) {
        return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    } else if constexpr (MASK == 2) {
        return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    } else if constexpr (MASK == 3) {
        return __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, false);  // quad_perm 3,2,1,0
    } else if constexpr (MASK == 7) {
        return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);  // row_half_mirror
    } else if constexpr (MASK == 8) {
        return __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else if constexpr (MASK == 15) {
        return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);  // row_mirror
    } else if constexpr (MASK < 32) {
        return __builtin_amdgcn_ds_swizzle(x, 0x1F | (MASK << 10));
    } else {
        return __shfl_xor(x, MASK);
    }
}

template <int MASK, typename T>
__device__ __forceinline__ T lane_xor(T x) {
    if constexpr (sizeof(T) == 8) {
        return static_cast<T>(join_words(lane_xor_word<MASK>(low_word(x)),
                                         lane_xor_word<MASK>(high_word(x))));
    } else {
        return lane_xor_word<MASK>(x);
    }
}

// (key, position) of this lane against (yk, yp): true when the other pair
// is the smaller.  Without positions (POS = false) keys alone decide.
template <bool POS, typename T>
__device__ __forceinline__ bool other_first(T k, int p, T yk, int yp) {
    return POS ? (yk < k || (yk == k && yp < p)) : yk < k;
}

// The median of three: one v_med3_i32 (the compiler matches this min/max
// form).  med3(x, y, INT_MIN) is the smaller of x and y, med3(x, y, INT_MAX)
// the larger, so one instruction keeps either side of a compare-exchange
// with the side chosen by a per-lane bound instead of a compare and select.
__device__ __forceinline__ int med3(int a, int b, int c) {
    return max(min(a, b), min(max(a, b), c));
}

// The bound that makes med3 keep the smaller value where bit BIT of the
// lane index is clear and the larger where it is set: INT_MIN or INT_MAX.
// The compiler sees that the bound takes one of two constants and would
// split every med3 into min, max and a select again, so the bound passes
// through an identity DPP move (quad_perm 0,1,2,3), which it cannot see
// through: one move per stage.
template <int BIT>
__device__ __forceinline__ int keep_bound(int lane) {
    const int b = (lane >> BIT) & 1 ? std::numeric_limits<int>::max()
                                    : std::numeric_limits<int>::min();
    return __builtin_amdgcn_mov_dpp(b, 0xE4, 0xF, 0xF, false);
}

// Keys alone of 32 bits take the med3 form; wider keys and (key, position)
// pairs compare and select.
template <bool POS, typename T>
constexpr bool kMed3Exchange = !POS && sizeof(T) == 4;

// One compare-exchange stage between each lane and lane ^ MASK, element by
// element: the lower lane keeps the smaller, the upper the larger.  With
// POS, positions travel with their keys and break ties.
template <int MASK, bool POS, int ITEMS, typename T>
__device__ __forceinline__ void lane_stage(T (&x)[ITEMS], int (&pos)[ITEMS], int lane) {
    const bool low = (lane & MASK) == 0;
    if constexpr (kMed3Exchange<POS, T>) {
        static_assert((MASK & (MASK - 1)) == 0, "half-cleaners pair lanes one bit apart");
        const int bound = keep_bound<__builtin_ctz(MASK)>(lane);
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) x[t] = med3(x[t], lane_xor<MASK>(x[t]), bound);
        return;
    }
#pragma unroll
    for (int t = 0; t < ITEMS; ++t) {
        const T yk = lane_xor<MASK>(x[t]);
        const int yp = POS ? lane_xor<MASK>(pos[t]) : 0;
        const bool take = low == other_first<POS>(x[t], pos[t], yk, yp);
        x[t] = take ? yk : x[t];
        if (POS) pos[t] = take ? yp : pos[t];
    }
}

// Orders x[0..N) (with positions when POS) ascending when it is bitonic.
template <bool POS, int N, typename T>
__device__ __forceinline__ void bitonic_clean_pos(T (&x)[N], int (&pos)[N]) {
    if constexpr (!POS) {
        bitonic_clean<N>(x);
    } else {
#pragma unroll
        for (int d = N / 2; d >= 1; d >>= 1) {
#pragma unroll
            for (int i = 0; i < N; ++i) {
                if ((i & d) == 0 && other_first<true>(x[i], pos[i], x[i + d], pos[i + d])) {
                    const T tk = x[i];
                    x[i] = x[i + d];
                    x[i + d] = tk;
                    const int tp = pos[i];
                    pos[i] = pos[i + d];
                    pos[i + d] = tp;
                }
            }
        }
    }
}

// Round R of the in-wavefront merge: pairs of runs of 2^R lanes.  A flip
// stage (element t against element ITEMS-1-t of the mirror lane, lane ^
// (2^(R+1)-1); the first run keeps the smaller) leaves each run bitonic;
// half-cleaners at lane distances 2^(R-1), ..., 1 and inside the lane sort
// it.
template <int D, bool POS, int ITEMS, typename T>
__device__ __forceinline__ void lane_half_cleaners(T (&x)[ITEMS], int (&pos)[ITEMS], int lane) {
    if constexpr (D >= 1) {
        lane_stage<D, POS>(x, pos, lane);
        lane_half_cleaners<D / 2, POS>(x, pos, lane);
    }
}

template <int R, bool POS, int ITEMS, typename T>
__device__ __forceinline__ void wave_round(T (&x)[ITEMS], int (&pos)[ITEMS], int lane) {
    constexpr int kMirror = (2 << R) - 1;
    const bool first = (lane & (1 << R)) == 0;
    T yk[ITEMS];
    int yp[ITEMS];
#pragma unroll
    for (int t = 0; t < ITEMS; ++t) {
        yk[t] = lane_xor<kMirror>(x[ITEMS - 1 - t]);
        yp[t] = POS ? lane_xor<kMirror>(pos[ITEMS - 1 - t]) : 0;
    }
    if constexpr (kMed3Exchange<POS, T>) {
        const int bound = keep_bound<R>(lane);
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) x[t] = med3(x[t], yk[t], bound);
    } else {
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) {
            const bool take = first == other_first<POS>(x[t], pos[t], yk[t], yp[t]);
            x[t] = take ? yk[t] : x[t];
            if (POS) pos[t] = take ? yp[t] : pos[t];
        }
    }
    lane_half_cleaners<(1 << R) / 2, POS>(x, pos, lane);
    bitonic_clean_pos<POS>(x, pos);
}

// Sorts the wavefront's 64 lanes x ITEMS elements (each lane's ITEMS already
// ascending) into one ascending run held lane-major, by six rounds of
// bitonic merges across lanes.  With POS the order is (key, position), all
// distinct, so the result is the stable order.  Data moves between lanes in
// registers (DPP) or through the LDS crossbar without touching its banks
// (swizzle, shuffle).
template <bool POS, int ITEMS, typename T>
__device__ __forceinline__ void wave_merge_rounds(T (&x)[ITEMS], int (&pos)[ITEMS], int lane) {
    wave_round<0, POS>(x, pos, lane);
    wave_round<1, POS>(x, pos, lane);
    wave_round<2, POS>(x, pos, lane);
    wave_round<3, POS>(x, pos, lane);
    wave_round<4, POS>(x, pos, lane);
    wave_round<5, POS>(x, pos, lane);
}

// Sorts a tile held in LDS: the keys' order images in kbuf (padded rows,
// KW = sizeof(Key)/4 words each, ITEMS elements of slack after the tile),
// with POS their positions in pbuf.  Each lane sorts its row, six rounds
// merge inside each wavefront, and in-LDS rounds merge the wavefronts'
// runs, until x (and pos) hold lane tid's ITEMS elements of the sorted tile.
// kbuf, pbuf and split (THREADS words) are scratch afterwards.
template <int THREADS, int ITEMS, bool POS, typename Key>
__device__ __forceinline__ void sort_tile(int* kbuf, int* pbuf, int* split, Key (&x)[ITEMS],
                                          int (&pos)[ITEMS], int tid, Key kmax) {
    constexpr int KW = sizeof(Key) / 4;
    constexpr int kTile = THREADS * ITEMS;
    // Each lane sorts its row of ITEMS elements.
    get_row<ITEMS>(kbuf, tid, x);
#pragma unroll
    for (int t = 0; t < ITEMS; ++t) pos[t] = tid * ITEMS + t;
    if constexpr (POS)
        bitonic_sort<ITEMS, true>(x, pos);
    else
        odd_even_sort<ITEMS>(x);

    // The first six rounds run inside each wavefront, across lanes: keys
    // alone (equal keys are indistinguishable, so any exact order of them is
    // the stable one), or (key, position) pairs with payloads.  Each
    // wavefront's run then holds one contiguous block of tile positions, so
    // the A-first merges of the LDS rounds below stay stable.
    constexpr int kWaveRun = ITEMS * 64;
    wave_merge_rounds<POS>(x, pos, tid & 63);

    // Merge rounds: runs of `run` elements merge pairwise into runs of 2*run.
    // The A run of a pair holds earlier positions than its B run, so taking
    // A on equal keys is the stable order.
    for (int run = kWaveRun; run < kTile; run *= 2) {
        __syncthreads();  // every read of the previous round is done
        put_row<ITEMS>(kbuf, tid, x);
        if constexpr (POS) put_row<ITEMS>(pbuf, tid, pos);
        __syncthreads();
        const int lanes = 2 * run / ITEMS;   // lanes per merged pair
        const int u = tid % lanes;           // this lane's place in it
        const int a0 = (tid - u) * ITEMS;    // the pair's A run; B run at a0 + run
        const int b0 = a0 + run;
        const int o_end = (u + 1) * ITEMS;
        // Co-rank of o_end: the largest x in [x_lo, x_hi] such that A[x-1]
        // comes before B[o_end-x] (A[x-1] <= B[o_end-x]; true at x_lo; the
        // passing points form a prefix), found by binary lifting: steps of
        // run, run/2, ..., 1 (they sum past the range, which is at most run
        // wide), each kept when its point passes.  Every tested point x in
        // (x_lo, x_hi] reads A[x-1] and B[o_end-x], both inside the pair's
        // runs.
        const int x_lo = o_end > run ? o_end - run : 0;
        const int x_hi = o_end < run ? o_end : run;
        int lo = x_lo;
        for (int step = run; step > 0; step >>= 1) {
            const int p = lo + step;
            const int pc = p < x_hi ? p : x_hi;
            const Key av = ld_elem<Key>(kbuf, stage_word(KW * (a0 + pc - 1)));
            const Key bv = ld_elem<Key>(kbuf, stage_word(KW * (b0 + o_end - pc)));
            lo = (p <= x_hi && av <= bv) ? p : lo;
        }
        split[tid] = lo;
        __syncthreads();
        const int s = u > 0 ? split[tid - 1] : 0;  // A elements before this lane's outputs
        const int bs = u * ITEMS - s;
        if constexpr (!POS) {
            // Candidates past a run's end read the next run (or the slack)
            // and are replaced by the largest image.  ITEMS consecutive
            // elements cross at most one 32-word pad: element t of a read
            // starting at word w sits at stage_word(w) + KW*t, plus 4 once
            // KW*t reaches the pad at 32 - (w & 31).
            Key a[ITEMS], b[ITEMS];
            const int wa = KW * (a0 + s), wb = KW * (b0 + bs);
            const int* const pa = kbuf + stage_word(wa);
            const int* const pb = kbuf + stage_word(wb);
            const int ca = 32 - (wa & 31), cb = 32 - (wb & 31);
#pragma unroll
            for (int t = 0; t < ITEMS; ++t) {
                a[t] = ld_elem<Key>(pa, KW * t + (KW * t >= ca ? 4 : 0));
                b[t] = ld_elem<Key>(pb, KW * t + (KW * t >= cb ? 4 : 0));
            }
            if (s + ITEMS > run || bs + ITEMS > run) {  // rare past the first rounds
#pragma unroll
                for (int t = 0; t < ITEMS; ++t) {
                    a[t] = t < run - s ? a[t] : kmax;
                    b[t] = t < run - bs ? b[t] : kmax;
                }
            }
#pragma unroll
            for (int t = 0; t < ITEMS; ++t) x[t] = min(a[t], b[ITEMS - 1 - t]);
            bitonic_clean<ITEMS>(x);
        } else {
            int ai = s, bi = bs;
            const int a_end = lo, b_end = o_end - lo;
#pragma unroll
            for (int t = 0; t < ITEMS; ++t) {
                const int ca = ai < run ? ai : run - 1;
                const int cb = bi < run ? bi : run - 1;
                const Key ka = ld_elem<Key>(kbuf, stage_word(KW * (a0 + ca)));
                const Key kb = ld_elem<Key>(kbuf, stage_word(KW * (b0 + cb)));
                const bool take_a = ai < a_end && (bi >= b_end || ka <= kb);
                x[t] = take_a ? ka : kb;
                pos[t] = pbuf[stage_word(take_a ? a0 + ca : b0 + cb)];
                ai += take_a ? 1 : 0;
                bi += take_a ? 0 : 1;
            }
        }
    }
}

template <int THREADS, int ITEMS, int VW, int ORDER>
__global__ __launch_bounds__(THREADS) void block_sort_kernel(
    const typename KeyOrder<ORDER>::T* __restrict__ src, const uint32_t* __restrict__ src_v,
    int64_t total, typename KeyOrder<ORDER>::T* dst, uint32_t* dst_v) {
    using K = KeyOrder<ORDER>;
    using Key = typename K::T;
    constexpr int KW = K::kWords;
    constexpr bool KV = VW > 0;
    constexpr int kTile = THREADS * ITEMS;
    static_assert(ITEMS >= 4 && (ITEMS & (ITEMS - 1)) == 0, "ITEMS: a power of two");
    // The in-LDS rounds read a lane's ITEMS candidates as consecutive padded
    // words that cross at most one pad (4 words after every 32).
    static_assert(KW * ITEMS <= 32, "a lane's row fits in 32 words");
    // LDS: keys and positions, padded as the merge stage (the padding also
    // spreads the runs' starts over the banks; unpadded, the lanes' run
    // reads conflict badly), keys with ITEMS elements of slack for candidate
    // reads past the last run; then payloads and splits.
    constexpr int kKeyWords = stage_word((kTile + ITEMS) * KW);
    constexpr int kPos = kKeyWords;
    constexpr int kPay = kPos + (KV ? stage_word(kTile) : 0);
    constexpr int kSplitAt = kPay + kTile * VW;
    __shared__ __attribute__((aligned(16))) int lds[kSplitAt + THREADS];
    int* const kbuf = lds;
    int* const pbuf = lds + kPos;
    int* const vbuf = lds + kPay;
    int* const split = lds + kSplitAt;

    const int tid = threadIdx.x;
    const int64_t t0 = blockIdx.x * static_cast<int64_t>(kTile);
    const int len = static_cast<int>(total - t0 < kTile ? total - t0 : kTile);
    // Whole tiles of 16-byte-aligned arrays move as 16-byte vectors.
    const bool vec_in = len == kTile && (reinterpret_cast<uintptr_t>(src + t0) & 15) == 0;
    const bool vec_out = len == kTile && (reinterpret_cast<uintptr_t>(dst + t0) & 15) == 0;

    // Load keys (coalesced) as order images; the tile's missing tail is the
    // largest image.
    if (vec_in) {
        const int32_t* const w = reinterpret_cast<const int32_t*>(src + t0);
#pragma unroll
        for (int r = 0; r < ITEMS * KW / 4; ++r) {
            const int q = 4 * (tid + r * THREADS);
            *reinterpret_cast<int4v*>(kbuf + stage_word(q)) =
                map_vec<ORDER, true>(load_stream4(w + q));
        }
    } else {
#pragma unroll
        for (int r = 0; r < ITEMS; ++r) {
            const int e = tid + r * THREADS;
            const Key x = e < len ? K::to_ord(src[t0 + e]) : K::kMax;
            st_elem<Key>(kbuf, stage_word(KW * e), x);
        }
    }
    if constexpr (KV) {
#pragma unroll
        for (int r = 0; r < ITEMS * VW; ++r) {
            const int w = tid + r * THREADS;
            if (w < len * VW) vbuf[w] = src_v[VW * t0 + w];
        }
    }
    __syncthreads();

    Key x[ITEMS];
    int pos[ITEMS];
    sort_tile<THREADS, ITEMS, KV>(kbuf, pbuf, split, x, pos, tid, K::kMax);
    __syncthreads();
    put_row<ITEMS>(kbuf, tid, x);
    if constexpr (KV) put_row<ITEMS>(pbuf, tid, pos);
    __syncthreads();

    // Store in tile order, coalesced; payloads follow their positions.
    if (vec_out) {
        int32_t* const w = reinterpret_cast<int32_t*>(dst + t0);
#pragma unroll
        for (int r = 0; r < ITEMS * KW / 4; ++r) {
            const int q = 4 * (tid + r * THREADS);
            store_stream4(w + q, map_vec<ORDER, false>(
                                     *reinterpret_cast<const int4v*>(kbuf + stage_word(q))));
        }
    } else {
#pragma unroll
        for (int r = 0; r < ITEMS; ++r) {
            const int e = tid + r * THREADS;
            if (e < len) dst[t0 + e] = K::from_ord(ld_elem<Key>(kbuf, stage_word(KW * e)));
        }
    }
    if constexpr (KV) {
#pragma unroll
        for (int r = 0; r < ITEMS; ++r) {
            const int e = tid + r * THREADS;
            if (e < len) {
                const int q = pbuf[stage_word(e)];
#pragma unroll
                for (int v = 0; v < VW; ++v) dst_v[VW * (t0 + e) + v] = vbuf[VW * q + v];
            }
        }
    }
}

// Block sort of 4-byte keys with payloads (VW words each) as 8-byte keys
// alone: element e of the tile sorts as the signed 64-bit value whose high
// word is its key's order image and whose low word is e.  These values are
// all distinct and order as (key, position), so sorting them is the stable
// order of the tile, with one 64-bit compare per exchange where the
// (key, position) pairs of block_sort_kernel take several.  Payloads stay
// in global memory: each lane gathers its outputs' payloads by position
// into registers, and a barrier separates every read of the tile from its
// writes (dst and dst_v may be src and src_v).  The tile's missing tail
// takes the largest image and positions past the end, which sort last and
// are never stored.
template <int THREADS, int ITEMS, int VW, int ORDER>
__global__ __launch_bounds__(THREADS) void block_sort_packed_kernel(
    const typename KeyOrder<ORDER>::T* src, const uint32_t* src_v, int64_t total,
    typename KeyOrder<ORDER>::T* dst, uint32_t* dst_v) {
    using K = KeyOrder<ORDER>;
    using P = long long;
    static_assert(K::kWords == 1 && VW > 0, "4-byte keys with payloads");
    static_assert(ITEMS >= 4 && (ITEMS & (ITEMS - 1)) == 0, "ITEMS: a power of two");
    static_assert(2 * ITEMS <= 32, "a lane's row fits in 32 words");
    constexpr int kTile = THREADS * ITEMS;
    constexpr int kKeyWords = stage_word((kTile + ITEMS) * 2);
    __shared__ __attribute__((aligned(16))) int lds[kKeyWords + THREADS];
    int* const kbuf = lds;
    int* const split = lds + kKeyWords;

    const int tid = threadIdx.x;
    const int64_t t0 = blockIdx.x * static_cast<int64_t>(kTile);
    const int len = static_cast<int>(total - t0 < kTile ? total - t0 : kTile);
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const int e = tid + r * THREADS;
        const int img = e < len ? K::to_ord(src[t0 + e]) : K::kMax;
        const uint64_t bits = (static_cast<uint64_t>(static_cast<uint32_t>(img)) << 32) |
                              static_cast<uint32_t>(e);
        st_elem<P>(kbuf, stage_word(2 * e), static_cast<P>(bits));
    }
    __syncthreads();

    P x[ITEMS];
    int pos[ITEMS];
    sort_tile<THREADS, ITEMS, false>(kbuf, kbuf, split, x, pos, tid,
                                     std::numeric_limits<P>::max());
    __syncthreads();
    put_row<ITEMS>(kbuf, tid, x);
    __syncthreads();

    // Output e = tid + r*THREADS (coalesced): its key, and its payload read
    // from the element's position before anything of the tile is written.
    int key[ITEMS];
    uint32_t pay[ITEMS][VW];
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const int e = tid + r * THREADS;
        key[r] = 0;
        if (e < len) {
            const P v = ld_elem<P>(kbuf, stage_word(2 * e));
            key[r] = K::from_ord(static_cast<int>(v >> 32));
            const int64_t q = t0 + static_cast<int>(static_cast<uint32_t>(v));
#pragma unroll
            for (int w = 0; w < VW; ++w) pay[r][w] = src_v[VW * q + w];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const int e = tid + r * THREADS;
        if (e < len) {
            dst[t0 + e] = key[r];
#pragma unroll
            for (int w = 0; w < VW; ++w) dst_v[VW * (t0 + e) + w] = pay[r][w];
        }
    }
}

// ---------------------------------------------------------------------------
// Batches of short merges.  One workgroup per tile of TILE outputs of the
// concatenated output C, whatever merges it holds: the plan finds the global
// co-rank (a, b) of every tile boundary (and the merge holding it); the tile
// kernel loads the tile's A and B ranges into LDS and cuts them into pieces
// at the merge starts that fall inside the tile.  Each lane finds the piece
// holding its first output and its co-rank inside that piece, then merges
// ITEMS outputs, passing into the next piece when one is exhausted (the A
// and B ranges of consecutive merges are consecutive).  Many short merges
// then share one workgroup instead of taking one each.

// Copies len elements (W words each, W = KeyOrder<ORDER>::kWords) from the
// global word array src to LDS words dst[0, W*len), mapping keys with
// to_ord (payloads use an identity order).  dst must sit at the same phase
// as src modulo 4 words, so 16-byte vectors line up on both sides; the
// partial vectors at the two ends (whole elements) go one element at a time.
template <int THREADS, int ORDER>
__device__ __forceinline__ void load_range(int* dst, const int32_t* src, int len, int tid) {
    using T = typename KeyOrder<ORDER>::T;
    constexpr int W = KeyOrder<ORDER>::kWords;
    const int words = W * len;
    const int head0 = (4 - (word_phase(src) & 3)) & 3;
    const int head = head0 < words ? head0 : words;
    const int nvec = (words - head) >> 2;
    const int tail = (words - head) & 3;
    for (int q = tid; q < nvec; q += THREADS) {
        const int w = head + 4 * q;
        *reinterpret_cast<int4v*>(dst + w) = map_vec<ORDER, true>(load_stream4(src + w));
    }
    if (W * tid < head) st_elem<T>(dst, W * tid, map_elem<ORDER, true>(ld_elem<T>(src, W * tid)));
    if (tid >= 4 && W * (tid - 3) <= tail) {
        const int w = head + 4 * nvec + W * (tid - 4);
        st_elem<T>(dst, w, map_elem<ORDER, true>(ld_elem<T>(src, w)));
    }
}

struct TileBound {
    int64_t a, b;  // global co-rank of the tile boundary: first A and B element
    int64_t p;     // merge holding the boundary
};

// Boundary w = 0..tiles of the tile grid: k = min(w*tile, m+n).  The merge
// holding it is found by first_start_after, guessed from an even share of
// the outputs per merge; then its co-rank inside that merge.
template <int G, int ORDER>
__global__ __launch_bounds__(256) void plan_tiles_kernel(
    const typename KeyOrder<ORDER>::T* __restrict__ A, const int64_t* __restrict__ a_off,
    int64_t m, const typename KeyOrder<ORDER>::T* __restrict__ B,
    const int64_t* __restrict__ b_off, int64_t n, int64_t pairs, int64_t tile, int64_t tiles,
    TileBound* __restrict__ tb) {
    static_assert(G >= 2, "group search");
    const int64_t gid = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
    if ((gid & ~int64_t(63)) / G > tiles) return;
    const int64_t w = gid / G;
    const bool live = w <= tiles;
    const int g_lane = static_cast<int>(gid % G);
    const int g_shift = static_cast<int>(threadIdx.x & 63) - g_lane;
    auto ao = [&](int64_t p) { return clamp_to<int64_t>(a_off[p], 0, m); };
    auto bo = [&](int64_t p) { return clamp_to<int64_t>(b_off[p], 0, n); };
    int64_t p = 0, k = 0, la = 0, lb = 0;
    const int64_t total = m + n;
    const int64_t c = live ? (w * tile < total ? w * tile : total) : 0;
    const double guess =
        total > 0 ? static_cast<double>(c) * static_cast<double>(pairs) / static_cast<double>(total)
                  : 0.0;
    const int64_t f = first_start_after<G>(
        c, pairs, guess, live, [&](int64_t x) { return ao(x) + bo(x); }, g_lane, g_shift);
    if (live) {
        p = f > 0 ? (f - 1 < pairs ? f - 1 : pairs - 1) : 0;
        const int64_t a1 = ao(p + 1), b1 = bo(p + 1);
        la = a1 > ao(p) ? a1 - ao(p) : 0;
        lb = b1 > bo(p) ? b1 - bo(p) : 0;
        k = clamp_to<int64_t>(c - (ao(p) + bo(p)), 0, la + lb);
    }
    const int64_t a_base = live ? ao(p) : 0, b_base = live ? bo(p) : 0;
    const int64_t i = co_rank_group<G, ORDER>(k, A + a_base, la, B + b_base, lb, g_lane, g_shift);
    if (!live || g_lane != 0) return;
    tb[w].a = a_base + i;
    tb[w].b = b_base + (k - i);
    tb[w].p = p;
}

// REG = true (keys alone, 16 words of output per lane: 4-byte keys x 16 or
// 8-byte keys x 8): each lane merges the slice direct_slice_wide gives it,
// and the tile leaves from registers (store_direct16, the quad transpose of
// the segment merge), with no LDS stage.  The launcher picks it when C is
// 16-byte aligned; every tile's output then is (tiles start at multiples of
// the tile length, a multiple of 4).
template <int THREADS, int ITEMS, int VW, int ORDER, bool REG = false>
__global__ __launch_bounds__(THREADS) void merge_tiles_kernel(
    const typename KeyOrder<ORDER>::T* __restrict__ A, const uint32_t* __restrict__ Av,
    const int64_t* __restrict__ a_off, int64_t m, const typename KeyOrder<ORDER>::T* __restrict__ B,
    const uint32_t* __restrict__ Bv, const int64_t* __restrict__ b_off, int64_t n, int64_t pairs,
    const TileBound* __restrict__ tb, typename KeyOrder<ORDER>::T* __restrict__ C,
    uint32_t* __restrict__ Cv) {
    using K = KeyOrder<ORDER>;
    using Key = typename K::T;
    constexpr int KW = K::kWords;
    constexpr bool KV = VW > 0;
    constexpr int VORDER = VW == 2 ? kKeyI64 : kKeyI32;
    constexpr int kTile = THREADS * ITEMS;
    static_assert(!REG || (VW == 0 && KW * ITEMS == 16), "register stores: 16 key words per lane");
    static_assert(kTile < 65536, "piece bounds are packed in 16 bits");
    // merge starts a tile holds in LDS (at least one candidate per lane)
    constexpr int kCap = kTile / 8 > THREADS ? kTile / 8 : THREADS;
    static_assert(kCap % THREADS == 0, "candidates per lane");
    constexpr int kWaves = THREADS / 64;
    // LDS: the tile's keys (A part, then B part) as images and its payloads;
    // once every lane holds its outputs in registers, the same words hold
    // the output stages (padded), unless the tile leaves from registers.
    // Then the piece bounds, each piece's first A and B index packed in one
    // word, and one count per wavefront.  A keys-only workgroup of 4-byte
    // keys needs 18.5 KB with register stores (8 share a CU) and 20.5 KB
    // with the stage (7).
    // (Each window has 8 spare words: its A and B parts each start at the
    // phase of their source modulo 4 words.)
    constexpr int kWin = 0;
    constexpr int kVWin = kWin + kTile * KW + 8;
    constexpr int kStage = 0;
    constexpr int kVStage = kStage + stage_word(kTile * KW);
    constexpr int kInWords = kVWin + (KV ? kTile * VW + 8 : 0);
    constexpr int kOutWords = REG ? 0 : kVStage + (KV ? stage_word(kTile * VW) : 0);
    constexpr int kPiece = kInWords > kOutWords ? kInWords : kOutWords;
    constexpr int kCount = kPiece + kCap + 2;
    __shared__ __attribute__((aligned(16))) int lds[kCount + kWaves];
    int* const win = lds + kWin;
    int* const vwin = lds + kVWin;
    // (no stage with register stores: its pointers are not used then)
    [[maybe_unused]] int* const stage = lds + (REG ? 0 : kStage);
    [[maybe_unused]] int* const vstage = lds + (REG ? 0 : kVStage);
    int* const pl = lds + kPiece;
    int* const cnt = lds + kCount;

    const int tid = threadIdx.x;
    const int64_t total = m + n;
    const int64_t k0 = blockIdx.x * static_cast<int64_t>(kTile);
    const int64_t k1 = k0 + kTile < total ? k0 + kTile : total;
    auto ao = [&](int64_t p) { return clamp_to<int64_t>(a_off[p], 0, m); };
    auto bo = [&](int64_t p) { return clamp_to<int64_t>(b_off[p], 0, n); };

    // Tile ranges, clamped into the arrays and the tile (any plan keeps
    // every access in range).
    const TileBound t0 = tb[blockIdx.x], t1 = tb[blockIdx.x + 1];
    const int64_t a0 = clamp_to<int64_t>(t0.a, 0, m);
    const int64_t b0 = clamp_to<int64_t>(t0.b, 0, n);
    const int c_max = static_cast<int>(k1 - k0);
    const int a_len = static_cast<int>(clamp_to<int64_t>(clamp_to<int64_t>(t1.a, a0, m) - a0, 0, c_max));
    const int b_len = static_cast<int>(clamp_to<int64_t>(clamp_to<int64_t>(t1.b, b0, n) - b0, 0,
                                                         c_max - a_len));
    const int c_len = a_len + b_len;
    const int64_t p0 = clamp_to<int64_t>(t0.p, 0, pairs > 0 ? pairs - 1 : 0);

    // Keys (as order images) and payloads of the tile: the A part at word
    // offA of the window, the B part at offB, each at its source's phase.
    const int32_t* const a_src = reinterpret_cast<const int32_t*>(A + a0);
    const int32_t* const b_src = reinterpret_cast<const int32_t*>(B + b0);
    const int offA = word_phase(a_src) & 3;
    const int offB = offA + KW * a_len + ((word_phase(b_src) - offA - KW * a_len) & 3);
    load_range<THREADS, ORDER>(win + offA, a_src, a_len, tid);
    load_range<THREADS, ORDER>(win + offB, b_src, b_len, tid);
    int vA = 0, vB = 0;
    if constexpr (KV) {
        const int32_t* const va_src = reinterpret_cast<const int32_t*>(Av) + VW * a0;
        const int32_t* const vb_src = reinterpret_cast<const int32_t*>(Bv) + VW * b0;
        vA = word_phase(va_src) & 3;
        vB = vA + VW * a_len + ((word_phase(vb_src) - vA - VW * a_len) & 3);
        load_range<THREADS, VORDER>(vwin + vA, va_src, a_len, tid);
        load_range<THREADS, VORDER>(vwin + vB, vb_src, b_len, tid);
    }
    // Pieces: piece 0 starts at the tile start; piece q >= 1 at the start of
    // merge p0+q when that start lies inside the tile.  The starts inside the
    // tile are a prefix of the candidates p0+1, p0+2, ..., and none is past
    // the merge that holds the tile's end (the next boundary's merge), so
    // only those candidates' offsets are read.
    const int64_t p_end = clamp_to<int64_t>(t1.p, p0, pairs > 0 ? pairs - 1 : 0);
    // The starts inside form a prefix of the candidates, so counting them
    // (ballots, then one count per wavefront) gives its length.
    int inside = 0;
#pragma unroll
    for (int r = 0; r < kCap / THREADS; ++r) {
        const int q = 1 + tid + r * THREADS;
        const int64_t p = p0 + q;
        bool in = false;
        if (p <= p_end) {
            const int64_t la = ao(p) - a0, lb = bo(p) - b0;
            in = la >= 0 && lb >= 0 && la + lb < c_len && la <= a_len && lb <= b_len;
            pl[q] = static_cast<int>(clamp_to<int64_t>(la, 0, a_len)) |
                    (static_cast<int>(clamp_to<int64_t>(lb, 0, b_len)) << 16);
        }
        inside += __popcll(__ballot(in));
    }
    if ((tid & 63) == 0) cnt[tid >> 6] = inside;
    if (tid == 0) pl[0] = 0;
    __syncthreads();
    int lo = 0;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) lo += cnt[wv];
    lo = lo < kCap ? lo : kCap;
    const int npieces = 1 + lo;
    // More merge starts than the LDS holds (only with many empty merges):
    // piece bounds are then read from the offsets in global memory.
    const bool overflow = lo == kCap && p0 + kCap + 1 <= p_end &&
                          ao(p0 + kCap + 1) + bo(p0 + kCap + 1) - k0 < c_len;
    int pieces = npieces;
    if (overflow) {
        int64_t l = p0 + kCap + 1, h = p_end + 1;  // merge starts inside the tile
        while (l < h) {
            const int64_t mid = (l + h) >> 1;
            if (ao(mid) + bo(mid) - k0 < c_len) l = mid + 1;
            else h = mid;
        }
        pieces = static_cast<int>(l - p0);
    }
    auto piece_a = [&](int q) -> int {
        if (q >= pieces) return a_len;
        if (q == 0) return 0;
        if (!overflow) return pl[q] & 0xFFFF;
        return static_cast<int>(clamp_to<int64_t>(ao(p0 + q) - a0, 0, a_len));
    };
    auto piece_b = [&](int q) -> int {
        if (q >= pieces) return b_len;
        if (q == 0) return 0;
        if (!overflow) return static_cast<int>(static_cast<unsigned>(pl[q]) >> 16);
        return static_cast<int>(clamp_to<int64_t>(bo(p0 + q) - b0, 0, b_len));
    };

    // The lane's slice: its first output (slice order of store_direct16
    // with register stores).
    const int o0 = (REG ? direct_slice_wide(tid) : tid) * ITEMS;
    Key x[ITEMS] = {};   // this lane's outputs (order images)
    int vx[ITEMS * (KV ? VW : 1)];  // their payload words
    if (o0 < c_len) {
        // The piece holding output o0: the last piece starting at or before it.
        int ql = 0, qh = pieces - 1;
        while (ql < qh) {
            const int mid = (ql + qh + 1) >> 1;
            if (piece_a(mid) + piece_b(mid) <= o0) ql = mid;
            else qh = mid - 1;
        }
        int q = ql;
        // Co-rank of o0 inside piece q (bisection, as in the segment merge).
        const int pa = piece_a(q), pb = piece_b(q);
        const int wa = piece_a(q + 1) - pa, wb = piece_b(q + 1) - pb;
        const int d = o0 - pa - pb;
        int lo2 = d > wb ? d - wb : 0, hi2 = d < wa ? d : wa;
        while (lo2 < hi2) {
            const int mid = (lo2 + hi2) >> 1;
            const Key av = ld_elem<Key>(win, offA + KW * (pa + mid));
            const Key bv = ld_elem<Key>(win, offB + KW * (pb + d - 1 - mid));
            if (av <= bv) lo2 = mid + 1;
            else hi2 = mid;
        }
        int i = pa + lo2, j = pb + (d - lo2);
        int ae = piece_a(q + 1), be = piece_b(q + 1);
        // Keys only, and all of this lane's outputs inside piece q: the
        // candidate network of the segment merge (ITEMS from each side,
        // masked at the piece's ends), which has no dependent LDS reads.
        const bool one_piece = !KV && o0 + ITEMS <= ae + be && o0 + ITEMS <= c_len;
        if (one_piece) {
            Key a[ITEMS], b[ITEMS];
#pragma unroll
            for (int t = 0; t < ITEMS; ++t) {
                a[t] = i + t < ae ? ld_elem<Key>(win, offA + KW * (i + t)) : K::kMax;
                b[t] = j + t < be ? ld_elem<Key>(win, offB + KW * (j + t)) : K::kMax;
            }
#pragma unroll
            for (int t = 0; t < ITEMS; ++t) x[t] = min(a[t], b[ITEMS - 1 - t]);
            bitonic_clean<ITEMS>(x);
        } else {
#pragma unroll
            for (int t = 0; t < ITEMS; ++t) {
                if (o0 + t < c_len) {
                    while (i == ae && j == be && q + 1 < pieces) {  // next merge
                        ++q;
                        ae = piece_a(q + 1);
                        be = piece_b(q + 1);
                    }
                    // (a side's end reads word 0 instead; that value is not taken)
                    const Key ka = ld_elem<Key>(win, i < a_len ? offA + KW * i : 0);
                    const Key kb = ld_elem<Key>(win, j < b_len ? offB + KW * j : 0);
                    const bool take_a = i < ae && (j >= be || ka <= kb);
                    x[t] = take_a ? ka : kb;
                    if constexpr (KV) {
                        const int src = take_a ? vA + VW * i : vB + VW * j;
#pragma unroll
                        for (int v = 0; v < VW; ++v) vx[VW * t + v] = vwin[src + v];
                    }
                    i += take_a ? 1 : 0;
                    j += take_a ? 0 : 1;
                }
            }
        }
    }
    if constexpr (REG) {
        // From registers: the wavefront's 64 slices as four 1 KB runs.
        int w[16];
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) {
            if constexpr (KW == 1) {
                w[t] = static_cast<int>(x[t]);
            } else {
                w[2 * t] = low_word(x[t]);
                w[2 * t + 1] = high_word(x[t]);
            }
        }
        const bool aligned = (word_phase(C + k0) & 3) == 0;
        store_direct16<ORDER>(reinterpret_cast<int32_t*>(C + k0), (tid >> 6) * 64 * ITEMS * KW,
                              KW * c_len, aligned, w, tid);
        return;
    }
    __syncthreads();  // the window is read; its words now hold the stages
    if (o0 < c_len) {
        int* const row = stage + stage_word(tid * ITEMS * KW);
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) {
            if (o0 + t < c_len) st_elem<Key>(row, KW * t, x[t]);
        }
        if constexpr (KV) {
            int* const vrow = vstage + stage_word(tid * ITEMS * VW);
#pragma unroll
            for (int t = 0; t < ITEMS * VW; ++t) {
                if (o0 + t / VW < c_len) vrow[t] = vx[t];
            }
        }
    }
    __syncthreads();
    constexpr int kVec = kTile * KW / 4 / THREADS;
    store_tile<THREADS, kVec, ORDER>(reinterpret_cast<int32_t*>(C + k0), KW * c_len, stage, tid);
    if constexpr (KV) {
        constexpr int kVVec = kTile * VW / 4 / THREADS;
        store_tile<THREADS, kVVec, VORDER>(reinterpret_cast<int32_t*>(Cv) + VW * k0, VW * c_len,
                                           vstage, tid);
    }
}

}  // namespace omerge
