// multiway_kernel.hpp -- the 4-way pass of the merge sort.
//
// Page "Practice - Sorting Foundations and Parallel Radix Sort"
// (pmpp.huatsai.dev/13-sorting/practice-sorting), its merge-sort item: the
// late stages of a merge sort are a few large merges, each cut into
// independent pieces by co-rank (page "Co-rank Function ... and Basic
// Parallel Merge Kernel").  A 2-way pass reads and writes every element once
// per doubling of the run length.  This pass merges runs four at a time
// (runs 4g .. 4g+3 into one), so the data crosses HBM once for two
// doublings.  Its output is that of two 2-way passes: the stable merge of
// the four runs, the earlier run first on equal keys.
//
// Splitting a 4-way merge.  Write X = merge(R0, R1) and Y = merge(R2, R3),
// neither formed in HBM; the group's output is merge(X, Y), X first on ties.
// A split of the output is four counts (i0, i1, i2, i3), how many elements
// of each run come before it.  Splits are taken at sample points, each with
// one co-rank and two bound searches, never a nested search:
//   * X point j is the element X[j*q].  The co-rank of j*q in (R0, R1) gives
//     (i0, i1), and the element is the first of R0[i0] and R1[i1] (R0 on
//     ties).  The elements of Y before it are those with smaller keys, so i2
//     and i3 are its key's lower bounds in R2 and R3.
//   * Y point j is the element Y[j*q], with (i2, i3) from the co-rank in
//     (R2, R3); the elements of X before it are those with keys no larger,
//     so i0 and i1 are upper bounds in R0 and R1.
// A point's output position is i0+i1+i2+i3.  The points of both kinds, in
// output order, cut the group into cells; a cell starts at a point (or the
// group's start) and ends at the next.  A cell holds at most q elements of
// X, since it contains no X point but its first element, and at most q of
// Y.  Y point j' comes before an X point exactly when Y[j'q] is among the
// i2+i3 elements of Y that come before it, so the number of Y points before
// it is the number of multiples of q in (0, i2+i3): each point knows its
// cell's index without sorting the points (and the same the other way).
//
// One workgroup merges one cell.  It loads the four windows into LDS
// (16-byte loads of the aligned body of each window, each followed by a
// block of sentinels: the largest key image), merges R0|R1 and R2|R3 there
// (each lane finds its slice by co-rank and orders its candidates with the
// min/max network of the block sort; the sentinels stand in for candidates
// past a window's end), writes X and Y back as padded rows, each side
// followed by a sentinel row, merges X|Y the same way, and stores the cell
// through the padded stage with 16-byte stores.  Keys only: equal keys are
// indistinguishable in a key-only output, so the splits fix every output
// bit, and a sentinel equal to a real key changes no output.
#pragma once

#include "batch_kernel.hpp"

namespace omerge {

// One cell of a 4-way pass: the window [s[r], e[r]) of run r of its group
// (absolute element indices into the pass's source) and its first output.
struct Cell4 {
    int64_t s[4];
    int64_t e[4];
    int64_t c0;
};

// Number of elements of the sorted S[0, len) that come before the key whose
// order image is v: those with S[i] < v when `strict` (a lower bound), with
// S[i] <= v otherwise (an upper bound).  G lanes per search (G divides 64),
// all lanes of the wavefront together (the votes and shuffles are
// wavefront-wide).  Each round tests G points of [lo, hi); the passing
// points form a prefix, and the answer lies after the last passing point
// and at or before the first failing one.  After the first (even) round the
// points go around the linear interpolation of where the images cross v,
// as in co_rank_group, and a round that narrows the interval less than an
// even split would turns interpolation off.  The interval update is exact
// whatever the placement, and every round shrinks it.
//
// A caller that knows more passes an interval [lo_in, hi_in] holding the
// answer (intersected with [0, len]) and a guess inside it; the first round
// then places its points around the guess, spread by 0.7*sqrt(width),
// unless that would cover more than half the interval.
template <int G, int ORDER>
__device__ __forceinline__ int64_t rank_group(typename KeyOrder<ORDER>::T v, bool strict,
                                              const typename KeyOrder<ORDER>::T* __restrict__ S,
                                              int64_t len, int g_lane, int g_shift,
                                              int64_t lo_in = 0, int64_t hi_in = INT64_MAX,
                                              double guess = -1.0) {
    static_assert(G >= 2 && G <= 64 && (64 % G) == 0, "group size");
    constexpr int kLog = bit_length(G) - 1;
    int64_t lo = lo_in > 0 ? (lo_in < len ? lo_in : len) : 0;
    int64_t hi = hi_in < len ? (hi_in > lo ? hi_in : lo) : len;
    // g = image - v - target is below 0 exactly at passing points.
    const double target = strict ? -0.5 : 0.5;
    double g_lo = 0.0, g_hi = 0.0;
    bool have_lo = false, have_hi = false;
    bool even_only = !OMERGE_PART_INTERP;
    for (int round = 0; round < 64; ++round) {
        if (__ballot(lo < hi) == 0) break;
        const int64_t span = hi - lo;
        double centre = 0.0, spread = 0.0;
        bool interp = false;
        if (round == 0 && guess >= 0.0 && OMERGE_PART_INTERP) {
            centre = guess;
            spread = fmax(1.0, 0.7 * sqrt(static_cast<double>(span)));
            interp = (G - 1) * spread < 0.5 * static_cast<double>(span);
        } else if (!even_only && have_lo && have_hi && g_hi > g_lo) {
            const double w = static_cast<double>(span + 1);  // from lo - 1 to hi
            const double unit = w / (g_hi - g_lo);
            centre = static_cast<double>(lo - 1) - g_lo * unit;
            spread = fmax(1.0, fmax(0.7 * sqrt(w), 0.5 * unit));
            interp = (G - 1) * spread < 0.5 * static_cast<double>(span);
        }
        const int64_t q = span >> kLog, r = span & (G - 1);
        const int live = interp || span >= G ? G : static_cast<int>(span);
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
            const auto s = KeyOrder<ORDER>::to_ord(S[p]);
            pass = strict ? s < v : s <= v;
            g = static_cast<double>(s) - static_cast<double>(v) - target;
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

// Geometry of one 4-way pass over `total` elements in runs of `run`: groups
// of four runs, full groups and a short last one, sample points every q
// elements of X and of Y, and cells.
struct MultiwayPlan {
    int64_t groups, full_groups;
    int64_t pts_full, cells_full;  // per full group
    int64_t points, cells;         // whole pass

    __host__ __device__ static int64_t inner_points(int64_t len, int64_t q) {
        return len > 0 ? (len + q - 1) / q - 1 : 0;  // multiples of q inside (0, len)
    }
    __host__ __device__ static MultiwayPlan make(int64_t total, int64_t run, int64_t q) {
        MultiwayPlan p;
        p.full_groups = total / (4 * run);
        const int64_t rem = total - p.full_groups * 4 * run;
        p.groups = p.full_groups + (rem > 0 ? 1 : 0);
        p.pts_full = 2 * inner_points(2 * run, q);
        p.cells_full = 1 + p.pts_full;
        const int64_t lx = rem < 2 * run ? rem : 2 * run;
        const int64_t last_pts = inner_points(lx, q) + inner_points(rem - lx, q);
        p.points = p.full_groups * p.pts_full + (rem > 0 ? last_pts : 0);
        p.cells = p.full_groups * p.cells_full + (rem > 0 ? 1 + last_pts : 0);
        return p;
    }
};

// An entry of the 4-way plan: sample point j (from 1) on side X or Y of
// group g, or (point = false) the start of group g.
struct MultiwayEntry {
    int64_t g, j;
    bool point, side_y;
};

__device__ __forceinline__ MultiwayEntry multiway_entry(int64_t w, int64_t total, int64_t run,
                                                        int64_t q, const MultiwayPlan& plan) {
    MultiwayEntry e{0, 0, w < plan.points, false};
    if (e.point) {
        const int64_t half = plan.pts_full / 2;
        if (w < plan.full_groups * plan.pts_full) {
            e.g = w / plan.pts_full;
            const int64_t r = w % plan.pts_full;
            e.side_y = r >= half;
            e.j = (e.side_y ? r - half : r) + 1;
        } else {
            e.g = plan.full_groups;
            const int64_t r = w - plan.full_groups * plan.pts_full;
            const int64_t rem = total - e.g * 4 * run;
            const int64_t nx = MultiwayPlan::inner_points(rem < 2 * run ? rem : 2 * run, q);
            e.side_y = r >= nx;
            e.j = (e.side_y ? r - nx : r) + 1;
        }
    } else {
        e.g = w - plan.points;
    }
    return e;
}

// The four counts of a point (runs R0..R3 of its group before its element),
// by a G-lane group: the co-rank of j*q in the point's own pair, then bounds
// of its element in the other pair's two runs (lanes [0, G/2) and [G/2, G)).
// Each search may be narrowed to [lo[r], hi[r]] with a guess (< 0: none).
// Every lane of the wavefront calls this; lanes that are not a point search
// empty ranges.  Arrays are indexed by constants only (a lane's pair by
// selects), so they stay in registers.
template <int G, int ORDER>
__device__ __forceinline__ void multiway_counts(
    const typename KeyOrder<ORDER>::T* __restrict__ src, const MultiwayEntry& e,
    const int64_t (&start)[4], const int64_t (&len)[4], int64_t q, int g_lane, int g_shift,
    const int64_t (&lo)[4], const int64_t (&hi)[4], const double (&guess)[4], int64_t (&cnt)[4]) {
    using K = KeyOrder<ORDER>;
    using Key = typename K::T;
    constexpr int H = G / 2;
    const bool y = e.side_y;
    // own pair (A, B) and the other pair (C, D)
    const int64_t sa = y ? start[2] : start[0], sb = y ? start[3] : start[1];
    const int64_t sc = y ? start[0] : start[2], sd = y ? start[1] : start[3];
    const int64_t la = e.point ? (y ? len[2] : len[0]) : 0;
    const int64_t lb = e.point ? (y ? len[3] : len[1]) : 0;
    const int64_t lc = e.point ? (y ? len[0] : len[2]) : 0;
    const int64_t ld = e.point ? (y ? len[1] : len[3]) : 0;
    const int64_t k2 = e.point ? e.j * q : 0;
    const int64_t i_first = co_rank_group<G, ORDER>(k2, src + sa, la, src + sb, lb, g_lane, g_shift,
                                                    y ? lo[2] : lo[0], y ? hi[2] : hi[0],
                                                    y ? guess[2] : guess[0]);
    const int64_t i_second = k2 - i_first;
    Key v = 0;
    if (e.point) {  // the point's element: the first of the two heads, the first run on ties
        const bool first = i_first < la && (i_second >= lb || K::to_ord(src[sa + i_first]) <=
                                                                   K::to_ord(src[sb + i_second]));
        v = K::to_ord(first ? src[sa + i_first] : src[sb + i_second]);
    }
    // lower bounds for an X point, upper bounds for a Y point
    const bool h = g_lane >= H;
    const int sub_lane = g_lane % H;
    const int sub_shift = static_cast<int>(threadIdx.x & 63) - sub_lane;
    const int64_t lo_c = y ? lo[0] : lo[2], lo_d = y ? lo[1] : lo[3];
    const int64_t hi_c = y ? hi[0] : hi[2], hi_d = y ? hi[1] : hi[3];
    const double gu_c = y ? guess[0] : guess[2], gu_d = y ? guess[1] : guess[3];
    const int64_t c = rank_group<H, ORDER>(v, !y, src + (h ? sd : sc), h ? ld : lc, sub_lane,
                                           sub_shift, h ? lo_d : lo_c, h ? hi_d : hi_c,
                                           h ? gu_d : gu_c);
    const int64_t c_first = static_cast<int64_t>(__shfl(static_cast<double>(c), g_shift));
    const int64_t c_second = static_cast<int64_t>(__shfl(static_cast<double>(c), g_shift + H));
    cnt[0] = y ? c_first : i_first;
    cnt[1] = y ? c_second : i_second;
    cnt[2] = y ? i_first : c_first;
    cnt[3] = y ? i_second : c_second;
}

// Plan of one 4-way pass.  Entries 0 .. points-1 are the sample points (per
// group: its X points j = 1, 2, ... then its Y points); entries points ..
// points+groups are the starts of the groups and, last, the end of the pass.
// A point writes the start of its cell and the end of the one before; a
// group start writes the start of the group's first cell and the end of the
// previous group's last cell.
//
// One G-lane group per entry, 256/G consecutive entries per workgroup, in
// two phases (as the partition kernel): phase 1 searches every STRIDE-th
// entry (and the first of the next workgroup) over whole runs; phase 2
// searches each other point inside the bounds its two searched neighbours
// give when both are points of the same side of the same group: along a
// side, the co-rank in the own pair never falls and grows by at most one
// per output, and the counts in the other pair never fall (the points'
// elements rise), so each count lies between the neighbours', with the
// first probes around the straight line between them.
template <int G, int ORDER, int STRIDE = 8>
__device__ __forceinline__ void plan_multiway_body(
    const typename KeyOrder<ORDER>::T* __restrict__ src, int64_t total, int64_t run, int64_t q,
    const MultiwayPlan& plan, Cell4* __restrict__ cells) {
    static_assert(G >= 4 && G <= 64 && (64 % G) == 0, "group search");
    constexpr int kGroups = 256 / G;  // entries per workgroup
    constexpr int kStride = kGroups >= STRIDE ? STRIDE : kGroups;
    constexpr int kCoarse = kGroups / kStride + 1;
    constexpr int kPhase1Lanes = (kCoarse * G + 63) / 64 * 64;
    __shared__ int64_t coarse_cnt[kCoarse][4];
    __shared__ int64_t coarse_id[kCoarse][2];  // group, and side*2^62 + j (-1: not a point)
    const int tid = threadIdx.x;
    const int64_t entries = plan.points + plan.groups + 1;
    const int64_t s0 = blockIdx.x * static_cast<int64_t>(kGroups);
    auto geometry = [&](const MultiwayEntry& e, int64_t (&start)[4], int64_t (&len)[4]) {
        const int64_t gbase = e.g * 4 * run;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t s = gbase + r * run;
            start[r] = s < total ? s : total;
            const int64_t t = s + run < total ? s + run : total;
            len[r] = t - start[r];
        }
    };
    const int64_t kNone[4] = {0, 0, 0, 0};
    const int64_t kAll[4] = {INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX};
    const double kNoGuess[4] = {-1.0, -1.0, -1.0, -1.0};

    // Phase 1.
    if (tid < kPhase1Lanes) {
        const int grp = tid / G, g_lane = tid % G;
        const int g_shift = (tid & 63) - g_lane;
        const int64_t w = s0 + static_cast<int64_t>(kStride) * grp;
        const bool act = grp < kCoarse && w < entries;
        MultiwayEntry e = multiway_entry(act ? w : entries, total, run, q, plan);
        e.point = e.point && act;
        int64_t start[4], len[4], cnt[4];
        geometry(e, start, len);
        multiway_counts<G, ORDER>(src, e, start, len, q, g_lane, g_shift, kNone, kAll, kNoGuess,
                                  cnt);
        if (act && g_lane == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) coarse_cnt[grp][r] = cnt[r];
            coarse_id[grp][0] = e.g;
            coarse_id[grp][1] = e.point ? (static_cast<int64_t>(e.side_y) << 62) + e.j : -1;
        } else if (grp < kCoarse && g_lane == 0) {
            coarse_id[grp][0] = -1;
            coarse_id[grp][1] = -1;
        }
    }
    __syncthreads();

    // Phase 2.
    const int grp = tid / G, g_lane = tid % G;
    const int g_shift = (tid & 63) - g_lane;
    const int64_t w = s0 + grp;
    if (s0 + (tid & ~63) / G >= entries) return;  // the whole wavefront is past the end
    const bool live = w < entries;
    const int jc = grp / kStride;
    const bool known = grp % kStride == 0;
    MultiwayEntry e = multiway_entry(live ? w : entries, total, run, q, plan);
    int64_t start[4], len[4], cnt[4];
    geometry(e, start, len);
    int64_t lo[4] = {0, 0, 0, 0}, hi[4] = {INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX};
    double guess[4] = {-1.0, -1.0, -1.0, -1.0};
    const int64_t my_id = (static_cast<int64_t>(e.side_y) << 62) + e.j;
    const bool narrow = live && e.point && !known && coarse_id[jc][0] == e.g &&
                        coarse_id[jc + 1][0] == e.g && coarse_id[jc][1] >= 0 &&
                        coarse_id[jc + 1][1] >= 0 &&
                        (coarse_id[jc][1] >> 62) == (my_id >> 62) &&
                        (coarse_id[jc + 1][1] >> 62) == (my_id >> 62);
    if (narrow) {
        const int64_t j0 = coarse_id[jc][1] & ((int64_t(1) << 62) - 1);
        const int64_t j1 = coarse_id[jc + 1][1] & ((int64_t(1) << 62) - 1);
        const double f = static_cast<double>(e.j - j0) / static_cast<double>(j1 - j0);
        const int pa = e.side_y ? 2 : 0;  // first run of the point's own pair
        const int64_t x = e.j * q, x0 = j0 * q, x1 = j1 * q;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t c0 = coarse_cnt[jc][r], c1 = coarse_cnt[jc + 1][r];
            // each count between the neighbours'; the own pair's co-rank of
            // x = j*q also within (x - x0) above and (x1 - x) below them
            int64_t l = c0, u = c1;
            if (r == pa) {
                l = c1 - (x1 - x) > c0 ? c1 - (x1 - x) : c0;
                u = c0 + (x - x0) < c1 ? c0 + (x - x0) : c1;
            }
            lo[r] = l;
            hi[r] = u;
            const double gs = static_cast<double>(c0) + f * static_cast<double>(c1 - c0);
            guess[r] = gs >= static_cast<double>(l) ? gs : -1.0;
        }
    }
    MultiwayEntry es = e;
    es.point = e.point && live && !known;
    multiway_counts<G, ORDER>(src, es, start, len, q, g_lane, g_shift, lo, hi, guess, cnt);
    if (!live || g_lane != 0) return;
    if (known) {
#pragma unroll
        for (int r = 0; r < 4; ++r) cnt[r] = coarse_cnt[jc][r];
    }

    if (e.point) {
        const int64_t other = e.side_y ? cnt[0] + cnt[1] : cnt[2] + cnt[3];  // other pair's elements before
        const int64_t cell = e.g * plan.cells_full + e.j + (other > 0 ? (other - 1) / q : 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            cells[cell].s[r] = start[r] + cnt[r];
            cells[cell - 1].e[r] = start[r] + cnt[r];
        }
        cells[cell].c0 = e.g * 4 * run + cnt[0] + cnt[1] + cnt[2] + cnt[3];
        return;
    }
    const int64_t hg = e.g;  // group start hg; hg == groups: the end of the pass
    if (hg < plan.groups) {
        const int64_t cell = hg * plan.cells_full;
        const int64_t b = hg * 4 * run;
#pragma unroll
        for (int r = 0; r < 4; ++r) cells[cell].s[r] = b + r * run < total ? b + r * run : total;
        cells[cell].c0 = b;
    }
    if (hg > 0) {
        const int64_t prev = hg == plan.groups ? plan.cells - 1 : hg * plan.cells_full - 1;
        const int64_t b = (hg - 1) * 4 * run;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            cells[prev].e[r] = b + (r + 1) * run < total ? b + (r + 1) * run : total;
    }
}

template <int G, int ORDER>
__global__ __launch_bounds__(256) void plan_multiway_kernel(
    const typename KeyOrder<ORDER>::T* __restrict__ src, int64_t total, int64_t run, int64_t q,
    MultiwayPlan plan, Cell4* __restrict__ cells) {
    plan_multiway_body<G, ORDER>(src, total, run, q, plan, cells);
}

// Co-rank of output rank k of the merge of A (la elements from LDS word aw)
// and B (lb from bw), by binary lifting: the largest x in [max(0, k-lb),
// min(k, la)] with A[x-1] <= B[k-x] (true at the low end; the passing points
// form a prefix).  The steps STEP, STEP/2, ..., 1 reach 2*STEP-1 past the
// low end, so STEP is at least half the interval's width.  Every read stays
// inside the arrays: the A index is clamped at 0, and B is read at most one
// element past its end (a sentinel).  Words are plain LDS words, or pass
// through the stage padding when PADDED.
template <int STEP, int KW, bool PADDED, typename Key>
__device__ __forceinline__ int co_rank_lds(const int* lds, int aw, int la, int bw, int lb, int k) {
    const int lo = k > lb ? k - lb : 0, hi = k < la ? k : la;
    int x = lo;
#pragma unroll
    for (int step = STEP; step > 0; step >>= 1) {
        const int p = x + step;
        const int c = p < hi ? p : hi;
        const int wa = aw + KW * (c > 0 ? c - 1 : 0), wb = bw + KW * (k - c);
        const Key a = ld_elem<Key>(lds, PADDED ? stage_word(wa) : wa);
        const Key b = ld_elem<Key>(lds, PADDED ? stage_word(wb) : wb);
        x = (p <= hi && a <= b) ? p : x;
    }
    return x;
}

// Calls f(t, element t) for the ITEMS elements of KW words that start at
// LDS word w.  In the padded layout (4 spare words after every 32) a window
// of at most 32 words crosses at most one pad: word j of it sits j words
// after the window's first, or 4 more once j reaches the pad, so each
// element is one of two reads (both made, both inside the array), chosen by
// one compare and one select.  Elements of 8 bytes start on even words and
// never straddle a pad.
template <int ITEMS, int KW, bool PADDED, typename Key, typename F>
__device__ __forceinline__ void for_window(const int* lds, int w, F f) {
    if constexpr (!PADDED) {
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) f(t, ld_elem<Key>(lds, w + KW * t));
    } else {
        static_assert(ITEMS * KW <= 32, "a window crosses at most one pad");
        const int* const base = lds + stage_word(w);
        const int ca = 32 - (w & 31);  // words before the next pad
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) {
            const Key before = ld_elem<Key>(base, KW * t);
            const Key after = ld_elem<Key>(base, KW * t + 4);
            f(t, KW * t < ca ? before : after);
        }
    }
}

// The lane's outputs [k0, k0 + ITEMS) of the merge of A and B in LDS,
// ascending, in x: from the co-rank of k0, the ITEMS smallest of the next
// ITEMS candidates of each side, by the min/max network.  Every side is
// followed by ITEMS sentinels (the largest image), so candidates past a
// side's end need no masking, and outputs past the merge's end are the
// largest image.  B's candidates fold into the network's first stage as
// they arrive, which keeps half the candidates out of registers.
template <int ITEMS, int STEP, int KW, bool PADDED, typename Key>
__device__ __forceinline__ void merge_slice_lds(const int* lds, int aw, int la, int bw, int lb,
                                                int k0, Key (&x)[ITEMS]) {
    const int sa = co_rank_lds<STEP, KW, PADDED, Key>(lds, aw, la, bw, lb, k0);
    for_window<ITEMS, KW, PADDED, Key>(lds, aw + KW * sa, [&](int t, Key e) { x[t] = e; });
    for_window<ITEMS, KW, PADDED, Key>(lds, bw + KW * (k0 - sa), [&](int t, Key e) {
        x[ITEMS - 1 - t] = min(x[ITEMS - 1 - t], e);
    });
    bitonic_clean<ITEMS>(x);
}

// Word j of a row of sentinels: the largest order image, KW words per key.
template <int KW>
__device__ __forceinline__ int sentinel_word(int j) {
    return KW == 1 || (j & 1) ? 0x7FFFFFFF : -1;
}

// LDS of the cell kernel.  Level 1 reads plain words: R0's window at its
// global word phase mod 4, a block of kRow sentinel words, R1 the same way,
// then from kYIn R2 and R3 likewise.  A pair's windows hold at most kQ
// elements and each window start moves up by at most 3 words to its phase.
// Level 2 reads padded rows of kRow words (the stage layout, which keeps the
// lanes' row writes free of bank conflicts): X's rows, a sentinel row, Y's
// rows, a sentinel row, at most THREADS + 2 rows, and 4 words past them that
// candidate reads may touch.  Level 2 then overwrites the rows with the
// cell's outputs, which leave through the stage.
template <int THREADS, int ITEMS, int KW>
struct MultiwayCfg {
    static constexpr int kQ = THREADS * ITEMS / 2;  // at most kQ elements of X and of Y per cell
    static constexpr int kRow = ITEMS * KW;         // words of a lane's slice and of a sentinel block
    static constexpr int kYIn = kQ * KW + 2 * kRow + 8;
    static constexpr int kIn = 2 * kYIn;
    static constexpr int kOut = stage_word((THREADS + 2) * kRow + 4) + 4;
    static constexpr int kLds = kIn > kOut ? kIn : kOut;
    static constexpr int kVec = ITEMS * KW / 4;      // 16-byte loads / stores per lane
    static constexpr int kLoose = 2 * (4 / KW - 1);  // end elements per window
    static constexpr int kStep1 = kQ / 2;  // level 1: widths at most kQ/2 (a pair holds kQ)
    static constexpr int kStep2 = kQ;      // level 2: widths at most kQ
    // Wavefronts per SIMD that the LDS allows (160 KB per CU, 4 SIMDs), at
    // most 8: the register budget follows from it.
    static constexpr int kWorkgroupsPerCu = (160 * 1024) / (4 * kLds);
    static constexpr int kWavesPerSimd =
        kWorkgroupsPerCu * THREADS / 256 < 8 ? (kWorkgroupsPerCu * THREADS / 256 > 0
                                                    ? kWorkgroupsPerCu * THREADS / 256
                                                    : 1)
                                             : 8;
    static_assert((ITEMS * KW) % 4 == 0, "rows of whole 16-byte vectors");
    static_assert((kQ & (kQ - 1)) == 0, "kQ: a power of two");
    static_assert(4 * kRow <= THREADS, "one lane per sentinel word");
};

// A cell's windows in words: global start, length, LDS start (the same
// phase mod 4), and the split into a head (up to the first 16-byte
// boundary), 16-byte body vectors and a tail.  Uniform over the workgroup.
struct CellWindows {
    int64_t gw[4], s[4], c0;
    int len[4], ow[4], head[4], nvec[4], tail[4];
};

// The descriptor's fields are clamped so that whatever it holds (unsorted
// runs give plans whose cells may collide or be left unwritten), every
// access stays inside the n-element source and output: windows inside
// [0, n), each pair's windows at most Q elements together (the LDS bound),
// and the cell's outputs inside [0, n).  On a plan of sorted runs the
// clamps change nothing.  GAP sentinel words follow each window.
template <int KW, int Y_IN, int Q, int GAP>
__device__ __forceinline__ CellWindows cell_windows(const Cell4& d, const int32_t* src32,
                                                    int64_t n) {
    CellWindows g;
    int64_t len64[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        g.s[r] = clamp_to<int64_t>(d.s[r], 0, n);
        len64[r] = clamp_to<int64_t>(d.e[r], g.s[r], n) - g.s[r];
    }
    len64[0] = len64[0] < Q ? len64[0] : Q;
    len64[1] = len64[1] < Q - len64[0] ? len64[1] : Q - len64[0];
    len64[2] = len64[2] < Q ? len64[2] : Q;
    len64[3] = len64[3] < Q - len64[2] ? len64[3] : Q - len64[2];
    const int64_t total = len64[0] + len64[1] + len64[2] + len64[3];
    g.c0 = clamp_to<int64_t>(d.c0, 0, n - total);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        g.len[r] = static_cast<int>(len64[r]);
        g.gw[r] = KW * g.s[r];
        const int nw = KW * g.len[r];
        const int ph = word_phase(src32 + g.gw[r]) & 3;
        const int h0 = (4 - ph) & 3;
        g.head[r] = h0 < nw ? h0 : nw;
        g.nvec[r] = (nw - g.head[r]) >> 2;
        g.tail[r] = (nw - g.head[r]) & 3;
        const int base = r == 0   ? 0
                         : r == 1 ? g.ow[0] + KW * g.len[0] + GAP
                         : r == 2 ? Y_IN
                                  : g.ow[2] + KW * g.len[2] + GAP;
        g.ow[r] = base + ((ph - base) & 3);
    }
    return g;
}

__device__ __forceinline__ int sel4(int r, int a, int b, int c, int e) {
    return r == 0 ? a : r == 1 ? b : r == 2 ? c : e;
}
__device__ __forceinline__ int64_t sel4(int r, int64_t a, int64_t b, int64_t c, int64_t e) {
    return r == 0 ? a : r == 1 ? b : r == 2 ? c : e;
}

// A cell's loads in flight: body vector qq of the concatenated windows
// (run r holds q_r <= qq < q_{r+1}) and at most one end element per lane.
template <int V, typename Key>
struct CellLoads {
    int4v body[V];
    Key loose;
    int loose_w;  // LDS word of the loose element, -1: none
};

template <int THREADS, int V, int KW, int LOOSE, typename Key>
__device__ __forceinline__ void issue_cell(const CellWindows& g, const Key* __restrict__ src,
                                           int tid, CellLoads<V, Key>& ld) {
    const int32_t* const src32 = reinterpret_cast<const int32_t*>(src);
    const int q1 = g.nvec[0], q2 = q1 + g.nvec[1], q3 = q2 + g.nvec[2], q4 = q3 + g.nvec[3];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int qq = tid + v * THREADS;
        const int r = qq < q1 ? 0 : qq < q2 ? 1 : qq < q3 ? 2 : 3;
        const int qi = qq - sel4(r, 0, q1, q2, q3);
        const int64_t g0 = sel4(r, g.gw[0] + g.head[0], g.gw[1] + g.head[1],
                                g.gw[2] + g.head[2], g.gw[3] + g.head[3]);
        if (qq < q4) ld.body[v] = load_stream4(src32 + g0 + 4 * qi);
    }
    ld.loose = 0;
    ld.loose_w = -1;
    if (tid < 4 * LOOSE) {
        const int r = tid / LOOSE, z = tid % LOOSE, zh = LOOSE / 2;
        const int hr = sel4(r, g.head[0], g.head[1], g.head[2], g.head[3]);
        const int nr = sel4(r, g.nvec[0], g.nvec[1], g.nvec[2], g.nvec[3]);
        const int tr = sel4(r, g.tail[0], g.tail[1], g.tail[2], g.tail[3]);
        const int e = z < zh ? z : (hr + 4 * nr) / KW + (z - zh);
        const bool have = z < zh ? KW * z < hr : KW * (z - zh) < tr;
        if (have) {
            ld.loose = src[sel4(r, g.s[0], g.s[1], g.s[2], g.s[3]) + e];
            ld.loose_w = sel4(r, g.ow[0], g.ow[1], g.ow[2], g.ow[3]) + KW * e;
        }
    }
}

template <int THREADS, int V, int KW, int ORDER, typename Key>
__device__ __forceinline__ void commit_cell(const CellWindows& g, const CellLoads<V, Key>& ld,
                                            int tid, int* lds) {
    const int q1 = g.nvec[0], q2 = q1 + g.nvec[1], q3 = q2 + g.nvec[2], q4 = q3 + g.nvec[3];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int qq = tid + v * THREADS;
        const int r = qq < q1 ? 0 : qq < q2 ? 1 : qq < q3 ? 2 : 3;
        const int qi = qq - sel4(r, 0, q1, q2, q3);
        const int l0 = sel4(r, g.ow[0] + g.head[0], g.ow[1] + g.head[1], g.ow[2] + g.head[2],
                            g.ow[3] + g.head[3]);
        if (qq < q4)
            *reinterpret_cast<int4v*>(lds + l0 + 4 * qi) = map_vec<ORDER, true>(ld.body[v]);
    }
    if (ld.loose_w >= 0) st_elem<Key>(lds, ld.loose_w, KeyOrder<ORDER>::to_ord(ld.loose));
    // the sentinel block after each window
    constexpr int kRow = V * 4;
    if (tid < 4 * kRow) {
        const int r = tid / kRow, j = tid % kRow;
        const int end = sel4(r, g.ow[0] + KW * g.len[0], g.ow[1] + KW * g.len[1],
                             g.ow[2] + KW * g.len[2], g.ow[3] + KW * g.len[3]);
        lds[end + j] = sentinel_word<KW>(j);
    }
}

// Body vectors of a cell's output from the padded stage, whose word j is
// output word j: vector i covers words [HEAD + 4i, HEAD + 4i + 4), which
// take the last 4 - HEAD words of stage quad i and the first HEAD of quad
// i + 1 (quads never straddle the padding).  HEAD is the output's phase,
// uniform, so the shift costs no instruction.
template <int THREADS, int V, int ORDER, int HEAD>
__device__ __forceinline__ void store_cell_body(int32_t* __restrict__ dst, int nvec,
                                                const int* stage, int tid) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int i = tid + v * THREADS;
        if (i < nvec) {
            const int4v a = *reinterpret_cast<const int4v*>(stage + stage_word(4 * i));
            int4v x = a;
            if constexpr (HEAD > 0) {
                const int4v b = *reinterpret_cast<const int4v*>(stage + stage_word(4 * i + 4));
                if constexpr (HEAD == 1) x = int4v{a.y, a.z, a.w, b.x};
                if constexpr (HEAD == 2) x = int4v{a.z, a.w, b.x, b.y};
                if constexpr (HEAD == 3) x = int4v{a.w, b.x, b.y, b.z};
            }
            store_stream4(dst + HEAD + 4 * i, map_vec<ORDER, false>(x));
        }
    }
}

// Stores a cell's len output words from the padded stage to dst: 16-byte
// stores on the aligned body, single elements before and after it.
template <int THREADS, int V, int ORDER>
__device__ __forceinline__ void store_cell(int32_t* __restrict__ dst, int len, const int* stage,
                                           int tid) {
    using T = typename KeyOrder<ORDER>::T;
    constexpr int W = KeyOrder<ORDER>::kWords;
    const int head0 = (4 - (word_phase(dst) & 3)) & 3;
    const int head = head0 < len ? head0 : len;
    const int nvec = (len - head) >> 2;
    const int tail = (len - head) & 3;
    switch (head) {
        case 0: store_cell_body<THREADS, V, ORDER, 0>(dst, nvec, stage, tid); break;
        case 1: store_cell_body<THREADS, V, ORDER, 1>(dst, nvec, stage, tid); break;
        case 2: store_cell_body<THREADS, V, ORDER, 2>(dst, nvec, stage, tid); break;
        default: store_cell_body<THREADS, V, ORDER, 3>(dst, nvec, stage, tid); break;
    }
    int* const d = reinterpret_cast<int*>(dst);
    if (W * tid < head)
        st_elem<T>(d, W * tid, map_elem<ORDER, false>(ld_elem<T>(stage, stage_word(W * tid))));
    if (tid >= 4 && W * (tid - 3) <= tail) {
        const int p = head + 4 * nvec + W * (tid - 4);
        st_elem<T>(d, p, map_elem<ORDER, false>(ld_elem<T>(stage, stage_word(p))));
    }
}

// One workgroup merges cells [blockIdx.x*CPW, +CPW) of the pass, one after
// another; the next cell's loads are issued as soon as the current cell is
// in LDS and stay in registers while it is merged.
template <int THREADS, int ITEMS, int CPW, int ORDER>
__global__ __launch_bounds__(
    THREADS, (MultiwayCfg<THREADS, ITEMS, KeyOrder<ORDER>::kWords>::kWavesPerSimd)) void
merge_multiway_kernel(
    const typename KeyOrder<ORDER>::T* __restrict__ src, int64_t n,
    const Cell4* __restrict__ cells, int64_t ncells,
    typename KeyOrder<ORDER>::T* __restrict__ dst) {
    using K = KeyOrder<ORDER>;
    using Key = typename K::T;
    constexpr int KW = K::kWords;
    using Cfg = MultiwayCfg<THREADS, ITEMS, KW>;
    __shared__ __attribute__((aligned(16))) int lds[Cfg::kLds];
    const int tid = threadIdx.x;
    const int32_t* const src32 = reinterpret_cast<const int32_t*>(src);
    const int64_t c_first = static_cast<int64_t>(blockIdx.x) * CPW;
    const int64_t c_end = c_first + CPW < ncells ? c_first + CPW : ncells;

    CellWindows nxt = cell_windows<KW, Cfg::kYIn, Cfg::kQ, Cfg::kRow>(cells[c_first], src32, n);
    CellLoads<Cfg::kVec, Key> ld;
    issue_cell<THREADS, Cfg::kVec, KW, Cfg::kLoose>(nxt, src, tid, ld);
    for (int64_t c = c_first; c < c_end; ++c) {
        if (c > c_first) __syncthreads();  // the previous cell's stores have read the stage
        const CellWindows cur = nxt;
        commit_cell<THREADS, Cfg::kVec, KW, ORDER>(cur, ld, tid, lds);
        __syncthreads();
        if (c + 1 < c_end) {
            nxt = cell_windows<KW, Cfg::kYIn, Cfg::kQ, Cfg::kRow>(cells[c + 1], src32, n);
            issue_cell<THREADS, Cfg::kVec, KW, Cfg::kLoose>(nxt, src, tid, ld);
        }

        // Level 1: R0|R1 into X and R2|R3 into Y, ITEMS outputs per lane:
        // lanes [0, nx) take X's slices and lanes [nx, nx+ny) Y's.  A cell
        // averages half its bound, so about half the wavefronts have no
        // slice; their branch is skipped whole (the merges dominate the
        // kernel's VALU work).
        const int lx = cur.len[0] + cur.len[1], ly = cur.len[2] + cur.len[3];
        const int total = lx + ly;
        const int nx = (lx + ITEMS - 1) / ITEMS, ny = (ly + ITEMS - 1) / ITEMS;
        Key x[ITEMS];
        if (tid < nx + ny) {
            const bool side_y = tid >= nx;
            const int u = tid - (side_y ? nx : 0);
            const int la = side_y ? cur.len[2] : cur.len[0];
            const int lb = side_y ? cur.len[3] : cur.len[1];
            const int k0 = u * ITEMS < la + lb ? u * ITEMS : la + lb;
            merge_slice_lds<ITEMS, Cfg::kStep1, KW, false>(lds, side_y ? cur.ow[2] : cur.ow[0], la,
                                                          side_y ? cur.ow[3] : cur.ow[1], lb, k0, x);
        }
        __syncthreads();  // every read of the inputs is done
        // X's rows, a sentinel row, Y's rows, a sentinel row
        if (tid < nx + ny) put_row<ITEMS>(lds, tid < nx ? tid : tid + 1, x);
        if (tid < 2 * Cfg::kRow) {
            const int row = tid < Cfg::kRow ? nx : nx + 1 + ny;
            const int j = tid % Cfg::kRow;
            lds[stage_word(row * Cfg::kRow + j)] = sentinel_word<KW>(j);
        }
        __syncthreads();

        // Level 2: X|Y into the cell's outputs, lanes [0, ceil(total/ITEMS)).
        if (tid * ITEMS < total)
            merge_slice_lds<ITEMS, Cfg::kStep2, KW, true>(lds, 0, lx, (nx + 1) * Cfg::kRow, ly,
                                                         tid * ITEMS, x);
        __syncthreads();
        if (tid * ITEMS < total) put_row<ITEMS>(lds, tid, x);
        __syncthreads();
        store_cell<THREADS, Cfg::kVec, ORDER>(reinterpret_cast<int32_t*>(dst) + KW * cur.c0,
                                              KW * total, lds, tid);
    }
}

}  // namespace omerge
