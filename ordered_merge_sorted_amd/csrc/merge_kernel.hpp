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
//     and the tile goes back to HBM through an LDS stage with coalesced
//     16-byte stores.
//
// gfx950 choices (none of these is on the pages):
//   * Ring slot of an element = its absolute element address (address/4)
//     modulo the power-of-two ring capacity.  A 16-byte-aligned vector in HBM
//     then lands on a 16-byte-aligned slot quad, so refills are
//     global_load_dwordx4 + ds_write_b128 with no wrap inside a vector.
//     Partial vectors at the two ends of a refill are loaded one element at
//     a time (never past the range, so never past the array).
//   * The refill for tile t+1 is issued into registers as soon as tile t's
//     split is known, before tile t is merged, and written to LDS only after
//     tile t's stores; the HBM latency hides behind the merge.
//   * Each lane searches the END of its slice; its start is its left
//     neighbour's end, read from a small LDS array, and the last lane's end
//     is the tile's split.  One search per lane per tile.
//   * The LDS stage is padded by one word every 32 so that lanes writing
//     their ITEMS outputs at stride ITEMS spread over the banks.
//   * All arithmetic is int32 compares and index arithmetic; no MFMA.
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

template <typename T>
__device__ __forceinline__ T clamp_to(T x, T lo, T hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

// Element-address phase: (address / 4) of p, as an int (only low bits used).
__device__ __forceinline__ int word_phase(const void* p) {
    return static_cast<int>(reinterpret_cast<uintptr_t>(p) >> 2);
}

template <int THREADS, int ITEMS, bool KV>
struct MergeCfg {
    static_assert(THREADS % 64 == 0, "whole 64-lane wavefronts");
    static_assert(ITEMS % 4 == 0, "refills and stores move 4 elements per lane");
    static constexpr int kTile = THREADS * ITEMS;  // outputs per tile
    static constexpr int kCap = next_pow2(kTile);  // ring capacity per side
    static constexpr int kMask = kCap - 1;
    static constexpr int kVec = ITEMS / 4;  // 16-byte vectors per lane per refill
    static constexpr int kStageWords = kTile + kTile / 32 + 1;
    // LDS layout in 32-bit words.
    static constexpr int kRing = 0;  // keys: A ring [0,kCap), B ring [kCap,2kCap)
    static constexpr int kValRing = kRing + 2 * kCap;  // payload rings (KV)
    static constexpr int kStage = kValRing + (KV ? 2 * kCap : 0);
    static constexpr int kValStage = kStage + kStageWords;
    static constexpr int kSplit = kValStage + (KV ? kStageWords : 0);
    static constexpr int kWords = kSplit + THREADS;
    static constexpr int kLdsBytes = kWords * 4;
};

// Padded stage index: one spare word every 32.
__device__ __forceinline__ int stage_at(int p) { return p + (p >> 5); }

// ---------------------------------------------------------------------------
// Partition and co-rank query kernels.

__global__ void partition_kernel(const int32_t* __restrict__ A, int64_t m,
                                 const int32_t* __restrict__ B, int64_t n,
                                 int64_t seg_len, int64_t count,
                                 int64_t* __restrict__ part) {
    const int64_t s = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
    if (s >= count) return;
    const int64_t total = m + n;
    const int64_t k = s < count - 1 ? s * seg_len : total;
    part[s] = co_rank_global(k, A, m, B, n);
}

__global__ void co_rank_kernel(const int32_t* __restrict__ A, int64_t m,
                               const int32_t* __restrict__ B, int64_t n,
                               const int64_t* __restrict__ ks, int64_t count,
                               int64_t* __restrict__ out) {
    const int64_t s = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
    if (s >= count) return;
    const int64_t k = clamp_to<int64_t>(ks[s], 0, m + n);
    out[s] = co_rank_global(k, A, m, B, n);
}

// ---------------------------------------------------------------------------
// Ring refill: copies a segment-relative range [r0, r1) of one side into its
// ring.  Issue and commit are split so the loads can be in flight while the
// current tile is merged.  Body vectors of side A and side B share one lane
// assignment, so a refill of at most TILE elements needs kVec vectors per
// lane.  Up to 3 head and 3 tail elements per side are loaded one by one by
// lanes 0..11.

struct SideRange {
    const int32_t* src;  // segment base of this array in global memory
    int base;            // ring slot of segment-relative index 0
    int r0;              // first segment-relative index to load
    int head;            // elements before the first 16-byte boundary
    int nvec;            // whole 16-byte vectors
    int tail;            // elements after the last whole vector

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

template <int THREADS, int ITEMS, int MASK>
struct Refill {
    static constexpr int kVec = ITEMS / 4;
    int4v body[kVec];
    int loose;        // one head/tail element (lanes 0..11)
    int loose_slot;   // its ring word index, or -1
    SideRange sa, sb;

    __device__ __forceinline__ void issue(const SideRange& a, const SideRange& b,
                                          int tid) {
        sa = a;
        sb = b;
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
            const int q = tid + v * THREADS;
            if (q < sa.nvec) {
                body[v] = *reinterpret_cast<const int4v*>(sa.src + sa.r0 + sa.head + 4 * q);
            } else if (q - sa.nvec < sb.nvec) {
                const int qb = q - sa.nvec;
                body[v] = *reinterpret_cast<const int4v*>(sb.src + sb.r0 + sb.head + 4 * qb);
            }
        }
        loose_slot = -1;
        if (tid < 12) {
            const SideRange& s = tid < 6 ? sa : sb;
            const int w = tid < 6 ? tid : tid - 6;
            int r = -1;
            if (w < 3) {
                if (w < s.head) r = s.r0 + w;
            } else if (w - 3 < s.tail) {
                r = s.r0 + s.head + 4 * s.nvec + (w - 3);
            }
            if (r >= 0) {
                loose = s.src[r];
                loose_slot = ((s.base + r) & MASK) + (tid < 6 ? 0 : MASK + 1);
            }
        }
    }

    // ring points at the A ring; the B ring follows it at MASK+1 words.
    __device__ __forceinline__ void commit(int* ring, int tid) const {
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
            const int q = tid + v * THREADS;
            if (q < sa.nvec) {
                const int slot = (sa.base + sa.r0 + sa.head + 4 * q) & MASK;
                *reinterpret_cast<int4v*>(ring + slot) = body[v];
            } else if (q - sa.nvec < sb.nvec) {
                const int qb = q - sa.nvec;
                const int slot = (sb.base + sb.r0 + sb.head + 4 * qb) & MASK;
                *reinterpret_cast<int4v*>(ring + MASK + 1 + slot) = body[v];
            }
        }
        if (loose_slot >= 0) ring[loose_slot] = loose;
    }
};

// Stores tile outputs [0, len) from the padded LDS stage to dst[0, len):
// 16-byte stores on the aligned body, single words at the ends.
template <int THREADS, int ITEMS>
__device__ __forceinline__ void store_tile(int32_t* __restrict__ dst, int len,
                                           const int* stage, int tid) {
    const int head0 = (4 - (word_phase(dst) & 3)) & 3;
    const int head = head0 < len ? head0 : len;
    const int nvec = (len - head) >> 2;
    const int tail = (len - head) & 3;
#pragma unroll
    for (int v = 0; v < ITEMS / 4; ++v) {
        const int q = tid + v * THREADS;
        if (q < nvec) {
            const int p = head + 4 * q;
            int4v x;
            x.x = stage[stage_at(p)];
            x.y = stage[stage_at(p + 1)];
            x.z = stage[stage_at(p + 2)];
            x.w = stage[stage_at(p + 3)];
            *reinterpret_cast<int4v*>(dst + p) = x;
        }
    }
    if (tid < head) dst[tid] = stage[stage_at(tid)];
    if (tid >= 4 && tid - 4 < tail) {
        const int p = head + 4 * nvec + (tid - 4);
        dst[p] = stage[stage_at(p)];
    }
}

// ---------------------------------------------------------------------------
// Segment merge kernel: one workgroup per segment of the output.

template <int THREADS, int ITEMS, bool KV>
__global__ __launch_bounds__(THREADS) void merge_segments_kernel(
    const int32_t* __restrict__ A, const uint32_t* __restrict__ Av, int64_t m,
    const int32_t* __restrict__ B, const uint32_t* __restrict__ Bv, int64_t n,
    const int64_t* __restrict__ part, int64_t seg_len,
    int32_t* __restrict__ C, uint32_t* __restrict__ Cv) {
    using Cfg = MergeCfg<THREADS, ITEMS, KV>;
    constexpr int kTile = Cfg::kTile;
    constexpr int kCap = Cfg::kCap;
    constexpr int kMask = Cfg::kMask;
    __shared__ __attribute__((aligned(16))) int lds[Cfg::kWords];
    int* const ring = lds + Cfg::kRing;
    int* const vring = lds + Cfg::kValRing;
    int* const stage = lds + Cfg::kStage;
    int* const vstage = lds + Cfg::kValStage;
    int* const split = lds + Cfg::kSplit;

    const int tid = threadIdx.x;
    const int64_t total = m + n;
    const int64_t seg = blockIdx.x;
    const int64_t k0 = seg * seg_len;
    const int64_t k1 = k0 + seg_len < total ? k0 + seg_len : total;
    const int c_len = static_cast<int>(k1 - k0);

    // Segment windows from the partition, clamped so that any partition
    // (even one made from unsorted input) keeps every access in range.
    const int64_t i0 = clamp_to<int64_t>(part[seg], k0 > n ? k0 - n : 0, k0 < m ? k0 : m);
    const int64_t i1 = clamp_to<int64_t>(part[seg + 1], k1 > n ? k1 - n : 0, k1 < m ? k1 : m);
    const int a_len = static_cast<int>(clamp_to<int64_t>(i1 - i0, 0, c_len));
    const int b_len = c_len - a_len;
    const int64_t j0 = k0 - i0;

    const int32_t* const As = A + i0;
    const int32_t* const Bs = B + j0;
    int32_t* const Cs = C + k0;
    const int a_base = word_phase(As) & kMask;
    const int b_base = word_phase(Bs) & kMask;
    // Payload rings use their own arrays' phases; d_a/d_b map a key slot to
    // the payload slot of the same element.
    const int32_t* const Avs = KV ? reinterpret_cast<const int32_t*>(Av + i0) : nullptr;
    const int32_t* const Bvs = KV ? reinterpret_cast<const int32_t*>(Bv + j0) : nullptr;
    const int va_base = KV ? (word_phase(Avs) & kMask) : 0;
    const int vb_base = KV ? (word_phase(Bvs) & kMask) : 0;
    const int d_a = (va_base - a_base) & kMask;
    const int d_b = (vb_base - b_base) & kMask;

    int a_cons = 0, b_cons = 0;  // consumed so far (segment-relative)
    int a_loaded = a_len < kTile ? a_len : kTile;
    int b_loaded = b_len < kTile ? b_len : kTile;

    // Initial fill: up to one tile of each side.
    {
        SideRange ra, rb, none;
        none.set(As, a_base, 0, 0);
        Refill<THREADS, ITEMS, kMask> fa, fb;
        ra.set(As, a_base, 0, a_loaded);
        rb.set(Bs, b_base, 0, b_loaded);
        fa.issue(ra, none, tid);
        fb.issue(none, rb, tid);
        fa.commit(ring, tid);
        fb.commit(ring, tid);
        if (KV) {
            SideRange va, vb, vnone;
            vnone.set(Avs, va_base, 0, 0);
            va.set(Avs, va_base, 0, a_loaded);
            vb.set(Bvs, vb_base, 0, b_loaded);
            fa.issue(va, vnone, tid);
            fb.issue(vnone, vb, tid);
            fa.commit(vring, tid);
            fb.commit(vring, tid);
        }
    }
    __syncthreads();

    for (int c_done = 0; c_done < c_len;) {
        const int c_tile = c_len - c_done < kTile ? c_len - c_done : kTile;
        const int wa = a_loaded - a_cons;  // A window in the ring: min(TILE, left)
        const int wb = b_loaded - b_cons;
        const int sa = (a_base + a_cons) & kMask;  // slot of the window's first A
        const int sb = (b_base + b_cons) & kMask;

        // Co-rank of the end of this lane's slice, searched in the ring.
        const int c_end = (tid + 1) * ITEMS < c_tile ? (tid + 1) * ITEMS : c_tile;
        const int e = co_rank<int>(
            c_end, wa, wb, [=](int x) { return ring[(sa + x) & kMask]; },
            [=](int x) { return ring[kCap + ((sb + x) & kMask)]; }, kMaxStepsTile);
        split[tid] = e;
        __syncthreads();
        // A elements this tile consumes; the same for every lane, so it is
        // moved to a scalar register and the refill bookkeeping stays scalar.
        const int x_t = __builtin_amdgcn_readfirstlane(split[THREADS - 1]);
        const int c_beg = tid * ITEMS < c_tile ? tid * ITEMS : c_tile;
        const int s = tid > 0 ? split[tid - 1] : 0;

        // Prefetch the next refill: exactly what this tile consumes, clamped
        // to what is left of the segment.
        const int a_cons2 = a_cons + x_t;
        const int b_cons2 = b_cons + (c_tile - x_t);
        const int a_loaded2 = a_cons2 + kTile < a_len ? a_cons2 + kTile : a_len;
        const int b_loaded2 = b_cons2 + kTile < b_len ? b_cons2 + kTile : b_len;
        Refill<THREADS, ITEMS, kMask> rf, rv;
        {
            SideRange ra, rb;
            ra.set(As, a_base, a_loaded, a_loaded2);
            rb.set(Bs, b_base, b_loaded, b_loaded2);
            rf.issue(ra, rb, tid);
            if (KV) {
                SideRange va, vb;
                va.set(Avs, va_base, a_loaded, a_loaded2);
                vb.set(Bvs, vb_base, b_loaded, b_loaded2);
                rv.issue(va, vb, tid);
            }
        }

        // Sequential merge of this lane's slice, in registers.
        int out[ITEMS];
        int src[ITEMS];
        {
            int a = s;
            int b = c_beg - s;
            const int a_end = e;
            const int b_end = c_end - e;
            int ka = ring[(sa + a) & kMask];
            int kb = ring[kCap + ((sb + b) & kMask)];
#pragma unroll
            for (int t = 0; t < ITEMS; ++t) {
                const bool take_a = a < a_end && (b >= b_end || ka <= kb);
                out[t] = take_a ? ka : kb;
                if (KV) {
                    src[t] = take_a ? Cfg::kValRing + ((sa + a + d_a) & kMask)
                                    : Cfg::kValRing + kCap + ((sb + b + d_b) & kMask);
                }
                a += take_a ? 1 : 0;
                b += take_a ? 0 : 1;
                if (t + 1 < ITEMS) {
                    const int w = take_a ? ((sa + a) & kMask) : kCap + ((sb + b) & kMask);
                    const int nxt = ring[w];
                    ka = take_a ? nxt : ka;
                    kb = take_a ? kb : nxt;
                }
            }
        }
        const int my_len = c_end - c_beg;
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) {
            if (t < my_len) {
                stage[stage_at(c_beg + t)] = out[t];
                if (KV) vstage[stage_at(c_beg + t)] = lds[src[t]];
            }
        }
        __syncthreads();

        store_tile<THREADS, ITEMS>(Cs + c_done, c_tile, stage, tid);
        if (KV) {
            store_tile<THREADS, ITEMS>(reinterpret_cast<int32_t*>(Cv + k0) + c_done,
                                       c_tile, vstage, tid);
        }
        rf.commit(ring, tid);
        if (KV) rv.commit(vring, tid);

        a_cons = a_cons2;
        b_cons = b_cons2;
        a_loaded = a_loaded2;
        b_loaded = b_loaded2;
        c_done += c_tile;
        __syncthreads();
    }
}

}  // namespace omerge
