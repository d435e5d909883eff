// CPU emulation of the HIP kernels, for tests only.  It compiles the product
// kernel headers unchanged against the stand-in HIP header next to it and
// runs each workgroup as THREADS host threads that meet at a std::barrier.
// Workgroups run one after another.  Exposes extern "C" entry points that the
// tests call through ctypes.
#include <algorithm>
#include <barrier>
#include <cstdlib>
#include <functional>
#include <thread>
#include <vector>

#include "hip/hip_runtime.h"
#include "multiway_kernel.hpp"

thread_local EmuDim3 threadIdx;
thread_local EmuDim3 blockIdx;
EmuDim3 blockDim;
EmuDim3 gridDim;

static std::barrier<>* g_barrier = nullptr;
void __syncthreads() { g_barrier->arrive_and_wait(); }

// Per-wavefront vote: lanes post their predicate, meet, read all 64, meet again.
struct WaveVote {
    std::barrier<> bar{64};
    int pred[64] = {};
    double val[64] = {};
    int ival[64] = {};
};
static std::vector<WaveVote>* g_waves = nullptr;
unsigned long long __ballot(int pred) {
    WaveVote& w = (*g_waves)[threadIdx.x / 64];
    const int lane = threadIdx.x % 64;
    w.pred[lane] = pred != 0;
    w.bar.arrive_and_wait();
    unsigned long long mask = 0;
    for (int l = 0; l < 64; ++l) mask |= static_cast<unsigned long long>(w.pred[l]) << l;
    w.bar.arrive_and_wait();
    return mask;
}

double __shfl(double var, int src) {
    WaveVote& w = (*g_waves)[threadIdx.x / 64];
    const int lane = threadIdx.x % 64;
    w.val[lane] = var;
    w.bar.arrive_and_wait();
    const double got = w.val[src & 63];
    w.bar.arrive_and_wait();
    return got;
}

int __shfl_xor(int var, int mask) {
    WaveVote& w = (*g_waves)[threadIdx.x / 64];
    const int lane = threadIdx.x % 64;
    w.ival[lane] = var;
    w.bar.arrive_and_wait();
    const int got = w.ival[(lane ^ mask) & 63];
    w.bar.arrive_and_wait();
    return got;
}

// Posts var for the caller's lane, reads lane `src` of the same wavefront.
static int wave_read(int var, int src) {
    WaveVote& w = (*g_waves)[threadIdx.x / 64];
    const int lane = threadIdx.x % 64;
    w.ival[lane] = var;
    w.bar.arrive_and_wait();
    const int got = w.ival[src & 63];
    w.bar.arrive_and_wait();
    return got;
}

int __builtin_amdgcn_update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask,
                                bool bound_ctrl) {
    (void)old;
    (void)bound_ctrl;
    if (row_mask != 0xF || bank_mask != 0xF) abort();
    const int lane = threadIdx.x % 64;
    const int row = lane & ~15, i = lane & 15;
    int from;
    if (ctrl >= 0 && ctrl <= 0xFF) {  // quad_perm: lane q of a quad reads quad lane sel[q]
        from = (lane & ~3) | ((ctrl >> (2 * (lane & 3))) & 3);
    } else if (ctrl >= 0x121 && ctrl <= 0x12F) {  // row_ror:n, rotate right within the row
        const int n = ctrl - 0x120;
        from = row | ((i + n) & 15);
    } else if (ctrl == 0x140) {  // row_mirror
        from = row | (15 - i);
    } else if (ctrl == 0x141) {  // row_half_mirror
        from = row | (i & 8) | (7 - (i & 7));
    } else {
        abort();
    }
    return wave_read(src, from);
}

int __builtin_amdgcn_mov_dpp(int src, int ctrl, int row_mask, int bank_mask, bool bound_ctrl) {
    return __builtin_amdgcn_update_dpp(0, src, ctrl, row_mask, bank_mask, bound_ctrl);
}

int __builtin_amdgcn_ds_swizzle(int src, int pattern) {
    if (pattern & 0x8000) abort();  // only bit mode
    const int and_mask = pattern & 31, or_mask = (pattern >> 5) & 31, xor_mask = (pattern >> 10) & 31;
    const int lane = threadIdx.x % 64;
    const int from = (lane & 32) | ((((lane & 31) & and_mask) | or_mask) ^ xor_mask);
    return wave_read(src, from);
}

// Runs `body` for every workgroup 0..blocks-1 with `threads` lanes each.
static void run_grid(int64_t blocks, int threads, const std::function<void()>& body) {
    std::barrier<> bar(threads);
    g_barrier = &bar;
    std::vector<WaveVote> waves(threads / 64);
    g_waves = &waves;
    blockDim = {static_cast<unsigned>(threads), 1, 1};
    gridDim = {static_cast<unsigned>(blocks), 1, 1};
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t) {
        pool.emplace_back([&, t] {
            threadIdx = {static_cast<unsigned>(t), 0, 0};
            for (int64_t b = 0; b < blocks; ++b) {
                blockIdx = {static_cast<unsigned>(b), 0, 0};
                body();
                bar.arrive_and_wait();  // the workgroup is done before the next starts
            }
        });
    }
    for (auto& th : pool) th.join();
    g_barrier = nullptr;
}

// The library's choice of store path: tiles leave from registers (REG) for
// 4-byte keys with no or 4-byte payloads and 8 outputs per lane, when every
// segment output is 16-byte aligned; otherwise through the LDS stage.
template <int I, int VW, int ORDER>
constexpr bool reg_shape() {
    constexpr int kw = omerge::KeyOrder<ORDER>::kWords;
    return ((kw == 1 && VW <= 1) || (kw == 2 && VW == 0)) && I == 8;
}
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Runs merge_segments_kernel<T, I, VW, ORDER, DESC, reg, SELF> over
// `blocks` workgroups (reg only where the shape allows it; SELF: each
// workgroup finds its own boundaries and part is not read).
template <int T, int I, int VW, int ORDER, bool DESC, bool SELF = false>
static void run_merge(bool reg, int64_t blocks, const typename omerge::KeyOrder<ORDER>::T* A,
                      const uint32_t* Av, int64_t m, const typename omerge::KeyOrder<ORDER>::T* B,
                      const uint32_t* Bv, int64_t n, const int64_t* part, int64_t seg_len,
                      typename omerge::KeyOrder<ORDER>::T* C, uint32_t* Cv,
                      const omerge::SegDesc* desc, int64_t c_total) {
    if constexpr (reg_shape<I, VW, ORDER>()) {
        if (reg) {
            run_grid(blocks, T, [&] {
                omerge::merge_segments_kernel<T, I, VW, ORDER, DESC, true, SELF>(
                    A, Av, m, B, Bv, n, part, seg_len, C, Cv, desc, c_total);
            });
            return;
        }
    }
    run_grid(blocks, T, [&] {
        omerge::merge_segments_kernel<T, I, VW, ORDER, DESC, false, SELF>(
            A, Av, m, B, Bv, n, part, seg_len, C, Cv, desc, c_total);
    });
}

// Partition + merge for one key order, payload width VW (words) and shape.
// self: one launch whose workgroups find their own boundaries (the
// partition is still written, for the caller's check, but not read).
template <int T, int I, int VW, int ORDER>
static void typed_cfg(const void* A, const void* Av, int64_t m, const void* B, const void* Bv,
                      int64_t n, int64_t seg_len, int64_t* part, void* C, void* Cv,
                      bool self = false) {
    using Key = typename omerge::KeyOrder<ORDER>::T;
    const Key* a = static_cast<const Key*>(A);
    const Key* b = static_cast<const Key*>(B);
    const int64_t count = (m + n + seg_len - 1) / seg_len + 1;
    // the library's partition shapes: 8 lanes per boundary and every 8th
    // boundary first for at most 49,152 boundaries, else 4 and 16
    if (count <= 49152)
        run_grid((count * 8 + 255) / 256, 256, [&] {
            omerge::partition_kernel<8, ORDER, 8, 8>(a, m, b, n, seg_len, count, part);
        });
    else
        run_grid((count * 4 + 255) / 256, 256, [&] {
            omerge::partition_kernel<4, ORDER, 4, 16>(a, m, b, n, seg_len, count, part);
        });
    if (m + n == 0) return;
    const bool reg = aligned16(C) && (VW == 0 || aligned16(Cv));
    if (self)
        run_merge<T, I, VW, ORDER, false, true>(reg, count - 1, a, static_cast<const uint32_t*>(Av),
                                                m, b, static_cast<const uint32_t*>(Bv), n, nullptr,
                                                seg_len, static_cast<Key*>(C),
                                                static_cast<uint32_t*>(Cv), nullptr, m + n);
    else
        run_merge<T, I, VW, ORDER, false>(reg, count - 1, a, static_cast<const uint32_t*>(Av), m,
                                          b, static_cast<const uint32_t*>(Bv), n, part, seg_len,
                                          static_cast<Key*>(C), static_cast<uint32_t*>(Cv), nullptr,
                                          m + n);
}

// Outputs per lane of the library's shapes (its items_for).
constexpr int production_items(int kw, int vw) {
    return kw == 1 && vw == 0 ? 8 : (kw + vw == 2 ? 8 : 4);
}
// Outputs per lane of the library's block sort (32 for 4-byte keys alone,
// 8 for 4-byte keys with payloads, packed) and of its tile path for short
// merges (16 for 4-byte keys alone), else the segment merge's count.
constexpr int production_sort_items(int kw, int vw) {
    return kw == 1 && vw == 0 ? 32 : kw == 1 ? 8 : production_items(kw, vw);
}
constexpr int production_tile_items(int kw, int vw) {
    return kw == 1 && vw == 0 ? 16 : production_items(kw, vw);
}
// Lanes of the library's block sort for each shape.
constexpr int production_sort_threads(int kw, int vw) {
    return kw == 1 && vw == 0 ? 512 : kw == 1 ? 1024 : kw == 2 && vw == 0 ? 1024 : 512;
}

// Which (order, payload words, shape) combinations this library holds:
// small shapes (128 lanes, 4 items) for every order keys-only and for a
// spread of orders with payloads; the library's shapes for float32 and
// float64 descending with every payload width.
constexpr bool emu_has(int variant, int order, int vw) {
    if (variant == 0) return order == (2 | 8) || order == (5 | 8);
    if (vw == 0) return true;
    if (vw == 1) return order == 0 || order == (2 | 8) || order == 3 || order == (5 | 8);
    return order == 1 || order == (3 | 8) || order == 5;
}

// variant | 2: the same shapes with each workgroup finding its own boundaries.
template <int ORDER, int VW>
static bool typed_go(int variant, const void* A, const void* Av, int64_t m, const void* B,
                     const void* Bv, int64_t n, int64_t seg_len, int64_t* part, void* C,
                     void* Cv) {
    const bool self = (variant & 2) != 0;
    variant &= 1;
    if constexpr (emu_has(1, ORDER, VW)) {
        if (variant == 1) {
            typed_cfg<128, 4, VW, ORDER>(A, Av, m, B, Bv, n, seg_len, part, C, Cv, self);
            return true;
        }
    }
    if constexpr (emu_has(0, ORDER, VW)) {
        if (variant == 0) {
            constexpr int kw = omerge::KeyOrder<ORDER>::kWords;
            typed_cfg<256, production_items(kw, VW), VW, ORDER>(A, Av, m, B, Bv, n, seg_len,
                                                                 part, C, Cv, self);
            return true;
        }
    }
    return false;
}

// One 4-way pass (plan + cell merges, MT lanes and MI keys per lane in the
// cell kernel) over runs of `run`.  Before the merges it checks what the
// cell kernel assumes of the plan: every cell written, windows inside their
// runs and in order, at most q elements of each pair per cell, outputs
// consecutive from 0 to N.  Returns 1 when they hold (and the merges ran),
// 0 otherwise.
//
// With garbage != 0 the cell array starts as pseudo-random 64-bit words
// (as unwritten device memory might) and the checks are skipped: for
// unsorted runs, whose plans may collide or leave cells unwritten, the
// sanitizers then show that the cell kernel's clamps keep every access in
// the arrays.
template <int MT, int MI, int ORDER>
static int multiway_pass(const typename omerge::KeyOrder<ORDER>::T* src, int64_t N, int64_t run,
                         typename omerge::KeyOrder<ORDER>::T* dst, uint64_t garbage = 0) {
    constexpr int64_t q = int64_t(MT) * MI / 2;
    const omerge::MultiwayPlan mp = omerge::MultiwayPlan::make(N, run, q);
    std::vector<omerge::Cell4> cells(mp.cells);
    uint64_t x = garbage;
    for (auto& c : cells) {
        int64_t* w = reinterpret_cast<int64_t*>(&c);
        for (int i = 0; i < 9; ++i) {
            x = x * 6364136223846793005ull + 1442695040888963407ull;  // LCG (Knuth's MMIX)
            w[i] = garbage ? static_cast<int64_t>(x) >> (x & 31) : -1;
        }
    }
    const int64_t entries = mp.points + mp.groups + 1;
    run_grid((entries * 8 + 255) / 256, 256, [&] {
        omerge::plan_multiway_kernel<8, ORDER>(src, N, run, q, mp, cells.data());
    });
    int64_t next = garbage ? N : 0;
    for (int64_t i = 0; !garbage && i < mp.cells; ++i) {
        const omerge::Cell4& c = cells[i];
        const int64_t g = c.s[0] / (4 * run);
        int64_t n_x = 0, n_y = 0;
        for (int r = 0; r < 4; ++r) {
            const int64_t lo = std::min(g * 4 * run + r * run, N);
            const int64_t hi = std::min(lo + run, N);
            if (c.s[r] < lo || c.e[r] < c.s[r] || c.e[r] > hi) return 0;
            (r < 2 ? n_x : n_y) += c.e[r] - c.s[r];
        }
        if (c.c0 != next || n_x > q || n_y > q || n_x + n_y == 0) return 0;
        next += n_x + n_y;
    }
    if (next != N) return 0;
    // three cells per workgroup: the loads of a cell are issued while the
    // previous one merges, and the last workgroup may hold fewer
    constexpr int kCells = 3;
    run_grid((mp.cells + kCells - 1) / kCells, MT, [&] {
        omerge::merge_multiway_kernel<MT, MI, kCells, ORDER>(src, N, cells.data(), mp.cells, dst);
    });
    return 1;
}

// The merge-sort pipeline of the library (block sort with ST lanes, then
// plan + merge per pass, ping-pong between out and a scratch copy), for one
// shape.
// MULTI: keys alone merge 4 runs per pass (after one 2-way pass when the
// doublings are odd), as the library does when built with
// OMERGE_SORT_MULTIWAY=1; otherwise every pass is 2-way, as its default.
template <int T, int I, int VW, int ORDER, int ST = T, int SI = I, bool MULTI = false,
          int MT = 256, int MI = 32>
static void sort_cfg(const void* in_k, const void* in_v, int64_t N, void* out_k, void* out_v,
                     int64_t seg_len) {
    using Key = typename omerge::KeyOrder<ORDER>::T;
    constexpr int kTile = ST * SI;  // the block sort's runs
    if (N == 0) return;
    int doublings = 0;
    for (int64_t run = kTile; run < N; run *= 2) ++doublings;
    const bool multi = MULTI && VW == 0 && doublings >= 2;
    const int two_way = multi ? doublings % 2 : doublings;
    const int four_way = multi ? doublings / 2 : 0;
    const int passes = two_way + four_way;
    // One scratch block laid out as the library lays out its own: keys, then
    // payloads at the next 256-byte boundary.
    const size_t key_bytes = static_cast<size_t>(N) * sizeof(Key);
    const size_t val_at = (key_bytes + 255) & ~size_t(255);
    std::vector<uint64_t> block((val_at + static_cast<size_t>(N) * 4 * VW) / 8 + 1);
    char* const scratch = reinterpret_cast<char*>(block.data());
    Key* bufk[2] = {static_cast<Key*>(out_k), reinterpret_cast<Key*>(scratch)};
    uint32_t* bufv[2] = {static_cast<uint32_t*>(out_v),
                         VW ? reinterpret_cast<uint32_t*>(scratch + val_at) : nullptr};
    int cur = passes % 2;
    const int64_t tiles = (N + kTile - 1) / kTile;
    // 4-byte keys with payloads block-sort as packed 8-byte keys, as the
    // library does.
    run_grid(tiles, ST, [&] {
        if constexpr (omerge::KeyOrder<ORDER>::kWords == 1 && VW > 0)
            omerge::block_sort_packed_kernel<ST, SI, VW, ORDER>(
                static_cast<const Key*>(in_k), static_cast<const uint32_t*>(in_v), N, bufk[cur],
                bufv[cur]);
        else
            omerge::block_sort_kernel<ST, SI, VW, ORDER>(static_cast<const Key*>(in_k),
                                                       static_cast<const uint32_t*>(in_v), N,
                                                       bufk[cur], bufv[cur]);
    });
    int64_t run = kTile;
    for (int pass = 0; pass < two_way; ++pass, run *= 2) {
        const int64_t per_pair = (2 * run + seg_len - 1) / seg_len;
        const int64_t full = N / (2 * run), rem = N - full * 2 * run;
        const int64_t segs = full * per_pair + (rem > 0 ? (rem + seg_len - 1) / seg_len : 0);
        std::vector<omerge::SegDesc> desc(segs);
        for (auto& d : desc) d = {-1, -1, -1, -1, -1};
        run_grid(((segs + 1) * 4 + 255) / 256, 256, [&] {
            omerge::plan_runs_kernel<4, ORDER>(bufk[cur], N, run, seg_len, per_pair, segs,
                                               desc.data());
        });
        const bool reg = aligned16(out_k) && (VW == 0 || aligned16(out_v));
        run_merge<T, I, VW, ORDER, true>(reg, segs, bufk[cur], bufv[cur], N, bufk[cur], bufv[cur],
                                         N, nullptr, seg_len, bufk[1 - cur], bufv[1 - cur],
                                         desc.data(), N);
        cur = 1 - cur;
    }
    for (int pass = 0; pass < four_way; ++pass, run *= 4) {
        if constexpr (VW == 0 && MULTI) {
            if (!multiway_pass<MT, MI, ORDER>(bufk[cur], N, run, bufk[1 - cur])) abort();
        }
        cur = 1 - cur;
    }
}

// The library's batched merge for one shape.
template <int T, int I, int VW, int ORDER>
static void batched_cfg(const void* A, const void* Av, const int64_t* a_off, int64_t m,
                        const void* B, const void* Bv, const int64_t* b_off, int64_t n,
                        int64_t pairs, int64_t seg_len, void* C, void* Cv) {
    using Key = typename omerge::KeyOrder<ORDER>::T;
    const int64_t total = m + n;
    if (total == 0) return;
    const int64_t segs = pairs + (total + seg_len - 1) / seg_len - 1;
    std::vector<omerge::SegDesc> desc(segs);
    for (auto& d : desc) d = {-1, -1, -1, -1, -1};
    const Key* a = static_cast<const Key*>(A);
    const Key* b = static_cast<const Key*>(B);
    run_grid(((segs + 1) * 4 + 255) / 256, 256, [&] {
        omerge::plan_batched_kernel<4, ORDER>(a, a_off, m, b, b_off, n, pairs, seg_len, segs,
                                              desc.data());
    });
    run_grid(segs, T, [&] {
        omerge::merge_segments_kernel<T, I, VW, ORDER, true>(
            a, static_cast<const uint32_t*>(Av), m, b, static_cast<const uint32_t*>(Bv), n,
            nullptr, seg_len, static_cast<Key*>(C), static_cast<uint32_t*>(Cv), desc.data(),
            total);
    });
}

// The library's tile path for batches of short merges, for one shape.
template <int T, int I, int VW, int ORDER>
static void tiles_cfg(const void* A, const void* Av, const int64_t* a_off, int64_t m,
                      const void* B, const void* Bv, const int64_t* b_off, int64_t n,
                      int64_t pairs, void* C, void* Cv) {
    using Key = typename omerge::KeyOrder<ORDER>::T;
    constexpr int kTile = T * I;
    const int64_t total = m + n;
    if (total == 0) return;
    const int64_t tiles = (total + kTile - 1) / kTile;
    std::vector<omerge::TileBound> tb(tiles + 1);
    for (auto& t : tb) t = {-1, -1, -1};
    const Key* a = static_cast<const Key*>(A);
    const Key* b = static_cast<const Key*>(B);
    run_grid(((tiles + 1) * 4 + 255) / 256, 256, [&] {
        omerge::plan_tiles_kernel<4, ORDER>(a, a_off, m, b, b_off, n, pairs, kTile, tiles,
                                            tb.data());
    });
    // the library's choice: register stores for keys alone with 16 words
    // per lane into a 16-byte-aligned output
    constexpr bool kReg = VW == 0 && omerge::KeyOrder<ORDER>::kWords * I == 16;
    if (kReg && aligned16(C)) {
        run_grid(tiles, T, [&] {
            omerge::merge_tiles_kernel<T, I, VW, ORDER, kReg>(
                a, static_cast<const uint32_t*>(Av), a_off, m, b, static_cast<const uint32_t*>(Bv),
                b_off, n, pairs, tb.data(), static_cast<Key*>(C), static_cast<uint32_t*>(Cv));
        });
        return;
    }
    run_grid(tiles, T, [&] {
        omerge::merge_tiles_kernel<T, I, VW, ORDER>(
            a, static_cast<const uint32_t*>(Av), a_off, m, b, static_cast<const uint32_t*>(Bv),
            b_off, n, pairs, tb.data(), static_cast<Key*>(C), static_cast<uint32_t*>(Cv));
    });
}

// Which (order, payload) combinations the sort / batch entries hold: the
// small shapes for int32 keys-only, float32 descending with 4-byte payloads,
// int64 with 8-byte payloads and float64 descending keys-only; the library
// shapes for int32 keys-only or with 8-byte payloads, int64 descending
// keys-only and float64 descending with 4-byte payloads.
constexpr bool emu_sort_has(int variant, int order, int vw) {
    if (variant == 0)
        return (order == 0 && (vw == 0 || vw == 2)) || (order == (5 | 8) && vw == 1) ||
               (order == (3 | 8) && vw == 0);
    return (order == 0 && (vw == 0 || vw == 2)) || (order == (2 | 8) && vw == 1) ||
           (order == 3 && vw == 2) || (order == (5 | 8) && vw == 0);
}

template <int ORDER, int VW>
static int sort_go(int variant, const void* in_k, const void* in_v, int64_t N, void* out_k,
                   void* out_v, int64_t seg_len) {
    if constexpr (emu_sort_has(1, ORDER, VW)) {
        if (variant == 1) {
            // small shapes run the 4-way passes (the library's build option)
            sort_cfg<128, 4, VW, ORDER, 128, 4, true, 64, 4>(in_k, in_v, N, out_k, out_v, seg_len);
            return 1;
        }
    }
    if constexpr (emu_sort_has(0, ORDER, VW)) {
        if (variant == 0) {
            constexpr int kw = omerge::KeyOrder<ORDER>::kWords;
            constexpr int st = production_sort_threads(kw, VW);
            // the library's shapes and passes (2-way)
            sort_cfg<256, production_items(kw, VW), VW, ORDER, st, production_sort_items(kw, VW),
                     false>(in_k, in_v, N, out_k, out_v, seg_len);
            return 1;
        }
    }
    return 0;
}

template <int ORDER, int VW>
static int batched_go(int variant, const void* A, const void* Av, const int64_t* a_off,
                      int64_t m, const void* B, const void* Bv, const int64_t* b_off, int64_t n,
                      int64_t pairs, int64_t seg_len, void* C, void* Cv) {
    if (seg_len == 0) {  // the tile path
        if constexpr (emu_sort_has(1, ORDER, VW)) {
            if (variant == 1) {
                tiles_cfg<128, 4, VW, ORDER>(A, Av, a_off, m, B, Bv, b_off, n, pairs, C, Cv);
                return 1;
            }
        }
        if constexpr (emu_sort_has(0, ORDER, VW)) {
            if (variant == 0) {
                constexpr int kw = omerge::KeyOrder<ORDER>::kWords;
                tiles_cfg<256, production_tile_items(kw, VW), VW, ORDER>(A, Av, a_off, m, B, Bv,
                                                                         b_off, n, pairs, C, Cv);
                return 1;
            }
        }
        return 0;
    }
    if constexpr (emu_sort_has(1, ORDER, VW)) {
        if (variant == 1) {
            batched_cfg<128, 4, VW, ORDER>(A, Av, a_off, m, B, Bv, b_off, n, pairs, seg_len, C,
                                           Cv);
            return 1;
        }
    }
    if constexpr (emu_sort_has(0, ORDER, VW)) {
        if (variant == 0) {
            constexpr int kw = omerge::KeyOrder<ORDER>::kWords;
            batched_cfg<256, production_items(kw, VW), VW, ORDER>(A, Av, a_off, m, B, Bv, b_off,
                                                                  n, pairs, seg_len, C, Cv);
            return 1;
        }
    }
    return 0;
}

template <int ORDER>
static bool typed_order(int variant, int vw, const void* A, const void* Av, int64_t m,
                        const void* B, const void* Bv, int64_t n, int64_t seg_len, int64_t* part,
                        void* C, void* Cv) {
    switch (vw) {
        case 0: return typed_go<ORDER, 0>(variant, A, Av, m, B, Bv, n, seg_len, part, C, Cv);
        case 1: return typed_go<ORDER, 1>(variant, A, Av, m, B, Bv, n, seg_len, part, C, Cv);
        case 2: return typed_go<ORDER, 2>(variant, A, Av, m, B, Bv, n, seg_len, part, C, Cv);
        default: return false;
    }
}

template <int T, int I, int VW, bool SELF = false>
static void merge_cfg(const int32_t* A, const uint32_t* Av, int64_t m, const int32_t* B,
                      const uint32_t* Bv, int64_t n, const int64_t* part, int64_t seg_len,
                      int32_t* C, uint32_t* Cv) {
    const int64_t segs = (m + n + seg_len - 1) / seg_len;
    const bool reg = aligned16(C) && (VW == 0 || aligned16(Cv));
    run_merge<T, I, VW, 0, false, SELF>(reg, segs, A, Av, m, B, Bv, n, SELF ? nullptr : part,
                                        seg_len, C, Cv, nullptr, m + n);
}

extern "C" {

// variant 0 = the shapes the library launches; 1 = small shapes (128 lanes,
// 4 items) that wrap the rings many times on small inputs; variant | 2 (in
// the merges) = the same shapes with each workgroup finding its own
// boundaries, the partition array unread.
int emu_tile(int variant, int kv) {
    if (variant == 0) return kv ? omerge::MergeCfg<256, 8, 1, 1>::kTile
                                : omerge::MergeCfg<256, 8, 1, 0>::kTile;
    return omerge::MergeCfg<128, 4, 1, 0>::kTile;
}

// lanes = lanes per boundary in the partition search (1, 4, 8, 16, 64; phase-1
// stride 8), or 416 for the library's launch (4 lanes, stride 16).
void emu_partition(int lanes, const int32_t* A, int64_t m, const int32_t* B, int64_t n,
                   int64_t seg_len, int64_t* part) {
    const int64_t count = (m + n + seg_len - 1) / seg_len + 1;
    const int64_t blocks = (count * lanes + 255) / 256;
    auto go = [&](auto kernel) {
        run_grid(blocks, 256, [&] { kernel(A, m, B, n, seg_len, count, part); });
    };
    switch (lanes) {
        case 1: go(omerge::partition_kernel<1, 0>); break;
        case 4: go(omerge::partition_kernel<4, 0>); break;
        case 8: go(omerge::partition_kernel<8, 0>); break;
        case 16: go(omerge::partition_kernel<16, 0>); break;
        // The library's launch: 4 lanes, every 16th boundary in phase 1.
        case 416: go(omerge::partition_kernel<4, 0, 4, 16>); break;
        default: go(omerge::partition_kernel<64, 0>); break;
    }
}

void emu_co_rank(const int32_t* A, int64_t m, const int32_t* B, int64_t n, const int64_t* ks,
                 int64_t count, int64_t* out) {
    const int64_t blocks = (count + 255) / 256;
    run_grid(blocks, 256, [&] { omerge::co_rank_kernel<0>(A, m, B, n, ks, count, out); });
}

void emu_direct(const int32_t* A, int64_t m, const int32_t* B, int64_t n, int32_t* C,
                int64_t per, int two) {
    const int64_t blocks = ((m + n + per - 1) / per + 255) / 256;
    run_grid(blocks, 256, [&] { omerge::direct_merge_kernel(A, m, B, n, C, per, two); });
}

void emu_merge_i32(int variant, const int32_t* A, int64_t m, const int32_t* B, int64_t n,
                   const int64_t* part, int64_t seg_len, int32_t* C) {
    switch (variant) {
        case 0: merge_cfg<256, 8, 0>(A, nullptr, m, B, nullptr, n, part, seg_len, C, nullptr); break;
        case 1: merge_cfg<128, 4, 0>(A, nullptr, m, B, nullptr, n, part, seg_len, C, nullptr); break;
        case 2: merge_cfg<256, 8, 0, true>(A, nullptr, m, B, nullptr, n, part, seg_len, C, nullptr); break;
        default: merge_cfg<128, 4, 0, true>(A, nullptr, m, B, nullptr, n, part, seg_len, C, nullptr);
    }
}

void emu_merge_kv(int variant, const int32_t* A, const uint32_t* Av, int64_t m, const int32_t* B,
                  const uint32_t* Bv, int64_t n, const int64_t* part, int64_t seg_len, int32_t* C,
                  uint32_t* Cv) {
    switch (variant) {
        case 0: merge_cfg<256, 8, 1>(A, Av, m, B, Bv, n, part, seg_len, C, Cv); break;
        case 1: merge_cfg<128, 4, 1>(A, Av, m, B, Bv, n, part, seg_len, C, Cv); break;
        case 2: merge_cfg<256, 8, 1, true>(A, Av, m, B, Bv, n, part, seg_len, C, Cv); break;
        default: merge_cfg<128, 4, 1, true>(A, Av, m, B, Bv, n, part, seg_len, C, Cv);
    }
}

// Partition and merge for a key order (kind | 8 if descending) and payload
// width vw (32-bit words: 0, 1 or 2).  Returns 0 if this library does not
// hold that combination (see emu_has).
int emu_merge_typed(int variant, int order, int vw, const void* A, const void* Av, int64_t m,
                    const void* B, const void* Bv, int64_t n, int64_t seg_len, int64_t* part,
                    void* C, void* Cv) {
#define EMU_ORDER(o) \
    case o: return typed_order<o>(variant, vw, A, Av, m, B, Bv, n, seg_len, part, C, Cv);
    switch (order) {
        EMU_ORDER(0)
        EMU_ORDER(1)
        EMU_ORDER(2)
        EMU_ORDER(3)
        EMU_ORDER(4)
        EMU_ORDER(5)
        EMU_ORDER(8)
        EMU_ORDER(9)
        EMU_ORDER(10)
        EMU_ORDER(11)
        EMU_ORDER(12)
        EMU_ORDER(13)
        default: return 0;
    }
#undef EMU_ORDER
}

// The merge sort (block sort + passes) for an order and payload width;
// returns 0 if this library does not hold the combination (emu_sort_has).
int emu_sort(int variant, int order, int vw, const void* in_k, const void* in_v, int64_t n,
             void* out_k, void* out_v, int64_t seg_len) {
#define EMU_SORT(o, w) \
    if (order == o && vw == w) return sort_go<o, w>(variant, in_k, in_v, n, out_k, out_v, seg_len);
    EMU_SORT(0, 0)
    EMU_SORT(0, 2)
    EMU_SORT(10, 1)
    EMU_SORT(3, 2)
    EMU_SORT(13, 0)
    EMU_SORT(13, 1)
    EMU_SORT(11, 0)
#undef EMU_SORT
    return 0;
}

// The batched merge for an order and payload width (same combinations);
// seg_len == 0 selects the tile path for short merges.
int emu_batched(int variant, int order, int vw, const void* A, const void* Av,
                const int64_t* a_off, int64_t m, const void* B, const void* Bv,
                const int64_t* b_off, int64_t n, int64_t pairs, int64_t seg_len, void* C,
                void* Cv) {
#define EMU_BATCH(o, w)                                                                       \
    if (order == o && vw == w)                                                                \
        return batched_go<o, w>(variant, A, Av, a_off, m, B, Bv, b_off, n, pairs, seg_len, C, \
                                Cv);
    EMU_BATCH(0, 0)
    EMU_BATCH(0, 2)
    EMU_BATCH(10, 1)
    EMU_BATCH(3, 2)
    EMU_BATCH(13, 0)
    EMU_BATCH(13, 1)
    EMU_BATCH(11, 0)
#undef EMU_BATCH
    return 0;
}

// One 4-way pass over runs of `run` for a key order (keys alone): variant 0
// = the library's cell kernel (256 lanes, 128 bytes of keys each), 1 = 64
// lanes x 4 keys (cells of at most 2 x 128 elements).  Returns 1 when the
// plan held every invariant the cell kernel assumes and the merges ran, 0
// when it did not, -1 for an order this library does not hold.
// garbage != 0: unsorted input allowed, cells start as garbage (see
// multiway_pass), no plan checks.
int emu_merge_runs4(int variant, int order, const void* src, int64_t n, int64_t run, void* dst,
                    uint64_t garbage) {
#define EMU_RUNS4(o)                                                                           \
    if (order == o) {                                                                          \
        using Key = typename omerge::KeyOrder<o>::T;                                           \
        const Key* s = static_cast<const Key*>(src);                                           \
        Key* d = static_cast<Key*>(dst);                                                       \
        if (variant == 1) return multiway_pass<64, 4, o>(s, n, run, d, garbage);               \
        return multiway_pass<256, omerge::KeyOrder<o>::kWords == 1 ? 32 : 16, o>(s, n, run, d, \
                                                                               garbage);       \
    }
    EMU_RUNS4(0)
    EMU_RUNS4(1)
    EMU_RUNS4(10)
    EMU_RUNS4(11)
    EMU_RUNS4(13)
#undef EMU_RUNS4
    return -1;
}

// Tile size (outputs) of a typed shape.
int emu_typed_tile(int variant, int order, int vw) {
    const int kw = (order & 7) >= 3 ? 2 : 1;
    return variant == 0 ? 256 * production_items(kw, vw) : 128 * 4;
}

// Run length (elements) of the block sort of a shape.
int emu_sort_tile(int variant, int order, int vw) {
    const int kw = (order & 7) >= 3 ? 2 : 1;
    return variant == 0 ? production_sort_threads(kw, vw) * production_sort_items(kw, vw)
                        : 128 * 4;
}

}  // extern "C"
