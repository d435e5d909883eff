// omerge.hip -- host launcher and C ABI of libomerge.so (declared in
// include/omerge.h).  Validates arguments, picks the launch geometry for the
// current device, and enqueues the partition kernel and the segment merge
// kernel on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "omerge.h"
#include "multiway_kernel.hpp"

// Scratch of merge_i32_no_alloc: the partition array of one merge, held in a
// file-scope device array (each GPU the library runs on has its own copy,
// for the life of the process).  2^20 + 1 co-ranks cover any total up to
// 2^32 (segments of at least 4,096 outputs there; smaller totals have at most
// one segment per resident workgroup).  Host code must not use the name
// `scratch` as a device address: it is a host-side stand-in.  The device
// address comes from hipGetSymbolAddress, once per device (no_alloc_scratch).
#define OMERGE_NO_ALLOC_ENTRIES ((1 << 20) + 1)
static __device__ __align__(256) int64_t scratch[OMERGE_NO_ALLOC_ENTRIES];

namespace omerge {
namespace {

constexpr int kVersion = 100;  // 0.1.0

// Kernel shapes (compile-time tunables; the defaults are the measured best
// on MI355X).  256 lanes = 4 wavefronts per workgroup.  Segment-merge tiles
// hold 2048 outputs for 4-byte keys alone and for 4+4-byte pairs, 1024 for
// the wider elements: about 8-16 KB of elements per tile, which fits six
// (keys alone) or three workgroups per CU in the 160 KB of LDS.  The block
// sort and the tile path for batches of short merges keep 16 outputs per
// lane for 4-byte keys alone (longer first runs, fewer tiles).
#ifndef OMERGE_THREADS
#define OMERGE_THREADS 256
#endif
#ifndef OMERGE_ITEMS_I32
#define OMERGE_ITEMS_I32 8
#endif
#ifndef OMERGE_SORT_ITEMS_I32  // block sort, 4-byte keys alone
#define OMERGE_SORT_ITEMS_I32 32
#endif
#ifndef OMERGE_SORT_ITEMS_I64  // block sort, 8-byte keys alone
#define OMERGE_SORT_ITEMS_I64 8
#endif
#ifndef OMERGE_TILE_ITEMS_I32  // tile path for short merges, 4-byte keys alone
#define OMERGE_TILE_ITEMS_I32 16
#endif
#ifndef OMERGE_ITEMS_KV
#define OMERGE_ITEMS_KV 8
#endif
#ifndef OMERGE_PART_LANES  // lanes per boundary in the partition search (1 = pages' loop)
#define OMERGE_PART_LANES 4
#endif
#ifndef OMERGE_PART_LANES2  // lanes per boundary in the partition's second phase
#define OMERGE_PART_LANES2 OMERGE_PART_LANES
#endif
#ifndef OMERGE_PART_STRIDE  // the partition's first phase searches every STRIDE-th boundary
#define OMERGE_PART_STRIDE 16
#endif
#ifndef OMERGE_PLAN_LANES  // lanes per boundary in the batch and sort-pass plans
#define OMERGE_PLAN_LANES OMERGE_PART_LANES
#endif
#ifndef OMERGE_PART_SMALL  // partitions of at most this many boundaries take the shape below
#define OMERGE_PART_SMALL 49152
#endif
#ifndef OMERGE_PART_LANES_SMALL  // lanes per boundary (both phases) of those partitions
#define OMERGE_PART_LANES_SMALL 8
#endif
#ifndef OMERGE_PART_STRIDE_SMALL
#define OMERGE_PART_STRIDE_SMALL 8
#endif
#ifndef OMERGE_TILES_PER_SEG  // tiles per workgroup segment of one merge, 4-byte keys alone
#define OMERGE_TILES_PER_SEG 2
#endif
#ifndef OMERGE_TILES_PER_SEG_STAGED  // the same, through the LDS stage (unaligned outputs)
#define OMERGE_TILES_PER_SEG_STAGED 4
#endif
#ifndef OMERGE_TILES_PER_SEG_KV  // the same for 4-byte keys with 4-byte payloads
#define OMERGE_TILES_PER_SEG_KV 3
#endif
#ifndef OMERGE_TILES_PER_SEG_WIDE_KEYS  // target for 8-byte keys alone, stored from registers
#define OMERGE_TILES_PER_SEG_WIDE_KEYS 3
#endif
#ifndef OMERGE_TILES_PER_SEG_WIDE  // target for the shapes with 8-byte keys or payloads
#define OMERGE_TILES_PER_SEG_WIDE 6
#endif
#ifndef OMERGE_TILES_PER_DESC_SEG  // the same for sort passes and batches
#define OMERGE_TILES_PER_DESC_SEG 8
#endif
#ifndef OMERGE_TILES_PER_SORT_SEG  // sort passes whose tiles are stored from registers
#define OMERGE_TILES_PER_SORT_SEG 4
#endif
#ifndef OMERGE_ITEMS_WIDE  // 64-bit keys, keys only
#define OMERGE_ITEMS_WIDE 8
#endif
#ifndef OMERGE_ITEMS_MIXED  // 12- and 16-byte elements (a 64-bit key or payload)
#define OMERGE_ITEMS_MIXED 4
#endif
#ifndef OMERGE_SORT_THREADS  // lanes of the block sort for 4-byte keys without payloads
#define OMERGE_SORT_THREADS 512
#endif
#ifndef OMERGE_SORT_THREADS_KV  // lanes of the block sort for 4-byte keys with 4-byte payloads
#define OMERGE_SORT_THREADS_KV 256
#endif
#ifndef OMERGE_SORT_THREADS_WIDE  // lanes of the block sort for 8-byte keys without payloads
#define OMERGE_SORT_THREADS_WIDE 1024
#endif
#ifndef OMERGE_SORT_PACKED  // 4-byte keys with payloads block-sort as packed 8-byte keys
#define OMERGE_SORT_PACKED 1
#endif
#ifndef OMERGE_SORT_THREADS_PACKED  // lanes and keys per lane of that block sort
#define OMERGE_SORT_THREADS_PACKED 1024
#endif
#ifndef OMERGE_SORT_ITEMS_PACKED
#define OMERGE_SORT_ITEMS_PACKED 8
#endif
#ifndef OMERGE_SORT_THREADS_MIXED  // lanes of the block sort for the other shapes
#define OMERGE_SORT_THREADS_MIXED 512
#endif
#ifndef OMERGE_SHORT_MERGE  // batches averaging fewer outputs per merge use the tile path
#define OMERGE_SHORT_MERGE 6144
#endif
// Sort passes of keys alone merge 4 runs at a time when 1.  Measured slower
// on MI355X than two 2-way passes (a 4-way pass over 2^28 int32 keys takes
// about 0.99 ms, two 2-way passes 0.74 ms): the cell kernel issues 1.54 VALU
// wavefront-instructions per element, against 0.56 per 2-way pass, which
// hides its VALU work under its HBM time.  So the sort keeps 2-way passes;
// omerge_merge_runs4 runs the 4-way pass on its own.
#ifndef OMERGE_SORT_MULTIWAY
#define OMERGE_SORT_MULTIWAY 0
#endif
#ifndef OMERGE_MULTIWAY_LANES  // lanes per sample point in the 4-way plan
#define OMERGE_MULTIWAY_LANES 8
#endif
#ifndef OMERGE_MULTIWAY_THREADS  // lanes of the 4-way cell kernel
#define OMERGE_MULTIWAY_THREADS 256
#endif
#ifndef OMERGE_MULTIWAY_ITEMS  // 4-byte keys per lane of the 4-way cell kernel (8-byte: half)
#define OMERGE_MULTIWAY_ITEMS 32
#endif
#ifndef OMERGE_MULTIWAY_CELLS  // cells per workgroup of the 4-way cell kernel
#define OMERGE_MULTIWAY_CELLS 4
#endif
// The reference copy's shape: 16-byte vectors per lane and lanes per
// workgroup.  Copying 2 x 2 GiB on MI355X, one vector per lane in 64-lane
// workgroups (1 KB per workgroup) measured fastest: 6.70-6.71 TB/s, against
// 6.52 with two vectors, 6.29 with four, 6.44-6.46 with one vector in
// 256-lane workgroups and 6.18-6.26 with four (the shape this reference
// used before); eight vectors in 256-lane workgroups fell to 0.38 TB/s.
#ifndef OMERGE_COPY_UNROLL
#define OMERGE_COPY_UNROLL 1
#endif
#ifndef OMERGE_COPY_THREADS
#define OMERGE_COPY_THREADS 64
#endif
constexpr int kThreads = OMERGE_THREADS;
constexpr int kPartLanes = OMERGE_PART_LANES;
constexpr int kPartLanes2 = OMERGE_PART_LANES2;
constexpr int kPlanLanes = OMERGE_PLAN_LANES;
// Segment-length windows: target R and the half-width searched around it.
struct SegWindow {
    int target, slack;
};
constexpr SegWindow kDescWindow{OMERGE_TILES_PER_DESC_SEG, 2};
constexpr SegWindow kSortRegWindow{OMERGE_TILES_PER_SORT_SEG, 2};
constexpr int kCopyUnroll = OMERGE_COPY_UNROLL;    // 16-byte vectors per lane in the copy
constexpr int kCopyThreads = OMERGE_COPY_THREADS;  // lanes per workgroup of the copy
constexpr bool kMultiway = OMERGE_SORT_MULTIWAY != 0;
constexpr int kMultiwayLanes = OMERGE_MULTIWAY_LANES;
constexpr int kMultiwayCells = OMERGE_MULTIWAY_CELLS;
// The 4-way cell kernel: 256 lanes, 128 bytes of keys per lane (32 4-byte or
// 16 8-byte keys), so a cell holds at most 2 x 4,096 or 2 x 2,048 elements
// (37 KB of LDS, four workgroups per CU).  Against 16 keys per lane (cells of
// half the size) the plan has half the points: on 2^28 int32 keys in runs of
// 2^14 to 2^26 the pass took 0.92-0.99 ms against 1.05-1.09 ms.
constexpr int kMultiwayThreads = OMERGE_MULTIWAY_THREADS;
constexpr int multiway_items(int kw) {
    return kw == 1 ? OMERGE_MULTIWAY_ITEMS : OMERGE_MULTIWAY_ITEMS / 2;
}

// Outputs per lane of the segment merge for KW key words and VW payload
// words per element: 32 bytes of element per lane for 4-byte keys alone
// (six workgroups per CU), 64 for the other shapes (three per CU; their
// LDS holds two rings and a stage per array).  The block sort and the tile
// path have their own counts for 4-byte keys alone.
constexpr int items_for(int kw, int vw) {
    return kw == 1 && vw == 0   ? OMERGE_ITEMS_I32
           : kw == 1 && vw == 1 ? OMERGE_ITEMS_KV
           : kw == 2 && vw == 0 ? OMERGE_ITEMS_WIDE
                                : OMERGE_ITEMS_MIXED;
}
constexpr int sort_items_for(int kw, int vw) {
    return kw == 1 && vw == 0   ? OMERGE_SORT_ITEMS_I32
           : kw == 2 && vw == 0 ? OMERGE_SORT_ITEMS_I64
                                : items_for(kw, vw);
}
constexpr int tile_items_for(int kw, int vw) {
    return kw == 1 && vw == 0 ? OMERGE_TILE_ITEMS_I32 : items_for(kw, vw);
}
constexpr int shape_index(int kw, int vw) { return (kw - 1) * 3 + vw; }
constexpr int kShapes = 6;

constexpr int64_t kMaxSegLen = int64_t(1) << 30;
// Element counts up to 2^59: byte sizes (at most 8 bytes per key or payload)
// and doubled run lengths then stay inside int64.
constexpr int64_t kMaxTotal = int64_t(1) << 59;
constexpr int64_t kMaxGridBlocks = int64_t(1) << 31;  // keeps blocks*256 < 2^39

thread_local hipError_t g_last_error = hipSuccess;

int hip_fail(hipError_t e) {
    g_last_error = e;
    return OMERGE_HIP_ERROR;
}

// Per-device launch facts, filled once per device and element shape.
struct DeviceInfo {
    int cus = 0;
    // per shape and store path, with a partition array (the first 2*kShapes)
    // or with each workgroup finding its own boundaries; 0 = not yet queried
    int wg_per_cu[4 * kShapes] = {};
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mutex;

// Resident workgroups per CU of `kernel` on the current device (cached per
// `shape`, an index below 4*kShapes), and the device's CU count.
int device_slots(int shape, const void* kernel, int* cus, int* wg_per_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return OMERGE_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    DeviceInfo& d = g_dev[dev];
    if (d.cus == 0) {
        int c = 0;
        e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e);
        d.cus = c > 0 ? c : 1;
    }
    if (d.wg_per_cu[shape] == 0) {
        int a = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, kernel, kThreads, 0);
        if (e != hipSuccess) return hip_fail(e);
        d.wg_per_cu[shape] = a > 0 ? a : 1;
    }
    *cus = d.cus;
    *wg_per_cu = d.wg_per_cu[shape];
    return OMERGE_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Device address of the file-scope `scratch` array on the current device,
// looked up once per device (with that device current) and kept.
constexpr int64_t kNoAllocMaxTotal = int64_t(1) << 32;
int64_t* g_scratch_addr[kMaxDevices] = {};
std::mutex g_scratch_mutex;

int no_alloc_scratch(int64_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return OMERGE_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (p == nullptr) return hip_fail(hipErrorInvalidSymbol);
        g_scratch_addr[dev] = static_cast<int64_t*>(p);
    }
    *out = g_scratch_addr[dev];
    return OMERGE_OK;
}

// Segment length: a whole number R of tiles per workgroup.  Two costs pull
// R in opposite directions.  The partition reads about ten random cache
// lines per boundary, so short segments make it expensive (the 2^28+2^28
// merge: 23 us of partition with 8,192-output segments, 40 us with 4,096).
// Long segments spread the workgroups resident at one time over a wide span
// of A, B and C (about slots*R tiles), and HBM serves such scattered streams
// more slowly than one compact moving window.  Measured on MI355X, per step,
// with tiles stored from registers (8 workgroups per CU): 4-byte keys alone
// run best at exactly R = 2 (2^28+2^28: 0.738 ms at 2, 0.741 at 3, 0.752 at
// 4, 0.780 at 5, the merge kernel alone 0.697, 0.713, 0.728 and 0.757 ms;
// 2^27+2^24 skewed: 0.213 ms at 2, 0.222-0.224 at 3 and 4), 4+4-byte pairs
// at exactly R = 3 (2^26+2^26 pairs: 0.387 ms at 2 and 3, 0.391 at 4), and
// 8-byte keys at 3 (through the stage at 6, 2% faster than at 3), searched
// one tile either side for the R whose last round of workgroups is fullest.
// Batches and staged sort passes (descriptor segments, cut again at every run
// or merge end) measured 2-5% faster per pass with R = 8 searched over
// [6, 10]; sort passes stored from registers take 4 over [2, 6].  Inputs
// with fewer tiles than the window's low end times the slots get the
// smallest R that keeps a single round.
int64_t choose_seg_len(int64_t total, int tile, int slots, SegWindow win) {
    const int64_t lo_r = win.target > win.slack ? win.target - win.slack : 1;
    const int64_t hi_r = win.target + win.slack;
    const int64_t tiles = ceil_div(total, tile);
    if (tiles <= int64_t(slots) * lo_r) {
        const int64_t r = ceil_div(tiles, slots);
        return (r < 1 ? 1 : r) * tile;
    }
    int64_t best_r = win.target;
    double best_score = -1.0;
    for (int64_t r = lo_r; r <= hi_r; ++r) {
        const int64_t segs = ceil_div(tiles, r);
        const int64_t rounds = ceil_div(segs, slots);
        const double eff = double(tiles) / double(rounds * r * slots);
        const int64_t off = r > win.target ? r - win.target : win.target - r;
        const double score = eff - 0.004 * double(off);  // prefer R near the target
        if (score > best_score) {
            best_score = score;
            best_r = r;
        }
    }
    return best_r * tile;
}

// Byte ranges [p, p+pb) and [q, q+qb) intersect.
bool overlaps(const void* p, int64_t pb, const void* q, int64_t qb) {
    if (!p || !q || pb <= 0 || qb <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + uintptr_t(pb);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + uintptr_t(qb);
    return a0 < b1 && b0 < a1;
}

// p is 16-byte aligned (or NULL).
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// An array of `len` elements of `size` bytes: NULL only when empty, aligned
// to its element size.
bool bad_array(const void* p, int64_t len, int size = 4) {
    if (len < 0) return true;
    if (len == 0) return false;
    return p == nullptr || (reinterpret_cast<uintptr_t>(p) & uintptr_t(size - 1)) != 0;
}

int check_sizes(int64_t m, int64_t n) {
    if (m < 0 || n < 0) return OMERGE_INVALID_ARG;
    if (m > kMaxTotal || n > kMaxTotal || m > kMaxTotal - n) return OMERGE_OVERFLOW;
    return OMERGE_OK;
}

int check_seg_len(int64_t seg_len) {
    if (seg_len <= 0 || seg_len > kMaxSegLen || (seg_len & 3) != 0) return OMERGE_INVALID_ARG;
    return OMERGE_OK;
}

// Launch helpers for one key order and payload width.  Keys are typed by
// the order (KeyOrder<ORDER>::T); payloads travel as VW 32-bit words.
template <int VW, int ORDER>
struct Path {
    using Key = typename KeyOrder<ORDER>::T;
    static constexpr int KW = KeyOrder<ORDER>::kWords;
    static constexpr int kItems = items_for(KW, VW);
    static constexpr int kTile = kThreads * kItems;
    // Single merges (measured per shape, above choose_seg_len): exactly 2
    // tiles per segment for 4-byte keys alone, 3 for 4+4-byte pairs; 3,
    // searched one tile either side, for 8-byte keys alone (2^28+2^28 int64:
    // 1.54 ms at 3, 1.55 at 4, 1.57-1.59 at 6); 6 for the 12- and 16-byte
    // shapes.  Through the LDS stage (unaligned outputs) 4-byte keys alone
    // ran best at 4 and 8-byte keys at 6.
    static constexpr SegWindow kMergeWindow =
        KW == 1 && VW == 0   ? SegWindow{OMERGE_TILES_PER_SEG, 0}
        : KW == 1 && VW == 1 ? SegWindow{OMERGE_TILES_PER_SEG_KV, 0}
        : KW == 2 && VW == 0 ? SegWindow{OMERGE_TILES_PER_SEG_WIDE_KEYS, 1}
                             : SegWindow{OMERGE_TILES_PER_SEG_WIDE, 1};
    static constexpr SegWindow kStagedMergeWindow =
        KW == 1 && VW == 0   ? SegWindow{OMERGE_TILES_PER_SEG_STAGED, 0}
        : KW == 2 && VW == 0 ? SegWindow{OMERGE_TILES_PER_SEG_WIDE, 1}
                             : kMergeWindow;
    static constexpr int kTileItems = tile_items_for(KW, VW);  // tile path
    static constexpr int kBatchTile = kThreads * kTileItems;
    static constexpr bool kTileReg = VW == 0 && KW * kTileItems == 16;
    // 4-byte keys with payloads sort their tiles as packed 8-byte keys
    // (block_sort_packed_kernel) unless built with OMERGE_SORT_PACKED=0.
    static constexpr bool kSortPacked = OMERGE_SORT_PACKED && KW == 1 && VW > 0;
    static constexpr int kSortItems =
        kSortPacked ? OMERGE_SORT_ITEMS_PACKED : sort_items_for(KW, VW);
    static constexpr int kShape = shape_index(KW, VW);
    // Block sort shape: the first sorted runs are kSortTile elements long.
    // Longer runs save whole merge passes (each one read and one write of
    // the array) at the price of more rounds inside the block sort, and the
    // lane count is capped by what LDS fits.  Measured on MI355X (2^27 keys,
    // or 2^26 for 12- and 16-byte elements): 512 lanes x 32 keys for 4-byte
    // keys alone (16,384-key runs like 1024 x 16, but one in-LDS round fewer
    // and 43% fewer VALU instructions per key; the 2^28 int32 sort took
    // 6.63-6.64 ms against 6.83-6.85); 1024 lanes x 8 keys for 8-byte keys
    // alone (4% faster than 256; 512 x 16 took the same time, 6.63-6.65 ms
    // for 2^27 int64 keys); 512 for the 12- and 16-byte shapes (3-4%); 256
    // for 4-byte keys with 4-byte payloads as (key, position) pairs, where
    // 512 and 1024 were slower; packed, those take 1024 lanes x 8 keys
    // (8,192-key runs, the 8-byte keys' shape).
    static constexpr int kSortThreads = kSortPacked                ? OMERGE_SORT_THREADS_PACKED
                                        : (KW == 1 && VW == 0)   ? OMERGE_SORT_THREADS
                                        : (KW == 1 && VW == 1) ? OMERGE_SORT_THREADS_KV
                                        : (KW == 2 && VW == 0) ? OMERGE_SORT_THREADS_WIDE
                                                               : OMERGE_SORT_THREADS_MIXED;
    static constexpr int kSortTile = kSortThreads * kSortItems;

    // Tiles stored from registers (no LDS stage): 4-byte keys with no or
    // 4-byte payloads, and 8-byte keys alone.  Launches take it when every
    // segment's output is 16-byte aligned; otherwise the staged kernel,
    // which stores 16-byte vectors at any output phase.  Slots are counted for the kernel the
    // aligned case runs.
    static constexpr bool kReg = ((KW == 1 && VW <= 1) || (KW == 2 && VW == 0)) && kItems == 8;

    template <bool DESC>
    static void launch_merge(bool reg, int64_t blocks, hipStream_t stream, const Key* A,
                             const uint32_t* Av, int64_t m, const Key* B, const uint32_t* Bv,
                             int64_t n, const int64_t* part, int64_t seg_len, Key* C, uint32_t* Cv,
                             const SegDesc* desc, int64_t c_total) {
        const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
        if constexpr (kReg) {
            if (reg) {
                hipLaunchKernelGGL((merge_segments_kernel<kThreads, kItems, VW, ORDER, DESC, true>),
                                   grid, block, 0, stream, A, Av, m, B, Bv, n, part, seg_len, C,
                                   Cv, desc, c_total);
                return;
            }
        }
        hipLaunchKernelGGL((merge_segments_kernel<kThreads, kItems, VW, ORDER, DESC, false>), grid,
                           block, 0, stream, A, Av, m, B, Bv, n, part, seg_len, C, Cv, desc,
                           c_total);
    }

    // A merge whose segments all fit the device at once, in one launch:
    // each workgroup finds its own two boundaries, so there is no partition
    // kernel and no partition array.  The searches lengthen each
    // workgroup's life, which only pays while the grid runs in one wave;
    // *done is false (nothing launched) for a larger grid.
    // Built for int32 keys in ascending order (merge_i32, merge_kv and the
    // typed calls with that order); the other orders keep two launches,
    // which keeps the library's build time down.
    static int merge_self(const Key* A, const uint32_t* Av, int64_t m, const Key* B,
                          const uint32_t* Bv, int64_t n, int64_t seg_len, Key* C, uint32_t* Cv,
                          bool reg, hipStream_t stream, bool* done) {
        *done = false;
        if constexpr (ORDER != kKeyI32) {
            return OMERGE_OK;
        } else {
            reg = reg && kReg;
            const void* kernel =
                reg ? reinterpret_cast<const void*>(
                          merge_segments_kernel<kThreads, kItems, VW, ORDER, false, kReg, true>)
                    : reinterpret_cast<const void*>(
                          merge_segments_kernel<kThreads, kItems, VW, ORDER, false, false, true>);
            int cus = 0, per_cu = 0;
            int rc =
                device_slots(2 * kShapes + 2 * kShape + (reg ? 1 : 0), kernel, &cus, &per_cu);
            if (rc != OMERGE_OK) return rc;
            const int64_t segs = ceil_div(m + n, seg_len);
            if (segs > static_cast<int64_t>(cus) * per_cu) return OMERGE_OK;
            const dim3 grid(static_cast<unsigned>(segs)), block(kThreads);
            if constexpr (kReg) {
                if (reg)
                    hipLaunchKernelGGL(
                        (merge_segments_kernel<kThreads, kItems, VW, ORDER, false, true, true>),
                        grid, block, 0, stream, A, Av, m, B, Bv, n, nullptr, seg_len, C, Cv,
                        nullptr, m + n);
            }
            if (!reg)
                hipLaunchKernelGGL(
                    (merge_segments_kernel<kThreads, kItems, VW, ORDER, false, false, true>), grid,
                    block, 0, stream, A, Av, m, B, Bv, n, nullptr, seg_len, C, Cv, nullptr,
                    m + n);
            *done = true;
            hipError_t e = hipGetLastError();
            return e == hipSuccess ? OMERGE_OK : hip_fail(e);
        }
    }

    // Segment length for the register-store kernel (reg, where the shape has
    // one) or the staged one; `win` overrides the single-merge window.
    static int seg_len(int64_t m, int64_t n, int64_t* out, bool reg = kReg,
                       const SegWindow* win = nullptr) {
        reg = reg && kReg;
        const void* kernel =
            reg ? reinterpret_cast<const void*>(
                      merge_segments_kernel<kThreads, kItems, VW, ORDER, false, kReg>)
                : reinterpret_cast<const void*>(
                      merge_segments_kernel<kThreads, kItems, VW, ORDER, false, false>);
        int cus = 0, per_cu = 0;
        int rc = device_slots(2 * kShape + (reg ? 1 : 0), kernel, &cus, &per_cu);
        if (rc != OMERGE_OK) return rc;
        *out = choose_seg_len(m + n, kTile, cus * per_cu,
                              win ? *win : (reg ? kMergeWindow : kStagedMergeWindow));
        return OMERGE_OK;
    }

    // Partition shape, by the number of boundaries.  The headline's 131,072
    // boundaries are bound by the random lines their probes fetch: 4 lanes
    // per boundary with every 16th boundary searched first measured fastest
    // there (8 lanes: 69 us against 42).  A few tens of thousands of
    // boundaries are bound by their dependent rounds instead: 8 lanes per
    // boundary (9-way splits where keys tie and interpolation cannot help)
    // and every 8th boundary first took the 21,846 boundaries of the
    // 2^26+2^26 key+payload step with 256 distinct keys from 23.5 to 22.5 us
    // and the step from 0.3873-0.3876 to 0.3825 ms, left a key+payload merge
    // of distinct keys as fast (0.397-0.400 ms), and took the 36,865
    // boundaries of the skewed 2^27+2^24 step from 0.2117-0.2123 to
    // 0.2096-0.2097 ms.
    static int partition(const Key* A, int64_t m, const Key* B, int64_t n, int64_t seg_len,
                         int64_t* part, hipStream_t stream) {
        const int64_t count = ceil_div(m + n, seg_len) + 1;
        const bool small = count <= OMERGE_PART_SMALL;
        const int64_t blocks =
            ceil_div(count * (small ? OMERGE_PART_LANES_SMALL : kPartLanes), 256);
        if (blocks > kMaxGridBlocks) return OMERGE_OVERFLOW;
        if (small)
            hipLaunchKernelGGL((partition_kernel<OMERGE_PART_LANES_SMALL, ORDER,
                                                 OMERGE_PART_LANES_SMALL, OMERGE_PART_STRIDE_SMALL>),
                               dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, A, m, B,
                               n, seg_len, count, part);
        else
            hipLaunchKernelGGL((partition_kernel<kPartLanes, ORDER, kPartLanes2, OMERGE_PART_STRIDE>),
                               dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, A, m, B,
                               n, seg_len, count, part);
        hipError_t e = hipGetLastError();
        return e == hipSuccess ? OMERGE_OK : hip_fail(e);
    }

    static int merge(const Key* A, const uint32_t* Av, int64_t m, const Key* B,
                     const uint32_t* Bv, int64_t n, const int64_t* part, int64_t seg_len, Key* C,
                     uint32_t* Cv, hipStream_t stream) {
        const int64_t segs = ceil_div(m + n, seg_len);
        if (segs > kMaxGridBlocks) return OMERGE_OVERFLOW;
        // Segment outputs start at multiples of seg_len (a multiple of 4).
        const bool reg = aligned16(C) && (VW == 0 || aligned16(Cv));
        launch_merge<false>(reg, segs, stream, A, Av, m, B, Bv, n, part, seg_len, C, Cv, nullptr,
                            m + n);
        hipError_t e = hipGetLastError();
        return e == hipSuccess ? OMERGE_OK : hip_fail(e);
    }

    // Segment merge of `segs` described segments (descriptor mode); `reg`:
    // every segment's output is known to be 16-byte aligned.
    static int merge_desc(const Key* A, const uint32_t* Av, int64_t m, const Key* B,
                          const uint32_t* Bv, int64_t n, const SegDesc* desc, int64_t segs,
                          int64_t seg_len, Key* C, uint32_t* Cv, int64_t c_total, bool reg,
                          hipStream_t stream) {
        if (segs == 0) return OMERGE_OK;
        launch_merge<true>(reg, segs, stream, A, Av, m, B, Bv, n, nullptr, seg_len, C, Cv, desc,
                           c_total);
        hipError_t e = hipGetLastError();
        return e == hipSuccess ? OMERGE_OK : hip_fail(e);
    }

    // A batch of short merges: one workgroup per tile of the concatenated
    // output, whatever merges it holds (plan the tile boundaries, then merge).
    static int batched_tiles(const Key* a, const void* Av, const int64_t* a_off, int64_t m,
                             const Key* b, const void* Bv, const int64_t* b_off, int64_t n,
                             int64_t pairs, void* C, void* Cv, hipStream_t stream) {
        const int64_t tiles = ceil_div(m + n, kBatchTile);
        const int64_t blocks = ceil_div((tiles + 1) * kPlanLanes, 256);
        if (tiles > kMaxGridBlocks || blocks > kMaxGridBlocks) return OMERGE_OVERFLOW;
        TileBound* tb = nullptr;
        hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&tb),
                                      static_cast<size_t>(tiles + 1) * sizeof(TileBound), stream);
        if (e != hipSuccess) return hip_fail(e);
        hipLaunchKernelGGL((plan_tiles_kernel<kPlanLanes, ORDER>),
                           dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a, a_off, m,
                           b, b_off, n, pairs, static_cast<int64_t>(kBatchTile), tiles, tb);
        e = hipGetLastError();
        int rc = e == hipSuccess ? OMERGE_OK : hip_fail(e);
        if (rc == OMERGE_OK) {
            // Keys alone with 16 words of output per lane store each tile
            // from registers when C is 16-byte aligned (every tile's output
            // then is); the other shapes and outputs go through the stage.
            if (kTileReg && aligned16(C))
                hipLaunchKernelGGL((merge_tiles_kernel<kThreads, kTileItems, VW, ORDER, kTileReg>),
                                   dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, stream,
                                   a, static_cast<const uint32_t*>(Av), a_off, m, b,
                                   static_cast<const uint32_t*>(Bv), b_off, n, pairs, tb,
                                   static_cast<Key*>(C), static_cast<uint32_t*>(Cv));
            else
                hipLaunchKernelGGL((merge_tiles_kernel<kThreads, kTileItems, VW, ORDER>),
                                   dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, stream,
                                   a, static_cast<const uint32_t*>(Av), a_off, m, b,
                                   static_cast<const uint32_t*>(Bv), b_off, n, pairs, tb,
                                   static_cast<Key*>(C), static_cast<uint32_t*>(Cv));
            e = hipGetLastError();
            rc = e == hipSuccess ? OMERGE_OK : hip_fail(e);
        }
        e = hipFreeAsync(tb, stream);
        if (rc == OMERGE_OK && e != hipSuccess) rc = hip_fail(e);
        return rc;
    }

    // A batch of `pairs` merges given by prefix offsets into A and B (device
    // arrays of pairs+1 entries).  Short merges on average (fewer than
    // OMERGE_SHORT_MERGE outputs each) take the tile path; otherwise every
    // merge is cut into segments, planned, and merged by the segment kernel.
    static int batched(const void* A, const void* Av, const int64_t* a_off, int64_t m,
                       const void* B, const void* Bv, const int64_t* b_off, int64_t n,
                       int64_t pairs, void* C, void* Cv, hipStream_t stream) {
        const int64_t total = m + n;
        if (total == 0) return OMERGE_OK;
        if (total < pairs * static_cast<int64_t>(OMERGE_SHORT_MERGE))
            return batched_tiles(static_cast<const Key*>(A), Av, a_off, m,
                                 static_cast<const Key*>(B), Bv, b_off, n, pairs, C, Cv, stream);
        int64_t sl = 0;
        int rc = seg_len(m, n, &sl, false, &kDescWindow);
        if (rc != OMERGE_OK) return rc;
        const int64_t segs = pairs + ceil_div(total, sl) - 1;
        const int64_t blocks = ceil_div((segs + 1) * kPlanLanes, 256);
        if (segs > kMaxGridBlocks || blocks > kMaxGridBlocks) return OMERGE_OVERFLOW;
        SegDesc* desc = nullptr;
        hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&desc),
                                      static_cast<size_t>(segs) * sizeof(SegDesc), stream);
        if (e != hipSuccess) return hip_fail(e);
        const Key* a = static_cast<const Key*>(A);
        const Key* b = static_cast<const Key*>(B);
        hipLaunchKernelGGL((plan_batched_kernel<kPlanLanes, ORDER>),
                           dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a, a_off, m,
                           b, b_off, n, pairs, sl, segs, desc);
        e = hipGetLastError();
        rc = e == hipSuccess ? OMERGE_OK : hip_fail(e);
        if (rc == OMERGE_OK)
            rc = merge_desc(a, static_cast<const uint32_t*>(Av), m, b,
                            static_cast<const uint32_t*>(Bv), n, desc, segs, sl,
                            static_cast<Key*>(C), static_cast<uint32_t*>(Cv), total,
                            /*reg=*/false, stream);
        e = hipFreeAsync(desc, stream);
        if (rc == OMERGE_OK && e != hipSuccess) rc = hip_fail(e);
        return rc;
    }

    // One 4-way pass (multiway_kernel.hpp): every group of four runs of
    // `run` keys of src[0, N) merges into the same positions of dst.  The
    // cell array is the caller's (`cells`, at least plan.cells entries) or,
    // when null, stream-ordered scratch.  Keys alone.
    static constexpr int kMwItems = multiway_items(KW);
    static constexpr int64_t kMwQ = int64_t(kMultiwayThreads) * kMwItems / 2;
    static int runs4(const Key* src, Key* dst, int64_t N, int64_t run, Cell4* cells,
                     hipStream_t stream) {
        static_assert(VW == 0, "the 4-way pass moves keys alone");
        if (N == 0) return OMERGE_OK;
        const MultiwayPlan mp = MultiwayPlan::make(N, run, kMwQ);
        const int64_t entries = mp.points + mp.groups + 1;
        if (ceil_div(mp.cells, kMultiwayCells) > kMaxGridBlocks ||
            ceil_div(entries * kMultiwayLanes, 256) > kMaxGridBlocks)
            return OMERGE_OVERFLOW;
        Cell4* c = cells;
        if (c == nullptr) {
            hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&c),
                                          static_cast<size_t>(mp.cells) * sizeof(Cell4), stream);
            if (e != hipSuccess) return hip_fail(e);
        }
        hipLaunchKernelGGL((plan_multiway_kernel<kMultiwayLanes, ORDER>),
                           dim3(static_cast<unsigned>(ceil_div(entries * kMultiwayLanes, 256))),
                           dim3(256), 0, stream, src, N, run, kMwQ, mp, c);
        hipError_t e = hipGetLastError();
        if (e == hipSuccess)
            hipLaunchKernelGGL(
                (merge_multiway_kernel<kMultiwayThreads, kMwItems, kMultiwayCells, ORDER>),
                dim3(static_cast<unsigned>(ceil_div(mp.cells, kMultiwayCells))),
                dim3(kMultiwayThreads), 0, stream, src, N, c, mp.cells, dst);
        if (e == hipSuccess) e = hipGetLastError();
        int rc = e == hipSuccess ? OMERGE_OK : hip_fail(e);
        if (cells == nullptr) {
            e = hipFreeAsync(c, stream);
            if (rc == OMERGE_OK && e != hipSuccess) rc = hip_fail(e);
        }
        return rc;
    }

    // Stable merge sort of N elements: block sort into runs of one tile,
    // then passes that merge adjacent runs, ping-ponging between the output
    // and a scratch copy so that the last pass lands in the output.  Keys
    // alone merge four runs per pass (multiway_kernel.hpp), after one 2-way
    // pass when the number of doublings is odd; with payloads every pass is
    // 2-way.
    static int sort(const void* in_k, const void* in_v, void* out_k, void* out_v, int64_t N,
                    hipStream_t stream) {
        if (N == 0) return OMERGE_OK;
        const int64_t tiles = ceil_div(N, kSortTile);
        if (tiles > kMaxGridBlocks) return OMERGE_OVERFLOW;
        int passes = 0;
        for (int64_t run = kSortTile; run < N; run *= 2) ++passes;
        const bool multi = kMultiway && VW == 0 && passes >= 2;
        const int two_way = multi ? passes % 2 : passes;
        const int four_way = multi ? passes / 2 : 0;
        // Pass segments start at multiples of seg_len inside pairs of runs
        // (multiples of the block-sort tile, itself a multiple of 4), and the
        // scratch copy is 256-byte aligned: with 16-byte-aligned outputs
        // every segment's output is 16-byte aligned.  Those passes store from
        // registers and measured fastest with 4-tile segments (2^28 int32
        // keys: 6.93 ms against 7.12 ms staged at 8; 2^27 pairs: 7.44 against
        // 7.91); the staged passes keep 8.
        const bool reg = kReg && aligned16(out_k) && (VW == 0 || aligned16(out_v));
        int64_t sl = 0;
        int rc = seg_len(N, 0, &sl, reg, reg ? &kSortRegWindow : &kDescWindow);
        if (rc != OMERGE_OK) return rc;
        size_t desc_need = 0;
        {
            int64_t run = kSortTile;
            for (int p = 0; p < two_way; ++p, run *= 2) {
                const int64_t per_pair = ceil_div(2 * run, sl);
                const int64_t full = N / (2 * run), rem = N - full * 2 * run;
                const int64_t segs = full * per_pair + (rem > 0 ? ceil_div(rem, sl) : 0);
                if (segs > kMaxGridBlocks) return OMERGE_OVERFLOW;
                desc_need = std::max(desc_need, static_cast<size_t>(segs) * sizeof(SegDesc));
            }
            for (int p = 0; p < four_way; ++p, run *= 4) {
                const MultiwayPlan mp = MultiwayPlan::make(N, run, kMwQ);
                if (mp.cells > kMaxGridBlocks || mp.points + mp.groups + 1 > kMaxGridBlocks)
                    return OMERGE_OVERFLOW;
                desc_need = std::max(desc_need, static_cast<size_t>(mp.cells) * sizeof(Cell4));
            }
        }
        // Scratch: keys, payloads and descriptors in one stream-ordered block,
        // each part 256-byte aligned (64-bit payloads after an odd number of
        // 32-bit keys would otherwise lose their 8-byte alignment).
        const size_t key_bytes = static_cast<size_t>(N) * sizeof(Key);
        const size_t val_at = (key_bytes + 255) & ~size_t(255);
        const size_t val_bytes = static_cast<size_t>(N) * 4 * VW;
        const size_t desc_at = (val_at + val_bytes + 255) & ~size_t(255);
        char* scratch = nullptr;
        if (passes > 0) {
            hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&scratch), desc_at + desc_need,
                                          stream);
            if (e != hipSuccess) return hip_fail(e);
        }
        Key* const sk = reinterpret_cast<Key*>(scratch);
        uint32_t* const sv = VW ? reinterpret_cast<uint32_t*>(scratch + val_at) : nullptr;
        SegDesc* const desc = reinterpret_cast<SegDesc*>(scratch + desc_at);
        Cell4* const cells = reinterpret_cast<Cell4*>(scratch + desc_at);
        Key* bufk[2] = {static_cast<Key*>(out_k), sk};
        uint32_t* bufv[2] = {static_cast<uint32_t*>(out_v), sv};
        // block sort target: the last pass then writes out
        int cur = (two_way + four_way) % 2;
        if constexpr (kSortPacked)
            hipLaunchKernelGGL((block_sort_packed_kernel<kSortThreads, kSortItems, VW, ORDER>),
                               dim3(static_cast<unsigned>(tiles)), dim3(kSortThreads), 0, stream,
                               static_cast<const Key*>(in_k), static_cast<const uint32_t*>(in_v),
                               N, bufk[cur], bufv[cur]);
        else
            hipLaunchKernelGGL((block_sort_kernel<kSortThreads, kSortItems, VW, ORDER>),
                               dim3(static_cast<unsigned>(tiles)), dim3(kSortThreads), 0, stream,
                               static_cast<const Key*>(in_k), static_cast<const uint32_t*>(in_v),
                               N, bufk[cur], bufv[cur]);
        hipError_t e = hipGetLastError();
        rc = e == hipSuccess ? OMERGE_OK : hip_fail(e);
        int64_t run = kSortTile;
        for (int p = 0; rc == OMERGE_OK && p < two_way; ++p, run *= 2) {
            const int64_t per_pair = ceil_div(2 * run, sl);
            const int64_t full = N / (2 * run), rem = N - full * 2 * run;
            const int64_t segs = full * per_pair + (rem > 0 ? ceil_div(rem, sl) : 0);
            const int64_t blocks = ceil_div((segs + 1) * kPlanLanes, 256);
            hipLaunchKernelGGL((plan_runs_kernel<kPlanLanes, ORDER>),
                               dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                               bufk[cur], N, run, sl, per_pair, segs, desc);
            e = hipGetLastError();
            rc = e == hipSuccess ? OMERGE_OK : hip_fail(e);
            if (rc == OMERGE_OK)
                rc = merge_desc(bufk[cur], bufv[cur], N, bufk[cur], bufv[cur], N, desc, segs, sl,
                                bufk[1 - cur], bufv[1 - cur], N, reg, stream);
            cur = 1 - cur;
        }
        for (int p = 0; rc == OMERGE_OK && p < four_way; ++p, run *= 4) {
            if constexpr (VW == 0) rc = runs4(bufk[cur], bufk[1 - cur], N, run, cells, stream);
            cur = 1 - cur;
        }
        if (scratch) {
            e = hipFreeAsync(scratch, stream);
            if (rc == OMERGE_OK && e != hipSuccess) rc = hip_fail(e);
        }
        return rc;
    }

    // Whole merge: partition, then merge.  The partition array is
    // stream-ordered scratch, or, when `fixed` is given, the caller's device
    // array of `fixed_cap` entries (then nothing is allocated, and a merge
    // needing more entries returns OMERGE_SCRATCH_LIMIT before any launch).
    static int full(const void* A, const void* Av, int64_t m, const void* B, const void* Bv,
                    int64_t n, void* C, void* Cv, hipStream_t stream, int64_t* fixed = nullptr,
                    int64_t fixed_cap = 0) {
        const int64_t total = m + n;
        if (total == 0) return OMERGE_OK;
        // The segment length suits the store path merge() will take.
        const bool reg = aligned16(C) && (VW == 0 || aligned16(Cv));
        int64_t sl = 0;
        int rc = seg_len(m, n, &sl, reg);
        if (rc != OMERGE_OK) return rc;
        bool done = false;
        rc = merge_self(static_cast<const Key*>(A), static_cast<const uint32_t*>(Av), m,
                        static_cast<const Key*>(B), static_cast<const uint32_t*>(Bv), n, sl,
                        static_cast<Key*>(C), static_cast<uint32_t*>(Cv), reg, stream, &done);
        if (rc != OMERGE_OK || done) return rc;
        const int64_t count = ceil_div(total, sl) + 1;
        int64_t* part = fixed;
        if (fixed != nullptr) {
            if (count > fixed_cap) return OMERGE_SCRATCH_LIMIT;
        } else {
            hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&part),
                                          static_cast<size_t>(count) * sizeof(int64_t), stream);
            if (e != hipSuccess) return hip_fail(e);
        }
        const Key* a = static_cast<const Key*>(A);
        const Key* b = static_cast<const Key*>(B);
        rc = partition(a, m, b, n, sl, part, stream);
        if (rc == OMERGE_OK)
            rc = merge(a, static_cast<const uint32_t*>(Av), m, b, static_cast<const uint32_t*>(Bv),
                       n, part, sl, static_cast<Key*>(C), static_cast<uint32_t*>(Cv), stream);
        if (fixed == nullptr) {
            hipError_t e = hipFreeAsync(part, stream);
            if (rc == OMERGE_OK && e != hipSuccess) rc = hip_fail(e);
        }
        return rc;
    }
};

// Argument checks shared by every merge entry point: kb / vb = key / payload
// bytes per element (vb = 0: keys only).
int check_merge_args(const void* A, const void* Av, int64_t m, const void* B, const void* Bv,
                     int64_t n, const void* C, const void* Cv, int kb, int vb) {
    int rc = check_sizes(m, n);
    if (rc != OMERGE_OK) return rc;
    const int64_t t = m + n;
    if (bad_array(A, m, kb) || bad_array(B, n, kb) || bad_array(C, t, kb)) return OMERGE_INVALID_ARG;
    if (vb && (bad_array(Av, m, vb) || bad_array(Bv, n, vb) || bad_array(Cv, t, vb)))
        return OMERGE_INVALID_ARG;
    const void* ins[4] = {A, B, Av, Bv};
    const int64_t lens[4] = {m * kb, n * kb, m * vb, n * vb};
    for (int i = 0; i < 4; ++i) {
        if (overlaps(C, t * kb, ins[i], lens[i]) || overlaps(Cv, t * vb, ins[i], lens[i]))
            return OMERGE_INVALID_ARG;
    }
    if (overlaps(C, t * kb, Cv, t * vb)) return OMERGE_INVALID_ARG;
    return OMERGE_OK;
}

// The partition of a segment merge: seg_len valid, part an aligned array of
// ceil(total/seg_len)+1 entries that no output (kb / vb bytes per element of
// C / Cv) overlaps.
int check_part(const int64_t* part, int64_t total, int64_t seg_len, const void* C, int kb,
               const void* Cv, int vb) {
    int rc = check_seg_len(seg_len);
    if (rc != OMERGE_OK) return rc;
    if (total == 0) return OMERGE_OK;
    if (part == nullptr || (reinterpret_cast<uintptr_t>(part) & 7) != 0) return OMERGE_INVALID_ARG;
    const int64_t part_bytes = (ceil_div(total, seg_len) + 1) * 8;
    if (overlaps(part, part_bytes, C, total * kb) || overlaps(part, part_bytes, Cv, total * vb))
        return OMERGE_INVALID_ARG;
    return OMERGE_OK;
}

// Key order codes of the C ABI (omerge_key_kind | OMERGE_DESCENDING) map onto
// KeyOrder's template argument one to one.
static_assert(int(OMERGE_KEY_I32) == int(kKeyI32) && int(OMERGE_KEY_U32) == int(kKeyU32) &&
                  int(OMERGE_KEY_F32) == int(kKeyF32) && int(OMERGE_KEY_I64) == int(kKeyI64) &&
                  int(OMERGE_KEY_U64) == int(kKeyU64) && int(OMERGE_KEY_F64) == int(kKeyF64) &&
                  int(OMERGE_DESCENDING) == int(kKeyDescending),
              "ABI order codes must match KeyOrder");

bool valid_order(int order) {
    const int kind = order & ~kKeyDescending;
    return kind >= kKeyI32 && kind <= kKeyF64;
}
int key_bytes(int order) { return (order & 7) >= kKeyI64 ? 8 : 4; }

// Calls op(Path<VW, ORDER>{}) for the run-time payload width (0, 4 or 8
// bytes) and order code, which valid_order has accepted: one instantiation
// per (width, order) pair.
template <int VW, typename Op>
int with_order(int order, Op&& op) {
#define OMERGE_CASE(o) \
    case o: return op(Path<VW, o>{});
    switch (order) {
        OMERGE_CASE(kKeyI32)
        OMERGE_CASE(kKeyU32)
        OMERGE_CASE(kKeyF32)
        OMERGE_CASE(kKeyI64)
        OMERGE_CASE(kKeyU64)
        OMERGE_CASE(kKeyF64)
        OMERGE_CASE(kKeyI32 | kKeyDescending)
        OMERGE_CASE(kKeyU32 | kKeyDescending)
        OMERGE_CASE(kKeyF32 | kKeyDescending)
        OMERGE_CASE(kKeyI64 | kKeyDescending)
        OMERGE_CASE(kKeyU64 | kKeyDescending)
        OMERGE_CASE(kKeyF64 | kKeyDescending)
        default: return OMERGE_INVALID_ARG;
    }
#undef OMERGE_CASE
}

template <typename Op>
int with_shape(int order, int payload_bytes, Op&& op) {
    if (payload_bytes == 0) return with_order<0>(order, op);
    if (payload_bytes == 4) return with_order<1>(order, op);
    return with_order<2>(order, op);
}

using PathI32 = Path<0, kKeyI32>;
using PathKV = Path<1, kKeyI32>;

}  // namespace
}  // namespace omerge

using namespace omerge;

extern "C" {

int merge_i32(const int32_t* A, int64_t m, const int32_t* B, int64_t n,
              int32_t* C, hipStream_t stream) {
    int rc = check_merge_args(A, nullptr, m, B, nullptr, n, C, nullptr, 4, 0);
    if (rc != OMERGE_OK) return rc;
    return PathI32::full(A, nullptr, m, B, nullptr, n, C, nullptr, stream);
}

int merge_i32_no_alloc(const int32_t* A, int64_t m, const int32_t* B, int64_t n,
                       int32_t* C, hipStream_t stream) {
    int rc = check_merge_args(A, nullptr, m, B, nullptr, n, C, nullptr, 4, 0);
    if (rc != OMERGE_OK) return rc;
    if (m + n == 0) return OMERGE_OK;
    if (m + n > kNoAllocMaxTotal) return OMERGE_SCRATCH_LIMIT;
    int64_t* part = nullptr;
    rc = no_alloc_scratch(&part);
    if (rc != OMERGE_OK) return rc;
    return PathI32::full(A, nullptr, m, B, nullptr, n, C, nullptr, stream, part,
                         OMERGE_NO_ALLOC_ENTRIES);
}

int merge_kv(const int32_t* A_keys, const uint32_t* A_vals, int64_t m,
             const int32_t* B_keys, const uint32_t* B_vals, int64_t n,
             int32_t* C_keys, uint32_t* C_vals, hipStream_t stream) {
    int rc = check_merge_args(A_keys, A_vals, m, B_keys, B_vals, n, C_keys, C_vals, 4, 4);
    if (rc != OMERGE_OK) return rc;
    return PathKV::full(A_keys, A_vals, m, B_keys, B_vals, n, C_keys, C_vals, stream);
}

int omerge_merge_keys(const void* A, int64_t m, const void* B, int64_t n, void* C,
                      int order, hipStream_t stream) {
    if (!valid_order(order)) return OMERGE_INVALID_ARG;
    int rc = check_merge_args(A, nullptr, m, B, nullptr, n, C, nullptr, key_bytes(order), 0);
    if (rc != OMERGE_OK) return rc;
    return with_shape(order, 0, [&](auto path) {
        return decltype(path)::full(A, nullptr, m, B, nullptr, n, C, nullptr, stream);
    });
}

int omerge_merge_pairs(const void* A_keys, const void* A_vals, int64_t m,
                       const void* B_keys, const void* B_vals, int64_t n, void* C_keys,
                       void* C_vals, int order, int payload_bytes, hipStream_t stream) {
    if (!valid_order(order) || (payload_bytes != 4 && payload_bytes != 8))
        return OMERGE_INVALID_ARG;
    int rc = check_merge_args(A_keys, A_vals, m, B_keys, B_vals, n, C_keys, C_vals,
                              key_bytes(order), payload_bytes);
    if (rc != OMERGE_OK) return rc;
    return with_shape(order, payload_bytes, [&](auto path) {
        return decltype(path)::full(A_keys, A_vals, m, B_keys, B_vals, n, C_keys, C_vals, stream);
    });
}

int omerge_merge_batched(const void* A_keys, const void* A_vals, const int64_t* a_offsets,
                         int64_t m, const void* B_keys, const void* B_vals,
                         const int64_t* b_offsets, int64_t n, int64_t num_merges, void* C_keys,
                         void* C_vals, int order, int payload_bytes, hipStream_t stream) {
    if (!valid_order(order) || (payload_bytes != 0 && payload_bytes != 4 && payload_bytes != 8))
        return OMERGE_INVALID_ARG;
    int rc = check_merge_args(A_keys, A_vals, m, B_keys, B_vals, n, C_keys, C_vals,
                              key_bytes(order), payload_bytes);
    if (rc != OMERGE_OK) return rc;
    if (num_merges < 0 || (m + n > 0 && num_merges == 0)) return OMERGE_INVALID_ARG;
    if (num_merges > kMaxGridBlocks) return OMERGE_OVERFLOW;
    if (m + n == 0) return OMERGE_OK;
    if (bad_array(a_offsets, num_merges + 1, 8) || bad_array(b_offsets, num_merges + 1, 8))
        return OMERGE_INVALID_ARG;
    const int64_t off_bytes = (num_merges + 1) * 8;
    const void* outs[2] = {C_keys, C_vals};
    const int64_t out_bytes[2] = {(m + n) * key_bytes(order), (m + n) * payload_bytes};
    for (int i = 0; i < 2; ++i) {
        if (overlaps(outs[i], out_bytes[i], a_offsets, off_bytes) ||
            overlaps(outs[i], out_bytes[i], b_offsets, off_bytes))
            return OMERGE_INVALID_ARG;
    }
    return with_shape(order, payload_bytes, [&](auto path) {
        const bool kv = payload_bytes != 0;
        return decltype(path)::batched(A_keys, kv ? A_vals : nullptr, a_offsets, m, B_keys,
                                       kv ? B_vals : nullptr, b_offsets, n, num_merges, C_keys,
                                       kv ? C_vals : nullptr, stream);
    });
}

int omerge_sort(const void* keys_in, const void* vals_in, void* keys_out, void* vals_out,
                int64_t n, int order, int payload_bytes, hipStream_t stream) {
    if (!valid_order(order) || (payload_bytes != 0 && payload_bytes != 4 && payload_bytes != 8))
        return OMERGE_INVALID_ARG;
    if (n < 0) return OMERGE_INVALID_ARG;
    if (n > kMaxTotal) return OMERGE_OVERFLOW;
    const int kb = key_bytes(order), vb = payload_bytes;
    if (bad_array(keys_in, n, kb) || bad_array(keys_out, n, kb)) return OMERGE_INVALID_ARG;
    if (vb && (bad_array(vals_in, n, vb) || bad_array(vals_out, n, vb))) return OMERGE_INVALID_ARG;
    // Outputs: disjoint from each other; each input is either its own output
    // (in place) or disjoint from both outputs.
    if (overlaps(keys_out, n * kb, vals_out, n * vb)) return OMERGE_INVALID_ARG;
    const void* ins[2] = {keys_in, vals_in};
    const int64_t in_bytes[2] = {n * kb, n * vb};
    const void* same[2] = {keys_out, vals_out};
    for (int i = 0; i < 2; ++i) {
        if (in_bytes[i] == 0 || ins[i] == same[i]) {
            if (overlaps(ins[i], in_bytes[i], same[1 - i], in_bytes[1 - i]))
                return OMERGE_INVALID_ARG;
            continue;
        }
        if (overlaps(ins[i], in_bytes[i], keys_out, n * kb) ||
            overlaps(ins[i], in_bytes[i], vals_out, n * vb))
            return OMERGE_INVALID_ARG;
    }
    if (n == 0) return OMERGE_OK;
    return with_shape(order, vb, [&](auto path) {
        return decltype(path)::sort(keys_in, vb ? vals_in : nullptr, keys_out,
                                    vb ? vals_out : nullptr, n, stream);
    });
}

int omerge_merge_runs4(const void* keys_in, void* keys_out, int64_t n, int64_t run, int order,
                       hipStream_t stream) {
    if (!valid_order(order) || n < 0 || run < 1) return OMERGE_INVALID_ARG;
    if (n > kMaxTotal) return OMERGE_OVERFLOW;
    const int kb = key_bytes(order);
    if (bad_array(keys_in, n, kb) || bad_array(keys_out, n, kb)) return OMERGE_INVALID_ARG;
    if (overlaps(keys_in, n * kb, keys_out, n * kb)) return OMERGE_INVALID_ARG;
    if (n == 0) return OMERGE_OK;
    return with_order<0>(order, [&](auto path) {
        using P = decltype(path);
        return P::runs4(static_cast<const typename P::Key*>(keys_in),
                        static_cast<typename P::Key*>(keys_out), n, run < n ? run : n, nullptr,
                        stream);
    });
}

int omerge_co_rank(const int32_t* A, int64_t m, const int32_t* B, int64_t n,
                   const int64_t* k, int64_t count, int64_t* i_out,
                   hipStream_t stream) {
    int rc = check_sizes(m, n);
    if (rc != OMERGE_OK) return rc;
    if (count < 0 || bad_array(A, m) || bad_array(B, n)) return OMERGE_INVALID_ARG;
    if (count == 0) return OMERGE_OK;
    if (count > kMaxTotal) return OMERGE_OVERFLOW;
    if (k == nullptr || i_out == nullptr || (reinterpret_cast<uintptr_t>(k) & 7) ||
        (reinterpret_cast<uintptr_t>(i_out) & 7))
        return OMERGE_INVALID_ARG;
    if (overlaps(i_out, count * 8, A, m * 4) || overlaps(i_out, count * 8, B, n * 4) ||
        overlaps(i_out, count * 8, k, count * 8))
        return OMERGE_INVALID_ARG;
    const int64_t blocks = ceil_div(count, kThreads);
    if (blocks > kMaxGridBlocks) return OMERGE_OVERFLOW;
    hipLaunchKernelGGL(co_rank_kernel<kKeyI32>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, A, m, B, n, k, count, i_out);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? OMERGE_OK : hip_fail(e);
}

int64_t omerge_segment_length(int64_t m, int64_t n, int kv) {
    if (check_sizes(m, n) != OMERGE_OK) return -1;
    int64_t seg_len = 0;
    const int rc = kv ? PathKV::seg_len(m, n, &seg_len) : PathI32::seg_len(m, n, &seg_len);
    return rc == OMERGE_OK ? seg_len : -1;
}

int64_t omerge_partition_count(int64_t total, int64_t seg_len) {
    if (total < 0 || total > kMaxTotal || check_seg_len(seg_len) != OMERGE_OK) return -1;
    return ceil_div(total, seg_len) + 1;
}

int omerge_partition(const int32_t* A, int64_t m, const int32_t* B, int64_t n,
                     int64_t seg_len, int64_t* part, hipStream_t stream) {
    int rc = check_sizes(m, n);
    if (rc != OMERGE_OK) return rc;
    if (bad_array(A, m) || bad_array(B, n)) return OMERGE_INVALID_ARG;
    rc = check_seg_len(seg_len);
    if (rc != OMERGE_OK) return rc;
    if (part == nullptr || (reinterpret_cast<uintptr_t>(part) & 7)) return OMERGE_INVALID_ARG;
    const int64_t part_bytes = (ceil_div(m + n, seg_len) + 1) * 8;
    if (overlaps(part, part_bytes, A, m * 4) || overlaps(part, part_bytes, B, n * 4))
        return OMERGE_INVALID_ARG;
    return PathI32::partition(A, m, B, n, seg_len, part, stream);
}

int omerge_merge_segments_i32(const int32_t* A, int64_t m, const int32_t* B,
                              int64_t n, const int64_t* part, int64_t seg_len,
                              int32_t* C, hipStream_t stream) {
    int rc = check_merge_args(A, nullptr, m, B, nullptr, n, C, nullptr, 4, 0);
    if (rc != OMERGE_OK) return rc;
    rc = check_part(part, m + n, seg_len, C, 4, nullptr, 0);
    if (rc != OMERGE_OK) return rc;
    if (m + n == 0) return OMERGE_OK;
    return PathI32::merge(A, nullptr, m, B, nullptr, n, part, seg_len, C, nullptr, stream);
}

int omerge_merge_segments_kv(const int32_t* A_keys, const uint32_t* A_vals,
                             int64_t m, const int32_t* B_keys,
                             const uint32_t* B_vals, int64_t n,
                             const int64_t* part, int64_t seg_len,
                             int32_t* C_keys, uint32_t* C_vals,
                             hipStream_t stream) {
    int rc = check_merge_args(A_keys, A_vals, m, B_keys, B_vals, n, C_keys, C_vals, 4, 4);
    if (rc != OMERGE_OK) return rc;
    rc = check_part(part, m + n, seg_len, C_keys, 4, C_vals, 4);
    if (rc != OMERGE_OK) return rc;
    if (m + n == 0) return OMERGE_OK;
    return PathKV::merge(A_keys, A_vals, m, B_keys, B_vals, n, part, seg_len, C_keys, C_vals,
                         stream);
}

int omerge_merge_i32_direct(const int32_t* A, int64_t m, const int32_t* B, int64_t n,
                            int32_t* C, int64_t per_thread, int two_searches,
                            hipStream_t stream) {
    int rc = check_merge_args(A, nullptr, m, B, nullptr, n, C, nullptr, 4, 0);
    if (rc != OMERGE_OK) return rc;
    if (per_thread < 1 || per_thread > (int64_t(1) << 30)) return OMERGE_INVALID_ARG;
    const int64_t total = m + n;
    if (total == 0) return OMERGE_OK;
    const int64_t blocks = ceil_div(ceil_div(total, per_thread), 256);
    if (blocks > kMaxGridBlocks) return OMERGE_OVERFLOW;
    hipLaunchKernelGGL(direct_merge_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, A, m, B, n, C, per_thread, two_searches);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? OMERGE_OK : hip_fail(e);
}

int omerge_stream_copy(const int32_t* src, int64_t n, int32_t* dst, hipStream_t stream) {
    if (bad_array(src, n) || bad_array(dst, n)) return OMERGE_INVALID_ARG;
    if (n > kMaxTotal) return OMERGE_OVERFLOW;
    if (overlaps(src, n * 4, dst, n * 4)) return OMERGE_INVALID_ARG;
    if (n == 0) return OMERGE_OK;
    const int64_t blocks = ceil_div(ceil_div(n, 4), int64_t(kCopyThreads) * kCopyUnroll);
    if (blocks > kMaxGridBlocks) return OMERGE_OVERFLOW;
    hipLaunchKernelGGL(stream_copy_kernel<kCopyUnroll>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kCopyThreads), 0, stream, src, n, dst);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? OMERGE_OK : hip_fail(e);
}

const char* omerge_status_string(int status) {
    switch (status) {
        case OMERGE_OK: return "ok";
        case OMERGE_INVALID_ARG: return "invalid argument";
        case OMERGE_OVERFLOW: return "size overflow";
        case OMERGE_HIP_ERROR: return "HIP error";
        case OMERGE_SCRATCH_LIMIT: return "exceeds the static scratch of merge_i32_no_alloc";
        default: return "unknown status";
    }
}

int omerge_last_hip_error(void) { return static_cast<int>(g_last_error); }

int omerge_version(void) { return kVersion; }

}  // extern "C"
