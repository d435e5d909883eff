/*
 * omerge.h -- C ABI of libomerge.so: stable merge of two sorted arrays on an
 * AMD Instinct MI355X (gfx950), by the co-rank method; the same kernels also
 * serve other key types and orders, batches of merges and a stable merge sort
 * (declared further down).
 *
 * The operation (page "Co-rank Function ... and Basic Parallel Merge Kernel",
 * pmpp.huatsai.dev/12-merge/02, overview and "Co-rank function definition";
 * page "merge_path.cu", gpu-preview.ayushworks.com/code/day36-merge): given A
 * (m keys) and B (n keys), each sorted ascending by signed 32-bit compare,
 * write C (m+n keys), the sorted sequence of all of them, where equal keys
 * keep A's elements before B's and each array's own order.  The output rank
 * space 0..m+n is cut into equal slices; the co-rank of a slice boundary k is
 * the i such that A[0..i) and B[0..k-i) are exactly the first k outputs.
 *
 * Conventions shared by every entry point below
 *   - Pointers to arrays are DEVICE pointers (HIP device memory, or memory the
 *     device can address).  The caller allocates and owns every buffer,
 *     including outputs; the library never frees a caller's buffer.
 *   - Arrays are contiguous and aligned to their element size (4 bytes; 8
 *     for 64-bit keys or payloads).  Any such alignment works; 16-byte-aligned
 *     arrays take the vector path on every full 16 bytes.  Merges and sorts
 *     of 4-byte keys (with or without 4-byte payloads) and of 8-byte keys
 *     alone into 16-byte-aligned outputs also store their tiles straight
 *     from registers, which is a few percent faster than the LDS-staged
 *     stores used otherwise.
 *   - Lengths are int64 and must be >= 0.  A pointer may be NULL only when its
 *     length is 0.  m + n == 0 is a no-op that returns OMERGE_OK.  A total
 *     above 2^59 elements returns OMERGE_OVERFLOW (byte sizes then fit int64).
 *   - Outputs must not overlap any input (checked by address range; for the
 *     stage calls below this includes the partition array and the co-rank
 *     queries).
 *   - A and B must be sorted ascending.  This is NOT checked.  Unsorted input
 *     gives an unspecified output, but the call still returns, every kernel
 *     still terminates and no access leaves the given arrays.
 *   - Work is enqueued on `stream` (NULL = the null stream) of the CURRENT HIP
 *     device and the call returns before it completes, like a kernel launch.
 *     Nothing synchronises the device.  Faults during execution surface at the
 *     caller's next synchronisation.  Calls on different streams are
 *     independent; the library keeps no mutable global state except a
 *     per-thread copy of the last HIP error code and a per-device cache of the
 *     device's compute-unit count.
 *   - Every entry point returns an omerge_status.  The library never prints
 *     and never exits the process.
 *
 * `struct ihipStream_t *` is the type HIP calls hipStream_t; it is spelled
 * out here so that this header needs no HIP header.
 */
#ifndef OMERGE_H
#define OMERGE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;

enum omerge_status {
    OMERGE_OK = 0,
    OMERGE_INVALID_ARG = 1, /* bad pointer, length, alignment or overlap   */
    OMERGE_OVERFLOW = 2,    /* sizes beyond what int64 / the grid can index */
    OMERGE_HIP_ERROR = 3,   /* a HIP call failed: see omerge_last_hip_error */
    OMERGE_SCRATCH_LIMIT = 4 /* larger than merge_i32_no_alloc's static scratch */
};

/*
 * merge_i32 -- stable merge of int32 keys (the pages' operation).
 *   A[m], B[n]  in:  sorted int32 keys (device).
 *   C[m+n]      out: merged keys (device).
 * Enqueues a partition kernel (one co-rank per segment boundary) and the
 * segment merge kernel on `stream`; the partition array is stream-ordered
 * scratch (hipMallocAsync/hipFreeAsync on `stream`).  A merge whose
 * segments all fit the device at once (about 8 million int32 keys on
 * MI355X) is one launch instead, each workgroup finding its own two
 * boundaries (the pages' block-level co-rank done by the block itself), with
 * no partition array.  Either way the output is the same.
 */
int merge_i32(const int32_t *A, int64_t m, const int32_t *B, int64_t n,
              int32_t *C, struct ihipStream_t *stream);

/*
 * merge_i32_no_alloc -- merge_i32 for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels and result as merge_i32, but it
 * calls no hipMalloc/hipMallocAsync/hipFree and no allocating library
 * routine: the partition array lives in a file-scope device array of the
 * library (2^20 + 1 co-ranks, 8 MiB on each GPU the library runs on, held
 * until the process ends); the one-launch path for small merges uses none.
 *   m + n at most 2^32; larger totals return OMERGE_SCRATCH_LIMIT before
 *   anything is enqueued.
 *   Every call on one GPU uses that GPU's one array, so calls that may
 *   overlap in time on one GPU (other streams, other host threads) RACE and
 *   must be serialised by the caller; calls in one stream are ordered.
 *   Nothing in the array needs clearing: each call writes every entry it
 *   reads.
 */
int merge_i32_no_alloc(const int32_t *A, int64_t m, const int32_t *B,
                       int64_t n, int32_t *C, struct ihipStream_t *stream);

/*
 * merge_kv -- stable merge of (int32 key, uint32 payload) pairs by key.
 * Only keys are compared; each payload moves with its key, so on equal keys
 * the payloads come out A's first, then B's, each in its array's order.
 * The pages merge keys only; carrying a payload is the plain extension.
 *   A_keys[m], A_vals[m], B_keys[n], B_vals[n]  in  (device).
 *   C_keys[m+n], C_vals[m+n]                    out (device; must not
 *                                                overlap each other).
 */
int merge_kv(const int32_t *A_keys, const uint32_t *A_vals, int64_t m,
             const int32_t *B_keys, const uint32_t *B_vals, int64_t n,
             int32_t *C_keys, uint32_t *C_vals, struct ihipStream_t *stream);

/*
 * Key types and orders of omerge_merge_keys / omerge_merge_pairs.
 *
 * The pages compare int keys (page "Co-rank Function ...") and float keys
 * (page "merge_path.cu", its kernels and CPU reference).  Every key type
 * below merges with the same kernels: each key is mapped to a signed integer
 * of its width by an order-preserving bijection of its bits on the way into
 * the kernel and mapped back on the way out, so the output keys are the
 * input keys' exact bit patterns.
 *   OMERGE_KEY_I32 / _I64  signed 32- / 64-bit integers (merge_i32's order).
 *   OMERGE_KEY_U32 / _U64  unsigned 32- / 64-bit integers.
 *   OMERGE_KEY_F32 / _F64  IEEE 754 binary32 / binary64 in the standard's
 *                          totalOrder: -NaN < -inf < negative finite < -0.0 <
 *                          +0.0 < positive finite < +inf < +NaN; NaNs of one
 *                          sign order by their fraction bits (larger = farther
 *                          from zero).  -0.0 and +0.0 are therefore NOT equal
 *                          keys here.
 * OR-ing OMERGE_DESCENDING reverses the order: A and B must then be sorted
 * descending, and C is descending.  In every order, equal keys keep A's
 * elements first, then each array's own order.  64-bit keys and payloads
 * must be 8-byte aligned.
 */
enum omerge_key_kind {
    OMERGE_KEY_I32 = 0,
    OMERGE_KEY_U32 = 1,
    OMERGE_KEY_F32 = 2,
    OMERGE_KEY_I64 = 3,
    OMERGE_KEY_U64 = 4,
    OMERGE_KEY_F64 = 5
};
#define OMERGE_DESCENDING 8

/*
 * omerge_merge_keys -- stable merge of keys of the type and order `order`
 * (an omerge_key_kind, optionally | OMERGE_DESCENDING).
 *   A[m], B[n]  in:  keys (4 or 8 bytes each, per the kind) sorted in that
 *                    order (device).
 *   C[m+n]      out: merged keys (device).
 * Same conventions, costs and scratch as merge_i32, which it equals for
 * order == OMERGE_KEY_I32.  An unknown order code is OMERGE_INVALID_ARG.
 *
 * omerge_merge_pairs -- the same for (key, payload) pairs, as merge_kv.
 * Payloads are payload_bytes (4 or 8) wide; they are never compared or
 * changed, and move with their keys.  Any other payload_bytes is
 * OMERGE_INVALID_ARG.
 */
int omerge_merge_keys(const void *A, int64_t m, const void *B, int64_t n,
                      void *C, int order, struct ihipStream_t *stream);
int omerge_merge_pairs(const void *A_keys, const void *A_vals, int64_t m,
                       const void *B_keys, const void *B_vals, int64_t n,
                       void *C_keys, void *C_vals, int order,
                       int payload_bytes, struct ihipStream_t *stream);

/*
 * omerge_merge_batched -- many independent stable merges in one call (page
 * "Practice - Sorting Foundations and Parallel Radix Sort",
 * pmpp.huatsai.dev/13-sorting/practice-sorting, its merge-sort stages: many
 * small merges are spread across workgroups, and a large one is cut into
 * pieces by co-rank).  Merge p (p = 0 .. num_merges-1) takes
 * A[a_offsets[p] .. a_offsets[p+1]) and B[b_offsets[p] .. b_offsets[p+1])
 * and writes C[a_offsets[p]+b_offsets[p] .. a_offsets[p+1]+b_offsets[p+1]),
 * i.e. C is the merges' outputs one after another.
 *   A_keys[m], B_keys[n]          in:  keys of `order` (as omerge_merge_keys),
 *                                      each merge's run sorted in that order.
 *   A_vals, B_vals                in:  payloads of payload_bytes (4 or 8)
 *                                      each, or NULL when payload_bytes == 0.
 *   a_offsets, b_offsets          in:  device int64 arrays of num_merges+1
 *                                      nondecreasing entries with
 *                                      a_offsets[0] = 0, a_offsets[num_merges]
 *                                      = m (likewise b with n).  NOT checked
 *                                      (device memory): other offsets give an
 *                                      unspecified output, but every access
 *                                      stays inside the arrays.
 *   C_keys[m+n], C_vals[m+n]      out.
 * num_merges >= 1 when m+n > 0.  Batches of short merges (fewer than 6,144
 * outputs per merge on average) are merged a tile of C at a time, many merges
 * per workgroup; others merge by segments.  Stream-ordered scratch of one
 * 24-byte bound per tile or one 40-byte descriptor per segment; otherwise as
 * merge_kv.
 *
 * omerge_sort -- stable merge sort of n keys (and their payloads): a block
 * sort of each tile, then passes that merge adjacent sorted runs, doubling
 * their length (the same page's merge-sort stages).  Equal keys keep their
 * input order.
 *   keys_in[n], vals_in[n]        in:  keys of `order`; payloads of
 *                                      payload_bytes (0 = none, vals NULL).
 *   keys_out[n], vals_out[n]      out: may be the inputs themselves (in
 *                                      place); otherwise disjoint from them.
 * Stream-ordered scratch of n keys and payloads plus the pass descriptors.
 */
int omerge_merge_batched(const void *A_keys, const void *A_vals,
                         const int64_t *a_offsets, int64_t m,
                         const void *B_keys, const void *B_vals,
                         const int64_t *b_offsets, int64_t n,
                         int64_t num_merges, void *C_keys, void *C_vals,
                         int order, int payload_bytes,
                         struct ihipStream_t *stream);
int omerge_sort(const void *keys_in, const void *vals_in, void *keys_out,
                void *vals_out, int64_t n, int order, int payload_bytes,
                struct ihipStream_t *stream);

/*
 * omerge_merge_runs4 -- one 4-way pass of a merge sort (the merge-sort
 * stages of the same page, four runs merged at once instead of two; each
 * group split into pieces by co-rank as in page "Co-rank Function ... and
 * Basic Parallel Merge Kernel").  keys_in holds sorted runs of `run` keys
 * (the last run may be short); every group of four consecutive runs (the
 * last group may hold fewer) is merged into the same positions of
 * keys_out, stably: equal keys keep their input order, so the earlier run
 * comes first.  Keys alone.
 *   keys_in[n]    in:  keys of `order` (as omerge_merge_keys), each run
 *                      sorted in that order.  NOT checked (device memory):
 *                      unsorted runs give an unspecified output, but every
 *                      access stays inside the arrays.
 *   keys_out[n]   out: disjoint from keys_in.
 *   run >= 1 (a run of n or more: one run, copied).
 * Stream-ordered scratch of one 72-byte descriptor per 4,096 keys (2,048
 * for 8-byte keys).  omerge_sort does not use this pass: on MI355X two 2-way
 * passes measured faster than one 4-way pass.
 */
int omerge_merge_runs4(const void *keys_in, void *keys_out, int64_t n,
                       int64_t run, int order, struct ihipStream_t *stream);

/*
 * omerge_co_rank -- device co-rank at arbitrary output ranks (page
 * "Co-rank Function ...", section "Binary-Search Implementation": bounds
 * i = min(k,m), i_low = max(0,k-n), j_low = max(0,k-m), half-step rounded up,
 * A wins ties).
 *   k[count]     in:  output ranks, each in [0, m+n] (device).  A rank out of
 *                     range is clamped into it.
 *   i_out[count] out: co-rank i of each rank; the B count is k - i (device).
 */
int omerge_co_rank(const int32_t *A, int64_t m, const int32_t *B, int64_t n,
                   const int64_t *k, int64_t count, int64_t *i_out,
                   struct ihipStream_t *stream);

/*
 * The two stages of merge_i32 / merge_kv, exposed so that a caller can hold
 * the partition (for example to split one merge across devices by output
 * rank, or to time the stages apart).
 *
 * omerge_segment_length -- the segment length (outputs per workgroup) that
 *   merge_i32 (kv = 0) or merge_kv (kv != 0) uses on the current device for
 *   these sizes and 16-byte-aligned outputs (merges into unaligned outputs
 *   pick their own).  Always a positive multiple of 4.  Returns -1 on bad
 *   sizes.
 * omerge_partition_count -- number of int64 entries the partition array needs
 *   for `total` = m+n outputs cut into segments of `seg_len`:
 *   ceil(total/seg_len) + 1.  Returns -1 on bad sizes.
 * omerge_partition -- part[s] = co-rank of k_s = min(s*seg_len, m+n) for
 *   s = 0 .. ceil((m+n)/seg_len)  (pages: block-level co-rank of the tiled
 *   kernel, page "Tiled and Circular Buffer Merge Kernel", section
 *   "Block-Level Co-Rank").  seg_len must be a positive multiple of 4 no
 *   larger than 2^30.  part is device memory of omerge_partition_count
 *   entries.
 * omerge_merge_segments_i32 / _kv -- the segment merge kernel alone, given a
 *   partition made by omerge_partition with the same seg_len.  The partition
 *   entries are clamped into their valid ranges before use, so a wrong
 *   partition gives a wrong output but never an access outside the arrays.
 */
int64_t omerge_segment_length(int64_t m, int64_t n, int kv);
int64_t omerge_partition_count(int64_t total, int64_t seg_len);
int omerge_partition(const int32_t *A, int64_t m, const int32_t *B, int64_t n,
                     int64_t seg_len, int64_t *part,
                     struct ihipStream_t *stream);
int omerge_merge_segments_i32(const int32_t *A, int64_t m, const int32_t *B,
                              int64_t n, const int64_t *part, int64_t seg_len,
                              int32_t *C, struct ihipStream_t *stream);
int omerge_merge_segments_kv(const int32_t *A_keys, const uint32_t *A_vals,
                             int64_t m, const int32_t *B_keys,
                             const uint32_t *B_vals, int64_t n,
                             const int64_t *part, int64_t seg_len,
                             int32_t *C_keys, uint32_t *C_vals,
                             struct ihipStream_t *stream);

/*
 * omerge_merge_i32_direct -- the same stable merge computed the way the
 * pages' global-memory kernels do it, kept as a measured ablation of the
 * LDS-tiled path: one lane per slice of `per_thread` outputs, reading A and B
 * and writing C in HBM directly, with no LDS.
 *   two_searches != 0: each lane finds the co-ranks of both ends of its slice
 *     and merges its two sub-arrays (page "Co-rank Function ... and Basic
 *     Parallel Merge Kernel", section "Basic Parallel Merge Kernel");
 *   two_searches == 0: each lane finds the co-rank of its slice start only and
 *     walks per_thread steps of the two-pointer merge (page "merge_path.cu",
 *     its co-rank kernel).
 * Arguments as merge_i32; per_thread in [1, 2^30].  The output is identical
 * to merge_i32's.
 */
int omerge_merge_i32_direct(const int32_t *A, int64_t m, const int32_t *B,
                            int64_t n, int32_t *C, int64_t per_thread,
                            int two_searches, struct ihipStream_t *stream);

/*
 * omerge_stream_copy -- measurement reference, not part of the merge: copies
 * n 32-bit words from src to dst (device, non-overlapping) with 16-byte
 * loads and stores, i.e. the same bytes a merge of n outputs must move.  A
 * benchmark times it beside the merge to measure the bandwidth this device
 * actually delivers, and uses its known byte count to calibrate hardware
 * traffic counters.
 */
int omerge_stream_copy(const int32_t *src, int64_t n, int32_t *dst,
                       struct ihipStream_t *stream);

/* Text for an omerge_status value (static storage; never NULL). */
const char *omerge_status_string(int status);

/* The hipError_t of the last HIP call that failed on this host thread
 * (0 if none has failed). */
int omerge_last_hip_error(void);

/* Library version as an integer: major*10000 + minor*100 + patch. */
int omerge_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OMERGE_H */
