/*
 * submconv.h -- C ABI of the MI355X (gfx950) submanifold 3x3x3 sparse convolution library.
 *
 * The operation is SubMConv3d: a 3x3x3 convolution whose output sites are exactly its input
 * sites (stride 1, no padding).  Every sparse convolution the TRELLIS.2-lineage models
 * construct is this op (lato.2_mrp_mlx README, "The scope, once measured"; pixal3d_mrp_mlx
 * working notes, "Measured facts"), with kernel size 3 and the k = 1 case (lato.2_mrp_mlx
 * README, "Status").
 *
 * Two pieces:
 *   1. an indice map per coordinate set: for every active voxel i and each of the 27 offsets
 *      d in {-1,0,1}^3, the row of the active voxel at coord_i + d, or -1.  It is built once
 *      and reused by every convolution on the same coordinates, the way the pages cache it
 *      per coordinate set like spconv's indice_key (lato.2_mrp_mlx README, header summary);
 *   2. the convolution
 *          out[i, o] = bias[o] + sum_{k : nbr[i,k] >= 0} sum_c W[o, dz+1, dy+1, dx+1, c] * f[nbr[i,k], c]
 *      with W in the KRSC layout [Cout, kz, ky, kx, Cin] (lato.2_mrp_mlx README, header
 *      summary) and the cross-correlation orientation f[c + d] (lato.2_mrp_mlx README,
 *      "Correctness", which notes that the mirrored c - d reading is silent when wrong).
 *
 * Conventions shared by every entry point
 *   - Tap index k = 9*(dz+1) + 3*(dy+1) + (dx+1) for d = (dz, dy, dx); the centre tap is 13.
 *     This is the KRSC flatten order, so W viewed as [Cout, 27, Cin] holds tap k at [:, k, :].
 *   - Coordinates are int32 rows (b, z, y, x); z pairs with kz, y with ky, x with kx.
 *     Neighbours never cross different b.
 *   - Array arguments are DEVICE pointers (hipMalloc'd or from any device allocator), row-major
 *     and contiguous, aligned at least to their element size.  16-byte aligned bases with
 *     16-byte-multiple row sizes take the vectorised kernels; anything else takes a slower
 *     element-wise path with identical results.
 *   - Scalars and out-parameters named in the signatures as host values are HOST pointers.
 *   - All device work is enqueued on `stream` (0 = the null stream).  Nothing throws across the
 *     ABI: every call returns an int status (subm_status_t); on error out-parameters are left
 *     as documented and subm_last_error() gives a thread-local message.
 *   - The library keeps a device memory pool per GPU (stream-ordered allocations whose release
 *     threshold is raised so freed memory is reused, not returned to the driver).
 */
#ifndef SUBMCONV_H
#define SUBMCONV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque handle of one indice map (one per coordinate set). */
typedef struct submconv_map* submconv_map_t;

typedef enum {
  SUBM_F32 = 0,  /* float32 storage */
  SUBM_F16 = 1,  /* IEEE binary16 storage */
  SUBM_BF16 = 2  /* bfloat16 storage */
} subm_dtype_t;

typedef enum {
  SUBM_OK = 0,
  SUBM_ERR_INVALID_ARG = 1,      /* null pointer, negative size, bad enum, aliasing, ... */
  SUBM_ERR_DUPLICATE_COORD = 2,  /* two rows share (b, z, y, x) */
  SUBM_ERR_COORD_RANGE = 3,      /* b outside [0, 65534] or a z/y/x extent above 65534 */
  SUBM_ERR_SHAPE_MISMATCH = 4,   /* n differs from the map's voxel count */
  SUBM_ERR_UNSUPPORTED = 5,      /* ksize or dtype the library does not implement */
  SUBM_ERR_OUT_OF_MEMORY = 6,    /* device allocation failed */
  SUBM_ERR_HIP = 7               /* any other HIP runtime error (message in subm_last_error) */
} subm_status_t;

/* Which structure a map build uses to find neighbours (see sparse_indice_map_build_ex). */
typedef enum {
  SUBM_MAP_AUTO = 0,  /* dense grid when the bounding box is small enough, else hash table */
  SUBM_MAP_HASH = 1,  /* always the hash table */
  SUBM_MAP_GRID = 2,  /* dense grid when it fits the grid budget (128 cells per voxel, at most
                         2^29 cells), else hash */
  SUBM_MAP_SUBDIVIDED = 3  /* reported only: the map was derived from a parent map by
                              sparse_indice_map_subdivide (sparse_structure.h); not a build
                              request */
} subm_map_mode_t;

#define SUBM_TAPS 27
#define SUBM_MAX_BATCH 65535       /* b must lie in [0, SUBM_MAX_BATCH): the hash structure packs b
                                      into 16 bits and keeps the all-ones key for its empty slots,
                                      so b = 65535 is the one batch index left out */
#define SUBM_MAX_EXTENT 65534      /* max - min of each of z, y, x must not exceed this */

/*
 * sparse_indice_map_build -- build the indice map (rulebook) of one coordinate set.
 *   coords   device int32 [n, 4], rows (b, z, y, x), 16-byte aligned.  Borrowed for the
 *            duration of the call (stream-ordered); the map keeps no reference to it.  Any row
 *            order; rows must be distinct.
 *   n        number of rows, 0 <= n <= 2^31 - 1.  n == 0 yields a valid empty map, no launch.
 *   stream   stream on which the build runs.
 *   out_map  host pointer; receives the new handle.  Set to NULL first, left NULL on error.
 * The map stores nbr[n, 27] (int32, row = ORIGINAL input row of the neighbour, -1 if absent),
 * the total pair count (entries >= 0, centre included) and the per-tap pair counts.
 * The call waits on the host until the build's kernels have run, to report the duplicate /
 * range errors (the duplicate check of the dense-grid structure is part of its neighbour
 * lookup); the pair counts are read on first use.
 * Errors: SUBM_ERR_INVALID_ARG, SUBM_ERR_DUPLICATE_COORD, SUBM_ERR_COORD_RANGE,
 *         SUBM_ERR_OUT_OF_MEMORY, SUBM_ERR_HIP.
 * Source: lato.2_mrp_mlx README, header summary (indice map with 27 lookups per voxel,
 * cached per coordinate set) and "Correctness" (batch isolation, isolated voxels).
 */
int sparse_indice_map_build(const int32_t* coords, int64_t n, hipStream_t stream,
                            submconv_map_t* out_map);

/*
 * sparse_indice_map_build_ex -- sparse_indice_map_build with an explicit structure request
 * (a subm_map_mode_t).  Both structures give the identical rulebook; the choice only changes
 * speed and memory.  An unknown mode returns SUBM_ERR_INVALID_ARG.
 */
int sparse_indice_map_build_ex(const int32_t* coords, int64_t n, int mode, hipStream_t stream,
                               submconv_map_t* out_map);

/*
 * sparse_indice_map_build_async -- sparse_indice_map_build_ex without any host wait: returns as
 * soon as the build is enqueued on `stream`, so a caller can enqueue its convolutions behind it
 * and keep the GPU busy.  Arguments and argument errors as sparse_indice_map_build_ex.
 * Coordinate errors (SUBM_ERR_DUPLICATE_COORD, SUBM_ERR_COORD_RANGE) are not reported by this
 * call but by sparse_indice_map_status and by every later call that reads the map on the host
 * (sparse_indice_map_info with pairs, _offset_counts, _mode, _copy_nbr, the per-offset
 * convolution, sparse_indice_map_subdivide); the map must still be freed.  Work enqueued on a map
 * whose status is not known yet is safe: every rulebook entry is -1 or a row of the set (all -1
 * for out-of-range coordinates), so kernels stay in bounds, but their results mean nothing if the
 * status turns out to be an error.  Several asynchronous builds may be in flight at once.
 * Source of the rulebook: as sparse_indice_map_build.
 */
int sparse_indice_map_build_async(const int32_t* coords, int64_t n, int mode, hipStream_t stream,
                                  submconv_map_t* out_map);

/*
 * sparse_indice_map_status -- the coordinate status of a map's build: SUBM_OK, or the error a
 * synchronous build would have returned (SUBM_ERR_DUPLICATE_COORD, SUBM_ERR_COORD_RANGE,
 * SUBM_ERR_HIP).  For a map from sparse_indice_map_build_async the first call waits on the host
 * for the build's kernels (not for work enqueued after them); later calls, and calls on
 * synchronously built or derived maps, return at once.  NULL returns SUBM_ERR_INVALID_ARG.
 * Source: lato.2_mrp_mlx README, "Correctness" (duplicate and out-of-range coordinates are the
 * failure modes the reference's checks look for).
 */
int sparse_indice_map_status(submconv_map_t map);

/*
 * sparse_indice_map_mode -- the structure a built map used: SUBM_MAP_HASH or SUBM_MAP_GRID
 * (SUBM_MAP_HASH for an empty map), or SUBM_MAP_SUBDIVIDED for a map derived from a parent map.
 * *mode is a host int.
 */
int sparse_indice_map_mode(submconv_map_t map, int* mode);

/*
 * sparse_indice_map_free -- release a map.  NULL is accepted (returns SUBM_OK).  No work that
 * uses the map may still be in flight on any stream other than the stream of its build, as for
 * freeing any device buffer; work on the build's own stream may still be in flight (it is
 * ordered before whatever reuses the memory), and that stream must still exist.  The rulebook
 * memory of a map that was only ever used on the stream of its build is kept by the library (at
 * most 8 blocks per device, until a build takes them or the process ends) and reused by a later
 * build of a similar size on that same stream, in stream order, so a build / convolve / free
 * loop enqueues no allocator work; other memory goes back to the device's memory pool in order
 * after the work on the build's stream.
 * Host wait: free blocks the calling thread until the map's own kernels have completed (the
 * build's lookup kernel and, if one was built, the neighbour-pool plan kernel: they write memory
 * of the map that goes back to the pool, and their completion events and pinned flag words are
 * recycled).  It does not wait for convolutions or copies enqueued on the map.
 * Source: lato.2_mrp_mlx README, header summary (the indice map is built once per coordinate set
 * and dropped with it).
 */
int sparse_indice_map_free(submconv_map_t map);

/*
 * sparse_indice_map_info -- host scalars of a built map: voxel count and total pair count
 * (number of nbr entries >= 0, centre tap included).  Either out pointer may be NULL.
 * Source: lato.2_mrp_mlx README, "Correctness" (indice-map hit rates are tested).
 */
int sparse_indice_map_info(submconv_map_t map, int64_t* n, int64_t* pairs);

/*
 * sparse_indice_map_offset_counts -- host int64[27]: pairs per tap k (hit count of each
 * offset).  counts must point to 27 host int64 values.
 */
int sparse_indice_map_offset_counts(submconv_map_t map, int64_t* counts);

/*
 * subm_release_cached_memory -- free the device memory the library keeps between calls on the
 * current device, and wait for the device.  Resident until then (per device):
 *   - the map-build workspace: grown to the largest build so far, never shrunk by itself:
 *     statistics and partials (~70 KB), the hash table area (32 bytes per row) and the dense
 *     grid area (4 bytes per cell of the set's bounding box with a one-cell margin, at most 128
 *     cells per row and 2 GiB), both sized for the largest build so far, rounded up to 64 MiB;
 *   - the rulebook blocks of freed maps kept for reuse on their stream (at most 8 and at most
 *     1 GiB; a block is 112 bytes per row);
 *   - the packed-weight buffers of the neighbour-pool kernel, one per stream that ran it (at most
 *     16; 27 x 128 x cin x 2 bytes, rounded up to 1 MiB).
 * Live maps keep their own memory (rulebook, plan), freed with them; the static array of
 * subm_conv3d_forward_noalloc (1,769,472 bytes) stays for the life of the process.  The call
 * waits for all work on the device (hipDeviceSynchronize) while it holds the library's locks, so
 * calls from other threads on this device block until it returns.  Later calls allocate again
 * as needed.
 */
int subm_release_cached_memory(void);

/*
 * sparse_indice_map_plan_state -- *state (host int) = the state of the map's neighbour-pool plan
 * (see subm_conv3d_forward): SUBM_PLAN_NONE (no eligible convolution has run on the map yet),
 * SUBM_PLAN_PENDING (enqueued; the host has not seen its overflow flag yet), SUBM_PLAN_READY
 * (eligible convolutions take the neighbour-pool kernel) or SUBM_PLAN_OVERFLOW (they take the
 * general kernels).  Never waits: a pending plan whose kernel has completed becomes READY or
 * OVERFLOW here.  Source: lato.2_mrp_mlx README, header summary (the structure cached per
 * coordinate set).
 */
enum { SUBM_PLAN_NONE = 0, SUBM_PLAN_PENDING = 1, SUBM_PLAN_READY = 2, SUBM_PLAN_OVERFLOW = 3 };
int sparse_indice_map_plan_state(submconv_map_t map, int* state);

/*
 * sparse_indice_map_row_order_state -- *state (host int) = the state of the map's sparse-row
 * order: SUBM_ORDER_NONE (not enqueued), SUBM_ORDER_ON (built: 27-tap convolutions on the
 * matrix-core walk visit rows with similar neighbour masks together) or SUBM_ORDER_OFF (enqueued,
 * but the map's rows average more than 9 of 27 neighbours, so the input order is kept).  The
 * second 16-bit 27-tap convolution with more than 32 output channels on a map of at least 65,536
 * rows, on the map's own stream, enqueues the order there (SUBMCONV_ROW_ORDER=0 disables it); the
 * outputs are the same bits either way (a skipped tap is one whose neighbour is absent, which adds
 * exact zeros).  Waits for the order's kernels when it is enqueued.  Source: lato.2_mrp_mlx
 * README, header summary (the neighbour sum over present offsets only).
 */
enum { SUBM_ORDER_NONE = 0, SUBM_ORDER_ON = 1, SUBM_ORDER_OFF = 2 };
int sparse_indice_map_row_order_state(submconv_map_t map, int* state);

/*
 * sparse_indice_map_copy_nbr -- copy the rulebook into caller memory.
 *   nbr     device int32 [n, 27] in input row order; nbr[i, k] is the input row of the active
 *           voxel at coord_i + offset(k), or -1.  Independent of any internal ordering.
 *   stream  stream on which the copy is enqueued (asynchronous).
 * Source: lato.2_mrp_mlx README, header summary (the 27-lookup neighbour map per voxel); the
 * copy exists so that tests can compare the map with the oracle's rulebook bit for bit.
 */
int sparse_indice_map_copy_nbr(submconv_map_t map, int32_t* nbr, hipStream_t stream);

/*
 * subm_conv3d_forward -- out = SubMConv3d(feats) on the map's coordinate set.
 *   map      built map of the coordinate set; may be NULL only when ksize == 1.
 *   n        number of rows of feats / out; must equal the map's voxel count when map != NULL.
 *   ksize    3 (27 taps through the map) or 1 (per-voxel linear map; the map is not read).
 *   cin,cout channel counts, >= 1.
 *   dtype    storage dtype shared by feats, weight, bias and out.  Products are accumulated in
 *            float32; the bias is added in float32; the result is rounded once to the storage
 *            dtype, to nearest even.
 *   feats    device [n, cin].
 *   weight   device KRSC [cout, ksize, ksize, ksize, cin].  The library never guesses a layout;
 *            a torch Conv3d weight [cout, cin, kz, ky, kx] must be permuted by the caller
 *            (lato.2_mrp_mlx README, header summary: rank alone does not tell the layouts apart).
 *   bias     device [cout], or NULL for no bias.
 *   out      device [n, cout]; must not be the same pointer as feats (partial overlap is
 *            undefined).  Fully overwritten.
 *   stream   stream on which the kernels are enqueued.  Never synchronises; validation is on the
 *            host only.  n == 0 returns SUBM_OK with no launch.  Work on another stream than the
 *            map's build is ordered after the build by the library (a stream wait on the build's
 *            last kernel, unless it has completed).
 * Row i of out is written only from rows of feats that are neighbours of i, so the result does
 * not depend on launch order and is bitwise reproducible run to run (no float atomics).
 * Kernels.  k = 3 with 16-bit storage, cout == 128, cin a multiple of 32, 16-byte aligned
 * feats / weight / out and at least 131,072 rows take the neighbour-pool kernel: the first such
 * call on a map enqueues the map's plan (cached with the map, freed with it; device memory of
 * about 0.3 KB per row), and every call enqueues a small kernel that packs the weights into a
 * library-owned per-(device, stream) buffer (27 x 128 x cin x 2 bytes, kept for later calls on
 * that stream) before the convolution.  Until the host has seen the plan's overflow flag (a tile
 * whose neighbours do not fit the kernel's LDS pool, e.g. rows in random order), the call also
 * enqueues the general kernel behind it, and each of the two does nothing unless the flags on
 * the device say it should; sparse_indice_map_plan_state reports the plan's state.  Every other
 * call takes the general kernels.  Both families compute the same sums (results differ by
 * summation order only, within the storage rounding).
 * Tuning and tests: the environment variable SUBMCONV_POOL=0 keeps the general kernels,
 * SUBMCONV_TILE=<name> forces one of their tile configurations (and the general kernels), and
 * SUBMCONV_PERSISTENT=0 launches one workgroup per row tile instead of one per compute unit
 * walking several tiles (the two agree bit for bit).
 * Errors: SUBM_ERR_INVALID_ARG, SUBM_ERR_SHAPE_MISMATCH, SUBM_ERR_UNSUPPORTED, SUBM_ERR_HIP.
 * Source: lato.2_mrp_mlx README, header summary and "Correctness"; trellis_sparse_mrp_mlx
 * commit log, "Extracted from lato.2_mrp_mlx" commit (the 128^3 / 128-channel timing).
 */
int subm_conv3d_forward(submconv_map_t map, int64_t n, int ksize, int cin, int cout,
                        int dtype, const void* feats, const void* weight, const void* bias,
                        void* out, hipStream_t stream);

/*
 * subm_conv3d_forward_noalloc -- subm_conv3d_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments, rules, results (bit for bit) and stream semantics, and it calls no hipMalloc, hipFree
 * or other allocating routine.  Its one scratch buffer (the packed weights of the neighbour-pool
 * kernel) is a static 1,769,472-byte array in device memory, held by every device the library runs
 * on until the process ends; a call that would need more (neighbour-pool kernel with cin > 256)
 * returns SUBM_ERR_UNSUPPORTED.  It never builds the map's neighbour-pool plan (that allocates):
 * until an allocating call (subm_conv3d_forward) has built it, eligible calls take the general
 * kernels.  All calls on one device share that array, so calls that overlap in time on one device
 * (on different streams, or from different threads without ordering) race; calls in stream order
 * do not.
 */
int subm_conv3d_forward_noalloc(submconv_map_t map, int64_t n, int ksize, int cin, int cout, int dtype,
                                const void* feats, const void* weight, const void* bias, void* out,
                                hipStream_t stream);

/*
 * subm_conv3d_forward_per_offset -- the same SubMConv3d (ksize 3) as subm_conv3d_forward, computed
 * the per-offset way: for each of the 27 offsets, gather the neighbour rows of that offset,
 * multiply them by that offset's weight slice, and add the products into the output rows.  This
 * is the straightforward loop over the offsets that the pages time their implementation against
 * (trellis_sparse_mrp_mlx commit log, "Extracted from lato.2_mrp_mlx" commit), kept as a second
 * design for comparison and for very sparse tap sets.
 *   Arguments as subm_conv3d_forward with ksize = 3, plus these limits (else
 *   SUBM_ERR_UNSUPPORTED): dtype SUBM_F16 or SUBM_BF16; cin a multiple of 8; cout a multiple of
 *   4; feats and weight 16-byte aligned, out 8-byte aligned; n * cin and 27 * cout * cin
 *   elements below 2^30.
 * Products are accumulated in float32 in a scratch buffer [n, cout] from the library's pool:
 * offset 13 (the centre) first, then offsets 0 .. 26 in order; the result is rounded once to the
 * storage dtype.  Bitwise reproducible run to run; it differs from subm_conv3d_forward only by
 * float32 summation order.  The first call on a map builds and caches the per-offset pair lists
 * (that call synchronises `stream` once); later calls never synchronise.
 * Errors: SUBM_ERR_INVALID_ARG, SUBM_ERR_SHAPE_MISMATCH, SUBM_ERR_UNSUPPORTED,
 *         SUBM_ERR_OUT_OF_MEMORY, SUBM_ERR_HIP.
 */
int subm_conv3d_forward_per_offset(submconv_map_t map, int64_t n, int cin, int cout, int dtype,
                                   const void* feats, const void* weight, const void* bias, void* out,
                                   hipStream_t stream);

/*
 * subm_timing_events -- measurement hook: the next convolution kernel that this thread launches
 * (through subm_conv3d_forward or any other entry point that convolves) records `start` when it
 * begins and `stop` when it completes.  Both events are bound to that kernel's own dispatch (no
 * marker packet joins the stream), so hipEventElapsedTime(start, stop) is the kernel's duration:
 * on the neighbour-pool path the pool kernel alone, without the weight packing launched before
 * it.  Events must be created with timing on the device of that call; NULL, NULL cancels a
 * pending request.  Only the next kernel takes the request.  Always returns SUBM_OK.
 * Source: none of the pages; it serves the roofline measurement of the convolution kernel.
 */
int subm_timing_events(hipEvent_t start, hipEvent_t stop);

/*
 * subm_mfma_rate -- measurement: the matrix-core rate of this GPU at the clock it holds under
 * that load.  Launches `blocks` workgroups of 256 threads (four waves); every wave issues
 * iters x 8 back-to-back v_mfma_f32_32x32x16_bf16 on register operands (32,768 FLOP each) with
 * no memory traffic in the loop.  sink: device float [blocks * 256] (each thread's folded
 * accumulators, written so that no work is dropped); clocks: device uint64 [2 * blocks]: per
 * workgroup the s_memtime (shader clock) and s_memrealtime (100 MHz) spans of its loop.  The
 * caller times the launch on `stream` (e.g. with events).  Errors: SUBM_ERR_INVALID_ARG (iters < 1,
 * blocks outside [1, 65535], a NULL pointer), SUBM_ERR_HIP.
 * Source: none of the pages; it gives the measured ceiling beside the published 2.5 PFLOP/s.
 */
int subm_mfma_rate(int64_t iters, int blocks, float* sink, uint64_t* clocks, hipStream_t stream);

/* Static string naming a status code ("SUBM_OK", ...); "unknown status" otherwise. */
const char* subm_status_string(int status);

/* Thread-local detail of the last error on this thread (empty string if none). */
const char* subm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SUBMCONV_H */
