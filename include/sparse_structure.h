/*
 * sparse_structure.h -- C ABI of the structure ops on either side of SubMConv3d in the sparse
 * U-Net decoders: subdivide, 2x downsample (max / mean) and 2x upsample (cached or masked),
 * plus the child indice map derived from a parent map.  Part of libsubmconv.so; status codes,
 * dtypes, pointer and stream conventions are those of submconv.h.
 *
 * All of them relate a COARSE coordinate set to a FINE one by the factor-2 cell relation
 * (a fine voxel f lies in the coarse cell floor(f / 2) per spatial axis, batch unchanged).  One
 * handle, sparse_subdivision_t, holds such a relation:
 *   coarse   int32 [n_coarse, 4] rows (b, z, y, x)
 *   fine     int32 [n_fine, 4]
 *   parent   int32 [n_fine]: the coarse row of every fine row
 *   members  for every coarse row m, its fine rows (ascending), used by the pooling.
 * Three builders make one, each from the pages' description of the op:
 *   sparse_subdivide             coarse = the input; fine = all 8 children of every voxel in
 *                                C order, parent-major (lato.2_mrp_mlx README, scope table, the
 *                                strided-conv row: coordinate expansion by 8;
 *                                trellis_sparse_mrp_mlx commit log, masked-upsample commit:
 *                                subdivide's children are in C order).  Child s of (b,z,y,x) is
 *                                (b, 2z + (s>>2 & 1), 2y + (s>>1 & 1), 2x + (s & 1)), row 8i + s.
 *   sparse_downsample_build      fine = the input; coarse = its distinct cells (2x pooling,
 *                                trellis_sparse_mrp_mlx commit log, the downsample-mode commit),
 *                                in ascending (b, z, y, x) order (the pages leave the order
 *                                open; sorted is the plain reading).  The handle is the structure
 *                                the matching upsample reuses (pixal3d_mrp_mlx working notes,
 *                                "Remaining ops to port": the upsample is cache-paired).
 *   sparse_upsample_masked_build coarse = the input; fine = the children flagged in an [n, 8]
 *                                0/1 mask, child s at (b, 2z + (s & 1), 2y + (s>>1 & 1),
 *                                2x + (s>>2 & 1)), spatial axis 0 fastest, the reverse of
 *                                subdivide's order; parent-major, s ascending; a voxel with no
 *                                flag emits nothing (trellis_sparse_mrp_mlx commit log,
 *                                masked-upsample commit).
 * and three operations use one:
 *   sparse_downsample_forward    fine features -> coarse features, max or mean over members;
 *   sparse_upsample_forward      coarse features -> fine features, each fine row a copy of its
 *                                parent's row (the subdivided / upsampled features);
 *   sparse_indice_map_subdivide  the indice map of a subdivide's fine set, derived from the
 *                                parent map with no hashing, sorting or search.
 *
 * Builders synchronise their stream (they return host counts and check coordinate ranges);
 * the forward operations never do.  Handles are immutable after the build and may be used from
 * any stream in stream order; freeing follows the rules of sparse_indice_map_free.
 */
#ifndef SPARSE_STRUCTURE_H
#define SPARSE_STRUCTURE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "submconv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sparse_subdivision* sparse_subdivision_t;

/* Pooling reduction of sparse_downsample_forward.  There is no default: the reduction differs
 * between models and is silent when wrong, so 0 is rejected (trellis_sparse_mrp_mlx commit log,
 * the downsample-mode commit). */
typedef enum {
  SUBM_POOL_MAX = 1,  /* per-channel maximum over the members */
  SUBM_POOL_MEAN = 2  /* per-channel sum over the members / member count, in float32 */
} subm_pool_mode_t;

/* Arrays of a handle: the coarse or fine coordinates (sparse_subdivision_coords and _copy) and
 * the parent index (sparse_subdivision_copy). */
typedef enum { SUBM_COARSE = 0, SUBM_FINE = 1, SUBM_PARENT = 2 } subm_subdivision_array_t;

/* Which builder made a handle (sparse_subdivision_kind). */
typedef enum { SUBM_SUBDIVIDE = 0, SUBM_DOWNSAMPLE = 1, SUBM_UPSAMPLE_MASKED = 2 } subm_subdivision_kind_t;

/*
 * sparse_subdivide -- the 8 children of every voxel.
 *   coords  device int32 [n, 4] rows (b, z, y, x), 16-byte aligned, borrowed for the call.
 *           b in [0, 65534]; |z|, |y|, |x| <= 2^30 - 1 so that children fit int32.
 *   n       0 <= n <= 2^28 - 1 (8n rows must be int32-indexable).
 *   out     host pointer receiving the handle (NULL on error).  n_coarse = n, n_fine = 8n.
 * Synchronises `stream` once (range check).  Errors: SUBM_ERR_INVALID_ARG, SUBM_ERR_COORD_RANGE,
 * SUBM_ERR_OUT_OF_MEMORY, SUBM_ERR_HIP.
 */
int sparse_subdivide(const int32_t* coords, int64_t n, hipStream_t stream, sparse_subdivision_t* out);

/*
 * sparse_downsample_build -- the 2x coarse set of a fine set and the fine-to-coarse relation.
 *   coords  device int32 [n, 4], 16-byte aligned, borrowed; rows must be distinct (not
 *           checked); b in [0, 65534]; per-axis extent (max - min) <= 65534, as for the map.
 *   n       0 <= n <= 2^31 - 1.
 *   out     receives the handle; n_fine = n, n_coarse = number of distinct cells.
 * Coarse rows are the distinct cells floor(c / 2) (toward minus infinity) in ascending
 * (b, z, y, x) order; members of a cell are its fine rows in ascending row order.  The fine
 * coordinates are copied into the handle.  Synchronises `stream` twice (range, cell count).
 * Errors: SUBM_ERR_INVALID_ARG, SUBM_ERR_COORD_RANGE, SUBM_ERR_OUT_OF_MEMORY, SUBM_ERR_HIP.
 */
int sparse_downsample_build(const int32_t* coords, int64_t n, hipStream_t stream, sparse_subdivision_t* out);

/*
 * sparse_upsample_masked_build -- masked 2x expansion.
 *   coords  device int32 [n, 4] coarse rows, 16-byte aligned, borrowed; b in [0, 65534];
 *           |z|, |y|, |x| <= 2^30 - 1.
 *   mask    device uint8 [n, 8]: child s of row i exists when mask[i*8 + s] != 0.  Borrowed.
 *   n       0 <= n <= 2^28 - 1.
 *   out     receives the handle; n_coarse = n, n_fine = number of nonzero mask bytes.
 * Synchronises `stream` once.  Errors as sparse_subdivide.
 */
int sparse_upsample_masked_build(const int32_t* coords, const uint8_t* mask, int64_t n, hipStream_t stream,
                                 sparse_subdivision_t* out);

/* Host counts of a handle; either pointer may be NULL. */
int sparse_subdivision_info(sparse_subdivision_t s, int64_t* n_coarse, int64_t* n_fine);

/* The builder that made the handle (a subm_subdivision_kind_t) into *kind (host int). */
int sparse_subdivision_kind(sparse_subdivision_t s, int* kind);

/* Device pointer to the handle's coarse (level SUBM_COARSE) or fine (SUBM_FINE) coordinates,
 * int32 [count, 4]; owned by the handle, valid until sparse_subdivision_free.  NULL for an
 * empty set. */
int sparse_subdivision_coords(sparse_subdivision_t s, int level, const int32_t** coords);

/* Device pointer to parent int32 [n_fine] (coarse row of each fine row), owned by the handle. */
int sparse_subdivision_parent(sparse_subdivision_t s, const int32_t** parent);

/*
 * sparse_subdivision_copy -- copy one array of the handle into caller device memory.
 *   what    SUBM_COARSE: int32 [n_coarse, 4]; SUBM_FINE: int32 [n_fine, 4]; SUBM_PARENT:
 *           int32 [n_fine].
 *   dst     device pointer with room for the array (may be NULL when the array is empty).
 *   stream  stream on which the copy is enqueued (asynchronous).
 */
int sparse_subdivision_copy(sparse_subdivision_t s, int what, void* dst, hipStream_t stream);

/* Release a handle.  NULL is accepted. */
int sparse_subdivision_free(sparse_subdivision_t s);

/*
 * sparse_downsample_forward -- coarse[m, c] = reduce over fine rows f of coarse row m of
 * fine[f, c]; reduce = max (SUBM_POOL_MAX) or mean (SUBM_POOL_MEAN).
 *   channels  >= 1.  dtype: SUBM_F32 / SUBM_F16 / SUBM_BF16, shared by both tensors.
 *   fine      device [n_fine, channels];  coarse  device [n_coarse, channels], overwritten,
 *             must not overlap fine.
 * Max is exact; mean sums in float32 in ascending member order and rounds once to nearest
 * even.  A coarse row with no member (possible only for a masked handle) is written as 0.
 * Never synchronises.  Errors: SUBM_ERR_INVALID_ARG (mode 0 or unknown included),
 * SUBM_ERR_UNSUPPORTED, SUBM_ERR_HIP.
 */
int sparse_downsample_forward(sparse_subdivision_t s, int channels, int dtype, int mode, const void* fine,
                              void* coarse, hipStream_t stream);

/*
 * sparse_upsample_forward -- fine[f, :] = coarse[parent[f], :] (exact copy).
 *   coarse  device [n_coarse, channels];  fine  device [n_fine, channels], overwritten, must
 *           not overlap coarse.
 * With a subdivide handle this gives the subdivided features; with a downsample handle it is
 * the cache-paired upsample; with a masked handle, the masked upsample's features.
 * Never synchronises.  Errors: SUBM_ERR_INVALID_ARG, SUBM_ERR_UNSUPPORTED, SUBM_ERR_HIP.
 */
int sparse_upsample_forward(sparse_subdivision_t s, int channels, int dtype, const void* coarse, void* fine,
                            hipStream_t stream);

/*
 * sparse_indice_map_subdivide -- indice map of the fine set of a subdivide handle, from the map
 * of its coarse set.  Every child of an active voxel is active, so the neighbour of child
 * 2p + o at offset d is child ((o + d) mod 2) of the parent neighbour at floor((o + d) / 2),
 * or absent with it: one parent rulebook read per child, no hash or sort.  The result is the
 * same rulebook sparse_indice_map_build gives on the fine coordinates (rows in the handle's
 * fine order), with the same counts.
 *   parent_map  map built on the handle's coarse coordinates (same n, same device).
 *   s           handle from sparse_subdivide (other kinds: SUBM_ERR_INVALID_ARG).
 *   out_map     receives the new map; free with sparse_indice_map_free.
 * Does not synchronise (the pair counts follow from the parent's per-tap counts).
 * Errors: SUBM_ERR_INVALID_ARG, SUBM_ERR_SHAPE_MISMATCH, SUBM_ERR_OUT_OF_MEMORY, SUBM_ERR_HIP.
 */
int sparse_indice_map_subdivide(submconv_map_t parent_map, sparse_subdivision_t s, hipStream_t stream,
                                submconv_map_t* out_map);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_STRUCTURE_H */
