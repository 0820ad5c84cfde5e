/*
 * sparse_norm.h -- C ABI of the per-voxel normalisation that follows SubMConv3d in the sparse
 * residual blocks: group normalisation in float32 (SparseGroupNorm32) and an activation, in one
 * call.  Part of libsubmconv.so; status codes, dtypes, pointer and stream conventions are those
 * of submconv.h.
 *
 * The pages list SparseGroupNorm32 and the activations among the per-voxel layers of the sparse
 * core (lato.2_mrp_mlx README, "Status"; pixal3d_mrp_mlx README, "Scope, measured against the
 * shared core") without defining them further.  The reading here is the usual one for a sparse
 * tensor:
 *   - the rows of batch item b are the contiguous range item_offsets[b] .. item_offsets[b+1] - 1
 *     (the sparse tensor's layout);
 *   - channels split into `groups` groups of channels / groups consecutive channels;
 *   - for item b and group g: mean and biased variance (divide by the count) over every row of
 *     the item and every channel of the group;
 *   - y = (x - mean) / sqrt(var + eps) * gamma[c] + beta[c], then the activation, in float32,
 *     rounded once to the storage dtype (to nearest even).
 */
#ifndef SPARSE_NORM_H
#define SPARSE_NORM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "submconv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Activation applied after the normalisation. */
typedef enum {
  SUBM_ACT_NONE = 0,
  SUBM_ACT_SILU = 1,  /* y * sigmoid(y) */
  SUBM_ACT_RELU = 2   /* max(y, 0) */
} subm_activation_t;

/*
 * sparse_group_norm_act -- y = act(group_norm(x)) per batch item.
 *   x             device [n, channels] in `dtype` (SUBM_F32 / SUBM_F16 / SUBM_BF16).
 *   n             rows, 0 <= n <= 2^31 - 1.  n == 0 returns SUBM_OK with no launch.
 *   channels      >= 1, a multiple of `groups`; a row (channels x element size) must be a
 *                 multiple of 16 bytes and at most 4096 bytes (else SUBM_ERR_UNSUPPORTED).
 *   item_offsets  device int64 [num_items + 1], non-decreasing from 0 to n (not checked on the
 *                 device: other values give unspecified results but every access stays inside
 *                 x and y).  An empty item is allowed.
 *   num_items     1 .. 65535.
 *   groups        >= 1.
 *   gamma, beta   device [channels] in `dtype`, or NULL for 1 and 0.
 *   eps           > 0.
 *   act           a subm_activation_t.
 *   x, y          16-byte aligned.
 *   y             device [n, channels] in `dtype`; may be the same pointer as x (in place);
 *                 any other overlap is undefined.
 * Scratch of about (num_items + min(n / 256, 1024)) * groups * 8 bytes comes from the library's
 * pool.  The statistics of a group are exact up to float32 rounding within blocks of rows and
 * float64 combination across them; the result is bitwise reproducible run to run.  Never
 * synchronises.
 * Errors: SUBM_ERR_INVALID_ARG, SUBM_ERR_UNSUPPORTED, SUBM_ERR_OUT_OF_MEMORY, SUBM_ERR_HIP.
 */
int sparse_group_norm_act(const void* x, int64_t n, int channels, int dtype, const int64_t* item_offsets,
                          int num_items, int groups, const void* gamma, const void* beta, float eps, int act,
                          void* y, hipStream_t stream);

/*
 * subm_conv3d_forward_group_norm_act -- out = act(group_norm(SubMConv3d(feats))), the
 * convolution followed by the normalisation of the residual blocks, with the group statistics
 * gathered in the convolution's epilogue.
 *   map .. bias   as subm_conv3d_forward (ksize 1 or 3); the convolution result is rounded to
 *                 the storage dtype exactly as subm_conv3d_forward rounds it, and the statistics
 *                 are taken of those rounded values, as a separate norm would see them.
 *   item_offsets .. act  as sparse_group_norm_act, with channels = cout.
 *   out           device [n, cout]; receives the convolution, then is normalised in place.
 * By default this runs the convolution and then the three-pass normalisation in place.  With
 * the environment variable SUBMCONV_GN_EPILOGUE=1, on the 16-bit fast path (more than 32 output
 * channels, groups not straddling a 64- or 128-channel column tile), the epilogue of the
 * convolution kernel writes per-tile, per-group partial sums instead, so the output is read
 * once less; measured on MI355X that costs more in the convolution (one workgroup per compute
 * unit leaves the epilogue's latency exposed) than the pass it saves, hence not the default.
 * Never synchronises.
 * Errors: those of subm_conv3d_forward and sparse_group_norm_act.
 * Source: the per-voxel layers that sandwich the convolution in the sparse blocks
 * (lato.2_mrp_mlx README, "Status").
 */
int subm_conv3d_forward_group_norm_act(submconv_map_t map, int64_t n, int ksize, int cin, int cout, int dtype,
                                       const void* feats, const void* weight, const void* bias,
                                       const int64_t* item_offsets, int num_items, int groups, const void* gamma,
                                       const void* beta, float eps, int act, void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_NORM_H */
