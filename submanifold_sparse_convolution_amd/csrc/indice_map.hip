// Indice map (rulebook) build for submanifold 3x3x3 convolution on gfx950.
//
// The pages build the map from sorted coordinate keys with 27 lookups per voxel, once per
// coordinate set (lato.2_mrp_mlx README, header summary).  Here the coordinate set goes into
// one of two direct-addressed structures in HBM instead of a sorted array, so there are no
// radix passes and no binary searches; the result, nbr[i, k] = input row of the voxel at
// coord_i + offset(k) or -1, is unique and therefore identical to any sorted-key construction.
//
//   GRID  a dense int32 volume over the bounding box of the set with a one-cell margin on each
//         spatial side (cell = row or -1).  Used when the box has at most kGridCellsPerVoxel
//         cells per voxel and 2^29 cells in total.  A neighbour is one load at
//         a fixed offset from the voxel's own cell; the margin keeps every +-1 step in bounds
//         and inside the voxel's own batch slab.
//   HASH  an open-addressing table (linear probing, 16-byte slots, load factor <= 1/2) keyed by
//         (b, z mod 2^16, y mod 2^16, x mod 2^16).  Used for sparse sets in large boxes.  The
//         modular reduction is injective on every coordinate and +-1 neighbour as long as each
//         axis' extent (max - min) is at most 65534, which the build enforces.
//
// The structure is chosen on the device from the set's bounds, so the whole build needs at most
// one host synchronisation (a synchronous build waits for the last kernel, which has then written
// the range and duplicate flags straight into pinned host memory; an asynchronous build skips even
// that wait).  Neither structure is ever cleared in full.  The grid and the hash table have areas
// of their own.  A grid cell holds tag + row, where the tag is a 32-bit base that advances by n
// with every build on the workspace: a cell counts as occupied only when cell - tag < n (unsigned),
// so every entry of an earlier build reads as empty with no reset at all; the host refills the
// grid with 0xFF bytes once, when the tags would pass 2^32 - 1.  The hash table area is all 0xFF
// bytes whenever no build is inserting, and the next build's first kernel puts a hash build's
// slots back.
//
// Kernels, all on the caller's stream:
//   map_bounds_kernel   puts back the previous build's slots if it was a hash build, then
//                       per-block min/max of (b, z, y, x) -> partials (at most 256), eight rows
//                       per thread in flight
//   map_insert_kernel   every block first reduces the partials itself and so derives the same
//                       plan (range checks, structure, strides) with no second launch and no
//                       signalling between blocks (that needs a device-scope fence, which writes
//                       back the whole L2 of each XCD); block 0 publishes it (and the range flags
//                       and mode to the host) and zeroes the map's counters.  Then GRID: a plain
//                       store of tag + row into each row's cell; HASH: CAS the key into the table
//                       (a key already taken raises the duplicate flag in host memory).
//   map_lookup_kernel   three threads per voxel, one per dz plane: 9 loads (GRID) or 9 probe
//                       sequences (HASH) each, all in flight; the block's rows are staged in LDS
//                       and written as one contiguous run of nbr; per-row 27-bit hit mask; hits
//                       counted per tap with wave ballots and added to one of 16 counter banks of
//                       the map, summed on the host when first needed.  GRID: a row whose own cell
//                       holds another row shares its coordinates with that row (the later store
//                       won), which raises the duplicate flag.
// The insert and lookup blocks are dealt out so that each of the eight XCDs (the hardware hands
// workgroups to them round-robin) takes one contiguous range of rows: the cells a row's
// neighbours share then meet in one L2.
#include <hip/hip_ext.h>

#include "internal.h"

namespace submconv {
namespace {

constexpr unsigned long long kEmptyKey = ~0ull;
constexpr int kThreads = 256;
constexpr int kMaxBoundsBlocks = 256;
constexpr int kMaxWideBlocks = 1024;
constexpr int kMaxInsertBlocks = 2048;  // with four voxels per thread in flight
constexpr int kLookupVoxels = 256;      // voxels per lookup block (three threads each)

struct __align__(16) Slot {
  unsigned long long key;
  int32_t val;
  int32_t pad;
};
static_assert(sizeof(Slot) == 16, "slot must be 16 bytes");

// The batch-range check needs no flag of its own: some b lies outside [0, SUBM_MAX_BATCH) exactly
// when the minimum or the maximum of b does.
struct __align__(16) BoundsPartial {
  int32_t mn[4];
  int32_t mx[4];
};

__device__ __forceinline__ unsigned long long pack_key(int32_t b, int32_t z, int32_t y, int32_t x) {
  return ((unsigned long long)(uint32_t)b << 48) | ((unsigned long long)((uint32_t)z & 0xFFFFu) << 32) |
         ((unsigned long long)((uint32_t)y & 0xFFFFu) << 16) | (unsigned long long)((uint32_t)x & 0xFFFFu);
}

// 64-bit finaliser of MurmurHash3 (Austin Appleby): spreads every key bit over the word.
__device__ __forceinline__ unsigned long long mix64(unsigned long long k) {
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdull;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ull;
  k ^= k >> 33;
  return k;
}

// Home slot in [0, slots): high word of hash * slots (no power-of-two capacity needed).
__device__ __forceinline__ unsigned long long home_slot(unsigned long long key, unsigned long long slots) {
  return __umul64hi(mix64(key), slots);
}

__device__ __forceinline__ int wave_min(int v) {
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

// Logical block of hardware block b of g: the blocks of XCD b mod 8 take one contiguous range.
__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t g) {
  const int64_t q = g / 8, r = g % 8, x = b % 8;
  return x * q + (x < r ? x : r) + b / 8;
}

// ------------------------------------------------------------------ bounds
__global__ __launch_bounds__(kThreads) void map_bounds_kernel(const int32_t* __restrict__ coords, int64_t n,
                                                              int nparts, BoundsPartial* __restrict__ partials,
                                                              const MapStats* __restrict__ prev,
                                                              void* __restrict__ hash_table) {
  // A previous hash build's slots back to empty (its lookup has finished: stream order).  Grid
  // entries need nothing: their tags tell them apart.
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (prev->mode == kModeHash) {
    int4* tab = static_cast<int4*>(hash_table);
    const int4 ff = make_int4(-1, -1, -1, -1);
    for (int64_t i = t0; i < prev->slots; i += stride) tab[i] = ff;
  }
  // Bounds: the first nparts blocks (the grid may be wider for a large previous build), eight
  // rows per thread in flight.
  if ((int)blockIdx.x >= nparts) return;
  int mn[4] = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX};
  int mx[4] = {INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
  constexpr int kBatch = 8;
  const int64_t pstride = (int64_t)nparts * kThreads;
  for (int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; i0 < n; i0 += kBatch * pstride) {
    int4 c[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + u * pstride;
      // (rows past the end repeat row i0, which changes no minimum or maximum)
      c[u] = *reinterpret_cast<const int4*>(coords + 4 * (i < n ? i : i0));
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      mn[0] = min(mn[0], c[u].x); mx[0] = max(mx[0], c[u].x);
      mn[1] = min(mn[1], c[u].y); mx[1] = max(mx[1], c[u].y);
      mn[2] = min(mn[2], c[u].z); mx[2] = max(mx[2], c[u].z);
      mn[3] = min(mn[3], c[u].w); mx[3] = max(mx[3], c[u].w);
    }
  }
  __shared__ int smn[kThreads / 64][4];
  __shared__ int smx[kThreads / 64][4];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int lo = wave_min(mn[a]);
    const int hi = wave_max(mx[a]);
    if (lane == 0) {
      smn[wave][a] = lo;
      smx[wave][a] = hi;
    }
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    const int a = threadIdx.x;
    int lo = smn[0][a], hi = smx[0][a];
    for (int w = 1; w < kThreads / 64; ++w) {
      lo = min(lo, smn[w][a]);
      hi = max(hi, smx[w][a]);
    }
    partials[blockIdx.x].mn[a] = lo;
    partials[blockIdx.x].mx[a] = hi;
  }
}

// ------------------------------------------------------------------ plan + insert
// The plan: bounds reduced from the partials, range checks, structure choice and strides.
struct Plan {
  int32_t mn[4];
  uint32_t flags;
  int mode;
  int64_t cells, sy, sz, sb;
};

// Every insert block reduces the (at most 256) partials itself, so all blocks agree on the plan
// without another launch.
__device__ void reduce_plan(const BoundsPartial* __restrict__ partials, int nparts, int64_t grid_budget_cells,
                            int mode_request, Plan& plan, int32_t (&mx_out)[4]) {
  __shared__ int s_mn[4], s_mx[4];
  __shared__ int rmn[kThreads / 64][4], rmx[kThreads / 64][4];
  const int t = threadIdx.x;
  int mn[4] = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX};
  int mx[4] = {INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
  for (int p = t; p < nparts; p += kThreads) {
    const BoundsPartial q = partials[p];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      mn[a] = min(mn[a], q.mn[a]);
      mx[a] = max(mx[a], q.mx[a]);
    }
  }
  const int wave = t / 64, lane = t % 64;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int lo = wave_min(mn[a]);
    const int hi = wave_max(mx[a]);
    if (lane == 0) {
      rmn[wave][a] = lo;
      rmx[wave][a] = hi;
    }
  }
  __syncthreads();
  if (t < 4) {
    int lo = rmn[0][t], hi = rmx[0][t];
    for (int w = 1; w < kThreads / 64; ++w) {
      lo = min(lo, rmn[w][t]);
      hi = max(hi, rmx[w][t]);
    }
    s_mn[t] = lo;
    s_mx[t] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    plan.mn[a] = s_mn[a];
    mx_out[a] = s_mx[a];
  }
  uint32_t flags = (s_mn[0] < 0 || s_mx[0] >= SUBM_MAX_BATCH) ? kFlagBatchRange : 0u;
  const int64_t ext_b = (int64_t)s_mx[0] - s_mn[0] + 1;
  const int64_t ext_z = (int64_t)s_mx[1] - s_mn[1];
  const int64_t ext_y = (int64_t)s_mx[2] - s_mn[2];
  const int64_t ext_x = (int64_t)s_mx[3] - s_mn[3];
  if (ext_z > SUBM_MAX_EXTENT || ext_y > SUBM_MAX_EXTENT || ext_x > SUBM_MAX_EXTENT) flags |= kFlagExtentRange;
  plan.mode = kModeHash;
  plan.cells = 0;
  plan.sy = plan.sz = plan.sb = 0;
  if ((flags & (kFlagBatchRange | kFlagExtentRange)) != 0) {
    plan.mode = kModeNone;
  } else {
    const int64_t gx = ext_x + 3, gy = ext_y + 3, gz = ext_z + 3;
    plan.sy = gx;
    plan.sz = gx * gy;
    plan.sb = plan.sz * gz;
    // ext_b <= 65535 and each g <= 65537, so compare in steps to avoid overflow.
    const bool small = plan.sb <= grid_budget_cells && ext_b <= grid_budget_cells / plan.sb;
    plan.cells = small ? plan.sb * ext_b : 0;
    plan.mode = (small && mode_request != SUBM_MAP_HASH) ? kModeGrid : kModeHash;
  }
  plan.flags = flags;
}

__device__ __forceinline__ int64_t grid_cell(const int32_t (&mn)[4], int64_t sb, int64_t sz, int64_t sy, int b, int z,
                                             int y, int x) {
  return (int64_t)(b - mn[0]) * sb + (int64_t)(z - mn[1] + 1) * sz + (int64_t)(y - mn[2] + 1) * sy +
         (int64_t)(x - mn[3] + 1);
}
__device__ __forceinline__ int64_t grid_cell(const MapStats& p, int b, int z, int y, int x) {
  return grid_cell(p.mn, p.sb, p.sz, p.sy, b, z, y, x);
}

__global__ __launch_bounds__(kThreads) void map_insert_kernel(const int32_t* __restrict__ coords, int64_t n,
                                                              const BoundsPartial* __restrict__ partials, int nparts,
                                                              int64_t grid_budget_cells, int64_t slots,
                                                              int mode_request, void* __restrict__ hash_table,
                                                              int32_t* __restrict__ grid, uint32_t tag,
                                                              uint32_t* __restrict__ banks,
                                                              MapStats* __restrict__ st,
                                                              MapHostFlags* __restrict__ host) {
  Plan plan;
  int32_t mx[4];
  reduce_plan(partials, nparts, grid_budget_cells, mode_request, plan, mx);
  const int t = threadIdx.x;
  if (blockIdx.x == 0) {  // publish the plan for the lookup kernel, the next build and the host
    if (t == 0) {
      // (constant indices: indexing the plan's arrays by thread would move them into LDS)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        st->mn[a] = plan.mn[a];
        st->mx[a] = mx[a];
      }
      host->flags = plan.flags;
      host->mode = plan.mode;
      st->flags = plan.flags;
      st->err_flags = 0;
      st->mode = plan.mode;
      st->cells = plan.cells;
      st->slots = slots;
      st->sy = plan.sy;
      st->sz = plan.sz;
      st->sb = plan.sb;
    }
    for (int k = t; k < kTapBanks * 27; k += kThreads) banks[k] = 0;
  }
  if (plan.mode == kModeNone) return;
  bool dup = false, overflow = false;
  if (plan.mode == kModeGrid) {
    // One contiguous run of rows per block, four rows per thread in flight; a plain store each
    // (two rows on one cell: the lookup sees it).
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t beg = xcd_block(blockIdx.x, gridDim.x) * per;
    const int64_t end = beg + per < n ? beg + per : n;
    for (int64_t i0 = beg + t; i0 < end; i0 += 4 * kThreads) {
      int4 c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * kThreads;
        c[u] = *reinterpret_cast<const int4*>(coords + 4 * (i < end ? i : i0));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * kThreads;
        if (i < end) grid[grid_cell(plan.mn, plan.sb, plan.sz, plan.sy, c[u].x, c[u].y, c[u].z, c[u].w)] =
            (int32_t)(tag + (uint32_t)i);
      }
    }
  } else {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    Slot* tab = static_cast<Slot*>(hash_table);
    for (int64_t i = (int64_t)blockIdx.x * kThreads + t; i < n; i += stride) {
      const int4 c = *reinterpret_cast<const int4*>(coords + 4 * i);
      const unsigned long long key = pack_key(c.x, c.y, c.z, c.w);
      unsigned long long s = home_slot(key, (unsigned long long)slots);
      bool placed = false;
      for (unsigned long long probe = 0; probe < (unsigned long long)slots; ++probe) {
        const unsigned long long prev = atomicCAS(&tab[s].key, kEmptyKey, key);
        if (prev == kEmptyKey) {
          tab[s].val = (int32_t)i;
          placed = true;
          break;
        }
        if (prev == key) {
          dup = true;
          placed = true;
          break;
        }
        s = (s + 1 == (unsigned long long)slots) ? 0 : s + 1;
      }
      overflow |= !placed;
    }
  }
  if (dup) host->duplicate = 1u;
  if (overflow) host->overflow = 1u;
}

// ------------------------------------------------------------------ lookup
// Three threads per voxel, one per dz plane (the plane index is uniform over each group of four
// waves): the plane's 9 neighbours are resolved with all 9 loads in flight, staged in LDS, and
// the block's rows written back as one contiguous block of nbr.
__device__ __forceinline__ int32_t probe_rest(const Slot* __restrict__ tab, unsigned long long slots,
                                              unsigned long long key, unsigned long long s) {
  // Continue a probe sequence after its home slot held another key.
  for (unsigned long long probe = 1; probe < slots; ++probe) {
    s = (s + 1 == slots) ? 0 : s + 1;
    const Slot e = tab[s];
    if (e.key == key) return e.val;
    if (e.key == kEmptyKey) return -1;
  }
  return -1;
}

__global__ __launch_bounds__(3 * kLookupVoxels) void map_lookup_kernel(const int32_t* __restrict__ coords, int64_t n,
                                                                      const void* __restrict__ hash_table,
                                                                      const int32_t* __restrict__ grid, uint32_t tag,
                                                                      int32_t* __restrict__ nbr,
                                                                      uint32_t* __restrict__ masks,
                                                                      uint32_t* __restrict__ banks,
                                                                      const MapStats* __restrict__ st,
                                                                      MapHostFlags* __restrict__ host) {
  __shared__ __align__(16) int32_t s_out[kLookupVoxels * 27];
  __shared__ uint32_t s_pm[3][kLookupVoxels];
  __shared__ uint32_t s_cnt[27];
  // Out-of-range coordinates (no structure built): every entry -1, so that work already enqueued
  // on the map by a caller who has not checked its status yet reads only valid entries.
  const int mode = st->mode;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int plane = t / kLookupVoxels;
  const int v = t - plane * kLookupVoxels;
  if (t < 27) s_cnt[t] = 0;
  const int64_t i0 = xcd_block(blockIdx.x, gridDim.x) * kLookupVoxels;
  const int64_t i = i0 + v;
  uint32_t pm = 0;  // hit bits of this plane's taps, at their tap positions
  if (i < n && mode == kModeNone) {
#pragma unroll
    for (int q = 0; q < 9; ++q) s_out[v * 27 + plane * 9 + q] = -1;
  } else if (i < n) {
    const int4 c = *reinterpret_cast<const int4*>(coords + 4 * i);
    if (mode == kModeGrid) {
      const int64_t sy = st->sy, sz = st->sz;
      const int64_t base = grid_cell(*st, c.x, c.y, c.z, c.w) + (plane - 1) * sz;
      int32_t val[9];
#pragma unroll
      for (int q = 0; q < 9; ++q) val[q] = grid[base + (q / 3 - 1) * sy + (q % 3 - 1)];
#pragma unroll
      for (int q = 0; q < 9; ++q) {
        const int k = plane * 9 + q;
        // an entry of this build is tag + row; anything else (empty, or an earlier build's) is absent
        const uint32_t r = (uint32_t)val[q] - tag;
        const int32_t row = r < (uint32_t)n ? (int32_t)r : -1;
        s_out[v * 27 + k] = row;
        pm |= (row >= 0 ? 1u : 0u) << k;
      }
      // The row's own cell holds another row when both have the same coordinates.
      if (plane == 1 && (uint32_t)val[4] - tag != (uint32_t)i) host->duplicate = 1u;
    } else {
      const Slot* tab = static_cast<const Slot*>(hash_table);
      const unsigned long long slots = (unsigned long long)st->slots;
      unsigned long long key[9], home[9];
      Slot e[9];
      const int dz = plane - 1;
#pragma unroll
      for (int q = 0; q < 9; ++q) {
        const int dy = q / 3 - 1, dx = q % 3 - 1;
        // Unsigned adds: wrap-around is harmless because only the low 16 bits enter the key.
        key[q] = pack_key(c.x, (int32_t)((uint32_t)c.y + (uint32_t)dz), (int32_t)((uint32_t)c.z + (uint32_t)dy),
                          (int32_t)((uint32_t)c.w + (uint32_t)dx));
        home[q] = home_slot(key[q], slots);
      }
#pragma unroll
      for (int q = 0; q < 9; ++q) e[q] = tab[home[q]];
#pragma unroll
      for (int q = 0; q < 9; ++q) {
        int32_t r;
        if (e[q].key == key[q]) r = e[q].val;
        else if (e[q].key == kEmptyKey) r = -1;
        else r = probe_rest(tab, slots, key[q], home[q]);
        const int k = plane * 9 + q;
        s_out[v * 27 + k] = r;
        pm |= (r >= 0 ? 1u : 0u) << k;
      }
    }
  }
  s_pm[plane][v] = pm;
  __syncthreads();
  const int64_t rows = (n - i0) < kLookupVoxels ? (n - i0) : kLookupVoxels;
  const int total = (int)rows * 27;
  int32_t* dst = nbr + i0 * 27;  // 16-byte aligned: i0 is a multiple of 256
  for (int e = 4 * t; e < total; e += 4 * 3 * kLookupVoxels) {
    if (e + 3 < total) *reinterpret_cast<int4*>(dst + e) = *reinterpret_cast<const int4*>(s_out + e);
    else
      for (int k = e; k < total; ++k) dst[k] = s_out[k];
  }
  if (plane == 0 && i < n) masks[i] = s_pm[0][v] | s_pm[1][v] | s_pm[2][v];
  // Per-tap hit counts: one ballot per tap of the plane and wave, LDS adds, 27 global adds per block.
#pragma unroll
  for (int q = 0; q < 9; ++q) {
    const int k = plane * 9 + q;
    const unsigned long long b = __ballot((pm >> k) & 1u);
    if (lane == 0 && b) atomicAdd(&s_cnt[k], (uint32_t)__popcll(b));
  }
  __syncthreads();
  if (t < 27 && s_cnt[t] != 0) atomicAdd(&banks[(blockIdx.x % kTapBanks) * 27 + t], s_cnt[t]);
}

__global__ __launch_bounds__(kThreads) void fill_kernel(int4* __restrict__ p, int64_t n16, int value) {
  const int4 v = make_int4(value, value, value, value);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += (int64_t)gridDim.x * kThreads) p[i] = v;
}

int clamp_blocks(int64_t b, int64_t cap) { return (int)(b < 1 ? 1 : (b > cap ? cap : b)); }

}  // namespace

int64_t map_hash_slots(int64_t n) { return n * 2 < 64 ? 64 : n * 2; }
int64_t map_grid_budget_cells(int64_t n) {
  const int64_t c = n * kGridCellsPerVoxel;
  return c < 4096 ? 4096 : (c > kGridMaxCells ? kGridMaxCells : c);
}
int map_bounds_blocks(int64_t n) { return clamp_blocks((n + 4 * kThreads - 1) / (4 * kThreads), kMaxBoundsBlocks); }
size_t map_hash_bytes(int64_t n) { return (size_t)map_hash_slots(n) * sizeof(Slot); }
size_t map_grid_bytes(int64_t n) { return (size_t)map_grid_budget_cells(n) * sizeof(int32_t); }
size_t map_partials_bytes(int64_t n) { return (size_t)map_bounds_blocks(n) * sizeof(BoundsPartial); }

hipError_t launch_map_build(const int32_t* coords, int64_t n, int mode_request, void* hash_table, int32_t* grid,
                            uint32_t tag, void* partials, int64_t prev_n, int32_t* nbr, uint32_t* masks,
                            uint32_t* banks, MapStats* stats, MapHostFlags* host_flags, hipEvent_t ready,
                            hipStream_t stream) {
  BoundsPartial* parts = static_cast<BoundsPartial*>(partials);
  const int nb = map_bounds_blocks(n);
  // Wide enough for the previous build's reset too (at most its hash slots, 2 per row).
  const int clear_blocks = clamp_blocks((map_hash_slots(prev_n) + 4 * kThreads - 1) / (4 * kThreads), kMaxWideBlocks);
  const int64_t slots = map_hash_slots(n);
  const int64_t budget = map_grid_budget_cells(n);
  // One voxel per insert thread up to kMaxInsertBlocks blocks (each hash CAS is a full round
  // trip), then more per thread.
  const int insert_blocks = clamp_blocks((n + kThreads - 1) / kThreads, kMaxInsertBlocks);
  const MapStats* cstats = stats;
  map_bounds_kernel<<<prev_n > 0 && clear_blocks > nb ? clear_blocks : nb, kThreads, 0, stream>>>(coords, n, nb, parts,
                                                                                                cstats, hash_table);
  const BoundsPartial* cparts = parts;
  map_insert_kernel<<<insert_blocks, kThreads, 0, stream>>>(coords, n, cparts, nb, budget, slots, mode_request,
                                                            hash_table, grid, tag, banks, stats, host_flags);
  // The event rides on the kernel's own completion (no marker packet between kernels).
  const void* chash = hash_table;
  const int32_t* cgrid = grid;
  hipExtLaunchKernelGGL(map_lookup_kernel, dim3((unsigned)((n + kLookupVoxels - 1) / kLookupVoxels)),
                        dim3(3 * kLookupVoxels), 0, stream, nullptr, ready, 0u, coords, n, chash, cgrid, tag, nbr,
                        masks, banks, cstats, host_flags);
  return hipGetLastError();
}

hipError_t launch_fill(void* p, size_t bytes, uint32_t value, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  fill_kernel<<<clamp_blocks((n16 + 4 * kThreads - 1) / (4 * kThreads), kMaxWideBlocks), kThreads, 0, stream>>>(
      static_cast<int4*>(p), n16, (int)value);
  return hipGetLastError();
}

}  // namespace submconv
