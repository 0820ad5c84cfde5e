// Indice map (rulebook) build for submanifold 3x3x3 convolution on gfx950.
//
// The pages build the map from sorted coordinate keys with 27 lookups per voxel, once per
// coordinate set (lato.2_mrp_mlx README, header summary).  Here the key set goes into an
// open-addressing hash table in HBM instead of a sorted array: one insert per voxel and one
// probe sequence per (voxel, tap), so no radix passes and no binary searches.  The result,
// nbr[i, k] = input row of the voxel at coord_i + offset(k) or -1, is unique and therefore
// identical to what any sorted-key construction gives.
//
// Key packing: (b, z mod 2^16, y mod 2^16, x mod 2^16) in 16-bit fields, b most significant.
// Reducing z, y, x modulo 2^16 is injective on every coordinate and every +-1 neighbour of it
// as long as each axis' extent (max - min) is at most 65534; the build checks that extent and
// the batch range [0, 65534] and reports SUBM_ERR_COORD_RANGE otherwise.  The all-ones key
// cannot occur (b <= 65534) and marks an empty slot.
//
// Kernels, all on the caller's stream:
//   map_clear_kernel    empty every slot; reset the statistics block
//   map_insert_kernel   CAS each key into the table (duplicate -> flag); per-column min/max
//   map_lookup_kernel   one thread per (voxel, tap): probe, write nbr coalesced, count hits
//   map_reduce_kernel   sum the per-block hit counts into per-tap and total pair counts
#include "internal.h"

namespace submconv {
namespace {

constexpr unsigned long long kEmptyKey = ~0ull;
constexpr int kThreads = 256;
constexpr int kMaxBlocks = 2048;

struct __align__(16) Slot {
  unsigned long long key;
  int32_t val;
  int32_t pad;
};
static_assert(sizeof(Slot) == 16, "slot must be 16 bytes");

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

__global__ __launch_bounds__(kThreads) void map_clear_kernel(Slot* __restrict__ table, int64_t slots,
                                                             BuildStats* __restrict__ st) {
  if (blockIdx.x == 0) {
    const int t = threadIdx.x;
    if (t < 4) {
      st->mn[t] = INT32_MAX;
      st->mx[t] = INT32_MIN;
    }
    if (t == 0) {
      st->flags = 0;
      st->pad = 0;
      st->pairs = 0;
    }
    if (t < 27) st->per_tap[t] = 0;
  }
  const Slot empty = {kEmptyKey, -1, 0};
  for (int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x; s < slots; s += (int64_t)gridDim.x * kThreads)
    table[s] = empty;
}

__device__ __forceinline__ int wave_min(int v) {
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

__global__ __launch_bounds__(kThreads) void map_insert_kernel(const int32_t* __restrict__ coords, int64_t n,
                                                              Slot* __restrict__ table, int64_t slots,
                                                              BuildStats* __restrict__ st) {
  int mn[4] = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX};
  int mx[4] = {INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
  uint32_t flags = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int32_t* c = coords + 4 * i;
    const int32_t b = c[0], z = c[1], y = c[2], x = c[3];
    mn[0] = min(mn[0], b); mx[0] = max(mx[0], b);
    mn[1] = min(mn[1], z); mx[1] = max(mx[1], z);
    mn[2] = min(mn[2], y); mx[2] = max(mx[2], y);
    mn[3] = min(mn[3], x); mx[3] = max(mx[3], x);
    if (b < 0 || b >= SUBM_MAX_BATCH) {
      flags |= kFlagBatchRange;
      continue;
    }
    const unsigned long long key = pack_key(b, z, y, x);
    unsigned long long s = home_slot(key, (unsigned long long)slots);
    bool placed = false;
    for (int64_t probe = 0; probe < slots; ++probe) {
      const unsigned long long prev = atomicCAS(&table[s].key, kEmptyKey, key);
      if (prev == kEmptyKey) {
        table[s].val = (int32_t)i;
        placed = true;
        break;
      }
      if (prev == key) {
        flags |= kFlagDuplicate;
        placed = true;
        break;
      }
      s = (s + 1 == (unsigned long long)slots) ? 0 : s + 1;
    }
    if (!placed) flags |= kFlagProbeOverflow;
  }
  // Block reduction of min / max / flags, then one atomic per quantity per block.
  __shared__ int smn[kThreads / 64][4];
  __shared__ int smx[kThreads / 64][4];
  __shared__ uint32_t sfl;
  if (threadIdx.x == 0) sfl = 0;
  __syncthreads();
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
  if (flags) atomicOr(&sfl, flags);
  __syncthreads();
  if (threadIdx.x < 4) {
    const int a = threadIdx.x;
    int lo = smn[0][a], hi = smx[0][a];
    for (int w = 1; w < kThreads / 64; ++w) {
      lo = min(lo, smn[w][a]);
      hi = max(hi, smx[w][a]);
    }
    if (lo != INT32_MAX) atomicMin(&st->mn[a], lo);
    if (hi != INT32_MIN) atomicMax(&st->mx[a], hi);
  }
  if (threadIdx.x == 0 && sfl) atomicOr(&st->flags, sfl);
}

__global__ __launch_bounds__(kThreads) void map_lookup_kernel(const int32_t* __restrict__ coords, int64_t n,
                                                              const Slot* __restrict__ table, int64_t slots,
                                                              int32_t* __restrict__ nbr,
                                                              uint32_t* __restrict__ partials) {
  __shared__ uint32_t hits[27];
  if (threadIdx.x < 27) hits[threadIdx.x] = 0;
  __syncthreads();
  const int64_t total = n * 27;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total; t += (int64_t)gridDim.x * kThreads) {
    const int64_t i = t / 27;
    const int k = (int)(t - i * 27);
    const int32_t* c = coords + 4 * i;
    const int32_t b = c[0];
    // Unsigned adds: wrap-around is harmless because only the low 16 bits enter the key.
    const int32_t z = (int32_t)((uint32_t)c[1] + (uint32_t)(k / 9 - 1));
    const int32_t y = (int32_t)((uint32_t)c[2] + (uint32_t)((k / 3) % 3 - 1));
    const int32_t x = (int32_t)((uint32_t)c[3] + (uint32_t)(k % 3 - 1));
    int32_t found = -1;
    if (b >= 0 && b < SUBM_MAX_BATCH) {
      const unsigned long long key = pack_key(b, z, y, x);
      unsigned long long s = home_slot(key, (unsigned long long)slots);
      for (int64_t probe = 0; probe < slots; ++probe) {
        const Slot e = table[s];
        if (e.key == key) {
          found = e.val;
          break;
        }
        if (e.key == kEmptyKey) break;
        s = (s + 1 == (unsigned long long)slots) ? 0 : s + 1;
      }
    }
    nbr[t] = found;
    if (found >= 0) atomicAdd(&hits[k], 1u);
  }
  __syncthreads();
  if (threadIdx.x < 27) partials[(int64_t)blockIdx.x * 27 + threadIdx.x] = hits[threadIdx.x];
}

__global__ __launch_bounds__(kThreads) void map_reduce_kernel(const uint32_t* __restrict__ partials, int blocks,
                                                              BuildStats* __restrict__ st) {
  // 9 threads per tap, each summing every 9th block; then an LDS reduction.
  __shared__ unsigned long long part[27][9];
  const int t = threadIdx.x;
  if (t < 27 * 9) {
    const int k = t % 27, r = t / 27;
    unsigned long long acc = 0;
    for (int b = r; b < blocks; b += 9) acc += partials[(int64_t)b * 27 + k];
    part[k][r] = acc;
  }
  __syncthreads();
  if (t < 27) {
    unsigned long long acc = 0;
    for (int r = 0; r < 9; ++r) acc += part[t][r];
    st->per_tap[t] = acc;
    part[t][0] = acc;
  }
  __syncthreads();
  if (t == 0) {
    unsigned long long total = 0;
    for (int k = 0; k < 27; ++k) total += part[k][0];
    st->pairs = total;
  }
}

int blocks_for(int64_t items) {
  const int64_t b = (items + kThreads - 1) / kThreads;
  return (int)(b < 1 ? 1 : (b > kMaxBlocks ? kMaxBlocks : b));
}

}  // namespace

int64_t map_table_slots(int64_t n) { return n * 2 < 64 ? 64 : n * 2; }

int map_partial_blocks(int64_t n) { return blocks_for(n * 27); }

hipError_t launch_map_build(const int32_t* coords, int64_t n, void* table, int64_t table_slots,
                            uint32_t* partials, int partial_blocks, int32_t* nbr, BuildStats* stats,
                            hipStream_t stream) {
  Slot* tab = static_cast<Slot*>(table);
  map_clear_kernel<<<blocks_for(table_slots), kThreads, 0, stream>>>(tab, table_slots, stats);
  map_insert_kernel<<<blocks_for(n), kThreads, 0, stream>>>(coords, n, tab, table_slots, stats);
  map_lookup_kernel<<<partial_blocks, kThreads, 0, stream>>>(coords, n, tab, table_slots, nbr, partials);
  map_reduce_kernel<<<1, kThreads, 0, stream>>>(partials, partial_blocks, stats);
  return hipGetLastError();
}

}  // namespace submconv
