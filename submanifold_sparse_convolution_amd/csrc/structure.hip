// Structure ops around SubMConv3d: subdivide, 2x downsample (max / mean), 2x upsample (cached and
// masked) and the child indice map of a subdivide.  The C entry points are declared in
// sparse_structure.h, which also states what each one computes and where the pages fix it.
//
// All of it is memory-bound integer and copy work, so the kernels are plain one-thread-per-item
// launches with coalesced 16-byte rows; the downsample's distinct cells in ascending order and the
// masked upsample's child positions come from the radix sort and prefix sum of sort_scan.hip.
#include <cstring>
#include <algorithm>
#include <climits>
#include <mutex>
#include <new>

#include "internal.h"
#include "sparse_structure.h"

namespace submconv {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 4096;
constexpr int32_t kChildLimit = (1 << 30) - 1;  // |coordinate| bound so that 2c + 1 fits int32

int grid_for(int64_t items, int per_thread = 1) {
  const int64_t b = (items + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  return (int)(b < 1 ? 1 : (b > kMaxBlocks ? kMaxBlocks : b));
}

// ---------------------------------------------------------------------------------------------
// Per-column minimum and maximum of (b, z, y, x): per-block partials, then one block reduces them
// (no atomics: with every wave hitting the same eight words they serialise in L2).

struct CoordRange {
  int32_t mn[4];
  int32_t mx[4];
};

constexpr int kRangeBlocks = 256;

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Block-wide min / max of 4 columns; the result is valid in thread 0.
__device__ __forceinline__ void block_range(int (&mn)[4], int (&mx)[4]) {
  __shared__ int s[kThreads / 64][8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    mn[c] = wave_min(mn[c]);
    mx[c] = wave_max(mx[c]);
  }
  if (lane == 0)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s[wave][c] = mn[c];
      s[wave][4 + c] = mx[c];
    }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < kThreads / 64; ++w)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        mn[c] = min(mn[c], s[w][c]);
        mx[c] = max(mx[c], s[w][4 + c]);
      }
}

__global__ __launch_bounds__(kThreads) void range_partial_kernel(const int4* __restrict__ coords, int64_t n,
                                                                 CoordRange* __restrict__ partials) {
  int mn[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
  int mx[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int4 c = coords[i];
    mn[0] = min(mn[0], c.x); mx[0] = max(mx[0], c.x);
    mn[1] = min(mn[1], c.y); mx[1] = max(mx[1], c.y);
    mn[2] = min(mn[2], c.z); mx[2] = max(mx[2], c.z);
    mn[3] = min(mn[3], c.w); mx[3] = max(mx[3], c.w);
  }
  block_range(mn, mx);
  if (threadIdx.x == 0)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      partials[blockIdx.x].mn[c] = mn[c];
      partials[blockIdx.x].mx[c] = mx[c];
    }
}

__global__ __launch_bounds__(kThreads) void range_final_kernel(const CoordRange* __restrict__ partials, int nparts,
                                                               CoordRange* __restrict__ r) {
  int mn[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
  int mx[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
  for (int b = threadIdx.x; b < nparts; b += kThreads)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mn[c] = min(mn[c], partials[b].mn[c]);
      mx[c] = max(mx[c], partials[b].mx[c]);
    }
  block_range(mn, mx);
  if (threadIdx.x == 0)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r->mn[c] = mn[c];
      r->mx[c] = mx[c];
    }
}

// ---------------------------------------------------------------------------------------------
// Subdivide: child s of row i at row 8i + s, offset (s>>2 & 1, s>>1 & 1, s & 1) on (z, y, x).

__global__ __launch_bounds__(kThreads) void subdivide_kernel(const int4* __restrict__ coarse, int64_t n,
                                                             int4* __restrict__ fine, int32_t* __restrict__ parent,
                                                             int32_t* __restrict__ seg_off) {
  const int64_t total = 8 * n;
  for (int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x; r < total; r += (int64_t)gridDim.x * kThreads) {
    const int64_t i = r >> 3;
    const int s = (int)(r & 7);
    const int4 c = coarse[i];
    fine[r] = make_int4(c.x, 2 * c.y + ((s >> 2) & 1), 2 * c.z + ((s >> 1) & 1), 2 * c.w + (s & 1));
    parent[r] = (int32_t)i;
    if (s == 0) seg_off[i] = (int32_t)r;
    if (r == 0) seg_off[n] = (int32_t)total;
  }
}

// ---------------------------------------------------------------------------------------------
// Masked upsample.  Row i's mask is 8 bytes; child s exists when byte s != 0, at offset
// (s & 1, s>>1 & 1, s>>2 & 1) on (z, y, x); children parent-major, s ascending.

__device__ __forceinline__ uint32_t mask_bits(const uint8_t* __restrict__ mask, int64_t i) {
  uint32_t bits = 0;
#pragma unroll
  for (int s = 0; s < 8; ++s) bits |= (mask[i * 8 + s] != 0 ? 1u : 0u) << s;
  return bits;
}

__global__ __launch_bounds__(kThreads) void mask_count_kernel(const uint8_t* __restrict__ mask, int64_t n,
                                                              int32_t* __restrict__ count) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    count[i] = __popc(mask_bits(mask, i));
}

// incl[i] = number of children of rows 0 .. i (inclusive scan of the counts).
__global__ __launch_bounds__(kThreads) void masked_emit_kernel(const int4* __restrict__ coarse,
                                                               const uint8_t* __restrict__ mask, int64_t n,
                                                               const int32_t* __restrict__ incl,
                                                               int4* __restrict__ fine, int32_t* __restrict__ parent,
                                                               int32_t* __restrict__ seg_off) {
  const int64_t total = 8 * n;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total; t += (int64_t)gridDim.x * kThreads) {
    const int64_t i = t >> 3;
    const int s = (int)(t & 7);
    const uint32_t bits = mask_bits(mask, i);
    const int32_t first = incl[i] - (int32_t)__popc(bits);
    if (s == 0) seg_off[i] = first;
    if (t == 0) seg_off[n] = incl[n - 1];
    if ((bits >> s) & 1u) {
      const int32_t pos = first + (int32_t)__popc(bits & ((1u << s) - 1u));
      const int4 c = coarse[i];
      fine[pos] = make_int4(c.x, 2 * c.y + (s & 1), 2 * c.z + ((s >> 1) & 1), 2 * c.w + ((s >> 2) & 1));
      parent[pos] = (int32_t)i;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Downsample build.  Key of a fine row = its coarse cell packed as
//   ((b - b0) << (bz + by + bx)) | ((zc - z0) << (by + bx)) | ((yc - y0) << bx) | (xc - x0)
// with zc = z >> 1 (arithmetic shift: floor division) and field widths just wide enough for the
// extents, so ascending keys are ascending (b, z, y, x) and the radix sort runs over few bits.

struct KeyPack {
  int32_t lo[4];   // b0, z0, y0, x0 (coarse minima)
  int shift[4];    // bit position of each field
};

template <typename K>
__global__ __launch_bounds__(kThreads) void cell_key_kernel(const int4* __restrict__ coords, int64_t n, KeyPack p,
                                                            K* __restrict__ keys, int32_t* __restrict__ rows) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int4 c = coords[i];
    const K k = ((K)(uint32_t)(c.x - p.lo[0]) << p.shift[0]) | ((K)(uint32_t)((c.y >> 1) - p.lo[1]) << p.shift[1]) |
                ((K)(uint32_t)((c.z >> 1) - p.lo[2]) << p.shift[2]) | ((K)(uint32_t)((c.w >> 1) - p.lo[3]) << p.shift[3]);
    keys[i] = k;
    rows[i] = (int32_t)i;
  }
}

template <typename K>
__global__ __launch_bounds__(kThreads) void cell_head_kernel(const K* __restrict__ keys, int64_t n,
                                                             int32_t* __restrict__ head) {
  for (int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x; p < n; p += (int64_t)gridDim.x * kThreads)
    head[p] = (p == 0 || keys[p] != keys[p - 1]) ? 1 : 0;
}

// cid[p] = 1 + coarse row of sorted position p (inclusive scan of the head flags).
template <typename K>
__global__ __launch_bounds__(kThreads) void cell_emit_kernel(const K* __restrict__ keys, const int32_t* __restrict__ rows,
                                                             const int32_t* __restrict__ cid, int64_t n, KeyPack p,
                                                             int4* __restrict__ coarse, int32_t* __restrict__ parent,
                                                             int32_t* __restrict__ seg_off,
                                                             int32_t* __restrict__ seg_rows) {
  // field c occupies bits [shift[c], shift[c - 1]) (x: [0, shift[2]))
  const K mz = ((K)1 << (p.shift[0] - p.shift[1])) - 1;
  const K my = ((K)1 << (p.shift[1] - p.shift[2])) - 1;
  const K mx = ((K)1 << p.shift[2]) - 1;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < n; q += (int64_t)gridDim.x * kThreads) {
    const int32_t m = cid[q] - 1;
    const int32_t row = rows[q];
    parent[row] = m;
    seg_rows[q] = row;
    const K k = keys[q];
    if (q == 0 || k != keys[q - 1]) {
      seg_off[m] = (int32_t)q;
      coarse[m] = make_int4((int32_t)(k >> p.shift[0]) + p.lo[0], (int32_t)((k >> p.shift[1]) & mz) + p.lo[1],
                            (int32_t)((k >> p.shift[2]) & my) + p.lo[2], (int32_t)(k & mx) + p.lo[3]);
    }
    if (q == n - 1) seg_off[m + 1] = (int32_t)n;
  }
}

// ---------------------------------------------------------------------------------------------
// Feature kernels.  A "chunk" is 16 bytes of a row when the row size and both base pointers allow
// it, else one element.

enum class DT { F32, F16, BF16 };

template <DT D> __device__ __forceinline__ float load_f(const void* p, int64_t idx);
template <> __device__ __forceinline__ float load_f<DT::F32>(const void* p, int64_t idx) {
  return static_cast<const float*>(p)[idx];
}
template <> __device__ __forceinline__ float load_f<DT::F16>(const void* p, int64_t idx) {
  return (float)static_cast<const _Float16*>(p)[idx];
}
template <> __device__ __forceinline__ float load_f<DT::BF16>(const void* p, int64_t idx) {
  return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[idx] << 16);
}
template <DT D> __device__ __forceinline__ void store_f(void* p, int64_t idx, float v);
template <> __device__ __forceinline__ void store_f<DT::F32>(void* p, int64_t idx, float v) {
  static_cast<float*>(p)[idx] = v;
}
template <> __device__ __forceinline__ void store_f<DT::F16>(void* p, int64_t idx, float v) {
  static_cast<_Float16*>(p)[idx] = (_Float16)v;  // round to nearest even
}
template <> __device__ __forceinline__ void store_f<DT::BF16>(void* p, int64_t idx, float v) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t h = __builtin_convertvector((f32x2_t){v, v}, bf16x2_t);  // round to nearest even
  static_cast<uint16_t*>(p)[idx] = (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xFFFFu);
}

// Row-by-word thread layout shared by the feature kernels: a block covers rpb rows per step,
// words consecutive threads per row (words = 16-byte chunks or elements of a row), so no thread
// divides its item index.  Rows wider than the block take several passes of the same threads.
struct RowLanes {
  int rpb;    // rows per block step
  int r;      // this thread's row within the step (r >= rpb: idle)
  int w0;     // first word of this thread
  int wstep;  // word stride
  __device__ RowLanes(int words) {
    if (words >= kThreads) {
      rpb = 1, r = 0, w0 = threadIdx.x, wstep = kThreads;
    } else {
      rpb = kThreads / words;
      r = threadIdx.x / words;
      w0 = threadIdx.x - r * words;
      wstep = words;
    }
  }
};

// Pooling: for every coarse row m and element group of E elements (E = 16 bytes / element size
// on the vector path, 1 otherwise), max or mean over the members.
template <DT D, int E, bool MAX>
__global__ __launch_bounds__(kThreads) void pool_kernel(const void* __restrict__ fine, void* __restrict__ coarse,
                                                        int64_t n_coarse, int channels,
                                                        const int32_t* __restrict__ seg_off,
                                                        const int32_t* __restrict__ seg_rows) {
  const int words = channels / E;
  const RowLanes L(words);
  if (L.r >= L.rpb) return;
  for (int64_t m = (int64_t)blockIdx.x * L.rpb + L.r; m < n_coarse; m += (int64_t)gridDim.x * L.rpb) {
    const int32_t lo = seg_off[m], hi = seg_off[m + 1];
    const int cnt = hi - lo;
    for (int w = L.w0; w < words; w += L.wstep) {
      const int c0 = w * E;
      float acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = MAX ? -__builtin_inff() : 0.f;
      if constexpr (E > 1) {
        // four members at a time: their row indices, then their words, all in flight together
        for (int32_t q0 = lo; q0 < hi; q0 += 4) {
          int64_t f[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) f[u] = q0 + u < hi ? (seg_rows != nullptr ? seg_rows[q0 + u] : q0 + u) : -1;
          uint4 raw[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            raw[u] = f[u] >= 0 ? *reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(fine) +
                                                                 (f[u] * channels + c0) * (16 / E))
                               : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (f[u] < 0) continue;
            const unsigned char* b = reinterpret_cast<const unsigned char*>(&raw[u]);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float v = load_f<D>(b, e);
              acc[e] = MAX ? fmaxf(acc[e], v) : acc[e] + v;
            }
          }
        }
      } else {
        for (int32_t q = lo; q < hi; ++q) {
          const int64_t f = seg_rows != nullptr ? seg_rows[q] : q;
          const float v = load_f<D>(fine, f * channels + c0);
          acc[0] = MAX ? fmaxf(acc[0], v) : acc[0] + v;
        }
      }
      const int64_t obase = m * channels + c0;
      if constexpr (E > 1) {
        uint4 raw;
        unsigned char* b = reinterpret_cast<unsigned char*>(&raw);
#pragma unroll
        for (int e = 0; e < E; ++e) store_f<D>(b, e, cnt == 0 ? 0.f : (MAX ? acc[e] : acc[e] / (float)cnt));
        *reinterpret_cast<uint4*>(static_cast<unsigned char*>(coarse) + obase * (16 / E)) = raw;
      } else {
        store_f<D>(coarse, obase, cnt == 0 ? 0.f : (MAX ? acc[0] : acc[0] / (float)cnt));
      }
    }
  }
}

// fine[f] = coarse[parent[f]], copied in words W (16, 4 or 2 bytes).
template <typename W>
__global__ __launch_bounds__(kThreads) void expand_kernel(const W* __restrict__ coarse, W* __restrict__ fine,
                                                          int64_t n_fine, int words,
                                                          const int32_t* __restrict__ parent) {
  const RowLanes L(words);
  if (L.r >= L.rpb) return;
  for (int64_t f = (int64_t)blockIdx.x * L.rpb + L.r; f < n_fine; f += (int64_t)gridDim.x * L.rpb) {
    const int64_t src = (int64_t)parent[f] * words;
    for (int w = L.w0; w < words; w += L.wstep) fine[f * words + w] = coarse[src + w];
  }
}

// Upsample of a subdivide: fine rows 8i .. 8i + 7 are all copies of coarse row i, so each coarse
// word is read once and stored eight times, with no parent index to read.
template <typename W>
__global__ __launch_bounds__(kThreads) void expand8_kernel(const W* __restrict__ coarse, W* __restrict__ fine,
                                                           int64_t n_coarse, int words) {
  const RowLanes L(words);
  if (L.r >= L.rpb) return;
  for (int64_t i = (int64_t)blockIdx.x * L.rpb + L.r; i < n_coarse; i += (int64_t)gridDim.x * L.rpb) {
    W* dst = fine + i * 8 * words;
    for (int w = L.w0; w < words; w += L.wstep) {
      const W v = coarse[i * words + w];
#pragma unroll
      for (int c = 0; c < 8; ++c) dst[c * words + w] = v;
    }
  }
}

// Blocks for a row-by-word launch over `rows` rows of `words` words.
int row_grid(int64_t rows, int words) {
  const int rpb = words >= kThreads ? 1 : kThreads / words;
  const int64_t b = (rows + rpb - 1) / rpb;
  return (int)(b < 1 ? 1 : (b > 16384 ? 16384 : b));
}

// ---------------------------------------------------------------------------------------------
// Child indice map.  Child r = 8i + s of parent i sits at 2 p_i + o with o = (s>>2 & 1, s>>1 & 1,
// s & 1).  Its neighbour at offset d is 2 p_i + t, t = o + d in {-1, 0, 1, 2}^3, i.e. child
// (t mod 2) of the voxel at p_i + floor(t / 2): nbr_child[r][k] = 8 nbr_parent[i][q] + s' when
// that parent neighbour exists (all its children exist), else -1.  A block owns 32 parents
// (256 children): parent rows staged in LDS, child rows staged in LDS and written coalesced.

constexpr int kChildParents = kThreads / 8;

__global__ __launch_bounds__(kThreads) void child_map_kernel(const int32_t* __restrict__ pnbr, int64_t np,
                                                             int32_t* __restrict__ cnbr, uint32_t* __restrict__ cmask) {
  __shared__ int32_t sp[kChildParents * 27];
  __shared__ __align__(16) int32_t sc[kThreads * 27];
  const int64_t p0 = (int64_t)blockIdx.x * kChildParents;
  const int64_t pcount = min((int64_t)kChildParents, np - p0);
  for (int e = threadIdx.x; e < pcount * 27; e += kThreads) sp[e] = pnbr[p0 * 27 + e];
  __syncthreads();
  const int tid = threadIdx.x;
  const int lp = tid >> 3, s = tid & 7;
  const int64_t r = p0 * 8 + tid;
  if (lp < pcount) {
    const int oz = (s >> 2) & 1, oy = (s >> 1) & 1, ox = s & 1;
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < 27; ++k) {
      const int tz = oz + k / 9 - 1, ty = oy + (k / 3) % 3 - 1, tx = ox + k % 3 - 1;
      const int q = 9 * ((tz >> 1) + 1) + 3 * ((ty >> 1) + 1) + ((tx >> 1) + 1);
      const int32_t pn = sp[lp * 27 + q];
      const int32_t v = pn >= 0 ? 8 * pn + (((tz & 1) << 2) | ((ty & 1) << 1) | (tx & 1)) : -1;
      sc[tid * 27 + k] = v;
      bits |= (v >= 0 ? 1u : 0u) << k;
    }
    cmask[r] = bits;
  }
  __syncthreads();
  // The block's rows are one contiguous, 16-byte aligned run (8 rows of 27 int32 per parent, a
  // multiple of 4 entries): 16-byte stores.  (Computing each 16-byte word from the parent rows
  // instead of staging the child rows in LDS measured 20 % slower.)
  const int words = (int)(pcount * 8 * 27 / 4);
  int4* dst4 = reinterpret_cast<int4*>(cnbr + p0 * 8 * 27);
  const int4* src4 = reinterpret_cast<const int4*>(sc);
  for (int e = tid; e < words; e += kThreads) dst4[e] = src4[e];
}

// ---------------------------------------------------------------------------------------------
// Host helpers.

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// One device allocation for a handle's arrays.
Status alloc_subdiv(SubdivData& d, bool with_seg_rows, hipStream_t stream) {
  const size_t c = align256((size_t)d.n_coarse * 16);
  const size_t f = align256((size_t)d.n_fine * 16);
  const size_t p = align256((size_t)d.n_fine * 4);
  const size_t o = align256((size_t)(d.n_coarse + 1) * 4);
  const size_t r = with_seg_rows ? align256((size_t)d.n_fine * 4) : 0;
  void* block = nullptr;
  Status s = device_alloc(&block, c + f + p + o + r, stream);
  if (!s.ok()) return s;
  unsigned char* b = static_cast<unsigned char*>(block);
  d.block = block;
  d.coarse = reinterpret_cast<int32_t*>(b);
  d.fine = reinterpret_cast<int32_t*>(b + c);
  d.parent = reinterpret_cast<int32_t*>(b + c + f);
  d.seg_off = reinterpret_cast<int32_t*>(b + c + f + p);
  d.seg_rows = with_seg_rows ? reinterpret_cast<int32_t*>(b + c + f + p + o) : nullptr;
  return Status{};
}

// Device scratch of enqueue_range: the result followed by the per-block partials.
constexpr size_t kRangeScratch = sizeof(CoordRange) * (kRangeBlocks + 1);

// Launches the range reduction into `dev_range` (kRangeScratch bytes) and a copy of the result
// into pinned host memory.
hipError_t enqueue_range(const int32_t* coords, int64_t n, CoordRange* dev_range, CoordRange* host_range,
                         hipStream_t stream) {
  const int blocks = (int)std::min<int64_t>(kRangeBlocks, (n + 4 * kThreads - 1) / (4 * kThreads));
  range_partial_kernel<<<blocks, kThreads, 0, stream>>>(reinterpret_cast<const int4*>(coords), n, dev_range + 1);
  range_final_kernel<<<1, kThreads, 0, stream>>>(dev_range + 1, blocks, dev_range);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return hipMemcpyAsync(host_range, dev_range, sizeof(CoordRange), hipMemcpyDeviceToHost, stream);
}

// Coordinates whose children must fit int32: b in [0, SUBM_MAX_BATCH), |z|, |y|, |x| <= 2^30 - 1.
const char* child_range_error(const CoordRange& r) {
  if (r.mn[0] < 0 || r.mx[0] >= SUBM_MAX_BATCH) return "batch index outside [0, 65534]";
  for (int c = 1; c < 4; ++c)
    if (r.mn[c] < -kChildLimit || r.mx[c] > kChildLimit) return "a coordinate exceeds 2^30 - 1 in magnitude";
  return nullptr;
}

int bit_width(uint32_t v) { return v == 0 ? 0 : 32 - __builtin_clz(v); }

struct Scratch {
  hipStream_t stream;
  void* p = nullptr;
  explicit Scratch(hipStream_t s) : stream(s) {}
  ~Scratch() { device_free(p, stream); }
};

bool common_checks(const int32_t* coords, int64_t n, int64_t max_n, sparse_subdivision_t* out, const char** err) {
  if (out == nullptr) { *err = "out is NULL"; return false; }
  *out = nullptr;
  if (n < 0) { *err = "n is negative"; return false; }
  if (n > max_n) { *err = "n exceeds the supported row count"; return false; }
  if (n > 0 && coords == nullptr) { *err = "coords is NULL"; return false; }
  if ((reinterpret_cast<uintptr_t>(coords) & 15u) != 0) { *err = "coords is not 16-byte aligned"; return false; }
  return true;
}

template <typename K>
Status downsample_sort(const int32_t* coords, int64_t n, const KeyPack& kp, int bits, SubdivData& d,
                       const Pinned& pin, hipStream_t stream) {
  // scratch: keys in / out, rows in / out, head flags, cell ids, sort and scan temporaries
  const size_t kb = align256((size_t)n * sizeof(K));
  const size_t rb = align256((size_t)n * 4);
  const size_t sort_tmp = radix_sort_scratch_bytes(n), scan_tmp = scan_scratch_bytes(n);
  const size_t tmp = align256(sort_tmp > scan_tmp ? sort_tmp : scan_tmp);
  Scratch scratch(stream);
  Status s = device_alloc(&scratch.p, 2 * kb + 4 * rb + tmp, stream);
  if (!s.ok()) return s;
  unsigned char* b = static_cast<unsigned char*>(scratch.p);
  K* keys_in = reinterpret_cast<K*>(b);
  K* keys_out = reinterpret_cast<K*>(b + kb);
  int32_t* rows_in = reinterpret_cast<int32_t*>(b + 2 * kb);
  int32_t* rows_out = reinterpret_cast<int32_t*>(b + 2 * kb + rb);
  int32_t* head = reinterpret_cast<int32_t*>(b + 2 * kb + 2 * rb);
  int32_t* cid = reinterpret_cast<int32_t*>(b + 2 * kb + 3 * rb);
  void* tmp_p = b + 2 * kb + 4 * rb;

  const int g = grid_for(n, 4);
  cell_key_kernel<K><<<g, kThreads, 0, stream>>>(reinterpret_cast<const int4*>(coords), n, kp, keys_in, rows_in);
  SUBM_HIP_TRY(hipGetLastError());
  bool in_alt = false;
  SUBM_HIP_TRY(launch_radix_sort_pairs<K>(keys_in, rows_in, keys_out, rows_out, n, bits, tmp_p, stream, &in_alt));
  const K* keys_sorted = in_alt ? keys_out : keys_in;
  const int32_t* rows_sorted = in_alt ? rows_out : rows_in;
  cell_head_kernel<K><<<g, kThreads, 0, stream>>>(keys_sorted, n, head);
  SUBM_HIP_TRY(hipGetLastError());
  SUBM_HIP_TRY(launch_scan(head, cid, n, false, tmp_p, stream));
  int32_t* host_count = static_cast<int32_t*>(pin.host);
  SUBM_HIP_TRY(hipMemcpyAsync(host_count, cid + (n - 1), sizeof(int32_t), hipMemcpyDeviceToHost, stream));
  SUBM_HIP_TRY(hipStreamSynchronize(stream));
  d.n_coarse = *host_count;
  s = alloc_subdiv(d, true, stream);
  if (!s.ok()) return s;
  SUBM_HIP_TRY(hipMemcpyAsync(d.fine, coords, (size_t)n * 16, hipMemcpyDeviceToDevice, stream));
  cell_emit_kernel<K><<<g, kThreads, 0, stream>>>(keys_sorted, rows_sorted, cid, n, kp, reinterpret_cast<int4*>(d.coarse),
                                                  d.parent, d.seg_off, d.seg_rows);
  SUBM_HIP_TRY(hipGetLastError());
  return Status{};
}

// a = coarse features [n_coarse, channels], b = fine features [n_fine, channels].
Status validate_features(const SubdivData& d, int channels, int dtype, const void* a, const void* b) {
  if (channels < 1 || channels > (1 << 24)) return make_status(SUBM_ERR_INVALID_ARG, "channels must be in [1, 2^24]");
  if (dtype != SUBM_F32 && dtype != SUBM_F16 && dtype != SUBM_BF16)
    return make_status(SUBM_ERR_UNSUPPORTED, "dtype must be SUBM_F32, SUBM_F16 or SUBM_BF16");
  if ((d.n_coarse > 0 && a == nullptr) || (d.n_fine > 0 && b == nullptr))
    return make_status(SUBM_ERR_INVALID_ARG, "a feature pointer is NULL");
  const uintptr_t elem = dtype == SUBM_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) % elem != 0)
    return make_status(SUBM_ERR_INVALID_ARG, "a pointer is not aligned to the element size");
  const uint64_t cb = (uint64_t)d.n_coarse * channels * elem, fb = (uint64_t)d.n_fine * channels * elem;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  if (pa < pb + fb && pb < pa + cb && cb > 0 && fb > 0)
    return make_status(SUBM_ERR_INVALID_ARG, "fine and coarse features overlap");
  int dev = -1;
  SUBM_HIP_TRY(hipGetDevice(&dev));
  if (dev != d.device) return make_status(SUBM_ERR_INVALID_ARG, "the handle was built on another device");
  return Status{};
}

template <DT D, int E>
hipError_t launch_pool(const SubdivData& d, int channels, bool max, const void* fine, void* coarse, hipStream_t stream) {
  const int g = row_grid(d.n_coarse, channels / E);
  if (max)
    pool_kernel<D, E, true><<<g, kThreads, 0, stream>>>(fine, coarse, d.n_coarse, channels, d.seg_off, d.seg_rows);
  else
    pool_kernel<D, E, false><<<g, kThreads, 0, stream>>>(fine, coarse, d.n_coarse, channels, d.seg_off, d.seg_rows);
  return hipGetLastError();
}

template <DT D>
hipError_t pool_dtype(const SubdivData& d, int channels, bool max, const void* fine, void* coarse, hipStream_t stream) {
  constexpr int S = D == DT::F32 ? 4 : 2;
  const bool vec = (channels * S) % 16 == 0 && (reinterpret_cast<uintptr_t>(fine) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(coarse) & 15u) == 0;
  if (vec) return launch_pool<D, 16 / S>(d, channels, max, fine, coarse, stream);
  return launch_pool<D, 1>(d, channels, max, fine, coarse, stream);
}

}  // namespace

hipError_t launch_child_map(const int32_t* parent_nbr, int64_t np, int32_t* nbr, uint32_t* masks, hipStream_t stream) {
  const int64_t blocks = (np + kChildParents - 1) / kChildParents;
  child_map_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(parent_nbr, np, nbr, masks);
  return hipGetLastError();
}

}  // namespace submconv

using namespace submconv;

extern "C" int sparse_subdivide(const int32_t* coords, int64_t n, hipStream_t stream, sparse_subdivision_t* out) {
  clear_error();
  const char* err = nullptr;
  if (!common_checks(coords, n, (int64_t(1) << 28) - 1, out, &err)) return fail(SUBM_ERR_INVALID_ARG, err);
  sparse_subdivision* h = new (std::nothrow) sparse_subdivision;
  if (h == nullptr) return fail(SUBM_ERR_OUT_OF_MEMORY, "host allocation of the handle failed");
  SubdivData& d = h->d;
  d.kind = SUBM_SUBDIVIDE;
  d.n_coarse = n;
  d.n_fine = 8 * n;
  if (hipGetDevice(&d.device) != hipSuccess) {
    delete h;
    return fail(SUBM_ERR_HIP, "hipGetDevice failed");
  }
  if (n == 0) {
    *out = h;
    return SUBM_OK;
  }
  const Pinned pin = pinned_block(d.device);
  Scratch range_buf(stream);
  Status s = pin.host == nullptr ? make_status(SUBM_ERR_OUT_OF_MEMORY, "pinned host block") : alloc_subdiv(d, false, stream);
  if (s.ok()) s = device_alloc(&range_buf.p, kRangeScratch, stream);
  if (!s.ok()) {
    device_free(d.block, stream);
    delete h;
    return fail(s);
  }
  CoordRange* host_range = static_cast<CoordRange*>(pin.host);
  hipError_t e = enqueue_range(coords, n, static_cast<CoordRange*>(range_buf.p), host_range, stream);
  if (e == hipSuccess) {
    subdivide_kernel<<<grid_for(8 * n, 4), kThreads, 0, stream>>>(reinterpret_cast<const int4*>(coords), n,
                                                                   reinterpret_cast<int4*>(d.fine), d.parent, d.seg_off);
    e = hipGetLastError();
  }
  if (e == hipSuccess)
    e = hipMemcpyAsync(d.coarse, coords, (size_t)n * 16, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    device_free(d.block, stream);
    delete h;
    return fail(hip_status(e, "subdivide"));
  }
  if (const char* msg = child_range_error(*host_range)) {
    device_free(d.block, stream);
    delete h;
    return fail(SUBM_ERR_COORD_RANGE, msg);
  }
  *out = h;
  return SUBM_OK;
}

extern "C" int sparse_upsample_masked_build(const int32_t* coords, const uint8_t* mask, int64_t n, hipStream_t stream,
                                            sparse_subdivision_t* out) {
  clear_error();
  const char* err = nullptr;
  if (!common_checks(coords, n, (int64_t(1) << 28) - 1, out, &err)) return fail(SUBM_ERR_INVALID_ARG, err);
  if (n > 0 && mask == nullptr) return fail(SUBM_ERR_INVALID_ARG, "mask is NULL");
  sparse_subdivision* h = new (std::nothrow) sparse_subdivision;
  if (h == nullptr) return fail(SUBM_ERR_OUT_OF_MEMORY, "host allocation of the handle failed");
  SubdivData& d = h->d;
  d.kind = SUBM_UPSAMPLE_MASKED;
  d.n_coarse = n;
  if (hipGetDevice(&d.device) != hipSuccess) {
    delete h;
    return fail(SUBM_ERR_HIP, "hipGetDevice failed");
  }
  if (n == 0) {
    *out = h;
    return SUBM_OK;
  }
  const Pinned pin = pinned_block(d.device);
  if (pin.host == nullptr) {
    delete h;
    return fail(SUBM_ERR_OUT_OF_MEMORY, "pinned host block");
  }
  // scratch: range, counts, inclusive scan, scan temporaries
  const size_t scan_tmp = scan_scratch_bytes(n);
  const size_t cb = align256((size_t)n * 4);
  Scratch scratch(stream);
  const size_t rb = align256(kRangeScratch);
  Status s = device_alloc(&scratch.p, rb + 2 * cb + align256(scan_tmp), stream);
  if (!s.ok()) {
    delete h;
    return fail(s);
  }
  unsigned char* b = static_cast<unsigned char*>(scratch.p);
  CoordRange* dev_range = reinterpret_cast<CoordRange*>(b);
  int32_t* count = reinterpret_cast<int32_t*>(b + rb);
  int32_t* incl = reinterpret_cast<int32_t*>(b + rb + cb);
  void* tmp_p = b + rb + 2 * cb;
  CoordRange* host_range = static_cast<CoordRange*>(pin.host);
  int32_t* host_total = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(pin.host) + 64);

  hipError_t e = enqueue_range(coords, n, dev_range, host_range, stream);
  if (e == hipSuccess) {
    mask_count_kernel<<<grid_for(n, 4), kThreads, 0, stream>>>(mask, n, count);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = launch_scan(count, incl, n, false, tmp_p, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(host_total, incl + (n - 1), sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    delete h;
    return fail(hip_status(e, "masked upsample count"));
  }
  if (const char* msg = child_range_error(*host_range)) {
    delete h;
    return fail(SUBM_ERR_COORD_RANGE, msg);
  }
  d.n_fine = *host_total;
  s = alloc_subdiv(d, false, stream);
  if (!s.ok()) {
    delete h;
    return fail(s);
  }
  e = hipMemcpyAsync(d.coarse, coords, (size_t)n * 16, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) {
    masked_emit_kernel<<<grid_for(8 * n, 4), kThreads, 0, stream>>>(reinterpret_cast<const int4*>(coords), mask, n, incl,
                                                                     reinterpret_cast<int4*>(d.fine), d.parent, d.seg_off);
    e = hipGetLastError();
  }
  if (e != hipSuccess) {
    device_free(d.block, stream);
    delete h;
    return fail(hip_status(e, "masked upsample emit"));
  }
  *out = h;
  return SUBM_OK;
}

extern "C" int sparse_downsample_build(const int32_t* coords, int64_t n, hipStream_t stream, sparse_subdivision_t* out) {
  clear_error();
  const char* err = nullptr;
  if (!common_checks(coords, n, INT32_MAX, out, &err)) return fail(SUBM_ERR_INVALID_ARG, err);
  sparse_subdivision* h = new (std::nothrow) sparse_subdivision;
  if (h == nullptr) return fail(SUBM_ERR_OUT_OF_MEMORY, "host allocation of the handle failed");
  SubdivData& d = h->d;
  d.kind = SUBM_DOWNSAMPLE;
  d.n_fine = n;
  if (hipGetDevice(&d.device) != hipSuccess) {
    delete h;
    return fail(SUBM_ERR_HIP, "hipGetDevice failed");
  }
  if (n == 0) {
    *out = h;
    return SUBM_OK;
  }
  const Pinned pin = pinned_block(d.device);
  if (pin.host == nullptr) {
    delete h;
    return fail(SUBM_ERR_OUT_OF_MEMORY, "pinned host block");
  }
  Scratch range_buf(stream);
  Status s = device_alloc(&range_buf.p, kRangeScratch, stream);
  if (!s.ok()) {
    delete h;
    return fail(s);
  }
  CoordRange* host_range = static_cast<CoordRange*>(pin.host);
  hipError_t e = enqueue_range(coords, n, static_cast<CoordRange*>(range_buf.p), host_range, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    delete h;
    return fail(hip_status(e, "downsample range"));
  }
  const CoordRange r = *host_range;
  if (r.mn[0] < 0 || r.mx[0] >= SUBM_MAX_BATCH) {
    delete h;
    return fail(SUBM_ERR_COORD_RANGE, "batch index outside [0, 65534]");
  }
  for (int c = 1; c < 4; ++c)
    if ((int64_t)r.mx[c] - (int64_t)r.mn[c] > SUBM_MAX_EXTENT) {
      delete h;
      return fail(SUBM_ERR_COORD_RANGE, "extent (max - min) of z, y or x exceeds 65534");
    }
  KeyPack kp{};
  int width[4];
  kp.lo[0] = r.mn[0];
  width[0] = bit_width((uint32_t)(r.mx[0] - r.mn[0]));
  for (int c = 1; c < 4; ++c) {
    kp.lo[c] = r.mn[c] >> 1;
    width[c] = bit_width((uint32_t)((r.mx[c] >> 1) - (r.mn[c] >> 1)));
  }
  kp.shift[3] = 0;
  kp.shift[2] = width[3];
  kp.shift[1] = width[3] + width[2];
  kp.shift[0] = width[3] + width[2] + width[1];
  const int bits = kp.shift[0] + width[0];
  // 32-bit keys while every field shift stays below 32
  s = bits < 32 ? downsample_sort<uint32_t>(coords, n, kp, bits < 1 ? 1 : bits, d, pin, stream)
                : downsample_sort<uint64_t>(coords, n, kp, bits, d, pin, stream);
  if (!s.ok()) {
    device_free(d.block, stream);
    delete h;
    return fail(s);
  }
  *out = h;
  return SUBM_OK;
}

extern "C" int sparse_subdivision_info(sparse_subdivision_t s, int64_t* n_coarse, int64_t* n_fine) {
  clear_error();
  if (s == nullptr) return fail(SUBM_ERR_INVALID_ARG, "handle is NULL");
  if (n_coarse != nullptr) *n_coarse = s->d.n_coarse;
  if (n_fine != nullptr) *n_fine = s->d.n_fine;
  return SUBM_OK;
}

extern "C" int sparse_subdivision_kind(sparse_subdivision_t s, int* kind) {
  clear_error();
  if (s == nullptr || kind == nullptr) return fail(SUBM_ERR_INVALID_ARG, "handle or kind is NULL");
  *kind = s->d.kind;
  return SUBM_OK;
}

extern "C" int sparse_subdivision_coords(sparse_subdivision_t s, int level, const int32_t** coords) {
  clear_error();
  if (s == nullptr || coords == nullptr) return fail(SUBM_ERR_INVALID_ARG, "handle or coords is NULL");
  if (level != SUBM_COARSE && level != SUBM_FINE) return fail(SUBM_ERR_INVALID_ARG, "level must be SUBM_COARSE or SUBM_FINE");
  const int64_t count = level == SUBM_COARSE ? s->d.n_coarse : s->d.n_fine;
  *coords = count == 0 ? nullptr : (level == SUBM_COARSE ? s->d.coarse : s->d.fine);
  return SUBM_OK;
}

extern "C" int sparse_subdivision_parent(sparse_subdivision_t s, const int32_t** parent) {
  clear_error();
  if (s == nullptr || parent == nullptr) return fail(SUBM_ERR_INVALID_ARG, "handle or parent is NULL");
  *parent = s->d.n_fine == 0 ? nullptr : s->d.parent;
  return SUBM_OK;
}

extern "C" int sparse_subdivision_copy(sparse_subdivision_t s, int what, void* dst, hipStream_t stream) {
  clear_error();
  if (s == nullptr) return fail(SUBM_ERR_INVALID_ARG, "handle is NULL");
  const void* src;
  size_t bytes;
  switch (what) {
    case SUBM_COARSE: src = s->d.coarse; bytes = (size_t)s->d.n_coarse * 16; break;
    case SUBM_FINE: src = s->d.fine; bytes = (size_t)s->d.n_fine * 16; break;
    case SUBM_PARENT: src = s->d.parent; bytes = (size_t)s->d.n_fine * 4; break;
    default: return fail(SUBM_ERR_INVALID_ARG, "what must be SUBM_COARSE, SUBM_FINE or SUBM_PARENT");
  }
  if (bytes == 0) return SUBM_OK;
  if (dst == nullptr) return fail(SUBM_ERR_INVALID_ARG, "dst is NULL");
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return fail(hip_status(e, "subdivision copy"));
  return SUBM_OK;
}

extern "C" int sparse_subdivision_free(sparse_subdivision_t s) {
  clear_error();
  if (s == nullptr) return SUBM_OK;
  if (s->d.block != nullptr) {
    DeviceGuard guard(s->d.device);
    device_free(s->d.block, nullptr);
  }
  delete s;
  return SUBM_OK;
}

extern "C" int sparse_downsample_forward(sparse_subdivision_t s, int channels, int dtype, int mode, const void* fine,
                                         void* coarse, hipStream_t stream) {
  clear_error();
  if (s == nullptr) return fail(SUBM_ERR_INVALID_ARG, "handle is NULL");
  if (mode != SUBM_POOL_MAX && mode != SUBM_POOL_MEAN)
    return fail(SUBM_ERR_INVALID_ARG, "mode must be SUBM_POOL_MAX or SUBM_POOL_MEAN (no default)");
  Status st = validate_features(s->d, channels, dtype, coarse, fine);
  if (!st.ok()) return fail(st);
  if (s->d.n_coarse == 0) return SUBM_OK;
  const bool max = mode == SUBM_POOL_MAX;
  hipError_t e;
  switch (dtype) {
    case SUBM_F32: e = pool_dtype<DT::F32>(s->d, channels, max, fine, coarse, stream); break;
    case SUBM_F16: e = pool_dtype<DT::F16>(s->d, channels, max, fine, coarse, stream); break;
    default: e = pool_dtype<DT::BF16>(s->d, channels, max, fine, coarse, stream); break;
  }
  if (e != hipSuccess) return fail(hip_status(e, "downsample launch"));
  return SUBM_OK;
}

extern "C" int sparse_upsample_forward(sparse_subdivision_t s, int channels, int dtype, const void* coarse, void* fine,
                                       hipStream_t stream) {
  clear_error();
  if (s == nullptr) return fail(SUBM_ERR_INVALID_ARG, "handle is NULL");
  Status st = validate_features(s->d, channels, dtype, coarse, fine);
  if (!st.ok()) return fail(st);
  if (s->d.n_fine == 0) return SUBM_OK;
  const size_t row = (size_t)channels * (dtype == SUBM_F32 ? 4 : 2);
  const uintptr_t ptrs = reinterpret_cast<uintptr_t>(coarse) | reinterpret_cast<uintptr_t>(fine);
  const int64_t nf = s->d.n_fine;
  if (s->d.kind == SUBM_SUBDIVIDE && row % 16 == 0 && ptrs % 16 == 0) {
    const int w = (int)(row / 16);
    expand8_kernel<uint4><<<row_grid(s->d.n_coarse, w), kThreads, 0, stream>>>(
        static_cast<const uint4*>(coarse), static_cast<uint4*>(fine), s->d.n_coarse, w);
  } else if (row % 16 == 0 && ptrs % 16 == 0) {
    const int w = (int)(row / 16);
    expand_kernel<uint4><<<row_grid(nf, w), kThreads, 0, stream>>>(static_cast<const uint4*>(coarse),
                                                                       static_cast<uint4*>(fine), nf, w, s->d.parent);
  } else if (row % 4 == 0 && ptrs % 4 == 0) {
    const int w = (int)(row / 4);
    expand_kernel<uint32_t><<<row_grid(nf, w), kThreads, 0, stream>>>(static_cast<const uint32_t*>(coarse),
                                                                          static_cast<uint32_t*>(fine), nf, w, s->d.parent);
  } else {
    const int w = (int)(row / 2);
    expand_kernel<uint16_t><<<row_grid(nf, w), kThreads, 0, stream>>>(static_cast<const uint16_t*>(coarse),
                                                                          static_cast<uint16_t*>(fine), nf, w, s->d.parent);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(hip_status(e, "upsample launch"));
  return SUBM_OK;
}

extern "C" int sparse_indice_map_subdivide(submconv_map_t parent_map, sparse_subdivision_t s, hipStream_t stream,
                                           submconv_map_t* out_map) {
  clear_error();
  if (out_map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "out_map is NULL");
  *out_map = nullptr;
  if (parent_map == nullptr || s == nullptr) return fail(SUBM_ERR_INVALID_ARG, "parent_map or handle is NULL");
  if (s->d.kind != SUBM_SUBDIVIDE) return fail(SUBM_ERR_INVALID_ARG, "the handle does not come from sparse_subdivide");
  if (parent_map->d.n != s->d.n_coarse) return fail(SUBM_ERR_SHAPE_MISMATCH, "parent map size differs from the coarse set");
  if (parent_map->d.device != s->d.device) return fail(SUBM_ERR_INVALID_ARG, "map and handle are on different devices");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != s->d.device) return fail(SUBM_ERR_INVALID_ARG, "the handle was built on another device");
  Status cs = map_counts(parent_map);
  if (!cs.ok()) return fail(cs);
  map_note_use(parent_map, stream);
  submconv_map* m = new (std::nothrow) submconv_map;
  if (m == nullptr) return fail(SUBM_ERR_OUT_OF_MEMORY, "host allocation of the map handle failed");
  const int64_t np = s->d.n_coarse;
  const int64_t nc = 8 * np;
  m->d.device = dev;
  m->d.n = nc;
  m->d.mode = kModeSubdivided;
  // Pairs per tap: child o hits tap d exactly when its parent hits tap floor((o + d) / 2).
  int64_t total = 0;
  for (int k = 0; k < 27; ++k) {
    const int d3[3] = {k / 9 - 1, (k / 3) % 3 - 1, k % 3 - 1};
    int64_t c = 0;
    for (int s8 = 0; s8 < 8; ++s8) {
      const int o[3] = {(s8 >> 2) & 1, (s8 >> 1) & 1, s8 & 1};
      int q[3];
      for (int a = 0; a < 3; ++a) q[a] = ((o[a] + d3[a]) >> 1) + 1;
      c += parent_map->d.per_tap[9 * q[0] + 3 * q[1] + q[2]];
    }
    m->d.per_tap[k] = c;
    total += c;
  }
  m->d.pairs = total;
  m->d.counts_ready = true;
  if (np == 0) {
    *out_map = m;
    return SUBM_OK;
  }
  void* nbr = nullptr;
  size_t nbr_bytes = 0;
  Status st = map_memory_take(dev, (size_t)nc * 28 * sizeof(int32_t), stream, &nbr, &nbr_bytes);
  if (!st.ok()) {
    delete m;
    return fail(st);
  }
  m->d.nbr = static_cast<int32_t*>(nbr);
  m->d.nbr_bytes = nbr_bytes;
  m->d.home = stream;
  m->d.masks = reinterpret_cast<uint32_t*>(m->d.nbr + (size_t)nc * 27);
  hipError_t e = launch_child_map(parent_map->d.nbr, np, m->d.nbr, m->d.masks, stream);
  // The kernel writes the map's memory after this call returns; freeing the map waits for it.
  if (e == hipSuccess) e = hipEventCreateWithFlags(&m->d.ready, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(m->d.ready, stream);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(stream);
    if (m->d.ready != nullptr) (void)hipEventDestroy(m->d.ready);
    map_memory_give(dev, nbr, nbr_bytes, stream, true);
    delete m;
    return fail(hip_status(e, "child map launch"));
  }
  *out_map = m;
  return SUBM_OK;
}
