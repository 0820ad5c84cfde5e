// Prefix sum and stable radix sort on the device (gfx950), for the structure builds: the
// downsample's distinct coarse cells in ascending (b, z, y, x) order and the masked upsample's
// child positions.
//
// Prefix sum of int32 (inclusive or exclusive), reduce-then-scan over tiles of 4096 values
// (256 threads x 16 consecutive values, read as four 16-byte words):
//   scan_tile_sums_kernel   one sum per tile
//   scan_sums_kernel        one 1024-thread workgroup turns the tile sums into tile offsets
//   scan_apply_kernel       each tile rescans its values from its offset
//
// Stable LSD radix sort of (key, int32 value) pairs, digits of at most 9 bits, as few passes as
// that allows (25-bit keys: three passes of 9, 8 and 8 bits):
//   radix_count_kernel      per tile, the number of items of each digit (digit-major layout,
//                           counts[d * tiles + tile])
//   (exclusive prefix sum of the counts in that order, the three kernels above) so all items
//                           of digit d precede those of digit d + 1, and within a digit the tiles
//                           keep their order
//   radix_scatter_kernel    each tile ranks its items stably and writes them to their places
// A tile's items are loaded at once (16 per thread) and ranked in 16 rounds of 256 consecutive
// items, one per thread.  Within a
// round a wave finds the lanes holding its own digit with eight ballots (one per digit bit); the
// lowest such lane records the count in LDS, and the four waves' counts are added in wave order,
// so equal digits keep the input order.  The same ballots let the count kernel add once per
// distinct digit and wave instead of once per item (input that is nearly sorted puts most of a
// wave's items on one digit, where per-item LDS atomics would serialise).
#include <utility>

#include "internal.h"

namespace submconv {
namespace {

constexpr int kST = 256;           // threads per tile workgroup
constexpr int kPer = 16;           // values per thread
constexpr int kTile = kST * kPer;  // values per tile
constexpr int kTop = 1024;         // threads of the tile-offset workgroup

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Exclusive prefix sum over the NT threads of a workgroup; *total receives the sum of all.
// s_w holds NT / 64 ints of LDS.  Contains two barriers; every thread must call it.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int x = s_w[i];
    off += i < w ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// The 16 values of this thread (zero past n).  `p` is 16-byte aligned.
__device__ __forceinline__ void load16(const int32_t* p, int64_t base, int64_t n, int (&v)[kPer]) {
  if (base + kPer <= n) {
    const int4* q = reinterpret_cast<const int4*>(p + base);
#pragma unroll
    for (int u = 0; u < kPer / 4; ++u) {
      const int4 x = q[u];
      v[4 * u] = x.x;
      v[4 * u + 1] = x.y;
      v[4 * u + 2] = x.z;
      v[4 * u + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < kPer; ++u) v[u] = base + u < n ? p[base + u] : 0;
  }
}

// Every kernel below returns at once when `gate` is non-null and *gate is zero (work enqueued
// ahead of a condition that only the device knows).
__device__ __forceinline__ bool gated(const uint32_t* gate) { return gate != nullptr && *gate == 0u; }

__global__ __launch_bounds__(kST) void scan_tile_sums_kernel(const int32_t* __restrict__ in, int64_t n,
                                                              int32_t* __restrict__ sums, const uint32_t* gate) {
  __shared__ int s_w[kST / 64];
  if (gated(gate)) return;
  int v[kPer];
  load16(in, (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kPer, n, v);
  int s = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) s += v[u];
  int total;
  (void)block_excl_scan<kST>(s, s_w, &total);
  if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

// In place: sums[t] becomes the sum of sums[0 .. t).
__global__ __launch_bounds__(kTop) void scan_sums_kernel(int32_t* __restrict__ sums, int64_t p, const uint32_t* gate) {
  __shared__ int s_w[kTop / 64];
  if (gated(gate)) return;
  const int64_t per = (p + kTop - 1) / kTop;
  const int64_t b = (int64_t)threadIdx.x * per;
  const int64_t e = b + per < p ? b + per : p;
  int v = 0;
  for (int64_t i = b; i < e; ++i) v += sums[i];
  int total;
  int off = block_excl_scan<kTop>(v, s_w, &total);
  for (int64_t i = b; i < e; ++i) {
    const int x = sums[i];
    sums[i] = off;
    off += x;
  }
}

// out may be in (each thread reads its own values before it writes them).
__global__ __launch_bounds__(kST) void scan_apply_kernel(const int32_t* in, int32_t* out, int64_t n,
                                                          const int32_t* __restrict__ sums, int exclusive,
                                                          const uint32_t* gate) {
  __shared__ int s_w[kST / 64];
  if (gated(gate)) return;
  const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kPer;
  int v[kPer];
  load16(in, base, n, v);
  int s = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) s += v[u];
  int total;
  int run = sums[blockIdx.x] + block_excl_scan<kST>(s, s_w, &total);
  int r[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    r[u] = exclusive ? run : run + v[u];
    run += v[u];
  }
  if (base + kPer <= n) {
    int4* q = reinterpret_cast<int4*>(out + base);
#pragma unroll
    for (int u = 0; u < kPer / 4; ++u) q[u] = make_int4(r[4 * u], r[4 * u + 1], r[4 * u + 2], r[4 * u + 3]);
  } else {
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (base + u < n) out[base + u] = r[u];
  }
}

constexpr int kMaxDigitBits = 9;
constexpr int kMaxBuckets = 1 << kMaxDigitBits;

// Lanes of this wave that are valid and hold digit d (digits of rb <= 9 bits).
__device__ __forceinline__ unsigned long long match_digit(uint32_t d, bool valid, int rb) {
  unsigned long long m = __ballot(valid);
  for (int b = 0; b < rb; ++b) {
    const unsigned long long bb = __ballot((d >> b) & 1u);
    m &= ((d >> b) & 1u) ? bb : ~bb;
  }
  return m;
}

// counts[d * tiles + tile] for the 2^rb digits of key bits [shift, shift + rb).
template <typename K>
__global__ __launch_bounds__(kST) void radix_count_kernel(const K* __restrict__ keys, int64_t n, int shift, int rb,
                                                           int64_t tiles, int32_t* __restrict__ counts,
                                                           const uint32_t* gate) {
  __shared__ int32_t h[kMaxBuckets];
  if (gated(gate)) return;
  const int t = threadIdx.x, lane = t & 63;
  const uint32_t mask = (1u << rb) - 1u;
  h[t] = 0;
  h[t + kST] = 0;
  const int64_t base = (int64_t)blockIdx.x * kTile;
  uint32_t d[kPer];  // all of this thread's keys in flight at once
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int64_t i = base + (int64_t)r * kST + t;
    d[r] = i < n ? (uint32_t)(keys[i] >> shift) & mask : 0u;
  }
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const bool valid = base + (int64_t)r * kST + t < n;
    const unsigned long long peers = match_digit(d[r], valid, rb);
    if (valid && (peers & below) == 0) atomicAdd(&h[d[r]], __popcll(peers));
  }
  __syncthreads();
  for (int dg = t; dg <= (int)mask; dg += kST) counts[(int64_t)dg * tiles + blockIdx.x] = h[dg];
}

// offsets[d * tiles + tile]: first output position of the tile's items of digit d.
template <typename K>
__global__ __launch_bounds__(kST) void radix_scatter_kernel(const K* __restrict__ keys_in,
                                                             const int32_t* __restrict__ vals_in,
                                                             K* __restrict__ keys_out, int32_t* __restrict__ vals_out,
                                                             int64_t n, int shift, int rb, int64_t tiles,
                                                             const int32_t* __restrict__ offsets,
                                                             const uint32_t* gate) {
  __shared__ int32_t s_run[kMaxBuckets];          // next output position of each digit in this tile
  __shared__ int32_t s_wc[kST / 64][kMaxBuckets];  // per-wave digit counts of the current round
  if (gated(gate)) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint32_t mask = (1u << rb) - 1u;
  const int64_t base = (int64_t)blockIdx.x * kTile;
  K key[kPer];  // all of this thread's items in flight at once
  int32_t val[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int64_t i = base + (int64_t)r * kST + t;
    key[r] = i < n ? keys_in[i] : K(0);
    val[r] = i < n ? vals_in[i] : 0;
  }
  // thread t owns digits t and t + 256
#pragma unroll
  for (int j = 0; j < kMaxBuckets / kST; ++j) {
    const int dg = t + j * kST;
    s_run[dg] = dg <= (int)mask ? offsets[(int64_t)dg * tiles + blockIdx.x] : 0;
#pragma unroll
    for (int k = 0; k < kST / 64; ++k) s_wc[k][dg] = 0;
  }
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const bool valid = base + (int64_t)r * kST + t < n;
    const uint32_t d = (uint32_t)(key[r] >> shift) & mask;
    const unsigned long long peers = match_digit(d, valid, rb);
    const int rank = __popcll(peers & below);
    if (valid && rank == 0) s_wc[w][d] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = s_run[d] + rank;
      for (int k = 0; k < w; ++k) pos += s_wc[k][d];
      keys_out[pos] = key[r];
      vals_out[pos] = val[r];
    }
    __syncthreads();
    // advance each owned digit's position past this round's items, clear the counts
#pragma unroll
    for (int j = 0; j < kMaxBuckets / kST; ++j) {
      const int dg = t + j * kST;
      int add = 0;
#pragma unroll
      for (int k = 0; k < kST / 64; ++k) {
        add += s_wc[k][dg];
        s_wc[k][dg] = 0;
      }
      s_run[dg] += add;
    }
    __syncthreads();
  }
}

int64_t tiles_of(int64_t n) { return (n + kTile - 1) / kTile; }
size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

size_t scan_scratch_bytes(int64_t n) { return align256((size_t)tiles_of(n) * sizeof(int32_t)); }

hipError_t launch_scan(const int32_t* in, int32_t* out, int64_t n, bool exclusive, void* scratch, hipStream_t stream,
                       const uint32_t* gate) {
  if (n <= 0) return hipSuccess;
  const int64_t p = tiles_of(n);
  int32_t* sums = static_cast<int32_t*>(scratch);
  scan_tile_sums_kernel<<<(unsigned)p, kST, 0, stream>>>(in, n, sums, gate);
  scan_sums_kernel<<<1, kTop, 0, stream>>>(sums, p, gate);
  const int32_t* csums = sums;
  scan_apply_kernel<<<(unsigned)p, kST, 0, stream>>>(in, out, n, csums, exclusive ? 1 : 0, gate);
  return hipGetLastError();
}

size_t radix_sort_scratch_bytes(int64_t n) {
  const int64_t m = kMaxBuckets * tiles_of(n);
  return align256((size_t)m * sizeof(int32_t)) + scan_scratch_bytes(m);
}

template <typename K>
hipError_t launch_radix_sort_pairs(K* keys, int32_t* vals, K* keys_alt, int32_t* vals_alt, int64_t n, int bits,
                                   void* scratch, hipStream_t stream, bool* result_in_alt, const uint32_t* gate) {
  *result_in_alt = false;
  if (n <= 0 || bits <= 0) return hipSuccess;
  const int64_t tiles = tiles_of(n);
  int32_t* counts = static_cast<int32_t*>(scratch);
  void* scan_tmp = static_cast<unsigned char*>(scratch) + align256((size_t)(kMaxBuckets * tiles) * sizeof(int32_t));
  // as few passes as digits of at most 9 bits allow, the bits spread evenly over them
  const int passes = (bits + kMaxDigitBits - 1) / kMaxDigitBits;
  K* kin = keys;
  int32_t* vin = vals;
  K* kout = keys_alt;
  int32_t* vout = vals_alt;
  for (int p = 0, shift = 0; p < passes; ++p) {
    const int rb = (bits - shift + (passes - p) - 1) / (passes - p);
    const K* ckin = kin;
    radix_count_kernel<K><<<(unsigned)tiles, kST, 0, stream>>>(ckin, n, shift, rb, tiles, counts, gate);
    hipError_t e = launch_scan(counts, counts, (int64_t(1) << rb) * tiles, true, scan_tmp, stream, gate);
    if (e != hipSuccess) return e;
    const int32_t* cvin = vin;
    const int32_t* coff = counts;
    radix_scatter_kernel<K><<<(unsigned)tiles, kST, 0, stream>>>(ckin, cvin, kout, vout, n, shift, rb, tiles, coff, gate);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    std::swap(kin, kout);
    std::swap(vin, vout);
    *result_in_alt = !*result_in_alt;
    shift += rb;
  }
  return hipSuccess;
}

template hipError_t launch_radix_sort_pairs<uint32_t>(uint32_t*, int32_t*, uint32_t*, int32_t*, int64_t, int, void*,
                                                      hipStream_t, bool*, const uint32_t*);
template hipError_t launch_radix_sort_pairs<uint64_t>(uint64_t*, int32_t*, uint64_t*, int32_t*, int64_t, int, void*,
                                                      hipStream_t, bool*, const uint32_t*);

}  // namespace submconv
