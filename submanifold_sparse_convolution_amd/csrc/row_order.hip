// Row order of a sparse map for the persistent 27-tap convolution (conv.hip), gfx950.
//
// The convolution computes a row block's tap for all of the block's rows as soon as one of them
// has that neighbour (an absent neighbour adds exact zeros).  On sets where rows have few
// neighbours each (the subdivided boxes: ~6.7 of 27 taps), every block of consecutive rows still
// reaches all 27 taps.  With rows of similar neighbour masks placed together, blocks reach fewer
// taps and the tile walk computes fewer stages; the outputs are the same bits.
//
// Built once per map, on the device:
//   order_gate_kernel     from the build's per-tap pair counts: on when a row has at most
//                         kOrderMaxTaps neighbours on average (one workgroup, writes the gate)
//   order_key_kernel      key = (row >> 16, the 12 highest bits of the mask without its
//                         always-set centre bit): the order stays within segments of 65,536 rows
//                         (256 tiles), so a tile's neighbours stay near each other in memory, and
//                         the key fits two 9-bit radix passes on sets of up to 4 M rows
//   (stable radix sort of (key, row), sort_scan.hip)
//   order_permute_kernel  rows[j], the rulebook row and the mask of rows[j] at position j
// Every kernel after the gate returns at once when the gate is off.  The block:
// [gate (256 B) | rows[n] | nbr[n][27] | masks[n]], 16-byte aligned parts.
#include "internal.h"

namespace submconv {
namespace {

constexpr int kOT = 256;
constexpr int64_t kOrderMaxTaps = 9;  // mean neighbours per row (of 27) at or below which the order is built
constexpr int kSegmentShift = 16;     // rows per segment: 65,536
constexpr int kMaskBits = 12;         // mask bits in the key
constexpr int kPermRows = 64;         // rows per workgroup of the permuted copy

__global__ __launch_bounds__(kOT) void order_gate_kernel(const uint32_t* __restrict__ banks, int64_t n,
                                                         uint32_t* __restrict__ gate) {
  __shared__ unsigned long long s_sum;
  if (threadIdx.x == 0) s_sum = 0ull;
  __syncthreads();
  unsigned long long v = 0ull;
  for (int k = threadIdx.x; k < kTapBanks * 27; k += kOT) v += banks[k];
  atomicAdd(&s_sum, v);
  __syncthreads();
  if (threadIdx.x == 0) *gate = s_sum <= (unsigned long long)(kOrderMaxTaps * n) ? 1u : 0u;
}

// Mask bits 0..12 and 14..26 as 26 bits (bit 13, the row itself, is set on every row), of which
// the highest kMaskBits.
__device__ __forceinline__ uint32_t mask_key(uint32_t m) {
  return (((m & 0x1FFFu) | ((m >> 14) << 13)) >> (26 - kMaskBits));
}

__global__ __launch_bounds__(kOT) void order_key_kernel(const uint32_t* __restrict__ masks, int64_t n,
                                                        const uint32_t* __restrict__ gate, uint32_t* __restrict__ keys,
                                                        int32_t* __restrict__ vals) {
  if (*gate == 0u) return;
  const int64_t i = (int64_t)blockIdx.x * kOT + threadIdx.x;
  if (i >= n) return;
  keys[i] = ((uint32_t)(i >> kSegmentShift) << kMaskBits) | mask_key(masks[i]);
  vals[i] = (int32_t)i;
}

// kPermRows positions per workgroup: their source rows into LDS, then the 27 ints of each row
// copied with consecutive threads on consecutive ints (reads of whole 108-byte rows, coalesced
// writes), seven loads in flight per thread.
__global__ __launch_bounds__(kOT) void order_permute_kernel(const int32_t* __restrict__ nbr,
                                                            const uint32_t* __restrict__ masks,
                                                            const int32_t* __restrict__ sorted, int64_t n,
                                                            const uint32_t* __restrict__ gate,
                                                            int32_t* __restrict__ rows, int32_t* __restrict__ onbr,
                                                            uint32_t* __restrict__ omasks) {
  __shared__ int32_t s_r[kPermRows];
  if (*gate == 0u) return;
  const int t = threadIdx.x;
  const int64_t j0 = (int64_t)blockIdx.x * kPermRows;
  const int cnt = (int)(n - j0 < kPermRows ? n - j0 : kPermRows);
  if (t < cnt) {
    const int32_t r = sorted[j0 + t];
    s_r[t] = r;
    rows[j0 + t] = r;
    omasks[j0 + t] = masks[r];
  }
  __syncthreads();
  constexpr int kIter = (kPermRows * 27 + kOT - 1) / kOT;
  const int total = cnt * 27;
  int32_t v[kIter];
#pragma unroll
  for (int u = 0; u < kIter; ++u) {
    const int i = t + u * kOT;
    const int jj = i < total ? i / 27 : 0;
    v[u] = i < total ? nbr[(int64_t)s_r[jj] * 27 + (i - jj * 27)] : 0;
  }
  int32_t* dst = onbr + j0 * 27;
#pragma unroll
  for (int u = 0; u < kIter; ++u)
    if (t + u * kOT < total) dst[t + u * kOT] = v[u];
}

size_t a16(size_t b) { return (b + 15) / 16 * 16; }

}  // namespace

OrderView order_view(void* block, int64_t n) {
  OrderView v;
  unsigned char* p = static_cast<unsigned char*>(block);
  v.gate = reinterpret_cast<uint32_t*>(p);
  size_t off = 256;
  v.rows = reinterpret_cast<int32_t*>(p + off);
  off += a16((size_t)n * 4);
  v.nbr = reinterpret_cast<int32_t*>(p + off);
  off += a16((size_t)n * 27 * 4);
  v.masks = reinterpret_cast<uint32_t*>(p + off);
  return v;
}

size_t order_block_bytes(int64_t n) { return 256 + a16((size_t)n * 4) + a16((size_t)n * 27 * 4) + a16((size_t)n * 4); }

size_t order_scratch_bytes(int64_t n) { return 4 * a16((size_t)n * 4) + radix_sort_scratch_bytes(n); }

hipError_t launch_row_order(const MapData* d, void* block, void* scratch, hipStream_t stream) {
  const int64_t n = d->n;
  if (n <= 0) return hipSuccess;
  const OrderView v = order_view(block, n);
  order_gate_kernel<<<1, kOT, 0, stream>>>(d->dev_banks, n, v.gate);
  int seg_bits = 0;  // n < 2^31: at most 15, so the key stays within 27 bits
  while ((int64_t(1) << seg_bits) < ((n + (int64_t(1) << kSegmentShift) - 1) >> kSegmentShift)) ++seg_bits;
  unsigned char* s = static_cast<unsigned char*>(scratch);
  uint32_t* k0 = reinterpret_cast<uint32_t*>(s);
  uint32_t* k1 = reinterpret_cast<uint32_t*>(s + a16((size_t)n * 4));
  int32_t* v0 = reinterpret_cast<int32_t*>(s + 2 * a16((size_t)n * 4));
  int32_t* v1 = reinterpret_cast<int32_t*>(s + 3 * a16((size_t)n * 4));
  order_key_kernel<<<(unsigned)((n + kOT - 1) / kOT), kOT, 0, stream>>>(d->masks, n, v.gate, k0, v0);
  bool alt = false;
  hipError_t e = launch_radix_sort_pairs<uint32_t>(k0, v0, k1, v1, n, kMaskBits + seg_bits, s + 4 * a16((size_t)n * 4),
                                                   stream, &alt, v.gate);
  if (e != hipSuccess) return e;
  const int32_t* sorted = alt ? v1 : v0;
  order_permute_kernel<<<(unsigned)((n + kPermRows - 1) / kPermRows), kOT, 0, stream>>>(d->nbr, d->masks, sorted, n,
                                                                                        v.gate, v.rows, v.nbr, v.masks);
  return hipGetLastError();
}

}  // namespace submconv
