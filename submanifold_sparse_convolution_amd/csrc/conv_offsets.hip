// SubMConv3d as a loop over the 27 offsets: gather -> GEMM -> scatter-add per offset.
//
// This is the straightforward loop over the offsets that the pages time their vectorised version against
// (trellis_sparse_mrp_mlx commit log, "Extracted from lato.2_mrp_mlx" commit: 5.9x slower on an
// M3 Ultra), built here as a second MI355X design beside the output-stationary kernel of
// conv.hip, computing the same
//
//   out[i, o] = bias[o] + sum_{k : nbr[i,k] >= 0} sum_c W[o, k, c] * f[nbr[i,k], c].
//
// For every tap k the map's rulebook column k is compacted once into a pair list
// (i, j = nbr[i, k]), i ascending (cached with the map).  One launch per tap then multiplies the
// gathered rows f[j] by W[:, k, :] on the matrix cores and adds the product into a float32
// accumulator row acc[i] (a read-modify-write: within one tap every i occurs once, and the taps
// run one after another, so there are no atomics and the sum order is fixed).  The centre tap
// runs first and writes acc = bias + W_13 f (every voxel is its own centre neighbour); a last
// kernel rounds acc once to the storage dtype.
//
// Per tap the kernel is a plain GEMM tile: 128 pairs x BN output channels, the gathered rows and
// the weight slice staged into LDS by direct-to-LDS loads (XOR-swizzled 16-byte chunks),
// v_mfma_f32_32x32x16 with the weights as operand A, and the fp32 tile staged through LDS so the
// accumulator rows are read and written in whole 16-byte runs.
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "internal.h"

namespace submconv {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------------------------
// Pair lists.  Blocks of 1024 rows (4 per thread, 256 consecutive rows per step): counts per
// (block, tap), an exclusive scan of the counts over blocks per tap, then the emit pass ranks
// every (row, tap) hit by wave ballots so that the pairs of a tap come out in ascending row order.

constexpr int kPairRows = 4 * kThreads;

__global__ __launch_bounds__(kThreads) void pair_count_kernel(const uint32_t* __restrict__ masks, int64_t n,
                                                              int32_t* __restrict__ counts) {
  __shared__ int32_t s_cnt[27];
  const int tid = threadIdx.x;
  if (tid < 27) s_cnt[tid] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * kPairRows;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int64_t row = r0 + it * kThreads + tid;
    const uint32_t m = row < n ? masks[row] : 0u;
    for (int k = 0; k < 27; ++k) {
      const uint64_t bal = __ballot((m >> k) & 1u);
      if ((tid & 63) == 0 && bal != 0) atomicAdd(&s_cnt[k], (int)__popcll(bal));
    }
  }
  __syncthreads();
  if (tid < 27) counts[(int64_t)blockIdx.x * 27 + tid] = s_cnt[tid];
}

// One block per tap: prefix[b * 27 + k] = sum of counts[b' * 27 + k] over b' < b.
__global__ __launch_bounds__(kThreads) void pair_scan_kernel(const int32_t* __restrict__ counts, int64_t nb,
                                                             int32_t* __restrict__ prefix) {
  __shared__ int32_t s[kThreads];
  const int k = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t carry = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += kThreads) {
    const int64_t b = b0 + tid;
    const int32_t v = b < nb ? counts[b * 27 + k] : 0;
    s[tid] = v;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {  // inclusive Hillis-Steele scan
      const int32_t add = tid >= o ? s[tid - o] : 0;
      __syncthreads();
      s[tid] += add;
      __syncthreads();
    }
    if (b < nb) prefix[b * 27 + k] = carry + s[tid] - v;
    carry += s[kThreads - 1];
    __syncthreads();
  }
}

struct TapBase {
  int64_t off[27];  // first pair of tap k in the pair arrays (tap 13 has none)
};

__global__ __launch_bounds__(kThreads) void pair_emit_kernel(const uint32_t* __restrict__ masks,
                                                             const int32_t* __restrict__ nbr, int64_t n,
                                                             const int32_t* __restrict__ prefix, TapBase base,
                                                             int32_t* __restrict__ pair_out, int32_t* __restrict__ pair_in) {
  __shared__ int32_t s_cnt[16 * 27];  // (step, wave) x tap hit counts, then their exclusive prefix
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * kPairRows;
  uint32_t m[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int64_t row = r0 + it * kThreads + tid;
    m[it] = row < n ? masks[row] : 0u;
    for (int k = 0; k < 27; ++k) {
      const uint64_t bal = __ballot((m[it] >> k) & 1u);
      if (lane == 0) s_cnt[(it * 4 + wave) * 27 + k] = (int32_t)__popcll(bal);
    }
  }
  __syncthreads();
  if (tid < 27) {
    int32_t run = 0;
    for (int q = 0; q < 16; ++q) {
      const int32_t c = s_cnt[q * 27 + tid];
      s_cnt[q * 27 + tid] = run;
      run += c;
    }
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int64_t row = r0 + it * kThreads + tid;
    for (int k = 0; k < 27; ++k) {
      const bool hit = (m[it] >> k) & 1u;
      const uint64_t bal = __ballot(hit);
      if (hit && k != 13) {
        const int64_t pos = base.off[k] + prefix[(int64_t)blockIdx.x * 27 + k] + s_cnt[(it * 4 + wave) * 27 + k] +
                            (int64_t)__popcll(bal & below);
        pair_out[pos] = (int32_t)row;
        pair_in[pos] = nbr[row * 27 + k];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Per-tap GEMM tile.

struct OffsetArgs {
  const void* feats;
  const void* weight;
  const void* bias;       // may be null
  float* acc;             // [n, cout] float32
  const int32_t* pair_out;  // null: identity (the centre tap)
  const int32_t* pair_in;
  int64_t count;          // pairs of this tap
  int tap;
  int cin;
  int cout;
  int row_bytes;
  uint32_t feats_bytes;
  uint32_t weight_bytes;
};

constexpr int kBM = 128;  // pairs per tile

template <int SLB, int BN>
struct OffsetShape {
  static constexpr int CH = SLB / 16;       // 16-byte chunks per row slice
  static constexpr int RPI = 64 / CH;       // rows per direct load (1 KB)
  static constexpr int WTM = BN / 2;        // output channels per wave (2 x 2 waves)
  static constexpr int WTN = kBM / 2;       // pairs per wave
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int KSTEPS = SLB / 32;   // 16-channel matrix-core steps per slice
  static constexpr int A_BYTES = BN * SLB, B_BYTES = kBM * SLB;
  static constexpr int SROW = BN * 4 + 16;  // epilogue staging row stride (bytes)
  static constexpr int LDS = (A_BYTES + B_BYTES) > kBM * SROW ? (A_BYTES + B_BYTES) : kBM * SROW;
  static constexpr int ALOADS = BN / RPI / 4, BLOADS = kBM / RPI / 4;  // direct loads per wave
  static_assert(BN % (4 * RPI) == 0 && kBM % (4 * RPI) == 0, "whole loads per wave");
};

// Swizzled position of logical chunk c of LDS row r (16-byte units).
template <int CH>
__device__ __forceinline__ int swz(int r, int c) {
  return c ^ ((r / (16 / CH)) % CH);
}

template <DT D, int SLB, int BN, bool FIRST>
__global__ __launch_bounds__(kThreads, 2) void offset_gemm_kernel(const OffsetArgs a) {
  using Sh = OffsetShape<SLB, BN>;
  constexpr int CH = Sh::CH, RPI = Sh::RPI, FM = Sh::FM, FN = Sh::FN, WTM = Sh::WTM, WTN = Sh::WTN;
  __shared__ __align__(16) unsigned char lds[Sh::LDS];
  unsigned char* sA = lds;                 // weights: BN rows
  unsigned char* sB = lds + Sh::A_BYTES;   // gathered feature rows: kBM rows

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: LDS load bases go to M0
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t p0 = (int64_t)blockIdx.x * kBM;
  const int o0 = blockIdx.y * BN;
  const int cout = a.cout, rb = a.row_bytes;
  const i32x4_t rsrc_f = make_rsrc(a.feats, a.feats_bytes);
  const i32x4_t rsrc_w = make_rsrc(a.weight, a.weight_bytes);

  // Per-lane load descriptors: the row each of this wave's loads covers and the logical chunk
  // this lane fetches; byte offsets of the rows (kOutOfRange for absent rows).
  uint32_t a_row_off[Sh::ALOADS], b_row_off[Sh::BLOADS];
  int a_chunk[Sh::ALOADS], b_chunk[Sh::BLOADS];
#pragma unroll
  for (int q = 0; q < Sh::ALOADS; ++q) {
    const int r = (wave * Sh::ALOADS + q) * RPI + lane / CH;
    a_chunk[q] = swz<CH>(r, lane % CH);
    const int o = o0 + r;
    a_row_off[q] = o < cout ? (uint32_t)(((int64_t)o * 27 + a.tap) * rb) : kOutOfRange;
  }
#pragma unroll
  for (int q = 0; q < Sh::BLOADS; ++q) {
    const int r = (wave * Sh::BLOADS + q) * RPI + lane / CH;
    b_chunk[q] = swz<CH>(r, lane % CH);
    const int64_t p = p0 + r;
    int64_t j = -1;
    if (p < a.count) j = a.pair_in != nullptr ? a.pair_in[p] : p;
    b_row_off[q] = j >= 0 ? (uint32_t)(j * rb) : kOutOfRange;
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  const int slices = (rb + SLB - 1) / SLB;
  for (int sl = 0; sl < slices; ++sl) {
    const int sbyte = sl * SLB;
#pragma unroll
    for (int q = 0; q < Sh::ALOADS; ++q) {
      const int cb = sbyte + a_chunk[q] * 16;
      const uint32_t off = (a_row_off[q] == kOutOfRange || cb >= rb) ? kOutOfRange : a_row_off[q] + cb;
      lds_dma16(rsrc_w, off, lds_offset(sA + (wave_u * Sh::ALOADS + q) * 1024));
    }
#pragma unroll
    for (int q = 0; q < Sh::BLOADS; ++q) {
      const int cb = sbyte + b_chunk[q] * 16;
      const uint32_t off = (b_row_off[q] == kOutOfRange || cb >= rb) ? kOutOfRange : b_row_off[q] + cb;
      lds_dma16(rsrc_f, off, lds_offset(sB + (wave_u * Sh::BLOADS + q) * 1024));
    }
    wait_vmcnt<0>();
    barrier_no_fence();
#pragma unroll
    for (int ks = 0; ks < Sh::KSTEPS; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      uint4 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 32 + (lane & 31);
        fa[i] = *reinterpret_cast<const uint4*>(sA + r * SLB + swz<CH>(r, c) * 16);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WTN + j * 32 + (lane & 31);
        fb[j] = *reinterpret_cast<const uint4*>(sB + r * SLB + swz<CH>(r, c) * 16);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<D>(fa[i], fb[j], acc[i][j]);
    }
    __syncthreads();  // every wave is done with this slice before the next overwrites it
  }

  // Stage the fp32 tile: lane l holds pair column l % 32 of each 32-block and, in registers
  // 4g .. 4g + 3, output channels 8g + 4 (l / 32) .. + 3 of each 32-row block of weights.
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int pr = wn * WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int oc = wm * WTM + i * 32 + 8 * g + 4 * (lane >> 5);
        *reinterpret_cast<float4*>(lds + pr * Sh::SROW + oc * 4) =
            make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
      }
    }
  __syncthreads();
  using T = typename Elem<D>::T;
  constexpr int C4 = BN / 4;  // float4 chunks per staged row
  for (int idx = tid; idx < kBM * C4; idx += kThreads) {
    const int r = idx / C4, c = idx - r * C4;
    const int64_t p = p0 + r;
    const int o = o0 + 4 * c;
    if (p >= a.count || o >= cout) continue;
    const int64_t i = a.pair_out != nullptr ? a.pair_out[p] : p;
    float4 v = *reinterpret_cast<const float4*>(lds + r * Sh::SROW + c * 16);
    float4* dst = reinterpret_cast<float4*>(a.acc + i * cout + o);
    if constexpr (FIRST) {
      if (a.bias != nullptr) {
        const T* b = reinterpret_cast<const T*>(a.bias) + o;
        v.x += to_float<D>(b[0]);
        v.y += to_float<D>(b[1]);
        v.z += to_float<D>(b[2]);
        v.w += to_float<D>(b[3]);
      }
    } else {
      const float4 old = *dst;
      v.x += old.x;
      v.y += old.y;
      v.z += old.z;
      v.w += old.w;
    }
    *dst = v;
  }
}

// out = acc rounded once to the storage dtype (4 values per thread).
template <DT D>
__global__ __launch_bounds__(kThreads) void round_out_kernel(const float4* __restrict__ acc, uint2* __restrict__ out,
                                                             int64_t quads) {
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < quads; t += (int64_t)gridDim.x * kThreads) {
    const float4 v = acc[t];
    out[t] = pack4<D>(v.x, v.y, v.z, v.w);
  }
}

template <DT D, int SLB, int BN>
hipError_t launch_taps(const MapData& m, const OffsetArgs& base, hipStream_t stream) {
  const dim3 block(kThreads);
  const unsigned gy = (unsigned)((base.cout + BN - 1) / BN);
  OffsetArgs a = base;
  a.tap = 13;
  a.pair_out = nullptr;
  a.pair_in = nullptr;
  a.count = m.n;
  offset_gemm_kernel<D, SLB, BN, true><<<dim3((unsigned)((a.count + kBM - 1) / kBM), gy), block, 0, stream>>>(a);
  for (int k = 0; k < 27; ++k) {
    if (k == 13 || m.per_tap[k] == 0) continue;
    a.tap = k;
    a.count = m.per_tap[k];
    a.pair_out = m.pair_out + m.pair_off[k];
    a.pair_in = m.pair_in + m.pair_off[k];
    offset_gemm_kernel<D, SLB, BN, false><<<dim3((unsigned)((a.count + kBM - 1) / kBM), gy), block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <DT D>
hipError_t launch_dtype(const MapData& m, const OffsetArgs& a, void* out, hipStream_t stream) {
  hipError_t e;
  const bool wide = a.row_bytes > 128;
  if (a.cout > 64)
    e = wide ? launch_taps<D, 256, 128>(m, a, stream) : launch_taps<D, 128, 128>(m, a, stream);
  else
    e = wide ? launch_taps<D, 256, 64>(m, a, stream) : launch_taps<D, 128, 64>(m, a, stream);
  if (e != hipSuccess) return e;
  const int64_t quads = m.n * a.cout / 4;
  const int64_t blocks = (quads + kThreads - 1) / kThreads;
  round_out_kernel<D><<<(unsigned)(blocks < 4096 ? blocks : 4096), kThreads, 0, stream>>>(
      reinterpret_cast<const float4*>(a.acc), static_cast<uint2*>(out), quads);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pair_lists(const MapData& m, int32_t* pair_out, int32_t* pair_in, int32_t* scratch,
                             hipStream_t stream) {
  const int64_t nb = (m.n + kPairRows - 1) / kPairRows;
  int32_t* counts = scratch;
  int32_t* prefix = scratch + nb * 27;
  TapBase base{};
  int64_t run = 0;
  for (int k = 0; k < 27; ++k) {
    base.off[k] = run;
    if (k != 13) run += m.per_tap[k];
  }
  pair_count_kernel<<<(unsigned)nb, kThreads, 0, stream>>>(m.masks, m.n, counts);
  pair_scan_kernel<<<27, kThreads, 0, stream>>>(counts, nb, prefix);
  pair_emit_kernel<<<(unsigned)nb, kThreads, 0, stream>>>(m.masks, m.nbr, m.n, prefix, base, pair_out, pair_in);
  return hipGetLastError();
}

size_t pair_scratch_ints(int64_t n) { return (size_t)((n + kPairRows - 1) / kPairRows) * 27 * 2; }

hipError_t launch_subm_conv_per_offset(const MapData& m, int cin, int cout, int dtype, const void* feats,
                                       const void* weight, const void* bias, void* out, float* acc,
                                       hipStream_t stream) {
  OffsetArgs a{};
  a.feats = feats;
  a.weight = weight;
  a.bias = bias;
  a.acc = acc;
  a.cin = cin;
  a.cout = cout;
  a.row_bytes = cin * 2;
  a.feats_bytes = (uint32_t)(m.n * a.row_bytes);
  a.weight_bytes = (uint32_t)((int64_t)cout * 27 * a.row_bytes);
  return dtype == SUBM_F16 ? launch_dtype<DT::F16>(m, a, out, stream) : launch_dtype<DT::BF16>(m, a, out, stream);
}

}  // namespace submconv
