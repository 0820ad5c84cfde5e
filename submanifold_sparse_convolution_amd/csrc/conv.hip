// Submanifold 3x3x3 (and 1x1x1) convolution forward on gfx950 (CDNA4).
//
//   out[i, o] = bias[o] + sum_{k : nbr[i,k] >= 0} sum_c W[o, k, c] * f[nbr[i,k], c]
//
// with W the KRSC weight [Cout, kz, ky, kx, Cin] viewed as [Cout, 27, Cin] and f gathered at
// coord_i + d (cross-correlation): lato.2_mrp_mlx README, header summary and "Correctness".
//
// Design: output-stationary implicit GEMM.  A 256-thread workgroup owns a tile of BM output
// rows x BN output channels and keeps its fp32 accumulators in registers for the whole
// reduction, so there are no atomics and no scatter: every output element is written once.
// The reduction runs over "stages" (tap k, 256-byte slice q of the input row):
//   A stage = BM gathered feature rows  f[nbr[row, k], q*256/s ...]   (zero where nbr = -1)
//   B stage = BN weight rows            W[o, k, q*256/s ...]
// Both operands are K-contiguous (a feature row and a KRSC weight row are both contiguous in
// Cin), so both are staged the same way: 16-byte chunks, global -> registers -> LDS, with the
// chunk index XOR-swizzled by the row (mod 16) so that the MFMA fragment reads
// (16 rows x 16 bytes per quarter-wave) hit distinct LDS banks.  The next stage's global loads
// are issued before the current stage's MFMAs, so HBM/L2 latency hides behind the matrix cores.
// Taps that no row of the tile uses are skipped (27-bit mask built from the tile's nbr rows).
//
// Matrix-core instructions (one 16x16 output block per instruction):
//   bf16 / fp16 : v_mfma_f32_16x16x32_{bf16,f16}; a lane supplies 8 consecutive K values
//   fp32        : 4 x v_mfma_f32_16x16x4_f32 over the same 16-byte fragments; instruction e
//                 takes element e of every lane, which only permutes the order of K
// Output block layout (both): lane l holds column l % 16, rows 4 * (l / 16) + {0..3}.
//
// Block -> tile mapping is XCD-aware: workgroups are dealt to the 8 XCDs round-robin, so
// block b goes to tile (b % 8) * per_xcd + b / 8 and each XCD walks one contiguous range of
// rows, whose neighbourhoods then stay in that XCD's L2.
#include <cstdlib>
#include <type_traits>

#include "internal.h"

namespace submconv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

enum class DT { F32, F16, BF16 };

template <DT D> struct Elem;
template <> struct Elem<DT::F32> { using T = float; static constexpr int kSize = 4; };
template <> struct Elem<DT::F16> { using T = uint16_t; static constexpr int kSize = 2; };
template <> struct Elem<DT::BF16> { using T = uint16_t; static constexpr int kSize = 2; };

template <DT D> __device__ __forceinline__ float to_float(typename Elem<D>::T v);
template <> __device__ __forceinline__ float to_float<DT::F32>(float v) { return v; }
template <> __device__ __forceinline__ float to_float<DT::F16>(uint16_t v) {
  return (float)__builtin_bit_cast(_Float16, v);
}
template <> __device__ __forceinline__ float to_float<DT::BF16>(uint16_t v) {
  return __uint_as_float((uint32_t)v << 16);
}

// float -> storage, round to nearest even, no flush to zero.
template <DT D> __device__ __forceinline__ typename Elem<D>::T from_float(float v);
template <> __device__ __forceinline__ float from_float<DT::F32>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_float<DT::F16>(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <> __device__ __forceinline__ uint16_t from_float<DT::BF16>(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// acc += A_frag * B_frag over one 64-byte K slice of 16 rows x 16 columns.
template <DT D> __device__ __forceinline__ f32x4_t mfma_step(const uint4& a, const uint4& b, f32x4_t c);
template <> __device__ __forceinline__ f32x4_t mfma_step<DT::BF16>(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4_t mfma_step<DT::F16>(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4_t mfma_step<DT::F32>(const uint4& a, const uint4& b, f32x4_t c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

struct ConvArgs {
  const void* feats;
  const void* weight;
  const void* bias;     // may be null
  void* out;
  const int32_t* nbr;   // [n, 27]; null when taps == 1
  int64_t n;
  int cin;
  int cout;
  int row_bytes;        // cin * element size
  int tiles_m;
  int per_xcd;
  int vec_out;          // 16-byte output stores allowed
  uint32_t feats_bytes;  // n * row_bytes (fast path: < 2^31)
  uint32_t weight_bytes; // cout * taps * row_bytes (fast path: < 2^31)
};

constexpr int kThreads = 256;
constexpr int kStageBytes = 256;  // bytes of one row per stage (16 chunks of 16 B)

template <DT D, int BM, int BN, int WM, bool VEC, int TAPS>
__global__ __launch_bounds__(kThreads, 2) void subm_conv_generic_kernel(const ConvArgs args) {
  using T = typename Elem<D>::T;
  constexpr int S = Elem<D>::kSize;
  constexpr int WN = 4 / WM;
  constexpr int WTM = BM / WM;
  constexpr int WTN = BN / WN;
  constexpr int FM = WTM / 16;
  constexpr int FN = WTN / 16;
  constexpr int APT = BM * 16 / kThreads;  // A chunks per thread
  constexpr int BPT = BN * 16 / kThreads;  // B chunks per thread
  static_assert(FM >= 1 && FN >= 1 && APT >= 1 && BPT >= 1, "tile too small");
  static_assert(BM * BN * S <= (BM + BN) * kStageBytes, "epilogue staging must fit");

  __shared__ __align__(16) unsigned char smem[(BM + BN) * kStageBytes];
  __shared__ int32_t s_nbr[TAPS == 27 ? BM * 27 : 1];
  __shared__ uint32_t s_mask;
  unsigned char* sA = smem;
  unsigned char* sB = smem + BM * kStageBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM;
  const int wn = wave / WM;

  const int bid = blockIdx.x;
  const int tile = (bid & 7) * args.per_xcd + (bid >> 3);
  if (tile >= args.tiles_m) return;
  const int64_t n = args.n;
  const int64_t row0 = (int64_t)tile * BM;
  const int o0 = blockIdx.y * BN;
  const int cin = args.cin, cout = args.cout, row_bytes = args.row_bytes;
  const unsigned char* feats = static_cast<const unsigned char*>(args.feats);
  const unsigned char* weight = static_cast<const unsigned char*>(args.weight);

  // ---- tile rulebook rows and the mask of taps present anywhere in the tile
  if (tid == 0) s_mask = 0;
  __syncthreads();
  uint32_t local_mask = 0;
  if constexpr (TAPS == 27) {
    const int32_t* nb = args.nbr + row0 * 27;
    const int valid = (int)((n - row0) < BM ? (n - row0) : BM);
    for (int idx = tid; idx < BM * 27; idx += kThreads) {
      const int r = idx / 27;
      const int v = r < valid ? nb[idx] : -1;
      s_nbr[idx] = v;
      if (v >= 0) local_mask |= 1u << (idx - r * 27);
    }
  } else {
    local_mask = 1u;
  }
  for (int off = 32; off > 0; off >>= 1) local_mask |= __shfl_xor(local_mask, off, 64);
  if (lane == 0 && local_mask) atomicOr(&s_mask, local_mask);
  __syncthreads();
  const uint32_t mask = s_mask;
  const int nq = (row_bytes + kStageBytes - 1) / kStageBytes;

  // Each thread always handles chunk column c = tid % 16 (16-byte offset inside the stage row)
  // of rows tid / 16 + 16 * u.
  const int ch = tid & 15;
  const int rsub = tid >> 4;

  uint4 ra[APT];
  uint4 rb[BPT];

  auto load_stage = [&](int k, int q) {
    const int cb = q * kStageBytes + ch * 16;  // byte offset in the input row
#pragma unroll
    for (int u = 0; u < APT; ++u) {
      const int r = rsub + 16 * u;
      int64_t j;
      if constexpr (TAPS == 27) {
        j = s_nbr[r * 27 + k];
      } else {
        j = (row0 + r < n) ? row0 + r : -1;
      }
      uint4 v = make_uint4(0, 0, 0, 0);
      if constexpr (VEC) {
        if (j >= 0 && cb < row_bytes) v = *reinterpret_cast<const uint4*>(feats + j * row_bytes + cb);
      } else {
        T e[16 / S];
        const T* src = reinterpret_cast<const T*>(feats) + j * cin;
#pragma unroll
        for (int t = 0; t < 16 / S; ++t) {
          const int col = cb / S + t;
          e[t] = (j >= 0 && col < cin) ? src[col] : T(0);
        }
        v = __builtin_bit_cast(uint4, e);
      }
      ra[u] = v;
    }
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int o = o0 + rsub + 16 * u;
      uint4 v = make_uint4(0, 0, 0, 0);
      const int64_t wrow = (int64_t)o * TAPS + k;
      if constexpr (VEC) {
        if (o < cout && cb < row_bytes) v = *reinterpret_cast<const uint4*>(weight + wrow * row_bytes + cb);
      } else {
        T e[16 / S];
        const T* src = reinterpret_cast<const T*>(weight) + wrow * cin;
#pragma unroll
        for (int t = 0; t < 16 / S; ++t) {
          const int col = cb / S + t;
          e[t] = (o < cout && col < cin) ? src[col] : T(0);
        }
        v = __builtin_bit_cast(uint4, e);
      }
      rb[u] = v;
    }
  };

  auto store_stage = [&]() {
#pragma unroll
    for (int u = 0; u < APT; ++u) {
      const int r = rsub + 16 * u;
      *reinterpret_cast<uint4*>(sA + r * kStageBytes + ((ch ^ (r & 15)) << 4)) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int r = rsub + 16 * u;
      *reinterpret_cast<uint4*>(sB + r * kStageBytes + ((ch ^ (r & 15)) << 4)) = rb[u];
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int lrow = lane & 15;   // fragment row (A) / column (B) within a 16-block
  const int lk = lane >> 4;     // which 16-byte chunk of the 64-byte K slice

  auto compute_stage = [&](int q) {
    const int rem_bytes = row_bytes - q * kStageBytes;
    const int ksteps = rem_bytes >= kStageBytes ? kStageBytes / 64 : (rem_bytes + 63) / 64;
    for (int kk = 0; kk < ksteps; ++kk) {
      const int c = kk * 4 + lk;
      const int sw = (c ^ lrow) << 4;
      uint4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const uint4*>(sA + (wm * WTM + i * 16 + lrow) * kStageBytes + sw);
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = *reinterpret_cast<const uint4*>(sB + (wn * WTN + j * 16 + lrow) * kStageBytes + sw);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_step<D>(af[i], bf[j], acc[i][j]);
    }
  };

  // ---- stage pipeline: registers hold stage s+1 while the matrix cores run stage s
  uint32_t rem = mask;
  bool have = rem != 0;
  int kc = 0, qc = 0;
  if (have) {
    kc = __builtin_ctz(rem);
    rem &= rem - 1;
    load_stage(kc, 0);
  }
  while (have) {
    __syncthreads();
    store_stage();
    __syncthreads();
    int kn = kc, qn = qc + 1;
    bool more = true;
    if (qn >= nq) {
      if (rem) {
        kn = __builtin_ctz(rem);
        rem &= rem - 1;
        qn = 0;
      } else {
        more = false;
      }
    }
    if (more) load_stage(kn, qn);
    compute_stage(qc);
    kc = kn;
    qc = qn;
    have = more;
  }

  // ---- epilogue: + bias (fp32), one RNE rounding, staged through LDS for coalesced stores
  float bcol[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int o = o0 + wn * WTN + j * 16 + lrow;
    bcol[j] = (args.bias != nullptr && o < cout) ? to_float<D>(reinterpret_cast<const T*>(args.bias)[o]) : 0.f;
  }
  __syncthreads();
  T* sC = reinterpret_cast<T*>(smem);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = wm * WTM + i * 16 + lk * 4 + e;
        const int col = wn * WTN + j * 16 + lrow;
        sC[r * BN + col] = from_float<D>(acc[i][j][e] + bcol[j]);
      }
  __syncthreads();
  T* out = reinterpret_cast<T*>(args.out);
  if (args.vec_out) {
    constexpr int CPR = BN * S / 16;  // 16-byte chunks per tile row
    for (int idx = tid; idx < BM * CPR; idx += kThreads) {
      const int r = idx / CPR, c = idx - r * CPR;
      const int64_t row = row0 + r;
      const int col = o0 + c * (16 / S);
      if (row < n && col < cout)
        *reinterpret_cast<uint4*>(out + row * cout + col) = *reinterpret_cast<const uint4*>(sC + r * BN + c * (16 / S));
    }
  } else {
    for (int idx = tid; idx < BM * BN; idx += kThreads) {
      const int r = idx / BN, c = idx - r * BN;
      const int64_t row = row0 + r;
      if (row < n && o0 + c < cout) out[row * cout + o0 + c] = sC[r * BN + c];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Fast path for 16-bit storage: 32x32x16 matrix-core tiles fed by direct global->LDS loads.
//
// Same output-stationary decomposition as the generic kernel, with:
//   * v_mfma_f32_32x32x16_{bf16,f16}: a 32 x 32 fp32 block per instruction (lane l holds column
//     l % 32, rows 8 * (v / 4) + 4 * (l / 32) + v % 4 for accumulator register v);
//   * stages of 64 input channels (128-byte row slices) loaded with global_load_lds_dwordx4:
//     each instruction moves 64 x 16 bytes straight into LDS (8 rows x 8 chunks), so no
//     registers hold data in flight and NS - 1 stages can be outstanding while one is consumed;
//     the gather's XOR swizzle (chunk ^ row mod 8) is applied on the global side by choosing
//     which chunk each lane fetches; an absent neighbour or a padding chunk fetches 16 zero
//     bytes from a device-side zero vector;
//   * every stage issues the same number of load instructions (trailing stages load zeros), so
//     a constant s_waitcnt vmcnt((NS - 2) * per-stage count) waits exactly for the oldest stage;
//     the workgroup barrier is a bare s_barrier (no memory fence, which on this architecture
//     would wait for every outstanding load and serialise the ring);
//   * tile height BM chosen at launch so that the number of tiles fills the 256 compute units
//     in whole rounds as closely as possible.
template <DT D> __device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c);
template <> __device__ __forceinline__ f32x16_t mfma32<DT::BF16>(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16_t mfma32<DT::F16>(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

constexpr int kRowSlice = 128;  // bytes of one row per stage (64 16-bit channels, 8 chunks of 16 B)

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Raw buffer resource (gfx9 layout): 48-bit base, stride 0, num_records = size in bytes; word 3
// selects 32-bit data format.  A load whose offset is >= num_records returns zeros, which is how
// absent neighbours and padding chunks are filled.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kOutOfRange = 0x80000000u;  // any offset at or above this reads zeros

__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// One direct buffer->LDS load: 64 lanes x 16 bytes from per-lane byte offsets into 1 KB of LDS
// at lds_addr + 16 * lane.  Issued from inline assembly so that the compiler does not track
// it: it would otherwise put a wait for every outstanding load before the LDS reads of the slot
// being consumed (it cannot tell the ring slots apart after a loop back-edge).  The kernel waits
// for these loads itself (s_waitcnt vmcnt before each barrier); they have no destination
// register.
__device__ __forceinline__ void lds_dma16(const i32x4_t& rsrc, uint32_t voffset, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voffset), "s"(rsrc), "s"(lds_addr));
}

// Workgroup barrier without a memory fence (a fence would wait for every outstanding load).
// The "memory" clobber keeps the compiler from moving LDS accesses across it; the waits that
// make LDS data valid are explicit s_waitcnt instructions placed before it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

template <int BM, int BN, int TAPS>
struct DmaShape {
  static constexpr int WM = BN >= 64 ? 2 : 4;    // waves along rows (compute)
  static constexpr int WN = 4 / WM;              // waves along output channels (compute)
  static constexpr int WTM = BM / WM;
  static constexpr int WTN = BN / WN;
  static constexpr int FM = WTM / 32;
  static constexpr int FN = WTN / 32;
  static constexpr int ADMA = BM / 32;           // load instructions per wave per stage (A rows)
  static constexpr int BDMA = BN / 32;           // (B rows)
  static constexpr int DMA = ADMA + BDMA;
  static constexpr int BUF = (BM + BN) * kRowSlice;
  static constexpr int NBR = TAPS == 27 ? BM * 27 * 4 : 0;
  // Two or four workgroups per compute unit (two or four waves per SIMD, so one hides another's
  // LDS and barrier waits) when a two-stage ring fits that often in the 160 KB LDS; otherwise
  // one workgroup with as many ring stages as fit (2 to 4).
  static constexpr int LDS2 = 2 * BUF + NBR + 256;
  static constexpr int FIT2 = (160 * 1024) / LDS2;  // two-stage rings that fit in one CU's LDS
  static constexpr int BPC = BM > 128 ? 1 : (FIT2 >= 4 ? 4 : (FIT2 >= 2 ? 2 : 1));
  static constexpr int NS_FIT = (160 * 1024 - NBR - 256) / BUF;
  static constexpr int NS = BPC > 1 ? 2 : (NS_FIT >= 4 ? 4 : (NS_FIT < 2 ? 2 : NS_FIT));
  static constexpr int LDS = NS * BUF + NBR + 256;
};

template <int V> using IC = std::integral_constant<int, V>;

template <DT D, int BM, int BN, int TAPS>
__global__ __launch_bounds__(kThreads, (DmaShape<BM, BN, TAPS>::BPC)) void subm_conv_dma_kernel(const ConvArgs args) {
  using Sh = DmaShape<BM, BN, TAPS>;
  constexpr int WM = Sh::WM, WTM = Sh::WTM, WTN = Sh::WTN, FM = Sh::FM, FN = Sh::FN;
  constexpr int ADMA = Sh::ADMA, BDMA = Sh::BDMA, DMA = Sh::DMA, BUF = Sh::BUF, NS = Sh::NS;
  static_assert(FM >= 1 && FN >= 1 && BDMA >= 1, "tile too small");
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  static_assert((BM / 2) * BN * 2 <= BUF, "epilogue staging must fit in two ring slots");
  static_assert((NS - 1) * DMA < 64, "outstanding loads exceed the vmcnt range");

  // One array per ring slot: the compiler can then see that the slot being filled by the
  // asynchronous loads and the slot being read by the matrix-core loop never alias, and does
  // not insert a wait for all outstanding loads before every LDS read.
  __shared__ __align__(16) unsigned char ring0[BUF];
  __shared__ __align__(16) unsigned char ring1[BUF];
  __shared__ __align__(16) unsigned char ring2[NS > 2 ? BUF : 16];
  __shared__ __align__(16) unsigned char ring3[NS > 3 ? BUF : 16];
  __shared__ uint32_t s_off[TAPS == 27 ? BM * 27 : 1];  // byte offset of each (row, tap) source row
  __shared__ uint32_t s_mask;
  auto ring = [&](auto I) -> unsigned char* {
    if constexpr (decltype(I)::value == 0) return ring0;
    else if constexpr (decltype(I)::value == 1) return ring1;
    else if constexpr (decltype(I)::value == 2) return ring2;
    else return ring3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM;
  const int wn = wave / WM;

  const int bid = blockIdx.x;
  const int tile = (bid & 7) * args.per_xcd + (bid >> 3);
  if (tile >= args.tiles_m) return;
  const int64_t n = args.n;
  const int64_t row0 = (int64_t)tile * BM;
  const int o0 = blockIdx.y * BN;
  const int cout = args.cout, row_bytes = args.row_bytes;
  const unsigned char* feats = static_cast<const unsigned char*>(args.feats);
  const unsigned char* weight = static_cast<const unsigned char*>(args.weight);

  if (tid == 0) s_mask = 0;
  __syncthreads();
  uint32_t local_mask = 0;
  if constexpr (TAPS == 27) {
    const int32_t* nb = args.nbr + row0 * 27;
    const int valid = (int)((n - row0) < BM ? (n - row0) : BM);
    for (int idx = tid; idx < BM * 27; idx += kThreads) {
      const int r = idx / 27;
      const int v = r < valid ? nb[idx] : -1;
      s_off[idx] = v >= 0 ? (uint32_t)v * (uint32_t)row_bytes : kOutOfRange;
      if (v >= 0) local_mask |= 1u << (idx - r * 27);
    }
  } else {
    local_mask = 1u;
  }
  for (int off = 32; off > 0; off >>= 1) local_mask |= __shfl_xor(local_mask, off, 64);
  if (lane == 0 && local_mask) atomicOr(&s_mask, local_mask);
  __syncthreads();
  const uint32_t mask = s_mask;
  const int nq = (row_bytes + kRowSlice - 1) / kRowSlice;
  const int total = __builtin_popcount(mask) * nq;  // stages in this tile

  // Load-side lane roles: lane l of a load instruction fills row (l / 8) of an 8-row group at
  // physical chunk l % 8.  Rows are swizzled as physical = logical ^ ((row / 2) % 8), which keeps
  // every 16-lane pass of a 16-byte fragment read (16 consecutive rows, one chunk) on distinct
  // banks; so lane l fetches logical chunk (l % 8) ^ ((row / 2) % 8) of its source row.
  const int lrow8 = lane >> 3;
  auto lchunk_of = [&](int group_base) { return (lane & 7) ^ (((group_base >> 1) + (lane >> 4)) & 7); };
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const i32x4_t rsrc_a = make_rsrc(feats, args.feats_bytes);
  const i32x4_t rsrc_b = make_rsrc(weight, args.weight_bytes);

  // Issue cursor: taps in ascending order, each split into nq channel slices.  prepare()
  // computes the per-lane source offsets of one stage; issue_range() emits a slice of its loads.
  uint32_t rem = mask;
  int ik = 0, iq = nq;
  uint32_t offs[DMA];
  auto prepare = [&](int stage_index) {
    const bool valid = stage_index < total;
    if (valid && iq >= nq) {
      ik = __builtin_ctz(rem);
      rem &= rem - 1;
      iq = 0;
    }
    const int k = ik, q = iq;
    if (valid) ++iq;
#pragma unroll
    for (int d = 0; d < ADMA; ++d) {
      const int g = wave * (BM / 4) + 8 * d;
      const int r = g + lrow8;
      const uint32_t cb = (uint32_t)(q * kRowSlice + lchunk_of(g) * 16);
      uint32_t base_off;
      if constexpr (TAPS == 27) {
        base_off = s_off[r * 27 + k];
      } else {
        base_off = (row0 + r < n) ? (uint32_t)(row0 + r) * (uint32_t)row_bytes : kOutOfRange;
      }
      offs[d] = (valid && (int)cb < row_bytes) ? base_off + cb : kOutOfRange;
    }
#pragma unroll
    for (int d = 0; d < BDMA; ++d) {
      const int g = wave * (BN / 4) + 8 * d;
      const int o = o0 + g + lrow8;
      const uint32_t cb = (uint32_t)(q * kRowSlice + lchunk_of(g) * 16);
      offs[ADMA + d] = (valid && (int)cb < row_bytes && o < cout)
                           ? ((uint32_t)o * TAPS + (uint32_t)k) * (uint32_t)row_bytes + cb
                           : kOutOfRange;
    }
  };
  auto issue_range = [&](unsigned char* base, int d0, int d1) {
#pragma unroll
    for (int d = 0; d < DMA; ++d) {
      if (d < d0 || d >= d1) continue;
      if (d < ADMA) {
        lds_dma16(rsrc_a, offs[d], lds_offset(base) + (uint32_t)((wave_u * (BM / 4) + 8 * d) * kRowSlice));
      } else {
        lds_dma16(rsrc_b, offs[d], lds_offset(base) + (uint32_t)((BM + wave_u * (BN / 4) + 8 * (d - ADMA)) * kRowSlice));
      }
    }
  };
  auto issue = [&](int stage_index, unsigned char* base) {
    prepare(stage_index);
    issue_range(base, 0, DMA);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int lrow = lane & 31;
  const int lk = lane >> 5;
  // Consume one stage (up to four 16-channel steps); after step kk, issue the kk-th quarter of
  // the loads of the stage NS - 1 ahead, so that address work overlaps the matrix cores.
  constexpr int DPS = (DMA + 3) / 4;
  // Every stage runs all four 16-channel steps: channels past Cin were loaded as zeros, so a
  // partial last slice only costs idle matrix-core work, and the straight-line code lets the
  // compiler keep exact LDS wait counts.
  auto compute_and_issue = [&](const unsigned char* buf, unsigned char* next) {
    const int rsw = (lrow >> 1) & 7;
    // Fragments of step kk + 1 are read while the matrix cores run step kk.
    uint4 af[2][FM], bf[2][FN];
    auto load_frags = [&](int kk, int slot) {
      const int sw = ((2 * kk + lk) ^ rsw) << 4;
#pragma unroll
      for (int i = 0; i < FM; ++i) af[slot][i] = *reinterpret_cast<const uint4*>(buf + (wm * WTM + i * 32 + lrow) * kRowSlice + sw);
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[slot][j] = *reinterpret_cast<const uint4*>(buf + (BM + wn * WTN + j * 32 + lrow) * kRowSlice + sw);
    };
    load_frags(0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) load_frags(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<D>(af[kk & 1][i], bf[kk & 1][j], acc[i][j]);
      issue_range(next, kk * DPS, (kk + 1) * DPS < DMA ? (kk + 1) * DPS : DMA);
    }
  };

  // One ring step: the oldest stage (slot S) is complete -> barrier -> consume slot S while
  // refilling the slot consumed in the previous step with the stage NS - 1 ahead.
  int st = 0;
  auto step = [&](auto S) {
    constexpr int cs = decltype(S)::value;
    constexpr int is = (cs + NS - 1) % NS;
    wait_vmcnt<(NS - 2) * DMA>();
    barrier_no_fence();
    prepare(st + NS - 1);
    compute_and_issue(ring(IC<cs>{}), ring(IC<is>{}));
    ++st;
  };
  // Prologue: stages 0 .. NS - 2 in flight; step s then issues stage s + NS - 1.
  issue(0, ring(IC<0>{}));
  if constexpr (NS > 2) issue(1, ring(IC<1>{}));
  if constexpr (NS > 3) issue(2, ring(IC<2>{}));
  while (st < total) {
    step(IC<0>{});
    if (st >= total) break;
    step(IC<1>{});
    if (st >= total) break;
    if constexpr (NS > 2) {
      step(IC<2>{});
      if (st >= total) break;
    }
    if constexpr (NS > 3) {
      step(IC<3>{});
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  // Epilogue: + bias (fp32), one RNE rounding, staged through two ring slots (rows below and
  // above BM / 2) for coalesced 16-byte stores.
  using T = typename Elem<D>::T;
  float bcol[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int o = o0 + wn * WTN + j * 32 + lrow;
    bcol[j] = (args.bias != nullptr && o < cout) ? to_float<D>(reinterpret_cast<const T*>(args.bias)[o]) : 0.f;
  }
  T* sC0 = reinterpret_cast<T*>(ring0);
  T* sC1 = reinterpret_cast<T*>(ring1);
  constexpr int HALF = BM / 2;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
        const int col = wn * WTN + j * 32 + lrow;
        T* dst = r < HALF ? sC0 + r * BN : sC1 + (r - HALF) * BN;
        dst[col] = from_float<D>(acc[i][j][v] + bcol[j]);
      }
  __syncthreads();
  T* out = reinterpret_cast<T*>(args.out);
  if (args.vec_out) {
    constexpr int CPR = BN * 2 / 16;
    for (int idx = tid; idx < BM * CPR; idx += kThreads) {
      const int r = idx / CPR, c = idx - r * CPR;
      const int64_t row = row0 + r;
      const int col = o0 + c * 8;
      const T* src = r < HALF ? sC0 + r * BN : sC1 + (r - HALF) * BN;
      if (row < n && col < cout) *reinterpret_cast<uint4*>(out + row * cout + col) = *reinterpret_cast<const uint4*>(src + c * 8);
    }
  } else {
    for (int idx = tid; idx < BM * BN; idx += kThreads) {
      const int r = idx / BN, c = idx - r * BN;
      const int64_t row = row0 + r;
      const T* src = r < HALF ? sC0 + r * BN : sC1 + (r - HALF) * BN;
      if (row < n && o0 + c < cout) out[row * cout + o0 + c] = src[c];
    }
  }
}

template <DT D, int BM, int BN, int TAPS>
hipError_t launch_dma(const ConvArgs& a0, hipStream_t stream) {
  ConvArgs a = a0;
  a.tiles_m = (int)((a.n + BM - 1) / BM);
  a.per_xcd = (a.tiles_m + 7) / 8;
  dim3 grid((unsigned)(8 * a.per_xcd), (unsigned)((a.cout + BN - 1) / BN));
  subm_conv_dma_kernel<D, BM, BN, TAPS><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

// Estimated relative time of a launch with tile height bm and bpc workgroups per compute unit:
// whole rounds of tiles over the 256 compute units, each round as long as bpc tiles of bm rows
// sharing one unit, plus a fixed per-tile overhead (the weight slices, bn rows, are loaded once
// per tile) worth 3/8 of bn rows.  Co-resident workgroups hide each other's waits; measured
// factors: 0.75 of the time for two per unit, 0.6 for four.
constexpr int kComputeUnits = 256;
inline double tile_cost(int64_t n, int col_tiles, int bm, int bn, int bpc) {
  const int64_t tiles = (n + bm - 1) / bm * col_tiles;
  const int64_t slots = (int64_t)kComputeUnits * bpc;
  const int64_t rounds = (tiles + slots - 1) / slots;
  const double overlap = bpc >= 4 ? 0.6 : (bpc == 2 ? 0.75 : 1.0);
  return (double)rounds * bpc * (bm + 3.0 * bn / 8.0) * overlap;
}

template <DT D, int BN, int TAPS>
hipError_t launch_dma_bn(const ConvArgs& a, hipStream_t stream) {
  const int col_tiles = (a.cout + BN - 1) / BN;
  const int bms[4] = {64, 128, 192, 256};
  const bool ok[4] = {BN >= 64, true, BN >= 64, true};
  const int bpcs[4] = {DmaShape<64, BN, TAPS>::BPC, DmaShape<128, BN, TAPS>::BPC, DmaShape<192, BN, TAPS>::BPC,
                       DmaShape<256, BN, TAPS>::BPC};
  int best = 3;
  double best_cost = tile_cost(a.n, col_tiles, 256, BN, bpcs[3]);
  for (int i = 2; i >= 0; --i) {
    if (!ok[i]) continue;
    const double c = tile_cost(a.n, col_tiles, bms[i], BN, bpcs[i]);
    if (c < best_cost) {
      best = i;
      best_cost = c;
    }
  }
  // SUBMCONV_TILE_M=64|128|192|256 forces the tile height (tuning and tests); ignored when that
  // height is not built for this channel width.
  if (const char* env = std::getenv("SUBMCONV_TILE_M")) {
    const int want = std::atoi(env);
    for (int i = 0; i < 4; ++i)
      if (bms[i] == want && ok[i]) best = i;
  }
  switch (bms[best]) {
    case 64: if constexpr (BN >= 64) return launch_dma<D, 64, BN, TAPS>(a, stream); break;
    case 128: return launch_dma<D, 128, BN, TAPS>(a, stream);
    case 192: if constexpr (BN >= 64) return launch_dma<D, 192, BN, TAPS>(a, stream); break;
    default: break;
  }
  return launch_dma<D, 256, BN, TAPS>(a, stream);
}

template <DT D, int TAPS>
hipError_t launch_dma_shape(const ConvArgs& a, hipStream_t stream) {
  if (a.cout <= 32) return launch_dma_bn<D, 32, TAPS>(a, stream);
  if (a.cout <= 64) return launch_dma_bn<D, 64, TAPS>(a, stream);
  return launch_dma_bn<D, 128, TAPS>(a, stream);
}

template <DT D, int BM, int BN, int WM, bool VEC, int TAPS>
hipError_t launch_tile(const ConvArgs& a0, hipStream_t stream) {
  ConvArgs a = a0;
  a.tiles_m = (int)((a.n + BM - 1) / BM);
  a.per_xcd = (a.tiles_m + 7) / 8;
  dim3 grid((unsigned)(8 * a.per_xcd), (unsigned)((a.cout + BN - 1) / BN));
  subm_conv_generic_kernel<D, BM, BN, WM, VEC, TAPS><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

template <DT D, bool VEC, int TAPS>
hipError_t launch_shape(const ConvArgs& a, hipStream_t stream) {
  if (a.cout <= 16) return launch_tile<D, 64, 16, 4, VEC, TAPS>(a, stream);
  if (a.cout <= 32) return launch_tile<D, 64, 32, 4, VEC, TAPS>(a, stream);
  if (a.cout <= 64) return launch_tile<D, 128, 64, 2, VEC, TAPS>(a, stream);
  return launch_tile<D, 128, 128, 2, VEC, TAPS>(a, stream);
}

template <DT D>
hipError_t launch_dtype(const ConvArgs& a, bool vec_in, int taps, hipStream_t stream) {
  if constexpr (D != DT::F32) {
    if (vec_in && a.cout > 16 && a.feats_bytes != 0 && a.weight_bytes != 0) {
      return taps == 27 ? launch_dma_shape<D, 27>(a, stream) : launch_dma_shape<D, 1>(a, stream);
    }
  }
  if (taps == 27) return vec_in ? launch_shape<D, true, 27>(a, stream) : launch_shape<D, false, 27>(a, stream);
  return vec_in ? launch_shape<D, true, 1>(a, stream) : launch_shape<D, false, 1>(a, stream);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
constexpr uint64_t kOffsetLimit = 0x7FFFF000ull;  // below kOutOfRange with room for a row slice

}  // namespace

hipError_t launch_subm_conv(const MapData* map, int64_t n, int ksize, int cin, int cout, int dtype,
                            const void* feats, const void* weight, const void* bias, void* out,
                            hipStream_t stream) {
  const int s = dtype == SUBM_F32 ? 4 : 2;
  ConvArgs a{};
  a.feats = feats;
  a.weight = weight;
  a.bias = bias;
  a.out = out;
  a.nbr = ksize == 3 ? map->nbr : nullptr;
  a.n = n;
  a.cin = cin;
  a.cout = cout;
  a.row_bytes = cin * s;
  a.vec_out = ((cout * s) % 16 == 0) && aligned16(out);
  const bool vec_in = (a.row_bytes % 16 == 0) && aligned16(feats) && aligned16(weight);
  const int taps = ksize == 3 ? 27 : 1;
  // The matrix-core path addresses operands with 31-bit byte offsets; larger tensors take the
  // generic kernel (size 0 marks "does not fit").
  const uint64_t fb = (uint64_t)n * (uint64_t)a.row_bytes;
  const uint64_t wb = (uint64_t)cout * (uint64_t)taps * (uint64_t)a.row_bytes;
  a.feats_bytes = fb < kOffsetLimit ? (uint32_t)fb : 0u;
  a.weight_bytes = wb < kOffsetLimit ? (uint32_t)wb : 0u;
  switch (dtype) {
    case SUBM_F32: return launch_dtype<DT::F32>(a, vec_in, taps, stream);
    case SUBM_F16: return launch_dtype<DT::F16>(a, vec_in, taps, stream);
    default: return launch_dtype<DT::BF16>(a, vec_in, taps, stream);
  }
}

}  // namespace submconv
