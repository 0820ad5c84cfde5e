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
#include "internal.h"

namespace submconv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

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
};

constexpr int kThreads = 256;
constexpr int kStageBytes = 256;  // bytes of one row per stage (16 chunks of 16 B)

template <DT D, int BM, int BN, int WM, bool VEC, int TAPS>
__global__ __launch_bounds__(kThreads, 2) void subm_conv_kernel(const ConvArgs args) {
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

template <DT D, int BM, int BN, int WM, bool VEC, int TAPS>
hipError_t launch_tile(const ConvArgs& a0, hipStream_t stream) {
  ConvArgs a = a0;
  a.tiles_m = (int)((a.n + BM - 1) / BM);
  a.per_xcd = (a.tiles_m + 7) / 8;
  dim3 grid((unsigned)(8 * a.per_xcd), (unsigned)((a.cout + BN - 1) / BN));
  subm_conv_kernel<D, BM, BN, WM, VEC, TAPS><<<grid, kThreads, 0, stream>>>(a);
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
  if (taps == 27) return vec_in ? launch_shape<D, true, 27>(a, stream) : launch_shape<D, false, 27>(a, stream);
  return vec_in ? launch_shape<D, true, 1>(a, stream) : launch_shape<D, false, 1>(a, stream);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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
  switch (dtype) {
    case SUBM_F32: return launch_dtype<DT::F32>(a, vec_in, taps, stream);
    case SUBM_F16: return launch_dtype<DT::F16>(a, vec_in, taps, stream);
    default: return launch_dtype<DT::BF16>(a, vec_in, taps, stream);
  }
}

}  // namespace submconv
