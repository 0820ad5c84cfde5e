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
//
// The kernels in this file, from the most general to the default fast path:
//   subm_conv_generic_kernel        the design above: fp32 storage, odd channel counts,
//                                   misaligned pointers, tensors beyond 31-bit byte offsets
//   subm_conv_mma_kernel            16-bit storage: 32x32x16 MFMA tiles fed by direct
//                                   global->LDS loads (no register staging)
//   subm_conv_ws_kernel             the same with separate load and matrix-core waves
//   subm_conv_ws_persistent_kernel  the default for k = 3 above 32 output channels: one
//                                   workgroup per CU walks several row tiles, eight load waves
//                                   beside four matrix-core waves
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace submconv {
namespace {


struct ConvArgs {
  const void* feats;
  const void* weight;
  const void* bias;     // may be null
  void* out;
  const int32_t* nbr;   // [n, 27]; null when taps == 1
  const uint32_t* masks;  // [n]: bit k set when nbr[i, k] >= 0; null when taps == 1
  int64_t n;
  int cin;
  int cout;
  int row_bytes;        // cin * element size
  int tiles_m;
  int per_xcd;
  int vec_out;          // 16-byte output stores allowed
  uint32_t feats_bytes;  // n * row_bytes (fast path: < 2^31)
  uint32_t weight_bytes; // cout * taps * row_bytes (fast path: < 2^31)
  // Group-norm partial sums of the rounded output (epilogue variant with statistics only):
  // gn_part[tile * gn_groups + g] = (mean, sum of squared deviations) of group g over the tile's
  // rows, groups of gn_cpg consecutive channels.
  float2* gn_part;
  int gn_cpg;
  int gn_groups;
  // non-null: flags [gate_n]; the kernel does nothing unless one is set (the fallback launched
  // beside a neighbour-pool convolution whose plan may have overflowed)
  const uint32_t* gate;
  int gate_n;
  // Row order of a sparse map (read by the persistent 27-tap walk only; null elsewhere): when
  // *order_gate is set, walk position j is input row order_rows[j], with rulebook row
  // order_nbr[j] and mask order_masks[j].
  const uint32_t* order_gate;
  const int32_t* order_rows;
  const int32_t* order_nbr;
  const uint32_t* order_masks;
};

// (every thread of the workgroup calls it)
__device__ __forceinline__ bool gated_off(const ConvArgs& a) {
  return a.gate != nullptr && !pool_any_flag(a.gate, a.gate_n);
}

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
//   * stages of SL-byte row slices (SL / 2 channels) loaded with buffer_load_dwordx4 ... lds:
//     each instruction moves 64 x 16 bytes straight into LDS, so no registers hold data in
//     flight and NS - 1 stages can be outstanding while one is consumed; the XOR swizzle of the
//     16-byte chunks is applied on the global side by choosing which chunk each lane fetches;
//     an absent neighbour or a padding chunk reads 16 zero bytes through an out-of-range offset;
//   * every stage issues the same number of load instructions (trailing stages load zeros), so
//     a constant s_waitcnt vmcnt((NS - 2) * per-stage count) waits exactly for the oldest stage;
//     the workgroup barrier is a bare s_barrier (no memory fence, which on this architecture
//     would wait for every outstanding load and serialise the ring).

// Output tile epilogue shared by the matrix-core kernels: + bias, one RNE rounding, staged in
// LDS (rows padded by 16 bytes, which spreads the 8-byte writes of 32 rows over the banks) in
// two halves of the rows, then coalesced 16-byte global stores by all NT threads.
//
// STATS: also the group-norm partial sums of the tile's rounded outputs, read back from the
// staged halves in 16-byte chunks: thread (chunk, row lane) sums x - K and (x - K)^2 per channel
// over its rows, with K the first value of the channel's group in the tile's first row (shifted
// sums stay accurate when the mean is large against the spread); the row lanes, then the
// channels of each group, are added in a fixed order.
template <DT D, int WM, int FM, int FN, int NT, bool STATS = false>
__device__ __forceinline__ void epilogue_store(const ConvArgs& args, const f32x16_t (&acc)[FM][FN], unsigned char* ring,
                                               const float* s_bias, int64_t row0, int o0, int tid, bool has_acc,
                                               int wm, int wn, int lane, int tile = 0) {
  using T = typename Elem<D>::T;
  constexpr int WN = 4 / WM, WTM = 32 * FM, WTN = 32 * FN, BM = WM * WTM, BN = WN * WTN;
  constexpr int HALF = BM / 2;
  constexpr int SROW = BN * 2 + 16;  // staging row stride in bytes
  const int64_t n = args.n;
  const int cout = args.cout;
  const int lrow = lane & 31, lk = lane >> 5;
  T* out = reinterpret_cast<T*>(args.out);
  // statistics lanes: 16-byte column chunk ck (8 channels) and row lane rl of RLS
  static_assert(!STATS || D != DT::F32, "statistics epilogue is for 16-bit storage");
  constexpr int NCK = BN / 8, RLS = NT / NCK;
  static_assert(64 % NCK == 0, "a wave holds whole rows of chunks");
  const int cpg = STATS ? args.gn_cpg : 1;
  const int ck = tid % NCK, rl = tid / NCK;
  const int vrows = (int)((n - row0) < BM ? (n - row0) : BM);
  float kk[8], a1[8], a2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) kk[e] = a1[e] = a2[e] = 0.f;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (has_acc && (wm * WTM) / HALF == pass) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 32 + lrow - pass * HALF;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = wn * WTN + j * 32 + 8 * g + 4 * lk;
            const float4 bb = *reinterpret_cast<const float4*>(s_bias + c);
            *reinterpret_cast<uint2*>(ring + r * SROW + c * 2) =
                pack4<D>(acc[i][j][4 * g] + bb.x, acc[i][j][4 * g + 1] + bb.y, acc[i][j][4 * g + 2] + bb.z,
                         acc[i][j][4 * g + 3] + bb.w);
          }
      }
    }
    __syncthreads();
    if constexpr (STATS) {
      if (pass == 0) {
        // K of each of this chunk's channels: its group's first channel in tile row 0 (a valid row)
        const T* row_0 = reinterpret_cast<const T*>(ring);
#pragma unroll
        for (int e = 0; e < 8; ++e) kk[e] = to_float<D>(row_0[(ck * 8 + e) / cpg * cpg]);
      }
      const int rend = vrows - pass * HALF < HALF ? vrows - pass * HALF : HALF;
#pragma unroll 4
      for (int r = rl; r < rend; r += RLS) {
        const uint4 raw = *reinterpret_cast<const uint4*>(ring + r * SROW + ck * 16);
        const T* x = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = to_float<D>(x[e]) - kk[e];
          a1[e] += d;
          a2[e] += d * d;
        }
      }
    }
    const int64_t rbase = row0 + pass * HALF;
    if (args.vec_out) {
      constexpr int CPR = BN * 2 / 16;
      for (int idx = tid; idx < HALF * CPR; idx += NT) {
        const int r = idx / CPR, c = idx - r * CPR;
        const int64_t row = rbase + r;
        const int col = o0 + c * 8;
        if (row < n && col < cout)
          *reinterpret_cast<uint4*>(out + row * cout + col) = *reinterpret_cast<const uint4*>(ring + r * SROW + c * 16);
      }
    } else {
      for (int idx = tid; idx < HALF * BN; idx += NT) {
        const int r = idx / BN, c = idx - r * BN;
        const int64_t row = rbase + r;
        if (row < n && o0 + c < cout) out[row * cout + o0 + c] = *reinterpret_cast<const T*>(ring + r * SROW + c * 2);
      }
    }
    __syncthreads();
  }
  if constexpr (STATS) {
    // Row lanes of one wave share their chunk with lanes l ^ NCK, l ^ 2 NCK, ...: a butterfly
    // of shuffles leaves the wave's sums in every lane; then the waves are added in order in LDS
    // (the ring is free now), and one thread per group adds its channels.
    constexpr int NW = NT / 64;
#pragma unroll
    for (int o = NCK; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a1[e] += __shfl_xor(a1[e], o);
        a2[e] += __shfl_xor(a2[e], o);
      }
    float* red = reinterpret_cast<float*>(ring);  // [2][NW][BN]
    float* tot = red + 2 * NW * BN;               // [2][BN]
    float* shf = tot + 2 * BN;                    // [BN]
    const int w = tid >> 6;
    if (lane < NCK)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        red[w * BN + ck * 8 + e] = a1[e];
        red[(NW + w) * BN + ck * 8 + e] = a2[e];
        if (w == 0) shf[ck * 8 + e] = kk[e];
      }
    __syncthreads();
    if (tid < BN) {
      float t1 = 0.f, t2 = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        t1 += red[q * BN + tid];
        t2 += red[(NW + q) * BN + tid];
      }
      tot[tid] = t1;
      tot[BN + tid] = t2;
    }
    __syncthreads();
    const int gt = BN / cpg;
    if (tid < gt && o0 + tid * cpg < cout) {
      float t1 = 0.f, t2 = 0.f;
      for (int c = tid * cpg; c < (tid + 1) * cpg; ++c) {
        t1 += tot[c];
        t2 += tot[BN + c];
      }
      const float mean_d = t1 / (float)(vrows * cpg);
      args.gn_part[(int64_t)tile * args.gn_groups + o0 / cpg + tid] =
          make_float2(shf[tid * cpg] + mean_d, fmaxf(t2 - t1 * mean_d, 0.f));
    }
  }
}

// Tile of the matrix-core kernel.  WM x WN = 4 waves; each wave owns FM 32-row blocks and FN
// 32-column blocks of the BM x BN output tile.  A stage is one SL-byte slice (SL / 2 channels)
// of every row of the tile (A) and of every weight row (B).
constexpr int kMaxStages = 8;

template <int WM, int FM, int FN, int SL, int TAPS>
struct MmaShape {
  static constexpr int WN = 4 / WM;
  static constexpr int WTM = 32 * FM, WTN = 32 * FN;  // rows / columns per wave
  static constexpr int BM = WM * WTM;                 // rows per tile
  static constexpr int BN = WN * WTN;                 // output channels per tile
  static constexpr int CH = SL / 16;                  // 16-byte chunks per row slice
  static constexpr int RPI = 64 / CH;                 // rows per 1 KB load instruction
  static constexpr int KSTEPS = SL / 32;              // 16-channel matrix-core steps per stage
  static constexpr int ADMA = BM / RPI / 4;           // A loads per wave per stage
  static constexpr int BDMA = (BN + 4 * RPI - 1) / (4 * RPI);  // B loads per wave per stage
  static constexpr int BNP = 4 * RPI * BDMA;          // B rows per stage (rows past BN load zeros)
  static constexpr int DMA = ADMA + BDMA;
  static constexpr int BUF = (BM + BNP) * SL;         // one ring slot
  // The tile's rulebook rows (BM x 27 int32, contiguous in the map) are copied into LDS with
  // NDMA direct loads per wave (whole 1 KB instructions, so the copy is padded).
  static constexpr int NDMA = TAPS == 27 ? (BM * 27 * 4 + 4095) / 4096 : 0;
  static constexpr int NBR = NDMA * 4096;
  static constexpr int NS_FIT = (160 * 1024 - NBR - 512) / BUF;
  static constexpr int NS = NS_FIT >= kMaxStages ? kMaxStages : NS_FIT;  // ring depth
  static_assert(BM % (4 * RPI) == 0, "A rows must split into whole load instructions per wave");
};

template <int V> using IC = std::integral_constant<int, V>;

template <DT D, int WM, int FM, int FN, int SL, int TAPS>
__global__ __launch_bounds__(kThreads, 1) void subm_conv_mma_kernel(const ConvArgs args) {
  using Sh = MmaShape<WM, FM, FN, SL, TAPS>;
  constexpr int WTM = Sh::WTM, WTN = Sh::WTN, BM = Sh::BM, BN = Sh::BN, BNP = Sh::BNP;
  constexpr int CH = Sh::CH, RPI = Sh::RPI, KSTEPS = Sh::KSTEPS;
  constexpr int ADMA = Sh::ADMA, BDMA = Sh::BDMA, DMA = Sh::DMA, BUF = Sh::BUF, NS = Sh::NS;
  static_assert(NS >= 2, "ring depth");
  static_assert((BM / 2) * (BN * 2 + 16) <= NS * BUF, "epilogue staging must fit in the ring");
  static_assert((NS - 1) * DMA < 64 && Sh::NDMA < 64, "outstanding loads exceed the vmcnt range");

  // The ring of NS stages in one array; slots are addressed at run time.  The direct loads are
  // invisible to the compiler, so it inserts no waits of its own for them.
  __shared__ __align__(16) unsigned char ring[NS * BUF];
  __shared__ __align__(16) int32_t s_nbr[TAPS == 27 ? Sh::NBR / 4 : 4];  // the tile's rulebook rows
  __shared__ __align__(16) float s_bias[BN];
  __shared__ uint32_t s_mask;

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
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // The tile's rulebook rows go straight into LDS (all loads in flight at once; bytes past the
  // map read as zeros and belong to rows >= n, which fetch() treats as absent), and the mask of
  // taps used anywhere in the tile is the OR of the rows' neighbour masks.  Taps no row uses
  // are skipped.
  if (tid == 0) s_mask = 0;
  using T = typename Elem<D>::T;
  if (tid < BN) {
    const int o = o0 + tid;
    s_bias[tid] = (args.bias != nullptr && o < cout) ? to_float<D>(reinterpret_cast<const T*>(args.bias)[o]) : 0.f;
  }
  uint32_t local_mask = 0;
  if constexpr (TAPS == 27) {
    const i32x4_t rsrc_n = make_rsrc(args.nbr, (uint32_t)(n * 27 * 4));
    const uint32_t gbase = (uint32_t)(row0 * 27 * 4);
#pragma unroll
    for (int d = 0; d < Sh::NDMA; ++d) {
      const uint32_t blk = (uint32_t)((wave_u * Sh::NDMA + d) * 1024);
      lds_dma16(rsrc_n, gbase + blk + (uint32_t)lane * 16u, lds_offset(s_nbr) + blk);
    }
#pragma unroll
    for (int u = 0; u < (BM + kThreads - 1) / kThreads; ++u) {
      const int64_t row = row0 + tid + u * kThreads;
      if (tid + u * kThreads < BM && row < n) local_mask |= args.masks[row];
    }
  } else {
    local_mask = 1u;
  }
  for (int off = 32; off > 0; off >>= 1) local_mask |= __shfl_xor(local_mask, off, 64);
  __syncthreads();
  if (lane == 0 && local_mask) atomicOr(&s_mask, local_mask);
  wait_vmcnt<0>();
  __syncthreads();
  const uint32_t mask = s_mask;
  const int nq = (row_bytes + SL - 1) / SL;
  const int total = __builtin_popcount(mask) * nq;  // stages in this tile

  // Load-side lane roles: lane l of a load instruction fills row l / CH of an RPI-row group at
  // physical chunk l % CH.  Rows are swizzled as physical = logical ^ ((row / (16 / CH)) % CH),
  // which keeps every 16-lane pass of a fragment read (16 consecutive rows, one chunk) on
  // distinct banks; so lane l fetches logical chunk (l % CH) ^ swizzle(its row).
  auto swz_of = [](int row) { return (row / (16 / CH)) % CH; };
  auto chunk_bytes = [&](int group_row) {
    return (uint32_t)(((lane % CH) ^ swz_of(group_row + lane / CH)) * 16);
  };
  const i32x4_t rsrc_a = make_rsrc(args.feats, args.feats_bytes);
  const i32x4_t rsrc_b = make_rsrc(args.weight, args.weight_bytes);

  // Per-lane constants: the chunk each load fetches, and the weight-row part of the B offsets.
  uint32_t lane_cb[DMA], base_b[BDMA];
  bool ok_b[BDMA];
#pragma unroll
  for (int d = 0; d < ADMA; ++d) lane_cb[d] = chunk_bytes(wave * (BM / 4) + RPI * d);
#pragma unroll
  for (int d = 0; d < BDMA; ++d) {
    const int g = BM + wave * (BNP / 4) + RPI * d;
    const int ol = g - BM + lane / CH;
    const int o = o0 + ol;
    lane_cb[ADMA + d] = chunk_bytes(g);
    ok_b[d] = ol < BN && o < cout;
    base_b[d] = (uint32_t)(ok_b[d] ? o : 0) * TAPS * (uint32_t)row_bytes + lane_cb[ADMA + d];
  }

  // Issue cursor: taps in ascending order, each split into nq slices of SL bytes.  fetch()
  // reads the source rows of the next stage from LDS a stage before they are needed; make()
  // turns them into this lane's load offsets (branch-free, so the scheduler can place it
  // between matrix-core instructions); issue() emits the stage's loads.
  uint32_t rem = mask;
  int ik = 0, iq = nq;
  int pk = 0, pq = 0;    // tap and slice of the fetched stage
  bool pvalid = false;   // the fetched stage exists
  int32_t raw[ADMA];     // rulebook entries (source rows) of the fetched stage, -1 if absent
  uint32_t offs[DMA];
  // Rows of this lane's A loads that exist (the last tile may be partial).
  bool row_ok[ADMA];
#pragma unroll
  for (int d = 0; d < ADMA; ++d) row_ok[d] = row0 + wave * (BM / 4) + RPI * d + lane / CH < n;
  auto fetch = [&](int stage_index) {
    pvalid = stage_index < total;
    const bool adv = pvalid && iq >= nq;
    const int nk = __builtin_ctz(rem | 0x80000000u);
    ik = adv ? nk : ik;
    rem = adv ? (rem & (rem - 1)) : rem;
    iq = adv ? 0 : iq;
    pk = ik;
    pq = iq;
    iq += pvalid ? 1 : 0;
#pragma unroll
    for (int d = 0; d < ADMA; ++d) {
      const int r = wave * (BM / 4) + RPI * d + lane / CH;
      if constexpr (TAPS == 27) {
        raw[d] = s_nbr[r * 27 + pk];
      } else {
        raw[d] = (int32_t)(row0 + r);
      }
    }
  };
  auto make = [&]() {
    const uint32_t sq = (uint32_t)(pq * SL);
    const uint32_t sb = (uint32_t)pk * (uint32_t)row_bytes + sq;
    const int limit = pvalid ? row_bytes - (int)sq : 0;  // chunks at or past this are padding
    // Products computed unconditionally and conditions combined with '&': a short-circuit
    // condition around the multiply becomes exec-masked control flow, which the scheduler cannot
    // move matrix-core instructions across.
#pragma unroll
    for (int d = 0; d < ADMA; ++d) {
      const uint32_t o = (uint32_t)raw[d] * (uint32_t)row_bytes + sq + lane_cb[d];
      const bool use = (raw[d] >= 0) & row_ok[d] & ((int)lane_cb[d] < limit);
      offs[d] = use ? o : kOutOfRange;
    }
#pragma unroll
    for (int d = 0; d < BDMA; ++d) {
      const bool use = ok_b[d] & ((int)lane_cb[ADMA + d] < limit);
      offs[ADMA + d] = use ? base_b[d] + sb : kOutOfRange;
    }
  };
  // Loads [d0, d1) of the stage (A loads first, then B).
  auto issue_range = [&](unsigned char* base, int d0, int d1) {
#pragma unroll
    for (int d = 0; d < DMA; ++d) {
      if (d < d0 || d >= d1) continue;
      if (d < ADMA)
        lds_dma16(rsrc_a, offs[d], lds_offset(base) + (uint32_t)((wave_u * (BM / 4) + RPI * d) * SL));
      else
        lds_dma16(rsrc_b, offs[d], lds_offset(base) + (uint32_t)((BM + wave_u * (BNP / 4) + RPI * (d - ADMA)) * SL));
    }
  };
  auto issue = [&](unsigned char* base) { issue_range(base, 0, DMA); };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Matrix-core side: a stage is KSTEPS 16-channel steps.  Lane l supplies row (or column)
  // l % 32 of a 32 x 16 operand block, channels 8 * (l / 32) .. + 7 of the step, from LDS
  // chunk 2 * step + l / 32 (swizzled).  All fragments of a stage are read one stage ahead, into
  // the register set that is not being multiplied, so every LDS read has a whole stage of
  // matrix-core work to hide behind and there is a single wait per stage.
  const int lrow = lane & 31;
  const int lk = lane >> 5;
  const int swz = swz_of(lrow);
  uint4 fa[2][KSTEPS][FM], fb[2][KSTEPS][FN];  // [set][step][block]
  auto read_step = [&](auto SET, auto KK, const unsigned char* buf) {
    constexpr int t = decltype(SET)::value, kk = decltype(KK)::value;
    const int off = ((2 * kk + lk) ^ swz) << 4;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[t][kk][i] = *reinterpret_cast<const uint4*>(buf + (wm * WTM + i * 32 + lrow) * SL + off);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[t][kk][j] = *reinterpret_cast<const uint4*>(buf + (BM + wn * WTN + j * 32 + lrow) * SL + off);
  };
  auto read_stage = [&](auto SET, const unsigned char* buf) {
    read_step(SET, IC<0>{}, buf);
    if constexpr (KSTEPS > 1) read_step(SET, IC<1>{}, buf);
    if constexpr (KSTEPS > 2) read_step(SET, IC<2>{}, buf);
    if constexpr (KSTEPS > 3) read_step(SET, IC<3>{}, buf);
  };
  auto multiply_step = [&](auto SET, auto KK) {
    constexpr int t = decltype(SET)::value, kk = decltype(KK)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<D>(fb[t][kk][j], fa[t][kk][i], acc[i][j]);
  };
  // Within a step: one LDS read and a few address instructions after each matrix-core
  // instruction.  A long run of reads fills the LDS queue and stalls the single wave on the
  // SIMD, and with it the matrix core; address work left in front of the step idles it.
  auto interleave = [&]() {
#pragma unroll
    for (int g = 0; g < FM * FN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // up to four VALU
    }
  };
  constexpr int DPS = (DMA + KSTEPS - 1) / KSTEPS;  // loads issued per step

  // Prologue: stages 0 .. NS - 1 fill every slot; wait for stage 0 and read it.
#pragma unroll
  for (int s0 = 0; s0 < NS; ++s0) {
    fetch(s0);
    make();
    issue(ring + s0 * BUF);
  }
  fetch(NS);
  wait_vmcnt<(NS - 1) * DMA>();
  barrier_no_fence();
  read_stage(IC<0>{}, ring);

  // Stage st (slot `slot`, fragments in register set SET):
  //   wait until this wave's loads of stage st + 1 have landed and its reads of stage st have
  //   returned; barrier (every wave's loads of st + 1 are in LDS, nobody reads slot st any
  //   more); read stage st + 1 into the other set; refill slot st with stage st + NS; multiply.
  // Nothing crosses a stage boundary (sched_barrier): the scheduler would otherwise hoist the
  // next stage's matrix-core instructions next to the reads that feed them.
  int st = 0, slot = 0;
  // Each step of the stage is its own scheduling group: the next stage's fragments for that
  // step, the step's matrix-core instructions, and a share of the loads that refill slot st.
  auto step_group = [&](auto SET, auto KK, unsigned char* cur, const unsigned char* next) {
    constexpr int t = decltype(SET)::value, kk = decltype(KK)::value;
    if constexpr (kk < KSTEPS) {
      read_step(IC<1 - t>{}, KK, next);
      multiply_step(SET, KK);
      issue_range(cur, kk * DPS, (kk + 1) * DPS < DMA ? (kk + 1) * DPS : DMA);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto step = [&](auto SET) {
    unsigned char* cur = ring + slot * BUF;
    const int next_slot = slot + 1 == NS ? 0 : slot + 1;
    const unsigned char* next = ring + next_slot * BUF;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(NS - 2) * DMA>();
    wait_lgkmcnt0();
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
    make();                  // stage st + NS, from the rulebook entries fetched a stage ago
    fetch(st + NS + 1);
    step_group(SET, IC<0>{}, cur, next);
    step_group(SET, IC<1>{}, cur, next);
    step_group(SET, IC<2>{}, cur, next);
    step_group(SET, IC<3>{}, cur, next);
    slot = next_slot;
    ++st;
  };
  // Whole pairs of stages in the loop (one exit, so the accumulators keep their registers),
  // then an odd last stage.
  while (st + 1 < total) {
    step(IC<0>{});
    step(IC<1>{});
  }
  if (st < total) step(IC<0>{});
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<0>();
  __syncthreads();

  // Epilogue: + bias (fp32), one RNE rounding, staged through the ring in two halves of the
  // rows for coalesced 16-byte stores.  With the weights as the first matrix-core operand, lane
  // l holds row l % 32 of its 32 x 32 block and, in accumulator registers 4g .. 4g + 3, the four
  // consecutive columns 8g + 4 (l / 32) .. + 3: one 8-byte LDS write each.
  epilogue_store<D, WM, FM, FN, kThreads>(args, acc, ring, s_bias, row0, o0, tid, true, wm, wn, lane);
}

// Warp-specialised variant: 512 threads, four compute waves (one per SIMD) that only read
// fragments from LDS and issue matrix-core instructions, and four load waves that only turn
// rulebook entries into addresses and issue the direct-to-LDS loads.  A compute wave therefore
// never stalls behind a load that cannot issue, and a load wave never waits for the matrix core.
// One workgroup barrier per stage hands ring slots between the two roles.
constexpr int kWsThreads = 512;

// KP selects how far ahead the compute waves read fragments: 0 = a whole stage (two register
// sets of a stage), 1 = one 16-channel step (two sets of a step, so wider slices fit the
// register budget of two waves per SIMD; the stage barrier then sits before the last step).
template <DT D, int WM, int FM, int FN, int SL, int TAPS, int KP, bool STATS = false>
__global__ __launch_bounds__(kWsThreads, 1) void subm_conv_ws_kernel(const ConvArgs args) {
  using Sh = MmaShape<WM, FM, FN, SL, TAPS>;
  constexpr int WTM = Sh::WTM, WTN = Sh::WTN, BM = Sh::BM, BN = Sh::BN, BNP = Sh::BNP;
  constexpr int CH = Sh::CH, RPI = Sh::RPI, KSTEPS = Sh::KSTEPS;
  constexpr int ADMA = Sh::ADMA, BDMA = Sh::BDMA, DMA = Sh::DMA, BUF = Sh::BUF, NS = Sh::NS;
  static_assert(NS >= 2, "ring depth");
  static_assert((BM / 2) * (BN * 2 + 16) <= NS * BUF, "epilogue staging must fit in the ring");
  static_assert((NS - 1) * DMA < 64 && Sh::NDMA < 64, "outstanding loads exceed the vmcnt range");

  __shared__ __align__(16) unsigned char ring[NS * BUF];
  __shared__ __align__(16) int32_t s_nbr[TAPS == 27 ? Sh::NBR / 4 : 4];
  __shared__ __align__(16) float s_bias[BN];
  __shared__ uint32_t s_mask;
  if (gated_off(args)) return;  // (whole workgroup: no barrier has run yet)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool loader = wave >= 4;
  const int cw = wave & 3;  // index of the wave within its role
  const int wm = cw % WM;
  const int wn = cw / WM;

  const int bid = blockIdx.x;
  const int tile = (bid & 7) * args.per_xcd + (bid >> 3);
  if (tile >= args.tiles_m) return;
  const int64_t n = args.n;
  const int64_t row0 = (int64_t)tile * BM;
  const int o0 = blockIdx.y * BN;
  const int cout = args.cout, row_bytes = args.row_bytes;
  const int cw_u = __builtin_amdgcn_readfirstlane(cw);

  // Rulebook rows into LDS (load waves) and the tap mask from the rows' neighbour masks.
  if (tid == 0) s_mask = 0;
  using T = typename Elem<D>::T;
  if (tid < BN) {
    const int o = o0 + tid;
    s_bias[tid] = (args.bias != nullptr && o < cout) ? to_float<D>(reinterpret_cast<const T*>(args.bias)[o]) : 0.f;
  }
  uint32_t local_mask = 0;
  if constexpr (TAPS == 27) {
    if (loader) {
      const i32x4_t rsrc_n = make_rsrc(args.nbr, (uint32_t)(n * 27 * 4));
      const uint32_t gbase = (uint32_t)(row0 * 27 * 4);
#pragma unroll
      for (int d = 0; d < Sh::NDMA; ++d) {
        const uint32_t blk = (uint32_t)((cw_u * Sh::NDMA + d) * 1024);
        lds_dma16(rsrc_n, gbase + blk + (uint32_t)lane * 16u, lds_offset(s_nbr) + blk);
      }
    }
#pragma unroll
    for (int u = 0; u < (BM + kWsThreads - 1) / kWsThreads; ++u) {
      const int64_t row = row0 + tid + u * kWsThreads;
      if (tid + u * kWsThreads < BM && row < n) local_mask |= args.masks[row];
    }
  } else {
    local_mask = 1u;
  }
  for (int off = 32; off > 0; off >>= 1) local_mask |= __shfl_xor(local_mask, off, 64);
  __syncthreads();
  if (lane == 0 && local_mask) atomicOr(&s_mask, local_mask);
  wait_vmcnt<0>();
  __syncthreads();
  const uint32_t mask = s_mask;
  const int nq = (row_bytes + SL - 1) / SL;
  const int total = __builtin_popcount(mask) * nq;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int lrow = lane & 31;
  const int lk = lane >> 5;
  auto swz_of = [](int row) { return (row / (16 / CH)) % CH; };

  if (loader) {
    // ---- load waves: the same lane roles, cursor and offsets as the single-role kernel, with
    // the four load waves taking the places of the four waves there.
    auto chunk_bytes = [&](int group_row) {
      return (uint32_t)(((lane % CH) ^ swz_of(group_row + lane / CH)) * 16);
    };
    const i32x4_t rsrc_a = make_rsrc(args.feats, args.feats_bytes);
    const i32x4_t rsrc_b = make_rsrc(args.weight, args.weight_bytes);
    uint32_t lane_cb[DMA], base_b[BDMA];
    bool ok_b[BDMA];
#pragma unroll
    for (int d = 0; d < ADMA; ++d) lane_cb[d] = chunk_bytes(cw * (BM / 4) + RPI * d);
#pragma unroll
    for (int d = 0; d < BDMA; ++d) {
      const int g = BM + cw * (BNP / 4) + RPI * d;
      const int ol = g - BM + lane / CH;
      const int o = o0 + ol;
      lane_cb[ADMA + d] = chunk_bytes(g);
      ok_b[d] = ol < BN && o < cout;
      base_b[d] = (uint32_t)(ok_b[d] ? o : 0) * TAPS * (uint32_t)row_bytes + lane_cb[ADMA + d];
    }
    bool row_ok[ADMA];
#pragma unroll
    for (int d = 0; d < ADMA; ++d) row_ok[d] = row0 + cw * (BM / 4) + RPI * d + lane / CH < n;
    uint32_t rem = mask;
    int ik = 0, iq = nq;
    int pk = 0, pq = 0;
    bool pvalid = false;
    int32_t raw[ADMA];
    uint32_t offs[DMA];
    auto fetch = [&](int stage_index) {
      pvalid = stage_index < total;
      const bool adv = pvalid && iq >= nq;
      const int nk = __builtin_ctz(rem | 0x80000000u);
      ik = adv ? nk : ik;
      rem = adv ? (rem & (rem - 1)) : rem;
      iq = adv ? 0 : iq;
      pk = ik;
      pq = iq;
      iq += pvalid ? 1 : 0;
#pragma unroll
      for (int d = 0; d < ADMA; ++d) {
        const int r = cw * (BM / 4) + RPI * d + lane / CH;
        if constexpr (TAPS == 27) {
          raw[d] = s_nbr[r * 27 + pk];
        } else {
          raw[d] = (int32_t)(row0 + r);
        }
      }
    };
    auto make = [&]() {
      const uint32_t sq = (uint32_t)(pq * SL);
      const uint32_t sb = (uint32_t)pk * (uint32_t)row_bytes + sq;
      const int limit = pvalid ? row_bytes - (int)sq : 0;
#pragma unroll
      for (int d = 0; d < ADMA; ++d) {
        const uint32_t o = (uint32_t)raw[d] * (uint32_t)row_bytes + sq + lane_cb[d];
        const bool use = (raw[d] >= 0) & row_ok[d] & ((int)lane_cb[d] < limit);
        offs[d] = use ? o : kOutOfRange;
      }
#pragma unroll
      for (int d = 0; d < BDMA; ++d) {
        const bool use = ok_b[d] & ((int)lane_cb[ADMA + d] < limit);
        offs[ADMA + d] = use ? base_b[d] + sb : kOutOfRange;
      }
    };
    auto issue = [&](unsigned char* base) {
#pragma unroll
      for (int d = 0; d < ADMA; ++d)
        lds_dma16(rsrc_a, offs[d], lds_offset(base) + (uint32_t)((cw_u * (BM / 4) + RPI * d) * SL));
#pragma unroll
      for (int d = 0; d < BDMA; ++d)
        lds_dma16(rsrc_b, offs[ADMA + d], lds_offset(base) + (uint32_t)((BM + cw_u * (BNP / 4) + RPI * d) * SL));
    };
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0) {
      fetch(s0);
      make();
      issue(ring + s0 * BUF);
    }
    fetch(NS);
    wait_vmcnt<(NS - 1) * DMA>();
    barrier_no_fence();
    int slot = 0;
    for (int st = 0; st < total; ++st) {
      // Barrier st: this wave's loads of stage st + 1 have landed; afterwards slot st is free.
      wait_vmcnt<(NS - 2) * DMA>();
      barrier_no_fence();
      make();
      issue(ring + slot * BUF);
      fetch(st + NS + 1);
      slot = slot + 1 == NS ? 0 : slot + 1;
    }
    wait_vmcnt<0>();
  } else {
    // ---- compute waves
    const int swz = swz_of(lrow);
    if constexpr (KP == 1) {
      // Fragments one 16-channel step ahead, in two register sets by step parity.
      uint4 ga[2][FM], gb[2][FN];
      auto read_step = [&](auto P, auto KK, const unsigned char* buf) {
        constexpr int p = decltype(P)::value, kk = decltype(KK)::value;
        const int off = ((2 * kk + lk) ^ swz) << 4;
#pragma unroll
        for (int i = 0; i < FM; ++i)
          ga[p][i] = *reinterpret_cast<const uint4*>(buf + (wm * WTM + i * 32 + lrow) * SL + off);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          gb[p][j] = *reinterpret_cast<const uint4*>(buf + (BM + wn * WTN + j * 32 + lrow) * SL + off);
      };
      auto mul_step = [&](auto P) {
        constexpr int p = decltype(P)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<D>(gb[p][j], ga[p][i], acc[i][j]);
      };
      auto interleave_step = [&]() {
#pragma unroll
        for (int g = 0; g < FM * FN; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
        }
      };
      // Step kk of the stage in slot `cur` (not the last): read step kk + 1, multiply step kk.
      auto inner = [&](auto KK, const unsigned char* cur) {
        constexpr int kk = decltype(KK)::value;
        if constexpr (kk < KSTEPS - 1) {
          __builtin_amdgcn_sched_barrier(0);
          read_step(IC<(kk + 1) & 1>{}, IC<kk + 1>{}, cur);
          mul_step(IC<kk & 1>{});
          interleave_step();
        }
      };
      barrier_no_fence();  // stage 0 has landed
      read_step(IC<0>{}, IC<0>{}, ring);
      int slot = 0;
      for (int st = 0; st < total; ++st) {
        const unsigned char* cur = ring + slot * BUF;
        const int next_slot = slot + 1 == NS ? 0 : slot + 1;
        inner(IC<0>{}, cur);
        inner(IC<1>{}, cur);
        inner(IC<2>{}, cur);
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkmcnt0();
        barrier_no_fence();  // barrier st: stage st + 1 in LDS; this wave is done with slot st
        __builtin_amdgcn_sched_barrier(0);
        read_step(IC<KSTEPS & 1>{}, IC<0>{}, ring + next_slot * BUF);
        mul_step(IC<(KSTEPS - 1) & 1>{});
        interleave_step();
        slot = next_slot;
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
    // Fragments of stage st + 1 are read during stage st.
    uint4 fa[2][KSTEPS][FM], fb[2][KSTEPS][FN];
    auto read_stage = [&](auto SET, const unsigned char* buf) {
      constexpr int t = decltype(SET)::value;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int off = ((2 * kk + lk) ^ swz) << 4;
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[t][kk][i] = *reinterpret_cast<const uint4*>(buf + (wm * WTM + i * 32 + lrow) * SL + off);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[t][kk][j] = *reinterpret_cast<const uint4*>(buf + (BM + wn * WTN + j * 32 + lrow) * SL + off);
      }
    };
    auto multiply = [&](auto SET) {
      constexpr int t = decltype(SET)::value;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<D>(fb[t][kk][j], fa[t][kk][i], acc[i][j]);
    };
    auto interleave = [&]() {
#pragma unroll
      for (int g = 0; g < KSTEPS * FM * FN; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
      }
    };
    barrier_no_fence();  // stage 0 has landed
    read_stage(IC<0>{}, ring);
    int st = 0, slot = 0;
    auto step = [&](auto SET) {
      constexpr int t = decltype(SET)::value;
      const int next_slot = slot + 1 == NS ? 0 : slot + 1;
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkmcnt0();
      barrier_no_fence();  // barrier st: stage st + 1 in LDS; this wave is done with slot st
      __builtin_amdgcn_sched_barrier(0);
      read_stage(IC<1 - t>{}, ring + next_slot * BUF);
      multiply(IC<t>{});
      interleave();
      slot = next_slot;
      ++st;
    };
    while (st + 1 < total) {
      step(IC<0>{});
      step(IC<1>{});
    }
    if (st < total) step(IC<0>{});
    __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();

  // Epilogue: compute waves stage + bias, one rounding; all 512 threads store.
  epilogue_store<D, WM, FM, FN, kWsThreads, STATS>(args, acc, ring, s_bias, row0, o0, tid, !loader, wm, wn, lane, tile);
}

// Persistent variant of the warp-specialised kernel (16-bit storage, k = 3, step-ahead
// fragments).  One workgroup per compute unit walks several row tiles in a row: the load waves
// keep filling the ring across tile boundaries, and the compute waves write a finished tile
// straight from their accumulators (bias, one RNE rounding, 8-byte stores; no LDS staging and
// no barrier), so the epilogue of one tile and the rulebook and first stages of the next overlap
// the loads in flight.  The tiles of a workgroup and their tap masks are computed by every wave
// before the roles split, so both roles run exactly the same number of stage barriers.
constexpr int kMaxBlockTiles = 256;
constexpr int kPersistentBlocks = 256;  // one workgroup per compute unit

// Orders ordinary LDS accesses against the direct loads, which the compiler does not see.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

template <DT D, int WM, int FM, int FN, int SL, int LW>
__global__ __launch_bounds__(64 * (4 + LW), 1) void subm_conv_ws_persistent_kernel(const ConvArgs args) {
  using Sh = MmaShape<WM, FM, FN, SL, 27>;
  constexpr int WTM = Sh::WTM, WTN = Sh::WTN, BM = Sh::BM, BN = Sh::BN;
  constexpr int CH = Sh::CH, RPI = Sh::RPI, KSTEPS = Sh::KSTEPS;
  // LW load waves beside the four compute waves: each loads BM / LW rows of A and its share of
  // the B rows.  (One wave sustains only so many direct-to-LDS loads: measured with a copy probe,
  // four waves per CU reach ~37 B/clk, eight ~49 B/clk.)
  constexpr int NT = 64 * (4 + LW);
  constexpr int QROWS = BM / LW;                         // A rows (and rulebook rows) per load wave
  constexpr int ADMA = QROWS / RPI;                      // A loads per load wave per stage
  constexpr int BDMA = (BN + LW * RPI - 1) / (LW * RPI); // B loads per load wave per stage
  constexpr int BNP = LW * RPI * BDMA;                   // B rows per stage (rows past BN load zeros)
  constexpr int DMA = ADMA + BDMA;
  constexpr int BUF = (BM + BNP) * SL;                   // one ring slot
  constexpr int QDMA = (QROWS * 27 * 4 + 1023) / 1024;   // 1 KB direct loads of rulebook rows per load wave
  constexpr int NS_FIT = (160 * 1024 - LW * QDMA * 1024 - 2048) / BUF;
  constexpr int NS = NS_FIT >= kMaxStages ? kMaxStages : NS_FIT;  // ring depth
  static_assert(QROWS % RPI == 0, "A rows split into whole load instructions per wave");
  static_assert(NS >= 2, "ring depth");
  static_assert((NS - 1) * DMA < 64 && QDMA < 64, "outstanding loads exceed the vmcnt range");
  static_assert((QROWS * 27 * 4) % 16 == 0 && (BM * 27 * 4) % 16 == 0, "rulebook rows in whole 16-byte chunks");
  static_assert(KSTEPS <= 4, "step-ahead schedule covers up to four steps per stage");

  __shared__ __align__(16) unsigned char ring[NS * BUF];
  __shared__ __align__(16) int32_t s_nbr[LW * QDMA * 256];  // one slot of QDMA KB per load wave
  __shared__ __align__(16) float s_bias[BN];
  __shared__ uint32_t s_tmask[kMaxBlockTiles];
  if (gated_off(args)) return;  // (whole workgroup: no barrier has run yet)
  // The walk's row order: the input order, or the map's sparse-row order when its gate is set
  // (same outputs: a row's taps are added in the same order, and only absent ones are skipped).
  const bool ordered = args.order_gate != nullptr && *args.order_gate != 0u;
  const int32_t* const nbr_w = ordered ? args.order_nbr : args.nbr;
  const uint32_t* const masks_w = ordered ? args.order_masks : args.masks;
  const int32_t* const rows_w = ordered ? args.order_rows : nullptr;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool loader = wave >= 4;
  const int cw = loader ? wave - 4 : wave;  // index of the wave within its role
  const int wm = cw % WM;
  const int wn = cw / WM;
  const int cw_u = __builtin_amdgcn_readfirstlane(cw);
  const int64_t n = args.n;
  const int o0 = blockIdx.y * BN;
  const int cout = args.cout, row_bytes = args.row_bytes;

  // This workgroup's tiles: virtual block bid + k * gridDim.x, mapped XCD-aware (gridDim.x is a
  // multiple of 8, so all of them stay on this workgroup's XCD).
  const int nblk = (int)gridDim.x, bid = (int)blockIdx.x;
  auto tile_of = [&](int k) { return (bid & 7) * args.per_xcd + (bid >> 3) + k * (nblk >> 3); };
  int ntiles = 0;
  while (ntiles < kMaxBlockTiles && (bid >> 3) + ntiles * (nblk >> 3) < args.per_xcd && tile_of(ntiles) < args.tiles_m)
    ++ntiles;
  if (ntiles == 0) return;  // whole workgroup: no barrier has run yet

  // Rulebook rows of tile k for this load wave's share of the rows, into its own slot (only this
  // wave reads it, so its own wait is enough).
  const i32x4_t rsrc_n = make_rsrc(nbr_w, (uint32_t)(n * 27 * 4));
  auto issue_rows = [&](int k) {
    const uint32_t gbase = (uint32_t)(((int64_t)tile_of(k) * BM + cw * QROWS) * 27 * 4);
#pragma unroll
    for (int d = 0; d < QDMA; ++d) {
      const uint32_t blk = (uint32_t)(d * 1024);
      const uint32_t off = blk + (uint32_t)lane * 16u;
      lds_dma16(rsrc_n, off < (uint32_t)(QROWS * 27 * 4) ? gbase + off : kOutOfRange,
                lds_offset(s_nbr) + (uint32_t)(cw_u * QDMA * 1024) + blk);
    }
  };
  // The load waves start on tile 0's rows now, under the tap-mask pass below.
  if (loader) issue_rows(0);
  using T = typename Elem<D>::T;
  if (tid < BN) {
    const int o = o0 + tid;
    s_bias[tid] = (args.bias != nullptr && o < cout) ? to_float<D>(reinterpret_cast<const T*>(args.bias)[o]) : 0.f;
  }
  for (int k = tid; k < ntiles; k += NT) s_tmask[k] = 0;
  __syncthreads();
  // Tap masks of all tiles: OR of the rows' neighbour masks, eight independent loads in flight.
  // BM is a multiple of 64, so the 64 consecutive rows of a wave's load lie in one tile: OR them
  // across the wave, then one LDS atomic per wave and load.
  static_assert(BM % 64 == 0, "a wave's rows lie in one tile");
  for (int idx0 = tid; idx0 < ntiles * BM; idx0 += 8 * NT) {
    uint32_t m[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = idx0 + u * NT;
      const int k = idx / BM;
      const int64_t row = (int64_t)tile_of(k < ntiles ? k : 0) * BM + (idx - k * BM);
      const bool ok = idx < ntiles * BM && row < n;
      m[u] = ok ? masks_w[row] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      uint32_t v = m[u];
      for (int off = 32; off > 0; off >>= 1) v |= __shfl_xor(v, off, 64);
      const int k = (idx0 + u * NT) / BM;
      if (lane == 0 && v != 0u) atomicOr(&s_tmask[k], v);
    }
  }
  __syncthreads();
  const int nq = (row_bytes + SL - 1) / SL;
  int total = 0;  // stages of the whole workgroup, identical in every wave
  for (int k = 0; k < ntiles; ++k) total += __builtin_popcount(s_tmask[k]) * nq;

  auto swz_of = [](int row) { return (row / (16 / CH)) % CH; };

  if (loader) {
    // Load waves issue ahead of the compute waves on their SIMD (measured 1-3 % faster; raising
    // the compute waves instead changes nothing).
    __builtin_amdgcn_s_setprio(2);
    auto chunk_bytes = [&](int group_row) {
      return (uint32_t)(((lane % CH) ^ swz_of(group_row + lane / CH)) * 16);
    };
    const i32x4_t rsrc_a = make_rsrc(args.feats, args.feats_bytes);
    const i32x4_t rsrc_b = make_rsrc(args.weight, args.weight_bytes);
    int32_t* my_nbr = s_nbr + cw * (QDMA * 256);
    uint32_t lane_cb[DMA], base_b[BDMA];
    bool ok_b[BDMA];
#pragma unroll
    for (int d = 0; d < ADMA; ++d) lane_cb[d] = chunk_bytes(cw * QROWS + RPI * d);
#pragma unroll
    for (int d = 0; d < BDMA; ++d) {
      const int g = BM + cw * (BNP / LW) + RPI * d;
      const int ol = g - BM + lane / CH;
      const int o = o0 + ol;
      lane_cb[ADMA + d] = chunk_bytes(g);
      ok_b[d] = ol < BN && o < cout;
      base_b[d] = (uint32_t)(ok_b[d] ? o : 0) * 27u * (uint32_t)row_bytes + lane_cb[ADMA + d];
    }
    bool row_ok[ADMA];
    // At a tile change the wait for the rows also drains the ring loads in flight, which have to
    // land anyway; prefetching the rows one stage earlier, with waits that leave them in flight,
    // measured 3-6 % slower.
    auto rows_landed = [&](int k) {
      const int64_t r0 = (int64_t)tile_of(k) * BM + cw * QROWS;
#pragma unroll
      for (int d = 0; d < ADMA; ++d) row_ok[d] = r0 + RPI * d + lane / CH < n;
      wait_vmcnt<0>();
      compiler_fence();
    };
    int ck = 0;  // tile of the fetch cursor
    uint32_t rem = s_tmask[0];
    int ik = 0, iq = nq;
    int pk = 0, pq = 0;
    bool pvalid = false;
    int32_t raw[ADMA];
    uint32_t offs[DMA];
    rows_landed(0);  // (issued before the tap-mask pass)
    auto fetch = [&](int stage_index) {
      pvalid = stage_index < total;
      if (pvalid && iq >= nq && rem == 0u) {  // this tile's stages are done: next tile with taps
        do {
          ++ck;
          rem = s_tmask[ck];
        } while (rem == 0u && ck + 1 < ntiles);
        compiler_fence();  // the last rows of the previous tile have been read
        issue_rows(ck);
        rows_landed(ck);
      }
      const bool adv = pvalid && iq >= nq;
      const int nk = __builtin_ctz(rem | 0x80000000u);
      ik = adv ? nk : ik;
      rem = adv ? (rem & (rem - 1)) : rem;
      iq = adv ? 0 : iq;
      pk = ik;
      pq = iq;
      iq += pvalid ? 1 : 0;
#pragma unroll
      for (int d = 0; d < ADMA; ++d) raw[d] = my_nbr[(RPI * d + lane / CH) * 27 + pk];
    };
    auto make = [&]() {
      const uint32_t sq = (uint32_t)(pq * SL);
      const uint32_t sb = (uint32_t)pk * (uint32_t)row_bytes + sq;
      const int limit = pvalid ? row_bytes - (int)sq : 0;
#pragma unroll
      for (int d = 0; d < ADMA; ++d) {
        const uint32_t o = (uint32_t)raw[d] * (uint32_t)row_bytes + sq + lane_cb[d];
        const bool use = (raw[d] >= 0) & row_ok[d] & ((int)lane_cb[d] < limit);
        offs[d] = use ? o : kOutOfRange;
      }
#pragma unroll
      for (int d = 0; d < BDMA; ++d) {
        const bool use = ok_b[d] & ((int)lane_cb[ADMA + d] < limit);
        offs[ADMA + d] = use ? base_b[d] + sb : kOutOfRange;
      }
    };
    auto issue = [&](unsigned char* base) {
#pragma unroll
      for (int d = 0; d < ADMA; ++d)
        lds_dma16(rsrc_a, offs[d], lds_offset(base) + (uint32_t)((cw_u * QROWS + RPI * d) * SL));
#pragma unroll
      for (int d = 0; d < BDMA; ++d)
        lds_dma16(rsrc_b, offs[ADMA + d], lds_offset(base) + (uint32_t)((BM + cw_u * (BNP / LW) + RPI * d) * SL));
    };
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0) {
      fetch(s0);
      make();
      issue(ring + s0 * BUF);
    }
    fetch(NS);
    wait_vmcnt<(NS - 1) * DMA>();
    barrier_no_fence();
    int slot = 0;
    for (int st = 0; st < total; ++st) {
      // Barrier st: this wave's loads of stage st + 1 have landed; afterwards slot st is free.
      wait_vmcnt<(NS - 2) * DMA>();
      barrier_no_fence();
      make();
      issue(ring + slot * BUF);
      fetch(st + NS + 1);
      slot = slot + 1 == NS ? 0 : slot + 1;
    }
    wait_vmcnt<0>();
  } else {
    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    const int lrow = lane & 31;
    const int lk = lane >> 5;
    const int swz = swz_of(lrow);
    uint4 ga[2][FM], gb[2][FN];
    auto read_step = [&](auto P, auto KK, const unsigned char* buf) {
      constexpr int p = decltype(P)::value, kk = decltype(KK)::value;
      const int off = ((2 * kk + lk) ^ swz) << 4;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        ga[p][i] = *reinterpret_cast<const uint4*>(buf + (wm * WTM + i * 32 + lrow) * SL + off);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        gb[p][j] = *reinterpret_cast<const uint4*>(buf + (BM + wn * WTN + j * 32 + lrow) * SL + off);
    };
    auto mul_step = [&](auto P) {
      constexpr int p = decltype(P)::value;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<D>(gb[p][j], ga[p][i], acc[i][j]);
    };
    auto interleave_step = [&]() {
#pragma unroll
      for (int g = 0; g < FM * FN; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
      }
    };
    auto inner = [&](auto KK, const unsigned char* cur) {
      constexpr int kk = decltype(KK)::value;
      if constexpr (kk < KSTEPS - 1) {
        __builtin_amdgcn_sched_barrier(0);
        read_step(IC<(kk + 1) & 1>{}, IC<kk + 1>{}, cur);
        mul_step(IC<kk & 1>{});
        interleave_step();
      }
    };
    // Finished tile: + bias, one rounding, each lane's four consecutive channels as 8 bytes.
    T* out = reinterpret_cast<T*>(args.out);
    auto write_tile = [&](int k) {
      const int64_t row0 = (int64_t)tile_of(k) * BM;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t row = row0 + wm * WTM + i * 32 + lrow;
        const int64_t orow = (rows_w != nullptr && row < n) ? (int64_t)rows_w[row] : row;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = wn * WTN + j * 32 + 8 * g + 4 * lk;
            const float4 bb = *reinterpret_cast<const float4*>(s_bias + c);
            if (row < n && o0 + c < cout)
              *reinterpret_cast<uint2*>(out + orow * cout + o0 + c) =
                  pack4<D>(acc[i][j][4 * g] + bb.x, acc[i][j][4 * g + 1] + bb.y, acc[i][j][4 * g + 2] + bb.z,
                           acc[i][j][4 * g + 3] + bb.w);
            acc[i][j][4 * g] = acc[i][j][4 * g + 1] = acc[i][j][4 * g + 2] = acc[i][j][4 * g + 3] = 0.f;
          }
      }
    };
    int k = 0;
    int left = __builtin_popcount(s_tmask[0]) * nq;  // stages left in tile k
    // A tile with no taps (no valid row: not produced by the tiling, kept for safety) is bias only.
    auto next_tiles = [&]() {
      while (left == 0 && k < ntiles) {
        write_tile(k);
        ++k;
        left = k < ntiles ? __builtin_popcount(s_tmask[k]) * nq : 0;
      }
    };
    next_tiles();
    barrier_no_fence();  // stage 0 has landed
    read_step(IC<0>{}, IC<0>{}, ring);
    int slot = 0;
    for (int st = 0; st < total; ++st) {
      const unsigned char* cur = ring + slot * BUF;
      const int next_slot = slot + 1 == NS ? 0 : slot + 1;
      inner(IC<0>{}, cur);
      inner(IC<1>{}, cur);
      inner(IC<2>{}, cur);
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkmcnt0();
      barrier_no_fence();  // barrier st: stage st + 1 in LDS; this wave is done with slot st
      __builtin_amdgcn_sched_barrier(0);
      read_step(IC<KSTEPS & 1>{}, IC<0>{}, ring + next_slot * BUF);
      mul_step(IC<(KSTEPS - 1) & 1>{});
      interleave_step();
      slot = next_slot;
      if (--left == 0) {
        __builtin_amdgcn_sched_barrier(0);
        next_tiles();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <DT D, int WM, int FM, int FN, int SL, int TAPS, int KP = 0, bool STATS = false>
hipError_t launch_ws(const ConvArgs& a0, hipStream_t stream) {
  using Sh = MmaShape<WM, FM, FN, SL, TAPS>;
  ConvArgs a = a0;
  a.tiles_m = (int)((a.n + Sh::BM - 1) / Sh::BM);
  a.per_xcd = (a.tiles_m + 7) / 8;
  dim3 grid((unsigned)(8 * a.per_xcd), (unsigned)((a.cout + Sh::BN - 1) / Sh::BN));
  launch_kernel_timed(subm_conv_ws_kernel<D, WM, FM, FN, SL, TAPS, KP, STATS>, grid, dim3(kWsThreads), stream, a);
  return hipGetLastError();
}

template <DT D, int WM, int FM, int FN, int SL, int TAPS>
hipError_t launch_mma(const ConvArgs& a0, hipStream_t stream) {
  using Sh = MmaShape<WM, FM, FN, SL, TAPS>;
  ConvArgs a = a0;
  a.tiles_m = (int)((a.n + Sh::BM - 1) / Sh::BM);
  a.per_xcd = (a.tiles_m + 7) / 8;
  dim3 grid((unsigned)(8 * a.per_xcd), (unsigned)((a.cout + Sh::BN - 1) / Sh::BN));
  launch_kernel_timed(subm_conv_mma_kernel<D, WM, FM, FN, SL, TAPS>, grid, dim3(kThreads), stream, a);
  return hipGetLastError();
}

// Persistent launch: one workgroup per compute unit (a multiple of 8, for the XCD mapping), each
// walking its tiles.  hipErrorNotSupported when a workgroup would get more than kMaxBlockTiles
// tiles or the output rows cannot take 8-byte stores (the caller then uses launch_ws).
template <DT D, int WM, int FM, int FN, int SL, int LW>
hipError_t launch_ws_persistent(const ConvArgs& a0, hipStream_t stream) {
  using Sh = MmaShape<WM, FM, FN, SL, 27>;
  ConvArgs a = a0;
  a.tiles_m = (int)((a.n + Sh::BM - 1) / Sh::BM);
  a.per_xcd = (a.tiles_m + 7) / 8;
  const int nblk = std::min(kPersistentBlocks, 8 * a.per_xcd);
  const int per_block = (a.per_xcd + nblk / 8 - 1) / (nblk / 8);
  if (per_block > kMaxBlockTiles || !a.vec_out || a.cout % 8 != 0) return hipErrorNotSupported;
  dim3 grid((unsigned)nblk, (unsigned)((a.cout + Sh::BN - 1) / Sh::BN));
  launch_kernel_timed(subm_conv_ws_persistent_kernel<D, WM, FM, FN, SL, LW>, grid, dim3(64 * (4 + LW)), stream, a);
  return hipGetLastError();
}

// Tile configurations of the matrix-core kernel: waves along rows, row blocks and column blocks
// per wave, stage slice bytes.
struct MmaTile {
  const char* name;
  int wm, fm, fn, sl;
};
constexpr MmaTile kTiles[] = {
    // 128 output channels per tile
    {"r192c128s128", 2, 3, 2, 128}, {"r192c128s64", 2, 3, 2, 64}, {"r128c128s64", 2, 2, 2, 64},
    {"r256c128s64", 2, 4, 2, 64},   {"r384c128s64", 4, 3, 4, 64}, {"r256c128s128", 2, 4, 2, 128},
    // 64 output channels per tile
    {"r192c64s128", 2, 3, 1, 128},  {"r256c64s64", 4, 2, 2, 64},  {"r384c64s64", 4, 3, 2, 64},
    {"r128c64s64", 2, 2, 1, 64},
    // 32 output channels per tile
    {"r256c32s64", 4, 2, 1, 64},    {"r128c32s64", 4, 1, 1, 64},
    // warp-specialised (separate load waves)
    {"ws256c128s64", 4, 2, 4, 64},  {"ws192c128s64", 2, 3, 2, 64}, {"ws256c128s64b", 2, 4, 2, 64},
    {"ws384c64s64", 4, 3, 2, 64},   {"ws512c64s64", 4, 4, 2, 64},
    // warp-specialised, fragments one step ahead
    {"ws192c128s128k", 2, 3, 2, 128}, {"ws192c128s64k", 2, 3, 2, 64}, {"ws256c64s128k", 4, 2, 2, 128},
    {"ws192c64s128k", 2, 3, 1, 128},
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

template <DT D, int TAPS>
hipError_t launch_tile_index(int t, const ConvArgs& a, hipStream_t stream) {
  switch (t) {
    case 0: return launch_mma<D, 2, 3, 2, 128, TAPS>(a, stream);
    case 1: return launch_mma<D, 2, 3, 2, 64, TAPS>(a, stream);
    case 2: return launch_mma<D, 2, 2, 2, 64, TAPS>(a, stream);
    case 3: return launch_mma<D, 2, 4, 2, 64, TAPS>(a, stream);
    case 4: return launch_mma<D, 4, 3, 4, 64, TAPS>(a, stream);
    case 5: return launch_mma<D, 2, 4, 2, 128, TAPS>(a, stream);
    case 6: return launch_mma<D, 2, 3, 1, 128, TAPS>(a, stream);
    case 7: return launch_mma<D, 4, 2, 2, 64, TAPS>(a, stream);
    case 8: return launch_mma<D, 4, 3, 2, 64, TAPS>(a, stream);
    case 9: return launch_mma<D, 2, 2, 1, 64, TAPS>(a, stream);
    case 10: return launch_mma<D, 4, 2, 1, 64, TAPS>(a, stream);
    case 11: return launch_mma<D, 4, 1, 1, 64, TAPS>(a, stream);
    case 12: return launch_ws<D, 4, 2, 4, 64, TAPS>(a, stream);
    case 13: return launch_ws<D, 2, 3, 2, 64, TAPS>(a, stream);
    case 14: return launch_ws<D, 2, 4, 2, 64, TAPS>(a, stream);
    case 15: return launch_ws<D, 4, 3, 2, 64, TAPS>(a, stream);
    case 16: return launch_ws<D, 4, 4, 2, 64, TAPS>(a, stream);
    case 17: return launch_ws<D, 2, 3, 2, 128, TAPS, 1>(a, stream);
    case 18: return launch_ws<D, 2, 3, 2, 64, TAPS, 1>(a, stream);
    case 19: return launch_ws<D, 4, 2, 2, 128, TAPS, 1>(a, stream);
    default: return launch_ws<D, 2, 3, 1, 128, TAPS, 1>(a, stream);
  }
}

// Tile choice (bf16 on the shell, dense, ellipsoid and subdivided workloads, all tiles measured
// side by side): above 64 output channels the warp-specialised 192 x 128 tile with 128-byte
// slices and step-ahead fragments is fastest on every workload; from 33 to 64 channels the
// 256 x 64 tile of the same kind.  Up to 32 channels, a 256-row tile when it saves rounds of
// tiles over the 256 compute units.
constexpr int kComputeUnits = 256;
constexpr bool persistent_enabled_default = true;
// SUBMCONV_PERSISTENT=0 selects the one-tile-per-workgroup launch, =1 the persistent walk even for
// the small sets that otherwise take a smaller one-tile launch (timing and tests).
inline bool persistent_enabled() {
  const char* v = std::getenv("SUBMCONV_PERSISTENT");
  return v == nullptr ? persistent_enabled_default : v[0] != '0';
}
inline bool persistent_forced() {
  const char* v = std::getenv("SUBMCONV_PERSISTENT");
  return v != nullptr && v[0] == '1';
}
// Sets of at most this many rows with 33..64 output channels fill at most half the CUs with
// 256-row tiles: a smaller one-tile launch spreads them wider (64^3 shell and torus, 22,406 rows:
// k = 3 17.2 us with 192-row tiles against 20.4 us for the persistent walk; k = 1 5.0 us with
// 128-row tiles against 6.3 us).
constexpr int64_t kSmallSetRows = 32768;
inline int64_t launch_rounds(int64_t n, int cout, int bm, int bn) {
  const int64_t tiles = (n + bm - 1) / bm * ((cout + bn - 1) / bn);
  return (tiles + kComputeUnits - 1) / kComputeUnits;
}

int tile_index(const char* name) {
  for (int t = 0; t < kNumTiles; ++t)
    if (std::strcmp(name, kTiles[t].name) == 0) return t;
  return -1;
}

template <DT D, int TAPS>
hipError_t launch_mma_auto(const ConvArgs& a, hipStream_t stream) {
  int best;
  const char* forced = std::getenv("SUBMCONV_TILE");
  const bool small64 = a.cout > 32 && a.cout <= 64 && a.n <= kSmallSetRows && !persistent_forced();
  if (TAPS == 27 && a.cout > 32 && !small64 && (forced == nullptr || tile_index(forced) < 0) && persistent_enabled()) {
    // the persistent walk of the same tiles the one-tile launch below would use
    // eight load waves: 2-3 % faster than four on the shell, dense, ellipsoid and subdivided
    // workloads, same outputs
    const hipError_t e = a.cout > 64 ? launch_ws_persistent<D, 2, 3, 2, 128, 8>(a, stream)
                                     : launch_ws_persistent<D, 4, 2, 2, 128, 8>(a, stream);
    if (e != hipErrorNotSupported) return e;
  }
  if (small64) {
    best = tile_index(TAPS == 27 ? "ws192c64s128k" : "r128c64s64");
  } else if (a.cout > 64) {
    best = tile_index("ws192c128s128k");
  } else if (a.cout > 32) {
    best = tile_index("ws256c64s128k");
  } else {
    const int64_t r128 = launch_rounds(a.n, a.cout, 128, 32);
    const int64_t r256 = launch_rounds(a.n, a.cout, 256, 32);
    best = tile_index(2 * r256 <= r128 + 1 ? "r256c32s64" : "r128c32s64");
  }
  // SUBMCONV_TILE=<name> forces a tile configuration (tuning and tests).
  if (const char* env = std::getenv("SUBMCONV_TILE")) {
    const int t = tile_index(env);
    if (t >= 0) best = t;
  }
  return launch_tile_index<D, TAPS>(best, a, stream);
}

template <DT D, int BM, int BN, int WM, bool VEC, int TAPS>
hipError_t launch_tile(const ConvArgs& a0, hipStream_t stream) {
  ConvArgs a = a0;
  a.tiles_m = (int)((a.n + BM - 1) / BM);
  a.per_xcd = (a.tiles_m + 7) / 8;
  dim3 grid((unsigned)(8 * a.per_xcd), (unsigned)((a.cout + BN - 1) / BN));
  launch_kernel_timed(subm_conv_generic_kernel<D, BM, BN, WM, VEC, TAPS>, grid, dim3(kThreads), stream, a);
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
      return taps == 27 ? launch_mma_auto<D, 27>(a, stream) : launch_mma_auto<D, 1>(a, stream);
    }
  }
  if (taps == 27) return vec_in ? launch_shape<D, true, 27>(a, stream) : launch_shape<D, false, 27>(a, stream);
  return vec_in ? launch_shape<D, true, 1>(a, stream) : launch_shape<D, false, 1>(a, stream);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
constexpr uint64_t kOffsetLimit = 0x7FFFF000ull;  // below kOutOfRange with room for a row slice

}  // namespace

// Convolution whose epilogue also writes group-norm partial sums per (row tile, group).  Taken
// only on the warp-specialised 16-bit fast path with groups that do not straddle column tiles;
// otherwise returns hipErrorNotSupported and writes nothing (the caller runs the plain
// convolution and a separate statistics pass).  *tile_rows receives the row-tile height.
hipError_t launch_subm_conv_gn_partials(const MapData* map, int64_t n, int ksize, int cin, int cout, int dtype,
                                        const void* feats, const void* weight, const void* bias, void* out,
                                        float2* part, int cpg, int groups, int* tile_rows, hipStream_t stream) {
  if (dtype == SUBM_F32 || cout <= 32) return hipErrorNotSupported;
  ConvArgs a{};
  a.feats = feats;
  a.weight = weight;
  a.bias = bias;
  a.out = out;
  a.nbr = ksize == 3 ? map->nbr : nullptr;
  a.masks = ksize == 3 ? map->masks : nullptr;
  a.n = n;
  a.cin = cin;
  a.cout = cout;
  a.row_bytes = cin * 2;
  a.vec_out = ((cout * 2) % 16 == 0) && aligned16(out);
  const bool vec_in = (a.row_bytes % 16 == 0) && aligned16(feats) && aligned16(weight);
  const int taps = ksize == 3 ? 27 : 1;
  const uint64_t fb = (uint64_t)n * (uint64_t)a.row_bytes;
  const uint64_t wb = (uint64_t)cout * (uint64_t)taps * (uint64_t)a.row_bytes;
  const uint64_t nb = ksize == 3 ? (uint64_t)n * 27u * 4u : 0u;
  if (!vec_in || fb >= kOffsetLimit || nb >= kOffsetLimit || wb >= kOffsetLimit) return hipErrorNotSupported;
  a.feats_bytes = (uint32_t)fb;
  a.weight_bytes = (uint32_t)wb;
  a.gn_part = part;
  a.gn_cpg = cpg;
  a.gn_groups = groups;
  const bool wide = cout > 64;  // the tiles launch_mma_auto picks: 192 x 128 above 64 channels, 256 x 64 below
  const int bn = wide ? 128 : 64;
  if (bn % cpg != 0) return hipErrorNotSupported;
  *tile_rows = wide ? 192 : 256;
  if (dtype == SUBM_F16) {
    if (taps == 27) return wide ? launch_ws<DT::F16, 2, 3, 2, 128, 27, 1, true>(a, stream) : launch_ws<DT::F16, 4, 2, 2, 128, 27, 1, true>(a, stream);
    return wide ? launch_ws<DT::F16, 2, 3, 2, 128, 1, 1, true>(a, stream) : launch_ws<DT::F16, 4, 2, 2, 128, 1, 1, true>(a, stream);
  }
  if (taps == 27) return wide ? launch_ws<DT::BF16, 2, 3, 2, 128, 27, 1, true>(a, stream) : launch_ws<DT::BF16, 4, 2, 2, 128, 27, 1, true>(a, stream);
  return wide ? launch_ws<DT::BF16, 2, 3, 2, 128, 1, 1, true>(a, stream) : launch_ws<DT::BF16, 4, 2, 2, 128, 1, 1, true>(a, stream);
}

hipError_t launch_subm_conv(const MapData* map, int64_t n, int ksize, int cin, int cout, int dtype,
                            const void* feats, const void* weight, const void* bias, void* out,
                            hipStream_t stream, const uint32_t* gate, int gate_n) {
  const int s = dtype == SUBM_F32 ? 4 : 2;
  ConvArgs a{};
  a.feats = feats;
  a.weight = weight;
  a.bias = bias;
  a.out = out;
  a.nbr = ksize == 3 ? map->nbr : nullptr;
  a.masks = ksize == 3 ? map->masks : nullptr;
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
  // The rulebook rows are copied with 32-bit byte offsets too (n x 27 int32).
  const uint64_t nb = ksize == 3 ? (uint64_t)n * 27u * 4u : 0u;
  a.feats_bytes = (fb < kOffsetLimit && nb < kOffsetLimit) ? (uint32_t)fb : 0u;
  a.weight_bytes = wb < kOffsetLimit ? (uint32_t)wb : 0u;
  a.gate = gate;
  a.gate_n = gate_n;
  if (ksize == 3 && map->order_block != nullptr && stream == map->order_stream) {
    const OrderView v = order_view(map->order_block, map->n);
    a.order_gate = v.gate;
    a.order_rows = v.rows;
    a.order_nbr = v.nbr;
    a.order_masks = v.masks;
  }
  switch (dtype) {
    case SUBM_F32: return launch_dtype<DT::F32>(a, vec_in, taps, stream);
    case SUBM_F16: return launch_dtype<DT::F16>(a, vec_in, taps, stream);
    default: return launch_dtype<DT::BF16>(a, vec_in, taps, stream);
  }
}

}  // namespace submconv
