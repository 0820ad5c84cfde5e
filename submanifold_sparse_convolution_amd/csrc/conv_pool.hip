// Neighbour-pool submanifold convolution for 128 output channels, 16-bit storage, gfx950.
//
//   out[i, o] = bias[o] + sum_{k : nbr[i,k] >= 0} sum_c W[o, k, c] * f[nbr[i,k], c]
//
// (lato.2_mrp_mlx README, header summary and "Correctness": KRSC weights, features gathered at
// coord_i + d.)  The same sum as the kernels of conv.hip, computed in a different order of
// memory traffic.
//
// Design.  A workgroup (eight waves, two per SIMD) owns a tile of 16 or 17 row blocks of 32
// consecutive rows and all 128 output channels; each wave keeps a 64-row x 128-channel block of
// fp32 accumulators (two row blocks x four output blocks; the seventeenth row block, when there is
// one, is shared by waves 0..3, each holding its 32-channel quarter).  The rows that the tile's
// rows reach through the nine taps of one dz (the tile's "sub-pool" for that dz: at most 768
// distinct rows on every workload measured, and sorted by row) are gathered ONCE per 32-channel
// slice into LDS and read by all nine taps, instead of being gathered again for every tap: the
// tile's rows reach about 3.1 distinct rows each on the 128^3 shell, against 20.9 gathered per
// row tap by tap.  A plan, built once per map by pool_plan_kernel, lists each sub-pool's rows and,
// for every (tap, row), the LDS slot of its neighbour (a zero row when it is absent).
//
// The reduction runs over steps (slice q of 32 input channels, dz, the nine (dy, dx) taps): per
// step a wave issues 2 x 8 (or 9) v_mfma_f32_32x32x16 (weights as operand A from a 6-slot LDS
// ring of half-steps, neighbour rows as operand B from the sub-pool), one barrier, and its share
// of the loads that run ahead: a quarter of a weight half-step three steps ahead (weights are
// pre-packed so that a half-step is one contiguous 4 KB block), a quarter of one slot-table tap
// four steps ahead (waves 0..3), one direct-to-LDS gather of the next sub-pool (steps 0..5 of each
// nine) and, once per sub-pool, an eighth of one group of row ids.  With two waves per SIMD one
// wave's MFMAs cover the other's waits for LDS reads (measured 1.6 % faster on the shell and 3 %
// on the dense grid than one wave per SIMD holding twice the rows).  A finished tile is rounded
// (one RNE conversion after + bias in fp32) and written through LDS as whole 256-byte rows.
//
// LDS (162,112 bytes): two sub-pool buffers of 769 x 64 bytes (slot 768 is a zero row), the
// weight ring, the slot table of the current tile, three groups of row ids, the bias.
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace submconv {
namespace {

constexpr int kPT = 256;        // threads of one plan group (the plan kernel runs three)
constexpr int kCT = 512;        // threads of the convolution: eight waves, two per SIMD
constexpr int kSL = 64;         // bytes of a row per slice (32 channels)
constexpr int kWH = 128 * 32;   // a weight half-step: 128 output channels x 16 input channels
constexpr int kWS = 6;          // weight half-steps held in LDS
constexpr int kUcap = 768;      // rows per sub-pool

template <int E>
struct PoolShape {
  static constexpr int NBLK = 16 + E;             // row blocks of 32 per tile
  static constexpr int TAPB = NBLK * 64;          // slot table bytes per tap (u16 per row)
  static constexpr int TABB = 27 * TAPB;
  static constexpr int WSLOTS = kUcap / 8;        // pool slots gathered by one wave (of eight)
  static constexpr int NJ = kUcap / 128;          // gather loads per wave per sub-pool
  static constexpr int IDB = kUcap * 4;           // row ids of one dz group
  static constexpr int RECB = TABB + 3 * IDB;     // plan record of one tile
  static constexpr int POOLB = (kUcap + 1) * kSL; // one sub-pool buffer, zero slot last
  static constexpr int O_W = 2 * POOLB;
  static constexpr int O_TAB = O_W + kWS * kWH;
  static constexpr int O_IDS = O_TAB + TABB;
  static constexpr int O_BIAS = O_IDS + 3 * IDB;
  static constexpr int LDSB = O_BIAS + 128 * 4;
  static_assert(kUcap % 64 == 0 && WSLOTS % 16 == 0, "whole gather loads per wave");
  static_assert(LDSB <= 160 * 1024, "LDS");
  static_assert((TAPB / 4) % 16 == 0 && (IDB / 8) % 16 == 0, "refills in whole 16-byte lanes");
  static_assert(NJ == 6, "the load schedule assumes 6 gathers per wave per sub-pool");
  static_assert(RECB % 16 == 0, "records in whole 16-byte chunks");
};

// Byte offset of pool slot s in a sub-pool buffer, with the 16-byte chunk index XOR-swizzled by
// (s >> 1) & 3.  Of the swizzles measured for one operand-B read (32 lanes of slots, one 16-byte
// chunk each), this one read fastest both for consecutive slots and for runs broken by gaps.
__host__ __device__ constexpr uint32_t slot_offset(uint32_t s) { return s * kSL + (((s >> 1) & 3u) << 4); }

// ------------------------------------------------------------------------------------------
// Plan: one workgroup of three 256-thread groups per tile, group g handling dz = g.  The tile's
// rulebook rows are read once with coalesced loads and transposed through LDS, so that a thread
// holds the nine entries of two adjacent rows in registers.  Per group, the distinct rows
// nbr[i, 9 dz + j] >= 0 of the tile's rows i are marked in a byte array over [lo, hi] (plain
// stores: many rows mark the same neighbour), turned into a bitmap with prefix counts, and ranked;
// the record gets the rows (in the order the gather lanes load them) and the slot table of the
// nine taps (byte offsets of the slots, slot 768 = the zero row for absent neighbours and rows
// past the tile).  A sub-pool beyond 768 rows or a range beyond 16,384 rows sets the (tile, dz)
// flag (flags[3 tile + dz] = 1, else 0) and stores 1 into *host_flag (zeroed by the host).  The
// marks reuse the staging area; 71 KB of LDS lets two workgroups share a compute unit.  nbr must
// be 16-byte aligned.
constexpr int kMarkBytes = 16384;
template <int E>
struct PlanShape {
  static constexpr int R = PoolShape<E>::NBLK * 32;
  static constexpr int STAGEB = R * 27 * 4;
  static constexpr int MARKB = 3 * kMarkBytes;
  static constexpr int AREAB = STAGEB > MARKB ? STAGEB : MARKB;
};
template <int E>
__global__ __launch_bounds__(3 * kPT, 2) void pool_plan_kernel(const int32_t* __restrict__ nbr, int64_t n, int nb,
                                                               int ntiles, unsigned char* __restrict__ plan,
                                                               uint32_t* __restrict__ flags, uint32_t* host_flag) {
  using P = PoolShape<E>;
  constexpr int R = P::NBLK * 32;
  constexpr int NW = kMarkBytes / 32;  // bitmap words per group
  __shared__ __align__(16) unsigned char area[PlanShape<E>::AREAB];
  __shared__ uint2 bits[3][NW];  // (bitmap word, exclusive prefix count)
  __shared__ int s_red[3][8];
  __shared__ uint32_t s_part[3][4];
  const int g = threadIdx.x >> 8, tid = threadIdx.x & 255, lane = tid & 63, wv = tid >> 6;
  const int dz = g;
  const int tile = (int)blockIdx.x;
  const int blk0 = (int)((int64_t)tile * nb / ntiles);
  const int blk1 = (int)((int64_t)(tile + 1) * nb / ntiles);
  const int64_t r0 = (int64_t)blk0 * 32;
  const int rows = (int)min((int64_t)(blk1 - blk0) * 32, n - r0);
  unsigned char* rec = plan + (size_t)tile * P::RECB;
  uint32_t* tab2 = reinterpret_cast<uint32_t*>(rec) + 9 * dz * (R / 2);  // slot offsets, two rows per word
  int32_t* idz = reinterpret_cast<int32_t*>(rec + P::TABB) + dz * kUcap;
  // 0. the tile's rulebook rows [rows][27], read with coalesced 16-byte loads (a tile starts at a
  //    multiple of 32 rows, 3,456 bytes) into LDS
  int32_t* stage = reinterpret_cast<int32_t*>(area);
  {
    const int nel = rows * 27;
    const int4* blk = reinterpret_cast<const int4*>(nbr + r0 * 27);
    constexpr int NV = (R * 27 / 4 + 3 * kPT - 1) / (3 * kPT);
    int4 x[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = (int)threadIdx.x + 3 * kPT * i;
      if (4 * v + 3 < nel) {
        x[i] = blk[v];
      } else {
        const int32_t* e = reinterpret_cast<const int32_t*>(blk) + 4 * v;
        x[i] = make_int4(4 * v < nel ? e[0] : -1, 4 * v + 1 < nel ? e[1] : -1, 4 * v + 2 < nel ? e[2] : -1,
                         4 * v + 3 < nel ? e[3] : -1);
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = (int)threadIdx.x + 3 * kPT * i;
      if (4 * v < R * 27) reinterpret_cast<int4*>(stage)[v] = x[i];
    }
  }
  __syncthreads();
  // this thread's rows 2 tid + h + 512 u, the nine entries of its dz
  constexpr int RU = (R + 2 * kPT - 1) / (2 * kPT);
  int nb9[RU][2][9];
#pragma unroll
  for (int u = 0; u < RU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 2 * tid + h + 2 * kPT * u;
#pragma unroll
      for (int j = 0; j < 9; ++j) nb9[u][h][j] = r < rows ? stage[r * 27 + 9 * dz + j] : -1;
    }
  // 1. range of the neighbour rows
  int lo = INT32_MAX, hi = -1;
#pragma unroll
  for (int u = 0; u < RU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        const int v = nb9[u][h][j];
        if (v >= 0) {
          lo = min(lo, v);
          hi = max(hi, v);
        }
      }
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, __shfl_xor(lo, off, 64));
    hi = max(hi, __shfl_xor(hi, off, 64));
  }
  if (lane == 0) {
    s_red[g][wv] = lo;
    s_red[g][4 + wv] = hi;
  }
  __syncthreads();  // (also: every group has read the staging area, which the marks reuse)
  lo = min(min(s_red[g][0], s_red[g][1]), min(s_red[g][2], s_red[g][3]));
  hi = max(max(s_red[g][4], s_red[g][5]), max(s_red[g][6], s_red[g][7]));
  const int64_t range = hi >= lo ? (int64_t)hi - lo + 1 : 0;
  const bool fits = range <= kMarkBytes;
  bool bad = !fits;
  const int nw = fits ? (int)((range + 31) / 32) : 0;  // bitmap words
  unsigned char* mark = area + g * kMarkBytes;
  // 2. marks of the rows present
  for (int k = tid; k < nw * 8; k += kPT) reinterpret_cast<uint32_t*>(mark)[k] = 0u;
  __syncthreads();
  if (fits) {
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 9; ++j) {
          const int v = nb9[u][h][j];
          if (v >= 0) mark[v - lo] = 1;
        }
  }
  __syncthreads();
  // 3. bitmap words and their exclusive prefix counts (each thread owns a run of words)
  const int per = (nw + kPT - 1) / kPT;
  const int k0 = min(nw, tid * per), k1 = min(nw, (tid + 1) * per);
  uint32_t cnt = 0;
  for (int k = k0; k < k1; ++k) {
    const uint4 x = reinterpret_cast<const uint4*>(mark)[2 * k];
    const uint4 y = reinterpret_cast<const uint4*>(mark)[2 * k + 1];
    const uint32_t m8[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    uint32_t word = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t m = m8[u];  // four mark bytes, 0 or 1 each
      word |= ((m & 1u) | ((m >> 7) & 2u) | ((m >> 14) & 4u) | ((m >> 21) & 8u)) << (4 * u);
    }
    bits[g][k].x = word;
    cnt += __popc(word);
  }
  uint32_t incl = cnt;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_part[g][wv] = incl;
  __syncthreads();
  {
    uint32_t c = incl - cnt;
    for (int k = 0; k < wv; ++k) c += s_part[g][k];
    for (int k = k0; k < k1; ++k) {
      bits[g][k].y = c;
      c += __popc(bits[g][k].x);
    }
  }
  const uint32_t total = s_part[g][0] + s_part[g][1] + s_part[g][2] + s_part[g][3];
  bad |= total > (uint32_t)kUcap;
  __syncthreads();
  // 4. rows by rank into LDS (the marks are dead), one bit per lane: a wave takes two words at a
  //    time; then the ids in gather order: slot c is loaded by wave c / 192, load (c % 192) / 16,
  //    lane group c % 16, and the ids of a lane group are contiguous; unused slots hold -1
  int32_t* by_rank = reinterpret_cast<int32_t*>(mark);
  for (int k = 2 * wv + (lane >> 5); k < nw; k += 8) {
    const uint2 wp = bits[g][k];
    const uint32_t bit = lane & 31;
    if ((wp.x >> bit) & 1u) {
      const uint32_t c = wp.y + __popc(wp.x & ((1u << bit) - 1u));
      if (c < (uint32_t)kUcap) by_rank[c] = lo + 32 * k + (int)bit;
    }
  }
  __syncthreads();
  for (int d = tid; d < kUcap; d += kPT) {
    const int grp = d / P::NJ, j = d - P::NJ * grp;
    const uint32_t c = (uint32_t)((grp >> 4) * P::WSLOTS + 16 * j + (grp & 15));
    idz[d] = c < total ? by_rank[c] : -1;
  }
  // 5. slot table of the nine taps (rows past the tile read the zero slot)
  auto slot_of = [&](int vj) -> uint32_t {
    uint32_t slot = kUcap;
    if (fits && vj >= 0) {
      const uint32_t d = (uint32_t)(vj - lo);
      const uint2 wp = bits[g][d >> 5];
      const uint32_t rank = wp.y + __popc(wp.x & ((1u << (d & 31)) - 1u));
      slot = rank < (uint32_t)kUcap ? rank : (uint32_t)kUcap;
    }
    return slot_offset(slot);
  };
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int r = 2 * tid + 2 * kPT * u;
    if (r >= R) break;
#pragma unroll
    for (int j = 0; j < 9; ++j) tab2[j * (R / 2) + r / 2] = slot_of(nb9[u][0][j]) | (slot_of(nb9[u][1][j]) << 16);
  }
  if (tid == 0) {
    flags[3 * tile + dz] = bad ? 1u : 0u;
    if (bad) *reinterpret_cast<volatile uint32_t*>(host_flag) = 1u;
  }
}

// Weights KRSC [128, 27, cin] -> packed [cin / 32][27][2 kk][4 ob][64 lanes][16 bytes]: half-step
// (q, t, kk) is one contiguous 4 KB block, and in it the operand-A fragment of output block ob is
// 1 KB in lane order: lane l = 32 lk + r holds output channel 32 ob + r, input channels
// 32 q + 8 (2 kk + lk) .. + 8.  Consecutive lanes then read consecutive 16-byte units, the
// pattern the LDS serves fastest.  One workgroup per (ob, t): it reads the 32 channels' rows of tap
// t (cin * 2 contiguous bytes each, 512 bytes at a time) into LDS and writes, for every 16-byte
// column c = 4 q + 2 kk + lk, the 32 rows' units as one contiguous 512-byte run.
__global__ __launch_bounds__(256) void pool_pack_kernel(const uint4* __restrict__ w, int cin, uint4* __restrict__ wpk) {
  __shared__ uint4 s_rows[32 * 33];  // [r][c - c0], rows padded by one unit against bank conflicts
  const int ob = (int)blockIdx.x / 27, t = (int)blockIdx.x % 27;
  const int row16 = cin / 8;  // 16-byte units per (co, tap) row
  for (int c0 = 0; c0 < row16; c0 += 32) {
    const int nc = min(32, row16 - c0);
    for (int i = threadIdx.x; i < 32 * nc; i += blockDim.x) {
      const int r = i / nc, c = i - r * nc;
      s_rows[r * 33 + c] = w[((int64_t)(32 * ob + r) * 27 + t) * row16 + c0 + c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 32 * nc; i += blockDim.x) {
      const int c = c0 + (i >> 5), r = i & 31;
      const int q = c >> 2, kk = (c >> 1) & 1, lk = c & 1;
      wpk[((((int64_t)(q * 27 + t) * 2 + kk) * 4 + ob) * 2 + lk) * 32 + r] = s_rows[r * 33 + (i >> 5)];
    }
    __syncthreads();
  }
}

struct PoolArgs {
  const void* feats;
  const void* wpk;
  const void* bias;
  void* out;
  const unsigned char* plan;
  const uint32_t* gate;  // non-null: overflow flags [3 ntiles]; the kernel does nothing when one is set
  int64_t n;
  int row_bytes;
  int qs;       // slices of 32 input channels
  int ntiles;
  int nb;       // row blocks of 32
  int per_wg;   // tiles per workgroup
  uint32_t feats_bytes;
  uint32_t wpk_bytes;
  uint32_t plan_bytes;
};

template <int V> using IC = std::integral_constant<int, V>;

// acc += a * b for the shared seventeenth block, as inline assembly with the accumulator in
// VGPRs: measured ~2 % faster on the shell than the builtin, whose scheduling and hazard waits
// around this ninth, conditional MFMA cost more than the explicit wait before the final write.
template <DT D>
__device__ __forceinline__ void mfma32_vgpr(f32x16_t& acc, const uint4& a, const uint4& b) {
  const i32x4_t av = __builtin_bit_cast(i32x4_t, a), bv = __builtin_bit_cast(i32x4_t, b);
  if constexpr (D == DT::BF16)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(av), "v"(bv));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(av), "v"(bv));
}

template <DT D, int E>
__global__ __launch_bounds__(kCT, 1) void pool_conv_kernel(const PoolArgs a) {
  using P = PoolShape<E>;
  using T = typename Elem<D>::T;
  __shared__ __align__(16) unsigned char lds[P::LDSB];

  const int tid = threadIdx.x;
  if (a.gate != nullptr && pool_any_flag(a.gate, 3 * a.ntiles)) return;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Waves w and w + 4 share a SIMD.  wq: the wave's quarter of a weight half-step (its 1 KB share
  // of the loads) and the rotation of its operand-A reads; waves 0..3 also load the slot table and
  // hold the shared seventeenth row block.
  const int wq = w & 3;
  const bool lo4 = w < 4;
  const int lr = lane & 31, lk = lane >> 5;
  // Workgroups are dealt to the eight XCDs round-robin: virtual block v takes the tiles
  // [v per_wg, (v + 1) per_wg), so each XCD walks one contiguous range of rows.
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  const int v = (G % 8 == 0) ? (b & 7) * (G >> 3) + (b >> 3) : b;
  const int tile0 = v * a.per_wg;
  const int ntl = min(a.per_wg, a.ntiles - tile0);
  if (ntl <= 0) return;
  const int Q = a.qs;
  const int S = 27 * Q;  // steps per tile

  const uint32_t lbase = lds_offset(lds);
  const i32x4_t rs_f = make_rsrc(a.feats, a.feats_bytes);
  const i32x4_t rs_w = make_rsrc(a.wpk, a.wpk_bytes);
  const i32x4_t rs_p = make_rsrc(a.plan, a.plan_bytes);

  if (tid < 128)
    reinterpret_cast<float*>(lds + P::O_BIAS)[tid] =
        a.bias != nullptr ? to_float<D>(reinterpret_cast<const T*>(a.bias)[tid]) : 0.f;
  if (tid < 8)
    *reinterpret_cast<uint4*>(lds + (tid >> 2) * P::POOLB + kUcap * kSL + (tid & 3) * 16) = make_uint4(0, 0, 0, 0);

  // Per-lane constants.  A gather lane of load j of wave w fills slot w * 96 + 16 j + lane / 4,
  // 16-byte unit lane % 4, so it fetches chunk (lane % 4) ^ ((slot >> 1) & 3) = (lane % 4) ^ ((lane / 8) % 4).
  const uint32_t gchunk = (uint32_t)(((lane & 3) ^ ((lane >> 3) & 3)) * 16);
  // Operand A position j of a wave holds output block (wq + j) % 4; its fragment is the 1 KB run
  // of that block in the half-step, 16 bytes per lane in lane order.
  uint32_t a_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a_off[j] = (uint32_t)(((wq + j) & 3) * 1024 + lane * 16);

  int ids[P::NJ];
  auto load_ids = [&](const unsigned char* base) {
    const uint2* p = reinterpret_cast<const uint2*>(base + (w * 16 + (lane >> 2)) * P::NJ * 4);
#pragma unroll
    for (int u = 0; u < P::NJ / 2; ++u) {
      const uint2 x = p[u];
      ids[2 * u] = (int)x.x;
      ids[2 * u + 1] = (int)x.y;
    }
  };
  auto read_ids = [&](int dz) { load_ids(lds + P::O_IDS + dz * P::IDB); };
  // gather load j of a sub-pool of slice q into pool buffer buf (live = false: reads nothing)
  auto gather1 = [&](int j, int q, int buf, bool live) {
    const uint32_t qoff = (uint32_t)(q * kSL) + gchunk;
    const uint32_t dst = lbase + (uint32_t)(buf * P::POOLB + w * P::WSLOTS * kSL);
    const uint32_t off = (live && ids[j] >= 0) ? (uint32_t)ids[j] * (uint32_t)a.row_bytes + qoff : kOutOfRange;
    lds_dma16(rs_f, off, dst + (uint32_t)(j * 16 * kSL));
  };
  // this wave's quarter of weight half-step (step = q * 27 + t, kk) -> half-slot: the packed
  // weights make a half-step one contiguous 4 KB block
  auto issue_w = [&](int step, int kk, int hslot) {
    const uint32_t src = (uint32_t)(2 * step + kk) * kWH + (uint32_t)(wq * 1024) + (uint32_t)lane * 16u;
    lds_dma16(rs_w, src, lbase + P::O_W + (uint32_t)(hslot * kWH + wq * 1024));
  };
  // slot-table tap t of a tile (tile < 0: nothing to load); waves 0..3
  auto issue_table = [&](int tile, int t) {
    const uint32_t off = tile < 0 ? kOutOfRange
                                  : (uint32_t)tile * P::RECB + (uint32_t)(t * P::TAPB + wq * (P::TAPB / 4)) + (uint32_t)lane * 16u;
    if (lane < P::TAPB / 64) lds_dma16(rs_p, off, lbase + P::O_TAB + (uint32_t)(t * P::TAPB + wq * (P::TAPB / 4)));
  };
  // row-id group dz of a tile (tile < 0: nothing to load); every wave loads an eighth
  auto issue_ids = [&](int tile, int dz) {
    const uint32_t off = tile < 0 ? kOutOfRange
                                  : (uint32_t)tile * P::RECB + (uint32_t)(P::TABB + dz * P::IDB + w * (P::IDB / 8)) +
                                        (uint32_t)lane * 16u;
    if (lane < P::IDB / 128) lds_dma16(rs_p, off, lbase + P::O_IDS + (uint32_t)(dz * P::IDB + w * (P::IDB / 8)));
  };

  // ---- prologue: the gathers of the first tile's sub-pool 0 go out as soon as this lane's row
  // ids arrive (straight from the record); slot-table taps 0..3 (the loop loads each tap four
  // steps ahead), row-id groups 1 and 2 and the first five weight half-steps follow.
  {
    load_ids(a.plan + (size_t)tile0 * P::RECB + P::TABB);
#pragma unroll
    for (int j = 0; j < P::NJ; ++j) gather1(j, 0, 0, true);
    const uint4* rec = reinterpret_cast<const uint4*>(a.plan + (size_t)tile0 * P::RECB);
    uint4* dst = reinterpret_cast<uint4*>(lds + P::O_TAB);
    for (int i = tid; i < 4 * P::TAPB / 16; i += kCT) dst[i] = rec[i];
    for (int i = tid; i < 2 * P::IDB / 16; i += kCT) dst[(P::TABB + P::IDB) / 16 + i] = rec[(P::TABB + P::IDB) / 16 + i];
    const uint4* wsrc = reinterpret_cast<const uint4*>(a.wpk);
    uint4* wdst = reinterpret_cast<uint4*>(lds + P::O_W);
    for (int i = tid; i < 5 * kWH / 16; i += kCT) wdst[i] = wsrc[i];  // half-steps (0,0) .. (2,0)
    wait_vmcnt<0>();
    __syncthreads();
  }

  // Accumulators: row blocks 2 w and 2 w + 1 of the tile, all four output blocks; waves
  // 0..3 also hold output block w of the seventeenth row block, when there is one (VGPRs).
  f32x16_t acc[2][4];
  f32x16_t accx;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) accx[e] = 0.f;

  constexpr int NB = 2 + E;  // operand-B fragments per half-step (the third: waves 0..3)
  constexpr int NU = 8 + E;  // MFMA units per half-step (unit 8: waves 0..3)
  uint32_t soff[NB], soff_n[NB];
  uint4 fa[2][4], fb[2][NB];

  auto read_slots = [&](int t, uint32_t* dst) {
    const uint16_t* tab = reinterpret_cast<const uint16_t*>(lds + P::O_TAB + t * P::TAPB);
#pragma unroll
    for (int i = 0; i < 2; ++i) dst[i] = tab[(2 * w + i) * 32 + lr];
    if constexpr (E) dst[2] = tab[16 * 32 + lr];
  };
  auto read_a = [&](auto SET, int hslot, int j) {
    constexpr int st = decltype(SET)::value;
    fa[st][j] = *reinterpret_cast<const uint4*>(lds + P::O_W + hslot * kWH + a_off[j]);
  };
  auto read_b = [&](auto SET, int kk, int pbuf, const uint32_t* so, int i) {
    constexpr int st = decltype(SET)::value;
    const uint32_t cx = (uint32_t)((2 * kk + lk) << 4);
    fb[st][i] = *reinterpret_cast<const uint4*>(lds + pbuf * P::POOLB + (so[i] ^ cx));
  };
  // MFMAs [LO, HI) of one half-step: unit u = 4 i + j (row block 2 w + i, operand A position j);
  // unit 8 is the shared block with this wave's own output block (waves 0..3).
  auto mfmas = [&](auto SET, auto LO, auto HI) {
    constexpr int st = decltype(SET)::value;
    constexpr int lo = decltype(LO)::value, hi = decltype(HI)::value;
#pragma unroll
    for (int u = lo; u < hi; ++u) {
      if (u < 8) {
        acc[u >> 2][u & 3] = mfma32<D>(fa[st][u & 3], fb[st][u >> 2], acc[u >> 2][u & 3]);
      } else if constexpr (E) {
        if (lo4) mfma32_vgpr<D>(accx, fa[st][0], fb[st][2]);
      }
    }
  };

  void* out = a.out;
  // Finished tile: + bias, one rounding.  Each 32-row block of a wave goes through a
  // wave-private LDS region, 16 rows at a time (rows padded to 272 bytes against bank
  // conflicts), so the stores are whole 256-byte rows, 16 bytes per lane.  `stage` is the LDS
  // byte offset of the eight regions; no load writes there any more.
  constexpr int kRowPad = 272;
  auto write_tile = [&](int tile, int stage) {
    if constexpr (E) asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");  // the last MFMA into accx is done
    int lanex = lane;  // (opaque: nothing derived from it is kept live across the main loop)
    asm volatile("" : "+v"(lanex));
    const int lrx = lanex & 31, lkx = lanex >> 5;
    const int blk0 = (int)((int64_t)tile * a.nb / a.ntiles);
    const int blk1 = (int)((int64_t)(tile + 1) * a.nb / a.ntiles);
    const int64_t r0 = (int64_t)blk0 * 32;
    const int valid = (int)min((int64_t)(blk1 - blk0) * 32, a.n - r0);  // rows of this tile
    unsigned char* obase = reinterpret_cast<unsigned char*>(out) + r0 * 256;
    const unsigned char* bbase = lds + P::O_BIAS + 16 * lkx;
    unsigned char* wst = lds + stage + w * 16 * kRowPad;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tr0 = (2 * w + i) * 32;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if ((lrx >> 4) == h) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x16_t& c = acc[i][j];
            const int ob = (wq + j) & 3;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              // accumulator element 4 g + e of lane (lr, lk) = output channel 32 ob + 8 g + 4 lk + e
              const int cb = 32 * ob + 8 * g;
              const float4 bb = *reinterpret_cast<const float4*>(bbase + cb * 4);
              *reinterpret_cast<uint2*>(wst + (lrx - 16 * h) * kRowPad + cb * 2 + 8 * lkx) =
                  pack4<D>(c[4 * g] + bb.x, c[4 * g + 1] + bb.y, c[4 * g + 2] + bb.z, c[4 * g + 3] + bb.w);
            }
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int rr = 4 * k + (lanex >> 4);
          const uint4 val = *reinterpret_cast<const uint4*>(wst + rr * kRowPad + (lanex & 15) * 16);
          const int row = tr0 + 16 * h + rr;
          if (row < valid) *reinterpret_cast<uint4*>(obase + (uint32_t)(row * 256 + (lanex & 15) * 16)) = val;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    }
    if constexpr (E) {
      if (lo4) {
        // block 16: this wave holds output block w of it
        const int trow = 16 * 32 + lrx;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cb = 32 * w + 8 * g;
          const float4 bb = *reinterpret_cast<const float4*>(bbase + cb * 4);
          if (trow < valid)
            *reinterpret_cast<uint2*>(obase + (uint32_t)(trow * 256 + cb * 2 + 8 * lkx)) =
                pack4<D>(accx[4 * g] + bb.x, accx[4 * g + 1] + bb.y, accx[4 * g + 2] + bb.z, accx[4 * g + 3] + bb.w);
          accx[4 * g] = accx[4 * g + 1] = accx[4 * g + 2] = accx[4 * g + 3] = 0.f;
        }
      }
    }
  };

  // step 0's slots and first half-step fragments, the row ids of the gathers of step 0
  read_slots(0, soff);
#pragma unroll
  for (int j = 0; j < 4; ++j) read_a(IC<0>{}, 0, j);
#pragma unroll
  for (int i = 0; i < 2; ++i) read_b(IC<0>{}, 0, 0, soff, i);
  if constexpr (E) {
    if (lo4) read_b(IC<0>{}, 0, 0, soff, 2);
  }
  read_ids(1);

  // One step (q, dz, g) of tile `tile`; `nxt` is the next tile of this workgroup (-1: none),
  // `sb` = q * 27 + dz * 9, `pbuf` the pool buffer of this sub-pool.
  auto step = [&](auto GG, int tile, int nxt, int q, int dz, int sb, int pbuf) {
    constexpr int g = decltype(GG)::value;
    // (2 s) mod 6 for the weight half-slots: S is a multiple of 3, so it is 2 (g mod 3)
    constexpr int hs = 2 * (g % 3);
    // Loads per step and wave, in this order: 1 weight quarter (waves 0..3: (s + 3, 0); waves
    // 4..7: (s + 2, 1)), 1 slot-table tap (waves 0..3), 1 gather of the next sub-pool (g <= 5,
    // possibly reading nothing), 1 row-id group (g == 0).  Wait until this wave's weight quarter
    // of step s - 2 ((s + 1, 0) or (s, 1)) has landed (vector-memory loads complete in order); the
    // barrier then makes every wave's share visible and frees the slots the loads below overwrite.
    constexpr int g2 = (g + 7) % 9, g1 = (g + 8) % 9;
    constexpr int after2 = (g2 <= 5 ? 1 : 0) + (g2 == 0 ? 1 : 0);  // step s - 2, after its weight load
    constexpr int all1 = 1 + (g1 <= 5 ? 1 : 0) + (g1 == 0 ? 1 : 0);  // step s - 1, all of it
    if (lo4)
      wait_vmcnt<after2 + 1 + all1 + 1>();
    else
      wait_vmcnt<after2 + all1>();
    barrier_no_fence();
    const bool last = q == Q - 1;
    const int src = last ? nxt : tile;
    const int t = dz * 9 + g;
    const int sl = sb + g;
    const int pbuf1 = g == 8 ? (pbuf ^ 1) : pbuf;
    const int hs1 = hs + 1, hs2 = hs + 2 == kWS ? 0 : hs + 2;
    const int nq = dz == 2 ? (last ? 0 : q + 1) : q;  // slice of the next sub-pool
    const bool glive = !(dz == 2 && last) || nxt >= 0;
    // ---- first half: MFMAs of (s, 0), written one per LDS read of (s, 1) or load of this step.
    // With two waves per SIMD the compiler's own schedule of this stream measured 2-3 % faster
    // than pinning that order with scheduling barriers.  The slots of step s + 1 are read first:
    // the second half needs them.
    read_slots(t == 26 ? 0 : t + 1, soff_n);
    auto one = [&](auto SETM, auto U) { mfmas(SETM, U, IC<decltype(U)::value + 1>{}); };
    one(IC<0>{}, IC<0>{}); read_a(IC<1>{}, hs1, 0);
    one(IC<0>{}, IC<1>{}); read_a(IC<1>{}, hs1, 1);
    one(IC<0>{}, IC<2>{}); read_a(IC<1>{}, hs1, 2);
    one(IC<0>{}, IC<3>{}); read_a(IC<1>{}, hs1, 3);
    one(IC<0>{}, IC<4>{}); read_b(IC<1>{}, 1, pbuf, soff, 0);
    one(IC<0>{}, IC<5>{}); read_b(IC<1>{}, 1, pbuf, soff, 1);
    if constexpr (E) {
      if (lo4) read_b(IC<1>{}, 1, pbuf, soff, 2);
    }
    // weight quarters: (s + 3, 0) into the half-slot of (s, 0), read last step, or (s + 2, 1)
    // into the half-slot of (s - 1, 1)
    one(IC<0>{}, IC<6>{});
    if (lo4)
      issue_w(sl + 3 < S ? sl + 3 : sl + 3 - S, 0, hs);
    else
      issue_w(sl + 2 < S ? sl + 2 : sl + 2 - S, 1, hs == 0 ? kWS - 1 : hs - 1);
    // slot-table tap of step s + 4 (the next slice's, or the next tile's in the last slice); the
    // gather of the next sub-pool: (q, dz + 1), (q + 1, 0) or the next tile's (0, 0), whose row
    // ids were read at the end of the previous sub-pool
    one(IC<0>{}, IC<7>{});
    if (lo4) issue_table(t >= 23 && last ? nxt : tile, t >= 23 ? t - 23 : t + 4);
    if constexpr (g <= 5) gather1(g, nq, pbuf ^ 1, glive);
    mfmas(IC<0>{}, IC<8>{}, IC<NU>{});
    if constexpr (g == 0) issue_ids(src, dz);
    // ---- second half: MFMAs of (s, 1), the first six followed by one read of (s + 1, 0)
    one(IC<1>{}, IC<0>{}); read_a(IC<0>{}, hs2, 0);
    one(IC<1>{}, IC<1>{}); read_a(IC<0>{}, hs2, 1);
    one(IC<1>{}, IC<2>{}); read_a(IC<0>{}, hs2, 2);
    one(IC<1>{}, IC<3>{}); read_a(IC<0>{}, hs2, 3);
    one(IC<1>{}, IC<4>{}); read_b(IC<0>{}, 0, pbuf1, soff_n, 0);
    one(IC<1>{}, IC<5>{}); read_b(IC<0>{}, 0, pbuf1, soff_n, 1);
    if constexpr (E) {
      if (lo4) read_b(IC<0>{}, 0, pbuf1, soff_n, 2);
    }
    one(IC<1>{}, IC<6>{}); if constexpr (g == 8) read_ids(dz == 0 ? 2 : dz - 1);  // the next sub-pool's gathers
    mfmas(IC<1>{}, IC<7>{}, IC<NU>{});
#pragma unroll
    for (int i = 0; i < NB; ++i) soff[i] = soff_n[i];
  };

  int pb = 0;
  for (int ti = 0; ti < ntl; ++ti) {
    const int tile = tile0 + ti;
    const int nxt = ti + 1 < ntl ? tile + 1 : -1;
    for (int q = 0; q < Q; ++q) {
      for (int dz = 0; dz < 3; ++dz) {
        const int sb = q * 27 + dz * 9;
        step(IC<0>{}, tile, nxt, q, dz, sb, pb);
        step(IC<1>{}, tile, nxt, q, dz, sb, pb);
        step(IC<2>{}, tile, nxt, q, dz, sb, pb);
        step(IC<3>{}, tile, nxt, q, dz, sb, pb);
        step(IC<4>{}, tile, nxt, q, dz, sb, pb);
        step(IC<5>{}, tile, nxt, q, dz, sb, pb);
        step(IC<6>{}, tile, nxt, q, dz, sb, pb);
        step(IC<7>{}, tile, nxt, q, dz, sb, pb);
        step(IC<8>{}, tile, nxt, q, dz, sb, pb);
        pb ^= 1;
      }
    }
    // The buffer of the tile's last sub-pool (pb ^ 1 after the toggle) is free once every wave
    // has finished reading it; the next tile's sub-pool 0 is in pb.
    barrier_no_fence();
    write_tile(tile, (pb ^ 1) * P::POOLB);
  }
  wait_vmcnt<0>();  // no direct-to-LDS load may still be in flight when the workgroup ends
}

}  // namespace

bool pool_tiling(int64_t n, PoolTiling* t) {
  const int64_t nb = (n + 31) / 32;
  if (nb < 256 * 16) return false;  // fewer than one full tile per compute unit
  const int64_t per_cu = (nb + 255) / 256;
  const int64_t k = (per_cu + 16) / 17;
  const int64_t T = std::min<int64_t>(256 * k, (nb + 15) / 16);
  const int64_t recb = (nb + T - 1) / T > 16 ? PoolShape<1>::RECB : PoolShape<0>::RECB;
  if (T * recb >= (int64_t)0x7FFFF000) return false;  // records addressed with 31-bit offsets
  if (nb >= ((int64_t)1 << 31) / 32 / 27) return false;  // (row indices of the rulebook are int32)
  t->nb = (int)nb;
  t->ntiles = (int)T;
  t->per_wg = (int)((T + 255) / 256);
  t->e = (nb + T - 1) / T > 16 ? 1 : 0;
  return true;
}

static size_t pool_records_bytes(const PoolTiling& t) {
  return (size_t)t.ntiles * (size_t)(t.e ? PoolShape<1>::RECB : PoolShape<0>::RECB);
}

int pool_flag_count(const PoolTiling& t) { return 3 * t.ntiles; }

size_t pool_plan_bytes(const PoolTiling& t) {
  return pool_records_bytes(t) + ((size_t)pool_flag_count(t) * 4 + 255) / 256 * 256;
}

uint32_t* pool_tile_flags(const PoolTiling& t, void* plan) {
  return reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(plan) + pool_records_bytes(t));
}

size_t pool_weight_bytes(int cin) { return (size_t)27 * 128 * (size_t)cin * 2; }

hipError_t launch_pool_plan(const int32_t* nbr, int64_t n, const PoolTiling& t, void* plan, uint32_t* host_flag,
                            hipEvent_t done, hipStream_t stream) {
  auto* rec = static_cast<unsigned char*>(plan);
  uint32_t* flags = pool_tile_flags(t, plan);
  if (t.e)
    hipExtLaunchKernelGGL(pool_plan_kernel<1>, dim3((unsigned)t.ntiles), dim3(3 * kPT), 0, stream, nullptr, done, 0u, nbr,
                          n, t.nb, t.ntiles, rec, flags, host_flag);
  else
    hipExtLaunchKernelGGL(pool_plan_kernel<0>, dim3((unsigned)t.ntiles), dim3(3 * kPT), 0, stream, nullptr, done, 0u, nbr,
                          n, t.nb, t.ntiles, rec, flags, host_flag);
  return hipGetLastError();
}

hipError_t launch_pool_conv(const PoolTiling& t, const void* plan, const uint32_t* gate, int64_t n, int cin, int dtype,
                            const void* feats, const void* weight, const void* bias, void* out, void* wpk,
                            hipStream_t stream) {
  const size_t wbytes = pool_weight_bytes(cin);
  pool_pack_kernel<<<4 * 27, 256, 0, stream>>>(static_cast<const uint4*>(weight), cin, static_cast<uint4*>(wpk));
  PoolArgs a{};
  a.feats = feats;
  a.wpk = wpk;
  a.bias = bias;
  a.out = out;
  a.plan = static_cast<const unsigned char*>(plan);
  a.gate = gate;
  a.n = n;
  a.row_bytes = cin * 2;
  a.qs = cin / 32;
  a.ntiles = t.ntiles;
  a.nb = t.nb;
  a.per_wg = t.per_wg;
  a.feats_bytes = (uint32_t)((uint64_t)n * (uint64_t)cin * 2);
  a.wpk_bytes = (uint32_t)wbytes;
  a.plan_bytes = (uint32_t)pool_records_bytes(t);
  const dim3 grid((unsigned)((t.ntiles + t.per_wg - 1) / t.per_wg));
  if (dtype == SUBM_BF16) {
    if (t.e) launch_kernel_timed(pool_conv_kernel<DT::BF16, 1>, grid, dim3(kCT), stream, a);
    else launch_kernel_timed(pool_conv_kernel<DT::BF16, 0>, grid, dim3(kCT), stream, a);
  } else {
    if (t.e) launch_kernel_timed(pool_conv_kernel<DT::F16, 1>, grid, dim3(kCT), stream, a);
    else launch_kernel_timed(pool_conv_kernel<DT::F16, 0>, grid, dim3(kCT), stream, a);
  }
  return hipGetLastError();
}

}  // namespace submconv
