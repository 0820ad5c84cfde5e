// Group normalisation per batch item in float32 followed by an activation (sparse_norm.h states
// the operation and where the pages name it).
//
// Three passes:
//   1. partials: the rows of every item are cut into segments of at most R consecutive rows
//      (segment s = b + k holds rows [max(off[b], kR), min(off[b+1], (k+1)R)) of item b, so the
//      segment index needs no search table); one block per segment reads its rows once and
//      forms, per group, the sums of x - K and (x - K)^2 with K the group's first value in the
//      segment (shifted sums: no cancellation when the mean is large against the spread), in
//      float32 and a fixed order, and stores the segment's mean and sum of squared deviations;
//   2. statistics: one block per item combines its segments, per group, with the pairwise update
//      of Chan, Golub and LeVeque in float64 (strided partial chains, then a fixed tree) and
//      stores the mean and 1 / sqrt(var + eps);
//   3. apply: one block per segment (a single item), per-channel scale rstd * gamma and shift
//      beta - mean * rstd * gamma in LDS, then y = act(x * scale + shift), rounded once.
// Every reduction runs in a fixed order, so the result is bitwise reproducible.
#include <algorithm>
#include <cmath>
#include <cstdlib>

#include "device_common.h"
#include "internal.h"
#include "sparse_norm.h"

namespace submconv {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSegmentsPerRun = 1024;  // segment length R grows with n to keep this bound

__device__ __forceinline__ int64_t clamp_off(const int64_t* off, int b, int64_t n) {
  const int64_t v = off[b];
  return v < 0 ? 0 : (v > n ? n : v);
}

// 16 bytes of storage -> E floats, and back (E = 16 / element size).
template <DT D, int E> __device__ __forceinline__ void unpack(const uint4& raw, float (&v)[E]) {
  const unsigned char* b = reinterpret_cast<const unsigned char*>(&raw);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if constexpr (D == DT::F32) v[e] = reinterpret_cast<const float*>(b)[e];
    else v[e] = to_float<D>(reinterpret_cast<const uint16_t*>(b)[e]);
  }
}

template <int ACT> __device__ __forceinline__ float activate(float y) {
  if constexpr (ACT == SUBM_ACT_SILU) return y / (1.f + __expf(-y));
  if constexpr (ACT == SUBM_ACT_RELU) return fmaxf(y, 0.f);
  return y;
}

// Segment s -> (item, rows [r0, r1)): the item is the largest b with b + off[b] / R <= s, which
// is strictly increasing in b.
struct Segment {
  int b;
  int64_t r0, r1;
};
__device__ __forceinline__ Segment find_segment(const int64_t* off, int items, int64_t n, int64_t R, int64_t s) {
  int lo = 0, hi = items - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mid + clamp_off(off, mid, n) / R <= s) lo = mid;
    else hi = mid - 1;
  }
  const int64_t k = s - lo;
  Segment g;
  g.b = lo;
  g.r0 = std::max(clamp_off(off, lo, n), k * R);
  g.r1 = std::min(clamp_off(off, lo + 1, n), (k + 1) * R);
  return g;
}

// Pass 1.  T = channels / E chunk lanes x RT = 256 / T row lanes.
template <DT D, int E>
__global__ __launch_bounds__(kThreads) void gn_partial_kernel(const void* __restrict__ x, int64_t n, int channels,
                                                              const int64_t* __restrict__ off, int items, int64_t R,
                                                              int groups, float2* __restrict__ part,
                                                              int32_t* __restrict__ part_rows) {
  __shared__ float s_acc[2][kThreads * E];
  __shared__ float s_shift[2048];
  const int tid = threadIdx.x;
  const int64_t s = blockIdx.x;
  const Segment seg = find_segment(off, items, n, R, s);
  const int64_t rows = seg.r1 > seg.r0 ? seg.r1 - seg.r0 : 0;
  const int cpg = channels / groups;
  if (rows == 0) {
    for (int g = tid; g < groups; g += kThreads) part[s * groups + g] = make_float2(0.f, 0.f);
    if (tid == 0) part_rows[s] = 0;
    return;
  }
  const unsigned char* xb = static_cast<const unsigned char*>(x);
  using T = typename Elem<D>::T;
  for (int g = tid; g < groups; g += kThreads) {
    const int64_t idx = seg.r0 * channels + (int64_t)g * cpg;
    s_shift[g] = D == DT::F32 ? reinterpret_cast<const float*>(xb)[idx] : to_float<D>(reinterpret_cast<const T*>(xb)[idx]);
  }
  __syncthreads();
  const int T_ = channels / E;  // chunk lanes (<= 256)
  const int RT = kThreads / T_;
  const int rl = tid / T_, cl = tid - (tid / T_) * T_;
  float a1[E], a2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) a1[e] = a2[e] = 0.f;
  if (rl < RT) {
    float k[E];
#pragma unroll
    for (int e = 0; e < E; ++e) k[e] = s_shift[(cl * E + e) / cpg];
#pragma unroll 4
    for (int64_t r = seg.r0 + rl; r < seg.r1; r += RT) {
      const uint4 raw = *reinterpret_cast<const uint4*>(xb + (r * channels + (int64_t)cl * E) * (16 / E));
      float v[E];
      unpack<D, E>(raw, v);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float d = v[e] - k[e];
        a1[e] += d;
        a2[e] += d * d;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    s_acc[0][tid * E + e] = a1[e];
    s_acc[1][tid * E + e] = a2[e];
  }
  __syncthreads();
  // per group: row lanes, then the group's channels, in order
  const float cnt = (float)(rows * cpg);
  for (int g = tid; g < groups; g += kThreads) {
    float t1 = 0.f, t2 = 0.f;
    for (int c = g * cpg; c < (g + 1) * cpg; ++c) {
      const int lane = c / E, e = c - (c / E) * E;
      for (int q = 0; q < RT; ++q) {
        t1 += s_acc[0][(q * T_ + lane) * E + e];
        t2 += s_acc[1][(q * T_ + lane) * E + e];
      }
    }
    const float mean_d = t1 / cnt;
    part[s * groups + g] = make_float2(s_shift[g] + mean_d, fmaxf(t2 - t1 * mean_d, 0.f));
  }
  if (tid == 0) part_rows[s] = (int32_t)rows;
}

// Pass 2: the partials of an item are combined with the pairwise update of Chan, Golub and
// LeVeque in float64, in two levels so that every compute unit takes part: level 1 combines
// chunks of kChunk consecutive partials of one item (slot s = b + p / kChunk for partial p of
// item b: the slots of consecutive items never collide, so no table is needed), level 2 combines
// the slots of each item.  Within a block, per group, TG threads run strided chains that are
// then added by a fixed pairwise tree, so the order never changes.
constexpr int kStatThreads = 1024;
constexpr int kChunkThreads = 256;
constexpr int kChunk = 64;      // partials per level-1 slot
constexpr int kChainLoads = 8;  // partials loaded ahead in each combination chain

__device__ __forceinline__ void chan_combine(double& na, double& ma, double& m2a, double nb, double mb, double m2b) {
  if (nb == 0.0) return;
  const double n = na + nb;
  const double d = mb - ma;
  const double r = nb / n;
  ma += d * r;
  m2a += m2b + d * d * na * r;
  na = n;
}

// Block-wide combination, per group g < groups, of the entries q in [q0, q1] given by
// get(q, g) -> (count, mean, M2); thread 0 of each group's lanes receives the result through
// `done(g, n, mean, M2)`.  NT threads; s_* hold NT doubles each.
template <int NT, typename Get, typename Done>
__device__ __forceinline__ void block_combine(int groups, int64_t q0, int64_t q1, Get get, Done done, double* s_n,
                                              double* s_m, double* s_q) {
  const int tid = threadIdx.x;
  int tg = 1;  // threads per group: the largest power of two with TG * groups <= NT
  while (tg * 2 * groups <= NT) tg *= 2;
  const int gpb = NT / tg;
  for (int g0 = 0; g0 < groups; g0 += gpb) {
    const int g = g0 + tid / tg, j = tid % tg;
    const bool on = tid / tg < gpb && g < groups;
    double na = 0.0, ma = 0.0, m2a = 0.0;
    if (on)
      for (int64_t q = q0 + j; q <= q1; q += (int64_t)kChainLoads * tg) {
        double c[kChainLoads], m[kChainLoads], v[kChainLoads];
#pragma unroll
        for (int u = 0; u < kChainLoads; ++u) {  // loads in flight before the dependent updates
          const int64_t qq = q + (int64_t)u * tg;
          get(qq <= q1 ? qq : q1, g, c[u], m[u], v[u]);  // clamped: no branches around the loads
          if (qq > q1) c[u] = 0.0;
        }
#pragma unroll
        for (int u = 0; u < kChainLoads; ++u) chan_combine(na, ma, m2a, c[u], m[u], v[u]);
      }
    s_n[tid] = na;
    s_m[tid] = ma;
    s_q[tid] = m2a;
    __syncthreads();
    for (int h = 1; h < tg; h <<= 1) {
      if (on && (j % (2 * h)) == 0) {
        double x = s_n[tid], y = s_m[tid], z = s_q[tid];
        chan_combine(x, y, z, s_n[tid + h], s_m[tid + h], s_q[tid + h]);
        s_n[tid] = x;
        s_m[tid] = y;
        s_q[tid] = z;
      }
      __syncthreads();
    }
    if (on && j == 0) done(g, s_n[tid], s_m[tid], s_q[tid]);
    __syncthreads();
  }
}

// Where the partials of item b live: segments (the separate statistics pass, count from
// part_rows) or row tiles of the convolution epilogue (interior tiles only, count from the tile
// height).  key(b) orders the items for the slot search; range(b) is [first, last] (first > last
// when empty).
template <bool TILES>
struct PartialSpace {
  const float2* part;
  const int32_t* part_rows;  // segments only
  const int64_t* off;
  int64_t n;
  int64_t R;  // segment length or tile height
  int cpg;
  __device__ int64_t key(int b) const {
    const int64_t lo = clamp_off(off, b, n);
    return TILES ? lo / R : b + lo / R;
  }
  __device__ void range(int b, int64_t& first, int64_t& last) const;
  __device__ void get(int64_t p, int g, int groups, double& c, double& m, double& v) const {
    const float2 x = part[p * groups + g];
    c = TILES ? (double)std::min(R, n - p * R) * cpg : (double)part_rows[p] * cpg;
    m = x.x;
    v = x.y;
  }
};

// Level 1: slot s = b + first-partial-chunk index; combines partials [max(first, kC), min(last, kC + kChunk - 1)].
template <bool TILES>
__global__ __launch_bounds__(kChunkThreads) void gn_chunk_kernel(PartialSpace<TILES> ps, int items, int groups,
                                                                 double* __restrict__ sn, double* __restrict__ sm,
                                                                 double* __restrict__ sq) {
  __shared__ double s_n[kChunkThreads], s_m[kChunkThreads], s_q[kChunkThreads];
  const int64_t s = blockIdx.x;
  int lo = 0, hi = items - 1;  // item: the largest b with b + key(b) / kChunk <= s
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mid + ps.key(mid) / kChunk <= s) lo = mid;
    else hi = mid - 1;
  }
  int64_t first, last;
  ps.range(lo, first, last);
  const int64_t k = s - lo;
  const int64_t q0 = std::max(first, k * kChunk), q1 = std::min(last, k * kChunk + kChunk - 1);
  block_combine<kChunkThreads>(
      groups, q0, q1, [&](int64_t q, int g, double& c, double& m, double& v) { ps.get(q, g, groups, c, m, v); },
      [&](int g, double c, double m, double v) {
        sn[s * groups + g] = c;
        sm[s * groups + g] = m;
        sq[s * groups + g] = v;
      },
      s_n, s_m, s_q);
}

// Level 2: one block per item: (first boundary piece,) its slots, (last boundary piece).
template <bool TILES>
__global__ __launch_bounds__(kStatThreads) void gn_finish_kernel(PartialSpace<TILES> ps, int groups, float eps,
                                                                 const double* __restrict__ sn,
                                                                 const double* __restrict__ sm,
                                                                 const double* __restrict__ sq,
                                                                 const float2* __restrict__ bpart,
                                                                 const int32_t* __restrict__ brows,
                                                                 float2* __restrict__ stats) {
  __shared__ double s_n[kStatThreads], s_m[kStatThreads], s_q[kStatThreads];
  const int b = blockIdx.x;
  int64_t first, last;
  ps.range(b, first, last);
  const int64_t q0 = b + (first <= last ? first / kChunk : 0), q1 = first <= last ? b + last / kChunk : q0 - 1;
  block_combine<kStatThreads>(
      groups, q0, q1,
      [&](int64_t q, int g, double& c, double& m, double& v) {
        c = sn[q * groups + g];
        m = sm[q * groups + g];
        v = sq[q * groups + g];
      },
      [&](int g, double c, double m, double v) {
        double cn = 0.0, cm = 0.0, cq = 0.0;
        if (TILES) {
          const float2 f = bpart[(int64_t)(2 * b) * groups + g];
          chan_combine(cn, cm, cq, (double)brows[2 * b] * ps.cpg, f.x, f.y);
        }
        chan_combine(cn, cm, cq, c, m, v);
        if (TILES) {
          const float2 l = bpart[(int64_t)(2 * b + 1) * groups + g];
          chan_combine(cn, cm, cq, (double)brows[2 * b + 1] * ps.cpg, l.x, l.y);
        }
        const double var = cn > 0.0 ? cq / cn : 0.0;
        stats[(int64_t)b * groups + g] =
            cn > 0.0 ? make_float2((float)cm, (float)(1.0 / sqrt(var + (double)eps))) : make_float2(0.f, 0.f);
      },
      s_n, s_m, s_q);
}

// Number of level-1 slots for `items` items over `partials` partial indices.
int64_t chunk_slots(int items, int64_t partials) { return items + partials / kChunk + 1; }

// Fused variant (statistics from the convolution epilogue).  The epilogue leaves per (row tile of
// BM rows, group) partials over whole tiles; a tile that straddles an item boundary is recomputed
// here from the stored output, only for the rows of the item (at most two such tiles per item).
struct ItemTiles {
  int64_t lo, hi;     // the item's rows
  int64_t t0, t1;     // its first and last tile
  bool b0, b1;        // first / last tile straddles an item boundary
};
__device__ __forceinline__ int64_t tile_rows(int64_t t, int64_t BM, int64_t n) {
  return std::min(BM, n - t * BM);
}
__device__ __forceinline__ ItemTiles item_tiles(const int64_t* off, int b, int64_t n, int64_t BM) {
  ItemTiles it;
  it.lo = clamp_off(off, b, n);
  it.hi = clamp_off(off, b + 1, n);
  it.t0 = it.lo / BM;
  it.t1 = it.hi > it.lo ? (it.hi - 1) / BM : it.t0;
  it.b0 = !(it.t0 * BM >= it.lo && it.t0 * BM + tile_rows(it.t0, BM, n) <= it.hi);
  it.b1 = !(it.t1 * BM >= it.lo && it.t1 * BM + tile_rows(it.t1, BM, n) <= it.hi);
  return it;
}

// One block per (item, side): the item's rows in its first (side 0) or last (side 1) tile when that
// tile straddles a boundary; an item inside one tile is side 0's alone.  bpart = (mean, M2) per
// group, brows = rows (0: nothing to add).
template <DT D>
__global__ __launch_bounds__(kThreads) void gn_boundary_kernel(const void* __restrict__ y, int64_t n, int channels,
                                                               const int64_t* __restrict__ off, int64_t BM, int groups,
                                                               float2* __restrict__ bpart, int32_t* __restrict__ brows) {
  using T = typename Elem<D>::T;
  __shared__ float s1s[kThreads], s2s[kThreads];
  const int b = blockIdx.x >> 1, side = blockIdx.x & 1;
  const ItemTiles it = item_tiles(off, b, n, BM);
  int64_t a = 0, e = 0;
  if (it.hi > it.lo) {
    if (side == 0 && it.b0) {
      a = it.lo;
      e = std::min(it.hi, it.t0 * BM + tile_rows(it.t0, BM, n));
    } else if (side == 1 && it.b1 && it.t1 != it.t0) {
      a = it.t1 * BM;
      e = it.hi;
    }
  }
  const int64_t slot = (int64_t)blockIdx.x;
  if (threadIdx.x == 0) brows[slot] = (int32_t)(e > a ? e - a : 0);
  const int cpg = channels / groups;
  const T* x = static_cast<const T*>(y);
  for (int g0 = 0; g0 < groups; g0 += kThreads) {
    const int gn = std::min(kThreads, groups - g0);
    const int RL = kThreads / gn;
    const int g = g0 + threadIdx.x % gn, rl = threadIdx.x / gn;
    float sh = 0.f, t1 = 0.f, t2 = 0.f;
    if (e > a && rl < RL) {
      sh = D == DT::F32 ? reinterpret_cast<const float*>(y)[a * channels + (int64_t)g * cpg]
                        : to_float<D>(x[a * channels + (int64_t)g * cpg]);
      for (int64_t r = a + rl; r < e; r += RL)
        for (int c = 0; c < cpg; ++c) {
          const int64_t idx = r * channels + (int64_t)g * cpg + c;
          const float v = D == DT::F32 ? reinterpret_cast<const float*>(y)[idx] : to_float<D>(x[idx]);
          const float d = v - sh;
          t1 += d;
          t2 += d * d;
        }
    }
    s1s[threadIdx.x] = t1;
    s2s[threadIdx.x] = t2;
    __syncthreads();
    if ((int)threadIdx.x < gn) {
      float u1 = 0.f, u2 = 0.f;
      for (int q = 0; q < RL; ++q) {
        u1 += s1s[q * gn + threadIdx.x];
        u2 += s2s[q * gn + threadIdx.x];
      }
      const float cnt = (float)((e > a ? e - a : 1) * cpg);
      const float mean_d = u1 / cnt;
      bpart[slot * groups + g] = e > a ? make_float2(sh + mean_d, fmaxf(u2 - u1 * mean_d, 0.f)) : make_float2(0.f, 0.f);
    }
    __syncthreads();
  }
}

template <>
__device__ void PartialSpace<false>::range(int b, int64_t& first, int64_t& last) const {
  const int64_t lo = clamp_off(off, b, n), hi = clamp_off(off, b + 1, n);
  first = b + lo / R;
  last = hi > lo ? b + (hi - 1) / R : first - 1;
}
template <>
__device__ void PartialSpace<true>::range(int b, int64_t& first, int64_t& last) const {
  const ItemTiles it = item_tiles(off, b, n, R);
  if (it.hi <= it.lo) {
    first = it.t0 + 1;
    last = it.t0;
    return;
  }
  first = it.t0 + (it.b0 ? 1 : 0);
  last = it.t1 - ((it.b1 && it.t1 != it.t0) ? 1 : 0);  // interior tiles [first, last]
}

// Pass 3: one block per segment (one item).
template <DT D, int E, int ACT>
__global__ __launch_bounds__(kThreads) void gn_apply_kernel(const void* __restrict__ x, void* __restrict__ y, int64_t n,
                                                            int channels, const int64_t* __restrict__ off, int items,
                                                            int64_t R, int groups, const float2* __restrict__ stats,
                                                            const void* __restrict__ gamma,
                                                            const void* __restrict__ beta) {
  using T = typename Elem<D>::T;
  __shared__ float s_scale[2048], s_shift[2048];
  const Segment seg = find_segment(off, items, n, R, blockIdx.x);
  if (seg.r1 <= seg.r0) return;
  const int cpg = channels / groups;
  const float2* st = stats + (int64_t)seg.b * groups;
  for (int c = threadIdx.x; c < channels; c += kThreads) {
    const float2 ms = st[c / cpg];
    const float ga = gamma != nullptr ? to_float<D>(static_cast<const T*>(gamma)[c]) : 1.f;
    const float be = beta != nullptr ? to_float<D>(static_cast<const T*>(beta)[c]) : 0.f;
    s_scale[c] = ms.y * ga;
    s_shift[c] = be - ms.x * ms.y * ga;
  }
  __syncthreads();
  const int words = channels / E;
  const int rpb = kThreads / words;  // words <= 256
  const int rl = threadIdx.x / words, w = threadIdx.x - rl * words;
  if (rl >= rpb) return;
  const unsigned char* xb = static_cast<const unsigned char*>(x);
  unsigned char* yb = static_cast<unsigned char*>(y);
  float sc[E], sh[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    sc[e] = s_scale[w * E + e];
    sh[e] = s_shift[w * E + e];
  }
#pragma unroll 4
  for (int64_t r = seg.r0 + rl; r < seg.r1; r += rpb) {
    const int64_t byte = (r * words + w) * 16;
    const uint4 raw = *reinterpret_cast<const uint4*>(xb + byte);
    float v[E];
    unpack<D, E>(raw, v);
    uint4 outw;
    unsigned char* ob = reinterpret_cast<unsigned char*>(&outw);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float o = activate<ACT>(fmaf(v[e], sc[e], sh[e]));
      if constexpr (D == DT::F32) reinterpret_cast<float*>(ob)[e] = o;
      else reinterpret_cast<uint16_t*>(ob)[e] = from_float<D>(o);
    }
    *reinterpret_cast<uint4*>(yb + byte) = outw;
  }
}

template <DT D, int E, int ACT>
hipError_t launch_apply(const void* x, void* y, int64_t n, int channels, const int64_t* off, int items, int groups,
                        const float2* stats, const void* gamma, const void* beta, int64_t R, int64_t segments,
                        hipStream_t stream) {
  gn_apply_kernel<D, E, ACT><<<(unsigned)segments, kThreads, 0, stream>>>(x, y, n, channels, off, items, R, groups,
                                                                          stats, gamma, beta);
  return hipGetLastError();
}

template <DT D>
hipError_t launch_dtype(const void* x, int64_t n, int channels, const int64_t* off, int items, int groups,
                        const void* gamma, const void* beta, float eps, int act, void* y, float2* part,
                        int32_t* part_rows, double* slots, float2* stats, int64_t R, int64_t segments,
                        hipStream_t stream) {
  constexpr int E = D == DT::F32 ? 4 : 8;
  gn_partial_kernel<D, E><<<(unsigned)segments, kThreads, 0, stream>>>(x, n, channels, off, items, R, groups, part,
                                                                       part_rows);
  const PartialSpace<false> ps{part, part_rows, off, n, R, channels / groups};
  const int64_t ns = chunk_slots(items, segments);
  double* sn = slots;
  double* sm = slots + ns * groups;
  double* sq = slots + 2 * ns * groups;
  gn_chunk_kernel<false><<<(unsigned)ns, kChunkThreads, 0, stream>>>(ps, items, groups, sn, sm, sq);
  gn_finish_kernel<false><<<(unsigned)items, kStatThreads, 0, stream>>>(ps, groups, eps, sn, sm, sq, nullptr, nullptr,
                                                                        stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (act) {
    case SUBM_ACT_SILU:
      return launch_apply<D, E, SUBM_ACT_SILU>(x, y, n, channels, off, items, groups, stats, gamma, beta, R, segments,
                                       stream);
    case SUBM_ACT_RELU:
      return launch_apply<D, E, SUBM_ACT_RELU>(x, y, n, channels, off, items, groups, stats, gamma, beta, R, segments,
                                       stream);
    default:
      return launch_apply<D, E, SUBM_ACT_NONE>(x, y, n, channels, off, items, groups, stats, gamma, beta, R, segments,
                                       stream);
  }
}

// Host checks shared by both entry points (no HIP call).
Status check_norm(int64_t n, int channels, int dtype, int num_items, int groups, float eps, int act) {
  if (dtype != SUBM_F32 && dtype != SUBM_F16 && dtype != SUBM_BF16)
    return make_status(SUBM_ERR_UNSUPPORTED, "dtype must be SUBM_F32, SUBM_F16 or SUBM_BF16");
  if (act != SUBM_ACT_NONE && act != SUBM_ACT_SILU && act != SUBM_ACT_RELU)
    return make_status(SUBM_ERR_INVALID_ARG, "act must be SUBM_ACT_NONE, SUBM_ACT_SILU or SUBM_ACT_RELU");
  if (n < 0 || n > INT32_MAX) return make_status(SUBM_ERR_INVALID_ARG, "n must be in [0, 2^31 - 1]");
  if (channels < 1 || channels > 4096) return make_status(SUBM_ERR_INVALID_ARG, "channels must be in [1, 4096]");
  if (groups < 1 || channels % groups != 0) return make_status(SUBM_ERR_INVALID_ARG, "groups must divide channels");
  if (num_items < 1 || num_items > 65535) return make_status(SUBM_ERR_INVALID_ARG, "num_items must be in [1, 65535]");
  if (!(eps > 0.f) || !std::isfinite(eps)) return make_status(SUBM_ERR_INVALID_ARG, "eps must be a positive finite number");
  const int elem = dtype == SUBM_F32 ? 4 : 2;
  if ((channels * elem) % 16 != 0 || channels * elem > 4096)
    return make_status(SUBM_ERR_UNSUPPORTED, "rows must be a multiple of 16 bytes and at most 4096 bytes");
  return Status{};
}

Status check_norm_pointers(const void* x, const void* y, const int64_t* off, const void* gamma, const void* beta,
                           int dtype) {
  const int elem = dtype == SUBM_F32 ? 4 : 2;
  if (x == nullptr || y == nullptr || off == nullptr) return make_status(SUBM_ERR_INVALID_ARG, "x, y or item_offsets is NULL");
  if (((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) != 0)
    return make_status(SUBM_ERR_UNSUPPORTED, "x and y must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(off) & 7u) != 0) return make_status(SUBM_ERR_INVALID_ARG, "item_offsets is not 8-byte aligned");
  if (((reinterpret_cast<uintptr_t>(gamma) | reinterpret_cast<uintptr_t>(beta)) % elem) != 0)
    return make_status(SUBM_ERR_INVALID_ARG, "gamma / beta not aligned to the element size");
  return Status{};
}

// The statistics in the convolution epilogue cost more than the separate pass they replace on
// this GPU (the kernel runs one workgroup per compute unit, so the epilogue's extra latency is
// exposed: config 5 layer, 64 channels, 32 groups: 1.09 ms fused vs 0.95 ms conv + norm), so the
// separate pass is the default; SUBMCONV_GN_EPILOGUE=1 selects the epilogue statistics.
bool epilogue_statistics_enabled() {
  const char* v = std::getenv("SUBMCONV_GN_EPILOGUE");
  return v != nullptr && v[0] == '1';
}

// Segment length of the partials / apply passes for n rows.
int64_t segment_rows(int64_t n) {
  const int64_t rmul = std::max<int64_t>(1, (n + 256 * (int64_t)kMaxSegmentsPerRun - 1) / (256 * (int64_t)kMaxSegmentsPerRun));
  return 256 * rmul;
}

template <DT D>
hipError_t launch_apply_act(const void* x, void* y, int64_t n, int channels, const int64_t* off, int items, int groups,
                            const float2* stats, const void* gamma, const void* beta, int act, hipStream_t stream) {
  constexpr int E = D == DT::F32 ? 4 : 8;
  const int64_t R = segment_rows(n);
  const int64_t segments = items + (n + R - 1) / R;
  switch (act) {
    case SUBM_ACT_SILU:
      return launch_apply<D, E, SUBM_ACT_SILU>(x, y, n, channels, off, items, groups, stats, gamma, beta, R, segments, stream);
    case SUBM_ACT_RELU:
      return launch_apply<D, E, SUBM_ACT_RELU>(x, y, n, channels, off, items, groups, stats, gamma, beta, R, segments, stream);
    default:
      return launch_apply<D, E, SUBM_ACT_NONE>(x, y, n, channels, off, items, groups, stats, gamma, beta, R, segments, stream);
  }
}

// Statistics from the convolution's tile partials, then the apply pass in place.
template <DT D>
hipError_t launch_from_tiles(void* y, int64_t n, int channels, const int64_t* off, int items, int groups,
                             const void* gamma, const void* beta, float eps, int act, const float2* part, int64_t BM,
                             float2* bpart, int32_t* brows, double* slots, float2* stats, hipStream_t stream) {
  gn_boundary_kernel<D><<<(unsigned)(2 * items), kThreads, 0, stream>>>(y, n, channels, off, BM, groups, bpart, brows);
  const PartialSpace<true> ps{part, nullptr, off, n, BM, channels / groups};
  const int64_t ns = chunk_slots(items, (n + BM - 1) / BM);
  double* sn = slots;
  double* sm = slots + ns * groups;
  double* sq = slots + 2 * ns * groups;
  gn_chunk_kernel<true><<<(unsigned)ns, kChunkThreads, 0, stream>>>(ps, items, groups, sn, sm, sq);
  gn_finish_kernel<true><<<(unsigned)items, kStatThreads, 0, stream>>>(ps, groups, eps, sn, sm, sq, bpart, brows,
                                                                       stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_apply_act<D>(y, y, n, channels, off, items, groups, stats, gamma, beta, act, stream);
}

}  // namespace
}  // namespace submconv

using namespace submconv;

extern "C" int sparse_group_norm_act(const void* x, int64_t n, int channels, int dtype, const int64_t* item_offsets,
                                     int num_items, int groups, const void* gamma, const void* beta, float eps, int act,
                                     void* y, hipStream_t stream) {
  clear_error();
  Status st = check_norm(n, channels, dtype, num_items, groups, eps, act);
  if (!st.ok()) return fail(st);
  if (n == 0) return SUBM_OK;
  st = check_norm_pointers(x, y, item_offsets, gamma, beta, dtype);
  if (!st.ok()) return fail(st);
  const int64_t R = segment_rows(n);
  const int64_t segments = num_items + (n + R - 1) / R;
  const size_t part_bytes = (size_t)segments * groups * sizeof(float2);
  const size_t rows_bytes = ((size_t)segments * sizeof(int32_t) + 255) / 256 * 256;
  const size_t stats_bytes = ((size_t)num_items * groups * sizeof(float2) + 255) / 256 * 256;
  const size_t slot_bytes = (size_t)chunk_slots(num_items, segments) * groups * 3 * sizeof(double);
  void* scratch = nullptr;
  st = device_alloc(&scratch, part_bytes + rows_bytes + stats_bytes + slot_bytes, stream);
  if (!st.ok()) return fail(st);
  unsigned char* base = static_cast<unsigned char*>(scratch);
  float2* part = reinterpret_cast<float2*>(base);
  int32_t* part_rows = reinterpret_cast<int32_t*>(base + part_bytes);
  float2* stats = reinterpret_cast<float2*>(base + part_bytes + rows_bytes);
  double* slots = reinterpret_cast<double*>(base + part_bytes + rows_bytes + stats_bytes);
  hipError_t e;
  switch (dtype) {
    case SUBM_F32:
      e = launch_dtype<DT::F32>(x, n, channels, item_offsets, num_items, groups, gamma, beta, eps, act, y, part,
                                part_rows, slots, stats, R, segments, stream);
      break;
    case SUBM_F16:
      e = launch_dtype<DT::F16>(x, n, channels, item_offsets, num_items, groups, gamma, beta, eps, act, y, part,
                                part_rows, slots, stats, R, segments, stream);
      break;
    default:
      e = launch_dtype<DT::BF16>(x, n, channels, item_offsets, num_items, groups, gamma, beta, eps, act, y, part,
                                 part_rows, slots, stats, R, segments, stream);
      break;
  }
  device_free(scratch, stream);
  if (e != hipSuccess) return fail(hip_status(e, "sparse_group_norm_act launch"));
  return SUBM_OK;
}

extern "C" int subm_conv3d_forward_group_norm_act(submconv_map_t map, int64_t n, int ksize, int cin, int cout,
                                                  int dtype, const void* feats, const void* weight, const void* bias,
                                                  const int64_t* item_offsets, int num_items, int groups,
                                                  const void* gamma, const void* beta, float eps, int act, void* out,
                                                  hipStream_t stream) {
  clear_error();
  Status st = check_conv(map, n, ksize, cin, cout, dtype, feats, weight, bias, out);
  if (st.ok()) st = check_norm(n, cout, dtype, num_items, groups, eps, act);
  if (!st.ok()) return fail(st);
  if (n == 0) return SUBM_OK;
  st = check_norm_pointers(out, out, item_offsets, gamma, beta, dtype);
  if (!st.ok()) return fail(st);
  map_note_use(map, stream);
  const MapData* md = map == nullptr ? nullptr : &map->d;
  // Scratch for the fused path (tile partials for the shortest tiles, boundary pieces, statistics).
  const int64_t max_tiles = (n + 191) / 192;
  const size_t part_bytes = ((size_t)max_tiles * groups * sizeof(float2) + 255) / 256 * 256;
  const size_t bpart_bytes = ((size_t)2 * num_items * groups * sizeof(float2) + 255) / 256 * 256;
  const size_t brows_bytes = ((size_t)2 * num_items * sizeof(int32_t) + 255) / 256 * 256;
  const size_t stats_bytes = ((size_t)num_items * groups * sizeof(float2) + 255) / 256 * 256;
  const size_t slot_bytes = (size_t)chunk_slots(num_items, max_tiles) * groups * 3 * sizeof(double);
  void* scratch = nullptr;
  st = device_alloc(&scratch, part_bytes + bpart_bytes + brows_bytes + stats_bytes + slot_bytes, stream);
  if (!st.ok()) return fail(st);
  unsigned char* base = static_cast<unsigned char*>(scratch);
  float2* part = reinterpret_cast<float2*>(base);
  float2* bpart = reinterpret_cast<float2*>(base + part_bytes);
  int32_t* brows = reinterpret_cast<int32_t*>(base + part_bytes + bpart_bytes);
  float2* stats = reinterpret_cast<float2*>(base + part_bytes + bpart_bytes + brows_bytes);
  double* slots = reinterpret_cast<double*>(base + part_bytes + bpart_bytes + brows_bytes + stats_bytes);
  int tile_rows = 0;
  hipError_t e = epilogue_statistics_enabled()
                     ? launch_subm_conv_gn_partials(md, n, ksize, cin, cout, dtype, feats, weight, bias, out, part,
                                                    cout / groups, groups, &tile_rows, stream)
                     : hipErrorNotSupported;
  if (e == hipSuccess) {
    e = dtype == SUBM_F16
            ? launch_from_tiles<DT::F16>(out, n, cout, item_offsets, num_items, groups, gamma, beta, eps, act, part,
                                         tile_rows, bpart, brows, slots, stats, stream)
            : launch_from_tiles<DT::BF16>(out, n, cout, item_offsets, num_items, groups, gamma, beta, eps, act, part,
                                          tile_rows, bpart, brows, slots, stats, stream);
    device_free(scratch, stream);
  } else if (e == hipErrorNotSupported) {
    (void)hipGetLastError();
    device_free(scratch, stream);
    // Plain convolution, then the separate normalisation in place.
    e = launch_subm_conv(md, n, ksize, cin, cout, dtype, feats, weight, bias, out, stream);
    if (e == hipSuccess) {
      const int rc = sparse_group_norm_act(out, n, cout, dtype, item_offsets, num_items, groups, gamma, beta, eps, act,
                                           out, stream);
      if (rc != SUBM_OK) return rc;
    }
  } else {
    device_free(scratch, stream);
  }
  if (e != hipSuccess) return fail(hip_status(e, "subm_conv3d_forward_group_norm_act launch"));
  return SUBM_OK;
}
