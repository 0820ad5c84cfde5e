// Matrix-core rate of this GPU at the clock it holds under that load, for the measured ceiling
// beside the published one: every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on register
// operands (eight independent accumulators, no memory traffic in the loop), two waves per SIMD.
// Each workgroup records its wave 0's s_memtime (shader clock) and s_memrealtime (a constant
// 100 MHz) spans around the loop, so the clock the loop ran at follows from their ratio.
#include "device_common.h"
#include "internal.h"

namespace submconv {
namespace {

constexpr int kRateThreads = 256;

// Two bf16 values in [1, 2) with random mantissas (no NaN or infinity, data that toggles).
__device__ __forceinline__ uint32_t bf16_pair(uint32_t r) {
  return (0x3F80u | (r & 0x7Fu)) | ((0x3F80u | ((r >> 16) & 0x7Fu)) << 16);
}

__global__ __launch_bounds__(kRateThreads) void mfma_rate_kernel(int64_t iters, float* __restrict__ sink,
                                                                 uint64_t* __restrict__ clocks) {
  uint32_t h = ((uint32_t)blockIdx.x * kRateThreads + threadIdx.x + 1u) * 2654435761u;
  auto next = [&]() {  // xorshift32 (Marsaglia)
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    return h;
  };
  const uint4 a = make_uint4(bf16_pair(next()), bf16_pair(next()), bf16_pair(next()), bf16_pair(next()));
  const uint4 b = make_uint4(bf16_pair(next()), bf16_pair(next()), bf16_pair(next()), bf16_pair(next()));
  f32x16_t acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = mfma32<DT::BF16>(a, b, acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[(int64_t)blockIdx.x * kRateThreads + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clocks[2 * (int64_t)blockIdx.x] = t1 - t0;
    clocks[2 * (int64_t)blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace
}  // namespace submconv

using namespace submconv;

extern "C" int subm_mfma_rate(int64_t iters, int blocks, float* sink, uint64_t* clocks, hipStream_t stream) {
  clear_error();
  if (iters < 1 || blocks < 1 || blocks > 65535) return fail(SUBM_ERR_INVALID_ARG, "iters >= 1 and 1 <= blocks <= 65535");
  if (sink == nullptr || clocks == nullptr) return fail(SUBM_ERR_INVALID_ARG, "sink or clocks is NULL");
  mfma_rate_kernel<<<blocks, kRateThreads, 0, stream>>>(iters, sink, clocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(hip_status(e, "subm_mfma_rate launch"));
  return SUBM_OK;
}
