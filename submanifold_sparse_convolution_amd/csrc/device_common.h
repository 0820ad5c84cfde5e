// Device helpers shared by the matrix-core kernels: storage types and conversions, the
// matrix-core instructions, buffer resources, direct-to-LDS loads and explicit waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace submconv {

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

template <DT D> __device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c);
template <> __device__ __forceinline__ f32x16_t mfma32<DT::BF16>(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16_t mfma32<DT::F16>(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Four fp32 values -> four 16-bit storage elements packed into 8 bytes, rounded to nearest even
// (hardware conversions: v_cvt_pk_bf16_f32, v_cvt_f16_f32).
template <DT D> __device__ __forceinline__ uint2 pack4(float a, float b, float c, float d);
template <> __device__ __forceinline__ uint2 pack4<DT::BF16>(float a, float b, float c, float d) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t lo = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  const bf16x2_t hi = __builtin_convertvector((f32x2_t){c, d}, bf16x2_t);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}
template <> __device__ __forceinline__ uint2 pack4<DT::F16>(float a, float b, float c, float d) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t lo = __builtin_convertvector((f32x2_t){a, b}, f16x2_t);
  const f16x2_t hi = __builtin_convertvector((f32x2_t){c, d}, f16x2_t);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

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

// Whether any of flags[0 .. count) is nonzero, the same answer in every thread of the workgroup.
// Every thread of the workgroup must call it: it synchronises the workgroup.
__device__ __forceinline__ bool pool_any_flag(const uint32_t* flags, int count) {
  __shared__ uint32_t s_any;
  if (threadIdx.x == 0) s_any = 0u;
  __syncthreads();
  uint32_t v = 0u;
  for (int k = threadIdx.x; k < count; k += blockDim.x) v |= flags[k];
  if (v != 0u) s_any = 1u;  // (every writer stores 1)
  __syncthreads();
  return s_any != 0u;
}

}  // namespace submconv
