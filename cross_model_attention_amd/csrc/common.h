// Device helpers shared by the libmapflow kernels (gfx950 / CDNA4, wave64).
//
// MFMA operand layouts used throughout (v_mfma_f32_16x16x32_{bf16,f16}; lane l, a = l / 16,
// c = l % 16):
//   A operand (16 x 32):  lane holds A[c][8a + e],  e = 0..7
//   B operand (32 x 16):  lane holds B[8a + e][c]
//   C / D     (16 x 16):  lane holds D[4a + i][c],  i = 0..3
// v_mfma_f32_16x16x4_f32: A lane holds A[c][a], B lane holds B[a][c], same C layout.
#pragma once


#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mf {

typedef short v8s __attribute__((__vector_size__(8 * sizeof(short))));
typedef _Float16 v8h __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float v4f __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t v4u __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));   // converts with v_cvt_pk_bf16_f32 (RNE)
typedef _Float16 h2 __attribute__((ext_vector_type(2))); // converts with v_cvt_pk_f16_f32 (RNE)

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ v4f mfma_bf16(v8s a, v8s b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f32(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f zero4() { return v4f{0.f, 0.f, 0.f, 0.f}; }

// 16-byte loads.  `nt` loads are streamed once (kept-block probabilities) and bypass reuse.
__device__ __forceinline__ v4u ld16(const void* p) { return *reinterpret_cast<const v4u*>(p); }
__device__ __forceinline__ v4u ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
}
__device__ __forceinline__ void st16(void* p, v4u v) { *reinterpret_cast<v4u*>(p) = v; }

// Device-memory pointers kept in LDS or registers lose the compiler's knowledge that they point
// to global memory, and accesses through them become flat accesses (which also count against the
// LDS wait counter).  This qualifier keeps them global.
#define MF_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ v4u ld16(const MF_GLOBAL void* p) {
  return *reinterpret_cast<const MF_GLOBAL v4u*>(p);
}

__device__ __forceinline__ v8s as_v8s(v4u v) { return __builtin_bit_cast(v8s, v); }
__device__ __forceinline__ v8h as_v8h(v4u v) { return __builtin_bit_cast(v8h, v); }
__device__ __forceinline__ v4u zero_u4() { return v4u{0u, 0u, 0u, 0u}; }

// bf16 <-> fp32 (bf16 is the upper half of an fp32 bit pattern).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even; inputs here are finite.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = static_cast<_Float16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// max / sum over the four 16-lane rows of a wave (lanes c, c+16, c+32, c+48), result in every
// lane: the gfx950 row-swap permutes exchange halves and row pairs without going through LDS
__device__ __forceinline__ float xrow_max(float v) {
  auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __builtin_fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float xrow_sum(float v) {
  auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// fp64 sum over the wave: rows by DPP on both 32-bit halves, then rows 0..3 added in order;
// uniform result.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0x128>(v);
  v += dpp_f64<0x124>(v);
  v += dpp_f64<0x122>(v);
  v += dpp_f64<0x121>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS (and scalar memory)
// operations, then the hardware barrier.  __syncthreads also carries a release fence, which
// waits for every outstanding global store and load of the wave; in a loop that streams stores
// and prefetches loads across block boundaries that fence would drain both at every barrier.
// Use it where only LDS data (including LDS filled by DMA after its own explicit wait) is
// exchanged between the waves.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per block row: {first token of the row, first token of its sequence, sequence length, I}.
struct BrowInfo {
  int tok0, seq0, n, I;
};
__device__ __forceinline__ BrowInfo load_info(const int32_t* info, int b) {
  const int4 v = reinterpret_cast<const int4*>(info)[b];
  return BrowInfo{v.x, v.y, v.z, v.w};
}

}  // namespace mf
