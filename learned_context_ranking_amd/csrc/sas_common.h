// Shared device helpers for the gfx950 kernels: vector types, MFMA wrappers, bf16
// conversion and wave-level reductions. Host code includes it only for the types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sas {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64;                 // tokens per block (the pages' b)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-byte global / LDS accesses of raw bf16 bit patterns.
__device__ __forceinline__ u16x8 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u16x8*>(p);
}
__device__ __forceinline__ void st16(uint16_t* p, u16x8 v) {
  *reinterpret_cast<u16x8*>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Lane l supplies A row l%32 and B column l%32 with the 8 k-values of half l/32; the
// accumulator element i of lane l is D[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(16x16) += A(16x32) * B(32x16); lane l supplies A row l%16 / B column l%16 with the
// 8 k-values of quarter l/16; accumulator element i of lane l is D[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 round-to-nearest-even (inputs here are finite).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4,
                                         float a5, float a6, float a7) {
  u16x8 v;
  v[0] = f2bf(a0); v[1] = f2bf(a1); v[2] = f2bf(a2); v[3] = f2bf(a3);
  v[4] = f2bf(a4); v[5] = f2bf(a5); v[6] = f2bf(a6); v[7] = f2bf(a7);
  return as_bf16x8(v);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Position of key k within its 16-key group when a transposed operand is staged in LDS
// so that each lane's 8 MFMA k-values are contiguous: a 32x32x16 accumulator gives lane
// half h the keys {4h..4h+3, 8+4h..8+4h+3}; swapping bits 2 and 3 of the key makes them
// positions 8h..8h+7.
__device__ __forceinline__ int perm32(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}
// The same for the 16x16x32 accumulator pairs used by the key-major backward: within a
// 32-query group, query q' = 16a + 4g + r (a<2, g<4, r<4) is stored at 8g + 4a + r.
__device__ __forceinline__ int perm16(int q) {
  return (q & ~31) | (((q >> 2) & 3) << 3) | (((q >> 4) & 1) << 2) | (q & 3);
}

}  // namespace sas
