// Shared device helpers for the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;

// bf16 storage is passed around as its 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x.bits) << 16); }

// Two packed bf16 (one 32-bit word) -> two floats, exact.
__device__ __forceinline__ float2 bf16x2_to_f32x2(uint32_t w) {
  return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

template <typename T>
__device__ __forceinline__ T wave_xor(T x, int mask) {
  return __shfl_xor(x, mask, kWave);
}

}  // namespace kda
