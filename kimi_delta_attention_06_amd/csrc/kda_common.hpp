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

// sum over the 16 lanes of each DPP row, returned to every lane of the row
template <int N>
__device__ __forceinline__ float row_shr_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 | N, 0xf,
                                                                       0xf, false));
}
__device__ __forceinline__ float row_sum16(float x) {
  x = row_shr_add<1>(x);
  x = row_shr_add<2>(x);
  x = row_shr_add<4>(x);
  x = row_shr_add<8>(x);
  // lane 15 of the row now holds the total: DPP row_newbcast:15 (writes every lane: no old value)
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x15f, 0xf, 0xf, false));
}

}  // namespace kda
