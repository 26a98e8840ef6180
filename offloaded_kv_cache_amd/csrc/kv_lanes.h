// kv_lanes.h - lane exchanges within a 64-wide wavefront without the LDS crossbar
// (gfx950): DPP lane selects inside rows of 16 lanes and the row / half-wave swaps.
#pragma once

#include "kv_internal.h"

namespace kvc {

// Lane exchanges without the LDS crossbar: the value of lane (lane ^ M). M = 1, 2, 8
// are DPP lane selects inside a row of 16 (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_ror:8); M = 4 is row_half_mirror (lane ^ 7) then quad_perm [3,2,1,0] (lane ^ 3);
// M = 16 and 32 are the row and half-wave swaps of gfx950, whose second result holds
// the partner's value in the lower rows and the first result in the upper ones.
typedef uint32_t swap2 __attribute__((ext_vector_type(2)));
template <int M>
__device__ inline uint32_t xchg32(uint32_t v, int lane) {
  if (M == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  if (M == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  if (M == 4) {
    const int t = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
    return (uint32_t)__builtin_amdgcn_mov_dpp(t, 0x1B, 0xF, 0xF, false);
  }
  if (M == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
  if (M == 16) {
    const swap2 r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  }
  const swap2 r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (lane & 32) ? r[0] : r[1];
}
template <int M>
__device__ inline double xchg64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = xchg32<M>((uint32_t)b, lane), hi = xchg32<M>((uint32_t)(b >> 32), lane);
  return __builtin_bit_cast(double, (hi << 32) | lo);
}

template <int M>
__device__ inline float xchgf(float v, int lane) {
  return __builtin_bit_cast(float, xchg32<M>(__builtin_bit_cast(uint32_t, v), lane));
}

}  // namespace kvc
