// kv_encode.h - per-wave record encoder shared by the append kernel and the
// decode kernel's fused single-token append (gfx950).
//
// Strata page ("KV 沉进内存、显存减半：Strata 让 12 GB 显卡跑满 262K 上下文"),
// section "4-bit KV 缓存：先旋转，再压到 4-bit": K and V are rotated by the
// 256-point Walsh-Hadamard matrix and stored as q4_0 blocks when written;
// section "三种 KV 格式横向对比": int8 (per-64 scales) and k8v4 (int8 K,
// rotated q4_0 V). The rounding rules are those of include/kvcache.h.
//
// One wave encodes one vector. Lane l holds elements e = l + 64k (k = 0..3).
// The rotation is done in fp64, where it is exact for fp16 inputs (partial sums
// are multiples of 2^-28 below 2^20): stages for bits 0..5 exchange between
// lanes, bits 6 and 7 are inside the lane.
#pragma once

#include "kv_internal.h"

namespace kvc {
namespace enc {

// Maximum over the wave of each of the lane's four values (exchanges of the four
// values are issued together).
__device__ inline void wave_max4(double (&v)[4]) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    double t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = __shfl_xor(v[k], o);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = fmax(v[k], t[k]);
  }
}

// Exact y = H x on the lane's four elements.
__device__ inline void wht256(double (&y)[4], int lane) {
#pragma unroll
  for (int bit = 0; bit < 6; ++bit) {
    const int m = 1 << bit;
    const bool upper = lane & m;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double o = __shfl_xor(y[k], m);
      y[k] = upper ? (o - y[k]) : (y[k] + o);
    }
  }
  const double a0 = y[0] + y[1], a1 = y[0] - y[1];  // bit 6
  const double a2 = y[2] + y[3], a3 = y[2] - y[3];
  y[0] = (a0 + a2) * 0.0625;                          // bit 7, then 1/16
  y[2] = (a0 - a2) * 0.0625;
  y[1] = (a1 + a3) * 0.0625;
  y[3] = (a1 - a3) * 0.0625;
}

// The record of one vector: codes of the lane's elements and the scales.
// int8: scale[k] is group k (elements 64k..64k+63 are exactly register k).
// q4: scale of block (lane >> 5) + 2k lives in register k of every lane of
// that half-wave.
template <int KIND>
__device__ inline void encode_vals(const uint16_t (&in)[4], int lane, int (&code)[4],
                                   uint16_t (&scale)[4]) {
  double x[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) x[k] = f16_to_f64(in[k]);
  if (KIND == kInt8) {
    double a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = fabs(x[k]);
    wave_max4(a);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      scale[k] = f64_to_f16_rne(a[k] / 127.0);
      code[k] = int8_code(x[k], f16_to_f64(scale[k]));
    }
  } else {
    wht256(x, lane);
    // per block (the 32 lanes of a half-wave, register k): largest |y|, then the
    // first element holding it, then its signed value
    double m[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = fabs(x[k]);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      double t[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) t[k] = __shfl_xor(m[k], o);
#pragma unroll
      for (int k = 0; k < 4; ++k) m[k] = fmax(m[k], t[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint64_t hit = __ballot(fabs(x[k]) == m[k]);
      const uint32_t half = (lane & 32) ? (uint32_t)(hit >> 32) : (uint32_t)hit;
      // (no hit only for NaN inputs, whose codes are unspecified)
      const double best = __shfl(x[k], (lane & 32) + (half ? __builtin_ctz(half) : (lane & 31)));
      scale[k] = f64_to_f16_rne(-best * 0.125);  // -m/8 is exact in fp64
      code[k] = q4_code(x[k], f16_to_f64(scale[k]));
    }
  }
}

// The lane's four fp16 inputs of a vector (elements lane + 64k).
__device__ inline void load_vals(const uint16_t* __restrict__ src, int lane, uint16_t (&in)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) in[k] = src[lane + 64 * k];
}

template <int KIND>
__device__ inline void encode(const uint16_t* __restrict__ src, int lane, int (&code)[4],
                              uint16_t (&scale)[4]) {
  uint16_t in[4];
  load_vals(src, lane, in);
  encode_vals<KIND>(in, lane, code, scale);
}

// K plane row of a token (token-major, slice-permuted code bytes).
template <int KIND>
__device__ inline void write_k_row(uint8_t* __restrict__ plane, int row, int lane,
                                   const int (&code)[4], const uint16_t (&scale)[4]) {
  uint8_t* codes = plane + (size_t)row * code_row_bytes(KIND);
  uint16_t* scales = reinterpret_cast<uint16_t*>(plane + kPageTokens * code_row_bytes(KIND)) +
                     row * n_scales(KIND);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = lane + 64 * k;
    const int j = e >> 5, r = e & 31;
    if (KIND == kInt8) {
      codes[64 * (r >> 3) + 8 * j + (r & 7)] = (uint8_t)(int8_t)code[k];
    } else {
      const int partner = __shfl_xor(code[k], 16);  // element e ^ 16, same block
      if (r < 16) codes[32 * (r >> 2) + 4 * j + (r & 3)] = (uint8_t)(code[k] | (partner << 4));
    }
  }
  if (KIND == kInt8) {
    if (lane < 4) {
      uint16_t s = scale[0];
      if (lane == 1) s = scale[1];
      if (lane == 2) s = scale[2];
      if (lane == 3) s = scale[3];
      scales[lane] = s;
    }
  } else if ((lane & 31) == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) scales[(lane >> 5) + 2 * k] = scale[k];
  }
}

template <int KIND>
__device__ inline void write_v_scales(uint8_t* __restrict__ plane, int row, int lane,
                                      const uint16_t (&scale)[4]) {
  uint16_t* sc = reinterpret_cast<uint16_t*>(plane + kHeadDim * code_row_bytes(KIND));
  if (KIND == kInt8) {
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) sc[k * kPageTokens + row] = scale[k];
    }
  } else if ((lane & 31) == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) sc[((lane >> 5) + 2 * k) * kPageTokens + row] = scale[k];
  }
}

// V codes of one token, written alone. int8: one byte per element. 4-bit: each
// byte of the element-major V plane pairs tokens 32G+i (low nibble) and 32G+16+i
// (high nibble); the token's nibble is replaced by an atomic AND then OR on the
// containing dword, so the partner's nibble is kept without a read round trip
// (nothing else writes these bytes while the token is appended).
template <int KIND>
__device__ inline void write_v_codes_one(uint8_t* __restrict__ plane, int row, int lane,
                                         const int (&code)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = lane + 64 * k;
    if (KIND == kInt8) {
      plane[(size_t)e * code_row_bytes(KIND) + row] = (uint8_t)(int8_t)code[k];
    } else {
      const size_t off = (size_t)e * code_row_bytes(KIND) + 16 * (row >> 5) + (row & 15);
      uint32_t* w = reinterpret_cast<uint32_t*>(plane + (off & ~(size_t)3));
      const int bit = 8 * (int)(off & 3) + ((row & 16) ? 4 : 0);
      atomicAnd(w, ~(0xFu << bit));
      atomicOr(w, (uint32_t)code[k] << bit);
    }
  }
}

}  // namespace enc
}  // namespace kvc
