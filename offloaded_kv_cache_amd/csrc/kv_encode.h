// kv_encode.h - per-wave record encoder of the decode kernel's fused single-token
// append (gfx950); the chunk append kernel (kv_append.hip) uses its scale rounding and
// exact code decisions.
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
// lanes (DPP lane selects and lane swaps, no LDS), bits 6 and 7 are inside the
// lane. Scales are rounded to fp16 and codes decided without branches on
// per-lane data and without fp64 division, each decision being the exact one.
#pragma once

#include "kv_lanes.h"

namespace kvc {
namespace enc {

// One butterfly stage (bit log2 M) and one max stage on the lane's four values. Lane
// exchanges are DPP selects and lane swaps (a lone vector is latency bound); the
// rounding is branch-free and the codes are decided without division.
// (partner + y in the lower lane of a pair, partner - y in the upper one, each as one fma
// with a sign of +-1: the product is exact, and so is the sum, whose exact value is
// representable, so the result is the exact butterfly)
template <int M>
__device__ inline void wht_stage(double (&y)[4], int lane) {
  const double sg = (lane & M) ? -1.0 : 1.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double o = xchg64<M>(y[k], lane);
    y[k] = __builtin_fma(sg, y[k], o);
  }
}
template <int M>
__device__ inline void max_stage(double (&v)[4], int lane) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = fmax(v[k], xchg64<M>(v[k], lane));
}

// Maximum over the wave of each of the lane's four values.
__device__ inline void wave_max4(double (&v)[4], int lane) {
  max_stage<1>(v, lane);
  max_stage<2>(v, lane);
  max_stage<4>(v, lane);
  max_stage<8>(v, lane);
  max_stage<16>(v, lane);
  max_stage<32>(v, lane);
}

// Exact y = H x on the lane's four elements.
__device__ inline void wht256(double (&y)[4], int lane) {
  wht_stage<1>(y, lane);
  wht_stage<2>(y, lane);
  wht_stage<4>(y, lane);
  wht_stage<8>(y, lane);
  wht_stage<16>(y, lane);
  wht_stage<32>(y, lane);
  const double a0 = y[0] + y[1], a1 = y[0] - y[1];  // bit 6
  const double a2 = y[2] + y[3], a3 = y[2] - y[3];
  y[0] = (a0 + a2) * 0.0625;                          // bit 7, then 1/16
  y[2] = (a0 - a2) * 0.0625;
  y[1] = (a1 + a3) * 0.0625;
  y[3] = (a1 - a3) * 0.0625;
}

// fp64 -> fp16, round to nearest even, without branches: x is rounded to fp32 with
// round-to-odd (the fp32 nearest, moved toward zero by one unit if it lies beyond x,
// and its last bit set whenever it is not x), then to fp16 with round to nearest even.
// fp32 keeps 13 bits more than fp16 (and reaches 2^-149 against fp16's 2^-24), so the
// odd last bit stands for every discarded bit and the second rounding is the one an
// exact rounding of x would make. Overflow gives infinity.
__device__ inline uint16_t f64_to_f16_fast(double x) {
  const float f = (float)x;
  const uint32_t fb = __builtin_bit_cast(uint32_t, f);
  const double fd = (double)f;
  const uint32_t beyond = fabs(fd) > fabs(x) ? 1u : 0u;  // toward zero by one unit (same sign)
  const uint32_t odd = ((fb - beyond) | 1u);
  const uint32_t r = fd != x ? odd : fb;
  return __builtin_bit_cast(uint16_t, (_Float16)__builtin_bit_cast(float, r));
}

// Codes decided exactly without a division: an fp32 estimate of x/d, then the exact
// tests of the rounding thresholds (c +- 1/2) * |d|, which are fp64 products of an
// 11-bit scale and a 6-bit constant. The estimate is within a small fraction of a unit
// of x/d (|x/d| is at most about 128), so at most one correction applies.
// The integer c with (c - 1/2) ad <= sx < (c + 1/2) ad (ties upward), ad > 0.
__device__ inline double round_quotient(double sx, double ad) {
  double c = __builtin_floor((double)((float)sx * __builtin_amdgcn_rcpf((float)ad)) + 0.5);
  c += sx >= (c + 0.5) * ad ? 1.0 : 0.0;
  c -= sx < (c - 0.5) * ad ? 1.0 : 0.0;
  return c;
}
// int8: round half away from zero of x/d, clamped to +-127 (d >= 0).
__device__ inline int int8_code_fast(double x, double d) {
  const double c = round_quotient(fabs(x), d == 0.0 ? 1.0 : d);
  const int ci = d == 0.0 ? 0 : (c > 127.0 ? 127 : (int)c);
  return x < 0 ? -ci : ci;
}
// q4: floor(y/d + 1/2) + 8, clamped to [0, 15].
__device__ inline int q4_code_fast(double y, double d) {
  const double c = round_quotient(d < 0 ? -y : y, d == 0.0 ? 1.0 : fabs(d)) + 8.0;
  return d == 0.0 ? 8 : (c < 0.0 ? 0 : (c > 15.0 ? 15 : (int)c));
}

// The record of one vector: codes of the lane's elements and the scales.
// int8: scale[k] is group k (elements 64k..64k+63 are exactly register k).
// fp8: every scale[k] is the vector's one scale.
// q4, fp4: scale of block (lane >> 5) + 2k lives in register k of every lane of
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
    wave_max4(a, lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      scale[k] = f64_to_f16_fast(a[k] / 127.0);
      const double d = f16_to_f64(scale[k]);
      code[k] = int8_code_fast(x[k], d);
    }
  } else if (KIND == kFp8) {
    // one scale for the vector: the largest |x| over the wave's four registers
    double a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = fabs(x[k]);
    wave_max4(a, lane);
    const double amax = fmax(fmax(a[0], a[1]), fmax(a[2], a[3]));
    const uint16_t s = f64_to_f16_fast(amax / 448.0);
    const double d = f16_to_f64(s);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      scale[k] = s;
      code[k] = fp8_code(x[k], d);
    }
  } else if (KIND == kFp4) {
    wht256(x, lane);
    // per block (the 32 lanes of a half-wave, register k): largest |y|, its exponent,
    // the power-of-two scale and the grid index of each element (exact comparisons)
    double m[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = fabs(x[k]);
    max_stage<1>(m, lane);
    max_stage<2>(m, lane);
    max_stage<4>(m, lane);
    max_stage<8>(m, lane);
    max_stage<16>(m, lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = fp4_block_exp(m[k]);
      scale[k] = m[k] == 0.0 ? (uint16_t)0 : fp16_pow2_bits(e);
      code[k] = m[k] == 0.0 ? 0 : fp4_code(x[k], e);
    }
  } else {
    wht256(x, lane);
    // per block (the 32 lanes of a half-wave, register k): largest |y|, then the
    // first element holding it, then its signed value
    double m[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = fabs(x[k]);
    max_stage<1>(m, lane);
    max_stage<2>(m, lane);
    max_stage<4>(m, lane);
    max_stage<8>(m, lane);
    max_stage<16>(m, lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint64_t hit = __ballot(fabs(x[k]) == m[k]);
      // (no hit only for NaN inputs, whose codes are unspecified)
      const int i_lo = (uint32_t)hit ? __builtin_ctz((uint32_t)hit) : 0;
      const int i_hi = 32 + ((uint32_t)(hit >> 32) ? __builtin_ctz((uint32_t)(hit >> 32)) : 0);
      // both halves' values read as scalars, then each lane keeps its half's
      const uint64_t xb = __builtin_bit_cast(uint64_t, x[k]);
      const uint32_t l0 = __builtin_amdgcn_readlane((uint32_t)xb, i_lo), l1 = __builtin_amdgcn_readlane((uint32_t)xb, i_hi);
      const uint32_t h0 = __builtin_amdgcn_readlane((uint32_t)(xb >> 32), i_lo),
                     h1 = __builtin_amdgcn_readlane((uint32_t)(xb >> 32), i_hi);
      const uint32_t sel = (lane & 32) ? ~0u : 0u;
      const double best = __builtin_bit_cast(double, ((uint64_t)(h0 ^ ((h0 ^ h1) & sel)) << 32) | (l0 ^ ((l0 ^ l1) & sel)));
      scale[k] = f64_to_f16_fast(-best * 0.125);  // -m/8 exact
      const double d = f16_to_f64(scale[k]);
      code[k] = q4_code_fast(x[k], d);
    }
  }
}

// The lane's four fp16 inputs of a vector (elements lane + 64k).
__device__ inline void load_vals(const uint16_t* __restrict__ src, int lane, uint16_t (&in)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) in[k] = src[lane + 64 * k];
}

// K plane row of a token (token-major, slice-permuted code bytes): its code bytes at
// `codes`, its n_scales(KIND) fp16 scales at `scales` (in the plane, or a staging copy).
template <int KIND>
__device__ inline void write_k_row_at(uint8_t* __restrict__ codes, uint16_t* __restrict__ scales, int lane,
                                      const int (&code)[4], const uint16_t (&scale)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = lane + 64 * k;
    const int j = e >> 5, r = e & 31;
    if (!four_bit(KIND)) {
      codes[64 * (r >> 3) + 8 * j + (r & 7)] = (uint8_t)code[k];
    } else {
      const int partner = (int)xchg32<16>((uint32_t)code[k], lane);  // element e ^ 16, same block
      if (r < 16) codes[32 * (r >> 2) + 4 * j + (r & 3)] = (uint8_t)(code[k] | (partner << 4));
    }
  }
  if (KIND == kFp8) {
    if (lane == 0) scales[0] = scale[0];
  } else if (KIND == kInt8) {
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
__device__ inline void write_k_row(uint8_t* __restrict__ plane, int row, int lane, const int (&code)[4],
                                   const uint16_t (&scale)[4]) {
  write_k_row_at<KIND>(plane + (size_t)row * code_row_bytes(KIND),
                       reinterpret_cast<uint16_t*>(plane + kPageTokens * code_row_bytes(KIND)) + row * n_scales(KIND),
                       lane, code, scale);
}

template <int KIND>
__device__ inline void write_v_scales(uint8_t* __restrict__ plane, int row, int lane,
                                      const uint16_t (&scale)[4]) {
  uint16_t* sc = reinterpret_cast<uint16_t*>(plane + kHeadDim * code_row_bytes(KIND));
  if (KIND == kFp8) {
    if (lane == 0) sc[row] = scale[0];
  } else if (KIND == kInt8) {
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) sc[k * kPageTokens + row] = scale[k];
    }
  } else if ((lane & 31) == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) sc[((lane >> 5) + 2 * k) * kPageTokens + row] = scale[k];
  }
}

// V codes of one token, written alone. int8, fp8: one byte per element. 4-bit: each
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
    if (!four_bit(KIND)) {
      plane[(size_t)e * code_row_bytes(KIND) + row] = (uint8_t)code[k];
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
