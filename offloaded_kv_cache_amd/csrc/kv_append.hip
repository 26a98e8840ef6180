// kv_append.hip - quantize-on-append into the paged pool (gfx950).
//
// Strata page ("KV 沉进内存、显存减半：Strata 让 12 GB 显卡跑满 262K 上下文"),
// section "4-bit KV 缓存：先旋转，再压到 4-bit": K and V are rotated by the
// 256-point Walsh-Hadamard matrix and stored as q4_0 blocks when written;
// section "三种 KV 格式横向对比": int8 (per-64 scales) and k8v4 (int8 K,
// rotated q4_0 V). The rounding rules are those of include/kvcache.h.
//
// One workgroup of 16 waves handles a 32-token group (tokens 32G .. 32G+31, which
// lie in one page) of one KV head: waves 0-7 encode the group's K vectors, waves 8-15
// its V vectors, four vectors per wave. Lane l of a wave holds vector l >> 4, elements
// 16 (l & 15) + i (i = 0..15): the rotation's stages for element bits 0-3 run inside the
// lane and those for bits 4-7 between the 16 lanes of a row, and a 32-element block is
// two neighbouring lanes, a 64-element group four. The fp64 rotation is exact for fp16
// inputs (partial sums are multiples of 2^-24 below 2^24 before the 1/16), so the order
// of its stages does not change the result; scales and codes follow the rounding rules
// of include/kvcache.h exactly (kv_encode.h). A V wave holds tokens (i, i + 16) in
// vectors v and v + 2, whose 4-bit codes share the bytes of the element-major V plane.
// The records are assembled in LDS and then written whole: the group's K rows and
// scale rows are contiguous in the token-major K plane, and in the element-major V
// plane each of the 256 element rows receives one 16-byte (4-bit codes) or 32-byte
// (8-bit codes) segment, instead of one byte per token. Tokens of the group outside
// the chunk keep their bytes: the segments of a partly covered group are merged with
// the bytes already in the pool, code by code (a 4-bit V byte holds two tokens), and
// only the covered tokens' K rows and scales are written. Appends to one page from
// different calls must be ordered.
#include <hip/hip_ext.h>

#include "kv_encode.h"

namespace kvc {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 32;                // tokens of a work item
constexpr int kAppendWaves = 16;
constexpr int kAppendThreads = 64 * kAppendWaves;

// Row of V element e in the LDS staging of the element-major V plane. A staging store
// has the 16 lanes of a row write elements 16 s + c (s = 0..15) of one token, rows 16 or
// 32 bytes apart, which would all fall in one LDS bank; xoring the row's low four bits
// with s puts them in different banks. A bijection of 0..255; the writer to global
// memory reads row e at the same place.
__device__ inline int vrow(int e) { return e ^ ((e >> 4) & 15); }

// ---- four vectors per wave: lane l holds vector l >> 4, elements 16 (l & 15) + i

// Butterfly stage of element bit log2(M) + 4 (M = 1, 2, 4, 8: lanes s and s ^ M of a row).
template <int M>
__device__ inline double mv_xchg(double v, int lane) {
  if (M != 4) return xchg64<M>(v, lane);
  // lane ^ 4 by the crossbar's swizzle (bit mode: and 0x1F, xor 4)
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)b, 0x101F);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)(b >> 32), 0x101F);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <int M>
__device__ inline void mv_lane_stage(double (&y)[16], int lane) {
  const double sg = (lane & M) ? -1.0 : 1.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = __builtin_fma(sg, y[i], mv_xchg<M>(y[i], lane));
}
// Exact H x / 16 of the lane's 16 elements (SCALED = false: H x, 16 times larger).
template <bool SCALED = true>
__device__ inline void mv_wht(double (&y)[16], int lane) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!(i & h)) {
        const double a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
  mv_lane_stage<1>(y, lane);
  mv_lane_stage<2>(y, lane);
  mv_lane_stage<4>(y, lane);
  mv_lane_stage<8>(y, lane);
  if (SCALED) {
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] *= 0.0625;
  }
}
__device__ inline double mv_absmax(const double (&y)[16]) {
  double m = fabs(y[0]);
#pragma unroll
  for (int i = 1; i < 16; ++i) m = fmax(m, fabs(y[i]));
  return m;
}

// Codes from an fp32 quotient, each checked against the rounding threshold nearest to
// it: y/d is formed as (float)y * rcp(d) (d is an fp16 value, exact in fp32; the estimate
// is within 2^-19 of y/d for the |y/d| <= 8.01 of q4 and within 2^-15 for the
// |x/d| <= 127.1 of int8). The code's offset and the rounding half are added in the same
// fma together with half the window (2^-16 for q4, 2^-12 for int8), so that a quotient
// within the window of a threshold is one whose shifted value lies less than a whole
// window above an integer: that is its fraction, and the integer part is the code. The
// fma's own rounding (at most 2^-20 for q4, 2^-18 for int8) and the estimate's error
// stay inside the window. Where a lane of the wave has such a quotient, the whole wave
// takes the exact decisions of kv_encode.h.
// q4: y16 = 16 y (the rotation without its 1/16): the quotient uses rcp(d) / 16 (exact).
__device__ inline void mv_q4_codes(const double (&y16)[16], double d, int (&code)[16]) {
  const float rd = d == 0.0 ? 0.0f : __builtin_amdgcn_rcpf((float)d) * 0.0625f;  // (d = 0: every code 8)
  bool near = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float q = fmaf((float)y16[i], rd, 8.5f + 0x1p-16f);  // y/d + 1/2 + 8, shifted by half the window
    near |= __builtin_amdgcn_fractf(q) < 0x1p-15f;
    code[i] = (int)__builtin_amdgcn_fmed3f(__builtin_floorf(q), 0.0f, 15.0f);
  }
  if (__any(near)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) code[i] = enc::q4_code_fast(y16[i] * 0.0625, d);
  }
}
__device__ inline void mv_int8_codes(const double (&x)[16], double d, int (&code)[16]) {
  const float rd = d == 0.0 ? 0.0f : __builtin_amdgcn_rcpf((float)d);  // (d = 0: every code 0)
  bool near = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float q = fmaf((float)fabs(x[i]), rd, 0.5f + 0x1p-12f);  // |x|/d + 1/2, shifted
    near |= __builtin_amdgcn_fractf(q) < 0x1p-11f;
    const int c = (int)fminf(__builtin_floorf(q), 127.0f);
    code[i] = x[i] < 0.0 ? -c : c;
  }
  if (__any(near)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) code[i] = enc::int8_code_fast(x[i], d);
  }
}

// Codes of the lane's 16 elements and the scale of its block (q4, fp4: the 32 elements
// of lanes 2b, 2b + 1), group (int8: 64 elements, lanes 4g .. 4g + 3) or vector (fp8).
template <int KIND>
__device__ inline uint16_t mv_encode(const uint16_t* __restrict__ src, int lane, int (&code)[16]) {
  double x[16];
  {
    const u4* p = reinterpret_cast<const u4*>(src + 16 * (lane & 15));
    const u4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t wa = a[i >> 1], wb = b[i >> 1];
      x[i] = f16_to_f64((uint16_t)(wa >> (16 * (i & 1))));
      x[8 + i] = f16_to_f64((uint16_t)(wb >> (16 * (i & 1))));
    }
  }
  uint16_t scale;
  if (KIND == kInt8) {
    double a = mv_absmax(x);
    a = fmax(a, xchg64<1>(a, lane));
    a = fmax(a, xchg64<2>(a, lane));
    scale = enc::f64_to_f16_fast(a / 127.0);
    mv_int8_codes(x, f16_to_f64(scale), code);
  } else if (KIND == kFp8) {
    double a = mv_absmax(x);
    a = fmax(a, xchg64<1>(a, lane));
    a = fmax(a, xchg64<2>(a, lane));
    a = fmax(a, xchg64<4>(a, lane));
    a = fmax(a, xchg64<8>(a, lane));
    scale = enc::f64_to_f16_fast(a / 448.0);
    const double d = f16_to_f64(scale);
#pragma unroll
    for (int i = 0; i < 16; ++i) code[i] = fp8_code(x[i], d);
  } else {
    if (KIND == kFp4) {
      mv_wht(x, lane);
      double m = mv_absmax(x);
      m = fmax(m, xchg64<1>(m, lane));
      const int e = fp4_block_exp(m);
      scale = m == 0.0 ? (uint16_t)0 : fp16_pow2_bits(e);
#pragma unroll
      for (int i = 0; i < 16; ++i) code[i] = m == 0.0 ? 0 : fp4_code(x[i], e);
    } else {
      // x = 16 y (the rotation without its 1/16, which the scale and the quotient take);
      // the block's largest |y| from its largest and smallest values, then the signed value
      // of the first element holding it (the lower lane's elements come first)
      mv_wht<false>(x, lane);
      double mx = x[0], mn = x[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        mx = fmax(mx, x[i]);
        mn = fmin(mn, x[i]);
      }
      double m = fmax(mx, -mn);
      m = fmax(m, xchg64<1>(m, lane));
      // pair of lanes: which signs reach m
      const bool pos_l = mx == m, neg_l = -mn == m;
      const uint32_t flags = (pos_l ? 1u : 0u) | (neg_l ? 2u : 0u);
      const uint32_t pflags = xchg32<1>(flags, lane);
      const uint32_t both = flags | pflags;
      double best;
      if (__any(both == 3u)) {
        // both signs reach m somewhere in a block of the wave: the first element holding it
        double first = 0.0;
        uint32_t hit = 0u;
#pragma unroll
        for (int i = 15; i >= 0; --i) {
          const bool h = fabs(x[i]) == m;
          first = h ? x[i] : first;
          hit |= h ? 1u : 0u;
        }
        const double pf = xchg64<1>(first, lane);
        const uint32_t ph = xchg32<1>(hit, lane);
        best = (lane & 1) ? (ph ? pf : first) : (hit ? first : pf);
      } else {
        best = (both & 1u) ? m : -m;
      }
      scale = enc::f64_to_f16_fast(-best * (0.125 * 0.0625));  // -m/8 of y, exact
      mv_q4_codes(x, f16_to_f64(scale), code);
    }
  }
  return scale;
}

// The 16 codes of a lane as bytes: code 4 q + b in byte b of word q.
__device__ inline void mv_bytes(const int (&c)[16], uint32_t (&w)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = (uint32_t)c[4 * q] | ((uint32_t)c[4 * q + 1] << 8) | ((uint32_t)c[4 * q + 2] << 16) | ((uint32_t)c[4 * q + 3] << 24);
}

// Staging of one token's K record: code row (slice-permuted bytes) and scales.
template <int KIND>
__device__ inline void mv_stage_k(uint8_t* __restrict__ row, uint16_t* __restrict__ sc, int lane,
                                  const int (&code)[16], uint16_t scale) {
  const int s = lane & 15, j = s >> 1;  // elements 16 s .. 16 s + 15 lie in block j
  if (!four_bit(KIND)) {
    // byte 64 (r >> 3) + 8 j + (r & 7) = code of element 32 j + r: two runs of 8 bytes
    u2 w0 = {0u, 0u}, w1 = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w0[i >> 2] |= ((uint32_t)code[i] & 0xFFu) << (8 * (i & 3));
      w1[i >> 2] |= ((uint32_t)code[8 + i] & 0xFFu) << (8 * (i & 3));
    }
    const int r0 = 16 * (s & 1);
    *reinterpret_cast<u2*>(row + 64 * (r0 >> 3) + 8 * j) = w0;
    *reinterpret_cast<u2*>(row + 64 * ((r0 + 8) >> 3) + 8 * j) = w1;
    if (KIND == kInt8) {
      if ((s & 3) == 0) sc[s >> 2] = scale;
    } else if (s == 0) {
      sc[0] = scale;
    }
  } else {
    // byte 32 sl + 4 j + w = code[32 j + 4 sl + w] | code[32 j + 16 + 4 sl + w] << 4: the
    // even lane (elements r < 16 of the block) takes the odd lane's codes; word sl of the
    // byte-packed codes holds elements 4 sl .. 4 sl + 3 of each lane
    uint32_t w[4];
    mv_bytes(code, w);
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = xchg32<1>(w[q], lane);
    if (!(s & 1)) {
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) *reinterpret_cast<uint32_t*>(row + 32 * sl + 4 * j) = w[sl] | (h[sl] << 4);
      sc[j] = scale;
    }
  }
}

template <int KK, int VK>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t n_tokens,
    int64_t start, const int32_t* __restrict__ block_table, int64_t group0, uint8_t* pool,
    int64_t n_pool_pages, int64_t page_bytes, int n_kv_heads, int32_t* status) {
  constexpr int KR = code_row_bytes(KK), KS = n_scales(KK);   // K code bytes and scales per token
  constexpr int VB = four_bit(VK) ? kGroup / 2 : kGroup;      // V code bytes per element row and group
  constexpr int VS = n_scales(VK);                            // V scale rows
  __shared__ __attribute__((aligned(16))) uint8_t kt[kGroup * KR];
  __shared__ __attribute__((aligned(16))) uint16_t ks[kGroup * KS];
  __shared__ __attribute__((aligned(16))) uint8_t vt[kHeadDim * VB];
  __shared__ __attribute__((aligned(16))) uint16_t vs[VS * kGroup];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y;
  const int64_t t0 = kGroup * (group0 + blockIdx.x);  // first token of the group
  // the tokens of the group in the chunk: [lo, hi), as offsets from t0 (uniform)
  const int lo = (int)(start > t0 ? start - t0 : 0);
  const int hi = (int)(start + n_tokens < t0 + kGroup ? start + n_tokens - t0 : kGroup);
  if (lo >= hi) return;
  const int32_t phys = block_table[t0 / kPageTokens];
  if (phys < 0 || phys >= n_pool_pages) {
    if (status && tid == 0) atomicOr(status, KV_STATUS_BAD_PAGE_ID);
    return;
  }
  uint8_t* kplane = pool + (int64_t)phys * page_bytes + (int64_t)h * (plane_bytes(KK) + plane_bytes(VK));
  uint8_t* vplane = kplane + plane_bytes(KK);
  const int row0 = (int)(t0 % kPageTokens);  // the group's first row in the page
  const size_t stride = (size_t)n_kv_heads * kHeadDim;
  auto src = [&](const uint16_t* x, int i) { return x + (size_t)(t0 + i - start) * stride + (size_t)h * kHeadDim; };

  const int vi = lane >> 4, s = lane & 15;  // the lane's vector and its 16 elements
  // the wave's four tokens: K waves 4w .. 4w + 3; V waves (i, i + 1, i + 16, i + 17), i = 2 (w - 8)
  const int ti = wave < 8 ? 4 * wave + vi : 2 * (wave - 8) + (vi & 1) + 16 * (vi >> 1);
  const int tc = ti < lo ? lo : (ti >= hi ? hi - 1 : ti);  // (tokens outside the chunk read a valid row)
  int code[16];
  if (wave < 8) {
    const uint16_t scale = mv_encode<KK>(src(k, tc), lane, code);
    mv_stage_k<KK>(kt + ti * KR, ks + ti * KS, lane, code, scale);
  } else {
    const uint16_t scale = mv_encode<VK>(src(v, tc), lane, code);
    // scale rows (one per block, group or vector), one entry per token
    if (VK == kFp8) {
      if (s == 0) vs[ti] = scale;
    } else if (VK == kInt8) {
      if ((s & 3) == 0) vs[(s >> 2) * kGroup + ti] = scale;
    } else if (!(s & 1)) {
      vs[(s >> 1) * kGroup + ti] = scale;
    }
    // element rows: 8-bit codes at byte ti; the 4-bit codes of tokens ti (vectors 0, 1) and
    // ti + 16 (vectors 2, 3, lanes 32 further) share byte ti
    if (!four_bit(VK)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) vt[vrow(16 * s + i) * VB + ti] = (uint8_t)code[i];
    } else {
      uint32_t w[4], p[4];
      mv_bytes(code, w);
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = xchg32<32>(w[q], lane);
      if (vi < 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t b = w[q] | (p[q] << 4);
#pragma unroll
          for (int t = 0; t < 4; ++t) vt[vrow(16 * s + 4 * q + t) * VB + ti] = (uint8_t)(b >> (8 * t));
        }
      }
    }
  }
  __syncthreads();

  // K rows [lo, hi) and their scale rows: contiguous in the plane
  {
    const int n16 = (hi - lo) * KR / 16;
    uint8_t* dst = kplane + (size_t)(row0 + lo) * KR;
    const u4* s16 = reinterpret_cast<const u4*>(kt + lo * KR);
    for (int c = tid; c < n16; c += kAppendThreads) reinterpret_cast<u4*>(dst)[c] = s16[c];
    uint16_t* sdst = reinterpret_cast<uint16_t*>(kplane + kPageTokens * KR) + (row0 + lo) * KS;
    for (int c = tid; c < (hi - lo) * KS; c += kAppendThreads) sdst[c] = ks[lo * KS + c];
  }
  // V element rows: one segment of VB bytes per row (16-byte pieces); a partly covered
  // group keeps the codes of its other tokens
  {
    const bool whole = lo == 0 && hi == kGroup;
    constexpr int kPieces = VB / 16;
    for (int c = tid; c < kHeadDim * kPieces; c += kAppendThreads) {
      const int e = c / kPieces, p = c % kPieces;
      u4* dst = reinterpret_cast<u4*>(vplane + (size_t)e * code_row_bytes(VK) + (row0 % kPageTokens / kGroup) * VB + 16 * p);
      u4 val = *reinterpret_cast<const u4*>(vt + vrow(e) * VB + 16 * p);
      if (!whole) {
        const u4 old = *dst;
        u4 keep;  // bits of the stored segment that belong to tokens outside the chunk
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t m = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int byte = 16 * p + 4 * w + b;
            if (four_bit(VK)) {
              const bool in_lo = byte >= lo && byte < hi, in_hi = byte + 16 >= lo && byte + 16 < hi;
              m |= (in_lo ? 0u : 0x0Fu) << (8 * b);
              m |= (in_hi ? 0u : 0xF0u) << (8 * b);
            } else {
              m |= (byte >= lo && byte < hi ? 0u : 0xFFu) << (8 * b);
            }
          }
          keep[w] = m;
        }
        val = (val & ~keep) | (old & keep);
      }
      *dst = val;
    }
  }
  // V scale rows: the entries of tokens [lo, hi)
  {
    uint16_t* sc = reinterpret_cast<uint16_t*>(vplane + kHeadDim * code_row_bytes(VK));
    const int n = hi - lo;
    for (int c = tid; c < VS * n; c += kAppendThreads) {
      const int r = c / n, i = lo + c % n;
      sc[r * kPageTokens + row0 + i] = vs[r * kGroup + i];
    }
  }
}

template <int KK, int VK>
void launch_append_v(dim3 grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop, const uint16_t* k,
                     const uint16_t* v, int64_t n_tokens, int64_t start_pos, const int32_t* block_table,
                     int64_t g0, uint8_t* pool, int64_t n_pool_pages, int64_t page_bytes, int n_kv_heads,
                     int32_t* status) {
  hipExtLaunchKernelGGL((append_kernel<KK, VK>), grid, dim3(kAppendThreads), 0, stream, start, stop, 0, k, v,
                        n_tokens, start_pos, block_table, g0, pool, n_pool_pages, page_bytes, n_kv_heads, status);
}

}  // namespace

hipError_t launch_append(int fmt, int n_kv_heads, const uint16_t* k, const uint16_t* v,
                         int64_t n_tokens, int64_t start_pos, const int32_t* block_table,
                         int32_t /*n_table*/, uint8_t* pool, int64_t n_pool_pages,
                         int32_t* status, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (n_tokens <= 0) return hipSuccess;
  const int64_t g0 = start_pos / kGroup, g1 = (start_pos + n_tokens - 1) / kGroup;
  const int64_t page_bytes = (int64_t)n_kv_heads * head_stride(fmt);
  const dim3 grid((unsigned)(g1 - g0 + 1), (unsigned)n_kv_heads);
  switch (fmt) {
    case KV_FMT_INT8:
      launch_append_v<kInt8, kInt8>(grid, stream, start, stop, k, v, n_tokens, start_pos, block_table, g0, pool,
                                    n_pool_pages, page_bytes, n_kv_heads, status);
      break;
    case KV_FMT_Q4_0:
      launch_append_v<kQ4, kQ4>(grid, stream, start, stop, k, v, n_tokens, start_pos, block_table, g0, pool,
                                n_pool_pages, page_bytes, n_kv_heads, status);
      break;
    case KV_FMT_FP4:
      launch_append_v<kFp4, kFp4>(grid, stream, start, stop, k, v, n_tokens, start_pos, block_table, g0, pool,
                                  n_pool_pages, page_bytes, n_kv_heads, status);
      break;
    case KV_FMT_FP8:
      launch_append_v<kFp8, kFp8>(grid, stream, start, stop, k, v, n_tokens, start_pos, block_table, g0, pool,
                                  n_pool_pages, page_bytes, n_kv_heads, status);
      break;
    default:
      launch_append_v<kInt8, kQ4>(grid, stream, start, stop, k, v, n_tokens, start_pos, block_table, g0, pool,
                                  n_pool_pages, page_bytes, n_kv_heads, status);
      break;
  }
  return hipGetLastError();
}

}  // namespace kvc
