// kv_append.hip - quantize-on-append into the paged pool (gfx950).
//
// Strata page ("KV 沉进内存、显存减半：Strata 让 12 GB 显卡跑满 262K 上下文"),
// section "4-bit KV 缓存：先旋转，再压到 4-bit": K and V are rotated by the
// 256-point Walsh-Hadamard matrix and stored as q4_0 blocks when written;
// section "三种 KV 格式横向对比": int8 (per-64 scales) and k8v4 (int8 K,
// rotated q4_0 V). The rounding rules are those of include/kvcache.h.
//
// One workgroup of four waves handles one token pair (32G+i, 32G+16+i) of one
// KV head: the two tokens whose 4-bit V codes share a byte of the element-major
// V plane. Waves 0 and 1 encode the K vectors of the two tokens, waves 2 and 3
// their V vectors; the V codes of the upper token pass through LDS and wave 2
// writes the shared bytes, so that every V byte has a single writer and a chunk
// of any length and alignment is appended without atomics.
//
// Lane l holds elements e = l + 64k (k = 0..3) of a vector. The rotation is
// done in fp64, where it is exact for fp16 inputs (partial sums are multiples
// of 2^-28 below 2^20): stages for bits 0..5 exchange between lanes, bits 6
// and 7 are inside the lane.
#include "kv_internal.h"

namespace kvc {
namespace {

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
__device__ inline void encode(const uint16_t* __restrict__ src, int lane, int (&code)[4],
                              uint16_t (&scale)[4]) {
  double x[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) x[k] = f16_to_f64(src[lane + 64 * k]);
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

template <int KK, int VK>
__global__ __launch_bounds__(256) void append_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t n_tokens,
    int64_t start, const int32_t* __restrict__ block_table, int64_t group0, uint8_t* pool,
    int64_t n_pool_pages, int64_t page_bytes, int n_kv_heads, int32_t* status) {
  __shared__ uint8_t vcode_hi[kHeadDim];  // V codes of the upper token (4-bit V)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int64_t grp = group0 + blockIdx.x / 16;
  const int i = blockIdx.x % 16;
  const int64_t t_lo = 32 * grp + i, t_hi = t_lo + 16;
  const bool in_lo = t_lo >= start && t_lo < start + n_tokens;
  const bool in_hi = t_hi >= start && t_hi < start + n_tokens;
  if (!in_lo && !in_hi) return;  // uniform over the workgroup
  const int64_t page = t_lo / kPageTokens;
  const int32_t phys = block_table[page];
  if (phys < 0 || phys >= n_pool_pages) {
    if (status && threadIdx.x == 0) atomicOr(status, KV_STATUS_BAD_PAGE_ID);
    return;
  }
  uint8_t* head = pool + (int64_t)phys * page_bytes + (int64_t)h * (plane_bytes(KK) + plane_bytes(VK));
  uint8_t* kplane = head;
  uint8_t* vplane = head + plane_bytes(KK);
  const int row_lo = (int)(t_lo % kPageTokens), row_hi = row_lo + 16;
  const size_t stride = (size_t)n_kv_heads * kHeadDim;

  const bool upper = wave & 1, is_v = wave >= 2;
  const bool in = upper ? in_hi : in_lo;
  const int64_t t = upper ? t_hi : t_lo;
  const int row = upper ? row_hi : row_lo;
  // 4-bit V bytes of lane elements (rows e, column of the pair)
  uint8_t* vbyte[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    vbyte[kk] = vplane + (size_t)(lane + 64 * kk) * code_row_bytes(VK) + 16 * (row_lo >> 5) + (row_lo & 15);
  // with one token of the pair outside the chunk, wave 2 keeps the other nibble
  uint8_t old[4] = {0, 0, 0, 0};
  if (VK == kQ4 && wave == 2 && !(in_lo && in_hi)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) old[kk] = *vbyte[kk];
  }

  int code[4] = {0, 0, 0, 0};
  uint16_t scale[4];
  if (in) {
    const size_t src = (size_t)(t - start) * stride + (size_t)h * kHeadDim;
    if (!is_v) {
      encode<KK>(k + src, lane, code, scale);
      write_k_row<KK>(kplane, row, lane, code, scale);
    } else {
      encode<VK>(v + src, lane, code, scale);
      write_v_scales<VK>(vplane, row, lane, scale);
      if (VK == kInt8) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) vplane[(size_t)(lane + 64 * kk) * code_row_bytes(VK) + row] = (uint8_t)(int8_t)code[kk];
      } else if (upper) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) vcode_hi[lane + 64 * kk] = (uint8_t)code[kk];
      }
    }
  }
  if (VK == kQ4) {
    __syncthreads();
    if (wave == 2) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int lo = in_lo ? code[kk] : (old[kk] & 0x0F);
        const int hi = in_hi ? vcode_hi[lane + 64 * kk] : (old[kk] >> 4);
        *vbyte[kk] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

}  // namespace

hipError_t launch_append(int fmt, int n_kv_heads, const uint16_t* k, const uint16_t* v,
                         int64_t n_tokens, int64_t start_pos, const int32_t* block_table,
                         int32_t /*n_table*/, uint8_t* pool, int64_t n_pool_pages,
                         int32_t* status, hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const int64_t g0 = start_pos / 32, g1 = (start_pos + n_tokens - 1) / 32;
  const int64_t pairs = (g1 - g0 + 1) * 16;
  const int64_t page_bytes = (int64_t)n_kv_heads * head_stride(fmt);
  dim3 grid((unsigned)pairs, (unsigned)n_kv_heads), block(256);
  switch (fmt) {
    case KV_FMT_INT8:
      hipLaunchKernelGGL((append_kernel<kInt8, kInt8>), grid, block, 0, stream, k, v, n_tokens,
                         start_pos, block_table, g0, pool, n_pool_pages, page_bytes, n_kv_heads,
                         status);
      break;
    case KV_FMT_Q4_0:
      hipLaunchKernelGGL((append_kernel<kQ4, kQ4>), grid, block, 0, stream, k, v, n_tokens,
                         start_pos, block_table, g0, pool, n_pool_pages, page_bytes, n_kv_heads,
                         status);
      break;
    default:
      hipLaunchKernelGGL((append_kernel<kInt8, kQ4>), grid, block, 0, stream, k, v, n_tokens,
                         start_pos, block_table, g0, pool, n_pool_pages, page_bytes, n_kv_heads,
                         status);
      break;
  }
  return hipGetLastError();
}

}  // namespace kvc
