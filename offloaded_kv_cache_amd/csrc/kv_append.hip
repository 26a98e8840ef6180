// kv_append.hip - quantize-on-append into the paged pool (gfx950).
//
// Strata page ("KV 沉进内存、显存减半：Strata 让 12 GB 显卡跑满 262K 上下文"),
// section "4-bit KV 缓存：先旋转，再压到 4-bit": K and V are rotated by the
// 256-point Walsh-Hadamard matrix and stored as q4_0 blocks when written;
// section "三种 KV 格式横向对比": int8 (per-64 scales) and k8v4 (int8 K,
// rotated q4_0 V). The rounding rules are those of include/kvcache.h.
//
// One workgroup of 16 waves handles a 32-token group (tokens 32G .. 32G+31, which
// lie in one page) of one KV head: waves 0-7 encode the group's K vectors, four
// tokens each; waves 8-15 its V vectors, the token pairs (i, i + 16) that share the
// bytes of a 4-bit V row, two pairs each (one vector per wave at a time,
// kv_encode.h). The records are assembled in LDS and then written whole: the
// group's K rows and scale rows are contiguous in the token-major K plane, and in
// the element-major V plane each of the 256 element rows receives one 16-byte
// (4-bit codes) or 32-byte (8-bit codes) segment, instead of one byte per token.
// Tokens of the group outside the chunk keep their bytes: the segments of a
// partly covered group are merged with the bytes already in the pool, code by code
// (a 4-bit V byte holds two tokens), and only the covered tokens' K rows and scales
// are written. Appends to one page from different calls must be ordered.
#include <hip/hip_ext.h>

#include "kv_encode.h"

namespace kvc {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kGroup = 32;                // tokens of a work item
constexpr int kAppendWaves = 16;
constexpr int kAppendThreads = 64 * kAppendWaves;

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

  if (wave < 8) {
    // K: tokens 4 wave .. 4 wave + 3 of the group, each record into its staging row
#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
      const int i = 4 * wave + u;
      if (i < lo || i >= hi) continue;  // uniform over the wave
      int code[4];
      uint16_t scale[4];
      enc::encode<KK, true>(src(k, i), lane, code, scale);
      enc::write_k_row_at<KK>(kt + i * KR, ks + i * KS, lane, code, scale);
    }
  } else {
    // V: token pairs (i, i + 16), i = 2 (wave - 8) and 2 (wave - 8) + 1
#pragma unroll 1
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * (wave - 8) + u;
      int lo_code[4] = {0, 0, 0, 0};
#pragma unroll 1
      for (int half = 0; half < 2; ++half) {
        const int ti = i + 16 * half;
        if (ti < lo || ti >= hi) continue;  // uniform over the wave
        int code[4];
        uint16_t scale[4];
        enc::encode<VK, true>(src(v, ti), lane, code, scale);
        // scale rows (one per group or block of elements, one entry per token)
        if (VK == kFp8) {
          if (lane == 0) vs[ti] = scale[0];
        } else if (VK == kInt8) {
          if (lane == 0) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) vs[kk * kGroup + ti] = scale[kk];
          }
        } else if ((lane & 31) == 0) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) vs[((lane >> 5) + 2 * kk) * kGroup + ti] = scale[kk];
        }
        // element rows: 8-bit codes at byte ti; 4-bit codes of the pair share byte i
        if (!four_bit(VK)) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) vt[(lane + 64 * kk) * VB + ti] = (uint8_t)code[kk];
        } else if (half == 0) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) lo_code[kk] = code[kk];
        } else {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) lo_code[kk] |= code[kk] << 4;
        }
      }
      if (four_bit(VK) && i + 16 >= lo && i < hi) {  // (a pair with at least one token in the chunk)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) vt[(lane + 64 * kk) * VB + i] = (uint8_t)lo_code[kk];
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
      u4 val = *reinterpret_cast<const u4*>(vt + e * VB + 16 * p);
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
