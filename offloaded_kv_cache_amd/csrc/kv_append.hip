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
// their V vectors (one vector per wave, kv_encode.h); the V codes of the upper
// token pass through LDS and wave 2 writes the shared bytes, so that every V
// byte has a single writer and a chunk of any length and alignment is appended
// without atomics.
#include "kv_encode.h"

namespace kvc {
namespace {

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
  if (four_bit(VK) && wave == 2 && !(in_lo && in_hi)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) old[kk] = *vbyte[kk];
  }

  int code[4] = {0, 0, 0, 0};
  uint16_t scale[4];
  if (in) {
    const size_t src = (size_t)(t - start) * stride + (size_t)h * kHeadDim;
    if (!is_v) {
      enc::encode<KK, false>(k + src, lane, code, scale);  // many vectors: LDS lane exchanges
      enc::write_k_row<KK>(kplane, row, lane, code, scale);
    } else {
      enc::encode<VK, false>(v + src, lane, code, scale);
      enc::write_v_scales<VK>(vplane, row, lane, scale);
      if (!four_bit(VK)) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) vplane[(size_t)(lane + 64 * kk) * code_row_bytes(VK) + row] = (uint8_t)code[kk];
      } else if (upper) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) vcode_hi[lane + 64 * kk] = (uint8_t)code[kk];
      }
    }
  }
  if (four_bit(VK)) {
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
    case KV_FMT_FP4:
      hipLaunchKernelGGL((append_kernel<kFp4, kFp4>), grid, block, 0, stream, k, v, n_tokens,
                         start_pos, block_table, g0, pool, n_pool_pages, page_bytes, n_kv_heads,
                         status);
      break;
    case KV_FMT_FP8:
      hipLaunchKernelGGL((append_kernel<kFp8, kFp8>), grid, block, 0, stream, k, v, n_tokens,
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
