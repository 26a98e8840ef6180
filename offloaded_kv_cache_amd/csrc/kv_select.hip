// kv_select.hip - page selection for streaming mode (gfx950).
//
// KV-offload news page (rebasdaily.com topic page on Qwen3.8-Flash-Next KV
// offload), section "新招不是全搬，而是分层放": attention over a fixed budget of
// selected tokens, with most of the cache in system memory; the page's account of
// the selection rule breaks off. The rule implemented (declared, see
// include/kvcache.h) works on exact integers:
//   S[p][g][e] = sum over page p's tokens of k * 2^24     (key sums, int64)
//   Q[g][e]    = sum over KV head g's query heads of q * 2^24
//   score[p]   = sum over g, e of Q[g][e] * S[p][g][e]    (128-bit integer)
// then the last page plus the k - 1 other pages of largest score (ties to the lower
// page index), in ascending order. Integer sums do not depend on their order, so
// the key sums can be accumulated with atomics and every selection is exact.
#include "kv_internal.h"

namespace kvc {
namespace {

constexpr int kThreads = 256;
constexpr double kTwo24 = 16777216.0;

typedef __int128 i128;

__device__ inline int64_t f16_to_int(uint16_t h) {  // exact: |h| * 2^24 < 2^40
  return (int64_t)(f16_to_f64(h) * kTwo24);
}

// Key sums of the tokens [start, start + n) that fall in logical page `first_page +
// blockIdx.x`, KV head blockIdx.y; thread e owns element e.
__global__ __launch_bounds__(kThreads) void key_sums_kernel(const uint16_t* __restrict__ k, int64_t n,
                                                           int64_t start, int64_t first_page,
                                                           int n_kv_heads, int64_t* __restrict__ sums) {
  const int e = threadIdx.x, g = blockIdx.y;
  const int64_t page = first_page + blockIdx.x;
  const int64_t t0 = max(start, page * kPageTokens), t1 = min(start + n, (page + 1) * kPageTokens);
  int64_t acc = 0;
  for (int64_t t = t0; t < t1; ++t) acc += f16_to_int(k[((t - start) * n_kv_heads + g) * kHeadDim + e]);
  atomicAdd(reinterpret_cast<unsigned long long*>(&sums[(page * n_kv_heads + g) * kHeadDim + e]),
            (unsigned long long)acc);
}

// Scores of a tile of kTilePages pages of selection set blockIdx.y (a layer or a
// sequence). The set's query sums Q[g][e] are formed once into LDS; thread (page j of the
// tile, part i) adds the products of its 16-element slice of every KV head, and one
// thread per page adds the page's kParts partial sums (128-bit integers).
constexpr int kTilePages = 16;
constexpr int kParts = kThreads / kTilePages;            // 16 threads per page
constexpr int kSlice = kHeadDim / kParts;                // 16 elements per thread and KV head
constexpr int kMaxKvHeads = 8;

__global__ __launch_bounds__(kThreads) void page_score_kernel(const uint16_t* __restrict__ q,
                                                             const int64_t* __restrict__ sums,
                                                             int64_t sums_pages, int n_pages,
                                                             int n_q_heads, int n_kv_heads,
                                                             i128* __restrict__ scores) {
  __shared__ int64_t qsum[kMaxKvHeads][kHeadDim];
  __shared__ i128 part[kTilePages][kParts];
  const int tid = threadIdx.x;
  q += (size_t)blockIdx.y * n_q_heads * kHeadDim;
  sums += (size_t)blockIdx.y * sums_pages * n_kv_heads * kHeadDim;
  scores += (size_t)blockIdx.y * n_pages;
  const int G = n_q_heads / n_kv_heads;
  for (int g = 0; g < n_kv_heads; ++g) {  // Q[g][e] for e = tid
    int64_t qs = 0;
    for (int i = 0; i < G; ++i) qs += f16_to_int(q[(g * G + i) * kHeadDim + tid]);
    qsum[g][tid] = qs;
  }
  __syncthreads();
  const int j = tid / kParts, i = tid % kParts;
  const int64_t page = (int64_t)blockIdx.x * kTilePages + j;
  i128 acc = 0;
  if (page < n_pages) {
    for (int g = 0; g < n_kv_heads; ++g) {
      const int64_t* sp = sums + (page * n_kv_heads + g) * kHeadDim + i * kSlice;
#pragma unroll
      for (int u = 0; u < kSlice; ++u) acc += (i128)qsum[g][i * kSlice + u] * (i128)sp[u];
    }
  }
  part[j][i] = acc;
  __syncthreads();
  if (i == 0 && page < n_pages) {
    i128 t = part[j][0];
    for (int u = 1; u < kParts; ++u) t += part[j][u];
    scores[page] = t;
  }
}

// The selection: the last page, then k - 1 rounds of "best page not yet taken".
constexpr int kMaxSelect = 256;
constexpr int kMaxPages = 32768;

__global__ __launch_bounds__(kThreads) void top_pages_kernel(const i128* __restrict__ scores, int n_pages,
                                                            int k_sel, int32_t* __restrict__ out) {
  __shared__ uint8_t taken[kMaxPages];
  scores += (size_t)blockIdx.x * n_pages;  // selection set blockIdx.x
  out += (size_t)blockIdx.x * k_sel;
  __shared__ i128 best_s[kThreads];
  __shared__ int best_p[kThreads];
  __shared__ int chosen[kMaxSelect];
  const int tid = threadIdx.x;
  if (n_pages <= k_sel) {
    for (int p = tid; p < n_pages; p += kThreads) out[p] = p;
    return;
  }
  for (int p = tid; p < n_pages; p += kThreads) taken[p] = 0;
  __syncthreads();
  if (tid == 0) {
    taken[n_pages - 1] = 1;
    chosen[0] = n_pages - 1;
  }
  __syncthreads();
  for (int r = 1; r < k_sel; ++r) {
    i128 bs = 0;
    int bp = -1;
    for (int p = tid; p < n_pages - 1; p += kThreads) {
      if (taken[p]) continue;
      const i128 s = scores[p];
      if (bp < 0 || s > bs) {  // pages visited in increasing order: equal scores keep the lower
        bs = s;
        bp = p;
      }
    }
    best_s[tid] = bs;
    best_p[tid] = bp;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
      if (tid < s) {
        const int po = best_p[tid + s];
        const i128 so = best_s[tid + s];
        const int pm = best_p[tid];
        if (po >= 0 && (pm < 0 || so > best_s[tid] || (so == best_s[tid] && po < pm))) {
          best_s[tid] = so;
          best_p[tid] = po;
        }
      }
      __syncthreads();
    }
    if (tid == 0) {
      taken[best_p[0]] = 1;
      chosen[r] = best_p[0];
    }
    __syncthreads();
  }
  if (tid == 0) {  // ascending order (k is small)
    for (int i = 1; i < k_sel; ++i) {
      const int v = chosen[i];
      int j = i - 1;
      while (j >= 0 && chosen[j] > v) {
        chosen[j + 1] = chosen[j];
        --j;
      }
      chosen[j + 1] = v;
    }
  }
  __syncthreads();
  for (int i = tid; i < k_sel; i += kThreads) out[i] = chosen[i];
}

}  // namespace

int select_max_pages() { return kMaxPages; }
int select_max_k() { return kMaxSelect; }
int select_max_kv_heads() { return kMaxKvHeads; }

hipError_t launch_key_sums(int n_kv_heads, const uint16_t* k, int64_t n_tokens, int64_t start_pos,
                           int64_t* sums, hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const int64_t p0 = start_pos / kPageTokens, p1 = (start_pos + n_tokens - 1) / kPageTokens;
  dim3 grid((unsigned)(p1 - p0 + 1), (unsigned)n_kv_heads), block(kThreads);
  hipLaunchKernelGGL(key_sums_kernel, grid, block, 0, stream, k, n_tokens, start_pos, p0, n_kv_heads, sums);
  return hipGetLastError();
}

hipError_t launch_select(int n_q_heads, int n_kv_heads, const uint16_t* q, const int64_t* sums,
                         int64_t sums_pages, int n_pages, int k_sel, int n_sets, int32_t* out, void* scores,
                         hipStream_t stream) {
  if (n_pages <= 0 || n_sets <= 0) return hipSuccess;
  const unsigned tiles = (unsigned)((n_pages + kTilePages - 1) / kTilePages);
  hipLaunchKernelGGL(page_score_kernel, dim3(tiles, (unsigned)n_sets), dim3(kThreads), 0, stream, q, sums,
                     sums_pages, n_pages, n_q_heads, n_kv_heads, (i128*)scores);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(top_pages_kernel, dim3((unsigned)n_sets), dim3(kThreads), 0, stream, (const i128*)scores,
                     n_pages, k_sel, out);
  return hipGetLastError();
}

}  // namespace kvc
