// kv_select.hip - page selection for streaming mode (gfx950).
//
// KV-offload news page (rebasdaily.com topic page on Qwen3.8-Flash-Next KV
// offload), section "新招不是全搬，而是分层放": attention over a fixed budget of
// selected tokens, with most of the cache in system memory; the page's account of
// the selection rule breaks off. The rule implemented (declared, see
// include/kvcache.h) works on exact integers and one rounding:
//   S[p][g][e] = sum over page p's tokens of k * 2^24     (key sums, int64)
//   R[p][g][e] = S[p][g][e] / 2^32 rounded once to fp16   (page representatives)
//   Q[g][e]    = sum over KV head g's query heads of q * 2^24
//   score[p]   = sum over g, e of Q[g][e] * R[p][g][e] * 2^24   (128-bit integer)
// then the last page plus the k - 1 other pages of largest score (ties to the lower
// page index), in ascending order. Integer sums do not depend on their order, so
// the key sums can be accumulated with atomics and every selection is exact; the
// scores read the 2-byte representatives, a quarter of the sums' bytes.
#include "kv_lanes.h"

namespace kvc {
namespace {

constexpr int kThreads = 256;
constexpr double kTwo24 = 16777216.0;

typedef __int128 i128;

__device__ inline int64_t f16_to_int(uint16_t h) {  // exact: |h| * 2^24 < 2^40
  return (int64_t)(f16_to_f64(h) * kTwo24);
}

// Key sums of the tokens [start, start + n) that fall in logical page `first_page +
// blockIdx.x`, KV head blockIdx.y; thread e owns element e. The representative is
// rounded from the sum the thread's own atomic add produced (its old value plus the
// addend), so within one call it is that of the complete sum.
__global__ __launch_bounds__(kThreads) void key_sums_kernel(const uint16_t* __restrict__ k, int64_t n,
                                                           int64_t start, int64_t first_page,
                                                           int n_kv_heads, int64_t* __restrict__ sums,
                                                           uint16_t* __restrict__ reps) {
  const int e = threadIdx.x, g = blockIdx.y;
  const int64_t page = first_page + blockIdx.x;
  const int64_t t0 = max(start, page * kPageTokens), t1 = min(start + n, (page + 1) * kPageTokens);
  int64_t acc = 0;
  for (int64_t t = t0; t < t1; ++t) acc += f16_to_int(k[((t - start) * n_kv_heads + g) * kHeadDim + e]);
  const int64_t at = (page * n_kv_heads + g) * kHeadDim + e;
  const unsigned long long old =
      atomicAdd(reinterpret_cast<unsigned long long*>(&sums[at]), (unsigned long long)acc);
  const int64_t now = (int64_t)(old + (unsigned long long)acc);  // |now| < 2^48: exact in fp64
  reps[at] = f64_to_f16_rne((double)now * 0x1p-32);
}

// An fp16 value times 2^24 as an integer, from its bits: magnitude m * 2^(max(E, 1) - 1)
// with m the significand (implicit bit included for E > 0), as |Q| * m < 2^54 fits int64
// the product with a query sum is formed before the shift.
__device__ inline i128 times_rep(int64_t qs, uint16_t h) {
  const int E = (h >> 10) & 31;
  const int64_t m = (int64_t)((h & 0x3FF) | (E ? 0x400 : 0));
  const i128 v = (i128)(qs * m) << (E ? E - 1 : 0);
  return (h & 0x8000) ? -v : v;
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
                                                             const uint16_t* __restrict__ reps,
                                                             int64_t reps_pages, int n_pages,
                                                             int n_q_heads, int n_kv_heads,
                                                             i128* __restrict__ scores) {
  __shared__ int64_t qsum[kMaxKvHeads][kHeadDim];
  __shared__ i128 part[kTilePages][kParts];
  const int tid = threadIdx.x;
  q += (size_t)blockIdx.y * n_q_heads * kHeadDim;
  reps += (size_t)blockIdx.y * reps_pages * n_kv_heads * kHeadDim;
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
      // the thread's 16 representatives: two 16-byte loads
      const uint4* rp = reinterpret_cast<const uint4*>(reps + (page * n_kv_heads + g) * kHeadDim + i * kSlice);
      const uint4 w[2] = {rp[0], rp[1]};
#pragma unroll
      for (int u = 0; u < kSlice; ++u) {
        const uint32_t word = (&w[u >> 3].x)[(u >> 1) & 3];
        acc += times_rep(qsum[g][i * kSlice + u], (uint16_t)(u & 1 ? word >> 16 : word & 0xFFFFu));
      }
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

// The selection: the last page, then k - 1 rounds of "best page not yet taken". Thread t
// owns pages t, t + 256, ... (the last page excepted) and keeps the best and second best
// of its pages not yet taken (a bit per page in LDS marks those taken); a round takes the
// best over the threads (equal scores: the lower page). The owner of the page taken moves
// its second best up, and looks at its pages again only when it wins a second time
// (its second best is then unknown). The round's arg-max runs inside each wave by lane
// exchanges, then over the four waves' results in LDS (double-buffered by round parity,
// so one barrier a round).
constexpr int kMaxSelect = 256;
constexpr int kMaxPages = 32768;
constexpr int kOwnWords = kMaxPages / kThreads / 32;  // taken bits of a thread's pages

__device__ inline bool better(i128 s, int p, i128 bs, int bp) {  // (s, p) ahead of (bs, bp)?
  return p >= 0 && (bp < 0 || s > bs || (s == bs && p < bp));
}

// (score, page) of lane ^ M
template <int M>
__device__ inline void xchg_pair(i128& s, int& p, int lane) {
  const unsigned __int128 u = (unsigned __int128)s;
  const uint32_t w0 = xchg32<M>((uint32_t)u, lane), w1 = xchg32<M>((uint32_t)(u >> 32), lane);
  const uint32_t w2 = xchg32<M>((uint32_t)(u >> 64), lane), w3 = xchg32<M>((uint32_t)(u >> 96), lane);
  s = (i128)(((unsigned __int128)w3 << 96) | ((unsigned __int128)w2 << 64) | ((unsigned __int128)w1 << 32) | w0);
  p = (int)xchg32<M>((uint32_t)p, lane);
}
template <int M>
__device__ inline void argmax_step(i128& s, int& p, int lane) {
  i128 os = s;
  int op = p;
  xchg_pair<M>(os, op, lane);
  if (better(os, op, s, p)) {
    s = os;
    p = op;
  }
}

// The best and second best of thread tid's pages not taken (page -1: none); the scores
// of 16 pages are loaded together, so that their latencies overlap.
struct Best2 {
  i128 s, s2;
  int p, p2;
};
__device__ inline Best2 own_best(const i128* __restrict__ scores, int last, int tid,
                                 const uint32_t (*taken)[kThreads]) {
  Best2 b = {0, 0, -1, -1};
  for (int j0 = 0; tid + kThreads * j0 < last; j0 += 16) {
    i128 sc[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int p = tid + kThreads * (j0 + u);
      sc[u] = p < last ? scores[p] : (i128)0;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = j0 + u, p = tid + kThreads * j;
      const bool free = p < last && !((taken[j >> 5][tid] >> (j & 31)) & 1u);
      if (!free) continue;
      if (better(sc[u], p, b.s, b.p)) {  // pages visited in increasing order
        b.s2 = b.s;
        b.p2 = b.p;
        b.s = sc[u];
        b.p = p;
      } else if (better(sc[u], p, b.s2, b.p2)) {
        b.s2 = sc[u];
        b.p2 = p;
      }
    }
  }
  return b;
}

__global__ __launch_bounds__(kThreads) void top_pages_kernel(const i128* __restrict__ scores, int n_pages,
                                                            int k_sel, int32_t* __restrict__ out) {
  scores += (size_t)blockIdx.x * n_pages;  // selection set blockIdx.x
  out += (size_t)blockIdx.x * k_sel;
  __shared__ i128 wbest_s[2][kThreads / 64];
  __shared__ int wbest_p[2][kThreads / 64];
  __shared__ int chosen[kMaxSelect];
  __shared__ uint32_t taken[kOwnWords][kThreads];  // column t: thread t's pages
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n_pages <= k_sel) {
    for (int p = tid; p < n_pages; p += kThreads) out[p] = p;
    return;
  }
  const int last = n_pages - 1;
#pragma unroll
  for (int w = 0; w < kOwnWords; ++w) taken[w][tid] = 0u;
  Best2 b = own_best(scores, last, tid, taken);
  if (tid == 0) chosen[0] = last;
  for (int r = 1; r < k_sel; ++r) {
    // arg-max inside the wave
    i128 ws = b.s;
    int wp = b.p;
    argmax_step<1>(ws, wp, lane);
    argmax_step<2>(ws, wp, lane);
    argmax_step<4>(ws, wp, lane);
    argmax_step<8>(ws, wp, lane);
    argmax_step<16>(ws, wp, lane);
    argmax_step<32>(ws, wp, lane);
    const int buf = r & 1;
    if (lane == 0) {
      wbest_s[buf][wave] = ws;
      wbest_p[buf][wave] = wp;
    }
    __syncthreads();
    // over the waves (every thread, the same answer)
    i128 gs = wbest_s[buf][0];
    int gp = wbest_p[buf][0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
      if (better(wbest_s[buf][w], wbest_p[buf][w], gs, gp)) {
        gs = wbest_s[buf][w];
        gp = wbest_p[buf][w];
      }
    if (tid == 0) chosen[r] = gp;
    if (gp % kThreads == tid) {  // the owner: mark it taken, move its second best up
      const int j = gp / kThreads;
      taken[j >> 5][tid] |= 1u << (j & 31);
      if (b.p2 != -2) {
        b.s = b.s2;
        b.p = b.p2;
        b.p2 = -2;  // unknown
      } else {
        b = own_best(scores, last, tid, taken);
      }
    }
  }
  __syncthreads();
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
                           int64_t* sums, uint16_t* reps, hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const int64_t p0 = start_pos / kPageTokens, p1 = (start_pos + n_tokens - 1) / kPageTokens;
  dim3 grid((unsigned)(p1 - p0 + 1), (unsigned)n_kv_heads), block(kThreads);
  hipLaunchKernelGGL(key_sums_kernel, grid, block, 0, stream, k, n_tokens, start_pos, p0, n_kv_heads, sums, reps);
  return hipGetLastError();
}

hipError_t launch_select(int n_q_heads, int n_kv_heads, const uint16_t* q, const uint16_t* reps,
                         int64_t reps_pages, int n_pages, int k_sel, int n_sets, int32_t* out, void* scores,
                         hipStream_t stream) {
  if (n_pages <= 0 || n_sets <= 0) return hipSuccess;
  const unsigned tiles = (unsigned)((n_pages + kTilePages - 1) / kTilePages);
  hipLaunchKernelGGL(page_score_kernel, dim3(tiles, (unsigned)n_sets), dim3(kThreads), 0, stream, q, reps,
                     reps_pages, n_pages, n_q_heads, n_kv_heads, (i128*)scores);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(top_pages_kernel, dim3((unsigned)n_sets), dim3(kThreads), 0, stream, (const i128*)scores,
                     n_pages, k_sel, out);
  return hipGetLastError();
}

}  // namespace kvc
