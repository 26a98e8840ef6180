// kv_read.hip - measurement helper (not part of the decode library's ABI): a plain read
// of exactly the bytes a decode launch streams, as the roofline reference for the split
// kernel. It reads, for every work item (split, sequence, KV head) of the decode launch's
// split-major grid, the KV-head part of each of the item's pages through the same block
// table, with 16-byte loads, and folds the words into one checksum per thread so that no
// load can be dropped. No arithmetic beyond the xor, no LDS beyond one word, no other
// barriers: its duration is what the memory system needs for the launch's pages in the
// launch's order and grouping. Like the split kernel, it runs one workgroup per item when
// the items fit one round of resident workgroups, and otherwise one round that takes the
// remaining items from a counter.
// Built into lib/libkvmeasure.so; only the benchmark loads it.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
constexpr int kMaxHeadBytes = 147456;  // a page's KV-head part at most (int8 K and V: 135,168 B)

__device__ inline __amdgpu_buffer_rsrc_t head_rsrc(const uint8_t* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, bytes, 0x00020000);
}

// One workgroup of NT threads per work item; an item's pages are read one after the other,
// each page's PER loads per thread issued together (words past the head part read an empty
// range: zeros, no memory).
template <int NT, int PER>
__global__ __launch_bounds__(NT) void read_pages(const uint8_t* __restrict__ pool, int64_t n_pool_pages,
                                                       int64_t page_bytes, int head_bytes, int n_kv_heads,
                                                       const int32_t* __restrict__ block_tables, int max_pages,
                                                       const int32_t* __restrict__ context_lens, int batch,
                                                       int pages_per_split, int n_items, uint32_t* __restrict__ counter,
                                                       uint32_t* __restrict__ out) {
  __shared__ int next_s;
  const int n_pairs = batch * n_kv_heads;
  for (int item = blockIdx.x; item < n_items;) {
    const int split = item / n_pairs, b = (item - split * n_pairs) / n_kv_heads, g = item % n_kv_heads;
    const int T = max(context_lens[b], 0);
    const int n_pages = min((T + 255) / 256, max_pages);  // (the table's row holds max_pages entries)
    const int p_begin = split * pages_per_split, p_end = min(n_pages, p_begin + pages_per_split);
    u4 acc = {0u, 0u, 0u, 0u};
    for (int pg = p_begin; pg < p_end; ++pg) {
      const int32_t phys = block_tables[(size_t)b * max_pages + pg];
      if (phys < 0 || phys >= n_pool_pages) continue;
      const auto r = head_rsrc(pool + phys * page_bytes + (int64_t)g * head_bytes, head_bytes);
      u4 w[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j)
        w[j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, (j * NT + threadIdx.x) * 16, 0, 0));
#pragma unroll
      for (int j = 0; j < PER; ++j) acc ^= w[j];
    }
    out[(size_t)item * NT + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (!counter) break;  // one workgroup per item
    // the next item past the first round, from the counter (every thread reads it after the barrier)
    if (threadIdx.x == 0) next_s = (int)gridDim.x + (int)atomicAdd(&counter[0], 1u);
    __syncthreads();
    item = next_s;
    __syncthreads();
  }
  // the last workgroup to finish leaves the counters at zero for the next launch
  if (counter && threadIdx.x == 0) {
    __threadfence();
    if (atomicAdd(&counter[1], 1u) == gridDim.x - 1) {
      atomicExch(&counter[0], 0u);
      atomicExch(&counter[1], 0u);
    }
  }
}

}  // namespace

// Reads the pages of a decode launch (see above). head_bytes: one KV head's K and V planes
// of a page (at most 147,456 B and a multiple of 16); page_bytes = n_kv_heads * head_bytes;
// threads: the decode launch's workgroup size, 256 or 512;
// pages_per_split and n_splits: the decode launch's split size and count; n_resident: the
// decode launch's round of resident workgroups (more items than that are taken from
// `counter`, two device words that are zero before the first such launch and are left at
// zero by each; 0 or a null counter: one workgroup per item); out: device buffer of
// n_splits * batch * n_kv_heads * threads words. The launch records start and stop (may be
// null) at the kernel's own start and end on `stream`. Returns 0, or -1 for arguments
// outside these limits (nothing is launched then).
extern "C" int kv_measure_read_pages(const uint8_t* pool, int64_t n_pool_pages, int head_bytes, int n_kv_heads,
                                     const int32_t* block_tables, int max_pages, const int32_t* context_lens,
                                     int batch, int pages_per_split, int n_splits, int threads, int n_resident,
                                     uint32_t* counter, uint32_t* out, hipStream_t stream, hipEvent_t start,
                                     hipEvent_t stop) {
  if (!pool || !block_tables || !context_lens || !out || head_bytes <= 0 || head_bytes % 16 ||
      head_bytes > kMaxHeadBytes || n_kv_heads <= 0 || batch <= 0 || max_pages <= 0 || pages_per_split <= 0 ||
      n_splits <= 0 || n_pool_pages <= 0 || n_resident < 0 || (threads != 256 && threads != 512))
    return -1;
  const int64_t page_bytes = (int64_t)n_kv_heads * head_bytes;
  const int per = (head_bytes / 16 + threads - 1) / threads;
  const int n_items = n_splits * batch * n_kv_heads;
  const bool counted = counter && n_resident > 0 && n_items > n_resident;
  if (!counted) counter = nullptr;
  const dim3 grid((unsigned)(counted ? n_resident : n_items));
#define KV_READ_CASE(NT, P)                                                                                \
  hipExtLaunchKernelGGL((read_pages<NT, P>), grid, dim3(NT), 0, stream, start, stop, 0, pool, n_pool_pages,     \
                        page_bytes, head_bytes, n_kv_heads, block_tables, max_pages, context_lens, batch,    \
                        pages_per_split, n_items, counter, out)
  // the smallest compiled word count per thread that covers the head part
  if (threads == 256) {
    if (per <= 18) KV_READ_CASE(256, 18);
    else if (per <= 26) KV_READ_CASE(256, 26);
    else if (per <= 33) KV_READ_CASE(256, 33);
    else KV_READ_CASE(256, 36);
  } else {
    if (per <= 9) KV_READ_CASE(512, 9);
    else if (per <= 13) KV_READ_CASE(512, 13);
    else KV_READ_CASE(512, 18);
  }
#undef KV_READ_CASE
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
