// kv_gather.hip - zero-copy page-in of missing pages from pinned host memory.
//
// Strata page ("KV 沉进内存、显存减半：Strata 让 12 GB 显卡跑满 262K 上下文"),
// section "KV 从显存搬进内存之后发生了什么": the authoritative KV copy stays in
// pinned host memory; before attention, pages missing from the device slots
// are copied over PCIe, zero-copy, into the slots the residency table chose.
//
// The kernel reads the host pages directly through the device mapping of the
// pinned allocation (no staging copy) and writes them to their slots; the
// (page, slot) list and the resulting block table travel in the kernel
// arguments, so the host needs no device-side buffer for them. Each workgroup
// moves one 64 KiB chunk of one page with 16-byte loads, eight in flight per
// thread, enough to keep many PCIe read requests outstanding.
#include <hip/hip_ext.h>

#include "kv_gather.h"

namespace kvc {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 65536;
constexpr int kThreads = 256;
constexpr int kUnroll = kChunk / (kThreads * 16);  // 16

__global__ __launch_bounds__(kThreads) void gather_kernel(GatherBatch batch, int64_t page_bytes,
                                                         const uint8_t* __restrict__ host_pool,
                                                         uint8_t* __restrict__ slot_pool,
                                                         int32_t* __restrict__ out_block_table) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = tid; i < batch.n_sel; i += kThreads) out_block_table[i] = batch.slots[i];
  }
  if ((int)blockIdx.y >= batch.n_miss) return;
  const u4* src = reinterpret_cast<const u4*>(host_pool + (int64_t)batch.miss_page[blockIdx.y] * page_bytes);
  u4* dst = reinterpret_cast<u4*>(slot_pool + (int64_t)batch.miss_slot[blockIdx.y] * page_bytes);
  const int64_t n16 = page_bytes / 16;
  const int64_t first = (int64_t)blockIdx.x * (kChunk / 16);
  u4 buf[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = first + (int64_t)u * kThreads + tid;
    if (i < n16) buf[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = first + (int64_t)u * kThreads + tid;
    if (i < n16) dst[i] = buf[u];
  }
}

// The same copy for a list of (source page, destination slot) pairs of any layers.
__global__ __launch_bounds__(kThreads) void gather_multi_kernel(MultiGatherBatch batch, int64_t page_bytes) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = tid; i < batch.n_entries; i += kThreads) batch.block_tables[i] = batch.slots[i];
  }
  if ((int)blockIdx.y >= batch.n_copies) return;
  const u4* src = reinterpret_cast<const u4*>(batch.src[blockIdx.y]);
  u4* dst = reinterpret_cast<u4*>(batch.dst[blockIdx.y]);
  const int64_t n16 = page_bytes / 16;
  const int64_t first = (int64_t)blockIdx.x * (kChunk / 16);
  u4 buf[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = first + (int64_t)u * kThreads + tid;
    if (i < n16) buf[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = first + (int64_t)u * kThreads + tid;
    if (i < n16) dst[i] = buf[u];
  }
}

}  // namespace

hipError_t launch_gather_multi_timed(const MultiGatherBatch& batch, int64_t page_bytes, hipStream_t stream,
                                     hipEvent_t start, hipEvent_t stop) {
  const unsigned chunks = (unsigned)((page_bytes + kChunk - 1) / kChunk);
  dim3 grid(chunks, (unsigned)(batch.n_copies > 0 ? batch.n_copies : 1)), block(kThreads);
  // events (or NULL) recorded at the kernel's own start and end
  hipExtLaunchKernelGGL(gather_multi_kernel, grid, block, 0, stream, start, stop, 0, batch, page_bytes);
  return hipGetLastError();
}

hipError_t launch_gather_multi(const MultiGatherBatch& batch, int64_t page_bytes, hipStream_t stream) {
  return launch_gather_multi_timed(batch, page_bytes, stream, nullptr, nullptr);
}

hipError_t launch_gather(const GatherBatch& batch, int64_t page_bytes, const uint8_t* host_pool,
                         uint8_t* slot_pool, int32_t* out_block_table, hipStream_t stream) {
  const unsigned chunks = (unsigned)((page_bytes + kChunk - 1) / kChunk);
  dim3 grid(chunks, (unsigned)(batch.n_miss > 0 ? batch.n_miss : 1)), block(kThreads);
  hipLaunchKernelGGL(gather_kernel, grid, block, 0, stream, batch, page_bytes, host_pool,
                     slot_pool, out_block_table);
  return hipGetLastError();
}

}  // namespace kvc
