// kv_api.hip - the C ABI: argument checks, workspace layout, dispatch, and the
// host-side CLOCK residency table.
//
// CLOCK table: Strata page ("KV 沉进内存、显存减半：Strata 让 12 GB 显卡跑满
// 262K 上下文"), section "KV 从显存搬进内存之后发生了什么" - before attention
// the selected blocks are looked up in a residency table with CLOCK (second
// chance) eviction, and missing pages are paged in. The page names the policy;
// the step rules (hits pinned first, misses placed in selection order, ref set
// on insert) are the textbook algorithm and are documented in kvcache.h.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kv_gather.h"
#include "kv_internal.h"

using namespace kvc;

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return KV_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(KV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_shape(const kv_shape* s) {
  if (!s) return fail(KV_EINVAL, "shape is NULL");
  if (s->format != KV_FMT_INT8 && s->format != KV_FMT_Q4_0 && s->format != KV_FMT_K8V4 &&
      s->format != KV_FMT_FP4 && s->format != KV_FMT_FP8)
    return fail(KV_EINVAL, "unknown format %d", s->format);
  if (s->head_dim != kHeadDim) return fail(KV_EUNSUPPORTED, "head_dim must be 256 (got %d)", s->head_dim);
  if (s->page_tokens != kPageTokens)
    return fail(KV_EUNSUPPORTED, "page_tokens must be 256 (got %d)", s->page_tokens);
  if (s->n_kv_heads < 1 || s->n_kv_heads > 65535)
    return fail(KV_EINVAL, "n_kv_heads out of range (%d)", s->n_kv_heads);
  if (s->n_q_heads < s->n_kv_heads || s->n_q_heads % s->n_kv_heads)
    return fail(KV_EINVAL, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                s->n_q_heads, s->n_kv_heads);
  if (s->n_q_heads / s->n_kv_heads > kMaxGroup)
    return fail(KV_EUNSUPPORTED, "at most %d query heads per KV head (got %d)", kMaxGroup,
                s->n_q_heads / s->n_kv_heads);
  return KV_OK;
}

int64_t page_bytes_of(const kv_shape* s) { return (int64_t)s->n_kv_heads * head_stride(s->format); }

std::mutex g_cu_mu;
int g_cus[64];  // per device, 0 until read

// Pages per split chosen so that the grid fills the 256 compute units once: two
// 4-wave workgroups per CU, or one 8-wave workgroup (int8 K), over all the
// (sequence, KV head, split) items of `total_pages` pages. Each sequence's last
// split may be partial, so the other batch - 1 sequences keep one workgroup per KV
// head in reserve (a second, nearly empty round of workgroups would double the time).
int32_t pages_per_split_for(const kv_shape* s, int32_t batch, int64_t total_pages) {
  const int64_t target = (int64_t)device_compute_units() * (8 / split_waves(k_kind(s->format)));
  int64_t room = target - (int64_t)(batch - 1) * s->n_kv_heads;
  if (room < s->n_kv_heads) room = s->n_kv_heads;
  int64_t pps = (total_pages * s->n_kv_heads + room - 1) / room;
  if (pps < 1) pps = 1;
  if (pps > 0x7FFFFFFF) pps = 0x7FFFFFFF;
  return (int32_t)pps;
}
int32_t auto_pages_per_split(const kv_shape* s, int32_t batch, int64_t max_pages_ctx) {
  return pages_per_split_for(s, batch, (int64_t)batch * max_pages_ctx);
}

struct WsLayout {
  size_t ml_off, o_off, total;
  int32_t n_splits;
};

WsLayout workspace_layout(const kv_shape* s, int32_t batch, int64_t max_context, int32_t pps) {
  const int64_t max_pages_ctx = (max_context + kPageTokens - 1) / kPageTokens;
  int64_t ns = (max_pages_ctx + pps - 1) / pps;
  if (ns < 1) ns = 1;
  WsLayout w;
  w.n_splits = (int32_t)ns;
  const size_t parts = (size_t)batch * s->n_q_heads * (size_t)ns;
  w.ml_off = 256;
  w.o_off = (w.ml_off + parts * 2 * sizeof(float) + 255) & ~(size_t)255;
  w.total = w.o_off + parts * kHeadDim * sizeof(float);
  return w;
}


// Checks a table and a selection without changing anything.
int validate_selection(const kv_residency* t, const int32_t* selection, int32_t n_sel,
                       const int32_t* out_slots) {
  if (!t || t->n_slots < 1 || t->n_pages < 0 || !t->slot_page || !t->ref ||
      (t->n_pages > 0 && !t->page_slot))
    return fail(KV_EINVAL, "bad residency table");
  if (t->hand < 0 || t->hand >= t->n_slots) return fail(KV_EINVAL, "hand out of range");
  if (n_sel < 0) return fail(KV_EINVAL, "negative selection size");
  if (n_sel > t->n_slots)
    return fail(KV_ENOSLOTS, "selection of %d pages exceeds %d slots", n_sel, t->n_slots);
  if (n_sel > 0 && (!selection || !out_slots)) return fail(KV_EINVAL, "NULL selection or out_slots");
  std::vector<uint8_t> seen(t->n_pages, 0);
  for (int32_t i = 0; i < n_sel; ++i) {
    const int32_t p = selection[i];
    if (p < 0 || p >= t->n_pages) return fail(KV_EINVAL, "page %d out of range [0, %d)", p, t->n_pages);
    if (seen[p]) return fail(KV_EINVAL, "page %d selected twice", p);
    seen[p] = 1;
  }
  return KV_OK;
}

}  // namespace

int kvc::device_compute_units() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return kDefaultComputeUnits;
  }
  std::lock_guard<std::mutex> lock(g_cu_mu);
  if (!g_cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      return kDefaultComputeUnits;
    }
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

extern "C" {

const char* kv_last_error(void) { return g_error.c_str(); }

const char* kv_version(void) { return "0.1.0"; }

int64_t kv_page_bytes(const kv_shape* shape) {
  if (int r = check_shape(shape)) return r;
  ok();
  return page_bytes_of(shape);
}

int kv_append_quantize(const kv_shape* shape, const void* k, const void* v, int64_t n_tokens,
                       int64_t start_pos, const int32_t* block_table, int32_t n_table, void* pool,
                       int64_t n_pool_pages, int32_t* status, void* stream) {
  return kv_append_quantize_timed(shape, k, v, n_tokens, start_pos, block_table, n_table, pool, n_pool_pages,
                                  status, stream, nullptr, nullptr);
}

int kv_append_quantize_timed(const kv_shape* shape, const void* k, const void* v, int64_t n_tokens,
                             int64_t start_pos, const int32_t* block_table, int32_t n_table, void* pool,
                             int64_t n_pool_pages, int32_t* status, void* stream, void* start_event,
                             void* stop_event) {
  if (int r = check_shape(shape)) return r;
  if (n_tokens < 0 || start_pos < 0) return fail(KV_EINVAL, "negative n_tokens or start_pos");
  if (n_tokens == 0) return ok();
  if (!k || !v || !block_table || !pool) return fail(KV_EINVAL, "NULL buffer");
  if (n_tokens > INT64_MAX - start_pos)  // (so that start_pos + n_tokens below cannot overflow)
    return fail(KV_EINVAL, "start_pos + n_tokens overflows");
  if (n_table < 1 || start_pos + n_tokens > (int64_t)n_table * kPageTokens)
    return fail(KV_EINVAL, "tokens [%lld, %lld) do not fit %d pages of 256", (long long)start_pos,
                (long long)(start_pos + n_tokens), n_table);
  if (n_pool_pages < 1) return fail(KV_EINVAL, "n_pool_pages must be >= 1");
  if (!aligned(k, 2) || !aligned(v, 2) || !aligned(block_table, 4) || !aligned(pool, 16) ||
      (status && !aligned(status, 4)))
    return fail(KV_EALIGN, "misaligned buffer (k, v: 2 B; block_table: 4 B; pool: 16 B)");
  if ((start_pos + n_tokens - 1) / 32 - start_pos / 32 + 1 > (int64_t)(0x7FFFFFFF / 16))
    return fail(KV_EINVAL, "too many tokens in one call");
  hipError_t e = launch_append(shape->format, shape->n_kv_heads, (const uint16_t*)k,
                               (const uint16_t*)v, n_tokens, start_pos, block_table, n_table,
                               (uint8_t*)pool, n_pool_pages, status, (hipStream_t)stream,
                               (hipEvent_t)start_event, (hipEvent_t)stop_event);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

size_t kv_decode_workspace_bytes(const kv_shape* shape, int32_t batch, int64_t max_context,
                                 int32_t pages_per_split) {
  if (check_shape(shape)) return 0;
  if (batch < 1 || max_context < 0 || max_context > 0x7FFFFFFF || pages_per_split < 0) {
    fail(KV_EINVAL, "bad batch, max_context or pages_per_split");
    return 0;
  }
  const int64_t max_pages_ctx = (max_context + kPageTokens - 1) / kPageTokens;
  const int32_t pps = pages_per_split ? pages_per_split : auto_pages_per_split(shape, batch, max_pages_ctx);
  ok();
  return workspace_layout(shape, batch, max_context, pps).total;
}

size_t kv_decode_mq_workspace_bytes(const kv_shape* shape, int32_t batch, int32_t n_q, int64_t max_context,
                                    int32_t pages_per_split) {
  if (check_shape(shape)) return 0;
  if (batch < 1 || n_q < 1 || (int64_t)batch * n_q > 65535 || max_context < 0 || max_context > 0x7FFFFFFF ||
      pages_per_split < 0) {
    fail(KV_EINVAL, "bad batch, n_q, max_context or pages_per_split");
    return 0;
  }
  const int64_t max_pages_ctx = (max_context + kPageTokens - 1) / kPageTokens;
  const int32_t pps = pages_per_split ? pages_per_split : auto_pages_per_split(shape, batch * n_q, max_pages_ctx);
  ok();
  return workspace_layout(shape, batch * n_q, max_context, pps).total;
}

int32_t kv_decode_split_pages(const kv_shape* shape, int32_t batch, int64_t max_context,
                              int64_t total_context) {
  if (check_shape(shape)) return 0;
  if (batch < 1 || batch > 65535 || max_context < 0 || max_context > 0x7FFFFFFF || total_context < 0 ||
      total_context > (int64_t)batch * max_context) {
    fail(KV_EINVAL, "bad batch, max_context or total_context");
    return 0;
  }
  const int64_t total = total_context > 0 ? total_context : (int64_t)batch * max_context;
  ok();
  // pages of the batch: the total rounded up per sequence is at most batch - 1 pages more
  const int64_t pages = (total + kPageTokens - 1) / kPageTokens + (total_context > 0 ? batch - 1 : 0);
  return pages_per_split_for(shape, batch, pages);
}

}  // extern "C"

namespace {

// Device memory of kv_decode_attention_noalloc: split partials, work counters and a status
// word, in place of a caller workspace (laid out as one). Every GPU the library runs on
// holds its own copy until the process ends; calls on one GPU share it.
static __device__ __align__(256) uint8_t scratch[KV_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxDevices];  // the device address of each device's copy, once looked up

// The current device's copy of `scratch` (the device of the caller's stream). Its address
// is looked up once per device, with that device current; host code uses only that
// address, never the array's name (a host-side stand-in). The first lookup also enqueues
// the clearing of the header (status word, work counters) on `stream`; every later call
// leaves the counters at zero, as the decode kernels do with a workspace.
int scratch_of_device(hipStream_t stream, uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(KV_EUNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
    e = launch_zero_words(static_cast<uint32_t*>(p), 64, stream);  // the 256-byte header
    if (e != hipSuccess) return hip_fail(e, "scratch header clear");
    g_scratch[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch[dev];
  return KV_OK;
}

int decode_phase(int phase, const kv_shape* shape, const void* q, int32_t batch, const void* pool,
                 int64_t n_pool_pages, const int32_t* block_tables, int32_t max_pages,
                 const int32_t* context_lens, int64_t max_context, float softmax_scale, float* out,
                 void* workspace, size_t workspace_bytes, int32_t pages_per_split, void* stream,
                 void* start_event = nullptr, void* stop_event = nullptr,
                 const void* k_new = nullptr, const void* v_new = nullptr, int32_t n_q = 1,
                 bool noalloc = false, int32_t* status = nullptr) {
  if (int r = check_shape(shape)) return r;
  if (n_q < 1) return fail(KV_EINVAL, "n_q must be >= 1 (got %d)", n_q);
  if (batch < 0 || (int64_t)batch * n_q > 65535)
    return fail(KV_EINVAL, "batch x n_q out of range (%d x %d)", batch, n_q);
  if (batch == 0) return ok();
  const int32_t rows = batch * n_q;  // query rows: the kernels treat each as a sequence
  if (!q || !pool || !block_tables || !context_lens || !out || (!workspace && !noalloc))
    return fail(KV_EINVAL, "NULL buffer");
  if (max_pages < 1) return fail(KV_EINVAL, "max_pages must be >= 1");
  if (max_context < 0 || max_context > 0x7FFFFFFF) return fail(KV_EINVAL, "max_context out of range");
  if (n_pool_pages < 1) return fail(KV_EINVAL, "n_pool_pages must be >= 1");
  if (pages_per_split < 0) return fail(KV_EINVAL, "pages_per_split must be >= 0");
  if (!(softmax_scale == softmax_scale)) return fail(KV_EINVAL, "softmax_scale is NaN");
  if (!aligned(q, 16) || !aligned(pool, 16) || !aligned(out, 16) || !aligned(workspace, 256) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(status, 4))
    return fail(KV_EALIGN, "misaligned buffer (q, pool, out: 16 B; workspace: 256 B; status: 4 B)");
  const int64_t bound = max_context < (int64_t)max_pages * kPageTokens ? max_context
                                                                       : (int64_t)max_pages * kPageTokens;
  const int64_t max_pages_ctx = (max_context + kPageTokens - 1) / kPageTokens;
  const int32_t pps = pages_per_split ? pages_per_split : auto_pages_per_split(shape, rows, max_pages_ctx);
  const WsLayout w = workspace_layout(shape, rows, max_context, pps);
  if (noalloc) {
    if (w.total > KV_NOALLOC_SCRATCH_BYTES)
      return fail(KV_ESMALL, "the call needs %zu bytes of split partials, beyond the library's %d-byte scratch array",
                  w.total, KV_NOALLOC_SCRATCH_BYTES);
    uint8_t* sp = nullptr;
    if (int r = scratch_of_device((hipStream_t)stream, &sp)) return r;
    workspace = sp;
  } else if (workspace_bytes < w.total) {
    return fail(KV_ESMALL, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                w.total);
  }
  uint8_t* ws = (uint8_t*)workspace;
  DecodeArgs a;
  a.fmt = shape->format;
  a.n_q_heads = shape->n_q_heads;
  a.n_kv_heads = shape->n_kv_heads;
  a.batch = rows;
  a.n_q = n_q;
  a.q = (const uint16_t*)q;
  a.pool = (const uint8_t*)pool;
  a.n_pool_pages = n_pool_pages;
  a.block_tables = block_tables;
  a.max_pages = max_pages;
  a.context_lens = context_lens;
  a.max_context = (int32_t)bound;
  a.pages_per_split = pps;
  a.n_splits = w.n_splits;
  a.n_cus = device_compute_units();
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.out = out;
  a.status = status ? status : (int32_t*)ws;
  a.sched = (uint32_t*)(ws + 4);
  a.part_ml = (float*)(ws + w.ml_off);
  a.part_o = (float*)(ws + w.o_off);
  if (k_new) {
    a.k_new = (const uint16_t*)k_new;
    a.v_new = (const uint16_t*)v_new;
    a.pool_w = (uint8_t*)const_cast<void*>(pool);
  }
  hipError_t e = launch_decode(a, phase, (hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

}  // namespace

extern "C" {

int kv_decode_attention(const kv_shape* shape, const void* q, int32_t batch, const void* pool,
                        int64_t n_pool_pages, const int32_t* block_tables, int32_t max_pages,
                        const int32_t* context_lens, int64_t max_context, float softmax_scale,
                        float* out, void* workspace, size_t workspace_bytes,
                        int32_t pages_per_split, void* stream) {
  return decode_phase(3, shape, q, batch, pool, n_pool_pages, block_tables, max_pages, context_lens,
                      max_context, softmax_scale, out, workspace, workspace_bytes, pages_per_split,
                      stream);
}

int kv_decode_attention_noalloc(const kv_shape* shape, const void* q, int32_t batch, const void* pool,
                                int64_t n_pool_pages, const int32_t* block_tables, int32_t max_pages,
                                const int32_t* context_lens, int64_t max_context, float softmax_scale,
                                float* out, int32_t* status, int32_t pages_per_split, void* stream) {
  return decode_phase(3, shape, q, batch, pool, n_pool_pages, block_tables, max_pages, context_lens,
                      max_context, softmax_scale, out, nullptr, 0, pages_per_split, stream, nullptr,
                      nullptr, nullptr, nullptr, 1, true, status);
}

int kv_decode_attention_mq(const kv_shape* shape, const void* q, int32_t batch, int32_t n_q,
                           const void* pool, int64_t n_pool_pages, const int32_t* block_tables,
                           int32_t max_pages, const int32_t* context_lens, int64_t max_context,
                           float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                           int32_t pages_per_split, void* stream) {
  return decode_phase(3, shape, q, batch, pool, n_pool_pages, block_tables, max_pages, context_lens,
                      max_context, softmax_scale, out, workspace, workspace_bytes, pages_per_split,
                      stream, nullptr, nullptr, nullptr, nullptr, n_q);
}

int kv_decode_split(const kv_shape* shape, const void* q, int32_t batch, const void* pool,
                    int64_t n_pool_pages, const int32_t* block_tables, int32_t max_pages,
                    const int32_t* context_lens, int64_t max_context, float softmax_scale,
                    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split,
                    void* stream) {
  return decode_phase(1, shape, q, batch, pool, n_pool_pages, block_tables, max_pages, context_lens,
                      max_context, softmax_scale, out, workspace, workspace_bytes, pages_per_split,
                      stream);
}

int kv_decode_split_timed(const kv_shape* shape, const void* q, int32_t batch, const void* pool,
                          int64_t n_pool_pages, const int32_t* block_tables, int32_t max_pages,
                          const int32_t* context_lens, int64_t max_context, float softmax_scale,
                          float* out, void* workspace, size_t workspace_bytes,
                          int32_t pages_per_split, void* stream, void* start_event,
                          void* stop_event) {
  return decode_phase(1, shape, q, batch, pool, n_pool_pages, block_tables, max_pages, context_lens,
                      max_context, softmax_scale, out, workspace, workspace_bytes, pages_per_split,
                      stream, start_event, stop_event);
}

int kv_append_decode(const kv_shape* shape, const void* k_new, const void* v_new, const void* q,
                     int32_t batch, void* pool, int64_t n_pool_pages, const int32_t* block_tables,
                     int32_t max_pages, const int32_t* context_lens, int64_t max_context,
                     float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                     int32_t pages_per_split, void* stream, void* start_event, void* stop_event) {
  if (batch > 0 && (!k_new || !v_new)) return fail(KV_EINVAL, "NULL buffer");
  if (batch > 0 && (!aligned(k_new, 2) || !aligned(v_new, 2)))
    return fail(KV_EALIGN, "misaligned buffer (k_new, v_new: 2 B)");
  int r = decode_phase(1, shape, q, batch, pool, n_pool_pages, block_tables, max_pages, context_lens,
                       max_context, softmax_scale, out, workspace, workspace_bytes, pages_per_split,
                       stream, start_event, stop_event, k_new, v_new);
  if (r != KV_OK) return r;
  return decode_phase(2, shape, q, batch, pool, n_pool_pages, block_tables, max_pages, context_lens,
                      max_context, softmax_scale, out, workspace, workspace_bytes, pages_per_split,
                      stream);
}

int kv_decode_combine(const kv_shape* shape, const void* q, int32_t batch, const void* pool,
                      int64_t n_pool_pages, const int32_t* block_tables, int32_t max_pages,
                      const int32_t* context_lens, int64_t max_context, float softmax_scale,
                      float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split,
                      void* stream) {
  return decode_phase(2, shape, q, batch, pool, n_pool_pages, block_tables, max_pages, context_lens,
                      max_context, softmax_scale, out, workspace, workspace_bytes, pages_per_split,
                      stream);
}

int kv_residency_reset(kv_residency* t) {
  if (!t || t->n_slots < 1 || t->n_pages < 0 || !t->slot_page || !t->ref ||
      (t->n_pages > 0 && !t->page_slot))
    return fail(KV_EINVAL, "bad residency table");
  for (int32_t s = 0; s < t->n_slots; ++s) {
    t->slot_page[s] = -1;
    t->ref[s] = 0;
  }
  for (int32_t p = 0; p < t->n_pages; ++p) t->page_slot[p] = -1;
  t->hand = 0;
  return ok();
}

int kv_residency_select(kv_residency* t, const int32_t* selection, int32_t n_sel, int32_t* out_slots,
                        int32_t* miss_pages, int32_t* miss_slots, int32_t* n_miss) {
  if (int r = validate_selection(t, selection, n_sel, out_slots)) return r;
  std::vector<uint8_t> pinned(t->n_slots, 0);
  for (int32_t i = 0; i < n_sel; ++i) {
    const int32_t s = t->page_slot[selection[i]];
    if (s >= 0) {
      t->ref[s] = 1;
      pinned[s] = 1;
    }
  }
  int32_t misses = 0;
  for (int32_t i = 0; i < n_sel; ++i) {
    const int32_t p = selection[i];
    if (t->page_slot[p] >= 0) continue;
    int32_t s;
    for (;;) {  // ends: at most n_sel - 1 slots are pinned, and a sweep clears every ref bit
      s = t->hand;
      t->hand = (t->hand + 1) % t->n_slots;
      if (t->slot_page[s] < 0) break;
      if (pinned[s]) continue;
      if (t->ref[s]) {
        t->ref[s] = 0;
        continue;
      }
      t->page_slot[t->slot_page[s]] = -1;
      break;
    }
    t->slot_page[s] = p;
    t->page_slot[p] = s;
    t->ref[s] = 1;
    pinned[s] = 1;
    if (miss_pages) miss_pages[misses] = p;
    if (miss_slots) miss_slots[misses] = s;
    ++misses;
  }
  for (int32_t i = 0; i < n_sel; ++i) out_slots[i] = t->page_slot[selection[i]];
  if (n_miss) *n_miss = misses;
  return ok();
}

int kv_gather_pages(const kv_shape* shape, kv_residency* t, const int32_t* selection, int32_t n_sel,
                    const void* host_pool, void* slot_pool, int32_t* out_block_table,
                    int32_t* out_n_miss, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (n_sel > 0 && (!host_pool || !slot_pool || !out_block_table))
    return fail(KV_EINVAL, "NULL buffer");
  if (!aligned(host_pool, 16) || !aligned(slot_pool, 16) || !aligned(out_block_table, 4))
    return fail(KV_EALIGN, "misaligned buffer (pools: 16 B, block table: 4 B)");
  {
    int32_t dummy = 0;
    if (int r = validate_selection(t, selection, n_sel, n_sel > 0 ? &dummy : nullptr)) return r;
  }
  if (n_sel > 0) {
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    hipError_t pe = hipPointerGetAttributes(&attr, host_pool);
    if (pe != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return fail(KV_EINVAL, "host_pool is not pinned, device-accessible host memory");
    }
  }
  std::vector<int32_t> slots(n_sel > 0 ? n_sel : 1), mp(n_sel > 0 ? n_sel : 1), ms(n_sel > 0 ? n_sel : 1);
  int32_t misses = 0;
  if (int r = kv_residency_select(t, selection, n_sel, slots.data(), mp.data(), ms.data(), &misses))
    return r;
  const int64_t pb = page_bytes_of(shape);
  // Launch in batches that fit the kernel-argument block; each batch writes
  // its slice of the block table and copies its share of the misses.
  int32_t done_sel = 0, done_miss = 0;
  while (done_sel < n_sel || done_miss < misses) {
    GatherBatch gb;
    gb.n_sel = n_sel - done_sel < kGatherMaxBatch ? n_sel - done_sel : kGatherMaxBatch;
    gb.n_miss = misses - done_miss < kGatherMaxBatch ? misses - done_miss : kGatherMaxBatch;
    for (int32_t i = 0; i < gb.n_sel; ++i) gb.slots[i] = slots[done_sel + i];
    for (int32_t i = 0; i < gb.n_miss; ++i) {
      gb.miss_page[i] = mp[done_miss + i];
      gb.miss_slot[i] = ms[done_miss + i];
    }
    hipError_t e = launch_gather(gb, pb, (const uint8_t*)host_pool, (uint8_t*)slot_pool,
                                 out_block_table + done_sel, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gather launch (the residency table was already updated)");
    done_sel += gb.n_sel;
    done_miss += gb.n_miss;
  }
  if (out_n_miss) *out_n_miss = misses;
  return ok();
}

}  // extern "C"

namespace {

// kv_gather_pages_layers with optional events: `start` is recorded at the start of the
// first copy kernel, `stop` at the end of the last one (none when there is nothing to do).
int gather_layers(const kv_shape* shape, int32_t n_layers, kv_residency* tables, const int32_t* selections,
                  int32_t n_sel, const void* const* host_pools, void* const* slot_pools,
                  int32_t* out_block_tables, int32_t* out_n_miss, void* stream, void* start_event,
                  void* stop_event) {
  if (int r = check_shape(shape)) return r;
  if (n_layers < 0 || n_sel < 0) return fail(KV_EINVAL, "negative size");
  if (n_layers == 0 || n_sel == 0) return ok();
  if (!tables || !selections || !host_pools || !slot_pools || !out_block_tables)
    return fail(KV_EINVAL, "NULL buffer");
  if (!aligned(out_block_tables, 4)) return fail(KV_EALIGN, "misaligned block tables (4 B)");
  // every argument is checked before any table changes
  for (int32_t l = 0; l < n_layers; ++l) {
    if (!host_pools[l] || !slot_pools[l]) return fail(KV_EINVAL, "NULL pool of layer %d", l);
    if (!aligned(host_pools[l], 16) || !aligned(slot_pools[l], 16))
      return fail(KV_EALIGN, "misaligned pool of layer %d (16 B)", l);
    int32_t dummy = 0;
    if (int r = validate_selection(&tables[l], selections + (size_t)l * n_sel, n_sel, &dummy)) return r;
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    hipError_t pe = hipPointerGetAttributes(&attr, host_pools[l]);
    if (pe != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return fail(KV_EINVAL, "host pool of layer %d is not pinned, device-accessible host memory", l);
    }
  }
  const int64_t pb = page_bytes_of(shape);
  const size_t total = (size_t)n_layers * n_sel;
  std::vector<int32_t> slots(total), mp(n_sel), ms(n_sel);
  std::vector<const uint8_t*> src;
  std::vector<uint8_t*> dst;
  for (int32_t l = 0; l < n_layers; ++l) {
    int32_t misses = 0;
    if (int r = kv_residency_select(&tables[l], selections + (size_t)l * n_sel, n_sel,
                                    slots.data() + (size_t)l * n_sel, mp.data(), ms.data(), &misses))
      return r;  // (earlier layers' tables were updated; nothing was enqueued)
    for (int32_t i = 0; i < misses; ++i) {
      src.push_back((const uint8_t*)host_pools[l] + (int64_t)mp[i] * pb);
      dst.push_back((uint8_t*)slot_pools[l] + (int64_t)ms[i] * pb);
    }
    if (out_n_miss) out_n_miss[l] = misses;
  }
  // launches of at most kMultiMaxCopies copies and kMultiMaxEntries block-table entries
  size_t done_e = 0, done_c = 0;
  while (done_e < total || done_c < src.size()) {
    MultiGatherBatch gb;
    const size_t ne = total - done_e < (size_t)kMultiMaxEntries ? total - done_e : kMultiMaxEntries;
    const size_t nc = src.size() - done_c < (size_t)kMultiMaxCopies ? src.size() - done_c : kMultiMaxCopies;
    gb.n_entries = (int32_t)ne;
    gb.n_copies = (int32_t)nc;
    gb.block_tables = out_block_tables + done_e;
    for (size_t i = 0; i < ne; ++i) gb.slots[i] = slots[done_e + i];
    for (size_t i = 0; i < nc; ++i) {
      gb.src[i] = src[done_c + i];
      gb.dst[i] = dst[done_c + i];
    }
    const bool first = done_e == 0 && done_c == 0;
    const bool last = done_e + ne == total && done_c + nc == src.size();
    hipError_t e = launch_gather_multi_timed(gb, pb, (hipStream_t)stream, first ? (hipEvent_t)start_event : nullptr,
                                             last ? (hipEvent_t)stop_event : nullptr);
    if (e != hipSuccess) return hip_fail(e, "gather launch (the residency tables were already updated)");
    done_e += ne;
    done_c += nc;
  }
  return ok();
}

}  // namespace

extern "C" {

int kv_gather_pages_layers(const kv_shape* shape, int32_t n_layers, kv_residency* tables,
                           const int32_t* selections, int32_t n_sel, const void* const* host_pools,
                           void* const* slot_pools, int32_t* out_block_tables, int32_t* out_n_miss,
                           void* stream) {
  return gather_layers(shape, n_layers, tables, selections, n_sel, host_pools, slot_pools, out_block_tables,
                       out_n_miss, stream, nullptr, nullptr);
}

int kv_gather_pages_layers_timed(const kv_shape* shape, int32_t n_layers, kv_residency* tables,
                                 const int32_t* selections, int32_t n_sel, const void* const* host_pools,
                                 void* const* slot_pools, int32_t* out_block_tables, int32_t* out_n_miss,
                                 void* stream, void* start_event, void* stop_event) {
  return gather_layers(shape, n_layers, tables, selections, n_sel, host_pools, slot_pools, out_block_tables,
                       out_n_miss, stream, start_event, stop_event);
}

int kv_page_key_sums(const kv_shape* shape, const void* k, int64_t n_tokens, int64_t start_pos,
                     int64_t* sums, void* reps, int64_t n_pages_cap, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (n_tokens < 0 || start_pos < 0) return fail(KV_EINVAL, "negative token count or position");
  if (n_tokens == 0) return ok();
  if (!k || !sums || !reps) return fail(KV_EINVAL, "NULL buffer");
  if (!aligned(k, 2) || !aligned(sums, 8) || !aligned(reps, 2))
    return fail(KV_EALIGN, "misaligned buffer (k: 2 B, sums: 8 B, reps: 2 B)");
  if (n_tokens > INT64_MAX - start_pos)  // (so that start_pos + n_tokens below cannot overflow)
    return fail(KV_EINVAL, "start_pos + n_tokens overflows");
  if ((start_pos + n_tokens - 1) / kPageTokens >= n_pages_cap)
    return fail(KV_EINVAL, "tokens up to position %lld need more than %lld pages of sums",
                (long long)(start_pos + n_tokens - 1), (long long)n_pages_cap);
  hipError_t e = launch_key_sums(shape->n_kv_heads, (const uint16_t*)k, n_tokens, start_pos, sums,
                                 (uint16_t*)reps, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "key-sum launch");
  return ok();
}

size_t kv_select_workspace_bytes(int64_t n_pages, int32_t n_sets) {
  if (n_pages < 0 || n_pages > select_max_pages() || n_sets < 0 || n_sets > 65535) {
    fail(KV_EINVAL, "n_pages (0..%d) or n_sets (0..65535) out of range", select_max_pages());
    return 0;
  }
  ok();
  const int64_t n = (int64_t)n_pages * n_sets;
  return (size_t)(n > 0 ? n : 1) * 16;
}

int kv_select_pages(const kv_shape* shape, const void* q, const void* reps, int64_t reps_pages,
                    int64_t n_pages, int32_t k_sel, int32_t n_sets, int32_t* out_selection,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (n_pages < 0 || n_pages > select_max_pages())
    return fail(KV_EINVAL, "n_pages out of range (0..%d)", select_max_pages());
  if (k_sel < 1 || k_sel > select_max_k()) return fail(KV_EINVAL, "k_sel out of range (1..%d)", select_max_k());
  if (shape->n_kv_heads > select_max_kv_heads())
    return fail(KV_EUNSUPPORTED, "page selection takes at most %d KV heads", select_max_kv_heads());
  if (n_sets < 0 || n_sets > 65535) return fail(KV_EINVAL, "n_sets out of range (0..65535)");
  if (reps_pages < n_pages) return fail(KV_EINVAL, "reps_pages (%lld) below n_pages (%lld)",
                                        (long long)reps_pages, (long long)n_pages);
  if (n_pages == 0 || n_sets == 0) return ok();
  if (!q || !reps || !out_selection || !workspace) return fail(KV_EINVAL, "NULL buffer");
  if (!aligned(q, 2) || !aligned(reps, 16) || !aligned(out_selection, 4) || !aligned(workspace, 16))
    return fail(KV_EALIGN, "misaligned buffer (q: 2 B, reps: 16 B, selection: 4 B, workspace: 16 B)");
  const size_t need = (size_t)n_pages * n_sets * 16;
  if (workspace_bytes < need)
    return fail(KV_ESMALL, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  hipError_t e = launch_select(shape->n_q_heads, shape->n_kv_heads, (const uint16_t*)q, (const uint16_t*)reps, reps_pages,
                               (int)n_pages, k_sel, n_sets, out_selection, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "selection launch");
  return ok();
}

uint16_t kv_host_f64_to_f16(double x) { return f64_to_f16_rne(x); }

int kv_host_encode_vector(int32_t kind, const uint16_t* x, uint8_t* codes, uint16_t* scales) {
  if (!x || !codes || !scales) return fail(KV_EINVAL, "NULL buffer");
  if (kind == kInt8) {
    for (int g = 0; g < 4; ++g) {
      double a = 0.0;
      for (int e = 64 * g; e < 64 * g + 64; ++e) {
        const double v = f16_to_f64(x[e]);
        const double av = v < 0 ? -v : v;
        if (av > a) a = av;
      }
      scales[g] = f64_to_f16_rne(a / 127.0);
      const double d = f16_to_f64(scales[g]);
      for (int e = 64 * g; e < 64 * g + 64; ++e)
        codes[e] = (uint8_t)(int8_t)int8_code(f16_to_f64(x[e]), d);
    }
    return ok();
  }
  if (kind == kFp8) {
    double a = 0.0;
    for (int e = 0; e < kHeadDim; ++e) {
      const double v = f16_to_f64(x[e]);
      const double av = v < 0 ? -v : v;
      if (av > a) a = av;
    }
    scales[0] = f64_to_f16_rne(a / 448.0);
    const double d = f16_to_f64(scales[0]);
    for (int e = 0; e < kHeadDim; ++e) codes[e] = (uint8_t)fp8_code(f16_to_f64(x[e]), d);
    return ok();
  }
  if (kind == kQ4 || kind == kFp4) {
    double y[kHeadDim];
    for (int e = 0; e < kHeadDim; ++e) y[e] = f16_to_f64(x[e]);
    for (int len = 1; len < kHeadDim; len <<= 1)  // Sylvester butterflies, exact in fp64
      for (int i = 0; i < kHeadDim; i += 2 * len)
        for (int j = i; j < i + len; ++j) {
          const double a = y[j], b = y[j + len];
          y[j] = a + b;
          y[j + len] = a - b;
        }
    for (int e = 0; e < kHeadDim; ++e) y[e] *= 0.0625;
    if (kind == kFp4) {
      for (int blk = 0; blk < 8; ++blk) {
        double a = 0.0;
        for (int e = 32 * blk; e < 32 * blk + 32; ++e) a = (y[e] < 0 ? -y[e] : y[e]) > a ? (y[e] < 0 ? -y[e] : y[e]) : a;
        const int ex = fp4_block_exp(a);
        scales[blk] = a == 0.0 ? (uint16_t)0 : fp16_pow2_bits(ex);
        for (int e = 32 * blk; e < 32 * blk + 32; ++e) codes[e] = (uint8_t)(a == 0.0 ? 0 : fp4_code(y[e], ex));
      }
      return ok();
    }
    for (int blk = 0; blk < 8; ++blk) {
      double m = y[32 * blk];
      for (int e = 32 * blk + 1; e < 32 * blk + 32; ++e) {
        const double am = m < 0 ? -m : m, ae = y[e] < 0 ? -y[e] : y[e];
        if (ae > am) m = y[e];
      }
      scales[blk] = f64_to_f16_rne(-m * 0.125);
      const double d = f16_to_f64(scales[blk]);
      for (int e = 32 * blk; e < 32 * blk + 32; ++e) codes[e] = (uint8_t)q4_code(y[e], d);
    }
    return ok();
  }
  return fail(KV_EINVAL, "kind must be 0 (int8), 1 (q4), 2 (fp4) or 3 (fp8)");
}

}  // extern "C"
