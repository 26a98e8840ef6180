// kv_internal.h - shared definitions of the HIP library (not installed).
//
// Record rules and page layout are those documented in include/kvcache.h; this
// header holds their constants, the exact fp64 -> fp16 rounding and the
// kernel launchers the C ABI dispatches to.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvcache.h"

namespace kvc {

constexpr int kHeadDim = 256;
constexpr int kPageTokens = 256;
constexpr int kDefaultComputeUnits = 256;  // MI355X (8 XCDs x 32 CUs): used when no device is visible

// Compute units of the current device (hipDeviceAttributeMultiprocessorCount, read once per
// device); kDefaultComputeUnits when no device can be queried (host-only use of the sizing
// functions). The split sizes and grids are chosen from it.
int device_compute_units();
constexpr int kMaxGroup = 8;  // query heads per KV head handled by one MFMA row tile

enum RecordKind : int { kInt8 = 0, kQ4 = 1, kFp4 = 2, kFp8 = 3 };
// q4_0 and fp4 records: rotated by H, 4-bit codes in the same byte layout, 8 fp16 scales;
// int8 and fp8 records: one byte per code in the same byte layout, not rotated
__host__ __device__ constexpr bool four_bit(int kind) { return kind == kQ4 || kind == kFp4; }

__host__ __device__ constexpr int code_row_bytes(int kind) { return four_bit(kind) ? 128 : 256; }
__host__ __device__ constexpr int n_scales(int kind) { return kind == kInt8 ? 4 : (kind == kFp8 ? 1 : 8); }
__host__ __device__ constexpr int plane_bytes(int kind) {
  return kPageTokens * code_row_bytes(kind) + kPageTokens * n_scales(kind) * 2;
}
__host__ __device__ constexpr int k_kind(int fmt) {
  return fmt == KV_FMT_Q4_0 ? kQ4 : (fmt == KV_FMT_FP4 ? kFp4 : (fmt == KV_FMT_FP8 ? kFp8 : kInt8));
}
__host__ __device__ constexpr int v_kind(int fmt) {
  return fmt == KV_FMT_INT8 ? kInt8 : (fmt == KV_FMT_FP4 ? kFp4 : (fmt == KV_FMT_FP8 ? kFp8 : kQ4));
}
// Waves per workgroup of the split-K decode kernel: 4 (two workgroups per CU) for
// 4-bit K; 8 (one workgroup per CU, half the registers per wave) for int8 K, whose
// tiles are twice as large.
__host__ __device__ constexpr int split_waves(int k_kind_) { return four_bit(k_kind_) ? 4 : 8; }
__host__ __device__ constexpr int64_t head_stride(int fmt) {
  return plane_bytes(k_kind(fmt)) + plane_bytes(v_kind(fmt));
}

// Round a double to the nearest fp16 (ties to even), once, from its bits.
// IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; values
// below 2^-14 are subnormal multiples of 2^-24; overflow gives infinity.
__host__ __device__ inline uint16_t f64_to_f16_rne(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int exp = (int)((b >> 52) & 0x7FF);
  const uint64_t frac = b & 0xFFFFFFFFFFFFFull;
  if (exp == 0x7FF) return (uint16_t)(sign | 0x7C00u | (frac ? 0x200u : 0u));
  if (exp == 0) return sign;                    // |x| < 2^-1022
  int e = exp - 1023;
  if (e >= 16) return (uint16_t)(sign | 0x7C00u);
  const uint64_t m = frac | (1ull << 52);       // |x| = m * 2^(e - 52)
  const bool normal = e >= -14;
  const int sh = normal ? 42 : 28 - e;          // target unit 2^(e-10), or 2^-24
  if (sh >= 64) return sign;
  uint64_t q = m >> sh;
  const uint64_t rem = m & ((1ull << sh) - 1);
  const uint64_t half = 1ull << (sh - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (normal) {
    if (q == 2048) { q = 1024; ++e; }
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | ((e + 15) << 10) | (uint16_t)(q - 1024));
  }
  return (uint16_t)(sign | q);                  // q == 1024 is the least normal
}

__host__ __device__ inline double f16_to_f64(uint16_t h) {
  return (double)__builtin_bit_cast(_Float16, h);
}

// int8 code of x for the stored scale d: round half away from zero, clamp.
// x/d is formed in fp64; it cannot fall within fp64 rounding of a half
// integer without being one, so the decision is the exact one.
__host__ __device__ inline int int8_code(double x, double d) {
  if (d == 0.0) return 0;
  const double q = x / d;
  if (q != q) return 0;  // (NaN, e.g. inf / inf: code 0, so the conversion below is defined)
  const double a = q < 0 ? -q : q;
  double r = __builtin_floor(a);
  if (a - r >= 0.5) r += 1.0;
  int c = (int)r;
  if (c > 127) c = 127;
  return q < 0 ? -c : c;
}

// q4 code of y for the stored scale d: round half up, offset 8, clamp.
__host__ __device__ inline int q4_code(double y, double d) {
  if (d == 0.0) return 8;
  const double q = y / d;
  if (q != q) return 8;  // (NaN, e.g. inf / inf: code 8, so the conversion below is defined)
  double r = __builtin_floor(q);
  if (q - r >= 0.5) r += 1.0;
  double c = r + 8.0;
  if (c < 0.0) c = 0.0;
  if (c > 15.0) c = 15.0;
  return (int)c;
}

// Launchers (stream-ordered, arguments already validated by the C ABI).
hipError_t launch_append(int fmt, int n_kv_heads, const uint16_t* k, const uint16_t* v,
                         int64_t n_tokens, int64_t start_pos, const int32_t* block_table,
                         int32_t n_table, uint8_t* pool, int64_t n_pool_pages,
                         int32_t* status, hipStream_t stream, hipEvent_t start = nullptr,
                         hipEvent_t stop = nullptr);

// fp4 record helpers (rules in include/kvcache.h). a = max |y| of a block (exact, a
// normal double or 0): the block exponent clamp(floor(log2 a) - 2, -23, 13).
__host__ __device__ inline int fp4_block_exp(double a) {
  const int ex = (int)((__builtin_bit_cast(uint64_t, a) >> 52) & 0x7FF) - 1023;  // floor(log2 a)
  const int e = ex - 2;
  return e < -23 ? -23 : (e > 13 ? 13 : e);
}
// 2^e as fp16 bits (exact for -24 <= e <= 15: normal from 2^-14, subnormal below).
__host__ __device__ inline uint16_t fp16_pow2_bits(int e) {
  return e >= -14 ? (uint16_t)((e + 15) << 10) : (uint16_t)(1u << (e + 24));
}
// 2^e as a double (exact).
__host__ __device__ inline double f64_pow2(int e) {
  return __builtin_bit_cast(double, (uint64_t)(e + 1023) << 52);
}
// Code of y in a block with exponent e (d = 2^e > 0): the e2m1 grid index of |y| / d,
// nearest with ties to the even index, saturating at 6; plus 8 for y < 0 (index > 0).
__host__ __device__ inline int fp4_code(double y, int e) {
  const double v = (y < 0 ? -y : y) * f64_pow2(-e);  // exact
  const int idx = (v > 0.25) + (v >= 0.75) + (v > 1.25) + (v >= 1.75) + (v > 2.5) + (v >= 3.5) + (v > 5.0);
  return idx + ((y < 0 && idx > 0) ? 8 : 0);
}

// fp8 record helpers (rules in include/kvcache.h). Code of x for the stored scale d > 0:
// |x| / d (an exact decision in fp64) to the nearest E4M3 magnitude, ties to the even
// mantissa, beyond 448 to 448; sign bit 0x80 for x < 0 unless the magnitude is 0.
// E4M3: magnitudes below 2^-6 are multiples of 2^-9 (exponent field 0); from 2^E
// (E >= -6) on, multiples of 2^(E-3) with exponent field E + 7.
__host__ __device__ inline int fp8_code(double x, double d) {
  if (d == 0.0) return 0;
  const double v = (x < 0 ? -x : x) / d;
  if (v != v) return 0;  // (NaN, e.g. inf / inf: code 0, never the NaN code)
  if (v >= 464.0) return x < 0 ? 0xFE : 0x7E;                // at and past the last midpoint
  const int ex = (int)((__builtin_bit_cast(uint64_t, v) >> 52) & 0x7FF) - 1023;  // floor(log2 v)
  const bool sub = v < 0x1p-6;
  const int ue = sub ? -9 : ex - 3;                           // unit 2^ue
  const double n = v * __builtin_bit_cast(double, (uint64_t)(1023 - ue) << 52);  // v / 2^ue, exact
  double r = __builtin_floor(n);
  const double f = n - r;
  if (f > 0.5 || (f == 0.5 && __builtin_fmod(r, 2.0) == 1.0)) r += 1.0;
  // subnormal: r in [0, 8] (8 = the least normal, field 1); normal: r in [8, 16]
  int c = sub ? (int)r : ((ex + 7) << 3) + (int)r - 8;
  if (c > 0x7E) c = 0x7E;
  return (x < 0 && c > 0) ? (c | 0x80) : c;
}

struct DecodeArgs {
  int fmt;
  int n_q_heads, n_kv_heads;
  int batch;                  // rows of q / out: sequences x queries per sequence
  int n_q = 1;                // queries per sequence (rows b * n_q .. b * n_q + n_q - 1)
  const uint16_t* q;
  const uint8_t* pool;
  int64_t n_pool_pages;
  const int32_t* block_tables;
  int32_t max_pages;
  const int32_t* context_lens;  // [batch / n_q]: query j of a sequence of length T sees T - n_q + j + 1 tokens
  int32_t max_context;        // clamp bound, already min(max_context, max_pages * 256)
  int32_t pages_per_split;
  int32_t n_splits;           // grid size along the context
  int32_t n_cus = kDefaultComputeUnits;  // compute units of the device (grid sizing)
  float scale_log2;           // softmax_scale * log2(e)
  float* out;
  int32_t* status;
  uint32_t* sched;            // two work counters, zero between launches
  float* part_ml;             // [batch][n_q_heads][n_splits][2]
  float* part_o;              // [batch][n_q_heads][n_splits][256]
  // optional: one token per sequence appended by the split kernel (position
  // context_lens[b] - 1) before attention reads it; null = no append
  const uint16_t* k_new = nullptr;  // [batch][n_kv_heads][256] fp16
  const uint16_t* v_new = nullptr;
  uint8_t* pool_w = nullptr;        // the pool, writable
};

// phase: 1 = split kernel only, 2 = combine only, 3 = both. start/stop (may be
// null) are recorded at the split kernel's own start and end.
hipError_t launch_decode(const DecodeArgs& a, int phase, hipStream_t stream,
                         hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// Sets n_words 32-bit words at p to zero with a small kernel on `stream` (a kernel rather
// than a memset, so that it can also be recorded into a HIP graph).
hipError_t launch_zero_words(uint32_t* p, int n_words, hipStream_t stream);

// Page selection (kv_select.hip).
hipError_t launch_key_sums(int n_kv_heads, const uint16_t* k, int64_t n_tokens, int64_t start_pos,
                           int64_t* sums, uint16_t* reps, hipStream_t stream);
hipError_t launch_select(int n_q_heads, int n_kv_heads, const uint16_t* q, const uint16_t* reps,
                         int64_t reps_pages, int n_pages, int k_sel, int n_sets, int32_t* out, void* scores,
                         hipStream_t stream);
int select_max_pages();
int select_max_k();
int select_max_kv_heads();

constexpr int kGatherMaxBatch = 256;  // selections per gather launch (kernel-argument size)

struct GatherBatch {
  int32_t n_sel;
  int32_t n_miss;
  int32_t slots[kGatherMaxBatch];       // slot of each selected page, in order
  int32_t miss_page[kGatherMaxBatch];   // page ids to copy
  int32_t miss_slot[kGatherMaxBatch];   // destination slots
};

// Page copies of several layers in one launch (kernel arguments): each copy has its
// own source (pinned host page) and destination (device slot); the block tables of all
// layers are one device array [n_layers][n_sel].
constexpr int kMultiMaxCopies = 96;
constexpr int kMultiMaxEntries = 256;  // block-table entries per launch
struct MultiGatherBatch {
  int32_t n_copies;
  int32_t n_entries;                       // block-table entries written by this launch
  int32_t* block_tables;                   // where entry 0 of this launch goes
  const uint8_t* src[kMultiMaxCopies];
  uint8_t* dst[kMultiMaxCopies];
  int32_t slots[kMultiMaxEntries];
};

hipError_t launch_gather_multi(const MultiGatherBatch& batch, int64_t page_bytes, hipStream_t stream);

hipError_t launch_gather(const GatherBatch& batch, int64_t page_bytes, const uint8_t* host_pool,
                         uint8_t* slot_pool, int32_t* out_block_table, hipStream_t stream);

}  // namespace kvc
