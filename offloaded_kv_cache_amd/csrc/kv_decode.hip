// kv_decode.hip - split-K GQA decode attention over the paged, block-quantized
// KV cache, for gfx950 (CDNA4).
//
// What is computed (KV-offload news page, section "缓存为何不能直接搬走？":
// a decode step reads the whole KV of every full-attention layer; Strata page
// "KV 沉进内存、显存减半：Strata 让 12 GB 显卡跑满 262K 上下文", section "4-bit
// KV 缓存：先旋转，再压到 4-bit": with rotated K the query is rotated by H so
// that <Hq, Hk> = <q, k>, and with rotated V the mixed output is multiplied by
// H): for every sequence and query head, softmax(scale * q'.k^) . v^ over the
// dequantized records, then H for rotated V.
//
// Kernel 1 (decode_split): one workgroup of four wavefronts per (split, KV
// head, sequence). A split is `pages_per_split` consecutive logical pages;
// wave w takes pages w, w+4, ... of it, one whole 256-token page at a time:
//   - Q.K on MFMA 16x16x32 f16. A = the rotated query of the group's heads,
//     each head as two fp16 rows (hi, lo) so the fp32 query is carried to
//     ~22 bits; B = 16 tokens x 32 elements of exact integer codes (q4: c-8,
//     int8: c), unpacked with bit tricks (1024 + c as fp16, then a packed
//     fp16 subtract). One MFMA covers one 32-element block, so the block (q4)
//     or group (int8) scale is applied to the fp32 accumulators afterwards.
//   - online softmax over the page in the log2 domain, with the wave's
//     running max and sum; probabilities are scaled by 2^14 and split into
//     fp16 hi/lo parts, kept in LDS.
//   - P.V on MFMA 16x16x32 f16 with the contraction over tokens. The V plane
//     is element-major, so a lane's 8 k-slots are 8 tokens of one element:
//     one dword of q4 codes (two 4-token runs) or two dwords of int8 codes.
//     The per-token scale d varies along the contraction, so it goes into B
//     exactly: d is split into parts with few enough bits that every
//     (code x part) product is exact in fp16 (q4: two parts of <= 8 and 3
//     bits; int8: three parts of <= 4 bits), one MFMA per part.
//   - the four waves merge their (max, sum, output) in LDS and the workgroup
//     writes one partial per query head.
// Kernel 2 (decode_combine): per (query head, sequence), the log-sum-exp
// merge of the partials, then the rotation back by H (fp32 butterflies) when
// V is stored rotated.
//
// Tokens past the context length are masked (score -inf, scale 0), so stale
// or uninitialised rows of a last, partly filled page never contribute.
// Nothing depends on the physical page ids except the addresses read.
#include "kv_internal.h"

namespace kvc {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr float kPScale = 16384.0f;  // probabilities are kept as p * 2^14 in fp16 hi/lo
constexpr float kPScaleInv = 1.0f / 16384.0f;

__device__ inline h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }

// Eight 4-bit codes (bytes b0..b3, low and high nibbles) -> c - 8 as fp16,
// slot order [lo0, lo1, lo2, lo3, hi0, hi1, hi2, hi3].
__device__ inline h8 unpack_q4(uint32_t x) {
  const uint32_t t01 = (x & 0xFFu) | ((x << 8) & 0xFF0000u);          // halves (b0, b1)
  const uint32_t t23 = ((x >> 16) & 0xFFu) | ((x >> 8) & 0xFF0000u);  // halves (b2, b3)
  const h2 lo01 = as_h2((t01 & 0x000F000Fu) | 0x64006400u) - (h2){1032, 1032};
  const h2 lo23 = as_h2((t23 & 0x000F000Fu) | 0x64006400u) - (h2){1032, 1032};
  // high nibble sits at bits 4..7: 1024 + 16c, scaled by 1/16 and shifted: c - 8
  const h2 hi01 = __builtin_elementwise_fma(as_h2((t01 & 0x00F000F0u) | 0x64006400u),
                                            (h2){0.0625, 0.0625}, (h2){-72, -72});
  const h2 hi23 = __builtin_elementwise_fma(as_h2((t23 & 0x00F000F0u) | 0x64006400u),
                                            (h2){0.0625, 0.0625}, (h2){-72, -72});
  return (h8){lo01[0], lo01[1], lo23[0], lo23[1], hi01[0], hi01[1], hi23[0], hi23[1]};
}

// Eight int8 codes (x0 bytes 0..3, x1 bytes 4..7) -> fp16, natural order.
__device__ inline h8 unpack_i8(uint32_t x0, uint32_t x1) {
  const uint32_t u0 = x0 ^ 0x80808080u, u1 = x1 ^ 0x80808080u;  // c + 128
  const h2 a = as_h2((u0 & 0xFFu) | ((u0 << 8) & 0xFF0000u) | 0x64006400u) - (h2){1152, 1152};
  const h2 b = as_h2(((u0 >> 16) & 0xFFu) | ((u0 >> 8) & 0xFF0000u) | 0x64006400u) - (h2){1152, 1152};
  const h2 c = as_h2((u1 & 0xFFu) | ((u1 << 8) & 0xFF0000u) | 0x64006400u) - (h2){1152, 1152};
  const h2 d = as_h2(((u1 >> 16) & 0xFFu) | ((u1 >> 8) & 0xFF0000u) | 0x64006400u) - (h2){1152, 1152};
  return (h8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ inline f4 mfma(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline float half_max(float v) {  // max over the 16 lanes of a lane group
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}
__device__ inline float half_sum(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}

// LDS of one wave while it works on a page.
//   sp:     first the page's scores (fp32 bits, log2 domain), then in place
//           p * 2^14 as two fp16 halves (hi | lo << 16), per head and token
//   dsplit: the page's V scales split into exact fp16 parts, per 4-token run:
//           q4   [8 blocks][64 runs][8]  = {hi x 4 tokens, lo x 4 tokens}
//           int8 [4 groups][64 runs][16] = {a x 4, b x 4, c x 4, pad x 4}
struct WaveLds {
  uint32_t sp[kMaxGroup][kPageTokens];
  _Float16 dsplit[4096];
};
__device__ inline int dsplit_q4(int blk, int run) { return (blk * 64 + run) * 8; }
__device__ inline int dsplit_i8(int grp, int run) { return (grp * 64 + run) * 16; }
static_assert(sizeof(WaveLds) == 16384, "wave LDS");

struct MergeLds {
  float m[4][kMaxGroup];
  float l[4][kMaxGroup];
  float o[4][kMaxGroup][kHeadDim];
};

constexpr int kWaves = 4;
constexpr size_t kSplitLds = (sizeof(WaveLds) * kWaves > sizeof(MergeLds) ? sizeof(WaveLds) * kWaves
                                                                         : sizeof(MergeLds));

// One 16-token tile of a K plane, as loaded by one lane (token = its column).
struct KTile {
  u4 c0, c1, c2, c3;  // code bytes of the lane's slice (q4: c0, c1; int8: all four)
  u4 d;               // the token's scales (q4: 8 fp16; int8: 4 fp16 in d.xy)
};

template <int KK>
__device__ inline KTile load_ktile(const uint8_t* kpl, int row, int grp) {
  KTile t;
  if (KK == kQ4) {
    const u4* cp = reinterpret_cast<const u4*>(kpl + (size_t)row * 128 + 32 * grp);
    t.c0 = cp[0];
    t.c1 = cp[1];
    t.c2 = t.c3 = (u4){0, 0, 0, 0};
    t.d = *reinterpret_cast<const u4*>(kpl + 256 * 128 + (size_t)row * 16);
  } else {
    const u4* cp = reinterpret_cast<const u4*>(kpl + (size_t)row * 256 + 64 * grp);
    t.c0 = cp[0];
    t.c1 = cp[1];
    t.c2 = cp[2];
    t.c3 = cp[3];
    const u2 dd = *reinterpret_cast<const u2*>(kpl + 256 * 256 + (size_t)row * 8);
    t.d = (u4){dd[0], dd[1], 0, 0};
  }
  return t;
}

__device__ inline float scale_at(u4 d, int j) {  // fp16 scale j of a packed row of scales
  const uint32_t w = d[j >> 1];
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((j & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

// Raw scores of one tile for the lane's two heads (rows 4grp..4grp+3 = head 2grp hi, lo,
// head 2grp+1 hi, lo).
template <int KK>
__device__ inline void qk_tile(const KTile& t, const h8 (&qa)[8], float& s0, float& s1) {
  s0 = 0.f;
  s1 = 0.f;
  if (KK == kQ4) {
    const uint32_t w[8] = {t.c0[0], t.c0[1], t.c0[2], t.c0[3], t.c1[0], t.c1[1], t.c1[2], t.c1[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f4 acc = mfma(qa[j], unpack_q4(w[j]), (f4){0.f, 0.f, 0.f, 0.f});
      const float d = scale_at(t.d, j);
      s0 = fmaf(d, acc[0] + acc[1], s0);
      s1 = fmaf(d, acc[2] + acc[3], s1);
    }
  } else {
    const uint32_t w[16] = {t.c0[0], t.c0[1], t.c0[2], t.c0[3], t.c1[0], t.c1[1], t.c1[2], t.c1[3],
                            t.c2[0], t.c2[1], t.c2[2], t.c2[3], t.c3[0], t.c3[1], t.c3[2], t.c3[3]};
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      f4 acc = mfma(qa[2 * gg], unpack_i8(w[4 * gg], w[4 * gg + 1]), (f4){0.f, 0.f, 0.f, 0.f});
      acc = mfma(qa[2 * gg + 1], unpack_i8(w[4 * gg + 2], w[4 * gg + 3]), acc);
      const float d = scale_at(t.d, gg);
      s0 = fmaf(d, acc[0] + acc[1], s0);
      s1 = fmaf(d, acc[2] + acc[3], s1);
    }
  }
}

// Two packed (hi | lo << 16) probabilities -> the two fp16 of one part.
__device__ inline uint32_t pick_part(uint32_t w0, uint32_t w1, int shift) {
  return ((w0 >> shift) & 0xFFFFu) | (((w1 >> shift) & 0xFFFFu) << 16);
}

template <int KK, int VK>
__global__ __launch_bounds__(256, 2) void decode_split(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ pool, int64_t n_pool_pages,
    const int32_t* __restrict__ block_tables, int max_pages, const int32_t* __restrict__ context_lens,
    int max_context, int n_q_heads, int n_kv_heads, int pages_per_split, int n_splits,
    float scale_log2, float* __restrict__ part_ml, float* __restrict__ part_o,
    int32_t* __restrict__ status) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kSplitLds];
  __shared__ float qs[kMaxGroup][kHeadDim];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;  // MFMA lane group and column
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = n_q_heads / n_kv_heads;

  int T = context_lens[b];
  if (T > max_context || T < 0) {
    if (tid == 0 && split == 0 && g == 0) atomicOr(status, KV_STATUS_CONTEXT_CLAMPED);
    T = T < 0 ? 0 : max_context;
  }
  const int n_pages = (T + kPageTokens - 1) / kPageTokens;
  const int p_begin = split * pages_per_split;
  const int p_end = min(n_pages, p_begin + pages_per_split);
  if (p_begin >= p_end) return;  // uniform over the workgroup

  // ---- query of the group's heads, rotated by H when K is stored rotated
  for (int hh = 0; hh < G; ++hh)
    qs[hh][tid] = (float)__builtin_bit_cast(_Float16, q[((size_t)b * n_q_heads + g * G + hh) * kHeadDim + tid]);
  __syncthreads();
  if (KK == kQ4) {
    for (int bit = 0; bit < 8; ++bit) {
      const int m = 1 << bit;
      float vals[kMaxGroup];
      for (int hh = 0; hh < G; ++hh) {
        const float mine = qs[hh][tid], other = qs[hh][tid ^ m];
        vals[hh] = (tid & m) ? (other - mine) : (mine + other);
      }
      __syncthreads();
      for (int hh = 0; hh < G; ++hh) qs[hh][tid] = vals[hh];
      __syncthreads();
    }
    for (int hh = 0; hh < G; ++hh) qs[hh][tid] *= 0.0625f;
    __syncthreads();
  }

  // A operands of Q.K: row r = 2*head + part; MFMA j covers block j (elements 32j..32j+31)
  const int a_head = col >> 1, a_part = col & 1;
  h8 qa[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      int e;
      if (KK == kQ4) e = 32 * j + (s < 4 ? 4 * grp + s : 16 + 4 * grp + (s - 4));
      else e = 32 * j + 8 * grp + s;
      const float f = qs[a_head < G ? a_head : 0][e];
      const _Float16 hi = (_Float16)f;
      const _Float16 lo = (_Float16)(f - (float)hi);
      qa[j][s] = a_head < G ? (a_part ? lo : hi) : (_Float16)0;
    }
  }

  WaveLds& wl = reinterpret_cast<WaveLds*>(lds_raw)[wave];

  // per-lane running state for the two heads of its row group (rows 4grp..4grp+3)
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f4 oacc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) oacc[t] = (f4){0.f, 0.f, 0.f, 0.f};

  const int64_t page_bytes = (int64_t)n_kv_heads * (plane_bytes(KK) + plane_bytes(VK));
  const int32_t* bt = block_tables + (size_t)b * max_pages;
  const int h0 = 2 * grp, h1 = 2 * grp + 1;

  for (int pg = p_begin + wave; pg < p_end; pg += kWaves) {
    const int32_t phys = bt[pg];
    if (phys < 0 || phys >= n_pool_pages) {
      if (lane == 0) atomicOr(status, KV_STATUS_BAD_PAGE_ID);
      continue;
    }
    const uint8_t* kpl = pool + (int64_t)phys * page_bytes + (int64_t)g * (plane_bytes(KK) + plane_bytes(VK));
    const uint8_t* vpl = kpl + plane_bytes(KK);
    const int valid = min(kPageTokens, T - pg * kPageTokens);  // tokens of this page in context

    // ---------------- Q.K: 16 tiles of 16 tokens, one tile of loads ahead
    float mx0 = -INFINITY, mx1 = -INFINITY;
    KTile cur = load_ktile<KK>(kpl, col, grp);
#pragma unroll 1
    for (int tile = 0; tile < 16; ++tile) {
      const int row = tile * 16 + col;
      const KTile nxt = load_ktile<KK>(kpl, min(tile + 1, 15) * 16 + col, grp);
      float s0, s1;
      qk_tile<KK>(cur, qa, s0, s1);
      const bool ok = row < valid;
      const float x0 = ok ? s0 * scale_log2 : -INFINITY;
      const float x1 = ok ? s1 * scale_log2 : -INFINITY;
      mx0 = fmaxf(mx0, x0);
      mx1 = fmaxf(mx1, x1);
      wl.sp[h0][row] = __builtin_bit_cast(uint32_t, x0);
      wl.sp[h1][row] = __builtin_bit_cast(uint32_t, x1);
      cur = nxt;
    }

    // ---------------- online softmax over the page (log2 domain)
    mx0 = half_max(mx0);
    mx1 = half_max(mx1);
    const float mn0 = fmaxf(m_run[0], mx0), mn1 = fmaxf(m_run[1], mx1);
    const float al0 = exp2f(m_run[0] - mn0), al1 = exp2f(m_run[1] - mn1);
    m_run[0] = mn0;
    m_run[1] = mn1;
    float sum0 = 0.f, sum1 = 0.f;
#pragma unroll 4
    for (int tile = 0; tile < 16; ++tile) {
      const int row = tile * 16 + col;
      const float p0 = exp2f(__builtin_bit_cast(float, wl.sp[h0][row]) - mn0);
      const float p1 = exp2f(__builtin_bit_cast(float, wl.sp[h1][row]) - mn1);
      sum0 += p0;
      sum1 += p1;
      const float ps0 = p0 * kPScale, ps1 = p1 * kPScale;
      const _Float16 hi0 = (_Float16)ps0, hi1 = (_Float16)ps1;
      const _Float16 lo0 = (_Float16)(ps0 - (float)hi0), lo1 = (_Float16)(ps1 - (float)hi1);
      wl.sp[h0][row] = (uint32_t)__builtin_bit_cast(uint16_t, hi0) | ((uint32_t)__builtin_bit_cast(uint16_t, lo0) << 16);
      wl.sp[h1][row] = (uint32_t)__builtin_bit_cast(uint16_t, hi1) | ((uint32_t)__builtin_bit_cast(uint16_t, lo1) << 16);
    }
    l_run[0] = l_run[0] * al0 + sum0;
    l_run[1] = l_run[1] * al1 + sum1;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      oacc[t][0] *= al0;
      oacc[t][1] *= al0;
      oacc[t][2] *= al1;
      oacc[t][3] *= al1;
    }

    // ---------------- V scales of the page, split into exact fp16 parts (0 past the context)
    {
      const uint16_t* vs = reinterpret_cast<const uint16_t*>(vpl + kHeadDim * code_row_bytes(VK));
      if (VK == kQ4) {
        const int blk = lane >> 3, t0 = (lane & 7) * 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u4 raw = *reinterpret_cast<const u4*>(vs + blk * kPageTokens + t0 + 8 * c);
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int tt = t0 + 8 * c + 4 * half;  // first token of this 4-token run
            h8 parts;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const uint32_t word = raw[2 * half + (u >> 1)];
              uint16_t bits = (uint16_t)((u & 1) ? (word >> 16) : (word & 0xFFFFu));
              if (tt + u >= valid) bits = 0;
              const _Float16 d = __builtin_bit_cast(_Float16, bits);
              const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFF8u));
              parts[u] = dh;
              parts[4 + u] = d - dh;
            }
            *reinterpret_cast<h8*>(&wl.dsplit[dsplit_q4(blk, tt >> 2)]) = parts;
          }
        }
      } else {
        const int grp4 = lane >> 4, t0 = (lane & 15) * 16;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u4 raw = *reinterpret_cast<const u4*>(vs + grp4 * kPageTokens + t0 + 8 * c);
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int tt = t0 + 8 * c + 4 * half;
            _Float16 parts[12];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const uint32_t word = raw[2 * half + (u >> 1)];
              uint16_t bits = (uint16_t)((u & 1) ? (word >> 16) : (word & 0xFFFFu));
              if (tt + u >= valid) bits = 0;
              const _Float16 d = __builtin_bit_cast(_Float16, bits);
              const _Float16 da = __builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFF80u));
              const _Float16 db8 = __builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFF8u));
              parts[u] = da;
              parts[4 + u] = db8 - da;
              parts[8 + u] = d - db8;
            }
            _Float16* dst = &wl.dsplit[dsplit_i8(grp4, tt >> 2)];
            *reinterpret_cast<h8*>(dst) = (h8){parts[0], parts[1], parts[2], parts[3],
                                               parts[4], parts[5], parts[6], parts[7]};
            *reinterpret_cast<h4*>(dst + 8) = (h4){parts[8], parts[9], parts[10], parts[11]};
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---------------- A operands of P.V (rows 2*head + part, k-slots = 8 tokens), built once
    // per page and parked in LDS over the consumed scores: afrag[i][lane]
    {
      u4 frag[8];
      const int shift = 16 * a_part;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u4 w0, w1;
        if (VK == kQ4) {
          const int t_lo = 32 * (2 * grp + (i >> 2)) + 4 * (i & 3);
          w0 = *reinterpret_cast<const u4*>(&wl.sp[a_head][t_lo]);
          w1 = *reinterpret_cast<const u4*>(&wl.sp[a_head][t_lo + 16]);
        } else {
          w0 = *reinterpret_cast<const u4*>(&wl.sp[a_head][64 * grp + 8 * i]);
          w1 = *reinterpret_cast<const u4*>(&wl.sp[a_head][64 * grp + 8 * i + 4]);
        }
        const u4 packed = (u4){pick_part(w0[0], w0[1], shift), pick_part(w0[2], w0[3], shift),
                               pick_part(w1[0], w1[1], shift), pick_part(w1[2], w1[3], shift)};
        frag[i] = a_head < G ? packed : (u4){0, 0, 0, 0};
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      u4* af = reinterpret_cast<u4*>(&wl.sp[0][0]);
#pragma unroll
      for (int i = 0; i < 8; ++i) af[i * 64 + lane] = frag[i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    const u4* afrag = reinterpret_cast<const u4*>(&wl.sp[0][0]);

    // ---------------- P.V
    if (VK == kQ4) {
      // lane column = head element 16*(2*blk + t) + col; its 32 code bytes hold 64 tokens
      u4 vc[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u4* src = reinterpret_cast<const u4*>(vpl + (size_t)(16 * t + col) * 128 + 32 * grp);
        vc[t][0] = src[0];
        vc[t][1] = src[1];
      }
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        u4 vn[2][2];
        const int nb = blk < 7 ? blk + 1 : 7;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u4* src = reinterpret_cast<const u4*>(vpl + (size_t)(16 * (2 * nb + t) + col) * 128 + 32 * grp);
          vn[t][0] = src[0];
          vn[t][1] = src[1];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int run = (32 * (2 * grp + (i >> 2)) + 4 * (i & 3)) >> 2;
          const h8 r0 = *reinterpret_cast<const h8*>(&wl.dsplit[dsplit_q4(blk, run)]);      // hi x4, lo x4
          const h8 r1 = *reinterpret_cast<const h8*>(&wl.dsplit[dsplit_q4(blk, run + 4)]);  // +16 tokens
          const h8 d1 = (h8){r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
          const h8 d2 = (h8){r0[4], r0[5], r0[6], r0[7], r1[4], r1[5], r1[6], r1[7]};
          const h8 pa = __builtin_bit_cast(h8, afrag[i * 64 + lane]);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const h8 c = unpack_q4(vc[t][i >> 2][i & 3]);
            oacc[2 * blk + t] = mfma(pa, c * d1, oacc[2 * blk + t]);
            oacc[2 * blk + t] = mfma(pa, c * d2, oacc[2 * blk + t]);
          }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          vc[t][0] = vn[t][0];
          vc[t][1] = vn[t][1];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      u4 vc[4];
      {
        const u4* src = reinterpret_cast<const u4*>(vpl + (size_t)col * 256 + 64 * grp);
        vc[0] = src[0]; vc[1] = src[1]; vc[2] = src[2]; vc[3] = src[3];
      }
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) {
        const int gg = nt >> 2;
        const int nn = nt < 15 ? nt + 1 : 15;
        u4 vn[4];
        {
          const u4* src = reinterpret_cast<const u4*>(vpl + (size_t)(16 * nn + col) * 256 + 64 * grp);
          vn[0] = src[0]; vn[1] = src[1]; vn[2] = src[2]; vn[3] = src[3];
        }
        const uint32_t w[16] = {vc[0][0], vc[0][1], vc[0][2], vc[0][3], vc[1][0], vc[1][1], vc[1][2], vc[1][3],
                                vc[2][0], vc[2][1], vc[2][2], vc[2][3], vc[3][0], vc[3][1], vc[3][2], vc[3][3]};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int run = (64 * grp + 8 * i) >> 2;
          const _Float16* r0 = &wl.dsplit[dsplit_i8(gg, run)];
          const _Float16* r1 = &wl.dsplit[dsplit_i8(gg, run + 1)];
          const h8 a0 = *reinterpret_cast<const h8*>(r0);
          const h4 a1 = *reinterpret_cast<const h4*>(r0 + 8);
          const h8 b0 = *reinterpret_cast<const h8*>(r1);
          const h4 b1 = *reinterpret_cast<const h4*>(r1 + 8);
          const h8 da = (h8){a0[0], a0[1], a0[2], a0[3], b0[0], b0[1], b0[2], b0[3]};
          const h8 db = (h8){a0[4], a0[5], a0[6], a0[7], b0[4], b0[5], b0[6], b0[7]};
          const h8 dc = (h8){a1[0], a1[1], a1[2], a1[3], b1[0], b1[1], b1[2], b1[3]};
          const h8 c = unpack_i8(w[2 * i], w[2 * i + 1]);
          const h8 pa = __builtin_bit_cast(h8, afrag[i * 64 + lane]);
          oacc[nt] = mfma(pa, c * da, oacc[nt]);
          oacc[nt] = mfma(pa, c * db, oacc[nt]);
          oacc[nt] = mfma(pa, c * dc, oacc[nt]);
        }
        vc[0] = vn[0]; vc[1] = vn[1]; vc[2] = vn[2]; vc[3] = vn[3];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---------------- merge the four waves and write this split's partials
  __syncthreads();
  MergeLds& ml = *reinterpret_cast<MergeLds*>(lds_raw);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int hh = 2 * grp + r;
    const float lsum = half_sum(l_run[r]);
    if (col == 0) {
      ml.m[wave][hh] = m_run[r];
      ml.l[wave][hh] = lsum;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) ml.o[wave][hh][16 * t + col] = oacc[t][2 * r] + oacc[t][2 * r + 1];
  }
  __syncthreads();
  const size_t S = (size_t)n_splits;
  for (int hh = 0; hh < G; ++hh) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml.m[w][hh]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = ml.m[w][hh];
      const float wt = mw == -INFINITY ? 0.f : exp2f(mw - M);
      L += wt * ml.l[w][hh];
      O += wt * ml.o[w][hh][tid];
    }
    const size_t idx = ((size_t)b * n_q_heads + g * G + hh) * S + split;
    part_o[idx * kHeadDim + tid] = O * kPScaleInv;
    if (tid == 0) {
      part_ml[2 * idx] = M;
      part_ml[2 * idx + 1] = L;
    }
  }
}

template <bool ROTATE>
__global__ __launch_bounds__(256) void decode_combine(
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    const int32_t* __restrict__ context_lens, int max_context, int n_q_heads,
    int pages_per_split, int n_splits, float* __restrict__ out) {
  __shared__ float buf[kHeadDim];
  const int tid = threadIdx.x, h = blockIdx.x, b = blockIdx.y;
  int T = context_lens[b];
  T = T < 0 ? 0 : (T > max_context ? max_context : T);
  const int n_pages = (T + kPageTokens - 1) / kPageTokens;
  const int ns = (n_pages + pages_per_split - 1) / pages_per_split;
  const size_t base = ((size_t)b * n_q_heads + h) * (size_t)n_splits;
  float o = 0.f;
  if (ns > 0) {
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[2 * (base + s)]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = part_ml[2 * (base + s)];
      const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
      L += w * part_ml[2 * (base + s) + 1];
      acc += w * part_o[(base + s) * kHeadDim + tid];
    }
    o = L > 0.f ? acc / L : 0.f;  // L == 0 only if every page of the sequence was skipped
  }
  if (ROTATE) {
    buf[tid] = o;
    __syncthreads();
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const int m = 1 << bit;
      const float mine = buf[tid], other = buf[tid ^ m];
      __syncthreads();
      buf[tid] = (tid & m) ? (other - mine) : (mine + other);
      __syncthreads();
    }
    o = buf[tid] * 0.0625f;
  }
  out[((size_t)b * n_q_heads + h) * kHeadDim + tid] = o;
}

template <int KK, int VK>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.n_splits, (unsigned)a.n_kv_heads, (unsigned)a.batch), block(256);
  hipLaunchKernelGGL((decode_split<KK, VK>), grid, block, 0, stream, a.q, a.pool, a.n_pool_pages,
                     a.block_tables, a.max_pages, a.context_lens, a.max_context, a.n_q_heads,
                     a.n_kv_heads, a.pages_per_split, a.n_splits, a.scale_log2, a.part_ml,
                     a.part_o, a.status);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  hipError_t e;
  switch (a.fmt) {
    case KV_FMT_INT8: e = launch_split<kInt8, kInt8>(a, stream); break;
    case KV_FMT_Q4_0: e = launch_split<kQ4, kQ4>(a, stream); break;
    default: e = launch_split<kInt8, kQ4>(a, stream); break;
  }
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)a.n_q_heads, (unsigned)a.batch), block(256);
  if (a.fmt == KV_FMT_INT8)
    hipLaunchKernelGGL((decode_combine<false>), grid, block, 0, stream, a.part_ml, a.part_o,
                       a.context_lens, a.max_context, a.n_q_heads, a.pages_per_split, a.n_splits,
                       a.out);
  else
    hipLaunchKernelGGL((decode_combine<true>), grid, block, 0, stream, a.part_ml, a.part_o,
                       a.context_lens, a.max_context, a.n_q_heads, a.pages_per_split, a.n_splits,
                       a.out);
  return hipGetLastError();
}

}  // namespace kvc
