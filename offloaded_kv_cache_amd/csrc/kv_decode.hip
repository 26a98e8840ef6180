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
// Kernel 1 (decode_split): one workgroup of NW wavefronts per work item
// (split, KV head, sequence); NW = 4 for q4 K (two workgroups per CU), 8 for
// int8 K (one per CU, half the registers per wave for the larger K tiles). A
// split is `pages_per_split` consecutive logical pages, processed one 256-token
// page at a time by the whole workgroup: wave w computes the scores of tokens
// (256/NW)w.. and the outputs of head elements (256/NW)w... Each wave holds its
// share of the next page in registers while it works on the current one, so
// HBM latency is hidden behind the math. Pages are read through a buffer
// resource with loop-invariant 32-bit lane offsets. The grid is at most one
// round of resident workgroups; items beyond it are taken from a counter in
// the workspace, so a batch of mixed lengths keeps every CU busy.
//
//   Q.K on MFMA 16x16x32 f16. A = the query of the group's heads (rotated by H
//   for q4 K), each head as two fp16 rows (hi, lo) carrying ~22 bits. B = 16
//   tokens x 32 elements of raw codes taken as fp16 subnormals: a 4-bit code c
//   sits in the low bits of a half and is worth c * 2^-24 (a nibble at bits
//   4..7 is worth 16c * 2^-24, so its A slot holds q/16); int8 codes are
//   offset to c + 128 and placed the same way. One MFMA is one 32-element
//   block, scaled afterwards by that block's (q4) or group's (int8) fp16 scale.
//   The offsets (8 for q4, 128 for int8) are removed with one more MFMA per
//   tile that forms sum_j d_j * Q_j, Q_j the block sums of the query.
//
//   Online softmax in the log2 domain with a workgroup-wide maximum per page
//   (wave maxima exchanged through LDS). Probabilities are scaled by 2^14,
//   split into fp16 hi/lo and written straight into the A-fragment layout of
//   the P.V MFMA.
//
//   P.V on MFMA 16x16x32 f16, contraction over tokens. The V plane is
//   element-major, so a lane's 8 k-slots are 8 tokens of one element (two
//   4-token runs of q4 nibbles, or 8 int8 bytes). The per-token scale d varies
//   along the contraction, so it is folded into B exactly: d is split into
//   parts with few enough bits that every code x part product is exact in
//   fp16, and each part is applied with one packed fp16 fma on a "1024 + code"
//   half (q4: B = (1024 + 16c) * (p/16) - 72p = (c - 8) p, parts of <= 7 and
//   4 bits; int8: B = (1024 + c + 128) * p - 1152p = c p, three parts of <= 4
//   bits). One MFMA per part. A page with a scale outside the range where these
//   constants are exact (q4: |d| >= 896, or 0 < |d| < 2^-10 where p/16 would
//   lose bits; int8: |d| >= 56) takes a slower path that forms (c - 8) or c
//   exactly and multiplies it by the parts (exact while |8 d| stays below the
//   fp16 maximum, i.e. rotated V elements below about 2^16 / 8 in magnitude).
//
//   The waves then share the page maximum and sum; each writes its elements of
//   the split's partial (max, sum, unnormalised output). With rotated V the
//   partial is rotated back by H first (H is linear, so merging rotated-back
//   partials equals rotating the merged output back).
//
// Kernel 2 (decode_combine): per (query head, sequence, 32-element chunk), the
// log-sum-exp merge of the partials.
//
// Tokens past the context length are masked (score -inf, scale 0), so stale
// or uninitialised rows of a partly filled page never contribute. Nothing
// depends on the physical page ids except the addresses read.
#include <hip/hip_ext.h>

#include "kv_encode.h"
#include "kv_lanes.h"

namespace kvc {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr float kPScale = 16384.0f;  // probabilities are kept as p * 2^14 in fp16 hi/lo
constexpr float kPScaleInv = 1.0f / 16384.0f;
constexpr float kTwo24 = 16777216.0f;
constexpr uint32_t kQ4FastBits = 0x6300;  // fp16 896: |d| below this, -72 * d_hi is exact and finite
constexpr uint32_t kQ4FastMinM1 = 0x13FF;  // fp16 2^-10 minus one: |d| from here up, d_lo / 16 is exact
constexpr uint32_t kI8FastBits = 0x5300;  // fp16 56: |d| below this, -1152 * d_part is exact and finite
constexpr int kQsStride = kHeadDim + 4;  // padded rows of the query in LDS (bank spread)

__device__ inline f4 mfma(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Page loads go through a buffer resource of the page's KV-head planes (uniform
// base, 32-bit per-lane offsets), so every load is "scalar base + vector offset +
// immediate" and no 64-bit lane address is kept; reads past the planes return 0.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw, untyped 32-bit-element buffer access
__device__ inline Rsrc page_rsrc(const uint8_t* head, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(head), (short)0, bytes, kRsrcWord3);
}
__device__ inline u4 ld16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline u2 ld8(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ inline uint32_t ld2(Rsrc r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// A value kept in a VGPR, opaque to constant folding, so that (x & m) | v
// becomes one v_and_or_b32 inside the hot loops.
__device__ inline uint32_t vgpr_const(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
  return r;
}

// Largest |d| of eight fp16 scales, as the bit pattern of |d| (NaN patterns compare
// above every finite value).
__device__ inline uint32_t max_abs_bits(u4 w) {
  typedef uint16_t us2 __attribute__((ext_vector_type(2)));
  const us2 a = __builtin_elementwise_max(__builtin_bit_cast(us2, w[0] & 0x7FFF7FFFu), __builtin_bit_cast(us2, w[1] & 0x7FFF7FFFu));
  const us2 b = __builtin_elementwise_max(__builtin_bit_cast(us2, w[2] & 0x7FFF7FFFu), __builtin_bit_cast(us2, w[3] & 0x7FFF7FFFu));
  const us2 m = __builtin_elementwise_max(a, b);
  return m[0] > m[1] ? m[0] : m[1];
}

// Smallest (|d| bits - 1) of eight fp16 scales, with 0 wrapping to 0xFFFF (so a zero
// scale never counts as small).
__device__ inline uint32_t min_abs_bits_m1(u4 w) {
  typedef uint16_t us2 __attribute__((ext_vector_type(2)));
  const us2 one = {1, 1};
  const us2 a = __builtin_elementwise_min(__builtin_bit_cast(us2, w[0] & 0x7FFF7FFFu) - one, __builtin_bit_cast(us2, w[1] & 0x7FFF7FFFu) - one);
  const us2 b = __builtin_elementwise_min(__builtin_bit_cast(us2, w[2] & 0x7FFF7FFFu) - one, __builtin_bit_cast(us2, w[3] & 0x7FFF7FFFu) - one);
  const us2 m = __builtin_elementwise_min(a, b);
  return m[0] < m[1] ? m[0] : m[1];
}

__device__ inline float half_max(float v, int lane) {  // max over the 16 lanes of a lane group
  v = fmaxf(v, xchgf<1>(v, lane));
  v = fmaxf(v, xchgf<2>(v, lane));
  v = fmaxf(v, xchgf<4>(v, lane));
  v = fmaxf(v, xchgf<8>(v, lane));
  return v;
}
__device__ inline float half_sum(float v, int lane) {
  v += xchgf<1>(v, lane);
  v += xchgf<2>(v, lane);
  v += xchgf<4>(v, lane);
  v += xchgf<8>(v, lane);
  return v;
}

// One butterfly stage (bit log2 M) of the Walsh-Hadamard transform on N values per lane:
// partner + v in the lower lane of a pair, partner - v in the upper one, each as one fma
// with a sign of +-1 (the same rounding as the add or subtract).
template <int M, int N>
__device__ inline void butterfly(float (&v)[N], int lane) {
  const float sg = (lane & M) ? -1.0f : 1.0f;
  float o[N];
#pragma unroll
  for (int i = 0; i < N; ++i) o[i] = xchgf<M>(v[i], lane);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaf(sg, v[i], o[i]);
}

// ---- Q.K operands --------------------------------------------------------

// Eight 4-bit codes of one dword (bytes w = 0..3, low nibble = element 4s+w,
// high nibble = element 16+4s+w of a block) as fp16 subnormals; slot order
// [lo0, lo2, hi0, hi2, lo1, lo3, hi1, hi3], high nibbles worth 16c.
__device__ inline h8 k_codes_q4(uint32_t x) {
  const uint32_t y = x >> 8;
  return __builtin_bit_cast(h8, (u4){x & 0x000F000Fu, x & 0x00F000F0u, y & 0x000F000Fu, y & 0x00F000F0u});
}
// Eight int8 codes (x0 bytes 0..3, x1 bytes 4..7) as fp16 subnormals of c + 128, in order.
__device__ inline h8 k_codes_i8(uint32_t x0, uint32_t x1) {
  const uint32_t u0 = x0 ^ 0x80808080u, u1 = x1 ^ 0x80808080u;
  return __builtin_bit_cast(h8, (u4){__builtin_amdgcn_perm(0u, u0, 0x0c010c00u), __builtin_amdgcn_perm(0u, u0, 0x0c030c02u),
                                     __builtin_amdgcn_perm(0u, u1, 0x0c010c00u), __builtin_amdgcn_perm(0u, u1, 0x0c030c02u)});
}

// One 16-token tile of a K plane, as loaded by one lane (token = its column).
struct KTile {
  u4 c0, c1, c2, c3;  // code bytes of the lane's slice (q4: c0, c1; int8: all four)
  u4 d;               // the token's scales (q4: 8 fp16; int8: 4 fp16 in d.xy, d.zw = 0;
                      // fp8: fp16 0 of d.x = the K scale, fp16 1 = the same token's V scale)
};

// Byte offsets (from the head's K plane) of the lane's part of K tile t (loop
// invariant): codes of token row 64w + 16t + col, slice grp; the token's scales.
// A wave owns tpw = 256 / (waves per workgroup) tokens of a page for Q.K.
template <int KK>
__device__ inline uint32_t ktile_code_off(int tpw, int wave, int t, int col, int grp) {
  return (uint32_t)((tpw * wave + 16 * t + col) * code_row_bytes(KK) + (four_bit(KK) ? 32 : 64) * grp);
}
template <int KK>
__device__ inline uint32_t ktile_scale_off(int tpw, int wave, int t, int col) {
  return (uint32_t)(kPageTokens * code_row_bytes(KK) + (tpw * wave + 16 * t + col) * n_scales(KK) * 2);
}

template <int KK>
__device__ inline KTile load_ktile(Rsrc r, uint32_t coff, uint32_t soff) {
  KTile t;
  t.c0 = ld16(r, coff);
  t.c1 = ld16(r, coff + 16);
  if (four_bit(KK)) {
    t.c2 = t.c3 = (u4){0, 0, 0, 0};
    t.d = ld16(r, soff);
  } else if (KK == kFp8) {
    t.c2 = ld16(r, coff + 32);
    t.c3 = ld16(r, coff + 48);
    // the V plane's scale row sits plane_bytes(kFp8) after the K plane's scale rows
    t.d = (u4){ld2(r, soff) | (ld2(r, soff + plane_bytes(kFp8)) << 16), 0u, 0u, 0u};
  } else {
    t.c2 = ld16(r, coff + 32);
    t.c3 = ld16(r, coff + 48);
    const u2 dd = ld8(r, soff);
    t.d = (u4){dd[0], dd[1], 0, 0};
  }
  return t;
}

__device__ inline float scale_at(u4 d, int j) {  // fp16 scale j of a packed row of scales
  const uint32_t w = d[j >> 1];
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((j & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

// Eight fp4 codes of one dword (byte w: low nibble = slot 2w, high nibble = slot
// 2w + 1) as fp16 values times the power of two of `scale` (the conversion uses its
// exponent), exact for the values of an fp4 record.
__device__ inline h8 fp4_vals(uint32_t x, float scale) {
  const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, scale, 0);
  const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, scale, 1);
  const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, scale, 2);
  const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, scale, 3);
  return (h8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
// Eight E4M3 codes (x0 bytes 0..3, x1 bytes 4..7) as their fp16 values, in order (the
// conversion at scale 1 is exact: every E4M3 value is an fp16 number).
__device__ inline h8 fp8_vals(uint32_t x0, uint32_t x1) {
  const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x0, 1.0f, false);
  const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x0, 1.0f, true);
  const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x1, 1.0f, false);
  const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x1, 1.0f, true);
  return (h8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Scores of one tile for the lane's two heads (rows 4grp..4grp+3 = head 2grp
// hi, lo, head 2grp+1 hi, lo), in units of q.k (before the softmax scale).
template <int KK>
__device__ inline void qk_tile(const KTile& t, const h8 (&qa)[8], h8 qc, float& s0, float& s1) {
  if constexpr (KK == kFp4) {
    // block j: the lane's eight elements (32j + 4grp + w and 32j + 16 + 4grp + w) as the
    // exact fp16 values of the record (scaled conversion by the block's 2^e); no scaling
    // or offset is left, so all eight blocks accumulate in one MFMA chain
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint32_t w[8] = {t.c0[0], t.c0[1], t.c0[2], t.c0[3], t.c1[0], t.c1[1], t.c1[2], t.c1[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = mfma(qa[j], fp4_vals(w[j], scale_at(t.d, j)), acc);
    s0 = acc[0] + acc[1];
    s1 = acc[2] + acc[3];
    return;
  }
  if constexpr (KK == kFp8) {
    // the codes' exact fp16 values in one MFMA chain over the 256 elements (int8's slot
    // order), then the token's one scale
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint32_t w[16] = {t.c0[0], t.c0[1], t.c0[2], t.c0[3], t.c1[0], t.c1[1], t.c1[2], t.c1[3],
                            t.c2[0], t.c2[1], t.c2[2], t.c2[3], t.c3[0], t.c3[1], t.c3[2], t.c3[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = mfma(qa[j], fp8_vals(w[2 * j], w[2 * j + 1]), acc);
    const float d = scale_at(t.d, 0);
    s0 = d * (acc[0] + acc[1]);
    s1 = d * (acc[2] + acc[3]);
    return;
  }
  float a0 = 0.f, b0 = 0.f, a1 = 0.f, b1 = 0.f;  // hi and lo rows, units of 2^-24
  if (KK == kQ4) {
    const uint32_t w[8] = {t.c0[0], t.c0[1], t.c0[2], t.c0[3], t.c1[0], t.c1[1], t.c1[2], t.c1[3]};
    // software-pipelined: block j's scaling runs while block j + 1's MFMA is in flight
    f4 cur = mfma(qa[0], k_codes_q4(w[0]), (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f4 nxt;
      if (j < 7) nxt = mfma(qa[j + 1], k_codes_q4(w[j + 1]), (f4){0.f, 0.f, 0.f, 0.f});
      const float d = scale_at(t.d, j);
      a0 = fmaf(d, cur[0], a0);
      b0 = fmaf(d, cur[1], b0);
      a1 = fmaf(d, cur[2], a1);
      b1 = fmaf(d, cur[3], b1);
      if (j < 7) cur = nxt;
    }
  } else {
    const uint32_t w[16] = {t.c0[0], t.c0[1], t.c0[2], t.c0[3], t.c1[0], t.c1[1], t.c1[2], t.c1[3],
                            t.c2[0], t.c2[1], t.c2[2], t.c2[3], t.c3[0], t.c3[1], t.c3[2], t.c3[3]};
    // two chained MFMAs per 64-element group; a group is scaled while the next group's
    // MFMAs are in flight
    f4 cur = mfma(qa[0], k_codes_i8(w[0], w[1]), (f4){0.f, 0.f, 0.f, 0.f});
    cur = mfma(qa[1], k_codes_i8(w[2], w[3]), cur);
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      f4 nxt;
      if (gg < 3) {
        nxt = mfma(qa[2 * gg + 2], k_codes_i8(w[4 * gg + 4], w[4 * gg + 5]), (f4){0.f, 0.f, 0.f, 0.f});
        nxt = mfma(qa[2 * gg + 3], k_codes_i8(w[4 * gg + 6], w[4 * gg + 7]), nxt);
      }
      const float d = scale_at(t.d, gg);
      a0 = fmaf(d, cur[0], a0);
      b0 = fmaf(d, cur[1], b0);
      a1 = fmaf(d, cur[2], a1);
      b1 = fmaf(d, cur[3], b1);
      if (gg < 3) cur = nxt;
    }
  }
  // sum_j d_j * Q_j per head (hi, lo rows), for the code offsets
  const f4 corr = mfma(qc, __builtin_bit_cast(h8, t.d), (f4){0.f, 0.f, 0.f, 0.f});
  const float off = KK == kQ4 ? 8.0f : 128.0f;
  s0 = fmaf(a0 + b0, kTwo24, -off * (corr[0] + corr[1]));
  s1 = fmaf(a1 + b1, kTwo24, -off * (corr[2] + corr[3]));
}

// ---- V share and P.V operands ---------------------------------------------

// The wave's share of a page's V plane: head elements 64w..64w+63 (four MFMA
// column tiles), all 256 tokens, plus the scales the wave turns into B parts.
template <int VK>
struct VShare {
  u4 c[4][four_bit(VK) ? 2 : 4];  // per column tile: the lane's 32 (4-bit) / 64 (int8) code bytes
  u2 s0, s1;                   // q4: 4 + 4 token scales; int8: s0, s1 = 8 consecutive scales
};

// Byte offset (from the head's K plane) of column tile nt of the wave's V share:
// the lane's 32 (q4) / 64 (int8) code bytes of head element epw * w + 16nt + col
// (a wave owns epw = 256 / (waves per workgroup) head elements for P.V).
template <int KK, int VK>
__device__ inline uint32_t vcode_off(int epw, int wave, int lane, int nt) {
  const int grp = lane >> 4, col = lane & 15;
  return (uint32_t)(plane_bytes(KK) + (epw * wave + 16 * nt + col) * code_row_bytes(VK) + (four_bit(VK) ? 32 : 64) * grp);
}
template <int VK>
__device__ inline void load_vcodes(VShare<VK>& v, Rsrc r, uint32_t off, int nt) {
#pragma unroll
  for (int u = 0; u < (four_bit(VK) ? 2 : 4); ++u) v.c[nt][u] = ld16(r, off + 16 * u);
}

// Byte offset (from the head's K plane) of the scales the lane turns into B parts.
template <int KK, int VK>
__device__ inline uint32_t vscale_off(int epw, int wave, int lane) {
  const uint32_t vs = plane_bytes(KK) + kHeadDim * code_row_bytes(VK);  // V scales
  if (four_bit(VK)) {
    // B-part entry (block of the wave bb, MFMA i, lane group gq): tokens t_lo..+3 and
    // t_lo+16..+19; lanes past the wave's blocks read its first block again
    const int nb = epw / 32, bb = (lane >> 5) < nb ? (lane >> 5) : 0, i = (lane >> 2) & 7, gq = lane & 3;
    const int t_lo = 32 * (2 * gq + (i >> 2)) + 4 * (i & 3);
    return vs + (uint32_t)(((nb * wave + bb) * kPageTokens + t_lo) * 2);
  } else {
    // entry (MFMA i, lane group gq) = tokens 64gq + 8i .. +7 of the wave's 64-element group
    const int i = (lane >> 2) & 7, gq = lane & 3;
    return vs + (uint32_t)(((epw * wave / 64) * kPageTokens + 64 * gq + 8 * i) * 2);
  }
}
template <int VK>
__device__ inline void load_vscales(VShare<VK>& v, Rsrc r, uint32_t off) {
  if (VK == kFp8) {
    // (fp8: the token's V scale comes with its K tile and is applied on the P side)
    v.s0 = v.s1 = (u2){0u, 0u};
  } else if (four_bit(VK)) {
    v.s0 = ld8(r, off);
    v.s1 = ld8(r, off + 32);
  } else {
    const u4 d = ld16(r, off);
    v.s0 = (u2){d[0], d[1]};
    v.s1 = (u2){d[2], d[3]};
  }
}

// Eight q4 codes of one dword (byte w: low nibble token t+w, high nibble token
// t+16+w) as halves "1024 + 16c", slot order [t..t+3, t+16..t+19].
__device__ inline u4 v_magic_q4(uint32_t x, uint32_t vmask, uint32_t vmagic) {
  const uint32_t t01 = __builtin_amdgcn_perm(0u, x, 0x0c010c00u);  // (b0, b1)
  const uint32_t t23 = __builtin_amdgcn_perm(0u, x, 0x0c030c02u);  // (b2, b3)
  return (u4){((t01 << 4) & vmask) | vmagic, ((t23 << 4) & vmask) | vmagic,
              (t01 & vmask) | vmagic, (t23 & vmask) | vmagic};
}
// Eight int8 codes as halves "1024 + c + 128", in order.
__device__ inline u4 v_magic_i8(uint32_t x0, uint32_t x1, uint32_t vmagic) {
  const uint32_t u0 = x0 ^ 0x80808080u, u1 = x1 ^ 0x80808080u;
  // selector byte 5 = byte 1 of vmagic = 0x64, the high byte of each half
  return (u4){__builtin_amdgcn_perm(vmagic, u0, 0x05010500u), __builtin_amdgcn_perm(vmagic, u0, 0x05030502u),
              __builtin_amdgcn_perm(vmagic, u1, 0x05010500u), __builtin_amdgcn_perm(vmagic, u1, 0x05030502u)};
}
__device__ inline h8 pk_fma8(u4 x, h8 m, h8 a) {
  return __builtin_elementwise_fma(__builtin_bit_cast(h8, x), m, a);
}

// LDS of a workgroup.
//   afrag:  the page's probabilities in P.V A-fragment layout, [MFMA i][lane] x 8 fp16
//   dpart:  per wave, the B parts of its V scales, part-major so that lanes write and read
//           consecutive 16 B: q4 [4 parts][block 2][i 8][lane group 4], int8 [6 parts][i 8]
//           [lane group 4], each an h8 in B slot order
//   wmax:   each wave's maximum score per head;  lsum: each wave's probability sums
template <int NW>
struct SplitLds {
  h8 afrag[8][64];
  h8 dpart[NW][256];
  float wmax[NW][kMaxGroup];
  float lsum[NW][kMaxGroup];
  float qs[kMaxGroup][kQsStride];
  float bsum[kMaxGroup][8];
  float wdmax[NW];  // fp8: each wave's largest V scale of the page
};

__device__ inline int32_t bt_row_entry(const int32_t* __restrict__ block_tables, int b, int max_pages, int pg) {
  return block_tables[(size_t)b * max_pages + pg];
}

// NW waves per workgroup (4: two workgroups per CU; 8: one, with half the per-wave
// registers, for the larger int8 K tiles). DYN: more work items than workgroups (taken
// from a counter); otherwise workgroup i does item i only. APPEND: the call also
// appends one token per sequence (k_new, v_new [batch][n_kv_heads][256] fp16, at
// position context_lens[b] - 1), written through pool_w (the pool's address).
// Rows b of q (batch of them) are n_q queries per sequence: row b is query
// j = b % n_q of sequence b / n_q, whose context length T gives it the first
// T - n_q + j + 1 tokens (causal attention of the sequence's n_q newest tokens).
template <int KK, int VK, int NW, bool DYN, bool APPEND>
// (The counter-fed q4 form is bounded for one workgroup per CU: bounded for two, it needs
// more than the 256 registers a wave then gets and spills to scratch memory; bounded for
// one, it keeps its values in VGPRs and AGPRs and, although only one of its workgroups
// then fits on a CU, measured 5-9% faster. Its grid is unchanged: workgroups past the
// resident ones start as others finish and take items from the same counter.)
__global__ __launch_bounds__(64 * NW, (NW == 4 && !(DYN && KK == kQ4)) ? 2 : 1) void decode_split(
    const uint16_t* __restrict__ q, const uint8_t* pool, int64_t n_pool_pages,
    const int32_t* __restrict__ block_tables, int max_pages, const int32_t* __restrict__ context_lens,
    int max_context, int n_q_heads, int n_kv_heads, int pages_per_split, int n_splits,
    float scale_log2, float* __restrict__ part_ml, float* __restrict__ part_o,
    int32_t* __restrict__ status, uint32_t* __restrict__ sched, int batch, int n_q,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, uint8_t* pool_w, int n_cus) {
  __shared__ __attribute__((aligned(16))) SplitLds<NW> lds;
  __shared__ int item_s;
  constexpr int TPW = kPageTokens / NW, KT = TPW / 16;  // Q.K: tokens and tiles per wave
  constexpr int EPW = kHeadDim / NW, NTW = EPW / 16;    // P.V: elements and column tiles per wave
  constexpr int HFN = NTW / 2;                           // P.V halves of two column tiles
  constexpr int kHPW = kMaxGroup / NW;                   // query head slots per wave (prologue)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;  // MFMA lane group and column
  const int G = n_q_heads / n_kv_heads;
  const int n_pairs = n_kv_heads * batch, n_items = n_splits * n_pairs;

  // Work items (split, sequence, KV head), split-major. Workgroup i takes item i; when
  // there are more items than workgroups (one round of resident workgroups), the rest
  // are taken from a counter in the workspace, so that the workgroups on every CU share
  // the items that have pages whatever the sequences' lengths. An item past a
  // sequence's last page is skipped.
  int item = blockIdx.x;
  for (bool first = true;; first = false) {
  if (!first) {
    if (!DYN) break;
    if (tid == 0) item_s = (int)gridDim.x + (int)atomicAdd(&sched[0], 1u);
    __syncthreads();
    item = item_s;
    __syncthreads();
  }
  if (item >= n_items) break;
  int split, b, g;
  if (n_q == 1) {
    split = item / n_pairs;
    b = (item - split * n_pairs) / n_kv_heads;
    g = item % n_kv_heads;
  } else {
    // Several query rows per sequence: the n_q rows of one (split, sequence, KV head) read
    // the same pages. Workgroups go to the eight XCDs round-robin by index, each XCD with its
    // own L2, so the rows of such a group take indices eight apart (one XCD) and close
    // together (dispatched about together), and the pages they share are read from HBM once.
    // Row groups come in chunks of eight: chunk c, XCD x holds group 8c + x, its row j at
    // index 8 (n_q c + j) + x; a last partial chunk of m < 8 groups is laid out row by row.
    const int R = n_items / n_q, full = (R / 8) * 8 * n_q;
    int r, j;
    if (item < full) {
      const int sx = item / 8;
      r = (sx / n_q) * 8 + item % 8;
      j = sx % n_q;
    } else {
      const int m = R % 8, l = item - full;
      r = (R / 8) * 8 + l % m;
      j = l / m;
    }
    const int n_seq_kv = n_pairs / n_q;  // (sequence, KV head) pairs
    split = r / n_seq_kv;
    const int rem = r - split * n_seq_kv;
    g = rem % n_kv_heads;
    b = (rem / n_kv_heads) * n_q + j;
  }

  // Issued together before anything waits: the query of the group's heads (element
  // tid; unconditional loads of a clamped head), the context length and the split's
  // first block-table entry (index clamped into the table).
  // Wave w holds head slots HPW w .. HPW w + HPW - 1, lane l elements l + 64k (k = 0..3)
  // of each: element bits 0-5 are the lane, bits 6-7 the register.
  float qv[kHPW * 4];
#pragma unroll
  for (int i = 0; i < kHPW; ++i) {
    const int hh = kHPW * wave + i, hc = min(hh, G - 1);
    const uint16_t* qh = q + ((size_t)b * n_q_heads + g * G + hc) * kHeadDim + lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x = (float)__builtin_bit_cast(_Float16, qh[64 * k]);
      qv[4 * i + k] = hh < G ? x : 0.f;
    }
  }
  const int p_begin = split * pages_per_split;
  const int bs = n_q == 1 ? b : b / n_q;            // the sequence of query row b
  const int later = n_q == 1 ? 0 : n_q - 1 - (b - bs * n_q);  // queries after row b's
  const int32_t phys_first = block_tables[(size_t)bs * max_pages + min(p_begin, max_pages - 1)];
  int T = context_lens[bs];
  const bool t_in_range = T <= max_context && T >= 0;
  if (!t_in_range) {
    if (tid == 0 && split == 0 && g == 0) atomicOr(status, KV_STATUS_CONTEXT_CLAMPED);
    T = T < 0 ? 0 : max_context;
  }
  T = T > later ? T - later : 0;
  const int n_pages = (T + kPageTokens - 1) / kPageTokens;
  const int p_end = min(n_pages, p_begin + pages_per_split);
  if (p_begin >= p_end) continue;  // uniform over the workgroup

  // Two workgroups share a CU when the grid is larger than the CU count; the one
  // dispatched second (blockIdx past the CU count) would otherwise lose every issue
  // tie to the older one's waves and finish its item well after it, leaving the CU
  // half occupied at the end. Its waves take a higher issue priority for the first
  // half of its pages, so the two finish close together.
  // The appended token (APPEND, length in range): written by the item whose pages hold
  // it, before any wave of the workgroup reads its page. On the item's first page it is
  // written before the first loads; on a later page, while the first page is in flight,
  // and the workgroup synchronises once before that page's loads are issued.
  int new_pg = -1;
  if (APPEND && t_in_range && T > 0 && (T - 1) / kPageTokens >= p_begin && (T - 1) / kPageTokens < p_end)
    new_pg = (T - 1) / kPageTokens;
  const bool new_first = new_pg == p_begin;
  // its K (even waves) or V (odd waves) inputs, loaded before the pages (waves 0 and 1 use them)
  uint16_t new_in[4] = {0, 0, 0, 0};
  if (APPEND && new_pg >= 0)
    enc::load_vals((wave & 1 ? v_new : k_new) + ((size_t)b * n_kv_heads + g) * kHeadDim, lane, new_in);
  const int32_t phys_new = new_pg >= 0 ? bt_row_entry(block_tables, bs, max_pages, new_pg) : -1;
  // (the appending workgroup, which also encodes the token, keeps it one page longer)
  const int boost_until = (!DYN && NW == 4 && ((int)blockIdx.x >= n_cus || new_pg >= 0))
                              ? min(p_end, p_begin + (p_end - p_begin) / 2 + (new_pg >= 0 ? 1 : 0))
                              : p_begin;
  if (boost_until > p_begin) __builtin_amdgcn_s_setprio(1);

  const int64_t head_bytes = plane_bytes(KK) + plane_bytes(VK);
  const int64_t page_bytes = (int64_t)n_kv_heads * head_bytes;
  const int32_t* bt = block_tables + (size_t)bs * max_pages;

  // Page base of logical page pg for this KV head (nullptr for an id outside the pool).
  auto page_base = [&](int pg) -> const uint8_t* {
    const int32_t phys = bt[pg];
    if (phys < 0 || phys >= n_pool_pages) return nullptr;
    return pool + (int64_t)phys * page_bytes + (int64_t)g * head_bytes;
  };

  __builtin_amdgcn_sched_barrier(0);
  // then the first page's share: KT K tiles (tokens TPW w ..) and the V share, issued
  // after the query so that the wait for the query does not also wait for the page
  KTile kt[KT];
  VShare<VK> vsh;
  const uint8_t* base = phys_first < 0 || phys_first >= n_pool_pages
                            ? nullptr
                            : pool + (int64_t)phys_first * page_bytes + (int64_t)g * head_bytes;
  // loop-invariant lane offsets of every load of a page
  uint32_t koff[KT], ksoff[KT], voff[NTW];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    koff[t] = ktile_code_off<KK>(TPW, wave, t, col, grp);
    ksoff[t] = ktile_scale_off<KK>(TPW, wave, t, col);
  }
#pragma unroll
  for (int t = 0; t < NTW; ++t) voff[t] = vcode_off<KK, VK>(EPW, wave, lane, t);
  const uint32_t vsoff = vscale_off<KK, VK>(EPW, wave, lane);
  // a bad page id reads an empty range (zeros, no memory) and is then skipped
  const Rsrc r0 = base ? page_rsrc(base, (int)head_bytes) : page_rsrc(pool, 0);
  // the K tiles now; the V share after the query's rotation, so that the query math
  // runs while the memory pipeline drains the first burst
  if (!new_first) {
#pragma unroll
    for (int t = 0; t < KT; ++t) kt[t] = load_ktile<KK>(r0, koff[t], ksoff[t]);
  }
  // The token's records: wave 0 encodes its K vector of this KV head, wave 1 its V
  // vector, from the inputs `in` (fp16 bits of elements lane + 64k), and writes them.
  auto append_token = [&](const uint16_t (&in)[4]) {
    const int row = (T - 1) % kPageTokens;
    if (phys_new < 0 || phys_new >= n_pool_pages) {
      if (tid == 0) atomicOr(status, KV_STATUS_BAD_PAGE_ID);
    } else if (wave < 2) {
      uint8_t* head = pool_w + (int64_t)phys_new * page_bytes + (int64_t)g * head_bytes;
      int code[4];
      uint16_t scale[4];
      if (KK == VK) {
        enc::encode_vals<KK>(in, lane, code, scale);
      } else if (wave == 0) {
        enc::encode_vals<KK>(in, lane, code, scale);
      } else {
        enc::encode_vals<VK>(in, lane, code, scale);
      }
      if (wave == 0) {
        enc::write_k_row<KK>(head, row, lane, code, scale);
      } else {
        enc::write_v_scales<VK>(head + plane_bytes(KK), row, lane, scale);
        enc::write_v_codes_one<VK>(head + plane_bytes(KK), row, lane, code);
      }
    }
    // the token's bytes are complete (and visible to the workgroup) before its page is read
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
  };
  // On the item's first page the token is written before the first loads.
  if (APPEND && new_first) append_token(new_in);
  if (new_first) {
#pragma unroll
    for (int t = 0; t < KT; ++t) kt[t] = load_ktile<KK>(r0, koff[t], ksoff[t]);
  }

  // The query prepared inside each wave for its head slots: rotation by H (q4 and fp4 K),
  // block sums for the code offsets (q4, int8), and the fp16 hi + lo A fragments written
  // straight into their MFMA layout in LDS; one workgroup barrier, then every wave reads
  // all eight fragments. (All head slots are prepared; unused ones hold zeros.)
  if (four_bit(KK)) {
    // element bits 0-5: butterflies between lanes; bits 6-7: a 4-point stage in registers
    butterfly<1>(qv, lane);
    butterfly<2>(qv, lane);
    butterfly<4>(qv, lane);
    butterfly<8>(qv, lane);
    butterfly<16>(qv, lane);
    butterfly<32>(qv, lane);
#pragma unroll
    for (int i = 0; i < kHPW; ++i) {
      float* x = qv + 4 * i;
      const float s01p = fmaf(1.0f, x[1], x[0]), s01m = fmaf(-1.0f, x[1], x[0]);
      const float s23p = fmaf(1.0f, x[3], x[2]), s23m = fmaf(-1.0f, x[3], x[2]);
      x[0] = fmaf(1.0f, s23p, s01p) * 0.0625f;
      x[1] = fmaf(1.0f, s23m, s01m) * 0.0625f;
      x[2] = fmaf(-1.0f, s23p, s01p) * 0.0625f;
      x[3] = fmaf(-1.0f, s23m, s01m) * 0.0625f;
    }
  }
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) load_vcodes<VK>(vsh, r0, voff[nt], nt);
  load_vscales<VK>(vsh, r0, vsoff);
  // Block sums by lane exchange (xchgf: each value with itself; this compiler folds the
  // second result of a row or half-wave swap of two different values into the first).
  if constexpr (KK == kQ4) {
    // block j = element bits 5-7 = 2k + lane bit 5: sums over lane bits 0-4
    static_assert(NW == 4, "q4 K: two head slots per wave");
#pragma unroll
    for (int u = 0; u < kHPW * 4; ++u) {
      float sum = half_sum(qv[u], lane);
      sum += xchgf<16>(sum, lane);
      if ((lane & 31) == 0) lds.bsum[kHPW * wave + u / 4][2 * (u % 4) + (lane >> 5)] = sum;
    }
  } else if constexpr (KK == kInt8) {
    // group j = element bits 6-7 = k: sums over all 64 lanes
    static_assert(NW == 8, "int8 K: one head slot per wave");
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float sum = half_sum(qv[u], lane);
      sum += xchgf<16>(sum, lane);
      sum += xchgf<32>(sum, lane);
      if (lane == 0) lds.bsum[wave][u] = sum;
    }
  }
  // A operands of Q.K: row r = 2 head + part (hi, lo) of lane 16 gq + r, fragment j = block j
  // (elements 32j .. 32j + 31); slot order within a lane's eight halves:
  //   q4:  [e, e+2, e+16, e+18, e+1, e+3, e+17, e+19], e = 32j + 4gq, high-nibble slots hold q/16
  //   fp4: [e, e+16, e+1, e+17, e+2, e+18, e+3, e+19], e = 32j + 4gq
  //   int8, fp8: e .. e + 7, e = 32j + 8gq
  {
    _Float16* af = reinterpret_cast<_Float16*>(&lds.afrag[0][0]);
    const int o = lane & 31;
    int gq, slot;
    if (KK == kQ4) {
      const int w = o & 3;
      gq = (o & 15) >> 2;
      slot = ((w & 1) << 2) | (w >> 1) | ((o >> 4) << 1);
    } else if (KK == kFp4) {
      gq = (o & 15) >> 2;
      slot = 2 * (o & 3) + (o >> 4);
    } else {
      gq = o >> 3;
      slot = o & 7;
    }
    const float sc = (KK == kQ4 && (o & 16)) ? 0.0625f : 1.0f;
#pragma unroll
    for (int u = 0; u < kHPW * 4; u += 2) {
      // hi = the value truncated to fp16, lo = the remainder truncated: ~21 bits together
      const float f0 = qv[u] * sc, f1 = qv[u + 1] * sc;
      const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(f0, f1));
      const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(f0 - (float)hi[0], f1 - (float)hi[1]));
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int hh = kHPW * wave + (u + v) / 4, k = (u + v) % 4;
        const int j = 2 * k + (lane >> 5);
        const int at = (j * 64 + 16 * gq + 2 * hh) * 8 + slot;
        af[at] = hi[v];
        af[at + 8] = lo[v];
      }
    }
  }
  __syncthreads();

  // A operands of Q.K and of the offset correction (row 2 head + part, k-slot j of lane
  // group 0 = block sum j)
  const int a_head = col >> 1, a_part = col & 1;
  const bool a_live = a_head < G;
  h8 qa[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qa[j] = lds.afrag[j][lane];
  h8 qc;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const float f = ((KK == kInt8 || KK == kQ4) && s < (KK == kQ4 ? 8 : 4)) ? lds.bsum[a_head][s] : 0.f;
    const _Float16 hi = (_Float16)f;
    const _Float16 lo = (_Float16)(f - (float)hi);
    qc[s] = (a_live && grp == 0) ? (a_part ? lo : hi) : (_Float16)0;
  }

  const uint32_t vmask = vgpr_const(0x00F000F0u), vmagic = vgpr_const(0x64006400u);
  const int h0 = 2 * grp, h1 = 2 * grp + 1;
  // per-lane running state for the two heads of its row group (rows 4grp..4grp+3)
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  // fp8: the accumulators hold the output in units of dunit (a power of two, the
  // previous page's largest V scale rounded down), so that p * d / dunit stays in fp16 range
  float dunit = 1.f;
  f4 oacc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) oacc[t] = (f4){0.f, 0.f, 0.f, 0.f};
  // On a later page the token is written here, once the query is prepared and its inputs
  // (loaded first) have long arrived, and before the loop issues any load of its page.
  if (APPEND && new_pg > p_begin) append_token(new_in);

  for (int pg = p_begin; pg < p_end; ++pg) {
    const bool page_ok = base != nullptr;
    if (!page_ok && tid == 0) atomicOr(status, KV_STATUS_BAD_PAGE_ID);
    const int valid = page_ok ? min(kPageTokens, T - pg * kPageTokens) : 0;  // tokens in context
    const uint8_t* next = pg + 1 < p_end ? page_base(pg + 1) : nullptr;

    // Next page's loads are issued without a branch so that the wait counters before
    // each use stay exact, and each part is issued as soon as its registers are
    // consumed, to overlap the math. After the last page, and for a bad page id, they
    // are issued against an empty range: they return zeros and read no memory.
    const Rsrc nr = next ? page_rsrc(next, (int)head_bytes) : page_rsrc(pool, 0);

    // ---------------- Q.K of the wave's TPW tokens, wave maximum per head
    float xs[KT][2];
    float vd[KT];  // fp8: V scale of the lane's token of tile t (0 past the context)
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const int row = TPW * wave + 16 * t + col;
      float s0, s1;
      qk_tile<KK>(kt[t], qa, qc, s0, s1);
      const bool ok = row < valid;
      vd[t] = (VK == kFp8 && ok) ? scale_at(kt[t].d, 1) : 0.f;
      xs[t][0] = ok ? s0 * scale_log2 : -INFINITY;
      xs[t][1] = ok ? s1 * scale_log2 : -INFINITY;
      mx0 = fmaxf(mx0, xs[t][0]);
      mx1 = fmaxf(mx1, xs[t][1]);
      kt[t] = load_ktile<KK>(nr, koff[t], ksoff[t]);  // next page's tile t
      __builtin_amdgcn_sched_barrier(0);
    }
    mx0 = half_max(mx0, lane);
    mx1 = half_max(mx1, lane);
    if (col == 0) {
      lds.wmax[wave][h0] = mx0;
      lds.wmax[wave][h1] = mx1;
    }
    if constexpr (VK == kFp8) {
      float dmx = vd[0];
#pragma unroll
      for (int t = 1; t < KT; ++t) dmx = fmaxf(dmx, vd[t]);
      dmx = half_max(dmx, lane);
      if (lane == 0) lds.wdmax[wave] = dmx;
    }

    // ---------------- B parts of the wave's V scales (0 past the context)
    bool fast;
    {
      h8* dp = lds.dpart[wave];
      if constexpr (VK == kFp8) {
        fast = true;  // no B parts: the V scale goes with the probability
      } else if constexpr (VK == kFp4) {
        // the scales of the lane's entry (block bb of the wave, MFMA i, lane group gq) in
        // B slot order [t, t+16, t+1, t+17, t+2, t+18, t+3, t+19] (0 past the context);
        // the products code * 2^e are exact, so every page takes the one path
        const int bb = lane >> 5, i = (lane >> 2) & 7, gq = lane & 3;
        const int t_lo = 32 * (2 * gq + (i >> 2)) + 4 * (i & 3);
        u4 wv = {vsh.s0[0], vsh.s0[1], vsh.s1[0], vsh.s1[1]};  // tokens t..t+3, t+16..t+19
        if (bb >= EPW / 32) wv = (u4){0u, 0u, 0u, 0u};
        if (valid < kPageTokens) {
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (t_lo + (u & 3) + 16 * (u >> 2) >= valid) wv[u >> 1] &= (u & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
        const u4 sv = {__builtin_amdgcn_perm(wv[2], wv[0], 0x05040100u), __builtin_amdgcn_perm(wv[2], wv[0], 0x07060302u),
                       __builtin_amdgcn_perm(wv[3], wv[1], 0x05040100u), __builtin_amdgcn_perm(wv[3], wv[1], 0x07060302u)};
        dp[(bb * 8 + i) * 4 + gq] = __builtin_bit_cast(h8, sv);
        fast = true;
      } else if (VK == kQ4) {
        const int bb = lane >> 5, i = (lane >> 2) & 7, gq = lane & 3;
        const int t_lo = 32 * (2 * gq + (i >> 2)) + 4 * (i & 3);
        // slot u = scale of token t_lo + (u & 3) + 16 (u >> 2): half (u & 1) of word u >> 1;
        // lanes past the wave's blocks (one block per wave at 8 waves) hold zeros
        u4 wv = {vsh.s0[0], vsh.s0[1], vsh.s1[0], vsh.s1[1]};
        if (bb >= EPW / 32) wv = (u4){0u, 0u, 0u, 0u};
        if (valid < kPageTokens) {  // a partial page: scales of rows past the context are 0
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (t_lo + (u & 3) + 16 * (u >> 2) >= valid) wv[u >> 1] &= (u & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
        const h8 d = __builtin_bit_cast(h8, wv);
        const h8 dh = __builtin_bit_cast(h8, wv & 0xFFF0FFF0u);  // <= 7 significant bits
        const h8 dl = d - dh;                                    // <= 4 significant bits
        // folded constants exact and finite: every |d| in [2^-10, 896) or 0
        fast = !__any(!(max_abs_bits(wv) < kQ4FastBits && min_abs_bits_m1(wv) >= kQ4FastMinM1));
        h8* e = dp + ((bb * 8 + i) * 4 + gq);  // = dp + lane
        if (fast) {
          e[0] = dh * (_Float16)0.0625f;
          e[64] = dh * (_Float16)(-72.0f);
          e[128] = dl * (_Float16)0.0625f;
          e[192] = dl * (_Float16)(-72.0f);
        } else {  // the parts themselves, for exact (c - 8) * part products
          e[0] = dh;
          e[128] = dl;
        }
      } else {
        const int i = (lane >> 2) & 7, gq = lane & 3;
        const int t0 = 64 * gq + 8 * i;
        // slot u = scale of token t0 + u: half (u & 1) of word u >> 1
        u4 wv = {vsh.s0[0], vsh.s0[1], vsh.s1[0], vsh.s1[1]};
        if (valid < kPageTokens) {  // a partial page: scales of rows past the context are 0
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (t0 + u >= valid) wv[u >> 1] &= (u & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
        const h8 d = __builtin_bit_cast(h8, wv);
        const h8 pa_ = __builtin_bit_cast(h8, wv & 0xFF80FF80u);   // <= 4 significant bits
        const h8 db8 = __builtin_bit_cast(h8, wv & 0xFFF8FFF8u);
        const h8 pb_ = db8 - pa_;                                  // <= 4 significant bits
        const h8 pc_ = d - db8;                                    // <= 3 significant bits
        if (lane < 32) {
          h8* e = dp + (i * 4 + gq);  // = dp + lane
          e[0] = pa_;
          e[32] = pa_ * (_Float16)(-1152.0f);
          e[64] = pb_;
          e[96] = pb_ * (_Float16)(-1152.0f);
          e[128] = pc_;
          e[160] = pc_ * (_Float16)(-1152.0f);
        }
        const uint32_t amax_bits = lane < 32 ? max_abs_bits(wv) : 0u;
        fast = !__any(!(amax_bits < kI8FastBits));
      }
    }
    load_vscales<VK>(vsh, nr, vsoff);  // next page's scales
    __syncthreads();  // (A) wave maxima visible

    // ---------------- online softmax: page maximum over the four waves, p of the wave's tokens
    float pm0 = lds.wmax[0][h0], pm1 = lds.wmax[0][h1];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      pm0 = fmaxf(pm0, lds.wmax[w][h0]);
      pm1 = fmaxf(pm1, lds.wmax[w][h1]);
    }
    const float mn0 = fmaxf(m_run[0], pm0), mn1 = fmaxf(m_run[1], pm1);
    // fp8: the page's unit (largest V scale of the page rounded down to a power of two;
    // 1 without tokens in context), its inverse, and the change of unit of the accumulators
    float vinv = 1.f, vratio = 1.f;
    if constexpr (VK == kFp8) {
      float dm = lds.wdmax[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) dm = fmaxf(dm, lds.wdmax[w]);
      const uint32_t eb = dm > 0.f ? (__builtin_bit_cast(uint32_t, dm) >> 23) : 127u;  // fp16 scales: normal fp32
      const float unit = __builtin_bit_cast(float, eb << 23);
      vinv = __builtin_bit_cast(float, (254u - eb) << 23);
      vratio = dunit * vinv;
      dunit = unit;
    }
    // reference point of the exponentials: the new maximum, or 0 while no token of
    // the split is in context (then every score and the old maximum are -inf, and
    // 2^(-inf) = 0 leaves the zero state unchanged)
    const float r0 = mn0 == -INFINITY ? 0.f : mn0, r1 = mn1 == -INFINITY ? 0.f : mn1;
    const float al0 = __builtin_amdgcn_exp2f(m_run[0] - r0);
    const float al1 = __builtin_amdgcn_exp2f(m_run[1] - r1);
    m_run[0] = mn0;
    m_run[1] = mn1;
    float sum0 = 0.f, sum1 = 0.f;
    _Float16* af = reinterpret_cast<_Float16*>(&lds.afrag[0][0]);
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const float p0 = __builtin_amdgcn_exp2f(xs[t][0] - r0);  // masked tokens: 2^(-inf) = 0
      const float p1 = __builtin_amdgcn_exp2f(xs[t][1] - r1);
      sum0 += p0;
      sum1 += p1;
      // fragment position of token TPW w + 16t + col for P.V MFMA i, lane (k-group kg,
      // row 2h + part), slot: k-group kg holds tokens 64kg..64kg+63, in the order in
      // which a lane's V code bytes come (q4: 4 + 4 nibble tokens, int8: 8 bytes)
      const int token = TPW * wave + 16 * t + col, kg = token >> 6, o = token & 63;
      int i, slot;
      if (VK == kFp4) {  // byte w of a dword: low nibble token t + w, high nibble t + 16 + w
        i = 4 * (o >> 5) + ((o & 15) >> 2);
        slot = 2 * (o & 3) + ((o >> 4) & 1);
      } else if (VK == kQ4) {
        i = 4 * (o >> 5) + ((o & 15) >> 2);
        slot = 4 * ((o >> 4) & 1) + (o & 3);
      } else {
        i = o >> 3;
        slot = o & 7;
      }
      const int base_idx = (i * 64 + 16 * kg) * 8 + slot;
      // (fp8: times the token's V scale in the page's unit, in [0, 2): exact)
      const float pk = VK == kFp8 ? kPScale * (vd[t] * vinv) : kPScale;
      const float ps0 = p0 * pk, ps1 = p1 * pk;
      const _Float16 hi0 = (_Float16)ps0, hi1 = (_Float16)ps1;
      const _Float16 lo0 = (_Float16)(ps0 - (float)hi0), lo1 = (_Float16)(ps1 - (float)hi1);
      // rows of heads >= G (zero query) are written too: they only feed output rows
      // that are never stored
      af[base_idx + (2 * h0) * 8] = hi0;
      af[base_idx + (2 * h0 + 1) * 8] = lo0;
      af[base_idx + (2 * h1) * 8] = hi1;
      af[base_idx + (2 * h1 + 1) * 8] = lo1;
    }
    l_run[0] = l_run[0] * al0 + sum0;
    l_run[1] = l_run[1] * al1 + sum1;
    const float ao0 = al0 * vratio, ao1 = al1 * vratio;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      oacc[t][0] *= ao0;
      oacc[t][1] *= ao0;
      oacc[t][2] *= ao1;
      oacc[t][3] *= ao1;
    }
    __syncthreads();  // (B) probabilities of all 256 tokens visible

    // ---------------- P.V for the wave's EPW head elements, in halves of two column tiles
    // (one q4 block each); after a half, its code registers take the next page's codes.
    const h8* dp = lds.dpart[wave];
    if (VK == kFp8 && valid < kPageTokens) {
      // E4M3 has NaN codes and 0 * NaN is NaN: bytes of rows past the context (stale or
      // never written) are cleared. Byte b of word w of slice u: token 64grp + 16u + 4w + b.
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int n = valid - (64 * grp + 16 * u + 4 * w);
            vsh.c[nt][u][w] &= n >= 4 ? ~0u : (n <= 0 ? 0u : (1u << (8 * n)) - 1u);
          }
    }
#pragma unroll
    for (int hf = 0; hf < HFN; ++hf) {
      if constexpr (VK == kFp8) {
        // B = the codes' exact fp16 values; the V scales are in the probabilities
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const h8 pa = lds.afrag[i][lane];
          const u4 w0 = vsh.c[2 * hf][i >> 1], w1 = vsh.c[2 * hf + 1][i >> 1];
          oacc[2 * hf] = mfma(pa, fp8_vals(w0[2 * (i & 1)], w0[2 * (i & 1) + 1]), oacc[2 * hf]);
          oacc[2 * hf + 1] = mfma(pa, fp8_vals(w1[2 * (i & 1)], w1[2 * (i & 1) + 1]), oacc[2 * hf + 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else if constexpr (VK == kFp4) {
        // B = code value (conversion at scale 1) times the token's 2^e: exact fp16
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const h8 pa = lds.afrag[i][lane];
          const h8 sc = dp[(hf * 8 + i) * 4 + grp];
          const h8 b0 = fp4_vals(vsh.c[2 * hf][i >> 2][i & 3], 1.0f) * sc;
          const h8 b1 = fp4_vals(vsh.c[2 * hf + 1][i >> 2][i & 3], 1.0f) * sc;
          oacc[2 * hf] = mfma(pa, b0, oacc[2 * hf]);
          oacc[2 * hf + 1] = mfma(pa, b1, oacc[2 * hf + 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
      if (fast) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const h8 pa = lds.afrag[i][lane];
          if (VK == kQ4) {
            const h8* e = dp + ((hf * 8 + i) * 4 + grp);
            const h8 dh16 = e[0], nh = e[64], dl16 = e[128], nl = e[192];
            const u4 x0 = v_magic_q4(vsh.c[2 * hf][i >> 2][i & 3], vmask, vmagic);
            const u4 x1 = v_magic_q4(vsh.c[2 * hf + 1][i >> 2][i & 3], vmask, vmagic);
            // the two column tiles' MFMAs alternate, so no MFMA waits on the one before it
            oacc[2 * hf] = mfma(pa, pk_fma8(x0, dh16, nh), oacc[2 * hf]);
            oacc[2 * hf + 1] = mfma(pa, pk_fma8(x1, dh16, nh), oacc[2 * hf + 1]);
            oacc[2 * hf] = mfma(pa, pk_fma8(x0, dl16, nl), oacc[2 * hf]);
            oacc[2 * hf + 1] = mfma(pa, pk_fma8(x1, dl16, nl), oacc[2 * hf + 1]);
          } else {
            const h8* e = dp + (i * 4 + grp);
            const h8 pa_ = e[0], na = e[32], pb_ = e[64], nb = e[96], pc_ = e[128], nc = e[160];
            const u4 w0 = vsh.c[2 * hf][i >> 1], w1 = vsh.c[2 * hf + 1][i >> 1];
            const u4 x0 = v_magic_i8(w0[2 * (i & 1)], w0[2 * (i & 1) + 1], vmagic);
            const u4 x1 = v_magic_i8(w1[2 * (i & 1)], w1[2 * (i & 1) + 1], vmagic);
            // the two column tiles' MFMAs alternate, so no MFMA waits on the one before it
            oacc[2 * hf] = mfma(pa, pk_fma8(x0, pa_, na), oacc[2 * hf]);
            oacc[2 * hf + 1] = mfma(pa, pk_fma8(x1, pa_, na), oacc[2 * hf + 1]);
            oacc[2 * hf] = mfma(pa, pk_fma8(x0, pb_, nb), oacc[2 * hf]);
            oacc[2 * hf + 1] = mfma(pa, pk_fma8(x1, pb_, nb), oacc[2 * hf + 1]);
            oacc[2 * hf] = mfma(pa, pk_fma8(x0, pc_, nc), oacc[2 * hf]);
            oacc[2 * hf + 1] = mfma(pa, pk_fma8(x1, pc_, nc), oacc[2 * hf + 1]);
          }
          __builtin_amdgcn_sched_barrier(0);  // keep each step's LDS operands short-lived
        }
      } else {
        // scales too large for the folded constants: exact codes first, then the parts
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const h8 pa = lds.afrag[i][lane];
          if (VK == kQ4) {
            const h8* e = dp + ((hf * 8 + i) * 4 + grp);
            const h8 dh = e[0], dl = e[128];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int nt = 2 * hf + u;
              const u4 xm = v_magic_q4(vsh.c[nt][i >> 2][i & 3], vmask, vmagic);
              const h8 c8 = __builtin_elementwise_fma(__builtin_bit_cast(h8, xm), (h8)(_Float16)0.0625f,
                                                      (h8)(_Float16)(-72.0f));  // c - 8, exact
              oacc[nt] = mfma(pa, c8 * dh, oacc[nt]);
              oacc[nt] = mfma(pa, c8 * dl, oacc[nt]);
            }
          } else {
            const h8* e = dp + (i * 4 + grp);
            const h8 pa_ = e[0], pb_ = e[64], pc_ = e[128];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int nt = 2 * hf + u;
              const u4 words = vsh.c[nt][i >> 1];
              const u4 xm = v_magic_i8(words[2 * (i & 1)], words[2 * (i & 1) + 1], vmagic);
              const h8 c8 = __builtin_bit_cast(h8, xm) - (h8)(_Float16)1152.0f;  // c, exact
              oacc[nt] = mfma(pa, c8 * pa_, oacc[nt]);
              oacc[nt] = mfma(pa, c8 * pb_, oacc[nt]);
              oacc[nt] = mfma(pa, c8 * pc_, oacc[nt]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      }
      // this half's code registers now take the next page's codes
      load_vcodes<VK>(vsh, nr, voff[2 * hf], 2 * hf);
      load_vcodes<VK>(vsh, nr, voff[2 * hf + 1], 2 * hf + 1);
    }
    base = next;
    if (pg + 1 == boost_until) __builtin_amdgcn_s_setprio(0);
  }

  // ---------------- this split's partials: common max, summed weights, each wave's elements
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const float lsum = half_sum(l_run[r], lane);
    if (col == 0) lds.lsum[wave][2 * grp + r] = lsum;
  }
  // the partial of heads 2grp + r at element EPW w + 16t + col (hi + lo rows)
  float po[2][NTW];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int t = 0; t < NTW; ++t) po[r][t] = (oacc[t][2 * r] + oacc[t][2 * r + 1]) * (kPScaleInv * dunit);
  if (four_bit(VK)) {
    // V is stored rotated: the partial is rotated back here (H is linear, so the merge of
    // rotated partials is the rotated merge). Element bits 0-3 (col) between lanes,
    // the tile bits inside the lane, the wave bits through LDS.
    {
      float pv[2 * NTW];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int t = 0; t < NTW; ++t) pv[NTW * r + t] = po[r][t];
      butterfly<1>(pv, lane);
      butterfly<2>(pv, lane);
      butterfly<4>(pv, lane);
      butterfly<8>(pv, lane);
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int t = 0; t < NTW; ++t) po[r][t] = pv[NTW * r + t];
    }
#pragma unroll
    for (int m = 1; m < NTW; m <<= 1)
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          if (!(t & m)) {
            const float x = po[r][t], y = po[r][t + m];
            po[r][t] = x + y;
            po[r][t + m] = x - y;
          }
    __syncthreads();  // the query rows in LDS are no longer read
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int t = 0; t < NTW; ++t) lds.qs[2 * grp + r][EPW * wave + 16 * t + col] = po[r][t];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int e = EPW * wave + 16 * t + col, lo = e & (EPW - 1);
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < NW; ++k) {  // NW-point transform over the wave bits
          const float x = lds.qs[2 * grp + r][lo + EPW * k];
          acc += (__builtin_popcount(k & wave) & 1) ? -x : x;
        }
        po[r][t] = acc * 0.0625f;
      }
  } else {
    __syncthreads();
  }
  const size_t S = (size_t)n_splits;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int hh = 2 * grp + r;
    if (hh < G) {
      const size_t idx = ((size_t)b * n_q_heads + g * G + hh) * S + split;
#pragma unroll
      for (int t = 0; t < NTW; ++t) part_o[idx * kHeadDim + EPW * wave + 16 * t + col] = po[r][t];
      if (wave == 0 && col == 0) {
        float l = lds.lsum[0][hh];
#pragma unroll
        for (int w = 1; w < NW; ++w) l += lds.lsum[w][hh];
        part_ml[2 * idx] = m_run[r];
        part_ml[2 * idx + 1] = l;
      }
    }
  }
  }  // work items

  // the last workgroup to finish leaves the counters at zero for the next launch
  if (DYN && tid == 0) {
    __threadfence();
    if (atomicAdd(&sched[1], 1u) == gridDim.x - 1) {
      atomicExch(&sched[0], 0u);
      atomicExch(&sched[1], 0u);
    }
  }
}

// Log-sum-exp merge of the partials of one (query head, sequence) for one chunk of
// 32 head elements (partials of rotated V were rotated back by the split kernel).
// 256 threads: eight groups of 32 (one thread per element) each merge an eighth of
// the splits; a thread's 16 partial values of a pass are loaded together with the
// split maxima, before the weights are known; the group sums are added in a fixed
// order. Every chunk's workgroup forms the (cheap) maximum and weights itself. The
// merge is latency-bound: 32-element chunks give twice the workgroups of 64-element
// ones, each with half the loads per thread, and finish sooner.
constexpr int kCombineThreads = 256;
constexpr int kCombineElems = 32;                              // head elements per workgroup
constexpr int kCombineGroups = kCombineThreads / kCombineElems;
constexpr int kCombineRun = 16;                                // splits per thread per pass
constexpr int kCombinePass = kCombineGroups * kCombineRun;     // splits per pass
constexpr int kCombineChunk = 1024;                            // split weights held in LDS

__global__ __launch_bounds__(kCombineThreads) void decode_combine(
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    const int32_t* __restrict__ context_lens, int max_context, int n_q_heads,
    int pages_per_split, int n_splits, int n_q, float* __restrict__ out) {
  __shared__ float wts[kCombineChunk];
  __shared__ float part[kCombineGroups][kCombineElems];
  __shared__ float red[2][kCombineThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int el = tid & (kCombineElems - 1), sg = tid / kCombineElems;
  const int e = kCombineElems * blockIdx.z + el;
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t base = ((size_t)b * n_q_heads + h) * (size_t)n_splits;
  // issued before the context length is known: split tid's maximum and weight sum, and
  // the first pass of partials (indices clamped to the grid's splits)
  const f2 ml_first = *reinterpret_cast<const f2*>(part_ml + 2 * (base + min(tid, n_splits - 1)));
  const float m_first = ml_first[0], l_first = ml_first[1];
  float v[kCombineRun];
#pragma unroll
  for (int u = 0; u < kCombineRun; ++u)
    v[u] = part_o[(base + min(sg * kCombineRun + u, n_splits - 1)) * kHeadDim + e];
  int T = context_lens[b / n_q];
  T = T < 0 ? 0 : (T > max_context ? max_context : T);
  const int later = n_q - 1 - b % n_q;  // (as in the split kernel)
  T = T > later ? T - later : 0;
  const int n_pages = (T + kPageTokens - 1) / kPageTokens;
  const int ns = min(n_splits, (n_pages + pages_per_split - 1) / pages_per_split);
  float o = 0.f, L = 0.f;
  if (ns > 0) {  // uniform over the workgroup
    float M = tid < ns ? m_first : -INFINITY;
    for (int s = tid + kCombineThreads; s < ns; s += kCombineThreads) M = fmaxf(M, part_ml[2 * (base + s)]);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (lane == 0) red[0][wave] = M;
    __syncthreads();
    M = red[0][0];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) M = fmaxf(M, red[0][w]);
    float acc = 0.f;
    for (int s0 = 0; s0 < ns; s0 += kCombineChunk) {  // chunks of splits whose weights fit in LDS
      const int cnt = min(kCombineChunk, ns - s0);
      __syncthreads();
      for (int s = tid; s < cnt; s += kCombineThreads) {
        const bool first = s0 == 0 && s == tid;  // (loaded at the start)
        const float ms = first ? m_first : part_ml[2 * (base + s0 + s)];
        const float ls = first ? l_first : part_ml[2 * (base + s0 + s) + 1];
        const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
        wts[s] = w;
        L += w * ls;
      }
      __syncthreads();
      for (int p0 = 0; p0 < cnt; p0 += kCombinePass) {
        const int first = p0 + sg * kCombineRun;  // this group's run of the pass
        if (s0 + p0 > 0) {
#pragma unroll
          for (int u = 0; u < kCombineRun; ++u)
            v[u] = part_o[(base + min(s0 + first + u, ns - 1)) * kHeadDim + e];
        }
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < kCombineRun; ++u) {
          const int s = first + u;
          a += s < cnt ? wts[min(s, kCombineChunk - 1)] * v[u] : 0.f;  // splits past ns add nothing
        }
        acc += a;
      }
    }
    part[sg][el] = acc;
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    if (lane == 0) red[1][wave] = L;
  }
  __syncthreads();
  if (ns > 0 && sg == 0) {
    o = part[0][el];
#pragma unroll
    for (int g = 1; g < kCombineGroups; ++g) o += part[g][el];
    L = red[1][0];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) L += red[1][w];
    o = L > 0.f ? o / L : 0.f;  // L == 0 only if every page of the sequence was skipped
  }
  if (sg == 0) out[((size_t)b * n_q_heads + h) * kHeadDim + e] = o;
}

template <int KK, int VK, bool DYN, bool APPEND>
void launch_split_v(const DecodeArgs& a, dim3 grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  constexpr int NW = split_waves(KK);
  hipExtLaunchKernelGGL((decode_split<KK, VK, NW, DYN, APPEND>), grid, dim3(64 * NW), 0, stream, start,
                        stop, 0, a.q, a.pool, a.n_pool_pages, a.block_tables, a.max_pages,
                        a.context_lens, a.max_context, a.n_q_heads, a.n_kv_heads, a.pages_per_split,
                        a.n_splits, a.scale_log2, a.part_ml, a.part_o, a.status, a.sched, a.batch,
                        a.n_q, a.k_new, a.v_new, a.pool_w, a.n_cus);
}

template <int KK, int VK>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  constexpr int NW = split_waves(KK);
  // one round of resident workgroups (two 4-wave or one 8-wave per CU), at most one per item
  const int64_t items = (int64_t)a.n_splits * a.n_kv_heads * a.batch;
  const int64_t resident = (int64_t)a.n_cus * (8 / NW);
  const dim3 grid((unsigned)(items < resident ? items : resident));
  const bool dyn = items > resident, app = a.k_new != nullptr;
  if (dyn && app) launch_split_v<KK, VK, true, true>(a, grid, stream, start, stop);
  else if (dyn) launch_split_v<KK, VK, true, false>(a, grid, stream, start, stop);
  else if (app) launch_split_v<KK, VK, false, true>(a, grid, stream, start, stop);
  else launch_split_v<KK, VK, false, false>(a, grid, stream, start, stop);
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void zero_words(uint32_t* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_words(uint32_t* p, int n_words, hipStream_t stream) {
  hipLaunchKernelGGL(zero_words, dim3(1), dim3(64), 0, stream, p, n_words);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int phase, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop) {
  if (phase & 1) {
    hipError_t e;
    switch (a.fmt) {
      case KV_FMT_INT8: e = launch_split<kInt8, kInt8>(a, stream, start, stop); break;
      case KV_FMT_Q4_0: e = launch_split<kQ4, kQ4>(a, stream, start, stop); break;
      case KV_FMT_FP4: e = launch_split<kFp4, kFp4>(a, stream, start, stop); break;
      case KV_FMT_FP8: e = launch_split<kFp8, kFp8>(a, stream, start, stop); break;
      default: e = launch_split<kInt8, kQ4>(a, stream, start, stop); break;
    }
    if (e != hipSuccess) return e;
  }
  if (phase & 2) {
    dim3 grid((unsigned)a.n_q_heads, (unsigned)a.batch, kHeadDim / kCombineElems), block(kCombineThreads);
    hipLaunchKernelGGL(decode_combine, grid, block, 0, stream, a.part_ml, a.part_o, a.context_lens,
                       a.max_context, a.n_q_heads, a.pages_per_split, a.n_splits, a.n_q, a.out);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace kvc
