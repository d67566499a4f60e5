// Split-sequence decode attention on the matrix cores (gfx950, wave64), with
// the dequantization fused into both products: the TurboQuant page (§2.3,
// end) puts dequantization inside the attention product instead of a
// separate pass; the Cocktail page (§3.2.3) computes attention per block and
// merges the block results.
//
// A wave consumes tiles of 32 cached tokens.  For each tile:
//   scores  S[m][t] = sum_d q[m][d] k_hat[t][d]   v_mfma_f32_16x16x32_f16,
//           A = the query tile (16 rows: up to 16 query heads sharing this KV
//           head), B = K codes (16 tokens per column block), 4 k-steps of 32
//           channels, two column blocks per tile;
//   output  O[m][c] += sum_t w[m][t] v_hat[t][c]  same instruction, A = the
//           softmax weights (binary32 split into two fp16 halves, hi + lo),
//           B = V codes, one k-step of 32 tokens, 8 column blocks of 16
//           channels.
// Codes enter the matrix cores as exact small fp16 integers OFF + c, built
// with a magic-exponent OR (OFF = 16 for 4-bit, 4 for 2-bit; 8-bit codes
// subtract their offset of 256 / 384 with one exact packed fp16 add, OFF =
// 0).  Group scales and zero-points stay in binary32 outside the
// products: per token t and channel group g
//   score = sum_g s[t][g] * (C_g[t] - (OFF + z[t][g]) * Q_g),  Q_g = sum_{d in g} q_d,
// which equals sum_d q_d s (c_td - z) up to binary32 rounding.  On the V side
// a packed fp16 add of -(OFF + z) turns each B element into c - z exactly
// before the product, so
//   O[c]  = sum_t (p_t s[t][g(c)]) (c_t - z[t][g(c)])
// carries no large offset that would cancel in binary32.
// The layouts of packed rows (kvq.h) are chosen for these operands: a
// K row is 16 slots of 8 channels, slot 4q + s holding channels
// 32 s + 8 q + v, so every k-step (32 channels) lies in one quantization
// group; a V row is 16 column words, word n holding channels n + 16 j, so a
// lane forms the B operand of column block j from its 8 token rows.
//
// Lane roles: l = lane, n16 = l & 15, q4 = l >> 4.
//  K-MFMA  A: row n16 = query, k-slots of lane group q4;
//          B: column n16 = token (nb*16 + n16), same k-slots;
//          C: column n16 = token, rows 4*q4 + i = queries (i < 4).
//  V-MFMA  A: row n16 = query, k-slots = tokens 8*q4 .. 8*q4+7 of the tile;
//          B: column n16 = channel 16 j + n16, same token slots;
//          C: column = channel 16 j + n16, rows 4*q4 + i = queries.
// Softmax state (running max, sum, V bias) lives with the C rows: lane
// (q4, n16) owns queries 4*q4 + i for its token column and its channels.
#pragma once
#include "kvq_dev.h"

namespace kvq {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef unsigned u4_t __attribute__((ext_vector_type(4)));
typedef unsigned u2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kNW = 4;    // waves per workgroup
constexpr int kTile = 32; // tokens per tile

__device__ __forceinline__ f4_t mfma(u4_t a, u4_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned perm(unsigned hi, unsigned lo, unsigned sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// perm selector placing byte `a` of lo at bits 0-7 and byte `a` of hi at bits 16-23
__host__ __device__ constexpr unsigned sel_bytes(int a) {
  return (0x0Cu << 24) | ((4u + a) << 16) | (0x0Cu << 8) | (unsigned)a;
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }


// (x & m) | c as one v_and_or_b32.  VOP3 encodings take no literal
// constants on this target, so with literal m and c the compiler emits an AND
// and an OR; passing m and c through an empty asm hides their values, so they
// are kept in registers (the asm has no side effects and is hoisted out of
// loops) and the selector fuses the pair.  The instruction itself stays
// compiler-generated, so its hazards against the matrix cores are tracked.
__device__ __forceinline__ unsigned opaque(unsigned v) {
  asm("" : "+v"(v));
  return v;
}
__device__ __forceinline__ unsigned and_or(unsigned x, unsigned m, unsigned c) {
  return (x & opaque(m)) | opaque(c);
}

__device__ __forceinline__ float f16lo(unsigned w) { return (float)__builtin_bit_cast(h2_t, w)[0]; }
__device__ __forceinline__ float f16hi(unsigned w) { return (float)__builtin_bit_cast(h2_t, w)[1]; }

// Two binary32 values -> (hi, lo) fp16 pairs with a + b == hi + lo to ~2^-22.
__device__ __forceinline__ void split_pair(float a, float b, unsigned& hi, unsigned& lo) {
  const h2_t h = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(a, b));
  hi = __builtin_bit_cast(unsigned, h);
  lo = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a - (float)h[0], b - (float)h[1]));
}

// ---------------------------------------------------------------------------
// K codecs: load a token row's 4 slices for lane group q4, and form k-step s
// as 4 fp16 pairs (channels v, v + 4 of the slice), value OFF + code.  The
// widening leaves an offset under the code (the exponent's implicit bit);
// the per-group bias (OFF + z) sum q removes it after the product.  A large
// offset inflates the binary32 partial sums of the matrix cores and costs
// absolute precision in the scores, so the 8-bit codecs subtract theirs
// exactly in fp16 first (OFF = 0).

struct KI4 {
  static constexpr int RB = 64, OFF = 16, BITS = 4;
  static constexpr bool SYM = false, F16 = false;
  u4_t r;
  __device__ __forceinline__ void load(const uint8_t* row, int q4) {
    r = ld_nt<u4_t>(row + q4 * 16);
  }
  __device__ __forceinline__ u4_t slice(int s) const {
    const unsigned w = r[s];
    u4_t o;
    o[0] = and_or(w << 6, 0x03C003C0u, 0x4C004C00u);
    o[1] = and_or(w << 2, 0x03C003C0u, 0x4C004C00u);
    o[2] = and_or(w >> 2, 0x03C003C0u, 0x4C004C00u);
    o[3] = and_or(w >> 6, 0x03C003C0u, 0x4C004C00u);
    return o;
  }
};

struct KI2 {
  static constexpr int RB = 32, OFF = 4, BITS = 2;
  static constexpr bool SYM = false, F16 = false;
  u2_t r;
  __device__ __forceinline__ void load(const uint8_t* row, int q4) {
    r = ld_nt<u2_t>(row + q4 * 8);
  }
  __device__ __forceinline__ u4_t slice(int s) const {
    const unsigned d = r[s >> 1];
    // byte 0 of the slice (channels 0-3) to the low half, byte 1 (4-7) to the high half
    const unsigned x = (s & 1) ? perm(0u, d, 0x0C030C02u) : perm(0u, d, 0x0C010C00u);
    u4_t o;
    o[0] = and_or(x << 8, 0x03000300u, 0x44004400u);
    o[1] = and_or(x << 6, 0x03000300u, 0x44004400u);
    o[2] = and_or(x << 4, 0x03000300u, 0x44004400u);
    o[3] = and_or(x << 2, 0x03000300u, 0x44004400u);
    return o;
  }
};

template <bool SYM_>
struct KI8 {
  static constexpr int RB = 128, OFF = 0, BITS = 8;
  static constexpr bool SYM = SYM_, F16 = false;
  // 256 + byte (offset binary for the signed codes: 384 + c) minus that
  // offset, as an exact fp16 pair: the code itself
  static constexpr unsigned kUnoffset = SYM_ ? 0xDE00DE00u : 0xDC00DC00u;  // -(384, 384) or -(256, 256)
  u4_t a, b;
  __device__ __forceinline__ void load(const uint8_t* row, int q4) {
    a = ld_nt<u4_t>(row + q4 * 32);
    b = ld_nt<u4_t>(row + q4 * 32 + 16);
  }
  __device__ __forceinline__ u4_t slice(int s) const {
    unsigned lo = s < 2 ? a[2 * s] : b[2 * s - 4];
    unsigned hi = s < 2 ? a[2 * s + 1] : b[2 * s - 3];
    if constexpr (SYM) {
      lo ^= 0x80808080u;
      hi ^= 0x80808080u;
    }
    u4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned w = (perm(hi, lo, sel_bytes(i)) << 2) | 0x5C005C00u;
      o[i] = __builtin_bit_cast(unsigned, __builtin_bit_cast(h2_t, w) + __builtin_bit_cast(h2_t, kUnoffset));
    }
    return o;
  }
};

// FP8 E4M3 codes ([KVQ-Eng] FP8 item): every E4M3 value is a normal fp16
// number (the smallest, 2^-9, is above fp16's normal range limit 2^-14), so
// the hardware's scaled conversion with scale 1 widens a pair of codes to
// an exact fp16 pair.  Bytes i and i + 1 of the slot's two words are
// gathered into one word (lo.i, hi.i, lo.i+1, hi.i+1) whose halves convert
// to the pairs of slots i and i + 1 (channel offsets i and i + 4, as INT8).
template <bool UPPER>
__device__ __forceinline__ unsigned e4m3_pair(unsigned x) {
  const h2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, UPPER);
  return __builtin_bit_cast(unsigned, h);
}
__host__ __device__ constexpr unsigned sel_pairs(int i) {  // i even
  return ((5u + i) << 24) | ((unsigned)(i + 1) << 16) | ((4u + i) << 8) | (unsigned)i;
}

struct KE4 {
  static constexpr int RB = 128, OFF = 0, BITS = 8;
  static constexpr bool SYM = true, F16 = false;
  u4_t a, b;
  __device__ __forceinline__ void load(const uint8_t* row, int q4) {
    a = ld_nt<u4_t>(row + q4 * 32);
    b = ld_nt<u4_t>(row + q4 * 32 + 16);
  }
  __device__ __forceinline__ u4_t slice(int s) const {
    const unsigned lo = s < 2 ? a[2 * s] : b[2 * s - 4];
    const unsigned hi = s < 2 ? a[2 * s + 1] : b[2 * s - 3];
    const unsigned x0 = perm(hi, lo, sel_pairs(0)), x2 = perm(hi, lo, sel_pairs(2));
    u4_t o;
    o[0] = e4m3_pair<false>(x0);
    o[1] = e4m3_pair<true>(x0);
    o[2] = e4m3_pair<false>(x2);
    o[3] = e4m3_pair<true>(x2);
    return o;
  }
};

// FP8 E5M2 codes: an E5M2 byte is the high byte of the fp16 number of the
// same value (same exponent field, two mantissa bits), so one byte permute
// per pair builds the exact fp16 operands: byte i of the slot's two words to
// bits 8-15 and 24-31 (channel offsets i and i + 4, as INT8).
__host__ __device__ constexpr unsigned sel_high_bytes(int i) {
  return ((4u + i) << 24) | (0x0Cu << 16) | ((unsigned)i << 8) | 0x0Cu;
}

struct KE5 {
  static constexpr int RB = 128, OFF = 0, BITS = 8;
  static constexpr bool SYM = true, F16 = false;
  u4_t a, b;
  __device__ __forceinline__ void load(const uint8_t* row, int q4) {
    a = ld_nt<u4_t>(row + q4 * 32);
    b = ld_nt<u4_t>(row + q4 * 32 + 16);
  }
  __device__ __forceinline__ u4_t slice(int s) const {
    const unsigned lo = s < 2 ? a[2 * s] : b[2 * s - 4];
    const unsigned hi = s < 2 ? a[2 * s + 1] : b[2 * s - 3];
    u4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = perm(hi, lo, sel_high_bytes(i));
    return o;
  }
};

struct KF16 {
  static constexpr int RB = 256, OFF = 0, BITS = 16;
  static constexpr bool SYM = false, F16 = true;
  u4_t r[4];
  __device__ __forceinline__ void load(const uint8_t* row, int q4) {
#pragma unroll
    for (int s = 0; s < 4; ++s) r[s] = ld_nt<u4_t>(row + q4 * 64 + 16 * s);
  }
  __device__ __forceinline__ u4_t slice(int s) const { return r[s]; }
};

// ---------------------------------------------------------------------------
// V codecs: load the lane's column word n16 of 8 token rows and form the B
// operand of column block j: 4 fp16 pairs (rows 2r, 2r + 1), each the fp16
// integer 1024 + f * code (the code masked in place under the exponent of
// 1024, whose ulp is 1; f = 16 when the code sits 4 bits up, odd blocks of
// 4-bit codes).  The tile loop adds the packed pair -(1024 + f * z) of the
// two rows, leaving f * (code - z) exactly; the output block then carries the
// factor f, removed when the wave's state leaves the loop.  Zero-point pairs
// are built from the rows' z bytes as ((z << ZSH[par]) & ZMASK[par]) | ZMAGIC,
// par = 1 for odd blocks when ZODD.

// kWeightScaleNote.  The V weights w = p s (p <= 1 the softmax numerator, s
// the token group's V scale; p alone for fp16 rows) enter the matrix cores as
// fp16 hi + lo pairs.  Most p of a long sequence are far below 1, so w would
// often be an fp16 subnormal, and the matrix cores do not multiply
// subnormal operands exactly (a row of 4097 E4M3 tokens lost 1.3e-4 of its
// norm that way).  Each codec therefore scales its weights by WS, a power of
// two as large as keeps s WS (the largest weight) below the fp16 maximum for
// any fp16 input (the bound is noted at each WS), so that only weights far
// too small to matter stay subnormal; WS is exact, and the output blocks
// carry it (fac) until the wave's state leaves the loop.
struct VI4 {
  static constexpr float WS = 4.0f;  // weight scale (see kWeightScaleNote): s 4 <= 34,935
  static constexpr int RB = 64, BITS = 4;
  static constexpr bool SYM = false, F16 = false, ZODD = true, ZP = true, MASK_ROWS = false;
  static constexpr unsigned ZMAGIC = 0xE400E400u;
  static constexpr unsigned ZMASK[2] = {0x000F000Fu, 0x00F000F0u};
  static constexpr int ZSH[2] = {0, 4};
  static constexpr float fac(int j) { return (j & 1) ? 16.0f * WS : WS; }
  unsigned r[8];
  __device__ __forceinline__ void load(const uint8_t* row0, int n16) {
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = ld_nt<unsigned>(row0 + k * RB + n16 * 4);
  }
  __device__ __forceinline__ void zero_row(int k) { r[k] = 0u; }
  __device__ __forceinline__ u4_t block(int j) const {
    u4_t o;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      o[p] = and_or(perm(r[2 * p + 1], r[2 * p], sel_bytes(j >> 1)), ZMASK[j & 1], 0x64006400u);
    return o;
  }
};

struct VI2 {
  static constexpr float WS = 1.0f;  // weight scale (see kWeightScaleNote): s <= 43,669
  static constexpr int RB = 32, BITS = 2;
  static constexpr bool SYM = false, F16 = false, ZODD = false, ZP = true, MASK_ROWS = false;
  static constexpr unsigned ZMAGIC = 0xE400E400u;
  static constexpr unsigned ZMASK[2] = {0x00030003u, 0x00030003u};
  static constexpr int ZSH[2] = {0, 0};
  static constexpr float fac(int) { return 1.0f; }
  unsigned x[4];  // rows 2p (low half) and 2p + 1 (high half)
  __device__ __forceinline__ void load(const uint8_t* row0, int n16) {
    unsigned r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = ld_nt<uint16_t>(row0 + k * RB + n16 * 2);
#pragma unroll
    for (int p = 0; p < 4; ++p) x[p] = perm(r[2 * p + 1], r[2 * p], 0x05040100u);
  }
  __device__ __forceinline__ void zero_row(int k) {
    x[k >> 1] &= (k & 1) ? 0x0000FFFFu : 0xFFFF0000u;
  }
  __device__ __forceinline__ u4_t block(int j) const {
    u4_t o;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = and_or(x[p] >> (2 * j), 0x00030003u, 0x64006400u);
    return o;
  }
};

template <bool SYM_>
struct VI8 {
  static constexpr float WS = 64.0f;  // weight scale (see kWeightScaleNote): s 64 <= 33,011
  static constexpr int RB = 128, BITS = 8;
  static constexpr bool SYM = SYM_, F16 = false, ZODD = false, ZP = true, MASK_ROWS = false;
  static constexpr unsigned ZMAGIC = 0xE400E400u;
  static constexpr unsigned ZMASK[2] = {0x00FF00FFu, 0x00FF00FFu};
  static constexpr int ZSH[2] = {0, 0};
  static constexpr float fac(int) { return WS; }
  unsigned w0[8], w1[8];  // codes 0-3 and 4-7 of the column word, per row (offset binary)
  __device__ __forceinline__ void load(const uint8_t* row0, int n16) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u2_t v = ld_nt<u2_t>(row0 + k * RB + n16 * 8);
      const unsigned vx = v[0], vy = v[1];
      w0[k] = SYM ? (vx ^ 0x80808080u) : vx;
      w1[k] = SYM ? (vy ^ 0x80808080u) : vy;
    }
  }
  __device__ __forceinline__ void zero_row(int k) {}
  __device__ __forceinline__ u4_t block(int j) const {
    const unsigned* w = (j >> 2) ? w1 : w0;
    u4_t o;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = perm(w[2 * p + 1], w[2 * p], sel_bytes(j & 3)) | 0x64006400u;
    return o;
  }
};

// E4M3 V codes: the B operand pairs (rows 2p, 2p + 1) of column blocks j and
// j + 1 come from one gathered word, converted half by half (see KE4).  No
// zero-point; rows past the valid range are cleared (a stray byte could be
// the NaN pattern, and 0 * NaN would poison the product).
struct VE4 {
  static constexpr float WS = 256.0f;  // weight scale (see kWeightScaleNote): s 256 <= 37,431
  static constexpr int RB = 128, BITS = 8;
  static constexpr bool SYM = true, F16 = false, ZODD = false, ZP = false, MASK_ROWS = true;
  static constexpr float fac(int) { return WS; }
  unsigned w0[8], w1[8];  // codes of channels n16 + 16 e, e = 0-3 and 4-7, per row
  __device__ __forceinline__ void load(const uint8_t* row0, int n16) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u2_t v = ld_nt<u2_t>(row0 + k * RB + n16 * 8);
      w0[k] = v[0];
      w1[k] = v[1];
    }
  }
  __device__ __forceinline__ void zero_row(int k) {
    w0[k] = 0u;
    w1[k] = 0u;
  }
  __device__ __forceinline__ u4_t block(int j) const {
    const unsigned* w = (j >> 2) ? w1 : w0;
    u4_t o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const unsigned x = perm(w[2 * p + 1], w[2 * p], sel_pairs(j & 2));
      o[p] = (j & 1) ? e4m3_pair<true>(x) : e4m3_pair<false>(x);
    }
    return o;
  }
};

// E5M2 V codes: the B operand pair (rows 2p, 2p + 1) of column block j is
// byte j mod 4 of the two rows' words moved to the high bytes.  No
// zero-point; rows past the valid range are cleared (a stray byte could be
// an infinity or NaN pattern).
struct VE5 {
  static constexpr float WS = 32768.0f;  // weight scale (see kWeightScaleNote): s 2^15 <= 37,450
  static constexpr int RB = 128, BITS = 8;
  static constexpr bool SYM = true, F16 = false, ZODD = false, ZP = false, MASK_ROWS = true;
  static constexpr float fac(int) { return WS; }
  unsigned w0[8], w1[8];  // codes of channels n16 + 16 e, e = 0-3 and 4-7, per row
  __device__ __forceinline__ void load(const uint8_t* row0, int n16) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u2_t v = ld_nt<u2_t>(row0 + k * RB + n16 * 8);
      w0[k] = v[0];
      w1[k] = v[1];
    }
  }
  __device__ __forceinline__ void zero_row(int k) {
    w0[k] = 0u;
    w1[k] = 0u;
  }
  __device__ __forceinline__ u4_t block(int j) const {
    const unsigned* w = (j >> 2) ? w1 : w0;
    u4_t o;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = perm(w[2 * p + 1], w[2 * p], sel_high_bytes(j & 3));
    return o;
  }
};

struct VF16 {
  static constexpr float WS = 32768.0f;  // weight scale (see kWeightScaleNote): the weight is p <= 1
  static constexpr int RB = 256, BITS = 16;
  static constexpr bool SYM = false, F16 = true, ZODD = false, ZP = false, MASK_ROWS = true;
  static constexpr float fac(int) { return WS; }
  u4_t r[8];
  __device__ __forceinline__ void load(const uint8_t* row0, int n16) {
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = ld_nt<u4_t>(row0 + k * RB + n16 * 16);
  }
  __device__ __forceinline__ void zero_row(int k) { r[k] = u4_t{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ u4_t block(int j) const {
    u4_t o;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      o[p] = perm(r[2 * p + 1][j >> 1], r[2 * p][j >> 1], (j & 1) ? 0x07060302u : 0x05040100u);
    return o;
  }
};

// ---------------------------------------------------------------------------
// Per-call parameters and per-(b, kv head) views.

struct AttnParams {
  int B, H, S, Hq, G, qtiles, max_len, num_splits, split_len, chunk_tokens;
  float qscale;  // sm_scale * log2(e)
  const uint16_t* q;
  const int* seq_len;
  float* out;
  float* ws;           // split partials [B][Hq][num_splits][kPartStride]
  float* oak_ksc;      // OAKEN: K outer-value score shares [B][Hq][max_len]
  const int* seg;
  unsigned* status;
  TensorArgs k, v;
  const int* pages;  // paged layout: block table [B][S / ptok]; null when contiguous
  int pshift;        // log2 tokens per page
  int npages;
  int dsq_sig;       // DSQ: significant tokens per 64-token group
};

// One tensor's view for a (b, kv head): code rows and token-axis metadata.
// Contiguous: row t of the (b, h) is token t.  Paged: the pointers are the
// pool bases and token t sits in row (pages[t >> pshift] H + h) 2^pshift +
// (t mod 2^pshift); at_tile rebases a view for the 32-token tile holding t
// (a tile never straddles a page) so that row t addresses it directly.
struct TokView {
  const uint8_t* codes;  // row 0 of this (b, h), or the pool base when paged
  const float* scale;    // [rows][ng]
  const uint8_t* zero;   // [rows][ng] (null when symmetric)
  const int* pages;      // paged: this sequence's block-table row (else null)
  int pshift;            // log2 tokens per page
  int hrow;              // this head's first row in a page: h << pshift
  int prow;              // rows of a page over all heads: H << pshift
  int npages;
  unsigned* status;
  const float* oscale = nullptr;  // Oaken: outer scales [rows][ng], rows as `scale`
};

// Block-table entry i, loaded on the vector path: a scalar load would share
// its wait counter with the LDS operations, so every LDS wait of the tile
// loop would also wait for it.  The opaque zero keeps the address
// non-uniform; callers make the value wave-uniform (readfirstlane) where
// they use it, one step later, so the page arithmetic stays scalar.
__device__ __forceinline__ int page_entry_v(const int* pages, int i) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return pages[i + z];
}

// Row offset that maps the tokens t of the page-aligned range starting at
// `tok` (within one page) to their pool rows: row = t + offset.  pg is the
// block-table entry of that page; one outside the pool reads page 0 and
// raises the flag.
__device__ __forceinline__ long long page_row_offset(const TokView& v, int pg, int tok) {
  if (pg < 0 || pg >= v.npages) {
    if ((threadIdx.x & 63) == 0) set_flag(v.status, kFlagPageRange);
    pg = 0;
  }
  return (long long)pg * v.prow + v.hrow + (tok & ((1 << v.pshift) - 1)) - tok;
}

template <int RB, int NG>
__device__ __forceinline__ TokView at_rows(const TokView& v, long long off) {
  TokView r = v;
  r.codes = v.codes + off * RB;
  r.scale = v.scale + off * NG;
  if (v.zero) r.zero = v.zero + off * NG;
  if (v.oscale) r.oscale = v.oscale + off * NG;
  return r;
}

// Channel-axis K metadata: per 64-token block, per channel.
struct ChanView {
  const float* scale;   // [S/64][128]
  const uint8_t* zero;  // [S/64][128]
};

// Running softmax state of a wave (lane-held, see the header comment).
template <int GI>
struct SoftState {
  float m[GI], l[GI];
  f4_t o[8];  // [column block j] rows 4*q4 + i
};

template <int GI>
__device__ __forceinline__ void soft_init(SoftState<GI>& st) {
#pragma unroll
  for (int i = 0; i < GI; ++i) {
    st.m[i] = -INFINITY;
    st.l[i] = 0.0f;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
}

}  // namespace kvq
