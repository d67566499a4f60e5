/*
 * CPU oracle for group-wise KV-cache quantization and quantized decode
 * attention.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests, by the
 * package's smoke check and by the bench's CPU-baseline leg, never by the
 * product path.  It shares no source with the HIP library.
 *
 * Plain scalar C, built with -O2 -ffp-contract=off (no fast-math), so every
 * float expression below is one IEEE-754 binary32 operation rounded to
 * nearest-even; attention is evaluated in binary64.
 *
 * Pages cited (titles as published):
 *  [Oaken]      "大模型KV缓存量化技术：原理、优化与实践" (jsqmd.com)
 *  [KVQ-Eng]    "大模型推理加速之KV Cache量化压缩原理与工程实现" (yunthe.com)
 *  [KVO-LLM]    "长上下文LLM推理中的KV Cache优化技术解析" (intelliparadigm.com)
 *  [Cocktail]   Cocktail chunk-adaptive mixed-precision KV-cache page (peacm.com)
 *  [TurboQuant] TurboQuant KV-cache page (bhfrc.com)
 *
 * Readings taken where the pages are silent:
 *  - Range widened to include zero: lo = min(0, min x), hi = max(0, max x),
 *    so the zero-point is an integer code inside [0, 2^b - 1].
 *  - An all-zero group has scale 0; then zero-point and codes are 0.
 *  - Rounding is half-to-even everywhere; x / s is a true division.
 *  - Dequantized values are formed in binary32, attention in binary64.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* fp16 input                                                               */
/* ---------------------------------------------------------------------- */

/* Exact binary16 -> binary32 (every half value is representable). */
float ora_f16_to_f32(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  float v;
  if (e == 0)
    v = ldexpf((float)m, -24); /* subnormal (or zero) */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexpf((float)(1024 + m), e - 25);
  return sign ? -v : v;
}

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* ---------------------------------------------------------------------- */
/* Group quantizers                                                         */
/* ---------------------------------------------------------------------- */

/*
 * Asymmetric b-bit quantization of one group of n elements read with the
 * given stride.  Scale from the group's range over 2^b - 1 levels
 * ([Oaken] §2.1, the static-quantization formula); code = round(x / s) + z
 * with s the scale and z the zero-point ([Cocktail] §3.2.2).
 * Writes the scale, the zero-point and n codes (contiguous).
 */
void ora_quant_group_asym(const uint16_t* x, long n, long stride, int bits, float* s_out,
                          uint8_t* z_out, uint8_t* q) {
  int qmax = (1 << bits) - 1;
  float lo = 0.0f, hi = 0.0f;
  for (long i = 0; i < n; ++i) {
    float v = ora_f16_to_f32(x[i * stride]);
    if (v < lo) lo = v;
    if (v > hi) hi = v;
  }
  float s = (hi - lo) / (float)qmax;
  *s_out = s;
  if (s == 0.0f) {
    *z_out = 0;
    for (long i = 0; i < n; ++i) q[i] = 0;
    return;
  }
  int z = clampi((int)rintf(-lo / s), 0, qmax);
  *z_out = (uint8_t)z;
  for (long i = 0; i < n; ++i) {
    float v = ora_f16_to_f32(x[i * stride]);
    q[i] = (uint8_t)clampi((int)rintf(v / s) + z, 0, qmax);
  }
}

/*
 * Symmetric INT8 of one group: scale = amax / 127, code = round(x / scale)
 * clamped to [-128, 127] ([KVQ-Eng], "INT8逐通道量化" listing).  The page
 * takes amax along the last axis, i.e. per token and head; here the scale
 * is formed in binary32 rather than the listing's fp16.
 */
void ora_quant_group_sym8(const uint16_t* x, long n, long stride, float* s_out, int8_t* q) {
  float amax = 0.0f;
  for (long i = 0; i < n; ++i) {
    float v = fabsf(ora_f16_to_f32(x[i * stride]));
    if (v > amax) amax = v;
  }
  float s = amax / 127.0f;
  *s_out = s;
  for (long i = 0; i < n; ++i) {
    if (s == 0.0f) {
      q[i] = 0;
      continue;
    }
    float v = ora_f16_to_f32(x[i * stride]);
    q[i] = (int8_t)clampi((int)rintf(v / s), -128, 127);
  }
}

/*
 * Token-axis groups: each of `rows` rows of D elements is split into D / g
 * contiguous groups ([TurboQuant] §2.3, per-group scaling along the head
 * dimension).  codes: rows x D (one code per byte, int8 for sym),
 * scale and zero: rows x (D / g).  zero may be NULL when sym.
 */
void ora_quant_rows(const uint16_t* x, long rows, int D, int g, int bits, int sym,
                    uint8_t* codes, float* scale, uint8_t* zero) {
  int ng = D / g;
  for (long r = 0; r < rows; ++r)
    for (int j = 0; j < ng; ++j) {
      const uint16_t* xg = x + r * D + (long)j * g;
      uint8_t* qg = codes + r * D + (long)j * g;
      if (sym)
        ora_quant_group_sym8(xg, g, 1, &scale[r * ng + j], (int8_t*)qg);
      else
        ora_quant_group_asym(xg, g, 1, bits, &scale[r * ng + j], &zero[r * ng + j], qg);
    }
}

/* ---------------------------------------------------------------------- */
/* FP8 E4M3 codes                                                           */
/* ---------------------------------------------------------------------- */

/*
 * [KVQ-Eng] §"主流KV Cache量化方案对比", item 1 (FP8): the cache is converted
 * from fp16 to 8-bit floating point, E4M3 or E5M2.  The E4M3 format used is
 * the OCP 8-bit one without infinities: 1 sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9, and
 * the all-ones pattern S.1111.111 is NaN, so the largest finite magnitude
 * is 1.75 * 2^8 = 448.
 *
 * Readings (the page names the formats only):
 *  - Scale: dynamic, one binary32 scale per token group (the page's practice
 *    section prefers dynamic per-vector scales), s = max|x| / 448, so the
 *    group's largest magnitude lands on the largest finite code.
 *  - Code: the E4M3 value nearest to the binary32 quotient x / s, ties to
 *    the code with an even mantissa; magnitudes beyond 448 saturate to 448;
 *    the code's sign bit is the quotient's sign bit.
 *  - An all-zero group has scale 0 and codes 0.
 *  - Dequantized value: E4M3 value * s in binary32 (exact product rounded once).
 */

/* Value of an E4M3 code, from the format definition (binary64, exact). */
double ora_e4m3_value(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return (c & 0x80) ? -v : v;
}

/* E4M3 code of a binary32 value: the nearest of the 127 finite non-negative
 * magnitudes (codes 0x00 .. 0x7E, increasing with the code), found by a
 * plain search; on a tie the even code wins; 448 and beyond give 448. */
uint8_t ora_e4m3_encode(float y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs(ora_e4m3_value((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      bd = d;
      best = c;
    }
  }
  if (a >= 448.0) best = 0x7E; /* saturation (distances lose all precision far above 448) */
  return (uint8_t)(sign | best);
}

/* One group of n elements: s = amax / 448, codes E4M3(x / s). */
void ora_quant_group_e4m3(const uint16_t* x, long n, float* s_out, uint8_t* q) {
  float amax = 0.0f;
  for (long i = 0; i < n; ++i) {
    float v = fabsf(ora_f16_to_f32(x[i]));
    if (v > amax) amax = v;
  }
  float s = amax / 448.0f;
  *s_out = s;
  for (long i = 0; i < n; ++i) q[i] = s == 0.0f ? 0 : ora_e4m3_encode(ora_f16_to_f32(x[i]) / s);
}

/* Token-axis groups of g channels, E4M3 codes: codes rows x D, scale rows x (D / g). */
void ora_quant_rows_e4m3(const uint16_t* x, long rows, int D, int g, uint8_t* codes, float* scale) {
  int ng = D / g;
  for (long r = 0; r < rows; ++r)
    for (int j = 0; j < ng; ++j)
      ora_quant_group_e4m3(x + r * D + (long)j * g, g, &scale[r * ng + j], codes + r * D + (long)j * g);
}

/* x_hat = value(code) * s in binary32. */
void ora_dequant_rows_e4m3(const uint8_t* codes, const float* scale, long rows, int D, int g,
                           float* out) {
  int ng = D / g;
  for (long r = 0; r < rows; ++r)
    for (int d = 0; d < D; ++d)
      out[r * D + d] = (float)ora_e4m3_value(codes[r * D + d]) * scale[r * ng + d / g];
}

/*
 * FP8 E5M2, the other format of [KVQ-Eng] §"主流KV Cache量化方案对比", item 1:
 * 1 sign bit, 5 exponent bits with bias 15, 2 mantissa bits (the exponent
 * of fp16); exponent field 0 holds the subnormals m * 2^-16, the all-ones
 * exponent infinities (mantissa 0) and NaNs, so the largest finite
 * magnitude is 1.75 * 2^15 = 57344.
 *
 * Readings (as for E4M3): one binary32 scale per token group,
 * s = max|x| / 57344; the code of x / s is the nearest finite E5M2 value,
 * ties to the even mantissa, magnitudes from 57344 up saturate to 57344
 * (the cache never holds an infinity), sign bit of the quotient kept; an
 * all-zero group has scale 0 and codes 0.
 */
double ora_e5m2_value(uint8_t c) {
  int e = (c >> 2) & 31, m = c & 3;
  double v;
  if (e == 31)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -16);
  else
    v = ldexp((double)(4 + m), e - 17);
  return (c & 0x80) ? -v : v;
}

/* E5M2 code of a binary32 value: the nearest of the 124 finite non-negative
 * magnitudes (codes 0x00 .. 0x7B, increasing with the code), found by a
 * plain search; on a tie the even code wins; 57344 and beyond give 57344. */
uint8_t ora_e5m2_encode(float y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c <= 0x7B; ++c) {
    double d = fabs(ora_e5m2_value((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      bd = d;
      best = c;
    }
  }
  if (a >= 57344.0) best = 0x7B; /* saturation */
  return (uint8_t)(sign | best);
}

/* One group of n elements: s = amax / 57344, codes E5M2(x / s). */
void ora_quant_group_e5m2(const uint16_t* x, long n, float* s_out, uint8_t* q) {
  float amax = 0.0f;
  for (long i = 0; i < n; ++i) {
    float v = fabsf(ora_f16_to_f32(x[i]));
    if (v > amax) amax = v;
  }
  float s = amax / 57344.0f;
  *s_out = s;
  for (long i = 0; i < n; ++i) q[i] = s == 0.0f ? 0 : ora_e5m2_encode(ora_f16_to_f32(x[i]) / s);
}

/* Token-axis groups of g channels, E5M2 codes: codes rows x D, scale rows x (D / g). */
void ora_quant_rows_e5m2(const uint16_t* x, long rows, int D, int g, uint8_t* codes, float* scale) {
  int ng = D / g;
  for (long r = 0; r < rows; ++r)
    for (int j = 0; j < ng; ++j)
      ora_quant_group_e5m2(x + r * D + (long)j * g, g, &scale[r * ng + j], codes + r * D + (long)j * g);
}

/* x_hat = value(code) * s in binary32. */
void ora_dequant_rows_e5m2(const uint8_t* codes, const float* scale, long rows, int D, int g,
                           float* out) {
  int ng = D / g;
  for (long r = 0; r < rows; ++r)
    for (int d = 0; d < D; ++d)
      out[r * D + d] = (float)ora_e5m2_value(codes[r * D + d]) * scale[r * ng + d / g];
}

/*
 * Channel-axis groups for K ([KVQ-Eng], advice to quantize K per channel):
 * x is `slices` slices of [T][D]; each channel of each block of gt
 * consecutive tokens is one group.  codes: slices x T x D,
 * scale and zero: slices x (T / gt) x D.
 */
void ora_quant_channel_blocks(const uint16_t* x, long slices, long T, int D, int gt, int bits,
                              uint8_t* codes, float* scale, uint8_t* zero) {
  long nb = T / gt;
  uint8_t* tmp = (uint8_t*)malloc((size_t)gt);
  for (long sl = 0; sl < slices; ++sl)
    for (long k = 0; k < nb; ++k)
      for (int d = 0; d < D; ++d) {
        const uint16_t* xg = x + (sl * T + k * gt) * D + d;
        long m = (sl * nb + k) * D + d;
        ora_quant_group_asym(xg, gt, D, bits, &scale[m], &zero[m], tmp);
        for (int j = 0; j < gt; ++j) codes[(sl * T + k * gt + j) * D + d] = tmp[j];
      }
  free(tmp);
}

/* Dequantization: x_hat = (q - z) * s in binary32, or q * s when sym. */
void ora_dequant_rows(const uint8_t* codes, const float* scale, const uint8_t* zero, long rows,
                      int D, int g, int sym, float* out) {
  int ng = D / g;
  for (long r = 0; r < rows; ++r)
    for (int d = 0; d < D; ++d) {
      float s = scale[r * ng + d / g];
      int c = sym ? (int)(int8_t)codes[r * D + d] : (int)codes[r * D + d] - (int)zero[r * ng + d / g];
      out[r * D + d] = (float)c * s;
    }
}

void ora_dequant_channel_blocks(const uint8_t* codes, const float* scale, const uint8_t* zero,
                                long slices, long T, int D, int gt, float* out) {
  long nb = T / gt;
  for (long sl = 0; sl < slices; ++sl)
    for (long t = 0; t < T; ++t)
      for (int d = 0; d < D; ++d) {
        long m = (sl * nb + t / gt) * D + d;
        int c = (int)codes[(sl * T + t) * D + d] - (int)zero[m];
        out[(sl * T + t) * D + d] = (float)c * scale[m];
      }
}

/* ---------------------------------------------------------------------- */
/* Oaken threshold grouping with group-shift outer values                   */
/* ---------------------------------------------------------------------- */

/*
 * One row of D elements, groups of g along the row ([Oaken] §3.1 online
 * stage, §3.2.1 threshold grouping, §3.2.2 group shift).
 * thr = {T_lo_outer, T_lo_inner, T_hi_inner, T_hi_outer}.
 *  - Outer: x > T_hi_outer or x < T_lo_outer (strict, §3.2.1).
 *  - Dense body: asymmetric 4-bit over the group's non-outer elements (inner
 *    and middle share it); outer positions store the zero-point so their
 *    dense value is exactly 0.
 *  - Outer value: shifted delta = x - T_hi_outer (above) or x - T_lo_outer
 *    (below), quantized with a per-group outer scale max|delta| / 31 to a
 *    5-bit magnitude plus a side bit; entries are listed in ascending
 *    channel order as idx | side << 7 | mag << 8.
 * codes: D, scale/zero/oscale: D / g, entries: up to D, *count set.
 */
void ora_oaken_row(const uint16_t* x, int D, int g, const float* thr, uint8_t* codes,
                   float* scale, uint8_t* zero, float* oscale, uint16_t* entries, int* count) {
  float t_lo = thr[0], t_hi = thr[3];
  int ng = D / g;
  int cnt = 0;
  for (int j = 0; j < ng; ++j) {
    float lo = 0.0f, hi = 0.0f, dmax = 0.0f;
    for (int i = j * g; i < (j + 1) * g; ++i) {
      float v = ora_f16_to_f32(x[i]);
      int outer = (v > t_hi) || (v < t_lo);
      if (outer) {
        float delta = v > t_hi ? v - t_hi : v - t_lo;
        if (fabsf(delta) > dmax) dmax = fabsf(delta);
      } else {
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
    }
    float s = (hi - lo) / 15.0f;
    int z = 0;
    if (s != 0.0f) z = clampi((int)rintf(-lo / s), 0, 15);
    float so = dmax / 31.0f;
    scale[j] = s;
    zero[j] = (uint8_t)z;
    oscale[j] = so;
    for (int i = j * g; i < (j + 1) * g; ++i) {
      float v = ora_f16_to_f32(x[i]);
      int above = v > t_hi;
      int outer = above || (v < t_lo);
      if (outer) {
        codes[i] = (uint8_t)z;
        float delta = above ? v - t_hi : v - t_lo;
        int mag = so == 0.0f ? 0 : clampi((int)rintf(fabsf(delta) / so), 0, 31);
        entries[cnt++] = (uint16_t)(i | (above << 7) | (mag << 8));
      } else {
        codes[i] = s == 0.0f ? 0 : (uint8_t)clampi((int)rintf(v / s) + z, 0, 15);
      }
    }
  }
  *count = cnt;
}

void ora_oaken_rows(const uint16_t* x, long rows, int D, int g, const float* thr, uint8_t* codes,
                    float* scale, uint8_t* zero, float* oscale, uint16_t* entries, int* counts) {
  int ng = D / g;
  for (long r = 0; r < rows; ++r)
    ora_oaken_row(x + r * D, D, g, thr, codes + r * D, scale + r * ng, zero + r * ng,
                  oscale + r * ng, entries + r * D, &counts[r]);
}

/* Reconstruction: dense (q - z) * s, outer T_hi + mag * s_out or T_lo - mag * s_out. */
void ora_oaken_dequant_rows(const uint8_t* codes, const float* scale, const uint8_t* zero,
                            const float* oscale, const uint16_t* entries, const int* counts,
                            long rows, int D, int g, const float* thr, float* out) {
  int ng = D / g;
  for (long r = 0; r < rows; ++r) {
    for (int d = 0; d < D; ++d)
      out[r * D + d] = (float)((int)codes[r * D + d] - (int)zero[r * ng + d / g]) * scale[r * ng + d / g];
    for (int e = 0; e < counts[r]; ++e) {
      uint16_t en = entries[r * D + e];
      int idx = en & 127, above = (en >> 7) & 1, mag = (en >> 8) & 31;
      float step = (float)mag * oscale[r * ng + idx / g];
      out[r * D + idx] = above ? thr[3] + step : thr[0] - step;
    }
  }
}

/* ---------------------------------------------------------------------- */
/* Offline calibration: nearest-rank percentiles of fp16 samples           */
/* ---------------------------------------------------------------------- */

/* Order-preserving key of an fp16 bit pattern (negatives below positives). */
static unsigned f16_key(uint16_t b) { return (b & 0x8000) ? (0xFFFFu - b) : (b | 0x8000u); }
static uint16_t f16_from_key(unsigned k) {
  return (uint16_t)(k >= 0x8000u ? (k & 0x7FFFu) : (0xFFFFu - k));
}

/* Accumulate a 65536-bin histogram of the values, indexed by ordered key. */
void ora_hist_f16(const uint16_t* x, long n, uint64_t* hist) {
  for (long i = 0; i < n; ++i) hist[f16_key(x[i])]++;
}

/*
 * Nearest-rank percentile ([Oaken] §3.1 offline stage: thresholds from the
 * sampled KV distribution).  p is given in basis points (2.5% = 250); the
 * result is the value of rank ceil(p * N / 10000) (at least 1).
 */
float ora_hist_percentile(const uint64_t* hist, long p_bp) {
  uint64_t n = 0;
  for (unsigned k = 0; k < 65536u; ++k) n += hist[k];
  uint64_t rank = (n * (uint64_t)p_bp + 9999u) / 10000u;
  if (rank < 1) rank = 1;
  uint64_t acc = 0;
  for (unsigned k = 0; k < 65536u; ++k) {
    acc += hist[k];
    if (acc >= rank) return ora_f16_to_f32(f16_from_key(k));
  }
  return NAN;
}

/* ---------------------------------------------------------------------- */
/* Cocktail chunk precision search and reorder                              */
/* ---------------------------------------------------------------------- */

/*
 * [Cocktail] §3.1.1: cosine similarity of the query embedding with each
 * chunk embedding; T_low = s_min + (s_max - s_min) * alpha,
 * T_high = s_max - (s_max - s_min) * beta; sim > T_high -> 16 (FP16),
 * T_low < sim <= T_high -> 4, sim <= T_low -> 2.
 */
void ora_chunk_bits(const double* qe, const double* ce, long n_chunks, int dim, double alpha,
                    double beta, double* sims, uint8_t* bits) {
  double qq = 0.0;
  for (int d = 0; d < dim; ++d) qq += qe[d] * qe[d];
  double smin = INFINITY, smax = -INFINITY;
  for (long i = 0; i < n_chunks; ++i) {
    double dot = 0.0, cc = 0.0;
    for (int d = 0; d < dim; ++d) {
      dot += qe[d] * ce[i * dim + d];
      cc += ce[i * dim + d] * ce[i * dim + d];
    }
    double s = dot / (sqrt(qq) * sqrt(cc));
    sims[i] = s;
    if (s < smin) smin = s;
    if (s > smax) smax = s;
  }
  double t_low = smin + (smax - smin) * alpha;
  double t_high = smax - (smax - smin) * beta;
  for (long i = 0; i < n_chunks; ++i)
    bits[i] = sims[i] > t_high ? 16 : (sims[i] > t_low ? 4 : 2);
}

/*
 * [Cocktail] §3.1.2: chunks of equal bit-width made contiguous.  Class
 * order FP16, INT4, INT2, stable inside a class.  perm[j] = original chunk
 * id at slot j; seg = {n_fp16, n_int4, n_int2, n_chunks}.  A bit value other
 * than 16 or 4 is placed in the INT2 class.
 */
void ora_reorder(const uint8_t* bits, long batch, long n_chunks, int32_t* perm, int32_t* seg) {
  for (long b = 0; b < batch; ++b) {
    const uint8_t* bb = bits + b * n_chunks;
    int32_t* pp = perm + b * n_chunks;
    long j = 0;
    for (int c = 0; c < 3; ++c) {
      long cnt = 0;
      for (long i = 0; i < n_chunks; ++i) {
        int cls = bb[i] == 16 ? 0 : (bb[i] == 4 ? 1 : 2);
        if (cls == c) {
          pp[j++] = (int32_t)i;
          ++cnt;
        }
      }
      seg[b * 4 + c] = (int32_t)cnt;
    }
    seg[b * 4 + 3] = (int32_t)n_chunks;
  }
}

/* ---------------------------------------------------------------------- */
/* Attention                                                                */
/* ---------------------------------------------------------------------- */

/*
 * Softmax attention of one query over tokens [t0, t1) of one KV head
 * (khat, vhat: [S][D] dequantized values).  Scores q.k * sm_scale (the
 * 1/sqrt(d) scaling in [KVO-LLM] §3.2's score estimate).  Returns the
 * running max m, the sum l of exp(score - m) and the normalized output o.
 * An empty range gives m = -inf, l = 0, o = 0.
 */
void ora_attention_partial(const uint16_t* q, const float* khat, const float* vhat, long t0,
                           long t1, int D, double sm_scale, double* m_out, double* l_out,
                           double* o) {
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (t1 <= t0) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  long n = t1 - t0;
  double* sc = (double*)malloc(sizeof(double) * (size_t)n);
  double m = -INFINITY;
  for (long t = t0; t < t1; ++t) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += (double)ora_f16_to_f32(q[d]) * (double)khat[t * D + d];
    sc[t - t0] = acc * sm_scale;
    if (sc[t - t0] > m) m = sc[t - t0];
  }
  double l = 0.0;
  for (long t = t0; t < t1; ++t) {
    double p = exp(sc[t - t0] - m);
    l += p;
    for (int d = 0; d < D; ++d) o[d] += p * (double)vhat[t * D + d];
  }
  for (int d = 0; d < D; ++d) o[d] /= l;
  *m_out = m;
  *l_out = l;
  free(sc);
}

/*
 * Decode attention for one sequence: q [Hq][D] fp16, khat/vhat
 * [Hkv][S][D].  Query head h reads KV head h / (Hq / Hkv) (consecutive query
 * heads share a KV head under GQA, [KVQ-Eng] cache-size section).
 * out: [Hq][D] in binary64.
 */
void ora_attention(const uint16_t* q, int Hq, int Hkv, int D, const float* khat,
                   const float* vhat, long S, double sm_scale, double* out) {
  int grp = Hq / Hkv;
  for (int h = 0; h < Hq; ++h) {
    int kv = h / grp;
    double m, l;
    ora_attention_partial(q + (long)h * D, khat + (long)kv * S * D, vhat + (long)kv * S * D, 0, S,
                          D, sm_scale, &m, &l, out + (long)h * D);
  }
}

/*
 * Log-sum-exp merge of per-segment partials ([Cocktail] §3.2.3: attention
 * computed per block and the block outputs merged):
 * M = max m_j, L = sum l_j e^(m_j - M), o = sum l_j e^(m_j - M) o_j / L.
 */
void ora_lse_merge(int parts, const double* m, const double* l, const double* o, int D,
                   double* out) {
  double M = -INFINITY;
  for (int j = 0; j < parts; ++j)
    if (m[j] > M) M = m[j];
  double L = 0.0;
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int j = 0; j < parts; ++j) {
    if (l[j] == 0.0) continue;
    double w = l[j] * exp(m[j] - M);
    L += w;
    for (int d = 0; d < D; ++d) out[d] += w * o[(long)j * D + d];
  }
  for (int d = 0; d < D; ++d) out[d] /= L;
}

/* ---------------------------------------------------------------------- */
/* KVO-LLM differential significant-token quantization (DSQ)               */
/* ---------------------------------------------------------------------- */

/*
 * [KVO-LLM] §3.1 (DSQ): tokens are grouped 64 at a time and the top 20 % of
 * each group by attention statistics are the significant tokens, marked in a
 * 1-bit mask; significant ("base") tokens are stored as INT8 with per-channel
 * scales, K of the other tokens as an INT2 difference from the base, V of the
 * other tokens as group-wise INT2.  The page's learnable scale compensation
 * is left out.
 *
 * Readings (the page gives the steps, not the arithmetic):
 *  - The statistic is an input: one binary32 importance score per token.
 *    Significant = the n_sig largest scores of the group (the page's 20 % of
 *    64 is 12.8; callers use n_sig = 13).  Scores are ordered by their bit
 *    patterns as a total order (-0 below +0, NaNs at the ends by sign), ties
 *    by the lower token index, so exactly n_sig tokens are chosen.
 *  - Significant K and V: symmetric INT8 per channel over the group's
 *    significant tokens, s_d = max|x| / 127, code = clamp(rne(x / s_d),
 *    -128, 127) (the INT8 listing's quantizer, applied per channel).
 *  - K base: one row per group, the mean of the dequantized significant K
 *    rows, base_d = fl(fl(sum_i fl(s_d * c_id)) / n_sig), summed in token
 *    order, so that the page's "difference from the base" has one base.
 *  - K difference of a non-significant token: delta = fl(k - base) in
 *    binary32, quantized as asymmetric INT2 in groups of g2 channels (the
 *    page fixes INT2, not its scale), exactly like a V group.
 *  - Rows are kept in token order within each class (slot i of a class is
 *    its i-th token); the mask restores positions.
 */
static unsigned dsq_key(float x) {
  uint32_t b;
  memcpy(&b, &x, 4);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

/* Asymmetric b-bit quantization of n binary32 values (same rule as
 * ora_quant_group_asym, for inputs that are not fp16). */
static void quant_group_asym_f32(const float* x, long n, int bits, float* s_out, uint8_t* z_out,
                                 uint8_t* q) {
  int qmax = (1 << bits) - 1;
  float lo = 0.0f, hi = 0.0f;
  for (long i = 0; i < n; ++i) {
    if (x[i] < lo) lo = x[i];
    if (x[i] > hi) hi = x[i];
  }
  float s = (hi - lo) / (float)qmax;
  *s_out = s;
  if (s == 0.0f) {
    *z_out = 0;
    for (long i = 0; i < n; ++i) q[i] = 0;
    return;
  }
  int z = clampi((int)rintf(-lo / s), 0, qmax);
  *z_out = (uint8_t)z;
  for (long i = 0; i < n; ++i) q[i] = (uint8_t)clampi((int)rintf(x[i] / s) + z, 0, qmax);
}

/*
 * One group of T = 64 tokens (k, v: [T][D] fp16; score: [T]).
 * Outputs (n_ns = T - n_sig):
 *   mask:   bit t set when token t is significant
 *   ksig, vsig [n_sig][D] int8 codes, kscale, vscale [D] channel scales
 *   base   [D] the K base row
 *   kc2, vc2 [n_ns][D] INT2 codes (one per byte), ks2, vs2 [n_ns][D/g2]
 *   scales, kz2, vz2 [n_ns][D/g2] zero-points.
 */
void ora_dsq_group(const uint16_t* k, const uint16_t* v, const float* score, int T, int D, int n_sig,
                   int g2, uint64_t* mask, int8_t* ksig, float* kscale, int8_t* vsig, float* vscale,
                   float* base, uint8_t* kc2, float* ks2, uint8_t* kz2, uint8_t* vc2, float* vs2,
                   uint8_t* vz2) {
  /* 1. significant tokens: rank by score, ties to the lower index */
  int sig_tok[64], ns_tok[64], n_s = 0, n_n = 0;
  uint64_t m = 0;
  for (int t = 0; t < T; ++t) {
    int rank = 0;
    for (int u = 0; u < T; ++u) {
      unsigned ku = dsq_key(score[u]), kt = dsq_key(score[t]);
      if (ku > kt || (ku == kt && u < t)) ++rank;
    }
    if (rank < n_sig) m |= (uint64_t)1 << t;
  }
  for (int t = 0; t < T; ++t) {
    if ((m >> t) & 1u) sig_tok[n_s++] = t;
    else ns_tok[n_n++] = t;
  }
  *mask = m;
  /* 2. significant K and V: INT8 per channel over the significant tokens */
  uint16_t col[64];
  int8_t qc[64];
  for (int d = 0; d < D; ++d) {
    for (int i = 0; i < n_s; ++i) col[i] = k[(long)sig_tok[i] * D + d];
    ora_quant_group_sym8(col, n_s, 1, &kscale[d], qc);
    for (int i = 0; i < n_s; ++i) ksig[(long)i * D + d] = qc[i];
    for (int i = 0; i < n_s; ++i) col[i] = v[(long)sig_tok[i] * D + d];
    ora_quant_group_sym8(col, n_s, 1, &vscale[d], qc);
    for (int i = 0; i < n_s; ++i) vsig[(long)i * D + d] = qc[i];
  }
  /* 3. K base: mean of the dequantized significant rows */
  for (int d = 0; d < D; ++d) {
    float acc = 0.0f;
    for (int i = 0; i < n_s; ++i) acc = acc + kscale[d] * (float)ksig[(long)i * D + d];
    base[d] = acc / (float)n_s;
  }
  /* 4. the other tokens: K difference and V, INT2 groups of g2 channels */
  int ng = D / g2;
  float dx[128];
  for (int j = 0; j < n_n; ++j) {
    const uint16_t* kr = k + (long)ns_tok[j] * D;
    const uint16_t* vr = v + (long)ns_tok[j] * D;
    for (int d = 0; d < D; ++d) dx[d] = ora_f16_to_f32(kr[d]) - base[d];
    for (int gi = 0; gi < ng; ++gi) {
      quant_group_asym_f32(dx + (long)gi * g2, g2, 2, &ks2[(long)j * ng + gi], &kz2[(long)j * ng + gi],
                           kc2 + (long)j * D + (long)gi * g2);
      ora_quant_group_asym(vr + (long)gi * g2, g2, 1, 2, &vs2[(long)j * ng + gi], &vz2[(long)j * ng + gi],
                           vc2 + (long)j * D + (long)gi * g2);
    }
  }
}

/*
 * Dequantized rows of one DSQ group in token order (khat, vhat: [T][D]):
 * significant tokens s_d * c, others base + (c - z) * s (K) and (c - z) * s
 * (V), each one binary32 operation per step.
 */
void ora_dsq_dequant_group(uint64_t mask, int T, int D, int g2, const int8_t* ksig, const float* kscale,
                           const int8_t* vsig, const float* vscale, const float* base,
                           const uint8_t* kc2, const float* ks2, const uint8_t* kz2, const uint8_t* vc2,
                           const float* vs2, const uint8_t* vz2, float* khat, float* vhat) {
  int ng = D / g2, i = 0, j = 0;
  for (int t = 0; t < T; ++t) {
    float* kr = khat + (long)t * D;
    float* vr = vhat + (long)t * D;
    if ((mask >> t) & 1u) {
      for (int d = 0; d < D; ++d) {
        kr[d] = kscale[d] * (float)ksig[(long)i * D + d];
        vr[d] = vscale[d] * (float)vsig[(long)i * D + d];
      }
      ++i;
    } else {
      for (int d = 0; d < D; ++d) {
        int gi = d / g2;
        float kd = (float)((int)kc2[(long)j * D + d] - (int)kz2[(long)j * ng + gi]) * ks2[(long)j * ng + gi];
        kr[d] = base[d] + kd;
        vr[d] = (float)((int)vc2[(long)j * D + d] - (int)vz2[(long)j * ng + gi]) * vs2[(long)j * ng + gi];
      }
      ++j;
    }
  }
}
