// Quantize-append kernels.
//
// Quantizer (per group, binary32, round half to even):
//   asymmetric ([Oaken page "大模型KV缓存量化技术：原理、优化与实践" §2.1 scale
//   formula; Cocktail page §3.2.2 code = round(x / s) + z]):
//     lo = min(0, min x), hi = max(0, max x), s = (hi - lo) / (2^b - 1),
//     z = clamp(rne(-lo / s)), q = clamp(rne(x / s) + z); all-zero group -> 0, 0, 0
//   symmetric INT8 ([KV-cache quantization engineering page, INT8 listing]):
//     s = max|x| / 127, q = clamp(rne(x / s), -128, 127)
//   FP8 E4M3 (the same page's FP8 item): s = max|x| / 448, q = E4M3 code of
//     x / s (nearest, ties to even, saturating at 448; see f8_pair)
// Every quotient is the IEEE binary32 one (the build keeps correctly rounded
// fp32 division and denormals; where a kernel avoids the divide, by the
// corrected constant division or the rounding check below, it reaches the
// same value), so codes, scales and zero-points are bit-identical to any
// other binary32 evaluation of these formulas.
//
// Thread layout of the token-axis, Oaken prefill and chunk-mixed INT4/INT2
// kernels: 8 lanes per 128-channel row, each lane holds 16 consecutive
// channels (two 16-byte loads); a group of GE channels is GE / 16 adjacent
// lanes, reduced with lane exchanges.  The one-token Oaken append, the
// streaming chunk kernels, the DSQ rows and the FP16 copies keep 16 lanes
// of 8 channels (quant8).
#include <algorithm>

#include "kvq_dev.h"

namespace kvq {
namespace {

// FP8 codes of two binary32 quotients, by the hardware conversion to the
// OCP formats (E4M3: no infinities, largest finite 448; E5M2: largest finite
// 57344): the nearest value, ties to the even mantissa, sign kept.  Each
// quotient is first clamped to the largest finite magnitude, so anything at
// or beyond it gives that magnitude (saturation) whatever the conversion does
// with overflows.  The cache never holds an infinity or NaN, so the codes of
// non-finite inputs are left unspecified.  Returns the two bytes in bits 0-15.
template <int F8>
__device__ __forceinline__ uint32_t f8_pair(float y0, float y1) {
  constexpr float kTop = F8 == 1 ? 448.0f : 57344.0f;
  y0 = __builtin_amdgcn_fmed3f(y0, -kTop, kTop);
  y1 = __builtin_amdgcn_fmed3f(y1, -kTop, kTop);
  if constexpr (F8 == 1) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false) & 0xFFFFu;
  else return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false) & 0xFFFFu;
}

// Rounded quotients without a division per element.  Every code below is
// rne(fl(x / s)) for one per-group s > 0: the correctly rounded binary32
// quotient, then rounded to an integer (ties to even).  With r = 1/s to
// within |r s - 1| <= 2^-22 (the hardware reciprocal, good to about 2^-23,
// after one Newton step), y = fl(x r) differs from fl(x / s) by less than
// |y| 2^-21 (the reciprocal's error plus the two roundings).  So where y lies
// farther than |y| 2^-19 from every half-integer, rne(y) = rne(fl(x / s));
// elsewhere (near-ties, exact ties, and anything not finite) `near` is set and
// the caller divides.  Every caller knows a power of two M >= |y| (M = 2^bits
// for the codes: |x / s| <= 2^bits - 1 up to rounding; 32 for the Oaken
// magnitudes), so the test is |y - rne(y)| < 0.5 - M 2^-19, exact (y - rne(y)
// is exact by Sterbenz, and both sides are representable).
__device__ __forceinline__ float recip_refined(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  return s != 0.0f ? fmaf(fmaf(-s, r0, 1.0f), r0, r0) : 0.0f;  // s = 0: every y is 0
}
template <int M>
__device__ __forceinline__ float rne_quot(float x, float r, bool& near) {
#pragma clang fp contract(off)
  constexpr float kAccept = 0.5f - (float)M * 0x1p-19f;
  const float y = x * r;
  const float n = rintf(y);
  near |= !(fabsf(y - n) < kAccept);
  return n;
}
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0ull; }

// The IEEE quotient fl(x / D) for x >= 0 and a constant D without a division:
// q0 = fl(x c) with c = fl(1/D), the residual x - q0 D exact by a fused
// multiply-add, then q0 + r c rounded once (Markstein's correction step with
// a correctly rounded reciprocal).  Checked on the CPU over every binade
// where a step can leave the normal range and one where none does (the rest
// are scaled copies), for the divisors used below.  x infinite or NaN is
// passed through, as the division would give.
template <int D>
__device__ __forceinline__ float div_const(float x) {
#pragma clang fp contract(off)
  constexpr float c = 1.0f / (float)D;
  const float q0 = x * c;
  const float q = fmaf(fmaf(-q0, (float)D, x), c, q0);
  return __builtin_isfinite(x) ? q : q0;
}

// rne_quot over a lane's N values with one test: the largest |y - rne(y)|
// against the same bound, so a lane with any near value divides all of them
// (each division gives the code the fast path would where that one is not
// near; a NaN y gives NaN either way).
template <int M, int N>
__device__ __forceinline__ bool rne_quot_lane(const float (&x)[N], float r, float (&n)[N]) {
  constexpr float kAccept = 0.5f - (float)M * 0x1p-19f;
  float dev = 0.0f;
#pragma unroll
  for (int k = 0; k < N; ++k) {
#pragma clang fp contract(off)
    const float y = x[k] * r;
    n[k] = rintf(y);
    dev = fmaxf(dev, fabsf(y - n[k]));
  }
  return !(dev < kAccept);
}

// Asymmetric codes clamp(rne(fl(x / s)) + z, 0, M - 1) of a lane's N values
// (M = 2^bits), z = clamp(rne(fl(-lo / s)), 0, M - 1) already formed as the
// exact float zf.  Each code comes from t = fl(x r + zf), one rounding: with
// |x / s| < M and 0 <= zf < M, t differs from fl(x / s) + zf by less than
// M 2^-21 (the reciprocal's error, the quotient's rounding and the sum's), so
// where every |t - rne(t)| of the lane (exact, by Sterbenz) stays below
// 0.5 - M 2^-19, rne(t) is the integer nearest fl(x / s) + zf, which is
// rne(fl(x / s)) + zf (zf an integer, and no tie).  Otherwise (near-ties,
// exact ties, anything not finite) the lane divides.  A NaN t gives NaN
// either way.
template <int M, int N>
__device__ __forceinline__ void asym_codes(const float (&x)[N], float s, float r, float zf, float (&q)[N]) {
  constexpr float kAccept = 0.5f - (float)M * 0x1p-19f;
  float dev = 0.0f;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float t = fmaf(x[k], r, zf);
    q[k] = rintf(t);
    dev = fmaxf(dev, fabsf(t - q[k]));
  }
  const bool near = !(dev < kAccept);
  if (wave_any(near) && near) {
#pragma unroll
    for (int k = 0; k < N; ++k) q[k] = rintf(x[k] / s) + zf;
  }
#pragma unroll
  for (int k = 0; k < N; ++k) q[k] = __builtin_amdgcn_fmed3f(q[k], 0.0f, (float)(M - 1));
}

template <int BITS, bool SYM, int GE>
__device__ __forceinline__ void quant8(const float (&x)[8], unsigned valid, uint32_t& plo,
                                       uint32_t& phi, float& s, int& z) {
  constexpr int LG = GE / 8;
  plo = 0;
  phi = 0;
  if constexpr (SYM) {
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
    amax = max_lanes<1, LG>(amax);
    s = div_const<127>(amax);
    z = 0;
    const float r = recip_refined(s);  // s = 0: all codes 0
    float n[8];
    const bool near = rne_quot_lane<128>(x, r, n);
    if (wave_any(near) && near) {
#pragma unroll
      for (int k = 0; k < 8; ++k) n[k] = rintf(x[k] / s);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t byte = (uint32_t)((int)__builtin_amdgcn_fmed3f(n[k], -128.0f, 127.0f) & 0xFF);
      if (k < 4) plo |= byte << (8 * k);
      else phi |= byte << (8 * (k - 4));
    }
  } else {
    constexpr float QMAX = (float)((1 << BITS) - 1);
    float lo = 0.0f, hi = 0.0f;
    float xm[8];  // invalid (excluded) values count as 0: they neither widen the range nor divide
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      xm[k] = ((valid >> k) & 1u) ? x[k] : 0.0f;
      lo = fminf(lo, xm[k]);
      hi = fmaxf(hi, xm[k]);
    }
    lo = min_lanes<1, LG>(lo);
    hi = max_lanes<1, LG>(hi);
    s = div_const<(1 << BITS) - 1>(hi - lo);
    const float r = recip_refined(s);  // s = 0: z = 0 and all codes 0
    float n[8];
    bool near = rne_quot_lane<(1 << BITS)>(xm, r, n);
    float zf = rne_quot<(1 << BITS)>(-lo, r, near);
    if (wave_any(near) && near) {
      zf = rintf(-lo / s);
#pragma unroll
      for (int k = 0; k < 8; ++k) n[k] = rintf(xm[k] / s);
    }
    zf = __builtin_amdgcn_fmed3f(zf, 0.0f, QMAX);
    z = (int)zf;
    uint64_t packed = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // an excluded value (xm = 0, so n = 0) takes the zero-point: it decodes to 0
      const float q = __builtin_amdgcn_fmed3f(n[k] + zf, 0.0f, QMAX);
      packed |= (uint64_t)(uint32_t)q << (BITS * k);
    }
    plo = (uint32_t)packed;
    phi = (uint32_t)(packed >> 32);
  }
}

typedef unsigned u4q_t __attribute__((ext_vector_type(4)));
typedef unsigned u2q_t __attribute__((ext_vector_type(2)));

// 16 bytes of input (8 fp16 values), streamed
__device__ __forceinline__ uint4 ld_row8(const uint16_t* p) {
  const u4q_t t = ld_nt<u4q_t>(p);
  const unsigned a = t[0], b = t[1], c = t[2], d = t[3];
  return make_uint4(a, b, c, d);
}
__device__ __forceinline__ void st_u4(uint8_t* p, uint4 v) { st_nt<u4q_t>(p, u4q_t{v.x, v.y, v.z, v.w}); }

__device__ __forceinline__ void unpack8(const uint4 raw, float (&v)[8]) {
  v[0] = lo_h2f(raw.x); v[1] = hi_h2f(raw.x);
  v[2] = lo_h2f(raw.y); v[3] = hi_h2f(raw.y);
  v[4] = lo_h2f(raw.z); v[5] = hi_h2f(raw.z);
  v[6] = lo_h2f(raw.w); v[7] = hi_h2f(raw.w);
}

template <int BITS>
__device__ __forceinline__ void store_codes8(uint8_t* row, int slot, uint32_t plo, uint32_t phi) {
  if constexpr (BITS == 8) {
    st_nt<u2q_t>(row + slot * 8, u2q_t{plo, phi});
  } else if constexpr (BITS == 4) {
    st_nt<uint32_t>(row + slot * 4, plo);
  } else {
    st_nt<uint16_t>(row + slot * 2, (uint16_t)plo);
  }
}

// Code v (0..7) of a lane's naturally packed codes.
template <int BITS>
__device__ __forceinline__ unsigned code_at(uint32_t plo, uint32_t phi, int v) {
  if constexpr (BITS == 8) return ((v < 4 ? plo : phi) >> (8 * (v & 3))) & 0xFFu;
  else return (plo >> (BITS * v)) & ((1u << BITS) - 1u);
}

// Slot of the K row that holds the 8 channels 8 li .. 8 li + 7 (kvq.h: slot
// 4 q + s holds channels 32 s + 8 q + v).
__device__ __forceinline__ int k_slot(int li) { return 4 * (li & 3) + (li >> 2); }

// Store a lane's 8 codes (channels 8 li + v) into a packed row.
//  K layout: the lane's codes form one slot.
//  V layout: column word n holds channels n + 16 j; the row's 16 lanes
//  exchange codes through `lrow` (128 entries of this row, wave-local).
template <int BITS, bool VL>
__device__ __forceinline__ void store_row_codes(uint8_t* row, int li, uint32_t plo, uint32_t phi,
                                                uint16_t* lrow) {
  if constexpr (!VL) {
    store_codes8<BITS>(row, k_slot(li), plo, phi);
  } else {
#pragma unroll
    for (int v = 0; v < 8; ++v) lrow[8 * li + v] = (uint16_t)code_at<BITS>(plo, phi, v);
    wave_lds_sync();
    uint64_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= (uint64_t)lrow[li + 16 * j] << (BITS * j);
    wave_lds_sync();
    store_codes8<BITS>(row, li, (uint32_t)w, (uint32_t)(w >> 32));
  }
}

// fp16 rows of the chunk-mixed FP16 pool.  K layout: slot 4 q + s (16 bytes)
// holds channels 32 s + 8 q + (0, 4, 1, 5, 2, 6, 3, 7); V layout: word n (16
// bytes) holds channels n + 16 j.
template <bool VL>
__device__ __forceinline__ void store_row_f16(uint8_t* row, int li, uint4 raw, uint16_t* lrow) {
  if constexpr (!VL) {
    uint4 o;
    o.x = __builtin_amdgcn_perm(raw.z, raw.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(raw.z, raw.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(raw.w, raw.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(raw.w, raw.y, 0x07060302u);
    st_u4(row + k_slot(li) * 16, o);
  } else {
    const uint32_t d[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int v = 0; v < 8; ++v) lrow[8 * li + v] = (uint16_t)(d[v >> 1] >> (16 * (v & 1)));
    wave_lds_sync();
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)lrow[li + 32 * k] | ((uint32_t)lrow[li + 32 * k + 16] << 16);
    wave_lds_sync();
    st_u4(row + li * 16, make_uint4(w[0], w[1], w[2], w[3]));
  }
}

// ---------------------------------------------------------------------------
// Uniform cache, token-axis groups.  x: [B][H][t_new][128], rows in that order.
// VL selects the V row layout.
// One token row per 16 lanes; lrow: the row's wave-local exchange area (V).
// Where token rows live: contiguous [B][H][S] rows, or pages of ptok rows per
// head, [npages][H][ptok], token t of sequence b in page pages[b][t / ptok].
struct PageMap {
  const int* pages;  // null: contiguous
  int ptok, npages;
};

// Unsigned division by a divisor fixed for a launch, n < 2^32, as one high
// multiply, an add and shifts (the round-up multiplier construction of
// Granlund and Montgomery): s = ceil(log2 d), m = floor(2^32 (2^s - d) / d)
// + 1, q = (t + ((n - t) >> 1)) >> (s - 1) with t = mulhi(n, m); d = 1: q = n.
// It replaces the 64-bit divides of the row index, which the compiler
// expands into some 80 instructions per lane.
struct FastDiv {
  uint32_t d, m, s;
};
FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  if (f.s == 0) return n;
  const uint32_t t = __umulhi(n, f.m);
  return (t + ((n - t) >> 1)) >> (f.s - 1);
}

// Codes of one lane's 16 values (channels 16 li .. 16 li + 15) of a token
// row, groups of GE channels over GE / 16 lanes: the quantizer of quant8 on
// twice the values per lane (the same groups, so the same scales and codes),
// codes returned as integers (two's complement bytes for symmetric INT8).
// F8: 0 integer codes, 1 FP8 E4M3, 2 FP8 E5M2.
template <int BITS, bool SYM, int GE, int F8 = 0>
__device__ __forceinline__ void quant16(const float (&x)[16], unsigned (&c)[16], float& s, int& z) {
  constexpr int LG = GE / 16;
  if constexpr (F8 != 0) {
    static_assert(BITS == 8, "FP8 codes are bytes");
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(x[k]));
    amax = max_lanes<1, LG>(amax);
    s = amax / (F8 == 1 ? 448.0f : 57344.0f);  // (the corrected step misrounds some of these quotients)
    z = 0;
#pragma unroll
    for (int k = 0; k < 16; k += 2) {
      const uint32_t w = f8_pair<F8>(x[k] / s, x[k + 1] / s);
      c[k] = s != 0.0f ? (w & 0xFFu) : 0u;
      c[k + 1] = s != 0.0f ? (w >> 8) : 0u;
    }
  } else if constexpr (SYM) {
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(x[k]));
    amax = max_lanes<1, LG>(amax);
    s = div_const<127>(amax);
    z = 0;
    const float r = recip_refined(s);  // s = 0: all codes 0
    float n[16];
    const bool near = rne_quot_lane<128>(x, r, n);
    if (wave_any(near) && near) {
#pragma unroll
      for (int k = 0; k < 16; ++k) n[k] = rintf(x[k] / s);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) c[k] = (unsigned)((int)__builtin_amdgcn_fmed3f(n[k], -128.0f, 127.0f) & 0xFF);
  } else {
    constexpr float QMAX = (float)((1 << BITS) - 1);
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      lo = fminf(lo, x[k]);
      hi = fmaxf(hi, x[k]);
    }
    lo = min_lanes<1, LG>(lo);
    hi = max_lanes<1, LG>(hi);
    s = div_const<(1 << BITS) - 1>(hi - lo);
    const float r = recip_refined(s);  // s = 0: z = 0 and all codes 0
    bool near = false;
    float zf = rne_quot<(1 << BITS)>(-lo, r, near);
    if (wave_any(near) && near) zf = rintf(-lo / s);
    zf = __builtin_amdgcn_fmed3f(zf, 0.0f, QMAX);
    z = (int)zf;
    float q[16];
    asym_codes<(1 << BITS)>(x, s, r, zf, q);
#pragma unroll
    for (int k = 0; k < 16; ++k) c[k] = (unsigned)q[k];
  }
}

// Eight codes of BITS bits, code k at bits BITS k (lo: the first 32 bits).
template <int BITS>
__device__ __forceinline__ void pack8(const unsigned* c, uint32_t& lo, uint32_t& hi) {
  lo = 0;
  hi = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (BITS * k < 32) lo |= c[k] << (BITS * k);
    else hi |= c[k] << (BITS * k - 32);
  }
}

// Store a lane's 16 codes (channels 16 li + k) into a packed row.
//  K layout: the lane's two 8-channel slots, k_slot(2 li) and k_slot(2 li + 1).
//  V layout: word n holds channels n + 16 j, so the lane's code k is code j
//  = li of word k; the row's 8 lanes exchange codes through `lc` (128 bytes
//  of this row, wave-local): code k to byte 8 k + li, then lane li reads
//  bytes 16 li .. 16 li + 15, words 2 li and 2 li + 1.
template <int BITS, bool VL>
__device__ __forceinline__ void store_row_codes16(uint8_t* row, int li, const unsigned (&c)[16], uint8_t* lc) {
  if constexpr (!VL) {
    uint32_t lo, hi;
    pack8<BITS>(c, lo, hi);
    store_codes8<BITS>(row, k_slot(2 * li), lo, hi);
    pack8<BITS>(c + 8, lo, hi);
    store_codes8<BITS>(row, k_slot(2 * li + 1), lo, hi);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) lc[8 * k + li] = (uint8_t)c[k];
    wave_lds_sync();
    const uint4 by = *reinterpret_cast<const uint4*>(lc + 16 * li);
    wave_lds_sync();
    if constexpr (BITS == 8) {
      st_u4(row + 16 * li, by);
    } else if constexpr (BITS == 4) {
      // bytes b0..b3 (each < 16) -> b0 | b1 << 4 | b2 << 8 | b3 << 12
      auto nib4 = [](uint32_t d) {
        const uint32_t t = d | (d >> 4);
        return (t & 0xFFu) | ((t >> 8) & 0xFF00u);
      };
      st_nt<u2q_t>(row + 8 * li, u2q_t{nib4(by.x) | nib4(by.y) << 16, nib4(by.z) | nib4(by.w) << 16});
    } else {
      // bytes b0..b3 (each < 4) -> b0 | b1 << 2 | b2 << 4 | b3 << 6
      auto crumb4 = [](uint32_t d) {
        const uint32_t t = d | (d >> 6);
        return (t & 0xFu) | ((t >> 12) & 0xF0u);
      };
      st_nt<uint32_t>(row + 4 * li, crumb4(by.x) | crumb4(by.y) << 8 | crumb4(by.z) << 16 | crumb4(by.w) << 24);
    }
  }
}

// rows = batch * H * t_new < 2^31 (checked by the caller), so the grid-strided
// row index never wraps.  Eight lanes per row, 16 channels per lane.
template <int BITS, bool SYM, int GE, bool VL, int F8 = 0>
__device__ __forceinline__ void quant_token_row(uint32_t row, const uint16_t* __restrict__ x, FastDiv ft,
                                                FastDiv fh, int S, const int* __restrict__ pos, uint32_t rows,
                                                uint8_t* __restrict__ codes, float* __restrict__ scale,
                                                uint8_t* __restrict__ zero, unsigned* __restrict__ status,
                                                uint8_t* lc, const PageMap& pm) {
  constexpr int NG = kD / GE, LG = GE / 16, RB = kD * BITS / 8;
  const int li = threadIdx.x & 7;
  if (row >= rows) return;  // all 8 lanes of a row leave together
  const uint32_t bh32 = fdiv(row, ft);
  const int t = (int)(row - bh32 * ft.d);
  const long long bh = bh32;
  const uint32_t b32 = fdiv(bh32, fh);
  const int b = (int)b32, H = (int)fh.d;
  const int p = pos[b];
  if (p < 0 || p + t >= S) {
    if (li == 0) set_flag(status, kFlagPosRange);
    return;
  }
  long long dst = bh * S + p + t;
  if (pm.pages) {
    const int tok = p + t;
    const int pg = pm.pages[(long long)b * (S / pm.ptok) + tok / pm.ptok];
    if (pg < 0 || pg >= pm.npages) {
      if (li == 0) set_flag(status, kFlagPageRange);
      return;
    }
    dst = ((long long)pg * H + (bh32 - b32 * fh.d)) * pm.ptok + tok % pm.ptok;
  }
  const uint16_t* src = x + (long long)row * kD + li * 16;
  float v[16];
  {
    float h[8];
    unpack8(ld_row8(src), h);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = h[k];
    unpack8(ld_row8(src + 8), h);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[8 + k] = h[k];
  }
  unsigned c[16];
  float s;
  int z;
  quant16<BITS, SYM, GE, F8>(v, c, s, z);
  store_row_codes16<BITS, VL>(codes + dst * RB, li, c, lc);
  if (li % LG == 0) {
    scale[dst * NG + li / LG] = s;
    if constexpr (!SYM && !F8) zero[dst * NG + li / LG] = (uint8_t)z;
  }
}

template <int BITS, bool SYM, int GE, bool VL, int F8>
__global__ __launch_bounds__(256) void k_quant_token(const uint16_t* __restrict__ x, FastDiv ft, FastDiv fh,
                                                     int S, const int* __restrict__ pos,
                                                     uint32_t rows, uint8_t* __restrict__ codes,
                                                     float* __restrict__ scale,
                                                     uint8_t* __restrict__ zero,
                                                     unsigned* __restrict__ status, PageMap pm) {
  __shared__ __align__(16) uint8_t lcode[VL ? 32 : 1][128];
  // blocks of 32 rows, grid-strided: a bounded grid keeps the dispatch cost low
  for (uint32_t r0 = blockIdx.x * 32u; r0 < rows; r0 += gridDim.x * 32u)
    quant_token_row<BITS, SYM, GE, VL, F8>(r0 + (threadIdx.x >> 3), x, ft, fh, S, pos, rows, codes, scale,
                                           zero, status, lcode[VL ? (threadIdx.x >> 3) : 0], pm);
}

// K and V of the same token-axis format in one launch: blockIdx.y selects the
// tensor (0: K rows, 1: V rows), so a decode-step append costs one launch.
template <int BITS, bool SYM, int GE, int F8>
__global__ __launch_bounds__(256) void k_quant_token_kv(const uint16_t* __restrict__ xk,
                                                        const uint16_t* __restrict__ xv, FastDiv ft, FastDiv fh,
                                                        int S, const int* __restrict__ pos, uint32_t rows,
                                                        TensorArgs tk, TensorArgs tv,
                                                        unsigned* __restrict__ status, PageMap pm) {
  __shared__ __align__(16) uint8_t lcode[32][128];
  for (uint32_t r0 = blockIdx.x * 32u; r0 < rows; r0 += gridDim.x * 32u) {
    const uint32_t row = r0 + (threadIdx.x >> 3);
    if (blockIdx.y == 0)
      quant_token_row<BITS, SYM, GE, false, F8>(row, xk, ft, fh, S, pos, rows, tk.codes, tk.scale, tk.zero,
                                                status, lcode[0], pm);
    else
      quant_token_row<BITS, SYM, GE, true, F8>(row, xv, ft, fh, S, pos, rows, tv.codes, tv.scale, tv.zero,
                                               status, lcode[threadIdx.x >> 3], pm);
  }
}

// ---------------------------------------------------------------------------
// Uniform cache, channel-axis groups of 64 tokens (K per channel, the KV-cache
// quantization engineering page's advice), appended as a stream: a block of
// 64 tokens is quantized once all its tokens are present; until then its
// tokens wait in the fp16 residual tail (one block per (b, h), rows in the
// fp16 K layout of store_row_f16).  An append of tokens [p, p + t_new) of a
// sequence therefore continues that sequence (p = its current length): the
// tail holds its tokens 64 floor(p / 64) .. p - 1.
//
// k_quant_channel: one workgroup per (block touched by the append, b h);
// block k0 = 64 floor(p / 64) + 64 blockIdx.x is quantized when it is
// complete after the append, its rows below p read from the tail, the others
// from the input.  The block's rows are staged in LDS as fp16; each
// channel's range is reduced over four 16-row quarters, then each thread
// codes 8 channels of 4 rows (their scales read once).  Codes in the K row
// layout.  k_channel_tail (launched after
// it on the same stream, so the tail is read before it is overwritten) then
// moves the new tokens of the block left incomplete into the tail.

// 8 channels 8 li .. 8 li + 7 of an fp16 K-layout row, in channel order
// (inverse of store_row_f16's K permutation).
__device__ __forceinline__ uint4 ld_row8_k16(const uint8_t* row, int li) {
  const uint4 t = ld_row8(reinterpret_cast<const uint16_t*>(row + k_slot(li) * 16));
  uint4 o;
  o.x = __builtin_amdgcn_perm(t.y, t.x, 0x05040100u);
  o.y = __builtin_amdgcn_perm(t.w, t.z, 0x05040100u);
  o.z = __builtin_amdgcn_perm(t.y, t.x, 0x07060302u);
  o.w = __builtin_amdgcn_perm(t.w, t.z, 0x07060302u);
  return o;
}

template <int BITS>
__global__ __launch_bounds__(256) void k_quant_channel(const uint16_t* __restrict__ x, int t_new,
                                                       int H, int S, const int* __restrict__ pos,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scale,
                                                       uint8_t* __restrict__ zero,
                                                       const uint8_t* __restrict__ tail,
                                                       unsigned* __restrict__ status, PageMap pm) {
  constexpr int QMAX = (1 << BITS) - 1, RB = kD * BITS / 8;
  const long long bh = blockIdx.y;
  const int b = (int)(bh / H);
  const int p = pos[b];
  if (p < 0 || p + t_new > S) {
    if (threadIdx.x == 0 && blockIdx.x == 0) set_flag(status, kFlagPosRange);
    return;
  }
  const int k0 = (p & ~63) + 64 * (int)blockIdx.x;
  if (k0 + 64 > p + t_new) return;  // incomplete after this append (or past it)
  // the block's first code row (its scales: row / 64): contiguous, or in its
  // page (a block never straddles a page; an entry outside the pool skips
  // the block and flags; the fp16 tail is per sequence)
  long long row0 = bh * S + k0;
  if (pm.pages) {
    const int pg = pm.pages[(long long)b * (S / pm.ptok) + k0 / pm.ptok];
    if (pg < 0 || pg >= pm.npages) {
      if (threadIdx.x == 0) set_flag(status, kFlagPageRange);
      return;
    }
    row0 = ((long long)pg * H + bh % H) * pm.ptok + k0 % pm.ptok;
  }
  // the block's 64 fp16 rows (16-byte aligned rows: 16-byte writes and reads)
  __shared__ __align__(16) uint16_t tile[64][kD + 8];
  __shared__ float lo_sh[4][kD], hi_sh[4][kD];
  __shared__ __align__(16) float s_sh[kD], r_sh[kD], z_sh[kD];
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int r = pass * 16 + (threadIdx.x >> 4), li = threadIdx.x & 15;
    const int t = k0 + r;
    // the input row is always read (row max(t, p) is in the input), so the
    // passes' loads issue together; a row still in the tail replaces it
    uint4 raw = ld_row8(x + (bh * t_new + (max(t, p) - p)) * kD + li * 8);
    if (t < p) raw = ld_row8_k16(tail + (bh * 64 + r) * 256, li);
    *reinterpret_cast<uint4*>(&tile[r][li * 8]) = raw;
  }
  __syncthreads();
  {
    // channels 2 cp and 2 cp + 1 over rows 16 qr .. 16 qr + 15
    const int cp = threadIdx.x & 63, qr = threadIdx.x >> 6;
    float lo0 = 0.0f, hi0 = 0.0f, lo1 = 0.0f, hi1 = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(&tile[16 * qr + r][2 * cp]);
      const float v0 = lo_h2f(w), v1 = hi_h2f(w);
      lo0 = fminf(lo0, v0);
      hi0 = fmaxf(hi0, v0);
      lo1 = fminf(lo1, v1);
      hi1 = fmaxf(hi1, v1);
    }
    lo_sh[qr][2 * cp] = lo0;
    hi_sh[qr][2 * cp] = hi0;
    lo_sh[qr][2 * cp + 1] = lo1;
    hi_sh[qr][2 * cp + 1] = hi1;
  }
  __syncthreads();
  if (threadIdx.x < kD) {
    const int c = threadIdx.x;
    const float lo = fminf(fminf(lo_sh[0][c], lo_sh[1][c]), fminf(lo_sh[2][c], lo_sh[3][c]));
    const float hi = fmaxf(fmaxf(hi_sh[0][c], hi_sh[1][c]), fmaxf(hi_sh[2][c], hi_sh[3][c]));
    const float s = div_const<QMAX>(hi - lo);
    int z = 0;
    if (s != 0.0f) z = min(max((int)rintf(-lo / s), 0), QMAX);
    s_sh[c] = s;
    r_sh[c] = recip_refined(s);
    z_sh[c] = (float)z;
    const long long m = (row0 / 64) * kD + c;
    scale[m] = s;
    zero[m] = (uint8_t)z;
  }
  __syncthreads();
  // thread (rows 4 rg .. 4 rg + 3, channels 8 cg .. 8 cg + 7): the channels'
  // scales read once for four rows; the 8 codes of a row form slot k_slot(cg)
  const int rg = threadIdx.x >> 4, cg = threadIdx.x & 15;
  float sv[8], rv[8], zv[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float4 a = *reinterpret_cast<const float4*>(&s_sh[8 * cg + 4 * h]);
    const float4 b2 = *reinterpret_cast<const float4*>(&r_sh[8 * cg + 4 * h]);
    const float4 c2 = *reinterpret_cast<const float4*>(&z_sh[8 * cg + 4 * h]);
    sv[4 * h] = a.x; sv[4 * h + 1] = a.y; sv[4 * h + 2] = a.z; sv[4 * h + 3] = a.w;
    rv[4 * h] = b2.x; rv[4 * h + 1] = b2.y; rv[4 * h + 2] = b2.z; rv[4 * h + 3] = b2.w;
    zv[4 * h] = c2.x; zv[4 * h + 1] = c2.y; zv[4 * h + 2] = c2.z; zv[4 * h + 3] = c2.w;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * rg + i;
    float v[8];
    unpack8(*reinterpret_cast<const uint4*>(&tile[r][8 * cg]), v);
    // rne(x / s) without a divide per value (rne_quot; s = 0: r = 0, z = 0, code 0)
    float n[8];
    bool near = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) n[k] = rne_quot<(1 << BITS)>(v[k], rv[k], near);
    if (wave_any(near) && near) {
#pragma unroll
      for (int k = 0; k < 8; ++k) n[k] = rintf(v[k] / sv[k]);
    }
    uint64_t w = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = (int)__builtin_amdgcn_fmed3f(n[k] + zv[k], 0.0f, (float)QMAX);
      w |= (uint64_t)c << (BITS * k);
    }
    store_codes8<BITS>(codes + (row0 + r) * RB, k_slot(cg), (uint32_t)w, (uint32_t)(w >> 32));
  }
}

// One workgroup per b h: the appended tokens of the block that stays
// incomplete (tokens 64 floor(e / 64) .. e - 1, e = p + t_new, those at or
// after p) go to the tail as fp16 K-layout rows.
__global__ __launch_bounds__(256) void k_channel_tail(const uint16_t* __restrict__ x, int t_new, int H,
                                                      int S, const int* __restrict__ pos,
                                                      uint8_t* __restrict__ tail) {
  const long long bh = blockIdx.x;
  const int b = (int)(bh / H);
  const int p = pos[b];
  if (p < 0 || p + t_new > S) return;  // flagged by k_quant_channel
  const int e = p + t_new, k0 = e & ~63;
  const int r0 = max(p, k0) - k0, r1 = e - k0;
  const int li = threadIdx.x & 15;
  for (int r = r0 + (threadIdx.x >> 4); r < r1; r += 16) {
    const uint4 raw = ld_row8(x + (bh * t_new + (k0 + r - p)) * kD + li * 8);
    store_row_f16<false>(tail + (bh * 64 + r) * 256, li, raw, nullptr);
  }
}

// ---------------------------------------------------------------------------
// Class pools of a chunk-mixed cache: contiguous [B][H][C][CT] rows per
// class, or pages: class cls of sequence b maps its class-local rows through
// its own block-table row pages[cls][b][.] (a chunk never straddles a page:
// chunk_tokens divides page_tokens).
struct ClassPages {
  const int* pages;  // null: contiguous; else int32 [3][B][S / ptok]
  int ptok, npages, B;
};

// First pool row of class-local chunk k of (b, h) in class cls's pool; -1
// for a block-table entry outside the pool.
__device__ __forceinline__ long long chunk_row0(const ClassPages& cp, int cls, long long bh, int H, int S,
                                                int CT, int k) {
  const long long lrow = (long long)k * CT;
  if (!cp.pages) return bh * S + lrow;
  const int b = (int)(bh / H);
  const int pg = cp.pages[((long long)cls * cp.B + b) * (S / cp.ptok) + lrow / cp.ptok];
  if (pg < 0 || pg >= cp.npages) return -1;
  return ((long long)pg * H + bh % H) * cp.ptok + lrow % cp.ptok;
}

// Chunk-mixed cache (the Cocktail page's reorder, §3.1.2, then quantization
// of the reordered chunks): one workgroup per (kMixSlots consecutive slots,
// b, h); a slot's source chunk is perm[b][slot], its class follows from
// seg[b].  FP16 chunks are copied (in the row layout of the FP16 pool).  A
// chunk is only chunk_tokens rows, so a workgroup takes several: the
// sequence's class counts and the slots' sources are read once, and the
// workgroups' per-slot prologue no longer dominates.
constexpr int kMixSlots = 8;

template <int GE, bool VL>
__global__ __launch_bounds__(256) void k_quant_mixed(
    const uint16_t* __restrict__ x, int H, int S, int CT, int C, const int* __restrict__ pos,
    const int* __restrict__ perm, const int* __restrict__ seg, uint8_t* __restrict__ c16,
    uint8_t* __restrict__ c4, float* __restrict__ s4, uint8_t* __restrict__ z4,
    uint8_t* __restrict__ c2, float* __restrict__ s2, uint8_t* __restrict__ z2,
    unsigned* __restrict__ status, ClassPages cp) {
  constexpr int NG = kD / GE, LG = GE / 16;
  __shared__ uint16_t lrows[VL ? 16 : 1][128];
  __shared__ __align__(16) uint8_t lcode[VL ? 32 : 1][128];
  __shared__ int lsrc[kMixSlots];
  const int j0 = blockIdx.x * kMixSlots;
  const long long bh = blockIdx.y;
  const int b = (int)(bh / H);
  if (pos[b] != 0) {
    if (threadIdx.x == 0 && j0 == 0) set_flag(status, kFlagPosRange);
    return;
  }
  const int n16 = seg[b * 4], n4 = seg[b * 4 + 1], n = seg[b * 4 + 3];
  if (j0 >= n || n > C) return;
  if (threadIdx.x < kMixSlots) {
    const int j = j0 + (int)threadIdx.x;
    lsrc[threadIdx.x] = j < n ? perm[(long long)b * C + j] : -1;
  }
  __syncthreads();
  const int li = threadIdx.x & 15;
  uint16_t* lrow = lrows[VL ? (threadIdx.x >> 4) : 0];
  for (int sl = 0; sl < kMixSlots; ++sl) {
    const int j = j0 + sl;
    if (j >= n) break;  // (uniform over the workgroup)
    const int src = lsrc[sl];
    if (src < 0 || src >= C) continue;
    const int cls = j < n16 ? 0 : (j < n16 + n4 ? 1 : 2);
    const int k = cls == 0 ? j : (cls == 1 ? j - n16 : j - n16 - n4);
    const uint16_t* xs = x + (bh * S + (long long)src * CT) * kD;
    const long long drow0 = chunk_row0(cp, cls, bh, H, S, CT, k);
    if (drow0 < 0) {
      if (threadIdx.x == 0) set_flag(status, kFlagPageRange);
      continue;
    }
    if (cls == 0) {  // FP16: copied, 16 lanes per row
      for (int r = threadIdx.x >> 4; r < CT; r += 16)
        store_row_f16<VL>(c16 + (drow0 + r) * kD * 2, li, ld_row8(xs + (long long)r * kD + li * 8), lrow);
      continue;
    }
    // INT4 / INT2: eight lanes per row, 16 channels per lane
    const int l8 = threadIdx.x & 7;
    uint8_t* lc = lcode[VL ? (threadIdx.x >> 3) : 0];
    for (int r = threadIdx.x >> 3; r < CT; r += 32) {
      const uint16_t* src = xs + (long long)r * kD + l8 * 16;
      const long long drow = drow0 + r;
      float v[16];
      {
        float h[8];
        unpack8(ld_row8(src), h);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = h[k];
        unpack8(ld_row8(src + 8), h);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[8 + k] = h[k];
      }
      unsigned c[16];
      float s;
      int z;
      if (cls == 1) {
        quant16<4, false, GE>(v, c, s, z);
        store_row_codes16<4, VL>(c4 + drow * 64, l8, c, lc);
        if (l8 % LG == 0) {
          s4[drow * NG + l8 / LG] = s;
          z4[drow * NG + l8 / LG] = (uint8_t)z;
        }
      } else {
        quant16<2, false, GE>(v, c, s, z);
        store_row_codes16<2, VL>(c2 + drow * 32, l8, c, lc);
        if (l8 % LG == 0) {
          s2[drow * NG + l8 / LG] = s;
          z2[drow * NG + l8 / LG] = (uint8_t)z;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk-mixed streaming append.  Tokens of the chunk not yet complete wait as
// fp16 rows in the FP16 pool's last chunk (the "waiting chunk"); a chunk
// completed by an append is read from there (its tokens below pos) and from
// the input, and copied or quantized into the next chunk of its class pool.

__device__ __forceinline__ int chunk_cls(unsigned v) { return v == 16u ? 0 : (v == 4u ? 1 : 2); }

// 8 channels 8 li .. 8 li + 7 of token row r of a chunk being completed, in
// channel order: from the waiting chunk (fp16 pool layout VL) when `waiting`,
// else from the input row xrow.  The V layout is transposed through lrow.
template <bool VL>
__device__ __forceinline__ uint4 chunk_row8(bool waiting, const uint8_t* wrow, const uint16_t* xrow,
                                            int li, uint16_t* lrow) {
  if constexpr (!VL) {
    return waiting ? ld_row8_k16(wrow, li) : ld_row8(xrow + li * 8);
  } else {
    // V pool word li holds channels li + 16 e; an input lane holds 8 li + e
    const uint4 w = waiting ? ld_row8(reinterpret_cast<const uint16_t*>(wrow + li * 16)) : ld_row8(xrow + li * 8);
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      lrow[waiting ? li + 16 * e : 8 * li + e] = (uint16_t)(d[e >> 1] >> (16 * (e & 1)));
    wave_lds_sync();
    uint4 o;
    o.x = (uint32_t)lrow[8 * li + 0] | ((uint32_t)lrow[8 * li + 1] << 16);
    o.y = (uint32_t)lrow[8 * li + 2] | ((uint32_t)lrow[8 * li + 3] << 16);
    o.z = (uint32_t)lrow[8 * li + 4] | ((uint32_t)lrow[8 * li + 5] << 16);
    o.w = (uint32_t)lrow[8 * li + 6] | ((uint32_t)lrow[8 * li + 7] << 16);
    wave_lds_sync();
    return o;
  }
}

// One workgroup per (i, b h), i = i0 + blockIdx.x: the i-th chunk this append
// completes in sequence b (original chunk id n + i, n = seg[b][3] = pos[b] /
// CT), with the bit-width bits[b][i]; its class-local index is that class's
// count plus the earlier chunks of the same class in this append.  Only chunk
// 0 reads waiting tokens, and only the sequence's final chunk can land in the
// waiting chunk's place (an all-FP16 sequence), so chunk 0 runs in a launch
// of its own before the others.
template <int GE, bool VL>
__global__ __launch_bounds__(256) void k_chunk_append(
    int i0, const uint16_t* __restrict__ x, int t_new, int H, int S, int CT, int C, const int* __restrict__ pos,
    const uint8_t* __restrict__ bits, int n_new, const int* __restrict__ seg, uint8_t* __restrict__ c16,
    uint8_t* __restrict__ c4, float* __restrict__ s4, uint8_t* __restrict__ z4, uint8_t* __restrict__ c2,
    float* __restrict__ s2, uint8_t* __restrict__ z2, unsigned* __restrict__ status, ClassPages cp) {
  constexpr int NG = kD / GE, LG = GE / 8;
  __shared__ uint16_t lrows[VL ? 16 : 1][128];
  const int i = i0 + (int)blockIdx.x;
  const long long bh = blockIdx.y;
  const int b = (int)(bh / H);
  const int p = pos[b], n = seg[b * 4 + 3];
  if (p < 0 || p + t_new > S || p / CT != n) {
    if (threadIdx.x == 0 && i == 0 && bh % H == 0) set_flag(status, kFlagPosRange);
    return;
  }
  const int j = n + i;
  if ((j + 1) * CT > p + t_new) return;  // not completed by this append
  const uint8_t* bb = bits + (long long)b * n_new;
  const int cls = chunk_cls(bb[i]);
  int k = seg[b * 4 + cls];
  for (int i2 = 0; i2 < i; ++i2) k += chunk_cls(bb[i2]) == cls;
  if (k >= C) return;
  const long long wrow0 = chunk_row0(cp, 0, bh, H, S, CT, C - 1);  // waiting chunk
  const long long drow0 = chunk_row0(cp, cls, bh, H, S, CT, k);
  if (wrow0 < 0 || drow0 < 0) {
    if (threadIdx.x == 0) set_flag(status, kFlagPageRange);
    return;
  }
  const int li = threadIdx.x & 15;
  uint16_t* lrow = lrows[VL ? (threadIdx.x >> 4) : 0];
  for (int r = threadIdx.x >> 4; r < CT; r += 16) {
    const int t = j * CT + r;
    const bool waiting = t < p;
    const uint4 raw = chunk_row8<VL>(waiting, c16 + (wrow0 + r) * kD * 2,
                                     x + (bh * t_new + (waiting ? 0 : t - p)) * kD, li, lrow);
    const long long drow = drow0 + r;
    if (cls == 0) {
      store_row_f16<VL>(c16 + drow * kD * 2, li, raw, lrow);
      continue;
    }
    float v[8];
    unpack8(raw, v);
    uint32_t plo, phi;
    float sc;
    int z;
    if (cls == 1) {
      quant8<4, false, GE>(v, 0xFFu, plo, phi, sc, z);
      store_row_codes<4, VL>(c4 + drow * 64, li, plo, phi, lrow);
      if (li % LG == 0) {
        s4[drow * NG + li / LG] = sc;
        z4[drow * NG + li / LG] = (uint8_t)z;
      }
    } else {
      quant8<2, false, GE>(v, 0xFFu, plo, phi, sc, z);
      store_row_codes<2, VL>(c2 + drow * 32, li, plo, phi, lrow);
      if (li % LG == 0) {
        s2[drow * NG + li / LG] = sc;
        z2[drow * NG + li / LG] = (uint8_t)z;
      }
    }
  }
}

// One workgroup per b h, after k_chunk_append (which reads the waiting chunk
// first): the appended tokens of the chunk left incomplete wait as fp16.
template <bool VL>
__global__ __launch_bounds__(256) void k_chunk_wait(const uint16_t* __restrict__ x, int t_new, int H, int S,
                                                    int CT, int C, const int* __restrict__ pos,
                                                    const int* __restrict__ seg, uint8_t* __restrict__ c16,
                                                    unsigned* __restrict__ status, ClassPages cp) {
  __shared__ uint16_t lrows[VL ? 16 : 1][128];
  const long long bh = blockIdx.x;
  const int b = (int)(bh / H);
  const int p = pos[b];
  if (p < 0 || p + t_new > S || p / CT != seg[b * 4 + 3]) return;  // flagged by k_chunk_append
  const long long wrow0 = chunk_row0(cp, 0, bh, H, S, CT, C - 1);  // the waiting chunk
  if (wrow0 < 0) {
    if (threadIdx.x == 0) set_flag(status, kFlagPageRange);
    return;
  }
  const int e = p + t_new, j0 = (e / CT) * CT;
  const int r0 = max(p, j0) - j0, r1 = e - j0;
  const int li = threadIdx.x & 15;
  uint16_t* lrow = lrows[VL ? (threadIdx.x >> 4) : 0];
  for (int r = r0 + (threadIdx.x >> 4); r < r1; r += 16) {
    const uint4 raw = ld_row8(x + (bh * t_new + (j0 + r - p)) * kD + li * 8);
    store_row_f16<VL>(c16 + (wrow0 + r) * kD * 2, li, raw, lrow);
  }
}

// ---------------------------------------------------------------------------
// Outer values of an Oaken row (the Oaken page, §3.2.2): delta = x - T_hi
// above the upper outer threshold, x - T_lo below the lower one; the group's
// outer scale s_out = max |delta| / 31 and each value's 5-bit shifted
// magnitude rne(|delta| / s_out).
//
// s_out without visiting the outer values: binary32 subtraction is monotone,
// so the largest fl(x - T_hi) over the values above T_hi is fl(max x - T_hi),
// and the largest fl(T_lo - x) (= |fl(x - T_lo)|) over the values below T_lo
// is fl(T_lo - min x); a group without such values gives a non-positive
// difference.  Hence max |delta| = max(fl(max x - T_hi), fl(T_lo - min x), 0)
// over all of the group's values, exactly.
template <int LG, int N>
__device__ __forceinline__ float oak_outer_scale(const float (&v)[N], float t_lo, float t_hi) {
  float mx = v[0], mn = v[0];
#pragma unroll
  for (int k = 1; k < N; ++k) {
    mx = fmaxf(mx, v[k]);
    mn = fminf(mn, v[k]);
  }
  mx = max_lanes<1, LG>(mx);
  mn = min_lanes<1, LG>(mn);
  return div_const<31>(fmaxf(fmaxf(mx - t_hi, t_lo - mn), 0.0f));
}

// One sparse entry (channel | side << 7 | mag << 8 | tag << 13) for the
// outer value v of a group with outer scale so (r = recip_refined(so); s_out
// = 0: magnitude 0).  tag: the row's token index mod 8, which decode reads in
// place of a search of the row pointers.
__device__ __forceinline__ uint16_t oak_entry_word(float v, float t_lo, float t_hi, float so, float r,
                                                   unsigned ch, unsigned tag) {
  const bool above = v > t_hi;
  const float d = above ? v - t_hi : t_lo - v;
  bool near = false;
  float m = rne_quot<32>(d, r, near);
  if (wave_any(near) && near) m = rintf(d / so);
  const unsigned mag = (unsigned)__builtin_amdgcn_fmed3f(m, 0.0f, 31.0f);
  return (uint16_t)(ch | (unsigned)above << 7 | mag << 8 | tag << 13);
}
__device__ __forceinline__ void store_entry(uint16_t* sp, unsigned e, unsigned cap, uint16_t w,
                                            bool& dropped) {
  if (e < cap)
    *reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(sp) + (e << 1)) = w;
  else
    dropped = true;
}

// A lane's entries for its outer values (bit k of `outer`: value k of the
// lane's 8 fp16 values in raw), one iteration per set bit in ascending
// channel order, to entries e, e + 1, ... of a list of capacity cap (< 2^31,
// so byte offsets fit 32 bits); `dropped` on overflow.
__device__ __forceinline__ void oak_lane_entries(const uint4 raw, unsigned outer, float t_lo, float t_hi,
                                                 float so, int li, unsigned tag, uint16_t* sp, unsigned e,
                                                 unsigned cap, bool& dropped) {
  const float r = recip_refined(so);
  while (outer) {
    const int k = __builtin_ctz(outer);
    outer &= outer - 1u;
    const unsigned w = (k & 4) ? ((k & 2) ? raw.w : raw.z) : ((k & 2) ? raw.y : raw.x);
    const float v = h2f((uint16_t)(w >> (16 * (k & 1))));
    store_entry(sp, e++, cap, oak_entry_word(v, t_lo, t_hi, so, r, (unsigned)(li * 8 + k), tag), dropped);
  }
}

// The dense INT4 body of one lane's 16 values of an Oaken row (outer values
// enter as 0, so they neither widen the range nor divide), in groups of 16 LG
// channels over LG lanes: s = (hi - lo) / 15, z = rne(-lo / s) and code
// clamp(rne(x / s) + z, 0, 15), the asymmetric quantizer of the token rows,
// returned as exact small floats.
template <int LG>
__device__ __forceinline__ void oak_dense16(const float (&xm)[16], float (&q)[16], float& s, int& z) {
  constexpr float QMAX = 15.0f;
  float lo = 0.0f, hi = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    lo = fminf(lo, xm[k]);
    hi = fmaxf(hi, xm[k]);
  }
  lo = min_lanes<1, LG>(lo);
  hi = max_lanes<1, LG>(hi);
  s = div_const<15>(hi - lo);
  const float r = recip_refined(s);  // s = 0: z = 0 and all codes 0
  bool near = false;
  float zf = rne_quot<16>(-lo, r, near);
  if (wave_any(near) && near) zf = rintf(-lo / s);
  zf = __builtin_amdgcn_fmed3f(zf, 0.0f, QMAX);
  z = (int)zf;
  asym_codes<16>(xm, s, r, zf, q);
}

// Eight 4-bit codes (exact floats 0..15) as one word, code k in bits 4k..4k+3:
// pairs joined exactly in float, each pair converted into its byte.
__device__ __forceinline__ uint32_t pack_nibbles8(const float* q) {
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[2 * b + 1], 16.0f, q[2 * b]), b, w);
  return w;
}

// Oaken (the Oaken page, §3.1 online stage, §3.2.1-3.2.2): per row, outer
// values (x > T_hi_outer or x < T_lo_outer) leave the dense INT4 body (coded
// z) and go to the row's sparse list as shifted deltas with a per-group
// 5-bit scale.  One workgroup per (b, h) walks the new rows in tiles of 64
// (eight lanes per row, 16 channels per lane, 32 rows at a time), the next
// tile's rows loaded while the current one is coded.  The rows' outer counts
// meet in LDS once per tile; every wave scans all 64 of them itself, so the
// running entry offset (and with it rowptr, a prefix sum of the counts)
// needs one barrier per tile.
template <int GE, bool VL>
__global__ __launch_bounds__(256) void k_quant_oaken(
    const uint16_t* __restrict__ x, int t_new, int H, int S, const int* __restrict__ pos,
    float t_lo, float t_hi, long long cap, uint8_t* __restrict__ codes, float* __restrict__ scale,
    uint8_t* __restrict__ zero, float* __restrict__ oscale, uint32_t* __restrict__ rowptr,
    uint16_t* __restrict__ sparse, unsigned* __restrict__ status, PageMap pm) {
  constexpr int NG = kD / GE, LG = GE / 16, U = 2, TR = 32 * U;
  static_assert(GE >= 16, "a group spans whole lanes");
  // V layout: code k of lane li goes to byte 8 k + li of its row's slot, so
  // that word n (channels n + 16 j) is bytes 8 n .. 8 n + 7
  __shared__ __align__(16) uint8_t lcode[VL ? 32 : 1][128];
  __shared__ unsigned row_cnt[2][TR];  // alternate tiles: one barrier per tile
  // the tile's rows as each thread loaded them, word-major (conflict-free):
  // pass 2 reads its outer values back from here
  __shared__ uint32_t lraw[8 * U][256];
  const long long bh = blockIdx.x;
  const int b = (int)(bh / H);
  const int p = pos[b];
  if (p < 0 || p + t_new > S) {
    if (threadIdx.x == 0) set_flag(status, kFlagPosRange);
    return;
  }
  uint32_t* rp = rowptr + bh * (S + 1);
  uint16_t* sp = sparse + bh * cap;
  const unsigned capu = (unsigned)cap;  // < 2^31 (validated)
  // running entry count: at most cap + 128 t_new < 2^32
  unsigned base = p == 0 ? 0u : rp[p];
  if (p == 0 && threadIdx.x == 0) rp[0] = 0u;
  const int rl = threadIdx.x >> 3, li = threadIdx.x & 7, lane = threadIdx.x & 63;
  uint8_t* lc = lcode[VL ? rl : 0];
  // rows past the last one load the last row (always readable); such rows
  // are neither counted nor stored
  const uint16_t* xr = x + bh * t_new * kD + li * 16;
  uint4 nxt[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint16_t* r = xr + (long long)min(32 * u + rl, t_new - 1) * kD;
    nxt[u][0] = ld_row8(r);
    nxt[u][1] = ld_row8(r + 8);
  }
  bool dropped = false;
  for (int t0 = 0, it = 0; t0 < t_new; t0 += TR, it ^= 1) {
    uint4 raw[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      raw[u][0] = nxt[u][0];
      raw[u][1] = nxt[u][1];
    }
    if (t0 + TR < t_new) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint16_t* r = xr + (long long)min(t0 + TR + 32 * u + rl, t_new - 1) * kD;
        nxt[u][0] = ld_row8(r);
        nxt[u][1] = ld_row8(r + 8);
      }
    }
    // pass 1: per row, the dense INT4 body, the scales and the outer mask;
    // the row's outer count (a lane's first entry within its row in bits 16
    // and up of meta)
    unsigned meta[U];
    float sos[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + 32 * u + rl;
      const bool active = t < t_new;
      float v[16], xm[16];
      {
        float h[8];
        unpack8(raw[u][0], h);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = h[k];
        unpack8(raw[u][1], h);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[8 + k] = h[k];
      }
      unsigned outer = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const bool o = ((v[k] > t_hi) | (v[k] < t_lo)) & active;
        outer |= (unsigned)o << k;
        xm[k] = o ? 0.0f : v[k];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lraw[8 * u + c][threadIdx.x] = (&raw[u][0].x)[c];
        lraw[8 * u + 4 + c][threadIdx.x] = (&raw[u][1].x)[c];
      }
      float q[16], s;
      int z;
      oak_dense16<LG>(xm, q, s, z);
      const float so = oak_outer_scale<LG>(v, t_lo, t_hi);
      const int lcnt = __popc(outer);
      int incl = lcnt;
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) {
        const int o = __shfl_up(incl, m, 8);
        if (li >= m) incl += o;
      }
      if (li == 7) row_cnt[it][32 * u + rl] = (unsigned)incl;  // 0 for an inactive row
      meta[u] = outer | (unsigned)(incl - lcnt) << 16;
      sos[u] = so;
      // codes: K layout, slots of channels 16 li .. +7 and 16 li + 8 .. +15;
      // V layout, words 2 li and 2 li + 1 through the row's LDS slot
      uint32_t w0, w1;
      if constexpr (!VL) {
        w0 = pack_nibbles8(q);
        w1 = pack_nibbles8(q + 8);
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) lc[8 * k + li] = (uint8_t)(unsigned)q[k];
        wave_lds_sync();
        const uint4 by = *reinterpret_cast<const uint4*>(lc + 16 * li);
        wave_lds_sync();
        // bytes b0..b3 (each < 16) of a word -> nibbles b0 | b1 << 4 | b2 << 8 | b3 << 12
        auto nib4 = [](uint32_t d) {
          const uint32_t t = d | (d >> 4);
          return (t & 0xFFu) | ((t >> 8) & 0xFF00u);
        };
        w0 = nib4(by.x) | nib4(by.y) << 16;
        w1 = nib4(by.z) | nib4(by.w) << 16;
      }
      if (active) {
        // the dense row: contiguous, or in its page (a table entry outside
        // the pool skips the row and flags; the sparse list is per sequence)
        long long dst = bh * S + p + t;
        bool dense_ok = true;
        if (pm.pages) {
          const int tok = p + t;
          const int pg = pm.pages[(long long)b * (S / pm.ptok) + tok / pm.ptok];
          dense_ok = pg >= 0 && pg < pm.npages;
          if (!dense_ok && li == 0) set_flag(status, kFlagPageRange);
          dst = ((long long)pg * H + bh % H) * pm.ptok + tok % pm.ptok;
        }
        if (dense_ok) {
          uint8_t* row = codes + dst * 64;
          if constexpr (!VL) {
            st_nt<uint32_t>(row + 4 * k_slot(2 * li), w0);
            st_nt<uint32_t>(row + 4 * k_slot(2 * li + 1), w1);
          } else {
            st_nt<u2q_t>(row + 8 * li, u2q_t{w0, w1});
          }
          if (li % LG == 0) {
            scale[dst * NG + li / LG] = s;
            zero[dst * NG + li / LG] = (uint8_t)z;
            oscale[dst * NG + li / LG] = so;
          }
        }
      }
    }
    __syncthreads();
    // each wave: inclusive scan of the tile's 64 row counts, lane r = row r
    const unsigned cnt = row_cnt[it][lane];
    unsigned scan = cnt;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const unsigned o = __shfl_up(scan, m, 64);
      if (lane >= m) scan += o;
    }
    const unsigned excl_row = scan - cnt;
    const unsigned tile_tot = __shfl(scan, 63, 64);
    // pass 2: rowptr, then the entries.  A lane's outer bits of the tile's
    // two rows form one mask (bit 16 u + k: value k of row u), walked in one
    // loop with the values read back from LDS, so a wave runs as many
    // iterations as its busiest lane has outer values in the whole tile
    // (about four at a 5 % outer rate), not that many per row.  Bits come in
    // ascending (row, channel) order: the lane's c-th entry of the tile is
    // its (c - before_u)-th of row u.
    unsigned mask = 0, before = 0, off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + 32 * u + rl;
      const unsigned rb = base + __shfl(excl_row, 32 * u + rl, 64);
      const unsigned rcnt = __shfl(cnt, 32 * u + rl, 64);
      const unsigned outer = meta[u] & 0xFFFFu;  // 0 for a row past the last
      off[u] = rb + (meta[u] >> 16) - before;    // mod 2^32
      before += __popc(outer);
      mask |= outer << (16 * u);
      if (t < t_new && li == 0) rp[(unsigned)(p + t + 1)] = min(rb + rcnt, capu);
    }
    const unsigned tag = (unsigned)(p + t0 + rl) & 7u;  // (p + t0 + 32 u + rl) mod 8
    const float so0 = sos[0], so1 = sos[1];
    const float rc0 = recip_refined(so0), rc1 = recip_refined(so1);
    const unsigned of0 = off[0], of1 = off[1];
    for (unsigned c = 0; mask; ++c) {
      const int j = __builtin_ctz(mask);
      mask &= mask - 1u;
      const bool r1 = (j & 16) != 0;
      const float v = h2f(reinterpret_cast<const uint16_t*>(&lraw[j >> 1][threadIdx.x])[j & 1]);
      store_entry(sp, (r1 ? of1 : of0) + c, capu,
                  oak_entry_word(v, t_lo, t_hi, r1 ? so1 : so0, r1 ? rc1 : rc0, (unsigned)(li * 16 + (j & 15)),
                                 tag),
                  dropped);
    }
    base += tile_tot;
  }
  if (dropped) set_flag(status, kFlagSparseFull);
}

// Oaken append of one token per sequence, K and V in one launch
// (blockIdx.y: 0 K rows, 1 V rows): 16 lanes per (b, h) row, 16 rows per
// workgroup.  With one new token the rows are independent: each continues its
// own (b, h) list at rowptr[pos].
template <int GE>
__global__ __launch_bounds__(256) void k_quant_oaken_one(const uint16_t* __restrict__ xk,
                                                         const uint16_t* __restrict__ xv, int BH, int H,
                                                         int S, const int* __restrict__ pos,
                                                         TensorArgs tk, TensorArgs tv,
                                                         unsigned* __restrict__ status, PageMap pm) {
  constexpr int NG = kD / GE, LG = GE / 8;
  __shared__ uint16_t lrows[16][128];
  const bool vl = blockIdx.y != 0;
  const TensorArgs& t = vl ? tv : tk;
  const uint16_t* x = vl ? xv : xk;
  const int rl = threadIdx.x >> 4, li = threadIdx.x & 15;
  const long long bh = (long long)blockIdx.x * 16 + rl;
  if (bh >= BH) return;  // all 16 lanes of a row leave together
  const int b = (int)((uint32_t)bh / (uint32_t)H);  // (bh < BH < 2^31: a 32-bit divide)
  const int p = pos[b];
  if (p < 0 || p + 1 > S) {
    if (li == 0) set_flag(status, kFlagPosRange);
    return;
  }
  uint32_t* rp = t.rowptr + bh * (S + 1);
  uint16_t* sp = t.sparse + bh * t.sparse_cap;
  const unsigned base = p == 0 ? 0u : rp[p];
  if (p == 0 && li == 0) rp[0] = 0u;
  float v[8];
  const uint4 raw = ld_row8(x + bh * kD + li * 8);
  unpack8(raw, v);
  unsigned outer = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) outer |= (unsigned)((v[k] > t.thr_hi) || (v[k] < t.thr_lo)) << k;
  uint32_t plo, phi;
  float s;
  int z;
  quant8<4, false, GE>(v, ~outer & 0xFFu, plo, phi, s, z);
  const float so = oak_outer_scale<LG>(v, t.thr_lo, t.thr_hi);
  const int lc = __popc(outer);
  int incl = lc;
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    const int o = __shfl_up(incl, m, 16);
    if (li >= m) incl += o;
  }
  const int rowtot = __shfl(incl, 15, 16);
  long long dst = bh * S + p;
  bool dense_ok = true;
  if (pm.pages) {  // the dense row in its page; the sparse list is per sequence
    const int pg = pm.pages[(long long)b * (S / pm.ptok) + p / pm.ptok];
    dense_ok = pg >= 0 && pg < pm.npages;
    if (!dense_ok && li == 0) set_flag(status, kFlagPageRange);
    dst = ((long long)pg * H + bh % H) * pm.ptok + p % pm.ptok;
  }
  if (dense_ok) {
    if (vl) store_row_codes<4, true>(t.codes + dst * 64, li, plo, phi, lrows[rl]);
    else store_row_codes<4, false>(t.codes + dst * 64, li, plo, phi, lrows[rl]);
    if (li % LG == 0) {
      t.scale[dst * NG + li / LG] = s;
      t.zero[dst * NG + li / LG] = (uint8_t)z;
      t.oscale[dst * NG + li / LG] = so;
    }
  }
  const unsigned cap = (unsigned)t.sparse_cap;  // < 2^31 (validated)
  const unsigned e = base + (unsigned)(incl - lc);
  bool dropped = false;
  oak_lane_entries(raw, outer, t.thr_lo, t.thr_hi, so, li, (unsigned)p & 7u, sp, e, cap, dropped);
  if (li == 0) {
    rp[p + 1] = min(base + (unsigned)rowtot, cap);
  }
  if (dropped) set_flag(status, kFlagSparseFull);
}

// ---------------------------------------------------------------------------
// KVO-LLM differential significant-token quantization (the KVO-LLM page,
// §3.1): per group of 64 tokens of one (b, h), the dsq_sig tokens with the
// largest scores are significant (1-bit mask); their K and V rows become
// INT8 with per-channel scales over the significant tokens; the other
// tokens become INT2 rows in groups of 32 channels, V directly and K as the
// difference from the base row, the mean of the dequantized significant K
// rows.  Class slots follow token order.
//
// Appends are a stream: the tokens of the group not yet complete wait in
// per-(b, h) fp16 tails (K rows in the K word order, V rows in the V word
// order of the fp16 pool layout) with their scores; k_quant_dsq takes one
// workgroup per group an append completes and gathers its 64 rows, those
// below pos from the tails and the rest from the input; k_dsq_tail (next on
// the stream, so the tails are read before they are rewritten) stores the
// new tokens of the group left incomplete.

// Scores ordered by bit pattern: a total order (-0 below +0, NaNs at the ends)
__device__ __forceinline__ unsigned dsq_key(float x) {
  const unsigned b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kDsqSigSlots = 16;  // significant-row slots per group
constexpr int kDsqOthSlots = 64;  // other-row slots per group
constexpr int kDsqPre = 4;        // other rows loaded ahead per row group

// 8 channels 8 li .. 8 li + 7 of an fp16 V-layout row (word n holds
// channels n + 16 j), in channel order (inverse of store_row_f16's V order).
__device__ __forceinline__ uint4 ld_row8_v16(const uint8_t* row, int li) {
  const uint16_t* h = reinterpret_cast<const uint16_t*>(row);
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c0 = 8 * li + 2 * k, c1 = c0 + 1;
    w[k] = (uint32_t)h[(c0 & 15) * 8 + (c0 >> 4)] | ((uint32_t)h[(c1 & 15) * 8 + (c1 >> 4)] << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(256) void k_quant_dsq(const uint16_t* __restrict__ xk,
                                                   const uint16_t* __restrict__ xv,
                                                   const float* __restrict__ score, int t_new, int H, int S,
                                                   int n_sig, const int* __restrict__ pos, TensorArgs kt,
                                                   TensorArgs vt, unsigned long long* __restrict__ mask_out,
                                                   unsigned* __restrict__ status, PageMap pm) {
  __shared__ float gsc[64];  // the group's scores
  __shared__ int s_tok[kDsqSigSlots];
  __shared__ int o_tok[kDsqOthSlots];
  __shared__ int8_t sig[2][kDsqSigSlots][kD];
  __shared__ float base[kD];
  __shared__ uint16_t lrows[16][kD];
  const int gi = blockIdx.x;
  const long long bh = blockIdx.y;
  const int b = (int)(bh / H);
  const int p = pos[b];
  if (p < 0 || p > S - t_new) {
    if (gi == 0 && threadIdx.x == 0) set_flag(status, kFlagPosRange);
    return;
  }
  const int k0 = (p & ~63) + 64 * gi;  // first token of the group
  if (k0 + 64 > p + t_new) return;     // still incomplete after this append
  // destination group: contiguous [B][H][S / 64], or group k0 mod ptok of
  // page pages[b][k0 / ptok] in the pool [npages][H][ptok / 64]
  long long gb = bh * (S / 64) + (k0 >> 6);
  if (pm.pages) {
    const int pg = pm.pages[(long long)b * (S / pm.ptok) + k0 / pm.ptok];
    if (pg < 0 || pg >= pm.npages) {
      if (threadIdx.x == 0) set_flag(status, kFlagPageRange);
      return;
    }
    gb = ((long long)pg * H + bh % H) * (pm.ptok / 64) + (k0 % pm.ptok) / 64;
  }
  const int n_oth = 64 - n_sig;
  // the group's tokens below p are read from the tails, the others from the input
  if (threadIdx.x < 64) {
    const int tok = k0 + threadIdx.x;
    gsc[threadIdx.x] = tok < p ? kt.oscale[bh * 64 + threadIdx.x] : score[bh * t_new + (tok - p)];
  }
  __syncthreads();
  // 1. significant tokens: rank of each token's score, ties to the lower index
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    const unsigned key = dsq_key(gsc[t]);
    int rank = 0;
    for (int u = 0; u < 64; ++u) {
      const unsigned ku = (unsigned)__shfl((int)key, u, 64);
      rank += (ku > key || (ku == key && u < t)) ? 1 : 0;
    }
    const bool is_sig = rank < n_sig;
    const unsigned long long m = __ballot(is_sig);
    const int below = __popcll(m & ((1ull << t) - 1ull));
    if (is_sig) s_tok[below] = t;
    else o_tok[t - below] = t;
    if (t == 0) mask_out[gb] = m;
  }
  __syncthreads();
  // 2. significant rows: INT8 per channel; thread = (tensor, channel)
  {
    // the base sum rounds each product and each sum (no fused multiply-add)
#pragma clang fp contract(off)
    const int tsr = threadIdx.x >> 7, d = threadIdx.x & 127;
    const uint16_t* x = (tsr ? xv : xk) + (bh * t_new - p) * kD + d;  // token t at x[t * kD]
    const uint16_t* tail = reinterpret_cast<const uint16_t*>((tsr ? vt : kt).codes16) + bh * 64 * kD;
    // channel d's half within an fp16 tail row: K word order (slot 4 q + s,
    // halves 0, 4, 1, 5, 2, 6, 3, 7) or V word order (word n, half j)
    const int toff = tsr ? ((d & 15) * 8 + (d >> 4))
                         : ((4 * ((d >> 3) & 3) + (d >> 5)) * 8 + (d & 3) * 2 + ((d >> 2) & 1));
    float xv_[kDsqSigSlots];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kDsqSigSlots; ++i) {
      const int tok = k0 + (i < n_sig ? s_tok[i] : 0);
      // the input row is always read (row max(tok, p) exists), so the
      // slots' loads issue together; a token still in the tails (rare)
      // replaces it from there
      uint16_t h = x[(long long)max(tok, p) * kD];
      if (tok < p) h = tail[(tok - k0) * kD + toff];
      xv_[i] = i < n_sig ? h2f(h) : 0.0f;
      amax = fmaxf(amax, fabsf(xv_[i]));
    }
    const float s = div_const<127>(amax);
    // rne(x / s) without a divide per value (rne_quot; slots past n_sig hold
    // 0 and code 0; s = 0 gives r = 0 and codes 0)
    const float r = recip_refined(s);
    bool near = false;
    float n[kDsqSigSlots];
#pragma unroll
    for (int i = 0; i < kDsqSigSlots; ++i) n[i] = rne_quot<128>(xv_[i], r, near);
    if (wave_any(near) && near) {
#pragma unroll
      for (int i = 0; i < kDsqSigSlots; ++i) n[i] = rintf(xv_[i] / s);
    }
    float acc = 0.0f;  // K base: sum in slot order, one rounding per operation
#pragma unroll
    for (int i = 0; i < kDsqSigSlots; ++i) {
      const int q = (int)__builtin_amdgcn_fmed3f(n[i], -128.0f, 127.0f);
      sig[tsr][i][d] = (int8_t)q;
      if (i < n_sig) acc = acc + s * (float)q;
    }
    (tsr ? vt : kt).scale[gb * kD + d] = s;
    if (tsr == 0) base[d] = acc / (float)n_sig;
  }
  __syncthreads();
  // 3. pack the significant rows: job = (tensor, slot, 8-byte word)
  for (int j = threadIdx.x; j < 2 * kDsqSigSlots * 16; j += blockDim.x) {
    const int tsr = j >> 8, row = (j >> 4) & 15, w = j & 15;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // K: word 4 q + s holds channels 32 s + 8 q + e; V: word n holds channels n + 16 e
      const int ch = tsr ? (w + 16 * e) : (32 * (w & 3) + 8 * (w >> 2) + e);
      const uint32_t byte = (uint8_t)sig[tsr][row][ch];
      if (e < 4) lo |= byte << (8 * e);
      else hi |= byte << (8 * (e - 4));
    }
    st_nt<u2q_t>((tsr ? vt : kt).codes + (gb * kDsqSigSlots + row) * kD + w * 8, u2q_t{lo, hi});
  }
  // 4. the other tokens: INT2 rows in groups of 32 channels; 16 lanes per row
  const int li = threadIdx.x & 15, rg = threadIdx.x >> 4;
  uint16_t* lrow = lrows[rg];
  // The input rows of kDsqPre slots are loaded before any of them is coded
  // (slots past n_oth load a row of the group, unused); rows still in the
  // tails (tokens below p) are read from there in place of theirs.
#pragma unroll
  for (int tsr = 0; tsr < 2; ++tsr) {
    const TensorArgs& t = tsr ? vt : kt;
    const uint16_t* xin = tsr ? xv : xk;
#pragma unroll
    for (int s0 = 0; s0 < kDsqOthSlots; s0 += 16 * kDsqPre) {
    uint4 raws[kDsqPre];
    int toks[kDsqPre];
#pragma unroll
    for (int j = 0; j < kDsqPre; ++j) {
      const int slot = s0 + rg + 16 * j;
      toks[j] = slot < n_oth ? k0 + o_tok[slot] : max(k0, p);
      raws[j] = ld_row8(xin + (bh * t_new + (max(toks[j], p) - p)) * kD + li * 8);
    }
#pragma unroll
    for (int j = 0; j < kDsqPre; ++j) {
      const int slot = s0 + rg + 16 * j;
      const long long dst = gb * kDsqOthSlots + slot;
      uint32_t plo = 0, phi = 0;
      float s = 0.0f;
      int z = 0;
      if (slot < n_oth) {
        float v[8];
        const int tok = toks[j];
        uint4 raw = raws[j];
        if (tok < p) {
          const uint8_t* trow = t.codes16 + (bh * 64 + (tok - k0)) * 256;
          raw = tsr ? ld_row8_v16(trow, li) : ld_row8_k16(trow, li);
        }
        unpack8(raw, v);
        if (tsr == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] - base[li * 8 + e];  // difference from the base
        }
        quant8<2, false, 32>(v, 0xFFu, plo, phi, s, z);
      }
      if (tsr) {
        // V: column word li of slot `slot` in the blocked order (the 8 words
        // of rows 8i .. 8i + 7 of one column are contiguous)
#pragma unroll
        for (int v = 0; v < 8; ++v) lrow[8 * li + v] = (uint16_t)code_at<2>(plo, phi, v);
        wave_lds_sync();
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) w |= (uint32_t)lrow[li + 16 * j] << (2 * j);
        wave_lds_sync();
        st_nt<uint16_t>(t.codes2 + gb * (kDsqOthSlots * 32) + (((slot >> 3) * 16 + li) * 16 + (slot & 7) * 2),
                        (uint16_t)w);
      } else {
        store_row_codes<2, false>(t.codes2 + dst * 32, li, plo, phi, lrow);
      }
      if ((li & 3) == 0) {
        t.scale2[dst * 4 + (li >> 2)] = s;
        t.zero2[dst * 4 + (li >> 2)] = (uint8_t)z;
      }
    }
    }
  }
}

// One workgroup per b h: the appended tokens of the group that stays
// incomplete (tokens 64 floor(e / 64) .. e - 1, e = p + t_new, those at or
// after p) go to the tails (K and V fp16 rows, scores).
__global__ __launch_bounds__(256) void k_dsq_tail(const uint16_t* __restrict__ xk,
                                                  const uint16_t* __restrict__ xv,
                                                  const float* __restrict__ score, int t_new, int H, int S,
                                                  const int* __restrict__ pos, TensorArgs kt, TensorArgs vt) {
  __shared__ uint16_t lrows[16][kD];
  const long long bh = blockIdx.x;
  const int b = (int)(bh / H);
  const int p = pos[b];
  if (p < 0 || p > S - t_new) return;  // flagged by k_quant_dsq
  const int e = p + t_new, k0 = e & ~63;
  const int r0 = max(p, k0) - k0, r1 = e - k0;
  const int li = threadIdx.x & 15, rg = threadIdx.x >> 4;
  // rows r0 .. r1 - 1 in passes of 16; every lane of a 16-lane row group
  // takes the same branch, and the V exchange is wave-local
  for (int rb = r0; rb < r1; rb += 16) {
    const int r = rb + rg;
    if (r < r1) {
      const long long src = (bh * t_new + (k0 + r - p)) * kD + li * 8;
      store_row_f16<false>(kt.codes16 + (bh * 64 + r) * 256, li, ld_row8(xk + src), nullptr);
      store_row_f16<true>(vt.codes16 + (bh * 64 + r) * 256, li, ld_row8(xv + src), lrows[rg]);
      if (li == 0) kt.oscale[bh * 64 + r] = score[bh * t_new + (k0 + r - p)];
    }
  }
}

constexpr int kThreads = 256;
constexpr long long kRowBlocks = 4096;  // grid bound of the row kernels (blocks of 32 rows)

}  // namespace

// ---------------------------------------------------------------------------
// Launchers

hipError_t launch_quant_token_kv(const CacheArgs& c, const uint16_t* xk, const uint16_t* xv, int t_new,
                                 const int* pos, hipStream_t st) {
  const TensorArgs& t = c.k;
  const PageMap pm{c.pages, c.ptok, c.npages};
  const long long rows = (long long)c.B * c.H * t_new;
  if (rows >= (1ll << 31)) return hipErrorInvalidValue;  // (rejected by kvq_quant_append)
  const FastDiv ft = make_fastdiv((uint32_t)t_new), fh = make_fastdiv((uint32_t)c.H);
  const dim3 grid((unsigned)std::min<long long>((rows + 31) / 32, kRowBlocks), 2);
#define KVQ_TOK(BITS, SYM, GE, F8)                                                                       \
  hipLaunchKernelGGL((k_quant_token_kv<BITS, SYM, GE, F8>), grid, dim3(kThreads), 0, st, xk, xv, ft, fh, \
                     c.S, pos, (uint32_t)rows, c.k, c.v, c.status, pm)
#define KVQ_TOK_G(BITS, SYM, F8)                  \
  switch (t.group) {                              \
    case 32: KVQ_TOK(BITS, SYM, 32, F8); break;   \
    case 64: KVQ_TOK(BITS, SYM, 64, F8); break;   \
    case 128: KVQ_TOK(BITS, SYM, 128, F8); break; \
    default: return hipErrorInvalidValue;         \
  }
  if (t.fmt == 1 || t.fmt == 2) {
    if (t.bits != 8 || t.sym) return hipErrorInvalidValue;
    if (t.fmt == 1) {
      KVQ_TOK_G(8, false, 1);
    } else {
      KVQ_TOK_G(8, false, 2);
    }
  } else if (t.sym) {
    if (t.bits != 8) return hipErrorInvalidValue;
    KVQ_TOK_G(8, true, 0);
  } else if (t.bits == 8) {
    KVQ_TOK_G(8, false, 0);
  } else if (t.bits == 4) {
    KVQ_TOK_G(4, false, 0);
  } else if (t.bits == 2) {
    KVQ_TOK_G(2, false, 0);
  } else {
    return hipErrorInvalidValue;
  }
#undef KVQ_TOK_G
#undef KVQ_TOK
  return hipGetLastError();
}

hipError_t launch_quant_token(const CacheArgs& c, const TensorArgs& t, bool vl, const uint16_t* x,
                              int t_new, const int* pos, hipStream_t st) {
  const PageMap pm{c.pages, c.ptok, c.npages};
  const long long rows = (long long)c.B * c.H * t_new;
  if (rows >= (1ll << 31)) return hipErrorInvalidValue;  // (rejected by kvq_quant_append)
  const FastDiv ft = make_fastdiv((uint32_t)t_new), fh = make_fastdiv((uint32_t)c.H);
  const uint32_t nr = (uint32_t)rows;
  const dim3 grid((unsigned)std::min<long long>((rows + 31) / 32, kRowBlocks));
#define KVQ_TOK(BITS, SYM, GE, F8)                                                                  \
  do {                                                                                              \
    if (vl)                                                                                         \
      hipLaunchKernelGGL((k_quant_token<BITS, SYM, GE, true, F8>), grid, dim3(kThreads), 0, st, x,  \
                         ft, fh, c.S, pos, nr, t.codes, t.scale, t.zero, c.status, pm);             \
    else                                                                                            \
      hipLaunchKernelGGL((k_quant_token<BITS, SYM, GE, false, F8>), grid, dim3(kThreads), 0, st, x, \
                         ft, fh, c.S, pos, nr, t.codes, t.scale, t.zero, c.status, pm);             \
  } while (0)
#define KVQ_TOK_G(BITS, SYM, F8)                  \
  switch (t.group) {                              \
    case 32: KVQ_TOK(BITS, SYM, 32, F8); break;   \
    case 64: KVQ_TOK(BITS, SYM, 64, F8); break;   \
    case 128: KVQ_TOK(BITS, SYM, 128, F8); break; \
    default: return hipErrorInvalidValue;         \
  }
  if (t.fmt == 1 || t.fmt == 2) {
    if (t.bits != 8 || t.sym) return hipErrorInvalidValue;
    if (t.fmt == 1) {
      KVQ_TOK_G(8, false, 1);
    } else {
      KVQ_TOK_G(8, false, 2);
    }
  } else if (t.sym) {
    if (t.bits != 8) return hipErrorInvalidValue;
    KVQ_TOK_G(8, true, 0);
  } else if (t.bits == 8) {
    KVQ_TOK_G(8, false, 0);
  } else if (t.bits == 4) {
    KVQ_TOK_G(4, false, 0);
  } else if (t.bits == 2) {
    KVQ_TOK_G(2, false, 0);
  } else {
    return hipErrorInvalidValue;
  }
#undef KVQ_TOK_G
#undef KVQ_TOK
  return hipGetLastError();
}

hipError_t launch_quant_channel(const CacheArgs& c, const TensorArgs& t, const uint16_t* x, int t_new,
                                const int* pos, hipStream_t st) {
  if (t.group != 64 || t_new < 1) return hipErrorInvalidValue;
  // blocks an append of t_new tokens can complete: floor((p mod 64 + t_new) / 64) <= (t_new + 63) / 64
  const dim3 grid((unsigned)((t_new + 63) / 64), (unsigned)(c.B * c.H));
  const PageMap pm{c.pages, c.ptok, c.npages};
  if (t.bits == 8)
    hipLaunchKernelGGL(k_quant_channel<8>, grid, dim3(kThreads), 0, st, x, t_new, c.H, c.S, pos,
                       t.codes, t.scale, t.zero, t.codes16, c.status, pm);
  else if (t.bits == 4)
    hipLaunchKernelGGL(k_quant_channel<4>, grid, dim3(kThreads), 0, st, x, t_new, c.H, c.S, pos,
                       t.codes, t.scale, t.zero, t.codes16, c.status, pm);
  else if (t.bits == 2)
    hipLaunchKernelGGL(k_quant_channel<2>, grid, dim3(kThreads), 0, st, x, t_new, c.H, c.S, pos,
                       t.codes, t.scale, t.zero, t.codes16, c.status, pm);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_channel_tail, dim3((unsigned)(c.B * c.H)), dim3(kThreads), 0, st, x, t_new, c.H,
                     c.S, pos, t.codes16);
  return hipGetLastError();
}

hipError_t launch_quant_mixed(const CacheArgs& c, const TensorArgs& t, bool vl, const uint16_t* x,
                              const int* pos, hipStream_t st) {
  const int C = c.S / c.chunk_tokens;
  const dim3 grid((unsigned)((C + kMixSlots - 1) / kMixSlots), (unsigned)(c.B * c.H));
  const ClassPages cp{c.pages, c.ptok, c.npages, c.B};
#define KVQ_MIX(GE)                                                                                \
  do {                                                                                             \
    if (vl)                                                                                        \
      hipLaunchKernelGGL((k_quant_mixed<GE, true>), grid, dim3(kThreads), 0, st, x, c.H, c.S,      \
                         c.chunk_tokens, C, pos, c.perm, c.seg, t.codes16, t.codes, t.scale,       \
                         t.zero, t.codes2, t.scale2, t.zero2, c.status, cp);                       \
    else                                                                                           \
      hipLaunchKernelGGL((k_quant_mixed<GE, false>), grid, dim3(kThreads), 0, st, x, c.H, c.S,     \
                         c.chunk_tokens, C, pos, c.perm, c.seg, t.codes16, t.codes, t.scale,       \
                         t.zero, t.codes2, t.scale2, t.zero2, c.status, cp);                       \
  } while (0)
  switch (t.group) {
    case 32: KVQ_MIX(32); break;
    case 64: KVQ_MIX(64); break;
    case 128: KVQ_MIX(128); break;
    default: return hipErrorInvalidValue;
  }
#undef KVQ_MIX
  return hipGetLastError();
}

hipError_t launch_chunk_append(const CacheArgs& c, const TensorArgs& t, bool vl, const uint16_t* x,
                               int t_new, const int* pos, const uint8_t* bits, int n_new, hipStream_t st) {
  const int C = c.S / c.chunk_tokens, CT = c.chunk_tokens;
  const ClassPages cp{c.pages, c.ptok, c.npages, c.B};
  hipError_t e = hipSuccess;
  // chunk 0 first, then the others (see k_chunk_append)
  for (int part = 0; part < 2 && e == hipSuccess; ++part) {
    const int i0 = part, cnt = part ? n_new - 1 : 1;
    if (cnt <= 0) break;
    const dim3 grid((unsigned)cnt, (unsigned)(c.B * c.H));
#define KVQ_CA(GE)                                                                                   \
  do {                                                                                               \
    if (vl)                                                                                          \
      hipLaunchKernelGGL((k_chunk_append<GE, true>), grid, dim3(kThreads), 0, st, i0, x, t_new, c.H, \
                         c.S, CT, C, pos, bits, n_new, c.seg, t.codes16, t.codes, t.scale, t.zero,   \
                         t.codes2, t.scale2, t.zero2, c.status, cp);                                \
    else                                                                                             \
      hipLaunchKernelGGL((k_chunk_append<GE, false>), grid, dim3(kThreads), 0, st, i0, x, t_new,     \
                         c.H, c.S, CT, C, pos, bits, n_new, c.seg, t.codes16, t.codes, t.scale,      \
                         t.zero, t.codes2, t.scale2, t.zero2, c.status, cp);                        \
  } while (0)
    switch (t.group) {
      case 32: KVQ_CA(32); break;
      case 64: KVQ_CA(64); break;
      case 128: KVQ_CA(128); break;
      default: return hipErrorInvalidValue;
    }
#undef KVQ_CA
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (vl)
    hipLaunchKernelGGL((k_chunk_wait<true>), dim3((unsigned)(c.B * c.H)), dim3(kThreads), 0, st, x, t_new,
                       c.H, c.S, CT, C, pos, c.seg, t.codes16, c.status, cp);
  else
    hipLaunchKernelGGL((k_chunk_wait<false>), dim3((unsigned)(c.B * c.H)), dim3(kThreads), 0, st, x,
                       t_new, c.H, c.S, CT, C, pos, c.seg, t.codes16, c.status, cp);
  return hipGetLastError();
}

hipError_t launch_quant_oaken(const CacheArgs& c, const TensorArgs& t, bool vl, const uint16_t* x,
                              int t_new, const int* pos, hipStream_t st) {
  const dim3 grid((unsigned)(c.B * c.H));
  const PageMap pm{c.pages, c.ptok, c.npages};
#define KVQ_OAK(GE)                                                                               \
  do {                                                                                            \
    if (vl)                                                                                       \
      hipLaunchKernelGGL((k_quant_oaken<GE, true>), grid, dim3(kThreads), 0, st, x, t_new, c.H,    \
                         c.S, pos, t.thr_lo, t.thr_hi, t.sparse_cap, t.codes, t.scale, t.zero,    \
                         t.oscale, t.rowptr, t.sparse, c.status, pm);                             \
    else                                                                                          \
      hipLaunchKernelGGL((k_quant_oaken<GE, false>), grid, dim3(kThreads), 0, st, x, t_new, c.H,   \
                         c.S, pos, t.thr_lo, t.thr_hi, t.sparse_cap, t.codes, t.scale, t.zero,    \
                         t.oscale, t.rowptr, t.sparse, c.status, pm);                             \
  } while (0)
  switch (t.group) {
    case 32: KVQ_OAK(32); break;
    case 64: KVQ_OAK(64); break;
    case 128: KVQ_OAK(128); break;
    default: return hipErrorInvalidValue;
  }
#undef KVQ_OAK
  return hipGetLastError();
}

hipError_t launch_quant_oaken_one(const CacheArgs& c, const uint16_t* xk, const uint16_t* xv,
                                 const int* pos, hipStream_t st) {
  const int BH = c.B * c.H;
  const PageMap pm{c.pages, c.ptok, c.npages};
  const dim3 grid((unsigned)((BH + 15) / 16), 2);
  switch (c.k.group) {
    case 32: hipLaunchKernelGGL((k_quant_oaken_one<32>), grid, dim3(kThreads), 0, st, xk, xv, BH, c.H, c.S, pos, c.k, c.v, c.status, pm); break;
    case 64: hipLaunchKernelGGL((k_quant_oaken_one<64>), grid, dim3(kThreads), 0, st, xk, xv, BH, c.H, c.S, pos, c.k, c.v, c.status, pm); break;
    case 128: hipLaunchKernelGGL((k_quant_oaken_one<128>), grid, dim3(kThreads), 0, st, xk, xv, BH, c.H, c.S, pos, c.k, c.v, c.status, pm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_dsq(const CacheArgs& c, const uint16_t* xk, const uint16_t* xv, const float* score,
                            int t_new, const int* pos, hipStream_t st) {
  // groups an append of t_new tokens can complete: floor((p mod 64 + t_new) / 64) <= (t_new + 63) / 64
  const dim3 grid((unsigned)((t_new + 63) / 64), (unsigned)(c.B * c.H));
  const PageMap pm{c.pages, c.ptok, c.npages};
  hipLaunchKernelGGL(k_quant_dsq, grid, dim3(kThreads), 0, st, xk, xv, score, t_new, c.H, c.S, c.dsq_sig, pos,
                     c.k, c.v, c.dsq_mask, c.status, pm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dsq_tail, dim3((unsigned)(c.B * c.H)), dim3(kThreads), 0, st, xk, xv, score, t_new, c.H,
                     c.S, pos, c.k, c.v);
  return hipGetLastError();
}

}  // namespace kvq
