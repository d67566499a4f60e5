// Split-sequence decode attention with the dequantization fused into the
// q.K and p.V loops ([TurboQuant page] §2.3, end: no separate dequant pass;
// [Cocktail page] §3.2.3: attention per block, block outputs merged).
//
// Work decomposition (gfx950, wave64):
//  - grid (split, kv_head x query_tile, batch); a workgroup is 4 waves.  The
//    split's token range is cut into 64-row (32 for fp16) tiles that the
//    waves take in turn, so the four waves stream adjacent memory.
//  - Inside a wave, a token row is handled by LPR lanes ("lanes per row");
//    lane (r, sub) owns channels [sub*DPL, (sub+1)*DPL) of rows
//    tile + r*NI + i, i < NI, so the rows a lane reads are consecutive and
//    their scales / zero-points come from one vector load.
//  - q.k_hat per row: scale and zero-point are applied once per group,
//    s * (sum q_d c_d - z * sum q_d), on binary32 codes widened from the
//    packed bytes; partial sums are reduced over the LPR lanes.
//  - Online softmax in base 2 (q pre-scaled by sm_scale*log2 e) with a
//    wave-uniform running max per query; p.v_hat accumulates
//    sum p s c - sum p s z per lane.
//  - Each wave folds its state into an LDS record (m, l, o[128]); the four
//    records are merged at the end and written as one split partial (or the
//    final output when there is one split).  kvq_merge combines splits:
//    M = max m_j, L = sum l_j 2^(m_j - M), o = sum 2^(m_j - M) o_j / L.
#pragma once
#include "kvq_dev.h"

namespace kvq {

constexpr int kNW = 4;  // waves per workgroup

struct DecodeParams {
  int B, H, S, Hq, G, qtiles, max_len, num_splits, split_len, chunk_tokens;
  float qscale;
  const uint16_t* q;
  const int* seq_len;
  float* out;
  float* ws;
  const int* seg;
  unsigned* status;
  TensorArgs k, v;
};

enum CodecKind { kTok = 0, kF16 = 1, kChan = 2, kOaken = 3 };

// Token-axis groups: per row, NG groups of 128/NG channels.
template <int BITS_, bool SYM_, int NG_>
struct TokCodec {
  static constexpr int kind = kTok, BITS = BITS_, NG = NG_, RB = kD * BITS_ / 8;
  static constexpr bool SYM = SYM_;
  static constexpr int MIN_LPR = (RB / 16 > NG_) ? RB / 16 : NG_;
  const uint8_t* codes;
  const float* scale;
  const uint8_t* zero;
};

// Raw fp16 rows.
struct F16Codec {
  static constexpr int kind = kF16, BITS = 16, NG = 1, RB = 2 * kD, MIN_LPR = 16;
  static constexpr bool SYM = false;
  const uint8_t* codes;
};

// Channel-axis groups of 64 tokens (K only): scale/zero [S/64][128].
template <int BITS_>
struct ChanCodec {
  static constexpr int kind = kChan, BITS = BITS_, NG = 1, RB = kD * BITS_ / 8, MIN_LPR = RB / 16;
  static constexpr bool SYM = false;
  const uint8_t* codes;
  const float* scale;
  const uint8_t* zero;
};

// Oaken: dense INT4 token-axis body plus the row's sparse outer entries.
template <int NG_>
struct OakenCodec {
  static constexpr int kind = kOaken, BITS = 4, NG = NG_, RB = 64, MIN_LPR = NG_ > 4 ? NG_ : 4;
  static constexpr bool SYM = false;
  const uint8_t* codes;
  const float* scale;
  const uint8_t* zero;
  const float* oscale;
  const uint32_t* rowptr;
  const uint16_t* sparse;
  long long cap;
  float t_lo, t_hi;
};

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int NI, int NG>
__device__ __forceinline__ void load_scale(const float* base, int row0, int j, float* out) {
  if constexpr (NG == 1) {
    if constexpr (NI >= 4) {
#pragma unroll
      for (int k = 0; k < NI / 4; ++k) {
        const float4 v = reinterpret_cast<const float4*>(base + row0)[k];
        out[4 * k] = v.x; out[4 * k + 1] = v.y; out[4 * k + 2] = v.z; out[4 * k + 3] = v.w;
      }
    } else if constexpr (NI == 2) {
      const float2 v = *reinterpret_cast<const float2*>(base + row0);
      out[0] = v.x; out[1] = v.y;
    } else {
      out[0] = base[row0];
    }
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i) out[i] = base[(long long)(row0 + i) * NG + j];
  }
}

template <int NI, int NG>
__device__ __forceinline__ void load_zero(const uint8_t* base, int row0, int j, float* out) {
  if constexpr (NG == 1) {
    uint32_t w[(NI + 3) / 4];
    if constexpr (NI == 16) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + row0);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (NI == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(base + row0);
      w[0] = v.x; w[1] = v.y;
    } else if constexpr (NI == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(base + row0);
    } else if constexpr (NI == 2) {
      w[0] = *reinterpret_cast<const uint16_t*>(base + row0);
    } else {
      w[0] = base[row0];
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) out[i] = (float)((w[i / 4] >> (8 * (i % 4))) & 0xFFu);
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i) out[i] = (float)base[(long long)(row0 + i) * NG + j];
  }
}

// Row meta (scale, zero-point) of a row-oriented codec for the lane's group.
template <class C, int NI>
__device__ __forceinline__ void row_meta(const C& c, int row0, int j, float* s, float* z) {
  if constexpr (C::kind == kTok || C::kind == kOaken) {
    load_scale<NI, C::NG>(c.scale, row0, j, s);
    if constexpr (C::SYM) {
#pragma unroll
      for (int i = 0; i < NI; ++i) z[i] = 128.0f;  // codes are read with the sign bit flipped
    } else {
      load_zero<NI, C::NG>(c.zero, row0, j, z);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      s[i] = 1.0f;
      z[i] = 0.0f;
    }
  }
}

// Sparse outer entries of one row, the ones lane `sub` of LPR handles:
// calls f(channel, x_hat) for each.
template <int LPR, int NG, class F>
__device__ __forceinline__ void for_outer(const OakenCodec<NG>& c, int row, uint32_t a, uint32_t e_end,
                                          int sub, F&& f) {
  const unsigned long long cap = (unsigned long long)c.cap;
  for (uint32_t e = a + sub; e < e_end && (unsigned long long)e < cap; e += LPR) {
    const uint32_t en = c.sparse[e];
    const int d = (int)(en & 127u);
    const float mag = (float)((en >> 8) & 31u);
    const float so = c.oscale[(long long)row * NG + d / (kD / NG)];
    const float xh = ((en >> 7) & 1u) ? c.t_hi + mag * so : c.t_lo - mag * so;
    f(d, xh);
  }
}

template <int LPR, int GT, int TR, class KC, class VC>
__device__ __forceinline__ void attend_segment(const KC& kc, const VC& vc, int t0, int t1, int wave,
                                               const float* __restrict__ q_lds, float* osp,
                                               float* canon) {
  constexpr int RPW = 64 / LPR, NI = TR / RPW, DPL = kD / LPR;
  constexpr int KWD = KC::RB / LPR / 4, VWD = VC::RB / LPR / 4;
  static_assert(NI >= 1 && KWD >= 1 && VWD >= 1, "lane layout");
  constexpr bool kOak = KC::kind == kOaken, vOak = VC::kind == kOaken;
  const int lane = threadIdx.x & 63, sub = lane % LPR, r = lane / LPR;
  const int kj = sub / (LPR / KC::NG), vj = sub / (LPR / VC::NG);

  float q[GT][DPL], qsum[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    qsum[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      q[g][e] = q_lds[g * kD + sub * DPL + e];
      qsum[g] += q[g][e];
    }
  }
  float m[GT], l[GT], bias[GT], o[GT][DPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
    bias[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[g][e] = 0.0f;
  }

  const int tb = t0 & ~(TR - 1);
  if (tb + wave * TR >= t1) return;  // this wave has no tile (wave-uniform)
  for (int tile = tb + wave * TR; tile < t1; tile += kNW * TR) {
    const int row0 = tile + r * NI;
    uint32_t kw[NI][KWD], vw[NI][VWD];
#pragma unroll
    for (int i = 0; i < NI; ++i)
      load_words<KWD>(kc.codes + (long long)(row0 + i) * KC::RB + sub * (KWD * 4), kw[i]);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      load_words<VWD>(vc.codes + (long long)(row0 + i) * VC::RB + sub * (VWD * 4), vw[i]);
    float ks[NI], kz[NI], vs[NI], vz[NI];
    row_meta<KC, NI>(kc, row0, kj, ks, kz);
    row_meta<VC, NI>(vc, row0, vj, vs, vz);
    bool valid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      valid[i] = (row0 + i >= t0) && (row0 + i < t1);
      if (!valid[i]) {
        ks[i] = 0.0f; kz[i] = 0.0f; vs[i] = 0.0f; vz[i] = 0.0f;
        if constexpr (VC::kind == kF16) {
#pragma unroll
          for (int k = 0; k < VWD; ++k) vw[i][k] = 0u;
        }
      }
    }
    uint32_t krp[NI + 1], vrp[NI + 1];
    if constexpr (kOak) {
#pragma unroll
      for (int i = 0; i <= NI; ++i) krp[i] = kc.rowptr[row0 + i];
    }
    if constexpr (vOak) {
#pragma unroll
      for (int i = 0; i <= NI; ++i) vrp[i] = vc.rowptr[row0 + i];
    }

    // ---- scores ----
    float qs[GT][DPL], cb[GT];
    if constexpr (KC::kind == kChan) {
      const int blk = tile >> 6;
      float sc[DPL], zc[DPL];
      const float* sp = kc.scale + (long long)blk * kD + sub * DPL;
      const uint8_t* zp = kc.zero + (long long)blk * kD + sub * DPL;
#pragma unroll
      for (int e = 0; e < DPL; e += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(sp + e);
        sc[e] = v4.x; sc[e + 1] = v4.y; sc[e + 2] = v4.z; sc[e + 3] = v4.w;
        const uint32_t zw = *reinterpret_cast<const uint32_t*>(zp + e);
#pragma unroll
        for (int k = 0; k < 4; ++k) zc[e + k] = (float)((zw >> (8 * k)) & 0xFFu);
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        cb[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
          qs[g][e] = q[g][e] * sc[e];
          cb[g] = fmaf(qs[g][e], zc[e], cb[g]);
        }
      }
    }
    float sco[GT][NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint32_t w[KWD];
#pragma unroll
      for (int k = 0; k < KWD; ++k) w[k] = KC::SYM ? (kw[i][k] ^ 0x80808080u) : kw[i][k];
      float c[DPL];
      codes_to_float<KC::BITS, DPL>(w, c);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float acc = 0.0f;
        if constexpr (KC::kind == kChan) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc = fmaf(qs[g][e], c[e], acc);
          sco[g][i] = acc - cb[g];
        } else {
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc = fmaf(q[g][e], c[e], acc);
          sco[g][i] = (KC::kind == kF16) ? acc : ks[i] * fmaf(-kz[i], qsum[g], acc);
        }
      }
      if constexpr (kOak) {
        if (valid[i])
          for_outer<LPR>(kc, row0 + i, krp[i], krp[i + 1], sub, [&](int d, float xh) {
#pragma unroll
            for (int g = 0; g < GT; ++g) sco[g][i] = fmaf(q_lds[g * kD + d], xh, sco[g][i]);
          });
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float sfull = sum_lanes<1, LPR>(sco[g][i]);
        sco[g][i] = valid[i] ? sfull : -INFINITY;
      }

    // ---- online softmax ----
    float p[GT][NI];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float tm = sco[g][0];
#pragma unroll
      for (int i = 1; i < NI; ++i) tm = fmaxf(tm, sco[g][i]);
      tm = max_lanes<LPR, 64>(tm);
      if (tm > m[g]) {
        const float a = fexp2(m[g] - tm);
        l[g] *= a;
        bias[g] *= a;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[g][e] *= a;
        if constexpr (vOak) {
          osp[g * kD + lane] *= a;
          osp[g * kD + 64 + lane] *= a;
        }
        m[g] = tm;
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        p[g][i] = fexp2(sco[g][i] - m[g]);
        l[g] += p[g][i];
      }
    }

    // ---- values ----
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint32_t w[VWD];
#pragma unroll
      for (int k = 0; k < VWD; ++k) w[k] = VC::SYM ? (vw[i][k] ^ 0x80808080u) : vw[i][k];
      float c[DPL];
      codes_to_float<VC::BITS, DPL>(w, c);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float wgt = p[g][i] * vs[i];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[g][e] = fmaf(wgt, c[e], o[g][e]);
        bias[g] = fmaf(wgt, vz[i], bias[g]);
      }
      if constexpr (vOak) {
        if (valid[i])
          for_outer<LPR>(vc, row0 + i, vrp[i], vrp[i + 1], sub, [&](int d, float xh) {
#pragma unroll
            for (int g = 0; g < GT; ++g) atomicAdd(&osp[g * kD + d], p[g][i] * xh);
          });
      }
    }
  }

  // ---- fold this wave's state into its LDS record ----
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    const float L = sum_lanes<LPR, 64>(l[g]);
    float ov[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) ov[e] = sum_lanes<LPR, 64>(o[g][e] - bias[g]);
    float* cg = canon + g * (kD + 2);
    if (r == 0) {
      const float cm = cg[kD], cl = cg[kD + 1];
      const float M = fmaxf(cm, m[g]);
      const float a1 = fexp2(cm - M), a2 = fexp2(m[g] - M);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        float add = ov[e];
        if constexpr (vOak) add += osp[g * kD + sub * DPL + e];
        cg[sub * DPL + e] = cg[sub * DPL + e] * a1 + add * a2;
      }
      __builtin_amdgcn_wave_barrier();
      if (sub == 0) {
        cg[kD] = M;
        cg[kD + 1] = cl * a1 + L * a2;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (vOak) {
      osp[g * kD + lane] = 0.0f;
      osp[g * kD + 64 + lane] = 0.0f;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Load the query tile into LDS (pre-scaled to base-2 logits) and reset the
// per-wave records.  Ends with a workgroup barrier.
template <int GT, bool OSP>
__device__ __forceinline__ void decode_prologue(const DecodeParams& P, int b, int kvh, int qt,
                                                float* q_lds, float* canon, float* osp) {
  for (int idx = threadIdx.x; idx < GT * kD; idx += blockDim.x) {
    const int g = idx / kD, d = idx % kD, gq = qt * GT + g;
    float v = 0.0f;
    if (gq < P.G) v = h2f(P.q[((long long)b * P.Hq + (long long)kvh * P.G + gq) * kD + d]) * P.qscale;
    q_lds[idx] = v;
  }
  for (int idx = threadIdx.x; idx < kNW * GT * (kD + 2); idx += blockDim.x)
    canon[idx] = (idx % (kD + 2) == kD) ? -INFINITY : 0.0f;
  if constexpr (OSP)
    for (int idx = threadIdx.x; idx < kNW * GT * kD; idx += blockDim.x) osp[idx] = 0.0f;
  __syncthreads();
}

// Merge the four wave records and write the split partial or the output.
template <int GT>
__device__ __forceinline__ void decode_epilogue(const DecodeParams& P, int b, int kvh, int qt,
                                                int split, const float* canon) {
  __syncthreads();
  for (int idx = threadIdx.x; idx < GT * kD; idx += blockDim.x) {
    const int g = idx / kD, d = idx % kD, gq = qt * GT + g;
    if (gq >= P.G) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, canon[(w * GT + g) * (kD + 2) + kD]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        const float* rec = canon + (w * GT + g) * (kD + 2);
        if (rec[kD] != -INFINITY) {
          const float f = fexp2(rec[kD] - M);
          L = fmaf(f, rec[kD + 1], L);
          O = fmaf(f, rec[d], O);
        }
      }
    }
    const long long hq = (long long)kvh * P.G + gq;
    if (P.num_splits == 1) {
      P.out[((long long)b * P.Hq + hq) * kD + d] = L > 0.0f ? O / L : 0.0f;
    } else {
      float* rec = P.ws + (((long long)b * P.Hq + hq) * P.num_splits + split) * kPartStride;
      rec[4 + d] = O;
      if (d == 0) {
        rec[0] = M;
        rec[1] = L;
      }
    }
  }
}

__device__ __forceinline__ int clamp_len(const DecodeParams& P, int b, bool report) {
  int len = P.seq_len[b];
  if (len < 0 || len > P.max_len) {
    if (report) set_flag(P.status, kFlagLenRange);
    len = len < 0 ? 0 : P.max_len;
  }
  return len;
}

template <class C>
__device__ __forceinline__ C make_codec(const TensorArgs& t, long long bh, int S);

}  // namespace kvq
