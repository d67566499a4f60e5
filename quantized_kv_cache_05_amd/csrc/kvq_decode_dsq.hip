// Decode over the differential significant-token cache (the KVO-LLM page,
// §3.1): every 64-token group holds up to 16 significant rows (int8 codes,
// per-channel scales) and up to 64 other rows (INT2, groups of 32 channels;
// K rows are differences from the group's base row).  Softmax attention does
// not depend on token order, so the two classes are attended slot by slot.
// A wave takes whole groups (operand layouts as in kvq_attn.h):
//  significant K  the channel scales are folded into the query, A = q_d s_d
//                 split into fp16 hi + lo, B = codes as 384 + c, so
//                 score = C - 384 sum_d q_d s_d;
//  base           base is the mean of the dequantized significant rows, so
//                 q . base is the mean of their scores: base is never read;
//  other K        score = q . base + sum_g s_g (C_g - (4 + z_g) Q_g), as for
//                 the token-axis INT2 cache;
//  softmax        one online update per group over all of its columns;
//  significant V  O_tmp = W B with B = c exactly (codes - 128 in fp16), then
//                 O += s_c O_tmp: the channel scale of output column c;
//  other V        weights p s_g, B = c - z exactly, as for the INT2 cache.
#include "kvq_attn_impl.h"

namespace kvq {
namespace {

constexpr int kSigSlots = 16;  // significant-row slots per group
constexpr int kOthSlots = 64;  // other-row slots per group
constexpr unsigned kSymZsub = 0xE480E480u;  // fp16 pair -(1024 + 128)

// A-operand row that holds query m (see QRows)
template <int QR>
__device__ __forceinline__ int arow_of_query(int m) {
  return QR == 1 ? 0 : (QR == 4 ? 4 * m : m);
}

template <int QR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_dsq(AttnParams P) {
  using QRW = QRows<QR>;
  constexpr int R = QR, GI = QRW::GI;
  __shared__ AttnLds<QR, 4> L;
  const int split = blockIdx.x, qt = blockIdx.y % P.qtiles, kvh = blockIdx.y / P.qtiles, b = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63, n16 = lane & 15, q4 = lane >> 4;
  const int nq = min(QR, P.G - qt * QR);
  u4_t qop[4];
  attn_prologue<QR, 4>(P, L, b, kvh, qt, nq, qop);
  const bool reporter = split == 0 && blockIdx.y == 0 && threadIdx.x == 0;
  const int len = clamp_seq_len(P, b, reporter);
  if ((len & 63) && reporter) set_flag(P.status, kFlagLenRange);
  const int g0 = (split * P.split_len) >> 6;  // split_len is a multiple of 64
  const int g1 = min(len >> 6, g0 + (P.split_len >> 6));
  const int nsig = P.dsq_sig, noth = kOthSlots - nsig;
  const float fnsig = (float)nsig;
  const int aq = QRW::arow_query(n16);
  const int mr = max(aq, 0);
  auto& W = L.u.wave[wave];
  SoftState<GI> st;
  soft_init(st);
  const long long bh = (long long)b * P.H + kvh;
  const long long Q = P.S / 64;
  const f4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int grp = g0 + wave; grp < g1; grp += kNW) {
    const long long gb = bh * Q + grp;
    const uint8_t* ksig = P.k.codes + gb * kSigSlots * kD;
    const uint8_t* vsig = P.v.codes + gb * kSigSlots * kD;
    const float* kss = P.k.scale + gb * kD;
    const float* vss = P.v.scale + gb * kD;
    const TokView ko{P.k.codes2 + gb * kOthSlots * 32, P.k.scale2 + gb * kOthSlots * 4,
                     P.k.zero2 + gb * kOthSlots * 4};
    const TokView vo{P.v.codes2 + gb * kOthSlots * 32, P.v.scale2 + gb * kOthSlots * 4,
                     P.v.zero2 + gb * kOthSlots * 4};
    // ---- loads (slots past the class counts are not read) ----
    const bool okS = n16 < nsig;
    KI8<true> kS;
    kS.a = u4_t{0u, 0u, 0u, 0u};
    kS.b = kS.a;
    if (okS) kS.load(ksig + n16 * kD, q4);
    KI2 kO[4];
    float sk[4][4], zk[4][4], sv[4][4], zd[4][4];
    bool okO[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int slot = 16 * cb + n16;
      okO[cb] = slot < noth;
      kO[cb].r = u2_t{0u, 0u};
#pragma unroll
      for (int g = 0; g < 4; ++g) sk[cb][g] = zk[cb][g] = sv[cb][g] = 0.0f;
      if (okO[cb]) {
        kO[cb].load(ko.codes + slot * KI2::RB, q4);
        load_tok_meta<4, false>(ko, slot, sk[cb], zk[cb]);
        load_tok_meta<4, true>(vo, slot, sv[cb], zd[cb]);
      }
    }
    float4 ksc[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c0 = 32 * s + 8 * q4;
      ksc[s][0] = *reinterpret_cast<const float4*>(kss + c0);
      ksc[s][1] = *reinterpret_cast<const float4*>(kss + c0 + 4);
    }
    VI8<true> vS;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 8 * q4 + k;
      vS.w0[k] = vS.w1[k] = 0x80808080u;  // code 0
      if (r < nsig) {
        const u2_t x = ld_nt<u2_t>(vsig + r * kD + n16 * 8);
        const unsigned x0 = x[0], x1 = x[1];
        vS.w0[k] = x0 ^ 0x80808080u;
        vS.w1[k] = x1 ^ 0x80808080u;
      }
    }
    float vsc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vsc[j] = vss[16 * j + n16];
    // ---- significant K: scaled query (hi + lo) and its channel sum ----
    u4_t qh[4], ql[4];
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c0 = 32 * s + 8 * q4;
      const float sc[8] = {ksc[s][0].x, ksc[s][0].y, ksc[s][0].z, ksc[s][0].w,
                           ksc[s][1].x, ksc[s][1].y, ksc[s][1].z, ksc[s][1].w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float a = L.q[mr][c0 + v] * sc[v], bq = L.q[mr][c0 + v + 4] * sc[v + 4];
        unsigned hi, lo;
        split_pair(a, bq, hi, lo);
        qh[s][v] = aq < 0 ? 0u : hi;
        ql[s][v] = aq < 0 ? 0u : lo;
        part += a + bq;
      }
    }
    // lanes of one A row differ in q4: their sum covers the row's 128 channels
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    float qs[GI];
#pragma unroll
    for (int i = 0; i < GI; ++i) qs[i] = __shfl(part, arow_of_query<QR>(QRW::slot_query(q4, i)), 64);
    f4_t c = zero4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u4_t kb = kS.slice(s);
      c = mfma(qh[s], kb, c);
      c = mfma(ql[s], kb, c);
    }
    float rawS[GI], mu[GI];
#pragma unroll
    for (int i = 0; i < GI; ++i) {
      rawS[i] = c[QRW::slot_elem(i)] - (float)KI8<true>::OFF * qs[i];
      mu[i] = sum16(okS ? rawS[i] : 0.0f) / fnsig;  // q . base
    }
    // ---- other K: differences from the base ----
    float rawO[4][GI];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      f4_t cc[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) cc[g] = mfma(qop[g], kO[cb].slice(g), zero4);
#pragma unroll
      for (int i = 0; i < GI; ++i) {
        const int m = min(QRW::slot_query(q4, i), R - 1);
        const int e = QRW::slot_elem(i);
        float a = mu[i];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          a = fmaf(sk[cb][g], fmaf(-(zk[cb][g] + (float)KI2::OFF), L.qg[m][g], cc[g][e]), a);
        rawO[cb][i] = a;
      }
    }
    // ---- online softmax (base 2), one update for the group ----
    float pS[GI], pO[4][GI];
    bool grow = false;
    float alpha[GI];
#pragma unroll
    for (int i = 0; i < GI; ++i) {
      const float ss = okS ? rawS[i] * P.qscale : -INFINITY;
      float so[4];
      float tm = ss;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        so[cb] = okO[cb] ? rawO[cb][i] * P.qscale : -INFINITY;
        tm = fmaxf(tm, so[cb]);
      }
      tm = max16(tm);
      const float mn = fmaxf(st.m[i], tm);
      alpha[i] = mn == -INFINITY ? 1.0f : fexp2(st.m[i] - mn);
      grow |= mn > st.m[i];
      st.m[i] = mn;
      pS[i] = okS ? fexp2(ss - mn) : 0.0f;
      float lsum = pS[i];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        pO[cb][i] = okO[cb] ? fexp2(so[cb] - mn) : 0.0f;
        lsum += pO[cb][i];
      }
      rawS[i] = lsum;  // reused: this lane's share of the group's weight sum
    }
    if (__any(grow)) {
#pragma unroll
      for (int i = 0; i < GI; ++i) {
        st.l[i] *= alpha[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) st.o[j][QRW::slot_elem(i)] *= alpha[i];
      }
    }
#pragma unroll
    for (int i = 0; i < GI; ++i) st.l[i] += rawS[i];
    // ---- significant V: W (16 slots, the other 16 zero) times the codes ----
#pragma unroll
    for (int i = 0; i < GI; ++i) {
      const int m = QRW::slot_query(q4, i);
      unsigned hi, lo;
      split_pair(pS[i], 0.0f, hi, lo);
      if (QRW::slot_owner(q4) && m < R) {
        W.w[0][0][m][n16] = (unsigned short)(hi & 0xFFFFu);
        W.w[0][0][m][16 + n16] = (unsigned short)(hi >> 16);
        W.w[0][1][m][n16] = (unsigned short)(lo & 0xFFFFu);
        W.w[0][1][m][16 + n16] = (unsigned short)(lo >> 16);
      }
    }
    wave_lds_sync();
    {
      u4_t wh = *reinterpret_cast<const u4_t*>(&W.w[0][0][mr][8 * q4]);
      u4_t wl = *reinterpret_cast<const u4_t*>(&W.w[0][1][mr][8 * q4]);
      if (aq < 0) wh = wl = u4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u4_t bb = vS.block(j);
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          const unsigned bv = bb[p2];
          const h2_t x = __builtin_bit_cast(h2_t, bv) + __builtin_bit_cast(h2_t, kSymZsub);
          bb[p2] = __builtin_bit_cast(unsigned, x);
        }
        f4_t t = mfma(wh, bb, zero4);
        t = mfma(wl, bb, t);
        st.o[j] += vsc[j] * t;
      }
    }
    wave_lds_sync();
    // ---- other V: two tiles of 32 slots ----
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int i = 0; i < GI; ++i) {
        const int m = QRW::slot_query(q4, i);
        const bool wr = QRW::slot_owner(q4) && m < R;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          unsigned hi, lo;
          split_pair(pO[2 * tau][i] * sv[2 * tau][g], pO[2 * tau + 1][i] * sv[2 * tau + 1][g], hi, lo);
          if (wr) {
            W.w[g][0][m][n16] = (unsigned short)(hi & 0xFFFFu);
            W.w[g][0][m][16 + n16] = (unsigned short)(hi >> 16);
            W.w[g][1][m][n16] = (unsigned short)(lo & 0xFFFFu);
            W.w[g][1][m][16 + n16] = (unsigned short)(lo >> 16);
          }
        }
      }
      VI2 vO;
      {
        unsigned rr[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int r = 32 * tau + 8 * q4 + k;
          rr[k] = 0u;
          if (r < noth) rr[k] = ld_nt<uint16_t>(vo.codes + r * VI2::RB + n16 * 2);
        }
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) vO.x[p2] = perm(rr[2 * p2 + 1], rr[2 * p2], 0x05040100u);
      }
      u4_t zsub[2][4];
      load_zsub<VI2, 4>(vo, 32 * tau + 8 * q4, zsub);
      wave_lds_sync();
      u4_t wa[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          wa[g][h] = *reinterpret_cast<const u4_t*>(&W.w[g][h][mr][8 * q4]);
          if (aq < 0) wa[g][h] = u4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u4_t bb = vO.block(j);
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          const unsigned bv = bb[p2], zv = zsub[0][j >> 1][p2];
          const h2_t x = __builtin_bit_cast(h2_t, bv) + __builtin_bit_cast(h2_t, zv);
          bb[p2] = __builtin_bit_cast(unsigned, x);
        }
        st.o[j] = mfma(wa[j >> 1][0], bb, st.o[j]);
        st.o[j] = mfma(wa[j >> 1][1], bb, st.o[j]);
      }
      wave_lds_sync();
    }
  }
  wave_record<QR, 4>(L, st, wave, nq);
  finish_split(P, L, b, kvh, qt, split, nq);
}

}  // namespace

hipError_t launch_decode_dsq(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
  if (c.k.group != 32 || c.v.group != 32 || c.dsq_sig < 1 || c.dsq_sig > kSigSlots) return hipErrorInvalidValue;
  const AttnParams P = make_attn_params(c, d);
  const dim3 grid((unsigned)d.num_splits, (unsigned)(c.H * d.qtiles), (unsigned)c.B);
  switch (d.qr) {
    case 1: hipLaunchKernelGGL((k_attn_dsq<1>), grid, dim3(kNW * 64), 0, st, P); break;
    case 4: hipLaunchKernelGGL((k_attn_dsq<4>), grid, dim3(kNW * 64), 0, st, P); break;
    case 16: hipLaunchKernelGGL((k_attn_dsq<16>), grid, dim3(kNW * 64), 0, st, P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
