// Decode over the differential significant-token cache (the KVO-LLM page,
// §3.1): every 64-token group holds up to 16 significant rows (int8 codes,
// per-channel scales) and up to 64 other rows (INT2, groups of 32 channels;
// K rows are differences from the group's base row).  Softmax attention does
// not depend on token order, so the two classes are attended slot by slot.
// A wave takes whole groups (operand layouts as in kvq_attn.h):
//  significant K  the channel scales are folded into the query, A = q_d s_d
//                 split into fp16 hi + lo, B = the signed codes c (widened
//                 exactly, the offset subtracted in fp16), so score = C;
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

// Weight scale of the significant V rows: the weights are p <= 1, so p 2^15
// stays finite in fp16.
constexpr float kSigWS = 32768.0f;


constexpr int kSigSlots = 16;  // significant-row slots per group
constexpr int kOthSlots = 64;  // other-row slots per group
constexpr unsigned kSymZsub = 0xE480E480u;  // fp16 pair -(1024 + 128)

// A-operand row that holds query m (see QRows)
template <int QR>
__device__ __forceinline__ int arow_of_query(int m) {
  return QR == 1 ? 0 : (QR == 4 ? 4 * m : m);
}

template <int QR, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_dsq(AttnParams P) {
  using QRW = QRows<QR>;
  constexpr int R = QR, GI = QRW::GI;
  __shared__ AttnLds<QR, 4, true> L;
  __shared__ float vscl[kNW][kD];  // per wave: the group's significant-V channel scales
  const int split = blockIdx.x, qt = blockIdx.y % P.qtiles, kvh = blockIdx.y / P.qtiles, b = blockIdx.z;
  // wave index as a wave-uniform value: group indices and group base
  // addresses then live in scalar registers, and loads take a scalar base
  // plus a 32-bit lane offset instead of a 64-bit address per lane
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, n16 = lane & 15, q4 = lane >> 4;
  const int nq = min(QR, P.G - qt * QR);
  u4_t qop[4];
  attn_prologue<QR, 4>(P, L, b, kvh, qt, nq, qop);
  // One query (QR 1): every A row holds the query, so row r may carry it on
  // k-step r mod 4 only; the four 32-channel group sums of a token then land
  // in the four C elements of one accumulator (rows 4 q4 + g).
  if constexpr (QR == 1) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if ((threadIdx.x & 3) != s) qop[s] = u4_t{0u, 0u, 0u, 0u};
  }
  const bool reporter = split == 0 && blockIdx.y == 0 && threadIdx.x == 0;
  const int len = clamp_seq_len(P, b, reporter);
  const int g0 = (split * P.split_len) >> 6;  // split_len is a multiple of 64
  const int g1 = min(len >> 6, g0 + (P.split_len >> 6));
  const int nsig = P.dsq_sig, noth = kOthSlots - nsig;
  const float fnsig = (float)nsig;
  const int aq = QRW::arow_query(n16);
  const int mr = max(aq, 0);
  auto& W = L.u.wave[wave];
  SoftState<GI> st;
  soft_init(st);
  // other-V zero-point bias of the lane's token columns, per softmax slot and
  // V group: sum of w (4 + z), in the running softmax frame (see below)
  float vb[GI][4];
#pragma unroll
  for (int i = 0; i < GI; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) vb[i][g] = 0.0f;
  const long long bh = (long long)b * P.H + kvh;
  const long long Q = P.S / 64;
  const f4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  // Loads are branch-free: a lane whose slot lies past its class count reads
  // a slot the wave reads anyway (no extra HBM bytes); its score is masked to
  // -inf and its weight is 0, and what it reads is finite.  A branch around a
  // load would make the compiler wait for it inside the branch.
  //
  // Two-stage pipeline: the K-side data of a group (significant and other K
  // rows, their metadata, the channel scales of the scaled-query table) is
  // loaded during the previous group's V products, into the registers its K
  // products have just released; the V-side data of a group is loaded when
  // its K products start.
  constexpr int NE = 16 * R, PER = (NE + 63) / 64;
  static_assert((NE & (NE - 1)) == 0, "entry count is a power of two");
  const bool okS = n16 < nsig;
  bool okO[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) okO[cb] = 16 * cb + n16 < noth;
  // first slot of group grp in the per-group arrays: contiguous [B][H][S / 64],
  // or, paged, group grp mod g of page pages[b][grp / g] in the pool
  // [npages][H][g] (g = page_tokens / 64 groups per page; an entry outside
  // the pool reads page 0 and flags)
  auto group_base = [&](int grp) -> long long {
    if constexpr (PAGED) {
      const int gsh = P.pshift - 6;
      int pg = P.pages[(long long)b * (P.S >> P.pshift) + (grp >> gsh)];
      if (pg < 0 || pg >= P.npages) {
        if (lane == 0) set_flag(P.status, kFlagPageRange);
        pg = 0;
      }
      return ((long long)pg * P.H + kvh) * (1 << gsh) + (grp & ((1 << gsh) - 1));
    } else {
      return bh * Q + grp;
    }
  };
  struct KSide {
    long long gb;               // the group's base (see group_base)
    float4 tsa[PER], tsb[PER];  // table channel scales, loaded first
    KI8<true> kS;
    KI2 kO[4];
    u4_t skr[4];      // scales of the slot's 4 channel groups (binary32 bits)
    unsigned zkr[4];  // zero-points of the slot's 4 groups (bytes)
  };
  auto load_k = [&](int grp, KSide& d) {
    const long long gb = group_base(grp);
    d.gb = gb;
    const float* kss = P.k.scale + gb * kD;
    // lane l builds table entry (l + 64 k) mod NE (NE = 16, 64 or 256): with
    // one query four lanes build each entry and store the same values, which
    // keeps the build free of branches
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = (lane + 64 * k) & (NE - 1);
      const int c0 = 32 * (e / (4 * R)) + 8 * (e & 3);
      d.tsa[k] = *reinterpret_cast<const float4*>(kss + c0);
      d.tsb[k] = *reinterpret_cast<const float4*>(kss + c0 + 4);
    }
    d.kS.load(P.k.codes + (gb * kSigSlots + (okS ? n16 : 0)) * kD, q4);
    const uint8_t* kc = P.k.codes2 + gb * kOthSlots * 32;
    const float* ks = P.k.scale2 + gb * kOthSlots * 4;
    const uint8_t* kz = P.k.zero2 + gb * kOthSlots * 4;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      // at most 16 significant tokens, so slots 0-47 always exist: only the
      // last column block needs the substitute slot
      const int rs = (cb < 3 || okO[cb]) ? 16 * cb + n16 : 0;
      d.kO[cb].load(kc + rs * KI2::RB, q4);
      d.skr[cb] = ld_nt<u4_t>(ks + rs * 4);
      d.zkr[cb] = ld_nt<unsigned>(kz + rs * 4);
    }
  };
  KSide kd;
  if (g0 + wave < g1) load_k(g0 + wave, kd);
  for (int grp = g0 + wave; grp < g1; grp += kNW) {
    const long long gb = kd.gb;  // this group's base, found with its K side
    const uint8_t* vsig = P.v.codes + gb * kSigSlots * kD;
    const float* vss = P.v.scale + gb * kD;
    const TokView vo{P.v.codes2 + gb * kOthSlots * 32, P.v.scale2 + gb * kOthSlots * 4,
                     P.v.zero2 + gb * kOthSlots * 4};
    // ---- V-side loads of this group ----
    u4_t svr[4];       // V scales of the score column's slot, 4 channel groups
    unsigned zvr[4];   // and its 4 zero-point bytes
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int rs = (cb < 3 || okO[cb]) ? 16 * cb + n16 : 0;
      svr[cb] = ld_nt<u4_t>(vo.scale + rs * 4);
      zvr[cb] = ld_nt<unsigned>(vo.zero + rs * 4);
    }
    // significant V rows 8 q4 + k; rows past the count (all of them for
    // q4 >= 2: the product's k-slots 16-31 carry zero weights) read row 0
    VI8<true> vS;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 8 * q4 + k;
      const u2_t x = ld_nt<u2_t>(vsig + (r < nsig ? r : 0) * kD + n16 * 8);
      const unsigned x0 = x[0], x1 = x[1];
      vS.w0[k] = x0 ^ 0x80808080u;
      vS.w1[k] = x1 ^ 0x80808080u;
    }
    const float2 vs2 = *reinterpret_cast<const float2*>(vss + 2 * lane);
    // other V, both tiles: blocked rows (the lane's 8 column words of rows
    // r0 .. r0 + 7 are one 16-byte run; rows 2p, 2p + 1 form word p; a run
    // wholly past the count reads run 0, whose weights are 0)
    u4_t vO[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int run = 4 * tau + q4;
      vO[tau] = ld_nt<u4_t>(vo.codes + (((8 * run < noth) ? run : 0) * 16 + n16) * 16);
    }
    // ---- significant K: the group's scaled query, built once per wave ----
    // Entry (s, m, qe) of the wave's LDS table holds the A-operand pairs of
    // query m, k-step s, lane group qe: channels c0 + v, c0 + v + 4 (v < 4,
    // c0 = 32 s + 8 qe) times their channel scales, split into fp16 hi + lo.
    // Each query's scaled sum sum_d q_d s_d is reduced over its entries.
    auto& T = L.qtab[wave];
    float part = 0.0f;
    {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e = (lane + 64 * k) & (NE - 1);
        {
          const int sl = e / (4 * R), m = (e >> 2) % R, qe = e & 3;
          const int c0 = 32 * sl + 8 * qe;
          const float4 sa = kd.tsa[k], sb = kd.tsb[k];
          const float sc[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
          u4_t hi4, lo4;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = L.q[m][c0 + v] * sc[v], bq = L.q[m][c0 + v + 4] * sc[v + 4];
            unsigned hi, lo;
            split_pair(a, bq, hi, lo);
            hi4[v] = hi;
            lo4[v] = lo;
            part += a + bq;
          }
          T.e[0][sl][m][qe] = hi4;
          T.e[1][sl][m][qe] = lo4;
        }
      }
      // the entries of query m differ in qe (bits 0-1) and, for R <= 4, in the
      // k-step (the bits above the query's); its sum ends in lane 4 m (lane 0
      // when R == 1)
      if constexpr (R == 1) {
        part = sum16(part);  // every 16-lane row holds all 16 entries
      } else {
        part = quad_sum(part);
        if constexpr (R == 4) {
          part += __shfl_xor(part, 16, 64);
          part += __shfl_xor(part, 32, 64);
        }
      }
    }
    float qs[GI];
#pragma unroll
    for (int i = 0; i < GI; ++i) qs[i] = R == 1 ? lane0(part) : __shfl(part, 4 * QRW::slot_query(q4, i), 64);
    // the significant-V weights enter the matrix cores scaled by kSigWS (kept
    // clear of fp16 subnormals, see kWeightScaleNote); the channel scales in
    // the table carry its inverse (both exact powers of two)
    *reinterpret_cast<float2*>(&vscl[wave][2 * lane]) = float2{vs2.x * (1.0f / kSigWS), vs2.y * (1.0f / kSigWS)};
    wave_lds_sync();
    f4_t c = zero4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u4_t kb = kd.kS.slice(s);
      u4_t qh = T.e[0][s][mr][q4], ql = T.e[1][s][mr][q4];
      if (aq < 0) qh = ql = u4_t{0u, 0u, 0u, 0u};
      c = mfma(qh, kb, c);
      c = mfma(ql, kb, c);
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
      if constexpr (QR == 1) {
        f4_t cc = zero4;  // element g: group g's sum (see the prologue)
#pragma unroll
        for (int g = 0; g < 4; ++g) cc = mfma(qop[g], kd.kO[cb].slice(g), cc);
        float a = mu[0];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const unsigned sbits = kd.skr[cb][g];  // scalar copy before the bit cast
          const float zf = (float)((kd.zkr[cb] >> (8 * g)) & 0xFFu);
          a = fmaf(__builtin_bit_cast(float, sbits), fmaf(-(zf + (float)KI2::OFF), L.qg[0][g], cc[g]), a);
        }
        rawO[cb][0] = a;
      } else {
        f4_t cc[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) cc[g] = mfma(qop[g], kd.kO[cb].slice(g), zero4);
#pragma unroll
        for (int i = 0; i < GI; ++i) {
          const int m = min(QRW::slot_query(q4, i), R - 1);
          const int e = QRW::slot_elem(i);
          float a = mu[i];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const unsigned sbits = kd.skr[cb][g];
            const float zf = (float)((kd.zkr[cb] >> (8 * g)) & 0xFFu);
            a = fmaf(__builtin_bit_cast(float, sbits), fmaf(-(zf + (float)KI2::OFF), L.qg[m][g], cc[g][e]), a);
          }
          rawO[cb][i] = a;
        }
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
#pragma unroll
        for (int g = 0; g < 4; ++g) vb[i][g] *= alpha[i];
      }
    }
#pragma unroll
    for (int i = 0; i < GI; ++i) st.l[i] += rawS[i];
    // ---- significant V: W (16 slots, the other 16 zero) times the codes ----
#pragma unroll
    for (int i = 0; i < GI; ++i) {
      const int m = QRW::slot_query(q4, i);
      unsigned hi, lo;
      split_pair(pS[i] * kSigWS, 0.0f, hi, lo);
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
        st.o[j] += vscl[wave][16 * j + n16] * t;
      }
    }
    wave_lds_sync();
    // ---- K-side loads of this wave's next group (its last group reloads
    // itself: lines still in cache, and no branch) ----
    load_k(grp + kNW < g1 ? grp + kNW : grp, kd);
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
          const unsigned s0 = svr[2 * tau][g], s1 = svr[2 * tau + 1][g];
          const float w0 = pO[2 * tau][i] * __builtin_bit_cast(float, s0);
          const float w1 = pO[2 * tau + 1][i] * __builtin_bit_cast(float, s1);
          const float z0 = (float)((zvr[2 * tau] >> (8 * g)) & 0xFFu);
          const float z1 = (float)((zvr[2 * tau + 1] >> (8 * g)) & 0xFFu);
          vb[i][g] = fmaf(w0, z0 + (float)KI2::OFF, fmaf(w1, z1 + (float)KI2::OFF, vb[i][g]));
          split_pair(w0, w1, hi, lo);
          if (wr) {
            W.w[g][0][m][n16] = (unsigned short)(hi & 0xFFFFu);
            W.w[g][0][m][16 + n16] = (unsigned short)(hi >> 16);
            W.w[g][1][m][n16] = (unsigned short)(lo & 0xFFFFu);
            W.w[g][1][m][16 + n16] = (unsigned short)(lo >> 16);
          }
        }
      }
      wave_lds_sync();
      // column blocks 2g, 2g + 1 use the weights of V group g
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u4_t wh = *reinterpret_cast<const u4_t*>(&W.w[g][0][mr][8 * q4]);
        u4_t wl = *reinterpret_cast<const u4_t*>(&W.w[g][1][mr][8 * q4]);
        if (aq < 0) wh = wl = u4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 2 * g; j < 2 * g + 2; ++j) {
          // 4 + code as fp16 (codes of block j at bits 2j of each half,
          // moved to mantissa bits 8-9 under the exponent of 4)
          u4_t bb;
#pragma unroll
          for (int p2 = 0; p2 < 4; ++p2) {
            const unsigned x = vO[tau][p2];
            const unsigned y = j < 4 ? (x << (8 - 2 * j)) : (x >> (2 * j - 8));
            bb[p2] = and_or(y, 0x03000300u, 0x44004400u);
          }
          st.o[j] = mfma(wh, bb, st.o[j]);
          st.o[j] = mfma(wl, bb, st.o[j]);
        }
      }
      wave_lds_sync();
    }
  }
  // other V entered the products as 4 + c: subtract each query's
  // sum of w (4 + z) over its token columns (16 lanes of a row group), per
  // V group (column blocks 2g, 2g + 1)
#pragma unroll
  for (int i = 0; i < GI; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float t = sum16(vb[i][g]);
      st.o[2 * g][QRW::slot_elem(i)] -= t;
      st.o[2 * g + 1][QRW::slot_elem(i)] -= t;
    }
  // tokens of the group not yet complete (streaming appends) wait as fp16
  // rows in the tails; the split holding token 64 floor(len / 64) attends
  // them (splits are 64-token aligned), with the plain fp16 codecs
  {
    const int lq = len & ~63;
    const int t0 = split * P.split_len, t1 = min(len, t0 + P.split_len);
    if (max(t0, lq) < t1) {
      const TokView kt{P.k.codes16 + (bh * 64 - lq) * KF16::RB, nullptr, nullptr};  // row t: tail row t - lq
      const TokView vt{P.v.codes16 + (bh * 64 - lq) * VF16::RB, nullptr, nullptr};
      const ChanView nc{nullptr, nullptr};
      u4_t qop16[4];  // the plain query operand (qop was specialised above)
      build_qop<QR>(L, qop16);
      attend_wave<QR, 1, 1, KF16, VF16, false, false, 1>(P, L, st, kt, vt, nc, NoOak{}, nq, max(t0, lq), t1,
                                                         wave, qop16);
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
  if (P.pages && P.pshift < 6) return hipErrorInvalidValue;  // pages hold whole groups
  const bool pg = P.pages != nullptr;
  switch (d.qr) {
    case 1:
      if (pg) hipLaunchKernelGGL((k_attn_dsq<1, true>), grid, dim3(kNW * 64), 0, st, P);
      else hipLaunchKernelGGL((k_attn_dsq<1, false>), grid, dim3(kNW * 64), 0, st, P);
      break;
    case 4:
      if (pg) hipLaunchKernelGGL((k_attn_dsq<4, true>), grid, dim3(kNW * 64), 0, st, P);
      else hipLaunchKernelGGL((k_attn_dsq<4, false>), grid, dim3(kNW * 64), 0, st, P);
      break;
    case 16:
      if (pg) hipLaunchKernelGGL((k_attn_dsq<16, true>), grid, dim3(kNW * 64), 0, st, P);
      else hipLaunchKernelGGL((k_attn_dsq<16, false>), grid, dim3(kNW * 64), 0, st, P);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
