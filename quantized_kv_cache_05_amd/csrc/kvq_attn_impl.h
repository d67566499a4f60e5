// The tile loop and epilogue of the matrix-core decode (see kvq_attn.h for the
// operand layouts).  Kernels in kvq_decode_*.hip instantiate attend_wave for
// their codecs and finish with finish_split.
#pragma once
#include <type_traits>

#include "kvq_attn.h"

namespace kvq {

// QR = query rows a workgroup serves (1, 4 or 16 query heads of one KV
// head).  Query rows sit in the A operands as follows:
//  QR 1:  every A row holds query 0; a lane uses C element 0;
//  QR 4:  A row 4m holds query m, the other rows are zero ("diagonal"): lane
//         group q4 then finds query q4 in C element 0, so every lane keeps one
//         softmax row, as for QR 1, instead of four mostly redundant ones;
//  QR 16: A row r holds query r; a lane keeps the four C rows 4*q4 + i.
// GI = softmax rows a lane keeps (1 or 4).
template <int QR>
struct QRows {
  static constexpr int R = QR;
  static constexpr bool DIAG = QR == 4;
  static constexpr int GI = QR == 16 ? 4 : 1;
  // query held by A-operand row r (-1: a zero row)
  __device__ static int arow_query(int r) {
    if constexpr (QR == 1) return 0;
    else if constexpr (DIAG) return (r & 3) ? -1 : (r >> 2);
    else return min(r, R - 1);
  }
  // query of softmax slot i of a lane in row group q4, and its C element
  __device__ static int slot_query(int q4, int i) { return QR == 1 ? 0 : (DIAG ? q4 : 4 * q4 + i); }
  static constexpr int slot_elem(int i) { return DIAG ? 0 : i; }
  // whether the lane owns (writes) slot i: one lane group for QR 1
  __device__ static bool slot_owner(int q4) { return QR != 1 || q4 == 0; }
};

// Workgroup-shared LDS: the query tile, per-group query sums, and a per-wave
// scratch area that the epilogue reuses for the wave records.
template <int QR, int NGV, bool CHANK_ = false>
struct AttnLds {
  static constexpr int R = QR;
  float q[R][128];       // query tile (fp16 values in binary32)
  float qg[R][4];        // sum of the query over each K channel group
  // channel-axis K: per wave, the block's scaled query as MFMA A-operand
  // entries [hi / lo][k-step s][query m][lane group q4] (see attend_wave);
  // row R stays zero for the A-operand rows that hold no query
  struct __attribute__((aligned(16))) QTab {
    u4_t e[2][4][R + 1][4];
  };
  // (a placeholder of one entry's alignment when K has token-axis groups)
  struct Empty {};
  typename std::conditional<CHANK_, QTab[kNW], Empty>::type qtab;
  struct __attribute__((aligned(16))) Wave {
    // softmax weights hi / lo, [V group][query][token]; row R as in QTab
    unsigned short w[NGV][2][R + 1][kTile];
  };
  struct Rec {
    float o[R][128 + 2];  // per query: output sum, then m, l
  };
  union __attribute__((aligned(16))) {
    Wave wave[kNW];
    Rec rec[kNW];
  } u;
};

// Meta of the token of a lane's score column (token nb*16 + n16).  Rows past
// the valid range are read too (they lie inside the allocation); callers mask
// what they produce (scores to -inf, weights to 0), so no branch and no early
// wait on the loads is needed here.
template <int NG, bool SYM>
__device__ __forceinline__ void load_tok_meta(const TokView& v, long long row, float (&s)[NG], float (&z)[NG]) {
  if constexpr (NG == 1) {
    s[0] = ld_nt<float>(v.scale + (unsigned)row);
  } else if constexpr (NG == 2) {
    const u2_t t = ld_nt<u2_t>(v.scale + (unsigned)(row * 2));
    const unsigned t0 = t[0], t1 = t[1];
    s[0] = __builtin_bit_cast(float, t0); s[1] = __builtin_bit_cast(float, t1);
  } else {
    const u4_t t = ld_nt<u4_t>(v.scale + (unsigned)(row * 4));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const unsigned tg = t[g];  // scalar copy before the bit cast (see the V product)
      s[g] = __builtin_bit_cast(float, tg);
    }
  }
  if constexpr (SYM) {
#pragma unroll
    for (int g = 0; g < NG; ++g) z[g] = 0.0f;
  } else {
    unsigned zw;
    if constexpr (NG == 1) zw = ld_nt<uint8_t>(v.zero + (unsigned)row);
    else if constexpr (NG == 2) zw = ld_nt<uint16_t>(v.zero + (unsigned)(row * 2));
    else zw = ld_nt<unsigned>(v.zero + (unsigned)(row * 4));
#pragma unroll
    for (int g = 0; g < NG; ++g) z[g] = (float)((zw >> (8 * g)) & 0xFFu);
  }
}

// -(1024 + f z) as packed fp16 pairs for the B operand of the V product:
// lane rows r0 .. r0 + 7 (pairs 2p, 2p + 1), one set per V group and block
// parity (see the V codecs).  The zero-point bytes of the 8 rows are
// contiguous (NGV per row); the row offset is a multiple of 8, so the loads
// are aligned.  Rows past the valid range multiply zero weights; the mask
// keeps their (arbitrary) bytes inside the mantissa, so the pairs stay finite.
// (load_zraw issues the loads of the zero-point words, zsub_one forms the
// pairs of one group and block parity, so that the loads can be issued well
// before any use and each set of pairs is formed just before its blocks.)
template <class VC, int NGV>
__device__ __forceinline__ void load_zraw(const TokView& vv, long long r0, unsigned (&zw)[2 * NGV]) {
  if constexpr (!VC::SYM) {
    const uint8_t* zp = vv.zero + (unsigned)(r0 * NGV);
    if constexpr (NGV == 1) {
      const u2_t t = ld_nt<u2_t>(zp);
      zw[0] = t[0];
      zw[1] = t[1];
    } else {
#pragma unroll
      for (int k = 0; k < NGV / 2; ++k) {
        const u4_t t = ld_nt<u4_t>(zp + 16 * k);
#pragma unroll
        for (int e = 0; e < 4; ++e) zw[4 * k + e] = t[e];
      }
    }
  }
}
template <class VC, int NGV>
__device__ __forceinline__ u4_t zsub_one(const unsigned (&zw)[2 * NGV], int g, int par) {
  u4_t z;
  if constexpr (VC::SYM) {
#pragma unroll
    for (int p = 0; p < 4; ++p) z[p] = VC::ZMAGIC | 0x00800080u;  // z = 128
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int ia = 2 * p * NGV + g, ib = (2 * p + 1) * NGV + g;
      // byte ia of the row bytes -> bits 0-7, byte ib -> bits 16-23
      const unsigned sel = (0x0Cu << 24) | ((4u + (ib & 3)) << 16) | (0x0Cu << 8) | (unsigned)(ia & 3);
      const unsigned x = perm(zw[ib >> 2], zw[ia >> 2], sel);
      z[p] = and_or(x << VC::ZSH[par], VC::ZMASK[par], VC::ZMAGIC);
    }
  }
  return z;
}

// Sum / max over the 16 lanes of a row group (lanes differing in bits 0-3),
// with DPP lane exchanges inside the 16-lane rows (no LDS round trip):
// quad_perm [1,0,3,2] and [2,3,0,1] pair the lanes of each quad,
// row_half_mirror (lane i <-> 7 - i of each 8-lane half) the two quads of a
// half, row_mirror (lane i <-> 15 - i) the two halves.  Each exchange pairs
// every lane with the mirror lane of the other part, so after the four all
// 16 lanes hold the same total (the operations are commutative, the order
// of the partial sums is the same on every lane).  Callers run the whole
// wave (a DPP read of an inactive lane would give 0).
__device__ __forceinline__ float sum16(float v) {
  v += dpp_row<kDppXor1>(v);
  v += dpp_row<kDppXor2>(v);
  v += dpp_row<kDppHalfMirror>(v);
  v += dpp_row<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_row<kDppXor1>(v));
  v = fmaxf(v, dpp_row<kDppXor2>(v));
  v = fmaxf(v, dpp_row<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_row<kDppMirror>(v));
  return v;
}
// Sum over the 4 lanes of each quad (DPP), and lane 0's value as a
// wave-uniform scalar (the whole wave active).
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_row<kDppXor1>(v);
  v += dpp_row<kDppXor2>(v);
  return v;
}
__device__ __forceinline__ float lane0(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// ---------------------------------------------------------------------------
// Oaken sparse side lists in the tile loop.  Reconstruction
// ([Oaken] §3.2.2): an outer value is T_hi + mag * s_out above the upper outer
// threshold and T_lo - mag * s_out below the lower one; the dense code at an
// outer position is the zero-point, so the dense part there is exactly 0 and
// the outer values only add.  The V row pointers of the next tile are loaded
// one tile ahead, so the entry loads go out with the tile's code loads.  No
// LDS atomics are used (they cost about as much as the rest of the tile), and
// every sum is taken in a fixed order, so decode is deterministic.
//
// K (score part of each row).  sum_{e in row t} q[idx] x_hat depends on
// the query and the entries only, not on the softmax, so a separate kernel
// (k_oak_kscore) forms it for every token beforehand, one thread per row
// summing its entries in order, into the decode workspace; the tile loop adds
// one float per token and query to the scores.
//
// V (outer-value output).  The entries of rows 8k .. 8k + 7 (octet k) take
// one lane each (one 2-byte load per octet).  The row of an entry is 8k plus
// the row tag the quantizer stores in the entry (bits 13-15: the token index
// mod 8; tiles start at multiples of 32).  Within an octet two entries share
// an address of the outer-value output only if they share row and channel,
// which a row's list never does, so with one output copy per row mod 8 every
// octet updates its copies by a plain read-modify-write with no conflicts;
// octets follow one another in program order.  The copies are summed when the
// wave records its result.  With 16 query rows a single copy is kept and each
// octet is applied one row at a time.

template <int QR>
constexpr int kOakCopies = QR == 16 ? 1 : 8;

template <int QR, int NG>
struct __attribute__((aligned(16))) OakWave {
  float so[kTile][NG];                 // V: outer scales of the tile's rows
  float pr[QR][kTile];                 // softmax numerators, per query and row (QR > 1)
  // one query row: per row, the numerator p times T_lo, T_hi and each group's
  // outer scale, so that an entry's share is one fma (p x_hat = p T + mag p s)
  float pv[QR == 1 ? kTile : 1][NG <= 2 ? 4 : 8];
  float pad[64];                       // per-lane sink of masked updates
  float osp[kOakCopies<QR>][QR][128];  // outer-value output per copy (row mod 8), wave frame
};

// One tensor's side list for a (b, kv head).
struct OakList {
  const uint32_t* rowptr;  // [S + 1]
  const uint16_t* sparse;  // [cap]; cap a multiple of 4, so the list is 8-byte aligned
  unsigned cap;            // 0: no list (sparse then points at 4 readable dummy entries)
  float t_lo, t_hi;
};

template <int QR, int NG>
struct OakCtx {
  OakList v;               // the V side list
  const float* ksc;        // K outer-value score shares of query row m, token t: ksc[m * ld + t]
  int ld;                  // row stride of ksc (tokens)
  OakWave<QR, NG>* w;      // this wave's LDS area
};
struct NoOak {};

// V row pointers of one tile for a lane: lane l holds rp of rows l mod 32
// and l mod 32 + 1 (both halves of the wave the same rows), row indices
// clamped to [t0, t1] so that rows outside the split own no entries.
struct OakRp {
  unsigned a, b;
};

__device__ __forceinline__ OakRp oak_rp_load(const OakList& l, int tile, int t0, int t1) {
  const int r = (int)(threadIdx.x & 31);
  const int ia = min(max(tile + r, t0), t1), ib = min(max(tile + r + 1, t0), t1);
  return OakRp{ld_nt<unsigned>(l.rowptr + ia), ld_nt<unsigned>(l.rowptr + ib)};
}

// Entry loads through the global address space: the list pointer would
// otherwise be taken as a flat address that might alias LDS, ordering every
// later LDS access behind the load.  The index is clamped into the list
// (entries outside a range are masked by the caller).
__device__ __forceinline__ unsigned oak_entry(const OakList& l, unsigned e) {
  typedef const __attribute__((address_space(1))) uint16_t gu16_t;
  return __builtin_nontemporal_load((gu16_t*)(l.sparse + min(e, max(l.cap, 1u) - 1u)));
}

// x_hat of entry en (idx | side << 7 | mag << 8 | tag << 13) with its row's outer scale,
// one binary32 product and one sum as in the reconstruction rule.
// (contraction off: the product is rounded before the sum; T_lo - step is
// formed as T_lo + (-step), the same binary32 result)
__device__ __forceinline__ float oak_value(unsigned en, float so, const OakList& l) {
#pragma clang fp contract(off)
  const bool hi = en & 128u;
  const float step = (float)((en >> 8) & 31u) * so;
  return (hi ? l.t_hi : l.t_lo) + (hi ? step : -step);
}

// V entries of one tile, before the softmax: the lane's entry of each octet
// (k = 0..3) and whether it lies in the octet's range.
struct OakOct {
  unsigned en[4];
  bool ok[4];
  unsigned ro[5];   // octet boundaries in the list (wave-uniform)
};

__device__ __forceinline__ OakOct oak_v_prep(const OakList& l, const OakRp& rp) {
  const unsigned lane = threadIdx.x & 63;
  OakOct o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o.ro[k] = min((unsigned)__builtin_amdgcn_readlane((int)rp.a, 8 * k), l.cap);
  o.ro[4] = min((unsigned)__builtin_amdgcn_readlane((int)rp.b, kTile - 1), l.cap);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o.en[k] = oak_entry(l, o.ro[k] + lane);
    o.ok[k] = o.ro[k] + lane < o.ro[k + 1];
  }
  return o;
}

// V entries after the softmax: p[m][row] x_hat into the wave's outer-value
// output (copy row mod 8), octet k by octet; entries past 64 in an octet take
// further rounds (rare).  The row is 8k + the entry's tag.
template <int QR, int NG>
__device__ __forceinline__ void oak_v_apply_one(OakWave<QR, NG>& W, const OakList& l, unsigned en, unsigned k,
                                                bool ok, int nq) {
  const unsigned lane = threadIdx.x & 63, idx = en & 127u, tag = en >> 13, row = 8u * k + tag;
  if constexpr (QR == 1) {
    const bool hi = en & 128u;
    const float mag = (float)((en >> 8) & 31u);
    float sg, tv;
    if constexpr (NG <= 2) {  // the row's four products in one 16-byte read
      const float4 pv = *reinterpret_cast<const float4*>(W.pv[row]);
      sg = (NG == 2 && idx >= 64u) ? pv.w : pv.z;
      tv = hi ? pv.y : pv.x;
    } else {
      const float* pv = W.pv[row];
      sg = pv[2 + idx / (128 / NG)];
      tv = hi ? pv[1] : pv[0];
    }
    const float val = fmaf(hi ? mag : -mag, sg, tv);
    if (ok) W.osp[tag][0][idx] += val;
    return;
  }
  const float xh = oak_value(en, W.so[row][NG == 1 ? 0u : idx / (128 / NG)], l);
  constexpr int NC = kOakCopies<QR>;
#pragma unroll
  for (int m = 0; m < QR; ++m) {
    if (m < nq) {
      const float val = W.pr[m][row] * xh;
      if constexpr (NC == 8) {
        float* a = ok ? &W.osp[tag][m][idx] : &W.pad[lane];
        *a += ok ? val : 0.0f;
      } else {  // one copy: one row of the octet at a time
#pragma unroll
        for (unsigned r = 0; r < 8; ++r) {
          const bool mine = ok && tag == r;
          float* a = mine ? &W.osp[0][m][idx] : &W.pad[lane];
          *a += mine ? val : 0.0f;
        }
      }
    }
  }
}

template <int QR, int NG>
__device__ __forceinline__ void oak_v_apply(OakWave<QR, NG>& W, const OakList& l, const OakOct& o, int nq) {
#pragma unroll
  for (int k = 0; k < 4; ++k) oak_v_apply_one<QR, NG>(W, l, o.en[k], (unsigned)k, o.ok[k], nq);
  // octets with more than 64 entries (rare): further rounds of 64
  const unsigned lane = threadIdx.x & 63;
  for (int k = 0; k < 4; ++k) {
    for (unsigned c = 1; o.ro[k] + 64u * c < o.ro[k + 1]; ++c) {
      const unsigned e = o.ro[k] + 64u * c + lane;
      oak_v_apply_one<QR, NG>(W, l, oak_entry(l, e), (unsigned)k, e < o.ro[k + 1], nq);
    }
  }
}

template <int NG>
__device__ __forceinline__ void load_f32s(const float* p, float (&v)[NG]) {
  if constexpr (NG == 1) {
    v[0] = ld_nt<float>(p);
  } else if constexpr (NG == 2) {
    const u2_t t = ld_nt<u2_t>(p);
    const unsigned t0 = t[0], t1 = t[1];
    v[0] = __builtin_bit_cast(float, t0);
    v[1] = __builtin_bit_cast(float, t1);
  } else {
    const u4_t t = ld_nt<u4_t>(p);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const unsigned tg = t[g];
      v[g] = __builtin_bit_cast(float, tg);
    }
  }
}

// The loaded inputs of one tile: K and V codes, token metadata, V zero-point
// words (no arithmetic on them yet, so issuing the loads waits for nothing).
template <class KC, class VC, int NGK, int NGV>
struct TileIn {
  KC kr[2];
  VC vr;
  float sk[2][NGK], zk[2][NGK], sv[2][NGV], zv[2][NGV];
  unsigned zraw[2 * NGV];
};

// ---------------------------------------------------------------------------
// One wave's share of a token range [t0, t1) of one (b, kv head): tiles of 32
// tokens starting at tile-aligned offsets, taken round robin by the waves in
// steps of TPS tiles.
//
//  KC / VC: codecs.  NGK / NGV: channel groups of K / V (token axis).
//  CHANK: K has channel-axis groups of 64 tokens (scale folded into the query).
//  PAGED: the views are paged (TokView), rebased for every tile; PK: K is
//         paged too (false: K is a per-sequence view, e.g. an fp16 tail).
//         With CHANK, the block scales (kc) are pool bases, indexed by the
//         page row of the block.
//  OAK: Oaken; oak holds the V side list, the K outer-value score shares
//       and the wave's LDS area (OakCtx); the score shares are added to the
//       scores and the V outer values enter the wave's outer-value output
//       inside the loop (see OakWave).
template <int QR, int NGK, int NGV, class KC, class VC, bool CHANK, bool OAK, int TPS, bool PAGED = false,
          bool PK = PAGED, class LDS, class OK = NoOak>
__device__ __forceinline__ void attend_wave(const AttnParams& P, LDS& L,
                                            SoftState<QRows<QR>::GI>& st, const TokView& kv_,
                                            const TokView& vv_, const ChanView& kc, const OK& oak,
                                            int nq, int t0, int t1, int wave,
                                            const u4_t (&qop)[4]) {
  using QRW = QRows<QR>;
  constexpr int R = QR, GI = QRW::GI;
  static_assert(LDS::R == QR, "LDS tables sized for QR query rows");
  const int lane = threadIdx.x & 63, n16 = lane & 15, q4 = lane >> 4;
  const int aq = QRW::arow_query(n16);  // query of this lane's A-operand row (-1: zero row)
  auto& W = L.u.wave[wave];
  // A-operand rows that hold no query (4 query rows) read row R of the
  // wave's LDS tables, kept zero here (read only after the LDS waits below)
  const int ar = aq < 0 ? R : aq;
  if constexpr (QRW::DIAG) {
    if (lane < 8 * NGV)
      *reinterpret_cast<u4_t*>(&W.w[lane >> 3][(lane >> 2) & 1][R][8 * (lane & 3)]) = u4_t{0u, 0u, 0u, 0u};
    if constexpr (CHANK) {
      if (lane < 32) L.qtab[wave].e[lane >> 4][(lane >> 2) & 3][R][lane & 3] = u4_t{0u, 0u, 0u, 0u};
    }
  }
  const int tb = t0 & ~(kTile * TPS - 1);
  // the running output is held in natural units between calls; inside, block
  // j accumulates with the codec's factor fac(j)
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (VC::fac(j) != 1.0f) st.o[j] *= VC::fac(j);
  // paged: the block-table entry of the next step is loaded one step ahead
  // (a step of kTile * TPS <= 64 tokens lies in one page: pages hold a
  // multiple of 64 tokens and steps start 64-aligned)
  static_assert(!PAGED || kTile * TPS <= 64, "a step must stay inside one page");
  int pg_next = 0;
  if constexpr (PAGED) pg_next = page_entry_v(vv_.pages, min(tb + wave * kTile * TPS, t1 - 1) >> vv_.pshift);
  // Oaken: row pointers of the wave's next tile, one tile ahead
  OakRp rp_next{};
  if constexpr (OAK) rp_next = oak_rp_load(oak.v, tb + wave * kTile * TPS, t0, t1);
  for (int step = tb + wave * kTile * TPS; step < t1; step += kNW * kTile * TPS) {
    TokView kv = kv_, vv = vv_;
    long long ro = 0;  // paged: pool row of token t = t + ro (this step's page)
    if constexpr (PAGED) {
      ro = page_row_offset(vv_, __builtin_amdgcn_readfirstlane(pg_next), step);
      if constexpr (PK && CHANK) kv.codes = kv_.codes + ro * KC::RB;
      else if constexpr (PK) kv = at_rows<KC::RB, NGK>(kv_, ro);
      vv = at_rows<VC::RB, NGV>(vv_, ro);
      pg_next = page_entry_v(vv_.pages, min(step + kNW * kTile * TPS, t1 - 1) >> vv_.pshift);
    }
    // the tile inputs; with channel-axis K the first tile's loads are issued
    // before the block scales are folded, so that both memory round trips
    // overlap instead of following one another
    using In = TileIn<KC, VC, NGK, NGV>;
    auto load_in = [&](In& in, int tile) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) in.kr[nb].load(kv.codes + (unsigned)((tile + nb * 16 + n16) * KC::RB), q4);
      in.vr.load(vv.codes + (unsigned)((tile + 8 * q4) * VC::RB), n16);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int t = tile + nb * 16 + n16;
        if constexpr (!CHANK && !KC::F16) load_tok_meta<NGK, KC::SYM>(kv, t, in.sk[nb], in.zk[nb]);
        // V zero-points enter through zsub below; only the scales are needed here
        if constexpr (!VC::F16) load_tok_meta<NGV, true>(vv, t, in.sv[nb], in.zv[nb]);
      }
      if constexpr (VC::ZP) load_zraw<VC, NGV>(vv, tile + 8 * q4, in.zraw);
    };
    In pre;
    if constexpr (CHANK) load_in(pre, step);
    // ---- channel-axis K: fold the block's scales into the query ----
    // The R x 128 products q[m][d] * s[d] are spread over the wave: entry
    // (s, m, q4e) covers channels 32 s + 8 q4e + (v, v + 4), v < 4; it is
    // split into fp16 hi + lo pairs and stored in the wave's LDS table, from
    // which the tile loop's A-operand lanes read it.  Each query's bias
    // sum_d q[m][d] s[d] (OFF + z[d]) is reduced over its entries.
    float cbias[GI];
    if constexpr (CHANK) {
      const long long blk = (step + ro) >> 6;  // a 64-token block never straddles a page
      const float* sp = kc.scale + blk * 128;
      const uint8_t* zp = kc.zero + blk * 128;
      auto& T = L.qtab[wave];
      constexpr int NE = 16 * R, PER = (NE + 63) / 64;
      float part = 0.0f;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e = lane + 64 * k;
        if (e < NE) {
          const int sl = e / (4 * R), m = (e >> 2) % R, qe = e & 3;
          const int c0 = 32 * sl + 8 * qe;
          const float4 sa = *reinterpret_cast<const float4*>(sp + c0);
          const float4 sb = *reinterpret_cast<const float4*>(sp + c0 + 4);
          const u2_t zz = *reinterpret_cast<const u2_t*>(zp + c0);
          const float sc[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
          u4_t hi4, lo4;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = L.q[m][c0 + v] * sc[v], b = L.q[m][c0 + v + 4] * sc[v + 4];
            unsigned hi, lo;
            split_pair(a, b, hi, lo);
            hi4[v] = hi;
            lo4[v] = lo;
            const float za = (float)((zz[0] >> (8 * v)) & 0xFFu) + (float)KC::OFF;
            const float zb = (float)((zz[1] >> (8 * v)) & 0xFFu) + (float)KC::OFF;
            part = fmaf(a, za, part);
            part = fmaf(b, zb, part);
          }
          T.e[0][sl][m][qe] = hi4;
          T.e[1][sl][m][qe] = lo4;
        }
      }
      // sum the entries of each query: lanes of query m differ in q4e (bits 0-1)
      // and, for R <= 4, in the k-step (the bits above the query's)
      if constexpr (R == 1) {
        part = sum16(part);  // the entries sit in lanes 0-15
      } else {
        part = quad_sum(part);
        if constexpr (R == 4) {
          part += __shfl_xor(part, 16, 64);
          part += __shfl_xor(part, 32, 64);
        }
      }
      // the sum of query m sits in lane 4 m (R > 1) or lane 0 (R == 1)
#pragma unroll
      for (int i = 0; i < GI; ++i)
        cbias[i] = R == 1 ? lane0(part) : __shfl(part, 4 * QRW::slot_query(q4, i), 64);
      wave_lds_sync();
    }
#pragma unroll
    for (int tt = 0; tt < TPS; ++tt) {
      const int tile = step + tt * kTile;
      if (tile >= t1) break;
      OakRp rpc{};
      if constexpr (OAK) {
        rpc = rp_next;
        rp_next = oak_rp_load(oak.v, tt + 1 < TPS ? tile + kTile : step + kNW * kTile * TPS, t0, t1);
      }
      if (tile + kTile <= t0) continue;
      // ---- loads ----
      // Oaken: the tile's V entries (octets), the rows' V outer scales and
      // the K score shares of the lane's score slots, issued ahead of the codes
      float oso[NGV];  // V outer scales of row lane & 31
      float oks[2][GI];
      OakOct oct{};
      if constexpr (OAK) {
        const long long t = tile + (lane & 31);
        load_f32s<NGV>(vv.oscale + (unsigned)(t * NGV), oso);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const unsigned tk = (unsigned)min(tile + nb * 16 + n16, oak.ld - 1);
#pragma unroll
          for (int i = 0; i < GI; ++i) {
            const unsigned m = (unsigned)min(QRW::slot_query(q4, i), nq - 1);
            oks[nb][i] = ld_nt<float>(oak.ksc + (m * (unsigned)oak.ld + tk));
          }
        }
        oct = oak_v_prep(oak.v, rpc);
        // issued before the code loads, so that the entry work below waits on
        // these alone (loads complete in order)
        __builtin_amdgcn_sched_barrier(0);
      }
      In in;
      if constexpr (CHANK) {
        if (tt == 0) in = pre;
        else load_in(in, tile);
      } else {
        load_in(in, tile);
      }
      KC (&kr)[2] = in.kr;
      VC& vr = in.vr;
      auto& sk = in.sk;
      auto& zk = in.zk;
      auto& sv = in.sv;
      bool ok[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int t = tile + nb * 16 + n16;
        ok[nb] = t >= t0 && t < t1;
      }
      if constexpr (VC::MASK_ROWS) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int t = tile + 8 * q4 + k;
          if (t < t0 || t >= t1) vr.zero_row(k);
        }
      }
      // -(OFF + z) of the B-operand rows as packed fp16 pairs, per V group
      // ---- Oaken: the rows' V outer scales into LDS ----
      if constexpr (OAK) {
        __builtin_amdgcn_sched_barrier(0);  // the code loads stay ahead of the entry work
#pragma unroll
        for (int g = 0; g < NGV; ++g) oak.w->so[lane & 31][g] = oso[g];  // (both halves: same values)
      }
      // ---- scores ----
      float sc[2][GI];
      if constexpr (CHANK) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          f4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
          const auto& T = L.qtab[wave];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const u4_t kb = kr[nb].slice(s);
            const u4_t qh = T.e[0][s][ar][q4], ql = T.e[1][s][ar][q4];
            c = mfma(qh, kb, c);
            c = mfma(ql, kb, c);
          }
#pragma unroll
          for (int i = 0; i < GI; ++i) sc[nb][i] = (c[QRW::slot_elem(i)] - cbias[i]) * P.qscale;
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          f4_t c[NGK];
#pragma unroll
          for (int g = 0; g < NGK; ++g) c[g] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < 4; ++s) c[s / (4 / NGK)] = mfma(qop[s], kr[nb].slice(s), c[s / (4 / NGK)]);
#pragma unroll
          for (int i = 0; i < GI; ++i) {
            const int m = min(QRW::slot_query(q4, i), R - 1);
            const int e = QRW::slot_elem(i);
            float a;
            if constexpr (KC::F16) {
              a = c[0][e];
            } else {
              a = 0.0f;
#pragma unroll
              for (int g = 0; g < NGK; ++g)
                a = fmaf(sk[nb][g], fmaf(-(zk[nb][g] + (float)KC::OFF), L.qg[m][g], c[g][e]), a);
            }
            sc[nb][i] = a * P.qscale;
          }
        }
      }
      // ---- Oaken: the outer K values' share of the score ----
      if constexpr (OAK) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int i = 0; i < GI; ++i)
            sc[nb][i] = fmaf(oks[nb][i], P.qscale, sc[nb][i]);  // (rows outside the range are masked below)
      }
      // ---- online softmax (base 2) ----
      float alpha[GI];
      bool grow = false;
#pragma unroll
      for (int i = 0; i < GI; ++i) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          if (!ok[nb]) sc[nb][i] = -INFINITY;
        const float tm = max16(fmaxf(sc[0][i], sc[1][i]));
        const float mn = fmaxf(st.m[i], tm);
        alpha[i] = mn == -INFINITY ? 1.0f : fexp2(st.m[i] - mn);
        grow |= mn > st.m[i];
        st.m[i] = mn;
      }
      if (__any(grow)) {
#pragma unroll
        for (int i = 0; i < GI; ++i) {
          const float a = alpha[i];
          st.l[i] *= a;
#pragma unroll
          for (int j = 0; j < 8; ++j) st.o[j][QRW::slot_elem(i)] *= a;
        }
        if constexpr (OAK) {  // the outer-value output copies follow the same frame
          auto& OW = *oak.w;
#pragma unroll
          for (int c = 0; c < kOakCopies<QR>; ++c) {
            if constexpr (QR == 1) {
              OW.osp[c][0][lane] *= alpha[0];
              OW.osp[c][0][lane + 64] *= alpha[0];
            } else {
#pragma unroll
              for (int i = 0; i < GI; ++i)
#pragma unroll
                for (int k = 0; k < 8; ++k) OW.osp[c][QRW::slot_query(q4, i)][n16 + 16 * k] *= alpha[i];
            }
          }
        }
      }
      float p[2][GI];
#pragma unroll
      for (int i = 0; i < GI; ++i)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          p[nb][i] = ok[nb] ? fexp2(sc[nb][i] - st.m[i]) : 0.0f;
          st.l[i] += p[nb][i];
        }
      // ---- Oaken: the softmax numerators of the rows, for the V entries ----
      if constexpr (OAK && QR == 1) {
        wave_lds_sync();  // the rows' outer scales, written by other lanes
        if (q4 == 0) {  // lanes 0-15 hold rows n16 and 16 + n16
          const OakList& lv = oak.v;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int row = nb * 16 + n16;
            const float pn = p[nb][0];
            float v[NGV <= 2 ? 4 : 8];
            v[0] = pn * lv.t_lo;
            v[1] = pn * lv.t_hi;
#pragma unroll
            for (int g = 0; g < NGV; ++g) v[2 + g] = pn * oak.w->so[row][g];
#pragma unroll
            for (int g = NGV + 2; g < (NGV <= 2 ? 4 : 8); ++g) v[g] = 0.0f;
            float* d = oak.w->pv[row];
#pragma unroll
            for (int g = 0; g < (NGV <= 2 ? 4 : 8); g += 4)
              *reinterpret_cast<float4*>(d + g) = float4{v[g], v[g + 1], v[g + 2], v[g + 3]};
          }
        }
      } else if constexpr (OAK) {
#pragma unroll
        for (int i = 0; i < GI; ++i) {
          const int m = QRW::slot_query(q4, i);
          if (QRW::slot_owner(q4) && m < R) {
            oak.w->pr[m][n16] = p[0][i];
            oak.w->pr[m][16 + n16] = p[1][i];
          }
        }
      }
      // ---- weights p * s_v (binary32) -> fp16 hi / lo in LDS ----
#pragma unroll
      for (int i = 0; i < GI; ++i) {
        const int m = QRW::slot_query(q4, i);
        const bool wr = QRW::slot_owner(q4) && m < R;
#pragma unroll
        for (int g = 0; g < NGV; ++g) {
          float w0, w1;
          if constexpr (VC::F16) {
            w0 = p[0][i] * VC::WS;
            w1 = p[1][i] * VC::WS;
          } else {
            w0 = ok[0] ? p[0][i] * (sv[0][g] * VC::WS) : 0.0f;
            w1 = ok[1] ? p[1][i] * (sv[1][g] * VC::WS) : 0.0f;
          }
          unsigned hi, lo;
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
      // ---- Oaken: V entries into the outer-value output ----
      if constexpr (OAK) oak_v_apply<QR, NGV>(*oak.w, oak.v, oct, nq);
      // ---- O += W V ----
      // blocks by V group and parity: each group's weights and -(OFF + z)
      // pairs are read / formed just before its blocks
      constexpr int JPG = 8 / NGV, NP = VC::ZODD ? 2 : 1;
#pragma unroll
      for (int g = 0; g < NGV; ++g) {
        u4_t wa[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) wa[h] = *reinterpret_cast<const u4_t*>(&W.w[g][h][ar][8 * q4]);
#pragma unroll
        for (int par = 0; par < NP; ++par) {
          u4_t zs{};
          if constexpr (VC::ZP) zs = zsub_one<VC, NGV>(in.zraw, g, par);
#pragma unroll
          for (int jj = 0; jj < JPG; ++jj) {
            const int j = g * JPG + jj;
            if (VC::ZODD && (j & 1) != par) continue;
            u4_t b = vr.block(j);
            if constexpr (VC::ZP) {
#pragma unroll
              for (int p2 = 0; p2 < 4; ++p2) {
                // copy vector elements to scalars before bit casts: clang miscompiles a bit cast
                // applied directly to an ext-vector element
                const unsigned bv = b[p2], zv = zs[p2];
                const h2_t x = __builtin_bit_cast(h2_t, bv) + __builtin_bit_cast(h2_t, zv);
                b[p2] = __builtin_bit_cast(unsigned, x);
              }
            }
            st.o[j] = mfma(wa[0], b, st.o[j]);
            st.o[j] = mfma(wa[1], b, st.o[j]);
          }
        }
      }
      wave_lds_sync();
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (VC::fac(j) != 1.0f) st.o[j] *= 1.0f / VC::fac(j);
}

// Fold the wave's state into its record (sum of l over the 16 token
// columns).  Caller: all waves, after a barrier.
template <int QR, int NGV, class LDS, class Extra>
__device__ __forceinline__ void wave_record(LDS& L, SoftState<QRows<QR>::GI>& st, int wave, int nq,
                                            Extra&& extra) {
  constexpr int GI = QRows<QR>::GI;
  const int lane = threadIdx.x & 63, n16 = lane & 15, q4 = lane >> 4;
  float lt[GI];
#pragma unroll
  for (int i = 0; i < GI; ++i) lt[i] = sum16(st.l[i]);
  __syncthreads();
  auto& rec = L.u.rec[wave];
  using QRW = QRows<QR>;
#pragma unroll
  for (int i = 0; i < GI; ++i) {
    const int m = QRW::slot_query(q4, i);
    if (!QRW::slot_owner(q4)) continue;
    if (m >= nq) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      rec.o[m][16 * j + n16] = st.o[j][QRW::slot_elem(i)] + extra(m, 16 * j + n16);
    }
    if (n16 == 0) {
      rec.o[m][128] = st.m[i];
      rec.o[m][129] = lt[i];
    }
  }
}

template <int QR, int NGV, class LDS>
__device__ __forceinline__ void wave_record(LDS& L, SoftState<QRows<QR>::GI>& st, int wave, int nq) {
  wave_record<QR, NGV>(L, st, wave, nq, [](int, int) { return 0.0f; });
}

// Merge the four wave records of each query and write the output (one
// split) or the split partial (m, l, unnormalized output) for k_merge.
// extra(m, d, M) may add a term to the unnormalized output of query m,
// channel d, in the frame of the workgroup maximum M.
template <class LDS, class Extra>
__device__ __forceinline__ void finish_split(const AttnParams& P, LDS& L, int b, int kvh, int qt,
                                             int split, int nq, Extra&& extra) {
  __syncthreads();
  const long long hq0 = (long long)kvh * P.G + (long long)qt * LDS::R;
  for (int idx = threadIdx.x; idx < nq * 128; idx += blockDim.x) {
    const int m = idx >> 7, d = idx & 127;
    const float M = wg_max(L, m);
    float Ls = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        const float mw = L.u.rec[w].o[m][128];
        if (mw != -INFINITY) {
          const float f = fexp2(mw - M);
          Ls = fmaf(f, L.u.rec[w].o[m][129], Ls);
          O = fmaf(f, L.u.rec[w].o[m][d], O);
        }
      }
      O += extra(m, d, M);
    }
    const long long hq = hq0 + m;
    if (P.num_splits == 1) {
      P.out[((long long)b * P.Hq + hq) * 128 + d] = Ls > 0.0f ? O / Ls : 0.0f;
    } else {
      float* r = P.ws + (((long long)b * P.Hq + hq) * P.num_splits + split) * kPartStride;
      r[4 + d] = O;
      if (d == 0) {
        r[0] = M;
        r[1] = Ls;
      }
    }
  }
}

template <class LDS>
__device__ __forceinline__ void finish_split(const AttnParams& P, LDS& L, int b, int kvh, int qt,
                                             int split, int nq) {
  finish_split(P, L, b, kvh, qt, split, nq, [](int, int, float) { return 0.0f; });
}

// Maximum of query m's running maxima over the four wave records.
template <class LDS>
__device__ __forceinline__ float wg_max(const LDS& L, int m) {
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kNW; ++w) M = fmaxf(M, L.u.rec[w].o[m][128]);
  return M;
}

// Workgroup prologue: the query tile in LDS, per-group query sums, the K
// A-operand of each k-step, and reset wave state.  Ends with a barrier.
// The K-product A operand of a lane from the query tile in LDS: k-step s
// holds fp16 pairs of channels (c0 + v, c0 + v + 4), c0 = 32 s + 8 q4, of the
// query on the lane's A row (zero rows stay zero).
template <int QR, class LDS>
__device__ __forceinline__ void build_qop(const LDS& L, u4_t (&qop)[4]) {
  const int lane = threadIdx.x & 63, n16 = lane & 15, q4 = lane >> 4;
  const int aq = QRows<QR>::arow_query(n16);
  const int m = max(aq, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c0 = 32 * s + 8 * q4;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const h2_t h = {(_Float16)L.q[m][c0 + v], (_Float16)L.q[m][c0 + v + 4]};
      qop[s][v] = aq < 0 ? 0u : __builtin_bit_cast(unsigned, h);
    }
  }
}

template <int QR, int NGK, class LDS>
__device__ __forceinline__ void attn_prologue(const AttnParams& P, LDS& L, int b, int kvh, int qt,
                                              int nq, u4_t (&qop)[4]) {
  constexpr int R = QR, GI = QRows<QR>::GI;
  for (int idx = threadIdx.x; idx < R * 128; idx += blockDim.x) {
    const int m = idx >> 7, d = idx & 127;
    float v = 0.0f;
    if (m < nq) v = h2f(P.q[((long long)b * P.Hq + (long long)kvh * P.G + (long long)qt * QR + m) * 128 + d]);
    L.q[m][d] = v;
  }
  for (int idx = threadIdx.x; idx < (int)(sizeof(L.u) / 4); idx += blockDim.x)
    reinterpret_cast<float*>(&L.u)[idx] = 0.0f;
  __syncthreads();
  if (threadIdx.x < R * NGK) {
    const int m = threadIdx.x / NGK, g = threadIdx.x % NGK, w = 128 / NGK;
    double s = 0.0;  // exact for up to 128 fp16 terms: one rounding to binary32
    for (int d = g * w; d < (g + 1) * w; ++d) s += (double)L.q[m][d];
    L.qg[m][g] = (float)s;
  }
  build_qop<QR>(L, qop);
  __syncthreads();
}

__device__ __forceinline__ int clamp_seq_len(const AttnParams& P, int b, bool report) {
  int len = P.seq_len[b];
  if (len < 0 || len > P.max_len) {
    if (report) set_flag(P.status, kFlagLenRange);
    len = len < 0 ? 0 : P.max_len;
  }
  return len;
}

}  // namespace kvq
