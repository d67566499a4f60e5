// Decode kernels for the Oaken cache.  The dense INT4 body goes through the
// matrix-core tile loop like any token-axis group; the sparse outer values
// (reconstruction from the Oaken page, §3.2.2: x_hat = T_hi + mag * s_out
// above the upper outer threshold, T_lo - mag * s_out below the lower one;
// the dense value at an outer position is 0) take two routes.  K's outer
// values enter the scores only through q . x_hat, which needs no softmax
// state: k_oak_kscore forms each token's share for every query of the group
// beforehand, fully parallel (one thread per row), into the decode
// workspace, and the tile loop adds one float per token.  V's outer values
// are weighted by the softmax numerators, so they are consumed inside the
// tile loop (OakWave in kvq_attn_impl.h), each tile's slice of the row-major
// entry list read as one contiguous range issued with the tile's codes.  The
// Oaken page (§2.3) names the access cost of sparse formats; both routes read
// the lists in order, on the streaming path.
#include "kvq_attn_impl.h"

namespace kvq {
namespace {

// Read (never used) in place of the entries of a list of capacity 0, so that
// the tile loop's entry loads need no branch.
alignas(16) __device__ uint16_t kNoEntries[4] = {0, 0, 0, 0};

__device__ __forceinline__ OakList make_list(const TensorArgs& t, long long bh, long long S) {
  return OakList{t.rowptr + bh * (S + 1), t.sparse_cap ? t.sparse + bh * t.sparse_cap : kNoEntries,
                 (unsigned)t.sparse_cap, t.thr_lo, t.thr_hi};
}

// K outer-value score shares: ksc[b][hq][t] = sum over row t's K entries of
// q[b][hq][idx] x_hat, for t < seq_len[b] (clamped to max_len; later rows
// are left unwritten, the tile loop masks them).  A workgroup takes
// kScoreRows rows of one (b, kv head), kScoreRPT per thread (rows tid +
// 256 r, so row-indexed loads and stores coalesce); their entries form one
// contiguous range of the list, staged into LDS with coalesced 8-byte loads
// (in rounds of kScoreBuf entries).  Each thread then sums each of its rows'
// entries in list order, four entries' LDS reads in flight at a time, so the
// result is deterministic.  Grid: (ceil(max_len / kScoreRows), H * qchunks,
// B), chunks of QN (1, 4 or 16) query heads of the group per workgroup,
// their queries in LDS as binary32.
constexpr int kScoreThreads = 256;
constexpr int kScoreRPT = 4;
constexpr int kScoreRows = kScoreThreads * kScoreRPT;
constexpr int kScoreBuf = 8192;  // entries staged per round
constexpr int kScoreWords = kScoreBuf / 4 / kScoreThreads;  // 8-byte loads per thread and round

template <int QN, int NG, bool PAGED>
__global__ __launch_bounds__(kScoreThreads) void k_oak_kscore(AttnParams P, float* __restrict__ ksc) {
  constexpr int kScoreQ = QN;
  __shared__ float qs[kScoreQ][kD];
  __shared__ u2_t ebuf[kScoreBuf / 4];
  const int qchunks = (P.G + kScoreQ - 1) / kScoreQ;
  const int h = blockIdx.y / qchunks, qc = blockIdx.y % qchunks, b = blockIdx.z;
  int len = P.seq_len[b];
  len = len < 0 ? 0 : min(len, P.max_len);  // (out-of-range lengths are reported by the decode kernel)
  const int tb = blockIdx.x * kScoreRows;     // first row of the workgroup
  if (tb >= len) return;                      // (uniform over the workgroup)
  const int nq = min(kScoreQ, P.G - qc * kScoreQ);
  const long long hq0 = (long long)b * P.Hq + (long long)h * P.G + qc * kScoreQ;  // first query row
  for (int i = threadIdx.x; i < nq * kD; i += kScoreThreads)
    qs[i / kD][i % kD] = (float)__builtin_bit_cast(_Float16, P.q[hq0 * kD + i]);
  const long long S = P.S, bh = (long long)b * P.H + h;
  const OakList l = make_list(P.k, bh, S);
  // the workgroup's entry range [lo, hi); each row's range is clamped into it
  const unsigned lo = min(l.rowptr[tb], l.cap), hi = min(l.rowptr[min(tb + kScoreRows, len)], l.cap);
  unsigned e0[kScoreRPT], e1[kScoreRPT];
  float so[kScoreRPT][NG];
#pragma unroll
  for (int r = 0; r < kScoreRPT; ++r) {
    const int t = tb + (int)threadIdx.x + r * kScoreThreads;
    e0[r] = e1[r] = lo;
    if (t < len) {
      e0[r] = min(max(l.rowptr[t], lo), hi);
      e1[r] = min(max(l.rowptr[t + 1], e0[r]), hi);
      long long row = bh * S + t;  // row of token t in the outer scales
      if constexpr (PAGED) {
        int pg = P.pages[(long long)b * (S >> P.pshift) + (t >> P.pshift)];
        if (pg < 0 || pg >= P.npages) {
          set_flag(P.status, kFlagPageRange);
          pg = 0;
        }
        row = (((long long)pg * P.H + h) << P.pshift) + (t & ((1 << P.pshift) - 1));
      }
      load_f32s<NG>(P.k.oscale + row * NG, so[r]);
    }
  }
  float acc[kScoreRPT][kScoreQ];
#pragma unroll
  for (int r = 0; r < kScoreRPT; ++r)
#pragma unroll
    for (int m = 0; m < kScoreQ; ++m) acc[r][m] = 0.0f;
  const uint2* words = reinterpret_cast<const uint2*>(l.sparse);
  const uint16_t* eb = reinterpret_cast<const uint16_t*>(ebuf);
  for (unsigned base = lo & ~3u; base < hi; base += kScoreBuf) {
    // stage words base / 4 .. of this round (hi <= cap, cap a multiple of 4:
    // every word read lies in the list)
    const unsigned wend = min((hi + 3u) >> 2, (base >> 2) + (unsigned)(kScoreBuf / 4));
    uint2 w[kScoreWords];
#pragma unroll
    for (int k = 0; k < kScoreWords; ++k) {
      const unsigned wi = (base >> 2) + threadIdx.x + (unsigned)(k * kScoreThreads);
      if (wi < wend) w[k] = words[wi];
    }
#pragma unroll
    for (int k = 0; k < kScoreWords; ++k) {
      const unsigned wi = (base >> 2) + threadIdx.x + (unsigned)(k * kScoreThreads);
      if (wi < wend) ebuf[threadIdx.x + k * kScoreThreads] = u2_t{w[k].x, w[k].y};
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kScoreRPT; ++r) {
      const unsigned a = max(e0[r], base), z = min(e1[r], base + (unsigned)kScoreBuf);
      for (unsigned e = a; e < z; e += 4) {
        unsigned en[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) en[k] = e + k < z ? eb[e + k - base] : 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (e + k >= z) break;
          const unsigned idx = en[k] & 127u;
          float s = so[r][0];
#pragma unroll
          for (int g = 1; g < NG; ++g) s = idx / (kD / NG) == (unsigned)g ? so[r][g] : s;
          const float xh = oak_value(en[k], s, l);
#pragma unroll
          for (int m = 0; m < kScoreQ; ++m)
            if (m < nq) acc[r][m] = fmaf(qs[m][idx], xh, acc[r][m]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < kScoreRPT; ++r) {
    const int t = tb + (int)threadIdx.x + r * kScoreThreads;
    if (t >= len) continue;
    float* o = ksc + hq0 * P.max_len + t;
#pragma unroll
    for (int m = 0; m < kScoreQ; ++m)
      if (m < nq) o[(long long)m * P.max_len] = acc[r][m];
  }
}

template <int QR, int NG, bool PAGED>
__global__ __launch_bounds__(256, 2) void k_attn_oaken(AttnParams P) {
  __shared__ AttnLds<QR, NG> L;
  __shared__ OakWave<QR, NG> OW[kNW];
  const int split = blockIdx.x, qt = blockIdx.y % P.qtiles, kvh = blockIdx.y / P.qtiles, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar addressing
  const int nq = min(QR, P.G - qt * QR);
  for (int i = threadIdx.x; i < (int)(sizeof(OW) / 4); i += blockDim.x) reinterpret_cast<float*>(OW)[i] = 0.0f;
  u4_t qop[4];
  attn_prologue<QR, NG>(P, L, b, kvh, qt, nq, qop);  // (ends with a barrier)
  const int len = clamp_seq_len(P, b, split == 0 && blockIdx.y == 0 && threadIdx.x == 0);
  const int t0 = split * P.split_len;
  const int t1 = min(len, t0 + P.split_len);
  const long long bh = (long long)b * P.H + kvh;
  const long long S = P.S;
  SoftState<QRows<QR>::GI> st;
  soft_init(st);
  if (t0 < t1) {
    // the side lists are per (sequence, head), paged or not
    const OakCtx<QR, NG> oc{make_list(P.v, bh, S),
                            P.oak_ksc + ((long long)b * P.Hq + (long long)kvh * P.G + qt * QR) * P.max_len,
                            P.max_len, &OW[wave]};
    TokView kv{P.k.codes + bh * S * KI4::RB, P.k.scale + bh * S * NG, P.k.zero + bh * S * NG};
    TokView vv{P.v.codes + bh * S * VI4::RB, P.v.scale + bh * S * NG, P.v.zero + bh * S * NG};
    kv.oscale = P.k.oscale + bh * S * NG;
    vv.oscale = P.v.oscale + bh * S * NG;
    if constexpr (PAGED) {  // the dense body and the outer scales live in pages: pool bases
      const int pshift = P.pshift;
      kv = TokView{P.k.codes, P.k.scale, P.k.zero, P.pages + (long long)b * (S >> pshift), pshift, kvh << pshift,
                   P.H << pshift, P.npages, P.status, P.k.oscale};
      vv = TokView{P.v.codes, P.v.scale, P.v.zero, kv.pages, pshift, kv.hrow, kv.prow, P.npages, P.status,
                   P.v.oscale};
    }
    const ChanView nc{nullptr, nullptr};
    attend_wave<QR, NG, NG, KI4, VI4, false, true, 2, PAGED>(P, L, st, kv, vv, nc, oc, nq, t0, t1, wave, qop);
  }
  // the wave's outer-value output is in the wave's frame, like its MFMA output
  wave_record<QR, NG>(L, st, wave, nq, [&](int m, int d) {
    float o = 0.0f;
#pragma unroll
    for (int c = 0; c < kOakCopies<QR>; ++c) o += OW[wave].osp[c][m][d];
    return o;
  });
  finish_split(P, L, b, kvh, qt, split, nq);
}

template <int QN, bool PAGED>
hipError_t go_kscore(const AttnParams& P, int ng, hipStream_t st) {
  const dim3 grid((unsigned)((P.max_len + kScoreRows - 1) / kScoreRows), (unsigned)(P.H * ((P.G + QN - 1) / QN)),
                  (unsigned)P.B);
  switch (ng) {
    case 1: hipLaunchKernelGGL((k_oak_kscore<QN, 1, PAGED>), grid, dim3(kScoreThreads), 0, st, P, P.oak_ksc); break;
    case 2: hipLaunchKernelGGL((k_oak_kscore<QN, 2, PAGED>), grid, dim3(kScoreThreads), 0, st, P, P.oak_ksc); break;
    case 4: hipLaunchKernelGGL((k_oak_kscore<QN, 4, PAGED>), grid, dim3(kScoreThreads), 0, st, P, P.oak_ksc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool PAGED>
hipError_t go_kscore_q(const AttnParams& P, int ng, hipStream_t st) {
  if (P.G == 1) return go_kscore<1, PAGED>(P, ng, st);
  if (P.G <= 4) return go_kscore<4, PAGED>(P, ng, st);
  return go_kscore<16, PAGED>(P, ng, st);
}

template <int QR, bool PAGED>
hipError_t go_pg(const AttnParams& P, int ng, dim3 grid, hipStream_t st) {
  switch (ng) {
    case 1: hipLaunchKernelGGL((k_attn_oaken<QR, 1, PAGED>), grid, dim3(kNW * 64), 0, st, P); break;
    case 2: hipLaunchKernelGGL((k_attn_oaken<QR, 2, PAGED>), grid, dim3(kNW * 64), 0, st, P); break;
    case 4: hipLaunchKernelGGL((k_attn_oaken<QR, 4, PAGED>), grid, dim3(kNW * 64), 0, st, P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int QR>
hipError_t go(const AttnParams& P, int ng, dim3 grid, hipStream_t st) {
  return P.pages ? go_pg<QR, true>(P, ng, grid, st) : go_pg<QR, false>(P, ng, grid, st);
}

}  // namespace

hipError_t launch_decode_oaken(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
  if (c.k.group != c.v.group) return hipErrorInvalidValue;
  if ((c.k.sparse_cap & 3) || (c.v.sparse_cap & 3)) return hipErrorInvalidValue;
  const AttnParams P = make_attn_params(c, d);
  const dim3 grid((unsigned)d.num_splits, (unsigned)(c.H * d.qtiles), (unsigned)c.B);
  const int ng = kD / c.v.group;
  if (ng != 1 && ng != 2 && ng != 4) return hipErrorInvalidValue;
  if (P.max_len > 0) {  // (with max_len 0 no token is attended and the score shares are never read)
    if (!P.oak_ksc) return hipErrorInvalidValue;
    const hipError_t e = P.pages ? go_kscore_q<true>(P, ng, st) : go_kscore_q<false>(P, ng, st);
    if (e != hipSuccess) return e;
  }
  switch (d.qr) {
    case 1: return go<1>(P, ng, grid, st);
    case 4: return go<4>(P, ng, grid, st);
    case 16: return go<16>(P, ng, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
