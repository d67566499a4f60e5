// Decode kernels for the uniform cache: token-axis K and V groups, or K with
// channel-axis groups of 64 tokens and token-axis V (see kvq_attn.h).
#include "kvq_attn_impl.h"

namespace kvq {
namespace {

// Occupancy target (waves per SIMD): two in general; four for the
// contiguous 4-query per-channel-K kernels with 4- or 2-bit codes and two V
// groups, and for the paged token-axis one-query kernels with at most two
// groups other than asymmetric INT8, which fit in 128 registers without
// spilling (the contiguous one-query kernels land there by themselves).
template <int QR, class KC, int NGV, bool CHANK, bool PAGED>
constexpr int kUniformWaves = ((CHANK && !PAGED && QR == 4 && NGV == 2 && KC::BITS <= 4) ||
                               (!CHANK && PAGED && QR == 1 && NGV <= 2 && !(KC::BITS == 8 && !KC::SYM)))
                                  ? 4
                                  : 2;

// Paged V view of (b, kvh): the pool bases and this sequence's block-table row.
template <class VC, int NGV>
__device__ __forceinline__ TokView paged_v(const AttnParams& P, int b, int kvh) {
  const int pshift = P.pshift;
  return TokView{P.v.codes, P.v.scale, VC::SYM ? nullptr : P.v.zero,
                 P.pages + (long long)b * (P.S >> pshift), pshift, kvh << pshift, P.H << pshift,
                 P.npages, P.status};
}

template <int QR, class KC, class VC, int NGK, int NGV, bool CHANK, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kUniformWaves<QR, KC, NGV, CHANK, PAGED>)))
void k_attn_uniform(AttnParams P) {
  __shared__ AttnLds<QR, NGV, CHANK> L;
  const int split = blockIdx.x, qt = blockIdx.y % P.qtiles, kvh = blockIdx.y / P.qtiles, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar addressing
  const int nq = min(QR, P.G - qt * QR);
  u4_t qop[4];
  attn_prologue<QR, NGK>(P, L, b, kvh, qt, nq, qop);
  const int len = clamp_seq_len(P, b, split == 0 && blockIdx.y == 0 && threadIdx.x == 0);
  const int t0 = split * P.split_len;
  const int t1 = min(len, t0 + P.split_len);
  // channel-axis K: tokens from lq on (the block not yet complete) are read
  // from the fp16 residual tail; splits are 64-token aligned, so one split
  // holds them all
  const int lq = CHANK ? (len & ~63) : len;
  SoftState<QRows<QR>::GI> st;
  soft_init(st);
  if (t0 < min(t1, lq)) {
    const long long bh = (long long)b * P.H + kvh;
    const long long S = P.S;
    TokView kv{P.k.codes + bh * S * KC::RB, nullptr, nullptr};
    ChanView kc{nullptr, nullptr};
    if constexpr (CHANK) {
      kc.scale = P.k.scale + bh * (S / 64) * 128;
      kc.zero = P.k.zero + bh * (S / 64) * 128;
    } else {
      kv.scale = P.k.scale + bh * S * NGK;
      kv.zero = KC::SYM ? nullptr : P.k.zero + bh * S * NGK;
    }
    TokView vv{P.v.codes + bh * S * VC::RB, P.v.scale + bh * S * NGV,
               VC::SYM ? nullptr : P.v.zero + bh * S * NGV};
    if constexpr (PAGED) {  // pools of pages: the views start at the pool bases
      vv = paged_v<VC, NGV>(P, b, kvh);
      kv = TokView{P.k.codes, CHANK ? nullptr : P.k.scale, (CHANK || KC::SYM) ? nullptr : P.k.zero, vv.pages,
                   vv.pshift, vv.hrow, vv.prow, P.npages, P.status};
      if constexpr (CHANK) kc = ChanView{P.k.scale, P.k.zero};  // blocks indexed by pool row / 64
    }
    attend_wave<QR, NGK, NGV, KC, VC, CHANK, false, 2, PAGED>(P, L, st, kv, vv, kc, NoOak{}, nq, t0,
                                                               min(t1, lq), wave, qop);
  }
  if constexpr (CHANK) {
    if (max(t0, lq) < t1) {
      const long long bh = (long long)b * P.H + kvh;
      const long long S = P.S;
      // row t of the view is tail row t - lq
      // (the tail is per sequence, paged or not)
      const TokView kt{P.k.codes16 + (bh * 64 - lq) * KF16::RB, nullptr, nullptr};
      TokView vv{P.v.codes + bh * S * VC::RB, P.v.scale + bh * S * NGV,
                 VC::SYM ? nullptr : P.v.zero + bh * S * NGV};
      if constexpr (PAGED) vv = paged_v<VC, NGV>(P, b, kvh);
      const ChanView nc{nullptr, nullptr};
      // the query operand is rebuilt here rather than kept live through the main loop
      u4_t qop16[4];
      build_qop<QR>(L, qop16);
      attend_wave<QR, 1, NGV, KF16, VC, false, false, 1, PAGED, false>(P, L, st, kt, vv, nc, NoOak{}, nq,
                                                                      max(t0, lq), t1, wave, qop16);
    }
  }
  wave_record<QR, NGV>(L, st, wave, nq);
  finish_split(P, L, b, kvh, qt, split, nq);
}

template <int QR, class KC, class VC, int NGK, int NGV, bool CHANK>
hipError_t go(const AttnParams& P, dim3 grid, hipStream_t st) {
  if (P.pages)
    hipLaunchKernelGGL((k_attn_uniform<QR, KC, VC, NGK, NGV, CHANK, true>), grid, dim3(kNW * 64), 0, st, P);
  else
    hipLaunchKernelGGL((k_attn_uniform<QR, KC, VC, NGK, NGV, CHANK, false>), grid, dim3(kNW * 64), 0, st, P);
  return hipGetLastError();
}

template <int QR, class KC, class VC, bool CHANK_OK = true>
hipError_t go_ng(const AttnParams& P, dim3 grid, bool chank, int ng, hipStream_t st) {
  if constexpr (!CHANK_OK) {
    if (chank) return hipErrorInvalidValue;
  } else if (chank) {
    switch (ng) {
      case 1: return go<QR, KC, VC, 1, 1, true>(P, grid, st);
      case 2: return go<QR, KC, VC, 1, 2, true>(P, grid, st);
      case 4: return go<QR, KC, VC, 1, 4, true>(P, grid, st);
    }
    return hipErrorInvalidValue;
  }
  switch (ng) {
    case 1: return go<QR, KC, VC, 1, 1, false>(P, grid, st);
    case 2: return go<QR, KC, VC, 2, 2, false>(P, grid, st);
    case 4: return go<QR, KC, VC, 4, 4, false>(P, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int QR>
hipError_t go_codec(const AttnParams& P, dim3 grid, hipStream_t st) {
  const bool chank = P.k.axis == 1;
  const int ng = kD / P.v.group;
  if (P.v.fmt == 1) return go_ng<QR, KE4, VE4, false>(P, grid, chank, ng, st);
  if (P.v.fmt == 2) return go_ng<QR, KE5, VE5, false>(P, grid, chank, ng, st);
  if (P.v.sym) return go_ng<QR, KI8<true>, VI8<true>, false>(P, grid, chank, ng, st);
  switch (P.v.bits) {
    case 8: return go_ng<QR, KI8<false>, VI8<false>>(P, grid, chank, ng, st);
    case 4: return go_ng<QR, KI4, VI4>(P, grid, chank, ng, st);
    case 2: return go_ng<QR, KI2, VI2, false>(P, grid, chank, ng, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

AttnParams make_attn_params(const CacheArgs& c, const DecodeLaunch& d) {
  AttnParams P;
  P.B = c.B; P.H = c.H; P.S = c.S; P.Hq = d.Hq; P.G = d.G; P.qtiles = d.qtiles;
  P.max_len = d.max_len; P.num_splits = d.num_splits; P.split_len = d.split_len;
  P.chunk_tokens = c.chunk_tokens; P.qscale = d.qscale; P.q = d.q; P.seq_len = d.seq_len;
  P.out = d.out; P.ws = d.ws; P.oak_ksc = d.oak_ksc; P.seg = c.seg; P.status = c.status;
  P.k = c.k; P.v = c.v;
  P.pages = c.pages;
  P.pshift = c.ptok ? __builtin_ctz((unsigned)c.ptok) : 0;
  P.npages = c.npages;
  P.dsq_sig = c.dsq_sig;
  return P;
}


// Log-sum-exp merge of split partials: one workgroup of 1024 threads per
// (b, query head): M = max m_j, L = sum l_j 2^(m_j - M), out = sum 2^(m_j - M) o_j / L.
// Thread t owns output channel t mod 128 and the splits j = t / 128 (mod 8);
// it issues the loads of up to kMergeRun of its splits at once and folds them
// into a running (max, sum, output) state, rescaled when the max grows, so a
// merge of up to 128 splits waits on one round of loads.  The eight states of
// each channel are then combined through LDS in a fixed order.
constexpr int kMergeThreads = 1024;
constexpr int kMergeRun = 16;

__global__ __launch_bounds__(kMergeThreads) void k_merge(const float* __restrict__ ws, int NS,
                                                        float* __restrict__ out) {
  constexpr int NP = kMergeThreads / kD;  // threads per output channel
  __shared__ float pm[NP], pl[NP];
  __shared__ float po[NP][kD];
  const long long bq = blockIdx.x;
  const int t = threadIdx.x, d = t & (kD - 1), part = t / kD;
  const float* rec0 = ws + bq * NS * kPartStride;
  float M = -INFINITY, Ls = 0.0f, O = 0.0f;
  for (int s0 = part; s0 < NS; s0 += kMergeRun * NP) {
    float m[kMergeRun], l[kMergeRun], o[kMergeRun];
#pragma unroll
    for (int k = 0; k < kMergeRun; ++k) {
      const int s = s0 + k * NP;
      // past the last split, read split s0 again (in range) and drop it below
      const float* r = rec0 + (long long)(s < NS ? s : s0) * kPartStride;
      m[k] = r[0];
      l[k] = r[1];
      o[k] = r[4 + d];
    }
    float mx = M;
#pragma unroll
    for (int k = 0; k < kMergeRun; ++k) {
      if (s0 + k * NP >= NS) m[k] = -INFINITY;
      mx = fmaxf(mx, m[k]);
    }
    if (mx != -INFINITY) {
      const float c = fexp2(M - mx);  // 0 while M is still -inf
      Ls *= c;
      O *= c;
#pragma unroll
      for (int k = 0; k < kMergeRun; ++k) {
        const float f = fexp2(m[k] - mx);  // 0 for an empty or dropped split
        Ls = fmaf(f, l[k], Ls);
        O = fmaf(f, o[k], O);
      }
      M = mx;
    }
  }
  if (d == 0) {
    pm[part] = M;
    pl[part] = Ls;
  }
  po[part][d] = O;
  __syncthreads();
  if (t < kD) {
    float Mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < NP; ++p) Mx = fmaxf(Mx, pm[p]);
    float Lt = 0.0f, Ot = 0.0f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float f = fexp2(pm[p] - Mx);
        Lt = fmaf(f, pl[p], Lt);
        Ot = fmaf(f, po[p][t], Ot);
      }
    }
    out[bq * kD + t] = Lt > 0.0f ? Ot / Lt : 0.0f;
  }
}

hipError_t launch_merge(const DecodeLaunch& d, int B, hipStream_t st) {
  hipLaunchKernelGGL(k_merge, dim3((unsigned)(B * d.Hq)), dim3(kMergeThreads), 0, st, d.ws, d.num_splits,
                     d.out);
  return hipGetLastError();
}

hipError_t launch_decode_uniform(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
  if (!decode_uniform_supported(c.k, c.v)) return hipErrorInvalidValue;
  const AttnParams P = make_attn_params(c, d);
  const dim3 grid((unsigned)d.num_splits, (unsigned)(c.H * d.qtiles), (unsigned)c.B);
  switch (d.qr) {
    case 1: return go_codec<1>(P, grid, st);
    case 4: return go_codec<4>(P, grid, st);
    case 16: return go_codec<16>(P, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
