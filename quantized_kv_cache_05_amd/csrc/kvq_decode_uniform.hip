// Decode kernels for the uniform cache: token-axis K and V groups, or K with
// channel-axis groups of 64 tokens and token-axis V (see kvq_attn.h).
#include "kvq_attn_impl.h"

namespace kvq {
namespace {

// Occupancy target (waves per SIMD): two in general; four for the 4-query
// per-channel-K kernels with 4- or 2-bit codes and two V groups, and for the
// paged one-query kernels with at most two groups other than asymmetric
// INT8, which fit in 128 registers without spilling (the contiguous
// one-query kernels land there by themselves).
template <int QR, class KC, int NGV, bool CHANK, bool PAGED>
constexpr int kUniformWaves = ((CHANK && QR == 4 && NGV == 2 && KC::BITS <= 4) ||
                               (PAGED && QR == 1 && NGV <= 2 && !(KC::BITS == 8 && !KC::SYM)))
                                  ? 4
                                  : 2;

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
      const int pshift = P.pshift;
      kv = TokView{P.k.codes, P.k.scale, KC::SYM ? nullptr : P.k.zero,
                   P.pages + (long long)b * (S >> pshift), pshift, kvh << pshift, P.H << pshift,
                   P.npages, P.status};
      vv = TokView{P.v.codes, P.v.scale, VC::SYM ? nullptr : P.v.zero, kv.pages, pshift, kv.hrow, kv.prow,
                   P.npages, P.status};
    }
    attend_wave<QR, NGK, NGV, KC, VC, CHANK, false, 2, PAGED>(P, L, st, kv, vv, kc, nullptr, 0, nq, t0,
                                                               min(t1, lq), wave, qop);
  }
  if constexpr (CHANK) {
    if (max(t0, lq) < t1) {
      const long long bh = (long long)b * P.H + kvh;
      const long long S = P.S;
      // row t of the view is tail row t - lq
      const TokView kt{P.k.codes16 + (bh * 64 - lq) * KF16::RB, nullptr, nullptr};
      const TokView vv{P.v.codes + bh * S * VC::RB, P.v.scale + bh * S * NGV,
                       VC::SYM ? nullptr : P.v.zero + bh * S * NGV};
      const ChanView nc{nullptr, nullptr};
      // the query operand is rebuilt here rather than kept live through the main loop
      u4_t qop16[4];
      build_qop<QR>(L, qop16);
      attend_wave<QR, 1, NGV, KF16, VC, false, false, 1>(P, L, st, kt, vv, nc, nullptr, 0, nq,
                                                         max(t0, lq), t1, wave, qop16);
    }
  }
  wave_record<QR, NGV>(L, st, wave, nq);
  finish_split(P, L, b, kvh, qt, split, nq);
}

template <int QR, class KC, class VC, int NGK, int NGV, bool CHANK>
hipError_t go(const AttnParams& P, dim3 grid, hipStream_t st) {
  if constexpr (!CHANK) {
    if (P.pages) {
      hipLaunchKernelGGL((k_attn_uniform<QR, KC, VC, NGK, NGV, false, true>), grid, dim3(kNW * 64), 0, st, P);
      return hipGetLastError();
    }
  }
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
  P.out = d.out; P.ws = d.ws; P.seg = c.seg; P.status = c.status;
  P.k = c.k; P.v = c.v;
  P.pages = c.pages;
  P.pshift = c.ptok ? __builtin_ctz((unsigned)c.ptok) : 0;
  P.npages = c.npages;
  P.dsq_sig = c.dsq_sig;
  return P;
}

bool decode_uniform_supported(const TensorArgs& k, const TensorArgs& v) {
  if (v.axis != 0) return false;
  if (v.group != 32 && v.group != 64 && v.group != 128) return false;
  if (k.bits != v.bits || k.sym != v.sym || k.fmt != v.fmt) return false;
  if (v.fmt == 1) return v.bits == 8 && !v.sym && k.axis == 0 && k.group == v.group;
  if (v.sym && v.bits != 8) return false;
  if (v.bits != 8 && v.bits != 4 && v.bits != 2) return false;
  if (k.axis == 0) return k.group == v.group;
  if (k.axis == 1) return k.group == 64 && !k.sym && (k.bits == 8 || k.bits == 4);
  return false;
}

// Log-sum-exp merge of split partials: one workgroup of 128 threads per
// (b, query head): M = max m_j, L = sum l_j 2^(m_j - M), out = sum 2^(m_j - M) o_j / L.
// Split weights are formed cooperatively in LDS, chunk by chunk, so each
// thread's loads of its output channel are independent of one another.
__global__ __launch_bounds__(128) void k_merge(const float* __restrict__ ws, int NS,
                                              float* __restrict__ out) {
  constexpr int CH = 512;  // splits per LDS chunk
  __shared__ float wgt[CH];
  __shared__ float red[128];
  const long long bq = blockIdx.x;
  const int d = threadIdx.x;
  const float* rec0 = ws + bq * NS * kPartStride;
  float M = -INFINITY;
  for (int s = d; s < NS; s += 128) M = fmaxf(M, rec0[(long long)s * kPartStride]);
  red[d] = M;
  __syncthreads();
  for (int w = 64; w > 0; w >>= 1) {
    if (d < w) red[d] = fmaxf(red[d], red[d + w]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();
  float Lp = 0.0f, O = 0.0f;
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < NS; c0 += CH) {
      const int n = min(CH, NS - c0);
      for (int s = d; s < n; s += 128) {
        const float* r = rec0 + (long long)(c0 + s) * kPartStride;
        const float ms = r[0];
        const float f = ms == -INFINITY ? 0.0f : fexp2(ms - M);
        wgt[s] = f;
        Lp = fmaf(f, r[1], Lp);
      }
      __syncthreads();
      const float* r = rec0 + (long long)c0 * kPartStride + 4 + d;
      int s = 0;
      for (; s + 8 <= n; s += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = r[(long long)(s + k) * kPartStride];
#pragma unroll
        for (int k = 0; k < 8; ++k) O = fmaf(wgt[s + k], v[k], O);
      }
      for (; s < n; ++s) O = fmaf(wgt[s], r[(long long)s * kPartStride], O);
      __syncthreads();
    }
  }
  red[d] = Lp;
  __syncthreads();
  for (int w = 64; w > 0; w >>= 1) {
    if (d < w) red[d] += red[d + w];
    __syncthreads();
  }
  const float L = red[0];
  out[bq * kD + d] = L > 0.0f ? O / L : 0.0f;
}

hipError_t launch_merge(const DecodeLaunch& d, int B, hipStream_t st) {
  hipLaunchKernelGGL(k_merge, dim3((unsigned)(B * d.Hq)), dim3(kD), 0, st, d.ws, d.num_splits, d.out);
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
