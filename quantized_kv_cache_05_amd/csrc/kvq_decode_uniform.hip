// Decode kernels for the uniform cache (token-axis K and V, or channel-axis
// K with token-axis V) and the split merge.
#include "kvq_decode_impl.h"

namespace kvq {
namespace {

template <class C>
struct Maker;
template <int BITS, bool SYM, int NG>
struct Maker<TokCodec<BITS, SYM, NG>> {
  using T = TokCodec<BITS, SYM, NG>;
  static __device__ __forceinline__ T make(const TensorArgs& t, long long bh, int S) {
    T c;
    c.codes = t.codes + bh * S * T::RB;
    c.scale = t.scale + bh * S * NG;
    c.zero = SYM ? nullptr : t.zero + bh * S * NG;
    return c;
  }
};
template <int BITS>
struct Maker<ChanCodec<BITS>> {
  using T = ChanCodec<BITS>;
  static __device__ __forceinline__ T make(const TensorArgs& t, long long bh, int S) {
    T c;
    c.codes = t.codes + bh * S * T::RB;
    c.scale = t.scale + bh * (S / 64) * kD;
    c.zero = t.zero + bh * (S / 64) * kD;
    return c;
  }
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int GT, class KC, class VC>
struct Layout {
  static constexpr int LPR = cmax(cmax(KC::MIN_LPR, VC::MIN_LPR), GT > 1 ? 8 : 1);
};

template <int GT, class KC, class VC>
__global__ __launch_bounds__(256) void k_decode_uniform(DecodeParams P) {
  constexpr int LPR = Layout<GT, KC, VC>::LPR;
  __shared__ float q_lds[GT * kD];
  __shared__ float canon[kNW * GT * (kD + 2)];
  const int split = blockIdx.x, qt = blockIdx.y % P.qtiles, kvh = blockIdx.y / P.qtiles, b = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  decode_prologue<GT, false>(P, b, kvh, qt, q_lds, canon, nullptr);
  int len = clamp_len(P, b, split == 0 && blockIdx.y == 0 && threadIdx.x == 0);
  if constexpr (KC::kind == kChan) {
    if (len & 63) {
      if (split == 0 && blockIdx.y == 0 && threadIdx.x == 0) set_flag(P.status, kFlagLenRange);
      len &= ~63;
    }
  }
  const int t0 = split * P.split_len;
  const int t1 = min(len, t0 + P.split_len);
  const long long bh = (long long)b * P.H + kvh;
  if (t0 < t1) {
    const KC kc = Maker<KC>::make(P.k, bh, P.S);
    const VC vc = Maker<VC>::make(P.v, bh, P.S);
    attend_segment<LPR, GT, 64>(kc, vc, t0, t1, wave, q_lds, nullptr, canon + wave * GT * (kD + 2));
  }
  decode_epilogue<GT>(P, b, kvh, qt, split, canon);
}

// kvq merge: one workgroup of 128 threads per (b, query head).
__global__ __launch_bounds__(128) void k_merge(const float* __restrict__ ws, int NS,
                                              float* __restrict__ out) {
  const long long bq = blockIdx.x;
  const int d = threadIdx.x;
  const float* rec0 = ws + bq * NS * kPartStride;
  float M = -INFINITY;
  for (int s = 0; s < NS; ++s) M = fmaxf(M, rec0[(long long)s * kPartStride]);
  float L = 0.0f, O = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < NS; ++s) {
      const float* rec = rec0 + (long long)s * kPartStride;
      if (rec[0] != -INFINITY) {
        const float f = fexp2(rec[0] - M);
        L = fmaf(f, rec[1], L);
        O = fmaf(f, rec[4 + d], O);
      }
    }
  }
  out[bq * kD + d] = L > 0.0f ? O / L : 0.0f;
}

DecodeParams make_params(const CacheArgs& c, const DecodeLaunch& d) {
  DecodeParams P;
  P.B = c.B; P.H = c.H; P.S = c.S; P.Hq = d.Hq; P.G = d.G; P.qtiles = d.qtiles;
  P.max_len = d.max_len; P.num_splits = d.num_splits; P.split_len = d.split_len;
  P.chunk_tokens = c.chunk_tokens; P.qscale = d.qscale; P.q = d.q; P.seq_len = d.seq_len;
  P.out = d.out; P.ws = d.ws; P.seg = c.seg; P.status = c.status; P.k = c.k; P.v = c.v;
  return P;
}

template <int GT, class KC, class VC>
hipError_t go(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
  const dim3 grid((unsigned)d.num_splits, (unsigned)(c.H * d.qtiles), (unsigned)c.B);
  hipLaunchKernelGGL((k_decode_uniform<GT, KC, VC>), grid, dim3(kNW * 64), 0, st, make_params(c, d));
  return hipGetLastError();
}

template <int GT, int BITS, bool SYM>
hipError_t go_ng(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
  const int ng = kD / c.v.group;
  if (c.k.axis == 1) {
    if constexpr (SYM || BITS == 2) {
      return hipErrorInvalidValue;
    } else {
      switch (ng) {
        case 1: return go<GT, ChanCodec<BITS>, TokCodec<BITS, false, 1>>(c, d, st);
        case 2: return go<GT, ChanCodec<BITS>, TokCodec<BITS, false, 2>>(c, d, st);
        case 4: return go<GT, ChanCodec<BITS>, TokCodec<BITS, false, 4>>(c, d, st);
        default: return hipErrorInvalidValue;
      }
    }
  }
  switch (ng) {
    case 1: return go<GT, TokCodec<BITS, SYM, 1>, TokCodec<BITS, SYM, 1>>(c, d, st);
    case 2: return go<GT, TokCodec<BITS, SYM, 2>, TokCodec<BITS, SYM, 2>>(c, d, st);
    case 4: return go<GT, TokCodec<BITS, SYM, 4>, TokCodec<BITS, SYM, 4>>(c, d, st);
    default: return hipErrorInvalidValue;
  }
}

template <int GT>
hipError_t go_bits(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
  if (c.v.sym) return go_ng<GT, 8, true>(c, d, st);
  switch (c.v.bits) {
    case 8: return go_ng<GT, 8, false>(c, d, st);
    case 4: return go_ng<GT, 4, false>(c, d, st);
    case 2: return go_ng<GT, 2, false>(c, d, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_uniform_supported(const TensorArgs& k, const TensorArgs& v) {
  if (v.axis != 0) return false;
  if (v.group != 32 && v.group != 64 && v.group != 128) return false;
  if (k.bits != v.bits || k.sym != v.sym) return false;
  if (v.sym && v.bits != 8) return false;
  if (v.bits != 8 && v.bits != 4 && v.bits != 2) return false;
  if (k.axis == 0) return k.group == v.group;
  if (k.axis == 1) return k.group == 64 && !k.sym && (k.bits == 8 || k.bits == 4);
  return false;
}

hipError_t launch_decode_uniform(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
  if (!decode_uniform_supported(c.k, c.v)) return hipErrorInvalidValue;
  if (d.gtile == 1) return go_bits<1>(c, d, st);
  if (d.gtile == 4) return go_bits<4>(c, d, st);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const DecodeLaunch& d, int B, hipStream_t st) {
  hipLaunchKernelGGL(k_merge, dim3((unsigned)(B * d.Hq)), dim3(kD), 0, st, d.ws, d.num_splits, d.out);
  return hipGetLastError();
}

}  // namespace kvq
