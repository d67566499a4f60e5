// Decode kernels for the Oaken cache: the dense INT4 body is dequantized like
// any token-axis group; each row's sparse outer entries add q[idx] * x_hat to
// the score and p * x_hat to output channel idx (an LDS accumulator per wave,
// rescaled with the running max) ([Oaken page] §3.2.2 reconstruction
// T_hi + delta * s / T_lo + delta * s; the dense value at an outer position is 0).
#include "kvq_decode_impl.h"

namespace kvq {
namespace {

template <int NG>
__device__ __forceinline__ OakenCodec<NG> make_oaken(const TensorArgs& t, long long bh, int S) {
  OakenCodec<NG> c;
  c.codes = t.codes + bh * S * 64;
  c.scale = t.scale + bh * S * NG;
  c.zero = t.zero + bh * S * NG;
  c.oscale = t.oscale + bh * S * NG;
  c.rowptr = t.rowptr + bh * (S + 1);
  c.sparse = t.sparse + bh * t.sparse_cap;
  c.cap = t.sparse_cap;
  c.t_lo = t.thr_lo;
  c.t_hi = t.thr_hi;
  return c;
}

template <int GT, int NG>
__global__ __launch_bounds__(256) void k_decode_oaken(DecodeParams P) {
  constexpr int LPR = (GT > 1 ? 8 : OakenCodec<NG>::MIN_LPR);
  __shared__ float q_lds[GT * kD];
  __shared__ float canon[kNW * GT * (kD + 2)];
  __shared__ float osp[kNW * GT * kD];
  const int split = blockIdx.x, qt = blockIdx.y % P.qtiles, kvh = blockIdx.y / P.qtiles, b = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  decode_prologue<GT, true>(P, b, kvh, qt, q_lds, canon, osp);
  const int len = clamp_len(P, b, split == 0 && blockIdx.y == 0 && threadIdx.x == 0);
  const int t0 = split * P.split_len;
  const int t1 = min(len, t0 + P.split_len);
  const long long bh = (long long)b * P.H + kvh;
  if (t0 < t1) {
    const OakenCodec<NG> kc = make_oaken<NG>(P.k, bh, P.S);
    const OakenCodec<NG> vc = make_oaken<NG>(P.v, bh, P.S);
    attend_segment<LPR, GT, 64>(kc, vc, t0, t1, wave, q_lds, osp + wave * GT * kD,
                                canon + wave * GT * (kD + 2));
  }
  decode_epilogue<GT>(P, b, kvh, qt, split, canon);
}

template <int GT>
hipError_t go(const CacheArgs& c, const DecodeParams& P, dim3 grid, hipStream_t st) {
  switch (kD / c.v.group) {
    case 1: hipLaunchKernelGGL((k_decode_oaken<GT, 1>), grid, dim3(kNW * 64), 0, st, P); break;
    case 2: hipLaunchKernelGGL((k_decode_oaken<GT, 2>), grid, dim3(kNW * 64), 0, st, P); break;
    case 4: hipLaunchKernelGGL((k_decode_oaken<GT, 4>), grid, dim3(kNW * 64), 0, st, P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_oaken(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
  if (c.k.group != c.v.group) return hipErrorInvalidValue;
  DecodeParams P;
  P.B = c.B; P.H = c.H; P.S = c.S; P.Hq = d.Hq; P.G = d.G; P.qtiles = d.qtiles;
  P.max_len = d.max_len; P.num_splits = d.num_splits; P.split_len = d.split_len;
  P.chunk_tokens = c.chunk_tokens; P.qscale = d.qscale; P.q = d.q; P.seq_len = d.seq_len;
  P.out = d.out; P.ws = d.ws; P.seg = c.seg; P.status = c.status; P.k = c.k; P.v = c.v;
  const dim3 grid((unsigned)d.num_splits, (unsigned)(c.H * d.qtiles), (unsigned)c.B);
  if (d.gtile == 1) return go<1>(c, P, grid, st);
  if (d.gtile == 4) return go<4>(c, P, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace kvq
