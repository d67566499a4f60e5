// Decode kernels for the Oaken cache: the dense INT4 body goes through the
// matrix cores like any token-axis group; each row's sparse outer entries add
// q[idx] * x_hat to the row's score and p * x_hat to output channel idx (LDS
// accumulators rescaled with the running maximum).  Reconstruction follows
// the Oaken page, §3.2.2: x_hat = T_hi + mag * s_out above, T_lo - mag * s_out
// below; the dense value at an outer position is exactly 0.
#include "kvq_attn_impl.h"

namespace kvq {
namespace {

__device__ __forceinline__ SparseView make_sparse(const TensorArgs& t, long long bh, long long S, int ng) {
  SparseView v;
  v.oscale = t.oscale + bh * S * ng;
  v.rowptr = t.rowptr + bh * (S + 1);
  v.sparse = t.sparse + bh * t.sparse_cap;
  v.cap = (unsigned)t.sparse_cap;
  v.t_lo = t.thr_lo;
  v.t_hi = t.thr_hi;
  return v;
}

template <int QR, int NG>
__global__ __launch_bounds__(256) void k_attn_oaken(AttnParams P) {
  __shared__ AttnLds<QR, NG, true> L;
  const int split = blockIdx.x, qt = blockIdx.y % P.qtiles, kvh = blockIdx.y / P.qtiles, b = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int nq = min(QR, P.G - qt * QR);
  u4_t qop[4];
  attn_prologue<QR, NG>(P, L, b, kvh, qt, nq, qop);
  const int len = clamp_seq_len(P, b, split == 0 && blockIdx.y == 0 && threadIdx.x == 0);
  const int t0 = split * P.split_len;
  const int t1 = min(len, t0 + P.split_len);
  SoftState<QRows<QR>::GI> st;
  soft_init(st);
  if (t0 < t1) {
    const long long bh = (long long)b * P.H + kvh;
    const long long S = P.S;
    const TokView kv{P.k.codes + bh * S * KI4::RB, P.k.scale + bh * S * NG, P.k.zero + bh * S * NG};
    const TokView vv{P.v.codes + bh * S * VI4::RB, P.v.scale + bh * S * NG, P.v.zero + bh * S * NG};
    const ChanView nc{nullptr, nullptr};
    const SparseView ks = make_sparse(P.k, bh, S, NG), vs = make_sparse(P.v, bh, S, NG);
    attend_wave<QR, NG, NG, KI4, VI4, false, true, 2>(P, L, st, kv, vv, nc, ks, vs, nq, t0, t1, wave,
                                                       qop);
  }
  wave_record<QR, NG, true>(L, st, wave, nq);
  finish_split(P, L, b, kvh, qt, split, nq);
}

template <int QR>
hipError_t go(const AttnParams& P, int ng, dim3 grid, hipStream_t st) {
  switch (ng) {
    case 1: hipLaunchKernelGGL((k_attn_oaken<QR, 1>), grid, dim3(kNW * 64), 0, st, P); break;
    case 2: hipLaunchKernelGGL((k_attn_oaken<QR, 2>), grid, dim3(kNW * 64), 0, st, P); break;
    case 4: hipLaunchKernelGGL((k_attn_oaken<QR, 4>), grid, dim3(kNW * 64), 0, st, P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_oaken(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
  if (c.k.group != c.v.group) return hipErrorInvalidValue;
  const AttnParams P = make_attn_params(c, d);
  const dim3 grid((unsigned)d.num_splits, (unsigned)(c.H * d.qtiles), (unsigned)c.B);
  const int ng = kD / c.v.group;
  switch (d.qr) {
    case 1: return go<1>(P, ng, grid, st);
    case 4: return go<4>(P, ng, grid, st);
    case 16: return go<16>(P, ng, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
