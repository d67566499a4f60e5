// Decode kernels for the chunk-mixed cache (the Cocktail page, §3.1.2 reorder
// and §3.2.3 per-block attention with a merge): a split covers a range of
// reordered chunk slots; its part in each class (FP16, INT4, INT2) is a
// contiguous row range of that class's pool, attended with that class's
// codecs into the same running softmax state, so the split emits one partial.
// The tokens of a chunk still being appended are attended by the last split.
#include "kvq_attn_impl.h"

namespace kvq {
namespace {

template <int QR, int NG>
__global__ __launch_bounds__(256, 2) void k_attn_mixed(AttnParams P) {
  __shared__ AttnLds<QR, NG> L;
  const int split = blockIdx.x, qt = blockIdx.y % P.qtiles, kvh = blockIdx.y / P.qtiles, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar addressing
  const int nq = min(QR, P.G - qt * QR);
  u4_t qop[4];
  attn_prologue<QR, NG>(P, L, b, kvh, qt, nq, qop);
  const int CT = P.chunk_tokens;
  const int C = P.S / CT;
  int n16 = P.seg[b * 4], n4 = P.seg[b * 4 + 1], n = P.seg[b * 4 + 3];
  // counts outside the pool capacity (never written by kvq_reorder_chunks) attend nothing
  if (n16 < 0 || n4 < 0 || n > C || n16 + n4 > n) n = n16 = n4 = 0;
  const int j0 = split * P.split_len;
  const int j1 = min(n, j0 + P.split_len);
  const long long bh = (long long)b * P.H + kvh;
  const long long S = P.S;
  SoftState<QRows<QR>::GI> st;
  soft_init(st);
  const ChanView nc{nullptr, nullptr};
  {
    const int a = max(j0, 0), e = min(j1, n16);
    if (a < e) {
      const TokView k16{P.k.codes16 + bh * S * KF16::RB, nullptr, nullptr};
      const TokView v16{P.v.codes16 + bh * S * VF16::RB, nullptr, nullptr};
      attend_wave<QR, 1, 1, KF16, VF16, false, false, 1>(P, L, st, k16, v16, nc, NoOak{}, nq,
                                                          a * CT, e * CT, wave, qop);
    }
  }
  {
    const int a = max(j0, n16), e = min(j1, n16 + n4);
    if (a < e) {
      const TokView k4{P.k.codes + bh * S * KI4::RB, P.k.scale + bh * S * NG, P.k.zero + bh * S * NG};
      const TokView v4{P.v.codes + bh * S * VI4::RB, P.v.scale + bh * S * NG, P.v.zero + bh * S * NG};
      attend_wave<QR, NG, NG, KI4, VI4, false, false, 2>(P, L, st, k4, v4, nc, NoOak{}, nq,
                                                          (a - n16) * CT, (e - n16) * CT, wave, qop);
    }
  }
  {
    const int a = max(j0, n16 + n4), e = min(j1, n);
    if (a < e) {
      const TokView k2{P.k.codes2 + bh * S * KI2::RB, P.k.scale2 + bh * S * NG, P.k.zero2 + bh * S * NG};
      const TokView v2{P.v.codes2 + bh * S * VI2::RB, P.v.scale2 + bh * S * NG, P.v.zero2 + bh * S * NG};
      attend_wave<QR, NG, NG, KI2, VI2, false, false, 2>(P, L, st, k2, v2, nc, NoOak{}, nq,
                                                          (a - n16 - n4) * CT, (e - n16 - n4) * CT,
                                                          wave, qop);
    }
  }
  // tokens of the chunk not yet complete (streaming appends) wait as fp16 in
  // the FP16 pool's last chunk: the last split attends seg[b][3] * CT ..
  // seq_len[b] - 1 of them
  if (P.seq_len && split == P.num_splits - 1 && n < C) {
    const int len = clamp_seq_len(P, b, blockIdx.y == 0 && threadIdx.x == 0);
    const int w0 = n * CT, w1 = min(len, w0 + CT - 1);
    if (w0 < w1) {
      const long long wr = bh * S + (long long)(C - 1) * CT - w0;  // row of token t: wr + t
      const TokView kw{P.k.codes16 + wr * KF16::RB, nullptr, nullptr};
      const TokView vw{P.v.codes16 + wr * VF16::RB, nullptr, nullptr};
      attend_wave<QR, 1, 1, KF16, VF16, false, false, 1>(P, L, st, kw, vw, nc, NoOak{}, nq, w0, w1, wave,
                                                          qop);
    }
  }
  wave_record<QR, NG>(L, st, wave, nq);
  finish_split(P, L, b, kvh, qt, split, nq);
}

template <int QR>
hipError_t go(const AttnParams& P, int ng, dim3 grid, hipStream_t st) {
  switch (ng) {
    case 1: hipLaunchKernelGGL((k_attn_mixed<QR, 1>), grid, dim3(kNW * 64), 0, st, P); break;
    case 2: hipLaunchKernelGGL((k_attn_mixed<QR, 2>), grid, dim3(kNW * 64), 0, st, P); break;
    case 4: hipLaunchKernelGGL((k_attn_mixed<QR, 4>), grid, dim3(kNW * 64), 0, st, P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mixed(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
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
