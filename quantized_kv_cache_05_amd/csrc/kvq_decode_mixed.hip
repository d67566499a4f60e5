// Decode kernels for the chunk-mixed cache ([Cocktail page] §3.1.2 / §3.2.3):
// a split covers a range of reordered chunk slots; the part of it in each
// class (FP16, INT4, INT2) is a contiguous row range of that class's pool,
// attended with that class's codec.  Per-class results are folded into the
// same per-wave record, so the split emits one partial.
#include "kvq_decode_impl.h"

namespace kvq {
namespace {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int GT, int NG>
__global__ __launch_bounds__(256) void k_decode_mixed(DecodeParams P) {
  using C16 = F16Codec;
  using C4 = TokCodec<4, false, NG>;
  using C2 = TokCodec<2, false, NG>;
  constexpr int L16 = 16;
  constexpr int L4 = cmax(C4::MIN_LPR, GT > 1 ? 8 : 1);
  constexpr int L2 = cmax(C2::MIN_LPR, GT > 1 ? 8 : 1);
  __shared__ float q_lds[GT * kD];
  __shared__ float canon[kNW * GT * (kD + 2)];
  const int split = blockIdx.x, qt = blockIdx.y % P.qtiles, kvh = blockIdx.y / P.qtiles, b = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  decode_prologue<GT, false>(P, b, kvh, qt, q_lds, canon, nullptr);
  const int CT = P.chunk_tokens;
  const int n16 = P.seg[b * 4], n4 = P.seg[b * 4 + 1], n = P.seg[b * 4 + 3];
  const int j0 = split * P.split_len;
  const int j1 = min(n, j0 + P.split_len);
  const long long bh = (long long)b * P.H + kvh;
  const long long rows = (long long)P.S;  // pool rows per (b, h)
  float* my = canon + wave * GT * (kD + 2);
  {
    const int a = max(j0, 0), e = min(j1, n16);
    if (a < e) {
      C16 k16, v16;
      k16.codes = P.k.codes16 + bh * rows * C16::RB;
      v16.codes = P.v.codes16 + bh * rows * C16::RB;
      attend_segment<L16, GT, 32>(k16, v16, a * CT, e * CT, wave, q_lds, nullptr, my);
    }
  }
  {
    const int a = max(j0, n16), e = min(j1, n16 + n4);
    if (a < e) {
      C4 k4, v4;
      k4.codes = P.k.codes + bh * rows * C4::RB;
      k4.scale = P.k.scale + bh * rows * NG;
      k4.zero = P.k.zero + bh * rows * NG;
      v4.codes = P.v.codes + bh * rows * C4::RB;
      v4.scale = P.v.scale + bh * rows * NG;
      v4.zero = P.v.zero + bh * rows * NG;
      attend_segment<L4, GT, 64>(k4, v4, (a - n16) * CT, (e - n16) * CT, wave, q_lds, nullptr, my);
    }
  }
  {
    const int a = max(j0, n16 + n4), e = min(j1, n);
    if (a < e) {
      C2 k2, v2;
      k2.codes = P.k.codes2 + bh * rows * C2::RB;
      k2.scale = P.k.scale2 + bh * rows * NG;
      k2.zero = P.k.zero2 + bh * rows * NG;
      v2.codes = P.v.codes2 + bh * rows * C2::RB;
      v2.scale = P.v.scale2 + bh * rows * NG;
      v2.zero = P.v.zero2 + bh * rows * NG;
      attend_segment<L2, GT, 64>(k2, v2, (a - n16 - n4) * CT, (e - n16 - n4) * CT, wave, q_lds,
                                 nullptr, my);
    }
  }
  decode_epilogue<GT>(P, b, kvh, qt, split, canon);
}

template <int GT>
hipError_t go(const CacheArgs& c, const DecodeParams& P, dim3 grid, hipStream_t st) {
  switch (kD / c.v.group) {
    case 1: hipLaunchKernelGGL((k_decode_mixed<GT, 1>), grid, dim3(kNW * 64), 0, st, P); break;
    case 2: hipLaunchKernelGGL((k_decode_mixed<GT, 2>), grid, dim3(kNW * 64), 0, st, P); break;
    case 4: hipLaunchKernelGGL((k_decode_mixed<GT, 4>), grid, dim3(kNW * 64), 0, st, P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mixed(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
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
