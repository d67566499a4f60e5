// Decode kernels for the chunk-mixed cache (the Cocktail page, §3.1.2 reorder
// and §3.2.3 per-block attention with a merge): a split covers a range of
// reordered chunk slots; its part in each class (FP16, INT4, INT2) is a
// contiguous row range of that class's pool, attended with that class's
// codecs into the same running softmax state, so the split emits one partial.
// The tokens of a chunk still being appended are attended by the last split.
// Paged, each class pool is a pool of pages with its own block-table row per
// sequence; steps of 32 or 64 class-local rows never straddle a page.
#include "kvq_attn_impl.h"

namespace kvq {
namespace {

// View of class cls's pool for (b, kvh) (row t of the view = class-local row
// t): contiguous, or paged through class cls's block-table row.
template <bool PAGED, int RB, int NGC>
__device__ __forceinline__ TokView class_view(const AttnParams& P, int cls, int b, int kvh, const uint8_t* codes,
                                              const float* scale, const uint8_t* zero) {
  const long long S = P.S, bh = (long long)b * P.H + kvh;
  if constexpr (PAGED) {
    const int pshift = P.pshift;
    return TokView{codes, scale, zero, P.pages + ((long long)cls * P.B + b) * (S >> pshift), pshift,
                   kvh << pshift, P.H << pshift, P.npages, P.status};
  } else {
    return TokView{codes + bh * S * RB, scale ? scale + bh * S * NGC : nullptr,
                   zero ? zero + bh * S * NGC : nullptr};
  }
}

template <int QR, int NG, bool PAGED>
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
  SoftState<QRows<QR>::GI> st;
  soft_init(st);
  const ChanView nc{nullptr, nullptr};
  {
    const int a = max(j0, 0), e = min(j1, n16);
    if (a < e) {
      const TokView k16 = class_view<PAGED, KF16::RB, 1>(P, 0, b, kvh, P.k.codes16, nullptr, nullptr);
      const TokView v16 = class_view<PAGED, VF16::RB, 1>(P, 0, b, kvh, P.v.codes16, nullptr, nullptr);
      attend_wave<QR, 1, 1, KF16, VF16, false, false, 1, PAGED>(P, L, st, k16, v16, nc, NoOak{}, nq, a * CT,
                                                                 e * CT, wave, qop);
    }
  }
  {
    const int a = max(j0, n16), e = min(j1, n16 + n4);
    if (a < e) {
      const TokView k4 = class_view<PAGED, KI4::RB, NG>(P, 1, b, kvh, P.k.codes, P.k.scale, P.k.zero);
      const TokView v4 = class_view<PAGED, VI4::RB, NG>(P, 1, b, kvh, P.v.codes, P.v.scale, P.v.zero);
      attend_wave<QR, NG, NG, KI4, VI4, false, false, 2, PAGED>(P, L, st, k4, v4, nc, NoOak{}, nq,
                                                                 (a - n16) * CT, (e - n16) * CT, wave, qop);
    }
  }
  {
    const int a = max(j0, n16 + n4), e = min(j1, n);
    if (a < e) {
      const TokView k2 = class_view<PAGED, KI2::RB, NG>(P, 2, b, kvh, P.k.codes2, P.k.scale2, P.k.zero2);
      const TokView v2 = class_view<PAGED, VI2::RB, NG>(P, 2, b, kvh, P.v.codes2, P.v.scale2, P.v.zero2);
      attend_wave<QR, NG, NG, KI2, VI2, false, false, 2, PAGED>(P, L, st, k2, v2, nc, NoOak{}, nq,
                                                                 (a - n16 - n4) * CT, (e - n16 - n4) * CT,
                                                                 wave, qop);
    }
  }
  // tokens of the chunk not yet complete (streaming appends) wait as fp16 in
  // the FP16 pool's last chunk, class-local rows (C - 1) CT on: the last
  // split attends seg[b][3] * CT .. seq_len[b] - 1 of them
  if (P.seq_len && split == P.num_splits - 1 && n < C) {
    const int len = clamp_seq_len(P, b, blockIdx.y == 0 && threadIdx.x == 0);
    const int w0 = n * CT, w1 = min(len, w0 + CT - 1);
    if (w0 < w1) {
      const TokView kw = class_view<PAGED, KF16::RB, 1>(P, 0, b, kvh, P.k.codes16, nullptr, nullptr);
      const TokView vw = class_view<PAGED, VF16::RB, 1>(P, 0, b, kvh, P.v.codes16, nullptr, nullptr);
      const int r0 = (C - 1) * CT;
      attend_wave<QR, 1, 1, KF16, VF16, false, false, 1, PAGED>(P, L, st, kw, vw, nc, NoOak{}, nq, r0,
                                                                 r0 + (w1 - w0), wave, qop);
    }
  }
  wave_record<QR, NG>(L, st, wave, nq);
  finish_split(P, L, b, kvh, qt, split, nq);
}

template <int QR, bool PAGED>
hipError_t go_pg(const AttnParams& P, int ng, dim3 grid, hipStream_t st) {
  switch (ng) {
    case 1: hipLaunchKernelGGL((k_attn_mixed<QR, 1, PAGED>), grid, dim3(kNW * 64), 0, st, P); break;
    case 2: hipLaunchKernelGGL((k_attn_mixed<QR, 2, PAGED>), grid, dim3(kNW * 64), 0, st, P); break;
    case 4: hipLaunchKernelGGL((k_attn_mixed<QR, 4, PAGED>), grid, dim3(kNW * 64), 0, st, P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int QR>
hipError_t go(const AttnParams& P, int ng, dim3 grid, hipStream_t st) {
  return P.pages ? go_pg<QR, true>(P, ng, grid, st) : go_pg<QR, false>(P, ng, grid, st);
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
