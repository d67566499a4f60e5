// Decode kernels for the Oaken cache.  The dense INT4 body goes through the
// matrix-core tile loop like any token-axis group; the sparse outer values
// (reconstruction from the Oaken page, §3.2.2: x_hat = T_hi + mag * s_out
// above the upper outer threshold, T_lo - mag * s_out below the lower one;
// the dense value at an outer position is 0) are consumed inside the same
// loop, tile by tile (OakWave in kvq_attn_impl.h): each tile's slice of the
// row-major entry list is read with coalesced 8-byte loads issued with the
// tile's codes, K entries add to the tile's scores before the softmax, V
// entries add to the wave's outer-value output after it.  The Oaken page
// (§2.3) names the access cost of sparse formats; reading each tile's entries
// as one contiguous range keeps them on the streaming path.
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
    const OakCtx<QR, NG> oc{{make_list(P.k, bh, S), make_list(P.v, bh, S)}, &OW[wave]};
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
  switch (d.qr) {
    case 1: return go<1>(P, ng, grid, st);
    case 4: return go<4>(P, ng, grid, st);
    case 16: return go<16>(P, ng, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
