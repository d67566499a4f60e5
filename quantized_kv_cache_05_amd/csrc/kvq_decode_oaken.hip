// Decode kernels for the Oaken cache.  The dense INT4 body goes through the
// matrix-core tile loop like any token-axis group; the sparse outer values
// are handled in bulk around it (reconstruction from the Oaken page, §3.2.2:
// x_hat = T_hi + mag * s_out above the upper outer threshold, T_lo - mag *
// s_out below the lower one; the dense value at an outer position is 0):
//  - K pre-pass: every outer K entry of the split adds q[m][idx] * x_hat to
//    query m's score slot of its token (LDS);
//  - tile loop: the slot is added to the dense score and replaced by the
//    final base-2 score;
//  - V post-pass: with the workgroup maximum M known, every outer V entry
//    adds 2^(score - M) * x_hat to output channel idx of query m (LDS).
// One lane per row walks the row's entries (row pointers staged in LDS).
#include "kvq_attn_impl.h"

namespace kvq {
namespace {

constexpr int kOakSpan = 2048;  // query x token score slots per workgroup

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

struct OakLds {
  unsigned rp[kOakSpan + 1];  // row pointers of the split's rows (K, then V)
  float sc[kOakSpan];         // [query][token] score slots
};

// Stage the row pointers of rows t0 .. t0 + n of one tensor; ends with a barrier.
__device__ __forceinline__ void stage_rowptr(const SparseView& sv, int t0, int n, unsigned* rp) {
  for (int i = threadIdx.x; i <= n; i += blockDim.x) rp[i] = sv.rowptr[t0 + i];
  __syncthreads();
}

// The outer scales of token t's row (one per channel group); paged rows go
// through the block table (an entry outside the pool reads page 0, as the
// dense body does, which flags it).
template <int NG>
__device__ __forceinline__ void row_oscale(const SparseView& sv, long long t, float (&so)[NG]) {
  long long row = t;
  if (sv.pages) {
    int pg = sv.pages[t >> sv.pshift];
    if (pg < 0 || pg >= sv.npages) pg = 0;
    row = (long long)pg * sv.prow + sv.hrow + (t & ((1 << sv.pshift) - 1));
  }
  if constexpr (NG == 1) {
    so[0] = sv.oscale[row];
  } else if constexpr (NG == 2) {
    const float2 v = *reinterpret_cast<const float2*>(sv.oscale + row * 2);
    so[0] = v.x; so[1] = v.y;
  } else {
    const float4 v = *reinterpret_cast<const float4*>(sv.oscale + row * 4);
    so[0] = v.x; so[1] = v.y; so[2] = v.z; so[3] = v.w;
  }
}

// One lane per row of the split: begin(r), then f(r, channel idx, x_hat) for
// each of row r's entries, then end(r), for every row r of the lane.  A lane
// takes kRowsInFlight rows at a time and issues, before any use, the loads of
// their outer scales and of the first kEntriesAhead entries of each row
// (clamped to a valid address, masked at use), so a batch of rows costs one
// memory round trip; the rare rows with more entries finish with a tail loop.
// 16 entries ahead cover all but ~1e-4 of the rows at 5 % outer values (a
// row holds Binomial(128, 0.05) entries), so a wave almost never waits on a
// tail round trip; 2 rows x 16 entries hold as many registers as 4 x 8.
constexpr int kRowsInFlight = 2, kEntriesAhead = 16;

template <int NG>
__device__ __forceinline__ float entry_value(const SparseView& sv, unsigned en, const float (&so)[NG],
                                             int& idx) {
  idx = (int)(en & 127u);
  const float mag = (float)((en >> 8) & 31u);
  float s = so[0];
#pragma unroll
  for (int g = 1; g < NG; ++g)
    if (idx >= g * (128 / NG)) s = so[g];
  return ((en >> 7) & 1u) ? sv.t_hi + mag * s : sv.t_lo - mag * s;
}

template <int NG, class B, class F, class E>
__device__ __forceinline__ void for_row_entries(const SparseView& sv, int t0, int n,
                                                const unsigned* rp, B&& begin, F&& f, E&& end) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kStride = kNW * 64;
  if (sv.cap == 0) return;  // no list: every entry was dropped at append time
  const unsigned last = sv.cap - 1;
  for (int r0 = wave * 64; r0 < n; r0 += kRowsInFlight * kStride) {
    unsigned a[kRowsInFlight], c[kRowsInFlight], en[kRowsInFlight][kEntriesAhead];
    float so[kRowsInFlight][NG];
#pragma unroll
    for (int k = 0; k < kRowsInFlight; ++k) {
      const int r = r0 + k * kStride + lane;
      const int rc = min(r, n - 1);
      a[k] = min(rp[rc], sv.cap);
      c[k] = r < n ? min(rp[rc + 1], sv.cap) - a[k] : 0u;
      row_oscale<NG>(sv, t0 + rc, so[k]);
#pragma unroll
      for (int j = 0; j < kEntriesAhead; ++j) en[k][j] = sv.sparse[min(a[k] + j, last)];
    }
#pragma unroll
    for (int k = 0; k < kRowsInFlight; ++k) {
      const int r = r0 + k * kStride + lane;
      if (r < n) begin(r);
#pragma unroll
      for (int j = 0; j < kEntriesAhead; ++j) {
        if (j < (int)c[k]) {
          int idx;
          const float xh = entry_value<NG>(sv, en[k][j], so[k], idx);
          f(r, idx, xh);
        }
      }
      for (unsigned j = kEntriesAhead; __any(j < c[k]); j += 4) {
        unsigned e4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) e4[q] = sv.sparse[min(a[k] + j + q, last)];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (j + q < c[k]) {
            int idx;
            const float xh = entry_value<NG>(sv, e4[q], so[k], idx);
            f(r, idx, xh);
          }
        }
      }
      if (r < n) end(r);
    }
  }
}

template <int QR, int NG, bool PAGED>
__global__ __launch_bounds__(256, 2) void k_attn_oaken(AttnParams P) {
  __shared__ AttnLds<QR, NG> L;
  __shared__ OakLds OL;
  __shared__ float osp[QR][128];
  __shared__ float mwg[QR];
  constexpr int span = kOakSpan / QR;
  const int split = blockIdx.x, qt = blockIdx.y % P.qtiles, kvh = blockIdx.y / P.qtiles, b = blockIdx.z;
  // wave-uniform wave index (scalar addressing), except when paged (see the
  // uniform decode kernel: the block-table entry must stay a vector load)
  const int wave = PAGED ? (int)(threadIdx.x >> 6) : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nq = min(QR, P.G - qt * QR);
  u4_t qop[4];
  attn_prologue<QR, NG>(P, L, b, kvh, qt, nq, qop);
  const int len = clamp_seq_len(P, b, split == 0 && blockIdx.y == 0 && threadIdx.x == 0);
  const int t0 = split * P.split_len;
  const int t1 = min(len, t0 + P.split_len);
  const int n = t1 - t0;  // <= span (split planning)
  const long long bh = (long long)b * P.H + kvh;
  const long long S = P.S;
  SparseView ks = make_sparse(P.k, bh, S, NG), vs = make_sparse(P.v, bh, S, NG);
  if constexpr (PAGED) {  // outer scales sit with the dense rows, in pages
    for (SparseView* sv : {&ks, &vs}) {
      sv->oscale = (sv == &ks ? P.k : P.v).oscale;
      sv->pages = P.pages + (long long)b * (S >> P.pshift);
      sv->pshift = P.pshift;
      sv->hrow = kvh << P.pshift;
      sv->prow = P.H << P.pshift;
      sv->npages = P.npages;
    }
  }
  SoftState<QRows<QR>::GI> st;
  soft_init(st);
  if (n > 0) {
    // K pre-pass: each lane sums its row's outer K contributions per query
    stage_rowptr(ks, t0, n, OL.rp);
    {
      float acc[QR];
      for_row_entries<NG>(
          ks, t0, n, OL.rp,
          [&](int) {
#pragma unroll
            for (int m = 0; m < QR; ++m) acc[m] = 0.0f;
          },
          [&](int, int idx, float xh) {
#pragma unroll
            for (int m = 0; m < QR; ++m)
              if (m < nq) acc[m] = fmaf(L.q[m][idx], xh, acc[m]);
          },
          [&](int r) {
#pragma unroll
            for (int m = 0; m < QR; ++m)
              if (m < nq) OL.sc[m * span + r] = acc[m];
          });
    }
    __syncthreads();
    TokView kv{P.k.codes + bh * S * KI4::RB, P.k.scale + bh * S * NG, P.k.zero + bh * S * NG};
    TokView vv{P.v.codes + bh * S * VI4::RB, P.v.scale + bh * S * NG, P.v.zero + bh * S * NG};
    if constexpr (PAGED) {  // the dense body lives in pages: the views start at the pool bases
      const int pshift = P.pshift;
      kv = TokView{P.k.codes, P.k.scale, P.k.zero, P.pages + (long long)b * (S >> pshift), pshift, kvh << pshift,
                   P.H << pshift, P.npages, P.status};
      vv = TokView{P.v.codes, P.v.scale, P.v.zero, kv.pages, pshift, kv.hrow, kv.prow, P.npages, P.status};
    }
    const ChanView nc{nullptr, nullptr};
    attend_wave<QR, NG, NG, KI4, VI4, false, true, 2, PAGED>(P, L, st, kv, vv, nc, OL.sc, span, nq, t0, t1,
                                                              wave, qop);
  }
  wave_record<QR, NG>(L, st, wave, nq);
  __syncthreads();
  // V post-pass in the frame of the workgroup maximum
  for (int i = threadIdx.x; i < QR * 128; i += blockDim.x) (&osp[0][0])[i] = 0.0f;
  if (threadIdx.x < nq) mwg[threadIdx.x] = wg_max(L, threadIdx.x);
  if (n > 0) {
    stage_rowptr(vs, t0, n, OL.rp);  // (barrier inside)
    float pr[QR];
    for_row_entries<NG>(
        vs, t0, n, OL.rp,
        [&](int r) {
#pragma unroll
          for (int m = 0; m < QR; ++m) {
            const float s = m < nq ? OL.sc[m * span + r] : -INFINITY;
            pr[m] = s == -INFINITY ? 0.0f : fexp2(s - mwg[m]);
          }
        },
        [&](int, int idx, float xh) {
#pragma unroll
          for (int m = 0; m < QR; ++m)
            if (m < nq) atomicAdd(&osp[m][idx], pr[m] * xh);
        },
        [&](int) {});
  }
  finish_split(P, L, b, kvh, qt, split, nq, [&](int m, int d, float) { return osp[m][d]; });
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

int oaken_max_split(int qr) { return kOakSpan / qr; }

hipError_t launch_decode_oaken(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st) {
  if (c.k.group != c.v.group) return hipErrorInvalidValue;
  if (d.split_len > kOakSpan / d.qr) return hipErrorInvalidValue;
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
