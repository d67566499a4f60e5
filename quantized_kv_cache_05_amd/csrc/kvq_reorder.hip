// Chunk reorder ([Cocktail page] §3.1.2): chunks of one bit-width are made
// contiguous, in class order FP16, INT4, INT2, keeping their original order
// inside a class.  One workgroup per sequence; each class is a stable
// partition built from wave ballots and a four-wave prefix.
#include "kvq_dev.h"

namespace kvq {
namespace {

__device__ __forceinline__ int chunk_class(int v) { return v == 16 ? 0 : (v == 4 ? 1 : 2); }

__global__ __launch_bounds__(256) void k_reorder(const uint8_t* __restrict__ bits, int n,
                                                 int* __restrict__ perm, int* __restrict__ seg,
                                                 unsigned* __restrict__ status) {
  const int b = blockIdx.x;
  const uint8_t* bb = bits + (long long)b * n;
  int* pp = perm + (long long)b * n;
  __shared__ int wave_tot[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
  int base = 0;
  bool bad = false;
  int counts[3];
  for (int c = 0; c < 3; ++c) {
    int cnt = 0;
    for (int i0 = 0; i0 < n; i0 += 256) {
      const int i = i0 + threadIdx.x;
      const int v = i < n ? (int)bb[i] : 2;
      if (c == 0 && i < n && v != 16 && v != 4 && v != 2) bad = true;
      const bool f = i < n && chunk_class(v) == c;
      const unsigned long long bal = __ballot(f);
      if (lane == 0) wave_tot[w] = __popcll(bal);
      __syncthreads();
      int off = 0, tot = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < w) off += wave_tot[k];
        tot += wave_tot[k];
      }
      if (f) pp[base + cnt + off + __popcll(bal & below)] = i;
      cnt += tot;
      __syncthreads();
    }
    counts[c] = cnt;
    base += cnt;
  }
  if (threadIdx.x == 0) {
    seg[b * 4 + 0] = counts[0];
    seg[b * 4 + 1] = counts[1];
    seg[b * 4 + 2] = counts[2];
    seg[b * 4 + 3] = n;
  }
  if (bad) set_flag(status, kFlagBadChunkBits);
}

}  // namespace

hipError_t launch_reorder(const CacheArgs& c, const uint8_t* bits, int n_chunks, hipStream_t st) {
  hipLaunchKernelGGL(k_reorder, dim3((unsigned)c.B), dim3(256), 0, st, bits, n_chunks, c.perm, c.seg,
                     c.status);
  return hipGetLastError();
}

}  // namespace kvq
