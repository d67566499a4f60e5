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

// Move pp[lo, hi) up by d slots (d >= 0), from the top down so that nothing
// is overwritten before it is read.  Every thread of the workgroup calls it.
__device__ __forceinline__ void shift_up(int* pp, int lo, int hi, int d) {
  for (int e = hi; e > lo; e -= 256) {
    const int s0 = max(lo, e - 256), idx = s0 + (int)threadIdx.x;
    const int v = idx < e ? pp[idx] : 0;
    __syncthreads();
    if (idx < e && d) pp[idx + d] = v;
    __syncthreads();
  }
}

// perm / seg after a streaming append: the m chunks completed in sequence b
// (original ids n .. n + m - 1, bit-widths bits[b][0 .. m)) join the end of
// their class, so the INT4 and INT2 slot ranges move up by the new chunks of
// the classes before them.  The result is the stable class partition of all
// complete chunks, as k_reorder builds it.  One workgroup per sequence.
__global__ __launch_bounds__(256) void k_chunk_seg(const uint8_t* __restrict__ bits, int n_new, int t_new,
                                                   int S, int CT, int C, const int* __restrict__ pos,
                                                   int* __restrict__ perm, int* __restrict__ seg,
                                                   unsigned* __restrict__ status) {
  const int b = blockIdx.x;
  const int p = pos[b];
  const int n16 = seg[b * 4], n4 = seg[b * 4 + 1], n2 = seg[b * 4 + 2], n = seg[b * 4 + 3];
  __syncthreads();  // every thread has read seg before it changes
  if (p < 0 || p + t_new > S || p / CT != n) return;  // flagged by the append kernels
  const int m = (p + t_new) / CT - n;
  if (m <= 0) return;
  const uint8_t* bb = bits + (long long)b * n_new;
  int a[3] = {0, 0, 0};
  bool bad = false;
  for (int i = 0; i < m; ++i) {
    const int v = bb[i];
    bad |= v != 16 && v != 4 && v != 2;
    ++a[chunk_class(v)];
  }
  int* pp = perm + (long long)b * C;
  shift_up(pp, n16 + n4, n, a[0] + a[1]);
  shift_up(pp, n16, n16 + n4, a[0]);
  if (threadIdx.x == 0) {
    int w[3] = {n16 + 0, n16 + a[0] + n4, n16 + a[0] + n4 + a[1] + n2};
    for (int i = 0; i < m; ++i) pp[w[chunk_class(bb[i])]++] = n + i;
    seg[b * 4 + 0] = n16 + a[0];
    seg[b * 4 + 1] = n4 + a[1];
    seg[b * 4 + 2] = n2 + a[2];
    seg[b * 4 + 3] = n + m;
    if (bad) set_flag(status, kFlagBadChunkBits);
  }
}

}  // namespace

hipError_t launch_append_chunks(const CacheArgs& c, const uint16_t* xk, const uint16_t* xv, int t_new,
                                const int* pos, const uint8_t* bits, int n_new, hipStream_t st) {
  hipError_t e = launch_chunk_append(c, c.k, false, xk, t_new, pos, bits, n_new, st);
  if (e == hipSuccess) e = launch_chunk_append(c, c.v, true, xv, t_new, pos, bits, n_new, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_chunk_seg, dim3((unsigned)c.B), dim3(256), 0, st, bits, n_new, t_new, c.S,
                     c.chunk_tokens, c.S / c.chunk_tokens, pos, c.perm, c.seg, c.status);
  return hipGetLastError();
}

hipError_t launch_reorder(const CacheArgs& c, const uint8_t* bits, int n_chunks, hipStream_t st) {
  hipLaunchKernelGGL(k_reorder, dim3((unsigned)c.B), dim3(256), 0, st, bits, n_chunks, c.perm, c.seg,
                     c.status);
  return hipGetLastError();
}

}  // namespace kvq
