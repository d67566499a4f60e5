// Input preparation that the method performs outside the decode loop:
//  - the chunk precision search of the Cocktail page (§3.1.1): cosine
//    similarity of a query embedding with every chunk embedding, thresholds
//    T_low = s_min + (s_max - s_min) * alpha and T_high = s_max - (s_max - s_min) * beta,
//    and the class of each chunk (16 above T_high, 4 above T_low, else 2);
//  - the offline calibration of the Oaken page (§3.1): the distribution of
//    sampled K / V values, summarised as a histogram of fp16 bit patterns,
//    and nearest-rank percentiles read from it.
// Both are computed exactly: the similarity of a chunk is one thread's
// sequential binary64 dot product (no contraction into fused multiply-adds),
// and the histogram and rank search are integer work.
#include "kvq_dev.h"

namespace kvq {
namespace {

// Binary64 arithmetic in program order, one rounding per operation (the
// kernel below forbids the compiler to fuse a product and a sum into one
// fused multiply-add, which HIP's default allows): each similarity is one
// thread's sequential sums over d, so rows cannot be split across lanes.
// The rows are read in slices of kSliceD values staged through LDS, loaded
// cooperatively so that a wave's load instruction covers 8 rows' 64-byte
// slices (not 64 rows' 8 bytes).  Each thread also forms the query's sum of
// squares in the same order, next to its chunk's two sums, so every thread
// has the same |q| without a separate pass.
constexpr int kChunkThreads = 1024;
constexpr int kSliceD = 8;
constexpr int kSimLds = 4096;  // similarities kept in LDS for the class pass (32 KiB)

// One workgroup of 1024 threads per sequence, 1024 chunks at a time, one
// chunk per thread.  Pass 1: similarities, their minimum and maximum; pass
// 2: classes, from LDS, from the output array, or recomputed bit-identically
// (beyond kSimLds chunks without an output array).
__global__ __launch_bounds__(kChunkThreads) void k_chunk_bits(const double* __restrict__ q_emb,
                                                              const double* __restrict__ c_emb, int n,
                                                              int dim, double alpha, double beta,
                                                              double* __restrict__ sims,
                                                              uint8_t* __restrict__ bits) {
#pragma clang fp contract(off)
  const int b = blockIdx.x;
  const double* qe = q_emb + (long long)b * dim;
  const double* ce = c_emb + (long long)b * n * dim;
  __shared__ double tile[kChunkThreads][kSliceD + 1];  // +1: conflict-free row reads
  __shared__ double sim_sh[kSimLds];
  __shared__ double wave_min[kChunkThreads / 64], wave_max[kChunkThreads / 64];
  const int t = threadIdx.x;
  // the similarities of chunks c0 .. c0 + 1023 (thread t: chunk c0 + t)
  // element j = t mod 8 of the slice at d0 of rows c0 + t / 8 + 128 m
  auto load_slice = [&](int c0, int d0, double (&v)[kSliceD]) {
#pragma unroll
    for (int m = 0; m < kSliceD; ++m) {
      const int c = c0 + (t >> 3) + 128 * m, d = d0 + (t & 7);
      v[m] = (c < n && d < dim) ? ce[(long long)c * dim + d] : 0.0;
    }
  };
  auto similarity_block = [&](int c0) -> double {
    double dot = 0.0, cc = 0.0, qq = 0.0;
    double nxt[kSliceD];
    load_slice(c0, 0, nxt);
    for (int d0 = 0; d0 < dim; d0 += kSliceD) {
      __syncthreads();  // the previous slice has been read
#pragma unroll
      for (int m = 0; m < kSliceD; ++m) tile[(t >> 3) + 128 * m][t & 7] = nxt[m];
      __syncthreads();
      if (d0 + kSliceD < dim) load_slice(c0, d0 + kSliceD, nxt);  // in flight during the sums
      const int dn = min(kSliceD, dim - d0);
      for (int j = 0; j < dn; ++j) {
        const double q = qe[d0 + j], c = tile[t][j];
        dot = dot + q * c;
        cc = cc + c * c;
        qq = qq + q * q;
      }
    }
    return dot / (sqrt(qq) * sqrt(cc));
  };
  double lo = INFINITY, hi = -INFINITY;
  for (int c0 = 0; c0 < n; c0 += kChunkThreads) {
    const double s = similarity_block(c0);
    const int i = c0 + t;
    if (i < n) {
      if (sims) sims[(long long)b * n + i] = s;
      if (i < kSimLds) sim_sh[i] = s;
      lo = fmin(lo, s);
      hi = fmax(hi, s);
    }
  }
  // minimum and maximum (exact in any order): across the wave, then the waves
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    lo = fmin(lo, __shfl_xor(lo, m, 64));
    hi = fmax(hi, __shfl_xor(hi, m, 64));
  }
  if ((t & 63) == 0) {
    wave_min[t >> 6] = lo;
    wave_max[t >> 6] = hi;
  }
  __syncthreads();
  double smin = wave_min[0], smax = wave_max[0];
#pragma unroll
  for (int w = 1; w < kChunkThreads / 64; ++w) {
    smin = fmin(smin, wave_min[w]);
    smax = fmax(smax, wave_max[w]);
  }
  const double range = smax - smin;
  const double t_low = smin + range * alpha;
  const double t_high = smax - range * beta;
  for (int c0 = 0; c0 < n; c0 += kChunkThreads) {
    const int i = c0 + t;
    double s = 0.0;
    if (c0 + kChunkThreads <= kSimLds) s = sim_sh[min(i, kSimLds - 1)];
    else if (sims) s = sims[(long long)b * n + min(i, n - 1)];
    else s = similarity_block(c0);  // every thread takes part (barriers inside)
    if (i < n) bits[(long long)b * n + i] = s > t_high ? 16 : (s > t_low ? 4 : 2);
  }
}

// Order-preserving key of an fp16 bit pattern: negative values below
// positive ones, -0 just below +0.
__device__ __forceinline__ unsigned f16_key(unsigned h) {
  return (h & 0x8000u) ? (0xFFFFu - h) : (h | 0x8000u);
}

constexpr int kHistHalf = 32768;  // keys per pass: one LDS counter array of 128 KiB

// Histogram of the keys in [key0, key0 + 32768) over x[0, n): per-workgroup
// 32-bit LDS counters, added to the 64-bit global bins at the end.
// A workgroup counts at most 2^31 elements (guaranteed by the launcher).
__global__ __launch_bounds__(1024) void k_hist_f16(const uint16_t* __restrict__ x, long long n,
                                                   long long per_group, unsigned key0,
                                                   unsigned long long* __restrict__ hist) {
  extern __shared__ unsigned cnt[];
  for (int i = threadIdx.x; i < kHistHalf; i += 1024) cnt[i] = 0u;
  __syncthreads();
  const long long a = (long long)blockIdx.x * per_group;
  const long long e = a + per_group < n ? a + per_group : n;
  // 8 fp16 values per 16-byte load where the slice allows it
  const long long a8 = (a + 7) & ~7ll, e8 = e & ~7ll;
  if (a8 < e8) {
    for (long long i = a8 + 8ll * threadIdx.x; i < e8; i += 8ll * 1024) {
      const uint4 w = *reinterpret_cast<const uint4*>(x + i);
      const unsigned v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const unsigned k0 = f16_key(v[k] & 0xFFFFu) - key0, k1 = f16_key(v[k] >> 16) - key0;
        if (k0 < (unsigned)kHistHalf) atomicAdd(&cnt[k0], 1u);
        if (k1 < (unsigned)kHistHalf) atomicAdd(&cnt[k1], 1u);
      }
    }
  }
  const long long head_end = a8 < e ? a8 : e;
  for (long long i = a + threadIdx.x; i < head_end; i += 1024) {
    const unsigned k = f16_key(x[i]) - key0;
    if (k < (unsigned)kHistHalf) atomicAdd(&cnt[k], 1u);
  }
  for (long long i = (e8 > a8 ? e8 : head_end) + threadIdx.x; i < e; i += 1024) {
    const unsigned k = f16_key(x[i]) - key0;
    if (k < (unsigned)kHistHalf) atomicAdd(&cnt[k], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kHistHalf; i += 1024)
    if (cnt[i]) atomicAdd(&hist[key0 + i], (unsigned long long)cnt[i]);
}

// Nearest-rank percentiles: for p (basis points), the value of the element
// of rank ceil(p * N / 10000) (at least 1) in ascending order.  One
// workgroup of 1024 threads; each thread owns 64 consecutive bins.
__global__ __launch_bounds__(1024) void k_percentiles(const unsigned long long* __restrict__ hist,
                                                      PercentileList pl, float* __restrict__ out) {
  __shared__ unsigned long long part[1024];
  const int t = threadIdx.x;
  unsigned long long mine = 0;
  for (int k = 0; k < 64; ++k) mine += hist[t * 64 + k];
  part[t] = mine;
  __syncthreads();
  // inclusive scan (Hillis-Steele)
  for (int off = 1; off < 1024; off <<= 1) {
    const unsigned long long add = t >= off ? part[t - off] : 0ull;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  const unsigned long long total = part[1023];
  const unsigned long long before = t ? part[t - 1] : 0ull;
  for (int j = 0; j < pl.count; ++j) {
    unsigned long long rank = (total * (unsigned long long)pl.p_bp[j] + 9999ull) / 10000ull;
    if (rank < 1) rank = 1;
    if (total == 0) {
      if (t == 0) out[j] = __builtin_nanf("");
      continue;
    }
    if (before < rank && rank <= part[t]) {
      unsigned long long acc = before;
      for (int k = 0; k < 64; ++k) {
        acc += hist[t * 64 + k];
        if (acc >= rank) {
          const unsigned key = (unsigned)(t * 64 + k);
          const unsigned h = key >= 0x8000u ? (key & 0x7FFFu) : (0xFFFFu - key);
          out[j] = h2f((uint16_t)h);
          break;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_bits(const double* q_emb, const double* c_emb, int batch, int n, int dim,
                             double alpha, double beta, double* sims, uint8_t* bits, hipStream_t st) {
  hipLaunchKernelGGL(k_chunk_bits, dim3((unsigned)batch), dim3(kChunkThreads), 0, st, q_emb, c_emb, n, dim,
                     alpha, beta, sims, bits);
  return hipGetLastError();
}

hipError_t launch_hist_f16(const uint16_t* x, long long n, unsigned long long* hist, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  // about 4 workgroups per compute unit, each a contiguous slice of >= 64 Ki values
  long long groups = 1024;
  long long per = (n + groups - 1) / groups;
  if (per < 65536) per = 65536;
  per = (per + 7) & ~7ll;
  groups = (n + per - 1) / per;
  const size_t lds = kHistHalf * sizeof(unsigned);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_hist_f16),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  for (unsigned key0 = 0; key0 < 65536u; key0 += kHistHalf) {
    hipLaunchKernelGGL(k_hist_f16, dim3((unsigned)groups), dim3(1024), lds, st, x, n, per, key0, hist);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_percentiles(const unsigned long long* hist, const PercentileList& pl, float* out,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_percentiles, dim3(1), dim3(1024), 0, st, hist, pl, out);
  return hipGetLastError();
}

}  // namespace kvq
