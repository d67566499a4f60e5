// Device helpers shared by the kvq kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

constexpr unsigned kFlagPosRange = 1u;
constexpr unsigned kFlagSparseFull = 2u;
constexpr unsigned kFlagLenRange = 4u;
constexpr unsigned kFlagBadChunkBits = 8u;
constexpr unsigned kFlagPageRange = 16u;

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// fp16 bit patterns packed two per 32-bit word -> floats.
__device__ __forceinline__ float lo_h2f(uint32_t w) { return h2f((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float hi_h2f(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int mask) { return __shfl_xor(v, mask, 64); }

// DPP lane exchange inside 16-lane rows (no LDS round trip): lane i reads
// lane i ^ 1 (quad_perm [1,0,3,2]), i ^ 2 (quad_perm [2,3,0,1]), 7 - i of its
// 8-lane half (row_half_mirror) or 15 - i of its row (row_mirror).  A
// reduction that applies them in this order pairs each lane with the mirror
// of the part it has already combined, so it covers lanes differing in bits
// 0-1, 0-2 or 0-3 like the xor exchanges 1, 2, 4, 8.  Callers keep every
// lane of a 16-lane row active (a read of an inactive lane gives 0).
// (The moved value has no "old" operand, so the compiler can fold the move
// into the instruction that consumes it, e.g. v_max_f32 with a DPP operand.)
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int M>
constexpr int dpp_step() { return M == 1 ? kDppXor1 : M == 2 ? kDppXor2 : M == 4 ? kDppHalfMirror : kDppMirror; }

// Sum / max over the lanes that differ only in bits [lo_bit, hi_bit) of the lane id.
template <int LO, int HI>
__device__ __forceinline__ float sum_lanes(float v) {
#pragma unroll
  for (int m = LO; m < HI; m <<= 1) v += shfl_xor_f(v, m);
  return v;
}
// max / min are exact in any order: within a 16-lane row (LO = 1, HI <= 16)
// through DPP, otherwise through lane permutes
template <int LO, int HI>
__device__ __forceinline__ float max_lanes(float v) {
  if constexpr (LO == 1 && HI <= 16) {
    if constexpr (HI > 1) v = fmaxf(v, dpp_row<dpp_step<1>()>(v));
    if constexpr (HI > 2) v = fmaxf(v, dpp_row<dpp_step<2>()>(v));
    if constexpr (HI > 4) v = fmaxf(v, dpp_row<dpp_step<4>()>(v));
    if constexpr (HI > 8) v = fmaxf(v, dpp_row<dpp_step<8>()>(v));
  } else {
#pragma unroll
    for (int m = LO; m < HI; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
  }
  return v;
}
template <int LO, int HI>
__device__ __forceinline__ float min_lanes(float v) {
  if constexpr (LO == 1 && HI <= 16) {
    if constexpr (HI > 1) v = fminf(v, dpp_row<dpp_step<1>()>(v));
    if constexpr (HI > 2) v = fminf(v, dpp_row<dpp_step<2>()>(v));
    if constexpr (HI > 4) v = fminf(v, dpp_row<dpp_step<4>()>(v));
    if constexpr (HI > 8) v = fminf(v, dpp_row<dpp_step<8>()>(v));
  } else {
#pragma unroll
    for (int m = LO; m < HI; m <<= 1) v = fminf(v, shfl_xor_f(v, m));
  }
  return v;
}

// Unpack the DPL codes a lane holds (little-endian, see kvq.h) into floats.
// BITS 8: one code per byte; 4: two per byte, low nibble first; 2: four per
// byte, lowest bits first.  Each byte is widened with a byte-select convert.
template <int BITS, int DPL>
__device__ __forceinline__ void codes_to_float(const uint32_t* w, float* c) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int k = 0; k < DPL / 4; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) c[4 * k + j] = (float)((w[k] >> (8 * j)) & 0xFFu);
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int k = 0; k < DPL / 8; ++k) {
      uint32_t ev = w[k] & 0x0F0F0F0Fu;
      uint32_t od = (w[k] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[8 * k + 2 * j] = (float)((ev >> (8 * j)) & 0xFFu);
        c[8 * k + 2 * j + 1] = (float)((od >> (8 * j)) & 0xFFu);
      }
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int k = 0; k < DPL / 16; ++k)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t m = (w[k] >> (2 * s)) & 0x03030303u;
#pragma unroll
        for (int j = 0; j < 4; ++j) c[16 * k + 4 * j + s] = (float)((m >> (8 * j)) & 0xFFu);
      }
  } else {  // 16: raw fp16
#pragma unroll
    for (int k = 0; k < DPL / 2; ++k) {
      c[2 * k] = lo_h2f(w[k]);
      c[2 * k + 1] = hi_h2f(w[k]);
    }
  }
}

// Load N 32-bit words from a 4*N-byte aligned address (16-byte vector loads
// where N allows).
template <int N>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t* w) {
  if constexpr (N == 1) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (N == 2) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      uint4 v = reinterpret_cast<const uint4*>(p)[k];
      w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
  }
}

__device__ __forceinline__ void set_flag(unsigned* status, unsigned f) { atomicOr(status, f); }

// Wave-local ordering of LDS traffic: the wave's earlier LDS writes are
// complete and visible to its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Streaming accesses: cache data and quantizer inputs are touched once per
// call, so loads and stores carry the non-temporal hint (they do not
// displace reusable lines); this measurably raises the achieved HBM
// bandwidth of the decode loop.
template <class T>
__device__ __forceinline__ T ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}
template <class T>
__device__ __forceinline__ void st_nt(void* p, T v) {
  __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
}

}  // namespace kvq
