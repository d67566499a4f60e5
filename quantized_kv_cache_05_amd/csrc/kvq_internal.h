// Host-side interface between the C-ABI layer (kvq_api.cpp) and the kernel
// launchers (kvq_quant.hip, kvq_reorder.hip, kvq_decode*.hip).  Plain structs:
// pointers already offset and validated by the API layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kD = 128;          // head_dim
constexpr int kPartStride = 132; // floats per split partial: m, l, 2 pad, o[128]
constexpr int kMaxQR = 16;       // query heads one decode workgroup serves

// Device view of one quantized tensor (K or V).
struct TensorArgs {
  int bits;       // 8, 4, 2 (UNIFORM), 4 (OAKEN)
  int sym;        // symmetric INT8
  int fmt;        // 0 integer codes, 1 FP8 E4M3 (bits 8, scale only)
  int axis;       // 0 token, 1 channel
  int group;      // channels (token axis) or tokens (channel axis)
  float thr_lo, thr_hi;  // OAKEN outer thresholds
  long long sparse_cap;
  uint8_t* codes;
  float* scale;
  uint8_t* zero;
  float* oscale;
  uint32_t* rowptr;
  uint16_t* sparse;
  uint8_t* codes16;
  uint8_t* codes2;
  float* scale2;
  uint8_t* zero2;
};

struct CacheArgs {
  int B, H, S;  // batch, kv heads, max_seq
  int mode;     // 0 uniform, 1 chunk mixed, 2 oaken
  int chunk_tokens;
  TensorArgs k, v;
  int* perm;
  int* seg;
  unsigned* status;
  const int* pages;  // paged: block table [B][S / ptok]; null when contiguous
  int ptok;          // tokens per page
  int npages;        // pages per pool
  int dsq_sig;                 // DSQ: significant tokens per 64-token group
  unsigned long long* dsq_mask;  // DSQ: [B][H][S / 64] significance masks
};

struct DecodeLaunch {
  const uint16_t* q;
  int Hq;        // query heads
  int G;         // query heads per KV head
  int qr;        // query heads per workgroup: 1, 4 or 16
  int qtiles;    // ceil(G / qr)
  const int* seq_len;
  int max_len;
  int num_splits;
  int split_len; // tokens (UNIFORM/OAKEN) or chunk slots (CHUNK_MIXED) per split
  float qscale;  // sm_scale * log2(e)
  float* out;
  float* ws;     // split partials, null when num_splits == 1
  float* oak_ksc;  // OAKEN: K outer-value score shares [B][Hq][max_len] (null otherwise)
};

// vl: write the V row layout (else the K row layout), see kvq.h.
// K and V in one launch; both tensors token-axis with equal bits, sym and group.
hipError_t launch_quant_token_kv(const CacheArgs& c, const uint16_t* xk, const uint16_t* xv, int t_new,
                                 const int* pos, hipStream_t st);
// Oaken append of one token per sequence, K and V in one launch (equal groups).
hipError_t launch_quant_oaken_one(const CacheArgs& c, const uint16_t* xk, const uint16_t* xv,
                                 const int* pos, hipStream_t st);
hipError_t launch_quant_token(const CacheArgs& c, const TensorArgs& t, bool vl, const uint16_t* x,
                              int t_new, const int* pos, hipStream_t st);
hipError_t launch_quant_channel(const CacheArgs& c, const TensorArgs& t, const uint16_t* x, int t_new,
                                const int* pos, hipStream_t st);
hipError_t launch_quant_mixed(const CacheArgs& c, const TensorArgs& t, bool vl, const uint16_t* x,
                              const int* pos, hipStream_t st);
hipError_t launch_quant_oaken(const CacheArgs& c, const TensorArgs& t, bool vl, const uint16_t* x,
                              int t_new, const int* pos, hipStream_t st);
hipError_t launch_reorder(const CacheArgs& c, const uint8_t* bits, int n_chunks, hipStream_t st);
// Cocktail streaming append of one tensor: complete chunks into their class
// pools, the rest into the FP16 pool's last chunk (perm / seg untouched).
hipError_t launch_chunk_append(const CacheArgs& c, const TensorArgs& t, bool vl, const uint16_t* x,
                               int t_new, const int* pos, const uint8_t* bits, int n_new, hipStream_t st);
// perm / seg after a streaming append (runs after launch_chunk_append of K and V).
hipError_t launch_chunk_seg(const CacheArgs& c, int t_new, const int* pos, const uint8_t* bits, int n_new,
                            hipStream_t st);
// Cocktail streaming append: complete chunks into their class pools, the
// rest into the FP16 pool's last chunk, then perm / seg.
hipError_t launch_append_chunks(const CacheArgs& c, const uint16_t* xk, const uint16_t* xv, int t_new,
                                const int* pos, const uint8_t* bits, int n_new, hipStream_t st);

// KVO-LLM DSQ: whole 64-token groups, K and V in one launch.
hipError_t launch_quant_dsq(const CacheArgs& c, const uint16_t* xk, const uint16_t* xv, const float* score,
                            int t_new, const int* pos, hipStream_t st);

// Cocktail chunk precision search and Oaken calibration histogram.
constexpr int kMaxPercentiles = 8;
struct PercentileList {
  int count;
  int p_bp[kMaxPercentiles];  // basis points, 0..10000
};
hipError_t launch_chunk_bits(const double* q_emb, const double* c_emb, int batch, int n, int dim,
                             double alpha, double beta, double* sims, uint8_t* bits, hipStream_t st);
hipError_t launch_hist_f16(const uint16_t* x, long long n, unsigned long long* hist, hipStream_t st);
hipError_t launch_percentiles(const unsigned long long* hist, const PercentileList& pl, float* out,
                              hipStream_t st);

// Returns hipErrorInvalidValue for a combination without a compiled kernel.
hipError_t launch_decode_uniform(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st);
hipError_t launch_decode_oaken(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st);
hipError_t launch_decode_mixed(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st);
hipError_t launch_decode_dsq(const CacheArgs& c, const DecodeLaunch& d, hipStream_t st);
// log-sum-exp merge of the split partials into the output
hipError_t launch_merge(const DecodeLaunch& d, int B, hipStream_t st);

// True when a uniform (K, V) pair has a compiled decode kernel.
bool decode_uniform_supported(const TensorArgs& k, const TensorArgs& v);

struct AttnParams;
AttnParams make_attn_params(const CacheArgs& c, const DecodeLaunch& d);

}  // namespace kvq
