// Kernel launchers for the sanitizer build of the host code: the driver only
// makes calls that argument validation refuses (or that have nothing to do),
// so reaching any launcher is an error and aborts.
#include <cstdio>
#include <cstdlib>

#include "kvq_internal.h"

namespace kvq {
namespace {
[[noreturn]] void reached(const char* what) {
  std::fprintf(stderr, "launcher reached in the validation build: %s\n", what);
  std::abort();
}
}  // namespace

hipError_t launch_quant_token_kv(const CacheArgs&, const uint16_t*, const uint16_t*, int, const int*, hipStream_t) {
  reached("quant_token_kv");
}
hipError_t launch_quant_oaken_one(const CacheArgs&, const uint16_t*, const uint16_t*, const int*, hipStream_t) {
  reached("quant_oaken_one");
}
hipError_t launch_quant_token(const CacheArgs&, const TensorArgs&, bool, const uint16_t*, int, const int*,
                              hipStream_t) {
  reached("quant_token");
}
hipError_t launch_quant_channel(const CacheArgs&, const TensorArgs&, const uint16_t*, int, const int*,
                                hipStream_t) {
  reached("quant_channel");
}
hipError_t launch_quant_mixed(const CacheArgs&, const TensorArgs&, bool, const uint16_t*, const int*,
                              hipStream_t) {
  reached("quant_mixed");
}
hipError_t launch_quant_oaken(const CacheArgs&, const TensorArgs&, bool, const uint16_t*, int, const int*,
                              hipStream_t) {
  reached("quant_oaken");
}
hipError_t launch_reorder(const CacheArgs&, const uint8_t*, int, hipStream_t) { reached("reorder"); }
hipError_t launch_chunk_append(const CacheArgs&, const TensorArgs&, bool, const uint16_t*, int, const int*,
                               const uint8_t*, int, hipStream_t) {
  reached("chunk_append");
}
hipError_t launch_chunk_seg(const CacheArgs&, int, const int*, const uint8_t*, int, hipStream_t) {
  reached("chunk_seg");
}
hipError_t launch_append_chunks(const CacheArgs&, const uint16_t*, const uint16_t*, int, const int*,
                                const uint8_t*, int, hipStream_t) {
  reached("append_chunks");
}
hipError_t launch_quant_dsq(const CacheArgs&, const uint16_t*, const uint16_t*, const float*, int, const int*,
                            hipStream_t) {
  reached("quant_dsq");
}
hipError_t launch_chunk_bits(const double*, const double*, int, int, int, double, double, double*, uint8_t*,
                             hipStream_t) {
  reached("chunk_bits");
}
hipError_t launch_hist_f16(const uint16_t*, long long, unsigned long long*, hipStream_t) { reached("hist_f16"); }
hipError_t launch_percentiles(const unsigned long long*, const PercentileList&, float*, hipStream_t) {
  reached("percentiles");
}
hipError_t launch_decode_uniform(const CacheArgs&, const DecodeLaunch&, hipStream_t) { reached("decode_uniform"); }
hipError_t launch_decode_oaken(const CacheArgs&, const DecodeLaunch&, hipStream_t) { reached("decode_oaken"); }
hipError_t launch_decode_mixed(const CacheArgs&, const DecodeLaunch&, hipStream_t) { reached("decode_mixed"); }
hipError_t launch_decode_dsq(const CacheArgs&, const DecodeLaunch&, hipStream_t) { reached("decode_dsq"); }
hipError_t launch_merge(const DecodeLaunch&, int, hipStream_t) { reached("merge"); }
}  // namespace kvq
