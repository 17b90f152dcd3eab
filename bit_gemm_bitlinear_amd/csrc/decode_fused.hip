// The decode kernel's instances that fuse the activation quantization of 2
// to 4 token rows (decode_kernels.hpp), in a translation unit of their own so
// that the build compiles them alongside decode.hip.
#include "decode_kernels.hpp"

namespace bl {

hipError_t launch_decode_rows(const DecodeArgs& a, int total_wgs, size_t lds_bytes, hipStream_t s,
                              bool epi) {
  return epi ? launch_decode_as<true, 4>(a, total_wgs, lds_bytes, s)
             : launch_decode_as<false, 4>(a, total_wgs, lds_bytes, s);
}

}  // namespace bl
