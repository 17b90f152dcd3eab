// The decode kernel's instances that fuse the activation quantization of 2
// to 4 token rows (decode_kernels.hpp; with the larger per-thread budget of
// the split shape when a row group needs it), in a translation unit of their
// own so that the build compiles them alongside decode.hip.
#include "decode_kernels.hpp"

namespace bl {

hipError_t launch_decode_rows(const DecodeArgs& a, int total_wgs, size_t lds_bytes, hipStream_t s,
                              bool epi, bool big) {
  if (big)
    return epi ? launch_decode_as<true, kFusedBigSlots>(a, total_wgs, lds_bytes, s)
               : launch_decode_as<false, kFusedBigSlots>(a, total_wgs, lds_bytes, s);
  return epi ? launch_decode_as<true, 4>(a, total_wgs, lds_bytes, s)
             : launch_decode_as<false, 4>(a, total_wgs, lds_bytes, s);
}

}  // namespace bl
