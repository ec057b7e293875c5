// gdn_decode_dv128.hip -- the decode kernel (gdn_decode.hpp) for value
// width 128, in a translation unit of its own so that it can take its own
// machine-scheduler flag (the build script has the measurement).
#include "gdn_decode.hpp"

namespace gdn {

template <typename IO>
static hipError_t dv128_dk(const DecodeParams& p, int dk, hipStream_t s) {
  switch (dk) {
    case 16: return launch_decode_t<IO, 16, 128>(p, s);
    case 32: return launch_decode_t<IO, 32, 128>(p, s);
    case 64: return launch_decode_t<IO, 64, 128>(p, s);
    case 128: return launch_decode_t<IO, 128, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_dv128(const DecodeParams& p, int dk, bool bf16, hipStream_t stream) {
  return bf16 ? dv128_dk<__bf16>(p, dk, stream) : dv128_dk<float>(p, dk, stream);
}

}  // namespace gdn
