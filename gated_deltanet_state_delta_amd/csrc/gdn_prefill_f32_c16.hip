// gdn_prefill_f32_c16.hip -- prefill kernel instantiations: f32 operands, chunk 16.
#include "gdn_prefill.hpp"

namespace gdn {
hipError_t prefill_f32_c16(PrefillParams p, int dk, int dv, hipStream_t s) {
  return dispatch_prefill_dk_dv<float, 16>(p, dk, dv, s);
}
}  // namespace gdn
