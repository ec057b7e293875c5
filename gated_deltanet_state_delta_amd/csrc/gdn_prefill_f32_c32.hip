// gdn_prefill_f32_c32.hip -- prefill kernel instantiations: f32 operands, chunk 32.
#include "gdn_prefill.hpp"

namespace gdn {
hipError_t prefill_f32_c32(PrefillParams p, int dk, int dv, hipStream_t s) {
  return dispatch_prefill_dk_dv<float, 32>(p, dk, dv, s);
}
}  // namespace gdn
