// gdn_prefill_f32_c64.hip -- prefill kernel instantiations: f32 operands, chunk 64.
#include "gdn_prefill.hpp"

namespace gdn {
hipError_t prefill_f32_c64(PrefillParams p, int dk, int dv, hipStream_t s) {
  return dispatch_prefill_dk_dv<float, 64>(p, dk, dv, s);
}
}  // namespace gdn
