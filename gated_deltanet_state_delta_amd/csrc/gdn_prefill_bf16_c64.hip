// gdn_prefill_bf16_c64.hip -- prefill kernel instantiations: bf16 operands, chunk 64.
#include "gdn_prefill.hpp"

namespace gdn {
hipError_t prefill_bf16_c64(PrefillParams p, int dk, int dv, hipStream_t s) {
  return dispatch_prefill_dk_dv<__bf16, 64>(p, dk, dv, s);
}
}  // namespace gdn
