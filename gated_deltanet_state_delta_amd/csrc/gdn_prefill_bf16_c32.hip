// gdn_prefill_bf16_c32.hip -- prefill kernel instantiations: bf16 operands, chunk 32.
#include "gdn_prefill.hpp"

namespace gdn {
hipError_t prefill_bf16_c32(PrefillParams p, int dk, int dv, hipStream_t s) {
  return dispatch_prefill_dk_dv<__bf16, 32>(p, dk, dv, s);
}
}  // namespace gdn
