// gdn_prefill_bf16_c16.hip -- prefill kernel instantiations: bf16 operands, chunk 16.
#include "gdn_prefill.hpp"

namespace gdn {
hipError_t prefill_bf16_c16(PrefillParams p, int dk, int dv, hipStream_t s) {
  return dispatch_prefill_dk_dv<__bf16, 16>(p, dk, dv, s);
}
}  // namespace gdn
