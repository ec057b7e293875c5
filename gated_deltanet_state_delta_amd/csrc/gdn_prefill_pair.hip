// gdn_prefill_pair.hip -- instantiations of the bf16 pair-role prefill kernel.
#include "gdn_prefill_pair.hpp"

namespace gdn {

hipError_t prefill_pair_bf16(PrefillParams p, int dk, hipStream_t s) {
  switch (dk) {
    case 64: return launch_prefill_pair_t<64>(p, s);
    case 128: return launch_prefill_pair_t<128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
