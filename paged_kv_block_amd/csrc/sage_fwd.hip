// sage_fwd.hip -- prequantized (int8 Q/K, fp8 E4M3 V) block-sparse attention.
#include "device_common.h"
#include "pkb_internal.h"

namespace pkb {

hipError_t launch_sage(const SageParams& p, hipStream_t stream) {
  (void)p;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace pkb
