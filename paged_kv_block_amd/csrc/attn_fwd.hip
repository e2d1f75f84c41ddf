// attn_fwd.hip -- launches of the paged attention kernel (attn_fwd_kernel.h)
// for page sizes that are multiples of 8: block-sparse rows, packed prefill and
// split-KV multi-token decode.  Other page sizes go to attn_ragged.hip.
#include "attn_fwd_kernel.h"

namespace pkb {

template <int D>
static hipError_t launch_d(const AttnParams& p, int waves, int mode, dim3 grid, hipStream_t st) {
  if (mode == kModeBsa) {
    if (waves == 1) return launch_one<D, 1, kModeBsa, false>(p, grid, st);
    if (waves == 2) return launch_one<D, 2, kModeBsa, false>(p, grid, st);
    if (waves == 4) return launch_one<D, 4, kModeBsa, false>(p, grid, st);
  } else if (mode == kModePrefill) {
    if (waves == 4) return launch_one<D, 4, kModePrefill, false>(p, grid, st);
  } else if (mode == kModeDecode) {
    if (waves == 4) return launch_one<D, 4, kModeDecode, false>(p, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn(const AttnParams& p, int D, int waves, int mode, dim3 grid,
                       hipStream_t stream) {
  if (p.page_size & 7) return launch_attn_ragged(p, D, waves, mode, grid, stream);
  if (D == 128) return launch_d<128>(p, waves, mode, grid, stream);
  if (D == 256) return launch_d<256>(p, waves, mode, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkb
