// attn_ragged.hip -- launches of the paged attention kernel (attn_fwd_kernel.h)
// for page sizes that are not a multiple of 8.  The block-sparse and decode
// pages put no constraint on the page size; the prefill page lists 16, 32, 64
// and 128, so prefill never comes here.  An 8-token chunk may then span pages,
// and the kernel copies each K/V row from its own page.
#include "attn_fwd_kernel.h"

namespace pkb {

template <int D>
static hipError_t launch_r(const AttnParams& p, int waves, int mode, dim3 grid, hipStream_t st) {
  if (mode == kModeBsa) {
    if (waves == 1) return launch_one<D, 1, kModeBsa, true>(p, grid, st);
    if (waves == 2) return launch_one<D, 2, kModeBsa, true>(p, grid, st);
    if (waves == 4) return launch_one<D, 4, kModeBsa, true>(p, grid, st);
  } else if (mode == kModeDecode) {
    if (waves == 4) return launch_one<D, 4, kModeDecode, true>(p, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_ragged(const AttnParams& p, int D, int waves, int mode, dim3 grid,
                              hipStream_t stream) {
  if (!(p.page_size & 7)) return hipErrorInvalidValue;
  if (D == 128) return launch_r<128>(p, waves, mode, grid, stream);
  if (D == 256) return launch_r<256>(p, waves, mode, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkb
