// Dispatch of the forward kernels by tile shape.  The kernels themselves are
// in bsfa_fwd_kernels.h, instantiated once per tile shape in
// bsfa_fwd_<bm>x<bn>.hip so that the shapes compile in parallel.
#include "bsfa_internal.h"

namespace bsfa {

int launch_fwd(const FwdParams& p, int head_dim, int bm, int bn, int causal, int mode, hipStream_t stream) {
  if (bm == 128 && bn == 128) return launch_fwd_128x128(p, head_dim, causal, mode, stream);
  if (bm == 128 && bn == 64) return launch_fwd_128x64(p, head_dim, causal, mode, stream);
  if (bm == 64 && bn == 128) return launch_fwd_64x128(p, head_dim, causal, mode, stream);
  if (bm == 64 && bn == 64) return launch_fwd_64x64(p, head_dim, causal, mode, stream);
  return 3;
}

}  // namespace bsfa
