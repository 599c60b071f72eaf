// Forward, diagnostic and tile-maximum kernels for 128 x 64 tiles
// (B_M = 128 query rows, B_N = 64 keys), both head dimensions.
#include "bsfa_fwd_kernels.h"

namespace bsfa {

int launch_fwd_128x64(const FwdParams& p, int head_dim, int causal, int mode, hipStream_t stream) {
  return launch_tile<128, 64>(p, head_dim, causal, mode, stream);
}

}  // namespace bsfa
