// Forward, diagnostic and tile-maximum kernels for 64 x 128 tiles
// (B_M = 64 query rows, B_N = 128 keys), both head dimensions.
#include "bsfa_fwd_kernels.h"

namespace bsfa {

int launch_fwd_64x128(const FwdParams& p, int head_dim, int causal, int mode, hipStream_t stream) {
  return launch_tile<64, 128>(p, head_dim, causal, mode, stream);
}

}  // namespace bsfa
