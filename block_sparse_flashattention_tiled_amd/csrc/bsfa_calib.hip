// Fixed-k threshold calibration on the GPU.
//
// "Block Sparse Flash Attention" (paperpeel.com/paper/2512.07011), Sec. 4.2
// and App. B.3: for each query block, the off-diagonal blocks are ordered by
// their maximum scores and the threshold is placed so that exactly the top k
// are retained; thresholds are averaged over calibration samples.
//
// Input: the tile maxima of every computed tile, [S, H, Mq, Mkv] (S samples,
// e.g. the batch axis of a tile-max pass).  Output: thresholds [H, Mq].
// Query block i of B_M x B_N tiles has the diagonal key blocks [d0, d1] (the
// ones overlapping its positions, Sec. 4.1); its off-diagonal computed tiles
// are the key blocks before d0 (causal) or every key block outside [d0, d1]
// (bidirectional).  With n_i of them: -inf if n_i <= k; +inf if k == 0;
// otherwise the midpoint of the k-th and (k+1)-th largest maxima, averaged
// over samples.
//
// One workgroup per (head, query block).  The order statistics are found by
// rank counting in LDS (rank = number of larger values, ties broken by
// position), which is exact and deterministic; O(n_i^2) comparisons per row.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bsfa_internal.h"

namespace bsfa {

constexpr int CALIB_THREADS = 256;

__global__ void __launch_bounds__(CALIB_THREADS)
    bsfa_calib_kernel(const float* __restrict__ tile_max, int S, int H, int Mq, int Mkv, int bm, int bn, int causal,
                      int k, float* __restrict__ thr) {
  extern __shared__ float vals[];
  __shared__ float sel[2];
  const int h = blockIdx.x / Mq;
  const int i = blockIdx.x % Mq;
  const int tid = threadIdx.x;
  const int d0 = (int)((int64_t)i * bm / bn);
  const int d1 = min((int)(((int64_t)(i + 1) * bm - 1) / bn), Mkv - 1);
  const int nd = d1 - d0 + 1;  // diagonal tiles
  const int n = causal ? d0 : Mkv - nd;
  if (n <= k) {
    if (tid == 0) thr[(size_t)h * Mq + i] = -INFINITY;
    return;
  }
  if (k == 0) {
    if (tid == 0) thr[(size_t)h * Mq + i] = INFINITY;
    return;
  }
  float acc = 0.f;
  for (int s = 0; s < S; ++s) {
    const float* row = tile_max + (((size_t)s * H + h) * Mq + i) * Mkv;
    for (int t = tid; t < n; t += CALIB_THREADS) vals[t] = row[t < d0 ? t : t + nd];
    __syncthreads();
    for (int t = tid; t < n; t += CALIB_THREADS) {
      const float x = vals[t];
      int rank = 0;
      for (int u = 0; u < n; ++u) {
        const float y = vals[u];
        rank += (y > x || (y == x && u < t)) ? 1 : 0;
      }
      if (rank == k - 1) sel[0] = x;
      if (rank == k) sel[1] = x;
    }
    __syncthreads();
    acc += 0.5f * (sel[0] + sel[1]);
    __syncthreads();
  }
  if (tid == 0) thr[(size_t)h * Mq + i] = acc / (float)S;
}

int launch_calibrate(const float* tile_max, int S, int H, int Mq, int Mkv, int bm, int bn, int causal, int k,
                     float* thr, hipStream_t stream) {
  const size_t lds = (size_t)Mkv * sizeof(float);
  hipLaunchKernelGGL(bsfa_calib_kernel, dim3((unsigned)((size_t)H * Mq)), dim3(CALIB_THREADS), lds, stream,
                     tile_max, S, H, Mq, Mkv, bm, bn, causal, k, thr);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // namespace bsfa
