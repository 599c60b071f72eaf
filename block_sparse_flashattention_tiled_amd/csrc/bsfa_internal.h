// Internal interface between the C ABI (bsfa_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsfa {

// Arguments of one forward launch; pointers are device pointers.
struct FwdParams {
  const uint16_t* q;  // bf16 [B, Hq, N, d]
  const uint16_t* k;  // bf16 [B, Hkv, N, d]
  const uint16_t* v;  // bf16 [B, Hkv, N, d]
  float* out;         // fp32 [B, Hq, N, d] (unless out_bf16 is set)
  uint16_t* out_bf16; // bf16 [B, Hq, N, d] or null: the output in bf16 instead of fp32
  float* lse;         // fp32 [B, Hq, N] or null
  int32_t* skip_counts;     // int32 [B, Hq, M] or null
  const float* thresholds;  // fp32 [Hq, T_len]
  uint8_t* tile_state;      // uint8 [B, Hq, M, Mkv] or null (diagnostic launches only)
  float* tile_max;          // fp32 [B, Hq, M, Mkv] or null (diagnostic launches only)
  const int32_t* seq_lens;  // int32 [B] or null: per-sequence lengths (each clamped to [0, N])
  int B, Hq, Hkv, G, N, T_len;
  int M;    // query blocks, ceil(N / B_M)
  int Mkv;  // key blocks, ceil(N / B_N)
  float scale;       // 1 / sqrt(d)
  float scale_log2;  // scale * log2(e)
  int remap;         // 1: XCD-aware workgroup order applies (set per paired launch)
  int gate;          // 0: threshold gate (s_max < tau); 1: gap gate (s_max < running max - tau)
  int pair_h0;       // paired launches: first query head, inside its KV group, that the launch covers
  int pair_hn;       // paired launches: query heads per KV group that the launch covers
  unsigned long long* work;  // pipelined (persistent) launches: 8 work-queue counters, zeroed before the launch
  int n_items;       // pipelined (persistent) launches: work items (the static grid's workgroups)
};

// Enqueue the forward kernel for B_M x B_N tiles (bm, bn in {64, 128});
// mode 0 = forward, 1 = forward with per-tile diagnostics, 2 = tile maxima
// only.  Returns a BSFA_* status.
int launch_fwd(const FwdParams& p, int head_dim, int bm, int bn, int causal, int mode, hipStream_t stream);

// One translation unit per tile shape (bsfa_fwd_<bm>x<bn>.hip).
int launch_fwd_128x128(const FwdParams& p, int head_dim, int causal, int mode, hipStream_t stream);
int launch_fwd_128x64(const FwdParams& p, int head_dim, int causal, int mode, hipStream_t stream);
int launch_fwd_64x128(const FwdParams& p, int head_dim, int causal, int mode, hipStream_t stream);
int launch_fwd_64x64(const FwdParams& p, int head_dim, int causal, int mode, hipStream_t stream);

// Persistent launches of the pipelined kernel: returns the next slot of 8
// work-queue counters in the library's ring for the current device, enqueued
// to be zeroed on `stream`, and the device's compute-unit count in *n_cu; null
// if the ring's device address or the unit count cannot be had.
unsigned long long* pipe_work_slot(hipStream_t stream, int* n_cu);

// Enqueue the fixed-k calibration over tile maxima [S, H, Mq, Mkv] ->
// thresholds [H, Mq] for B_M x B_N tiles (bm = bn = 1 for square tiles of any
// size: the diagonal of query block i is then key block i).
int launch_calibrate(const float* tile_max, int S, int H, int Mq, int Mkv, int bm, int bn, int causal, int k,
                     float* thr, hipStream_t stream);

// Largest number of key blocks the calibration kernel handles (one row of
// tile maxima must fit in LDS).
constexpr int kCalibMaxBlocks = 16384;

}  // namespace bsfa
