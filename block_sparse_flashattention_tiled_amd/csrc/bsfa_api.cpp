// C ABI of the block-sparse FlashAttention prefill library (declared in
// include/bsfa.h).  Host code only: argument checks, parameter packing and
// dispatch to the HIP kernels.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bsfa.h"
#include "bsfa_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_shape(const bsfa_shape& s, int causal, const bsfa_block& blk) {
  if (s.batch < 1 || s.n_heads_q < 1 || s.n_heads_kv < 1 || s.seq_len < 1 || s.head_dim < 1 || s.thr_len < 1)
    return BSFA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return BSFA_ERR_SHAPE;
  if (s.n_heads_q % s.n_heads_kv) return BSFA_ERR_SHAPE;
  if (blk.bm < 1 || blk.bn < 1) return BSFA_ERR_SHAPE;
  if ((blk.bm != 64 && blk.bm != 128) || (blk.bn != 64 && blk.bn != 128)) return BSFA_ERR_UNSUPPORTED;
  if (s.head_dim != 64 && s.head_dim != 128) return BSFA_ERR_UNSUPPORTED;
  // the kernels index heads, rows and thresholds with 32-bit integers
  const int64_t lim = INT32_MAX;
  const int64_t m = (s.seq_len + blk.bm - 1) / blk.bm;  // query blocks; the last may be partial
  if (s.seq_len > lim / 2 || s.batch > lim || s.n_heads_q > lim) return BSFA_ERR_SHAPE;
  if (s.batch * s.n_heads_q > lim / m) return BSFA_ERR_SHAPE;    // workgroups
  if (s.n_heads_q > lim / s.thr_len) return BSFA_ERR_SHAPE;      // threshold index
  if (s.batch * s.n_heads_q > lim / s.seq_len) return BSFA_ERR_SHAPE;  // (b, h) row base
  // one head's K or V is read as a buffer of N d 2 bytes with 32-bit signed
  // byte offsets (the tile's first row times the row pitch, plus the lane's
  // chunk): longer heads have no kernel
  if (s.seq_len * s.head_dim * 2 > lim) return BSFA_ERR_UNSUPPORTED;
  return BSFA_OK;
}

bsfa::FwdParams shape_params(const bsfa_shape& shape, const bsfa_block& block) {
  bsfa::FwdParams p{};
  p.B = (int)shape.batch;
  p.Hq = (int)shape.n_heads_q;
  p.Hkv = (int)shape.n_heads_kv;
  p.G = p.Hq / p.Hkv;
  p.N = (int)shape.seq_len;
  p.M = (int)((shape.seq_len + block.bm - 1) / block.bm);
  p.Mkv = (int)((shape.seq_len + block.bn - 1) / block.bn);
  p.T_len = (int)shape.thr_len;
  p.scale = (float)(1.0 / sqrt((double)shape.head_dim));
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)shape.head_dim));
  return p;
}

// out is fp32 unless out_bf16 is set (then out is null)
int prefill_impl(const void* q, const void* k, const void* v, float* out, uint16_t* out_bf16, float* lse,
                 int32_t* skip_counts, const float* thresholds, bsfa_shape shape, int causal, bsfa_block block,
                 int gate, uint8_t* tile_state, float* tile_max, int diagnostics, void* stream,
                 const int32_t* seq_lens = nullptr) {
  const int st = check_shape(shape, causal, block);
  if (st != BSFA_OK) return st;
  if (gate != BSFA_GATE_THRESHOLD && gate != BSFA_GATE_GAP) return BSFA_ERR_SHAPE;
  if (!q || !k || !v || !(out || out_bf16) || !thresholds) return BSFA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out ? (const void*)out : out_bf16, 16))
    return BSFA_ERR_ALIGN;
  if (!aligned(thresholds, 4) || (lse && !aligned(lse, 4)) || (skip_counts && !aligned(skip_counts, 4)) ||
      (tile_max && !aligned(tile_max, 4)) || (seq_lens && !aligned(seq_lens, 4)))
    return BSFA_ERR_ALIGN;

  bsfa::FwdParams p = shape_params(shape, block);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = out;
  p.out_bf16 = out_bf16;
  p.gate = gate;
  p.lse = lse;
  p.skip_counts = skip_counts;
  p.thresholds = thresholds;
  p.tile_state = tile_state;
  p.tile_max = tile_max;
  p.seq_lens = seq_lens;
  return bsfa::launch_fwd(p, (int)shape.head_dim, block.bm, block.bn, causal, diagnostics,
                          static_cast<hipStream_t>(stream));
}

// One launch per level; ks clamped to the number of key blocks (k >= n_i
// means "keep all" for every query block alike).
int calibrate_impl(const float* tile_max, int64_t n_samples, int64_t n_heads, int64_t mq, int64_t mkv,
                          int bm, int bn, int causal, const int64_t* ks, int64_t n_levels, float* thresholds,
                          void* stream) {
  if (n_samples < 1 || n_heads < 1 || mq < 1 || mkv < 1 || n_levels < 1 || (causal != 0 && causal != 1))
    return BSFA_ERR_SHAPE;
  if (!ks || !tile_max || !thresholds) return BSFA_ERR_NULL;
  for (int64_t l = 0; l < n_levels; ++l)
    if (ks[l] < 0) return BSFA_ERR_SHAPE;
  if (mkv > bsfa::kCalibMaxBlocks) return BSFA_ERR_UNSUPPORTED;
  if (n_heads > INT32_MAX / mq || n_samples > INT32_MAX || n_levels > INT32_MAX / (n_heads * mq))
    return BSFA_ERR_SHAPE;
  if (!aligned(tile_max, 4) || !aligned(thresholds, 4)) return BSFA_ERR_ALIGN;
  const int64_t level_size = n_heads * mq;
  for (int64_t l = 0; l < n_levels; ++l) {
    const int kk = (int)(ks[l] < mkv ? ks[l] : mkv);
    const int st = bsfa::launch_calibrate(tile_max, (int)n_samples, (int)n_heads, (int)mq, (int)mkv, bm, bn, causal,
                                          kk, thresholds + l * level_size, static_cast<hipStream_t>(stream));
    if (st != BSFA_OK) return st;
  }
  return BSFA_OK;
}

}  // namespace

extern "C" {

int bsfa_validate(bsfa_shape shape, int causal, bsfa_block block) { return check_shape(shape, causal, block); }

const char* bsfa_status_string(int status) {
  switch (status) {
    case BSFA_OK: return "ok";
    case BSFA_ERR_NULL: return "a required pointer is NULL";
    case BSFA_ERR_SHAPE: return "inconsistent or out-of-range shape";
    case BSFA_ERR_UNSUPPORTED: return "unsupported head_dim / tile combination";
    case BSFA_ERR_ALIGN: return "misaligned pointer";
    case BSFA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int bsfa_prefill(const void* q, const void* k, const void* v, float* out, float* lse, int32_t* skip_counts,
                 const float* thresholds, bsfa_shape shape, int causal, bsfa_block block, void* stream) {
  return prefill_impl(q, k, v, out, nullptr, lse, skip_counts, thresholds, shape, causal, block,
                      BSFA_GATE_THRESHOLD, nullptr, nullptr, 0, stream);
}

int bsfa_prefill_ex(const void* q, const void* k, const void* v, float* out, float* lse, int32_t* skip_counts,
                    const float* thresholds, bsfa_shape shape, int causal, bsfa_block block, uint8_t* tile_state,
                    float* tile_max, void* stream) {
  return prefill_impl(q, k, v, out, nullptr, lse, skip_counts, thresholds, shape, causal, block,
                      BSFA_GATE_THRESHOLD, tile_state, tile_max, 1, stream);
}

int bsfa_prefill_bf16(const void* q, const void* k, const void* v, void* out, float* lse, int32_t* skip_counts,
                      const float* thresholds, bsfa_shape shape, int causal, bsfa_block block, void* stream) {
  return prefill_impl(q, k, v, nullptr, static_cast<uint16_t*>(out), lse, skip_counts, thresholds, shape, causal,
                      block, BSFA_GATE_THRESHOLD, nullptr, nullptr, 0, stream);
}

int bsfa_prefill_gated(const void* q, const void* k, const void* v, float* out, float* lse, int32_t* skip_counts,
                       const float* thresholds, bsfa_shape shape, int causal, bsfa_block block, int gate,
                       uint8_t* tile_state, float* tile_max, void* stream) {
  const int diagnostics = (tile_state || tile_max) ? 1 : 0;
  return prefill_impl(q, k, v, out, nullptr, lse, skip_counts, thresholds, shape, causal, block, gate, tile_state,
                      tile_max, diagnostics, stream);
}

int bsfa_prefill_varlen(const void* q, const void* k, const void* v, float* out, float* lse, int32_t* skip_counts,
                        const float* thresholds, bsfa_shape shape, int causal, bsfa_block block,
                        const int32_t* seq_lens, uint8_t* tile_state, float* tile_max, void* stream) {
  if (!seq_lens) return BSFA_ERR_NULL;
  const int diagnostics = (tile_state || tile_max) ? 1 : 0;
  return prefill_impl(q, k, v, out, nullptr, lse, skip_counts, thresholds, shape, causal, block,
                      BSFA_GATE_THRESHOLD, tile_state, tile_max, diagnostics, stream, seq_lens);
}

int bsfa_tile_max(const void* q, const void* k, float* tile_max, bsfa_shape shape, int causal, bsfa_block block,
                  void* stream) {
  const int st = check_shape(shape, causal, block);
  if (st != BSFA_OK) return st;
  if (!q || !k || !tile_max) return BSFA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(tile_max, 4)) return BSFA_ERR_ALIGN;
  bsfa::FwdParams p = shape_params(shape, block);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.tile_max = tile_max;
  return bsfa::launch_fwd(p, (int)shape.head_dim, block.bm, block.bn, causal, 2, static_cast<hipStream_t>(stream));
}

int bsfa_calibrate_fixed_k(const float* tile_max, int64_t n_samples, int64_t n_heads, int64_t n_blocks, int causal,
                           int64_t k, float* thresholds, void* stream) {
  if (k < 0) return BSFA_ERR_SHAPE;
  // square tiles: the diagonal of query block i is key block i, whatever the size
  return calibrate_impl(tile_max, n_samples, n_heads, n_blocks, n_blocks, 1, 1, causal, &k, 1, thresholds, stream);
}

int bsfa_calibrate_levels(const float* tile_max, int64_t n_samples, int64_t n_heads, int64_t n_blocks, int causal,
                          const int64_t* ks, int64_t n_levels, float* thresholds, void* stream) {
  return calibrate_impl(tile_max, n_samples, n_heads, n_blocks, n_blocks, 1, 1, causal, ks, n_levels, thresholds,
                        stream);
}

int bsfa_calibrate(const float* tile_max, bsfa_shape shape, int causal, bsfa_block block, const int64_t* ks,
                   int64_t n_levels, float* thresholds, void* stream) {
  const int st = check_shape(shape, causal, block);
  if (st != BSFA_OK) return st;
  const int64_t mq = (shape.seq_len + block.bm - 1) / block.bm;
  const int64_t mkv = (shape.seq_len + block.bn - 1) / block.bn;
  return calibrate_impl(tile_max, shape.batch, shape.n_heads_q, mq, mkv, block.bm, block.bn, causal, ks, n_levels,
                        thresholds, stream);
}

}  // extern "C"
