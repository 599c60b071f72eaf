/*
 * bsfa.h - C ABI of the block-sparse FlashAttention prefill library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the one defined in "Block Sparse Flash Attention"
 * (paperpeel.com/paper/2512.07011): FlashAttention-2 style tiled attention
 * (Sec. 2 "FlashAttention", App. B.2) in which every score tile is computed
 * exactly and its maximum scaled score is compared with a calibrated
 * threshold for its head and query block (Sec. 4, 4.1).  A tile below the
 * threshold is skipped: its V block is not loaded, the P.V product is not
 * performed and the running max / sum / output are not updated (Sec. 4.4).
 * Diagonal tiles always pass (Sec. 4.1).  Under causal masking, tiles with no
 * visible (query, key) pair are not computed at all (App. B.2).
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller (for instance
 *    torch tensors).  No call allocates device memory, and none keeps a
 *    reference after it returns.
 *  - The library's one piece of state is a ring of 1,024 slots of eight
 *    64-bit work-queue counters per device (64 KB of module data, loaded with the
 *    library).  Each launch of the pipelined kernel (128 x 128 tiles at
 *    d = 128; one or two per call) takes the next slot and zeroes it on the
 *    call's stream before the kernel, which then hands out its work items
 *    from that slot.  Calls are therefore reentrant, on any mix of streams and
 *    host threads, as long as at most 1,024 such launches are in flight at
 *    once on one device.
 *  - Every argument check runs on the host before anything is enqueued; on
 *    error the call returns a non-zero status and writes nothing.
 *  - Work is enqueued on ``stream`` (a hipStream_t; NULL = the default
 *    stream).  No call synchronises.  A launch failure reported by the HIP
 *    runtime is returned as BSFA_ERR_LAUNCH; faults during execution surface
 *    at the caller's next synchronisation, as for any HIP work.
 *  - No C++ exception crosses this interface.
 *  - Results are deterministic: every output element is reduced in a fixed
 *    order whichever workgroup computes it.  The only atomics hand out work
 *    items.
 */
#ifndef BSFA_H
#define BSFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem shape.  Query head h reads KV head h / (n_heads_q / n_heads_kv)
 * (contiguous groups; the pages do not fix the grouped-query mapping). */
typedef struct {
  int64_t batch;      /* B    >= 1 */
  int64_t n_heads_q;  /* H_q  >= 1 */
  int64_t n_heads_kv; /* H_kv >= 1, H_q % H_kv == 0 */
  int64_t seq_len;    /* N    >= 1.  M = ceil(N / bm) query blocks and
                         M_KV = ceil(N / bn) key blocks; when N is not a
                         multiple of a tile side the last block is partial
                         and positions >= N do not exist: they are
                         neither keys nor queries, take no part in any tile
                         maximum, and their output rows are not written.  (The
                         pages instead pad to a multiple of the tile by
                         repeating the last token, App. B.3; a caller who wants
                         that result pads before the call.)  One head's K or V
                         must fit in 2^31 - 1 bytes, N * d * 2 <= INT32_MAX
                         (N <= 8,388,607 at d = 128, N <= 16,777,215 at
                         d = 64): longer heads return BSFA_ERR_UNSUPPORTED;
                         N > INT32_MAX / 2 returns BSFA_ERR_SHAPE. */
  int64_t head_dim;   /* d in {64, 128} */
  int64_t thr_len;    /* T_len >= 1: thresholds per head.  Query block i uses
                         entry min(i, T_len - 1): blocks past the table reuse
                         its last entry (App. B.3). */
} bsfa_shape;

/* Tile shape B_M x B_N (App. B.2): bm query rows by bn keys, each 64 or 128
 * (square, or rectangular like the 128 x 64 tiles of the pages' A100 kernel,
 * Sec. 5.1).  The tile is also the skip granularity: one gate per query
 * block and key block.  The DIAGONAL tiles of query block i, which bypass the
 * gate (Sec. 4.1), are the key blocks whose positions overlap the query
 * block's: key block j with j*bn < (i+1)*bm and (j+1)*bn > i*bm (j = i for
 * square tiles).  Thresholds are per query block. */
typedef struct {
  int32_t bm;
  int32_t bn;
} bsfa_block;

enum {
  BSFA_OK = 0,
  BSFA_ERR_NULL = 1,        /* a required pointer is NULL */
  BSFA_ERR_SHAPE = 2,       /* inconsistent or out-of-range shape */
  BSFA_ERR_UNSUPPORTED = 3, /* valid shape this build has no kernel for */
  BSFA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  BSFA_ERR_LAUNCH = 5       /* the HIP runtime refused the launch */
};

/* Gates of bsfa_prefill_gated.  Both compare a tile's s_max (maximum scaled
 * score over its visible entries) in the scaled-score domain; diagonal tiles
 * always pass; NaN comparisons keep the tile. */
enum {
  BSFA_GATE_THRESHOLD = 0, /* the pages' gate (Sec. 4.1, 4.4): skip iff s_max < tau */
  BSFA_GATE_GAP = 1        /* skip iff s_max < M - tau, M = largest s_max of the tiles of
                              this (head, query block) kept so far, in key-block order:
                              the running-maximum comparison of BLASST and of
                              SpargeAttention's in-kernel P.V skip (Sec. 3 "Related Work") */
};

/* Tile states written by bsfa_prefill_ex. */
enum {
  BSFA_TILE_PRUNED = 0,   /* causal: no visible pair (after the diagonal), never computed */
  BSFA_TILE_KEPT = 1,     /* off-diagonal, s_max >= threshold (or threshold NaN) */
  BSFA_TILE_SKIPPED = 2,  /* off-diagonal, s_max < threshold: no V load, no P.V */
  BSFA_TILE_DIAGONAL = 3  /* diagonal tile: bypasses the gate */
};

/*
 * bsfa_prefill - block-sparse attention forward (prefill) for one layer.
 *
 *  q           bf16  [B, H_q,  N, d] contiguous, read only
 *  k           bf16  [B, H_kv, N, d] contiguous, read only
 *  v           bf16  [B, H_kv, N, d] contiguous, read only; rows of V in tiles
 *                    that every query block skips are never read
 *  out         fp32  [B, H_q,  N, d] fully overwritten:
 *                    O[q] = sum_{k in R(q)} softmax(S)[q,k] V[k] with
 *                    S = Q K^T / sqrt(d) (Sec. 2) and R(q) the visible keys
 *                    of the kept tiles of q's query block
 *  lse         fp32  [B, H_q, N] natural-log sum of exp(S) over R(q); NULL = not written
 *  skip_counts int32 [B, H_q, M] number of skipped tiles per query block;
 *                    NULL = not written
 *  thresholds  fp32  [H_q, T_len] in the scaled-score domain (the same units
 *                    as S).  A tile (i, j) off the diagonal is skipped iff
 *                    max_{visible (q,k) in tile} S[q,k] < thresholds[h, min(i, T_len-1)]
 *                    (strict, Sec. 4.4).  -inf keeps every tile (dense
 *                    attention); +inf keeps only the diagonal; NaN keeps all.
 *  shape, causal (0 or 1), block: see above.
 *  stream      hipStream_t or NULL.
 *
 * Returns BSFA_OK or an error status (see the enum); nothing is written on error.
 */
int bsfa_prefill(const void* q, const void* k, const void* v, float* out, float* lse, int32_t* skip_counts,
                 const float* thresholds, bsfa_shape shape, int causal, bsfa_block block, void* stream);

/*
 * bsfa_prefill_ex - bsfa_prefill plus per-tile diagnostics (each nullable):
 *  tile_state uint8 [B, H_q, M, M_KV]: BSFA_TILE_* of every tile
 *  tile_max   fp32  [B, H_q, M, M_KV]: the gate's s_max (maximum scaled score over
 *             the visible entries) of every computed tile, NaN where not computed.
 * Same contract as bsfa_prefill otherwise.  Slower: for testing and
 * calibration, not for production.
 */
int bsfa_prefill_ex(const void* q, const void* k, const void* v, float* out, float* lse, int32_t* skip_counts,
                    const float* thresholds, bsfa_shape shape, int causal, bsfa_block block,
                    uint8_t* tile_state, float* tile_max, void* stream);

/*
 * bsfa_prefill_bf16 - bsfa_prefill writing the output in bf16: out is
 * bf16 [B, H_q, N, d] (16-byte aligned), each element the fp32 result of
 * bsfa_prefill rounded to nearest even.  Lets the call replace an attention
 * whose output is consumed in bf16 ("drop-in replacement", Sec. 1) without a
 * separate conversion pass.  lse stays fp32.  Same contract otherwise.
 */
int bsfa_prefill_bf16(const void* q, const void* k, const void* v, void* out, float* lse, int32_t* skip_counts,
                      const float* thresholds, bsfa_shape shape, int causal, bsfa_block block, void* stream);

/*
 * bsfa_prefill_gated - bsfa_prefill with a choice of gate and optional
 * per-tile diagnostics.
 *  gate        BSFA_GATE_THRESHOLD: identical to bsfa_prefill.
 *              BSFA_GATE_GAP: thresholds[h, min(i, T_len-1)] is the gap tau;
 *              key blocks are visited in increasing order and off-diagonal
 *              tile j is skipped iff s_max(i, j) < M - tau, M the largest
 *              s_max of the tiles kept before it (-inf before the first),
 *              so the first visited tile is always kept.  tau = +inf keeps
 *              everything.
 *  tile_state, tile_max  as for bsfa_prefill_ex; both NULL = production launch.
 * Errors as for bsfa_prefill, plus BSFA_ERR_SHAPE for an unknown gate.
 */
int bsfa_prefill_gated(const void* q, const void* k, const void* v, float* out, float* lse, int32_t* skip_counts,
                       const float* thresholds, bsfa_shape shape, int causal, bsfa_block block, int gate,
                       uint8_t* tile_state, float* tile_max, void* stream);

/*
 * bsfa_prefill_varlen - a batch of sequences of different lengths, each
 * attended independently (the mixed-length workload of Sec. 5.2,
 * "Variable-length analysis").
 *  q, k, v, out, lse  laid out as for bsfa_prefill with N = shape.seq_len the
 *              longest (padded) length: sequence b occupies positions
 *              [0, seq_lens[b]) of its rows.
 *  seq_lens    int32 [B] DEVICE array, required: the length of each sequence;
 *              values are clamped to [0, N].
 *  Sequence b is computed exactly as bsfa_prefill would compute it alone at
 *  length seq_lens[b] (partial last block, positions past it do not exist),
 *  with the same threshold table.  Rows of out / lse past seq_lens[b], counts
 *  of query blocks past its last block, and the diagnostics of those blocks
 *  are not written; diagnostics of key blocks past its last block read as not
 *  computed (BSFA_TILE_PRUNED, NaN).
 *  tile_state, tile_max  optional diagnostics as for bsfa_prefill_ex.
 */
int bsfa_prefill_varlen(const void* q, const void* k, const void* v, float* out, float* lse, int32_t* skip_counts,
                        const float* thresholds, bsfa_shape shape, int causal, bsfa_block block,
                        const int32_t* seq_lens, uint8_t* tile_state, float* tile_max, void* stream);

/*
 * bsfa_tile_max - calibration pass: the tile maxima alone.
 *  q, k      as for bsfa_prefill
 *  tile_max  fp32 [B, H_q, M, M_KV]: max over the visible entries of each
 *            computed tile of the scaled scores S = Q K^T / sqrt(d), NaN where a
 *            tile is not computed (causal, no visible pair).  Bit-identical to
 *            the tile_max output
 *            of bsfa_prefill_ex on the same inputs.
 * This is the measurement the threshold calibration of Sec. 4.2 sorts: "the
 * off-diagonal blocks ordered by their maximum scores".  QK^T only: no V is
 * read, nothing else is written.  shape.thr_len is not used (must be >= 1).
 */
int bsfa_tile_max(const void* q, const void* k, float* tile_max, bsfa_shape shape, int causal, bsfa_block block,
                  void* stream);

/*
 * bsfa_calibrate_fixed_k - fixed-k threshold table from tile maxima of
 * SQUARE tiles (Sec. 4.2; App. B.3 "Threshold tensor"); bsfa_calibrate
 * covers every tile shape.
 *  tile_max    fp32 [S, H, M, M] device: tile maxima of S calibration samples
 *              (e.g. the batch of a bsfa_tile_max call), NaN-free on computed
 *              tiles
 *  thresholds  fp32 [H, M] device, written: for query block i with n_i
 *              off-diagonal computed tiles (causal: i; bidirectional: M - 1),
 *              -inf if n_i <= k, +inf if k == 0, otherwise the midpoint of the
 *              k-th and (k+1)-th largest off-diagonal maxima, averaged over the
 *              S samples.  With S = 1 and distinct maxima, bsfa_prefill with
 *              this table keeps exactly min(k, n_i) off-diagonal tiles of every
 *              query block.  Use with shape.thr_len = M.
 * Errors: BSFA_ERR_SHAPE (counts < 1, k < 0), BSFA_ERR_UNSUPPORTED (M > 16384).
 */
int bsfa_calibrate_fixed_k(const float* tile_max, int64_t n_samples, int64_t n_heads, int64_t n_blocks, int causal,
                           int64_t k, float* thresholds, void* stream);

/*
 * bsfa_calibrate_levels - the threshold tensor for several sparsity levels at
 * once (App. B.3 "Threshold tensor": one table per sparsity level, the level
 * chosen at inference time by selecting its slice).
 *  tile_max    as for bsfa_calibrate_fixed_k
 *  ks          HOST array of n_levels values of k (each >= 0)
 *  thresholds  fp32 [n_levels, H, M] device, written: slice l is exactly what
 *              bsfa_calibrate_fixed_k returns for k = ks[l].  Pass
 *              thresholds + l * H * M (with shape.thr_len = M) to bsfa_prefill
 *              to run at level l.
 * Square tiles, as bsfa_calibrate_fixed_k.
 * Errors: as bsfa_calibrate_fixed_k, BSFA_ERR_NULL for ks == NULL,
 * BSFA_ERR_SHAPE for n_levels < 1 or a negative k.
 */
int bsfa_calibrate_levels(const float* tile_max, int64_t n_samples, int64_t n_heads, int64_t n_blocks, int causal,
                          const int64_t* ks, int64_t n_levels, float* thresholds, void* stream);

/*
 * bsfa_calibrate - fixed-k threshold tensor for any tile shape and length
 * (Sec. 4.2; App. B.3 "Threshold tensor").
 *  tile_max    fp32 [B, H_q, M, M_KV] device: the output of bsfa_tile_max for
 *              the same shape, causal flag and block; its B batch elements are
 *              the calibration samples
 *  shape, causal, block  as given to that bsfa_tile_max call (M = ceil(N/bm),
 *              M_KV = ceil(N/bn))
 *  ks          HOST array of n_levels values of k (each >= 0): off-diagonal
 *              tiles kept per query block
 *  thresholds  fp32 [n_levels, H_q, M] device, written.  Query block i has
 *              n_i off-diagonal computed tiles: the key blocks that end
 *              before it starts (causal), or every key block outside its
 *              diagonal ones (bidirectional).  Entry (l, h, i) is -inf if
 *              n_i <= ks[l], +inf if ks[l] == 0, otherwise the midpoint of the
 *              k-th and (k+1)-th largest of those maxima, averaged over the B
 *              samples.  For square tiles and N a multiple of bm this equals
 *              bsfa_calibrate_levels.  Use slice l with shape.thr_len = M.
 * Errors: as bsfa_validate for shape / causal / block; BSFA_ERR_NULL,
 * BSFA_ERR_SHAPE (n_levels < 1, a negative k), BSFA_ERR_UNSUPPORTED
 * (M_KV > 16384), BSFA_ERR_ALIGN.
 */
int bsfa_calibrate(const float* tile_max, bsfa_shape shape, int causal, bsfa_block block, const int64_t* ks,
                   int64_t n_levels, float* thresholds, void* stream);

/*
 * bsfa_validate - host-only check of a shape / mask / tile combination.
 * Makes no HIP call.  Returns BSFA_OK if bsfa_prefill would accept it
 * (pointer checks aside).
 */
int bsfa_validate(bsfa_shape shape, int causal, bsfa_block block);

/* bsfa_status_string - static, human-readable text for a status code. */
const char* bsfa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BSFA_H */
