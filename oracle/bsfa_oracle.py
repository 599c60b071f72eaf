"""CPU float64 oracle for block-sparse FlashAttention prefill (BSFA form).

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It is the definition
the HIP path is checked against and it shares no code with that path: it
imports nothing from the kernel package and the kernel package imports
nothing from here.

Source: "Block Sparse Flash Attention" (paperpeel.com/paper/2512.07011).

What is computed, per batch b and query head h (KV head g = h // G):

* Scores are the scaled dot products S = Q K^T / sqrt(d)            (Sec. 2,
  "Scaled dot-product attention"; App. B.2 step (3)).
* Queries are cut into blocks of B_M rows, keys into blocks of B_N columns;
  tile (i, j) pairs query block i with key block j (App. B.2).  ``block`` is
  B_M = B_N (an int) or the pair (B_M, B_N).  M_Q = ceil(N / B_M) and
  M_KV = ceil(N / B_N): when N is not a multiple of a side the last block is
  partial, and positions >= N do not exist (a reading: the pages pad to a
  multiple by repeating the last token, App. B.3, which makes the padding
  tokens keys of every query).  Under causal masking key k is visible to
  query q iff k <= q, and a tile holding no visible pair (its first key after
  the query block's last query) is not computed (App. B.2, "approximately
  half for causal").
* The diagonal tiles of query block i are the key blocks whose positions
  overlap the block's own (Sec. 4.1).  With square tiles that is j = i; the
  pages' kernels use 128 x 64 tiles (Sec. 5.1) and 128 x 224 (App. A.3)
  without saying which tiles count as diagonal, and overlap is the reading
  taken here: it keeps, for every query q, the tile holding key q.
* Each computed tile has a maximum score s_max(i, j), taken over its visible
  entries (Sec. 4.1).
* The threshold for head h and query block i is T[h, min(i, T_len - 1)]:
  per (head, position) (Sec. 4.1, 4.2), with positions past the table
  reusing its last entry (App. B.3, "Practical considerations").
* Tile (i, j) is skipped iff it is not diagonal and s_max(i, j) < T
  (strict, Sec. 4.4); diagonal tiles always pass (Sec. 4.1).  A NaN threshold
  compares false, so nothing is skipped.
* A skipped tile takes no part in the running max, sum or output (Sec. 4.4).
  Online softmax over the kept tiles is an exact rearrangement of one softmax
  over the kept entries (App. B.2), so the oracle evaluates that softmax
  directly: lse[q] = log sum_{k in R(q)} exp S[q, k] and
  O[q] = sum_{k in R(q)} exp(S[q, k] - lse[q]) V[k], where R(q) is the set
  of visible keys in kept tiles.  R(q) always holds k = q (diagonal tile).

Readings where the pages are silent (each is listed in the design notes):
the gate uses the scaled score; the tile max runs over visible entries only;
GQA groups are contiguous (g = h // (H_q / H_kv)); lse is the natural log of
the scaled scores over R(q); ties (s_max == T) are kept.

A second gate, for comparison (``gate_mode="gap"``): the running-maximum
reference that the pages attribute to BLASST and to SpargeAttention's
in-kernel P.V skip (Sec. 3 "Related Work": gating on the gap to a running
maximum rather than on a stored threshold).  The pages give no formula; the
reading used here: key blocks are visited in increasing order (App. B.2) and
off-diagonal tile j is skipped iff s_max(i, j) < M - tau, where M is the
largest s_max among the tiles kept before j (-inf before the first) and tau
is the table entry of (head, query block), read as the gap.

Threshold calibration (Sec. 4.2, App. B.3): for each query block, sort the
off-diagonal computed tiles by their maxima and put the threshold so exactly
the top k are retained - here the midpoint between the k-th and (k+1)-th
largest maxima, or -inf when the block has at most k off-diagonal tiles -
then average over calibration samples (the batch axis).
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "to_f64",
    "tile_shape",
    "diagonal_blocks",
    "block_scores",
    "block_tile_maxima",
    "threshold_for",
    "gate",
    "gate_gap",
    "masked_softmax_attention",
    "run_blocks",
    "run",
    "tile_maxima",
    "calibrate_row",
    "calibrate_fixed_k",
    "STATE_PRUNED",
    "STATE_KEPT",
    "STATE_SKIPPED",
    "STATE_DIAGONAL",
]

# tile_state codes
STATE_PRUNED = 0  # causal: tile above the diagonal, never computed
STATE_KEPT = 1  # off-diagonal tile that passed the gate
STATE_SKIPPED = 2  # off-diagonal tile below its threshold
STATE_DIAGONAL = 3  # diagonal tile (bypasses the gate)


def to_f64(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly; float arrays pass through."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def tile_shape(block) -> Tuple[int, int]:
    """(B_M, B_N) of ``block``: an int is a square tile, a pair is (B_M, B_N)."""
    if isinstance(block, (tuple, list)):
        bm, bn = int(block[0]), int(block[1])
    else:
        bm = bn = int(block)
    if bm < 1 or bn < 1:
        raise ValueError("tile sides must be positive")
    return bm, bn


def diagonal_blocks(i: int, bm: int, bn: int, m_kv: int) -> List[int]:
    """Key blocks j < m_kv whose positions [j B_N, (j+1) B_N) overlap those of
    query block i, [i B_M, (i+1) B_M): the tiles that bypass the gate
    (Sec. 4.1; overlap is the reading for B_M != B_N).  Positions past N need
    no clipping: key block j exists iff j < m_kv, and then j B_N < N."""
    return [j for j in range(m_kv) if j * bn < (i + 1) * bm and (j + 1) * bn > i * bm]


def block_scores(q_rows: np.ndarray, k_cols: np.ndarray, head_dim: int) -> np.ndarray:
    """Scaled scores S = Q_i K^T / sqrt(d) of one query block (Sec. 2; App. B.2 step (3))."""
    return (q_rows @ k_cols.T) / math.sqrt(head_dim)


def _visible(q0: int, n_rows: int, n_keys: int, causal: bool) -> np.ndarray:
    """Visibility of keys [0, n_keys) to query rows [q0, q0 + n_rows)."""
    qpos = np.arange(q0, q0 + n_rows)[:, None]
    kpos = np.arange(n_keys)[None, :]
    if causal:
        return kpos <= qpos
    return np.ones((n_rows, n_keys), dtype=bool)


def block_tile_maxima(s: np.ndarray, vis: np.ndarray, bn: int) -> np.ndarray:
    """s_max(i, j) over the visible entries of each computed key block j of
    ``bn`` keys (Sec. 4.1); the last key block may be partial."""
    n_tiles = -(-s.shape[1] // bn)
    out = np.empty(n_tiles)
    for j in range(n_tiles):
        cols = slice(j * bn, min((j + 1) * bn, s.shape[1]))
        out[j] = s[:, cols][vis[:, cols]].max()
    return out


def threshold_for(thresholds: np.ndarray, h: int, i: int) -> float:
    """T[h, i] with positions past the table reusing the last entry (App. B.3)."""
    t_len = thresholds.shape[1]
    return float(thresholds[h, min(i, t_len - 1)])


def gate(tile_max_row: np.ndarray, diag: Sequence[int], tau: float) -> np.ndarray:
    """Skip decision of the computed tiles of one query block (Sec. 4.1, 4.4).

    ``diag``: the block's diagonal key blocks.  Skip iff not diagonal and
    s_max < tau (strict).  ``tau`` NaN compares false.
    """
    skip = tile_max_row < tau
    skip[list(diag)] = False  # diagonal bypass
    return skip


def gate_gap(tile_max_row: np.ndarray, diag: Sequence[int], tau: float) -> np.ndarray:
    """Skip decisions of the gap gate for one query block (see the module notes).

    Tiles are visited in increasing key-block order; tile j not in ``diag`` is
    skipped iff s_max(i, j) < M - tau with M the largest s_max of the tiles
    kept so far.  IEEE arithmetic throughout: -inf - (-inf) is NaN, and a NaN
    comparison keeps the tile.
    """
    n = tile_max_row.shape[0]
    skip = np.zeros(n, dtype=bool)
    m = -np.inf
    with np.errstate(invalid="ignore"):
        for j in range(n):
            if j not in diag and tile_max_row[j] < np.float64(m) - np.float64(tau):
                skip[j] = True
            else:
                m = max(m, float(tile_max_row[j]))
    return skip


def masked_softmax_attention(s: np.ndarray, keep: np.ndarray, v_rows: np.ndarray):
    """lse and output of softmax restricted to ``keep`` (App. B.2 + Sec. 4.4).

    lse[q] = log sum_{k: keep} exp s[q, k];  O[q] = sum_{k: keep} exp(s[q,k] - lse[q]) V[k].
    Every row must keep at least one entry.
    """
    if not keep.any(axis=1).all():
        raise ValueError("a query row keeps no key")
    # only keys some row keeps enter the arithmetic: a skipped tile's V rows
    # are never read (Sec. 4.4)
    cols = np.flatnonzero(keep.any(axis=0))
    s_kept = np.where(keep[:, cols], s[:, cols], -np.inf)
    m = s_kept.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s_kept - m).sum(axis=1))
    p = np.exp(s_kept - lse[:, None])  # exp(-inf) = 0 outside keep
    return p @ v_rows[cols], lse


def run_blocks(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    thresholds: np.ndarray,
    causal: bool,
    block,
    blocks: Iterable[Tuple[int, int, int]],
    skip_override: Optional[np.ndarray] = None,
    gate_mode: str = "threshold",
) -> List[dict]:
    """Evaluate selected query blocks ``(b, h, i)``.

    q: [B, H_q, N, d], k/v: [B, H_kv, N, d] (bf16 bits or floats);
    thresholds: [H_q, T_len]; ``block``: B_M = B_N or (B_M, B_N).
    ``skip_override`` ([B, H_q, M_Q, M_KV] bool) replaces the gate's
    decisions when given (diagonal tiles must stay kept).  ``gate_mode``:
    "threshold" (the pages' gate) or "gap" (``gate_gap``).

    Each result holds ``out`` [rows, d], ``lse`` [rows], ``tile_max`` [M_KV]
    (NaN where not computed), ``tile_state`` [M_KV] uint8 and ``skip_count``.
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    if gate_mode not in ("threshold", "gap"):
        raise ValueError("gate_mode must be 'threshold' or 'gap'")
    G = Hq // Hkv
    bm, bn = tile_shape(block)
    M_kv = -(-N // bn)
    results = []
    cache = {}
    for b, h, i in blocks:
        g = h // G
        key = (b, g)
        if key not in cache:
            cache.clear()
            cache[key] = (to_f64(k[b, g]), to_f64(v[b, g]))
        kf, vf = cache[key]
        r_end = min((i + 1) * bm, N)
        n_keys = r_end if causal else N
        q_rows = to_f64(q[b, h, i * bm : r_end])
        s = block_scores(q_rows, kf[:n_keys], d)
        vis = _visible(i * bm, r_end - i * bm, n_keys, causal)
        tmax = block_tile_maxima(s, vis, bn)
        diag = diagonal_blocks(i, bm, bn, M_kv)
        tau = threshold_for(thresholds, h, i)
        if skip_override is not None:
            skip = np.array(skip_override[b, h, i, : tmax.shape[0]], dtype=bool)
            if skip[diag].any():
                raise ValueError("a diagonal tile cannot be skipped")
        elif gate_mode == "gap":
            skip = gate_gap(tmax, diag, tau)
        else:
            skip = gate(tmax, diag, tau)
        keep = vis & ~np.repeat(skip, bn)[None, :n_keys]
        out, lse = masked_softmax_attention(s, keep, vf[:n_keys])
        tile_max = np.full(M_kv, np.nan)
        tile_max[: tmax.shape[0]] = tmax
        state = np.full(M_kv, STATE_PRUNED, dtype=np.uint8)
        state[: tmax.shape[0]] = np.where(skip, STATE_SKIPPED, STATE_KEPT)
        state[diag] = STATE_DIAGONAL
        results.append(
            {
                "b": b,
                "h": h,
                "i": i,
                "out": out,
                "lse": lse,
                "tile_max": tile_max,
                "tile_state": state,
                "skip_count": int(skip.sum()),
                "tau": tau,
            }
        )
    return results


def run(q, k, v, thresholds, causal: bool, block, skip_override=None, gate_mode: str = "threshold") -> dict:
    """Whole-layer oracle: out [B,H_q,N,d], lse [B,H_q,N], skip_counts [B,H_q,M_Q],
    tile_state [B,H_q,M_Q,M_KV] (uint8), tile_max [B,H_q,M_Q,M_KV] (NaN where not
    computed)."""
    B, Hq, N, d = q.shape
    bm, bn = tile_shape(block)
    M, M_kv = -(-N // bm), -(-N // bn)
    out = np.empty((B, Hq, N, d))
    lse = np.empty((B, Hq, N))
    skip_counts = np.empty((B, Hq, M), dtype=np.int64)
    tile_state = np.empty((B, Hq, M, M_kv), dtype=np.uint8)
    tile_max = np.empty((B, Hq, M, M_kv))
    blocks = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(M)]
    for r in run_blocks(q, k, v, thresholds, causal, block, blocks, skip_override, gate_mode):
        b, h, i = r["b"], r["h"], r["i"]
        rows = slice(i * bm, min((i + 1) * bm, N))
        out[b, h, rows] = r["out"]
        lse[b, h, rows] = r["lse"]
        skip_counts[b, h, i] = r["skip_count"]
        tile_state[b, h, i] = r["tile_state"]
        tile_max[b, h, i] = r["tile_max"]
    return {
        "out": out,
        "lse": lse,
        "skip_counts": skip_counts,
        "tile_state": tile_state,
        "tile_max": tile_max,
    }


def tile_maxima(q, k, causal: bool, block, heads: Optional[Sequence[int]] = None,
                rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """s_max of every computed tile: [B, H_q, M_Q, M_KV] float64, NaN where not
    computed.  ``heads`` / ``rows`` restrict the evaluation (other entries stay NaN).
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    bm, bn = tile_shape(block)
    M, M_kv = -(-N // bm), -(-N // bn)
    out = np.full((B, Hq, M, M_kv), np.nan)
    heads = range(Hq) if heads is None else heads
    rows = range(M) if rows is None else rows
    for b in range(B):
        for h in heads:
            kf = to_f64(k[b, h // G])
            for i in rows:
                r_end = min((i + 1) * bm, N)
                n_keys = r_end if causal else N
                s = block_scores(to_f64(q[b, h, i * bm : r_end]), kf[:n_keys], d)
                tm = block_tile_maxima(s, _visible(i * bm, r_end - i * bm, n_keys, causal), bn)
                out[b, h, i, : tm.shape[0]] = tm
    return out


def calibrate_row(tile_max_row: np.ndarray, i: int, k: int, causal: bool, block=1) -> float:
    """Fixed-k threshold of query block i from one sample's tile maxima row [M_KV] (Sec. 4.2).

    The off-diagonal computed tiles - key blocks not among the diagonal ones
    and, under causal masking, starting before the query block ends - are
    sorted by their maxima, largest first.  With n of them: -inf if n <= k,
    +inf if k == 0 (no off-diagonal tile retained), otherwise the midpoint of
    the k-th and (k+1)-th largest, so that (barring ties) exactly the top k
    are retained.  ``block``: (B_M, B_N); an int means a square tile, and any
    square size gives the same index sets (causal: j < i; else j != i).
    """
    if k < 0:
        raise ValueError("k must be >= 0")
    bm, bn = tile_shape(block)
    M_kv = tile_max_row.shape[0]
    diag = diagonal_blocks(i, bm, bn, M_kv)
    cols = [j for j in range(M_kv) if j not in diag and (not causal or j * bn < (i + 1) * bm)]
    if len(cols) <= k:
        return -np.inf
    if k == 0:
        return np.inf
    vals = np.sort(tile_max_row[cols])[::-1]
    if np.isnan(vals).any():
        raise ValueError("tile maxima missing for a calibrated row")
    return 0.5 * (vals[k - 1] + vals[k])


def calibrate_fixed_k(tile_max: np.ndarray, k: int, causal: bool, block=1) -> np.ndarray:
    """Fixed-k thresholds [H_q, M_Q] from sample tile maxima [S, H_q, M_Q, M_KV]
    (Sec. 4.2, App. B.3).

    Each (head, query block) gets ``calibrate_row`` per sample; the samples'
    thresholds are then averaged ("averaging across calibration samples").
    """
    S, Hq, M, _ = tile_max.shape
    thr = np.zeros((Hq, M))
    for h in range(Hq):
        for i in range(M):
            thr[h, i] = sum(calibrate_row(tile_max[s_idx, h, i], i, k, causal, block)
                            for s_idx in range(S)) / S
    return thr
