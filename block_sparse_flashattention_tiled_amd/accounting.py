"""Work and traffic accounting for block-sparse FlashAttention prefill.

Counting only: no attention arithmetic lives here.  Each count follows a
statement of "Block Sparse Flash Attention" (paperpeel.com/paper/2512.07011):

* every tile runs two equally expensive contractions, S = Q_i K_j^T and
  P~_ij V_j, each of 2 B_M B_N d FLOPs (Sec. 2 "FlashAttention"; App. B.2);
* a skipped tile saves the P.V contraction and the B_N d elements of V_j, i.e.
  half of the key/value traffic (Sec. 4.3);
* causal attention computes about half of the M_Q x M_KV tiles (App. B.2);
* the threshold table holds one value per (level, layer, head, query block)
  (Sec. 4.2; App. B.3 "Threshold tensor", "Storage overhead");
* for N >> d_model the QK and PV terms scale as N^2 d_model against
  N d_model^2 for the projections (App. B.1).

The fixed-k helpers count the tiles a fixed-k table is designed to skip: a
query block with n off-diagonal computed tiles keeps min(k, n) of them plus
its diagonal tile (Sec. 4, 4.1, 4.2).  The ``grid_*`` helpers do the same for
any tile B_M x B_N and length N (partial last blocks): the diagonal tiles of
a query block are the key blocks overlapping its positions, and under causal
masking a tile is computed when its first key is not after the block's last
query.
"""

from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

__all__ = [
    "tile_matmul_flops",
    "computed_tiles",
    "off_diagonal_tiles",
    "designed_skipped_tiles",
    "designed_skip_fraction",
    "k_for_target",
    "executed_flops",
    "dense_equivalent_flops",
    "algorithmic_bytes",
    "quadratic_term_ops",
    "projection_term_ops",
    "score_matrix_elements",
    "threshold_count",
    "threshold_table_bytes",
    "v_share_of_kv_traffic",
    "grid_rows",
    "grid_computed_tiles",
    "grid_designed_skipped_tiles",
    "grid_designed_skip_fraction",
    "grid_k_for_target",
    "grid_executed_flops",
]


def tile_matmul_flops(bm: int, bn: int, d: int) -> int:
    """FLOPs of one tile contraction, Q_i K_j^T or P~ V_j: 2 B_M B_N d."""
    return 2 * bm * bn * d


def computed_tiles(m: int, causal: bool) -> int:
    """Tiles computed for one head with M square blocks (causal: lower triangle)."""
    return m * (m + 1) // 2 if causal else m * m


def off_diagonal_tiles(i: int, m: int, causal: bool) -> int:
    """Off-diagonal computed tiles of query block i."""
    return i if causal else m - 1


def designed_skipped_tiles(m: int, k: int, causal: bool) -> int:
    """Tiles one head skips under a fixed-k table: sum_i max(0, n_i - k)."""
    return sum(max(0, off_diagonal_tiles(i, m, causal) - k) for i in range(m))


def designed_skip_fraction(m: int, k: int, causal: bool) -> float:
    """Skipped / computed tiles for a fixed-k table."""
    return designed_skipped_tiles(m, k, causal) / computed_tiles(m, causal)


def k_for_target(m: int, target: float, causal: bool) -> Optional[int]:
    """The k whose designed skip fraction is closest to ``target``.

    ``None`` stands for "no gating" (threshold -inf everywhere), returned for
    a target of 0.  Ties go to the larger k (fewer skips).
    """
    if target <= 0.0:
        return None
    kmax = m - 1
    best_k, best_err = kmax, float("inf")
    for k in range(kmax, -1, -1):
        err = abs(designed_skip_fraction(m, k, causal) - target)
        if err < best_err - 1e-15:
            best_k, best_err = k, err
    return best_k


def executed_flops(batch: int, heads: int, m: int, block: int, d: int, skipped: int, causal: bool) -> int:
    """MFMA FLOPs actually issued: QK^T on every computed tile, P.V on kept ones.

    ``skipped`` is the total number of skipped tiles over all (batch, head).
    """
    t = tile_matmul_flops(block, block, d)
    comp = computed_tiles(m, causal) * batch * heads
    return comp * t + (comp - skipped) * t


def dense_equivalent_flops(batch: int, heads: int, m: int, block: int, d: int, causal: bool) -> int:
    """FLOPs of the same tiled computation with nothing skipped."""
    return executed_flops(batch, heads, m, block, d, 0, causal)


def algorithmic_bytes(batch: int, heads: int, m: int, block: int, d: int, skipped: int, causal: bool,
                      out_bytes: int = 4) -> Dict[str, int]:
    """Bytes the method must move between HBM and the compute units.

    Per computed tile: K_j (block * d bf16).  Per kept tile: V_j.  Per query
    block: Q_i, O_i (``out_bytes`` per element), lse, one threshold and one
    skip count.  Re-reads of K_j / V_j by different query blocks are counted
    (they are the tile stream), so this is an upper bound on compulsory HBM
    traffic and a lower bound on cache-to-CU traffic.
    """
    comp = computed_tiles(m, causal) * batch * heads
    kept = comp - skipped
    qblocks = m * batch * heads
    tile = block * d * 2
    parts = {
        "k_tiles": comp * tile,
        "v_tiles": kept * tile,
        "q": qblocks * tile,
        "out": qblocks * block * d * out_bytes,
        "lse": qblocks * block * 4,
        "thresholds": qblocks * 4,
        "skip_counts": qblocks * 4,
    }
    parts["total"] = sum(parts.values())
    return parts


def quadratic_term_ops(n: int, d_model: int) -> int:
    """N^2 d_model: the size of each of the QK and PV terms over all heads (App. B.1)."""
    return n * n * d_model


def projection_term_ops(n: int, d_model: int) -> int:
    """N d_model^2: the size of the linear-projection term (App. B.1)."""
    return n * d_model * d_model


def score_matrix_elements(n: int) -> int:
    """Elements of one head's N x N score matrix (App. B.1)."""
    return n * n


def threshold_count(layers: int, heads: int, n_max: int, bm: int, levels: int = 1) -> int:
    """Entries of T in R^{S x L x H x ceil(N_max / B_M)} (Sec. 4.2; App. B.3)."""
    return levels * layers * heads * math.ceil(n_max / bm)


def threshold_table_bytes(layers: int, heads: int, n_max: int, bm: int, levels: int, elem_bytes: int) -> int:
    """Storage of the threshold table."""
    return threshold_count(layers, heads, n_max, bm, levels) * elem_bytes


def v_share_of_kv_traffic(bn: int, d: int) -> float:
    """Share of one tile's K+V load that a skip avoids: V_j over K_j + V_j (Sec. 4.3)."""
    return (bn * d) / (2 * bn * d)


def grid_rows(n: int, bm: int, bn: int, causal: bool):
    """Per query block of a length-``n`` sequence cut into ``bm`` x ``bn`` tiles:
    (computed tiles, off-diagonal computed tiles)."""
    m, m_kv = -(-n // bm), -(-n // bn)
    rows = []
    for i in range(m):
        last_q = min((i + 1) * bm, n) - 1
        computed = min(last_q // bn + 1, m_kv) if causal else m_kv
        first_diag = (i * bm) // bn
        last_diag = min(last_q // bn, m_kv - 1)
        rows.append((computed, computed - (last_diag - first_diag + 1)))
    return rows


def grid_computed_tiles(n: int, bm: int, bn: int, causal: bool) -> int:
    """Tiles computed for one head."""
    return sum(c for c, _ in grid_rows(n, bm, bn, causal))


def grid_designed_skipped_tiles(n: int, bm: int, bn: int, k: int, causal: bool) -> int:
    """Tiles one head skips under a fixed-k table: sum_i max(0, n_i - k)."""
    return sum(max(0, off - k) for _, off in grid_rows(n, bm, bn, causal))


def grid_designed_skip_fraction(n: int, bm: int, bn: int, k: int, causal: bool) -> float:
    return grid_designed_skipped_tiles(n, bm, bn, k, causal) / grid_computed_tiles(n, bm, bn, causal)


def grid_k_for_target(n: int, bm: int, bn: int, target: float, causal: bool) -> Optional[int]:
    """The k whose designed skip fraction is closest to ``target`` (None for 0: no gating;
    ties go to the larger k)."""
    if target <= 0.0:
        return None
    kmax = max(off for _, off in grid_rows(n, bm, bn, causal))
    best_k, best_err = kmax, float("inf")
    for k in range(kmax, -1, -1):
        err = abs(grid_designed_skip_fraction(n, bm, bn, k, causal) - target)
        if err < best_err - 1e-15:
            best_k, best_err = k, err
    return best_k


def grid_executed_flops(batch: int, heads: int, n: int, bm: int, bn: int, d: int, skipped: int,
                        causal: bool) -> int:
    """MFMA FLOPs issued on full tiles: QK^T on every computed tile, P.V on kept ones
    (partial tiles are counted whole, as the kernel computes them)."""
    t = tile_matmul_flops(bm, bn, d)
    comp = grid_computed_tiles(n, bm, bn, causal) * batch * heads
    return comp * t + (comp - skipped) * t
