"""Work/traffic counters against the figures the pages print (tests/golden/paper_figures.json)."""

import json
import math
import os

import pytest

from block_sparse_flashattention_tiled_amd import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "paper_figures.json")))


def test_tile_contraction_flops():
    for c in GOLD["tile_contraction"]["cases"]:
        assert acc.tile_matmul_flops(c["bm"], c["bn"], c["d"]) == 2 * c["bm"] * c["bn"] * c["d"]
    # both contractions of a tile are counted once each
    assert acc.dense_equivalent_flops(1, 1, 1, 128, 128, True) == 2 * acc.tile_matmul_flops(128, 128, 128)


def test_llama_128k_terms():
    g = GOLD["llama_128k_terms"]
    assert g["heads"] * g["head_dim"] == g["d_model"]
    quad = acc.quadratic_term_ops(g["n"], g["d_model"])
    proj = acc.projection_term_ops(g["n"], g["d_model"])
    # printed to two significant digits
    assert float(f"{quad:.1e}") == g["quadratic_term_printed"]
    assert float(f"{proj:.1e}") == g["projection_term_printed"]
    # "approximately 32:1" (N / d_model = 31.25 at N = 128,000)
    assert abs(quad / proj - g["ratio_printed"]) <= g["ratio_abs_tol"]
    # the same total from the tile counts: QK over all heads of a non-causal layer
    m = g["n"] // 128
    t = acc.tile_matmul_flops(128, 128, g["head_dim"]) * acc.computed_tiles(m, False) * g["heads"]
    assert t == 2 * quad


def test_score_matrix_128k():
    g = GOLD["score_matrix_128k"]
    e = acc.score_matrix_elements(g["n"])
    assert e > g["elements_over"]
    assert e * 2 / 1e9 == pytest.approx(g["fp16_gb_printed"], rel=g["rel_tol"])


def test_threshold_storage():
    g = GOLD["threshold_storage_llama"]
    n = acc.threshold_count(g["layers"], g["heads"], g["n_max"], g["bm"])
    assert n == 524288
    assert n == pytest.approx(g["count_printed"], rel=g["rel_tol"])
    assert round(100 * n / g["params"], 3) == g["percent_printed"]
    q = GOLD["threshold_storage_qwen"]
    b = acc.threshold_table_bytes(q["layers"], q["heads"], q["n_max"], q["bm"], q["levels"], q["elem_bytes"])
    assert b / 2**20 == pytest.approx(q["mib_printed"], abs=q["abs_tol"])


def test_v_share_and_causal_half():
    g = GOLD["v_share"]
    assert acc.v_share_of_kv_traffic(g["bn"], g["d"]) == g["share_printed"]
    c = GOLD["causal_half"]
    frac = acc.computed_tiles(c["m"], True) / acc.computed_tiles(c["m"], False)
    assert frac == pytest.approx(c["fraction_printed"], abs=c["abs_tol"])


def test_skip_halves_kv_bytes_of_a_tile():
    full = acc.algorithmic_bytes(1, 1, 1, 128, 128, 0, False)
    # one computed tile that is also the diagonal: K and V both read
    assert full["k_tiles"] == full["v_tiles"] == 128 * 128 * 2


@pytest.mark.parametrize(
    "m,k,causal,skipped,computed",
    [
        (16, 4, True, 66, 136),  # sum_{i=5}^{15} (i - 4) = 66 of 16*17/2
        (4, 0, True, 6, 10),     # only diagonal tiles kept
        (4, 3, True, 0, 10),     # every block has <= 3 off-diagonal tiles
        (8, 2, False, 8 * 5, 64),
    ],
)
def test_designed_fixed_k_counts(m, k, causal, skipped, computed):
    assert acc.designed_skipped_tiles(m, k, causal) == skipped
    assert acc.computed_tiles(m, causal) == computed


@pytest.mark.parametrize(
    "m,target,causal,k",
    [(16, 0.5, True, 4), (64, 0.5, True, 18), (256, 0.6, True, 57), (256, 0.8, True, 26),
     (256, 0.9, True, 12), (1024, 0.95, True, 25), (256, 0.75, False, 63), (256, 0.0, True, None)],
)
def test_k_for_target(m, target, causal, k):
    assert acc.k_for_target(m, target, causal) == k
    if k is not None:
        f = acc.designed_skip_fraction(m, k, causal)
        for kk in (k - 1, k + 1):
            if 0 <= kk < m:
                assert abs(f - target) <= abs(acc.designed_skip_fraction(m, kk, causal) - target)


def test_executed_flops_counts_kept_pv_only():
    b, h, m, blk, d = 1, 2, 8, 64, 64
    t = acc.tile_matmul_flops(blk, blk, d)
    comp = acc.computed_tiles(m, True) * b * h
    assert acc.executed_flops(b, h, m, blk, d, 10, True) == 2 * comp * t - 10 * t


@pytest.mark.parametrize("causal", [True, False])
def test_grid_counts_reduce_to_the_square_ones(causal):
    for m in (1, 2, 7, 64):
        n = 128 * m
        assert acc.grid_computed_tiles(n, 128, 128, causal) == acc.computed_tiles(m, causal)
        for k in (0, 1, 5, m + 3):
            assert acc.grid_designed_skipped_tiles(n, 128, 128, k, causal) == \
                acc.designed_skipped_tiles(m, k, causal)
        for tgt in (0.0, 0.6, 0.9):
            assert acc.grid_k_for_target(n, 128, 128, tgt, causal) == acc.k_for_target(m, tgt, causal)
        assert acc.grid_executed_flops(2, 3, n, 128, 128, 64, 11, causal) == \
            acc.executed_flops(2, 3, m, 128, 64, 11, causal)


def _brute_grid(n, bm, bn, causal):
    """(computed, off-diagonal) per query block by enumerating positions."""
    m, m_kv = -(-n // bm), -(-n // bn)
    rows = []
    for i in range(m):
        qs = range(i * bm, min((i + 1) * bm, n))
        comp = off = 0
        for j in range(m_kv):
            ks = range(j * bn, min((j + 1) * bn, n))
            if causal and not any(kk <= qq for qq in qs for kk in ks):
                continue
            comp += 1
            off += 0 if set(qs) & set(ks) else 1
        rows.append((comp, off))
    return rows


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,bm,bn", [(1024, 128, 64), (1000, 128, 64), (960, 64, 128), (77, 128, 64),
                                     (300, 48, 32), (256, 32, 48)])
def test_grid_rows_by_enumeration(n, bm, bn, causal):
    assert acc.grid_rows(n, bm, bn, causal) == _brute_grid(n, bm, bn, causal)


def test_grid_128x64_causal_closed_form():
    # query block i of 128 rows sees key blocks 0..2i+1 of 64 keys, two of them diagonal
    m = 16
    rows = acc.grid_rows(128 * m, 128, 64, True)
    assert rows == [(2 * i + 2, 2 * i) for i in range(m)]
    assert acc.grid_computed_tiles(128 * m, 128, 64, True) == m * (m + 1)
