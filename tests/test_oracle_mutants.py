"""Plant plausible mistakes in the oracle (CPU) and check that a pin catches each.

Each mutant replaces one function of the oracle module for the duration of a
test; the pin that guards the corresponding passage must then fail.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import bsfa_oracle as ob
import test_oracle_gap_gate as gap_pins
import test_oracle_pins as pins
import test_oracle_rect as rect_pins


def _mut_gate_le(tile_max_row, diag, tau):  # '<=' instead of the strict '<'
    skip = tile_max_row <= tau
    skip[list(diag)] = False
    return skip


def _mut_gate_no_bypass(tile_max_row, diag, tau):  # diagonal gated like the rest
    return tile_max_row < tau


def _mut_unscaled(q_rows, k_cols, head_dim):  # scores without 1/sqrt(d)
    return q_rows @ k_cols.T


def _mut_threshold_wrap(thresholds, h, i):  # wraps positions instead of reusing the last
    return float(thresholds[h, i % thresholds.shape[1]])


def _mut_tile_max_all(s, vis, block):  # maximum over masked entries too
    n = s.shape[1] // block
    return np.array([s[:, j * block:(j + 1) * block].max() for j in range(n)])


_ORIG_RUN_BLOCKS = ob.run_blocks


def _mut_gqa_modulo(q, k, v, thresholds, causal, block, blocks, skip_override=None, gate_mode="threshold"):
    # KV head h % H_kv instead of the contiguous h // G: permute q heads so the
    # real routine sees the interleaved grouping
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    perm = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)])
    res = _ORIG_RUN_BLOCKS(q[:, perm], k, v, thresholds[perm], causal, block,
                           [(b, int(np.flatnonzero(perm == h)[0]), i) for b, h, i in blocks], skip_override,
                           gate_mode)
    for r, (b, h, i) in zip(res, blocks):
        r["h"] = h
    return res


def _mut_gap_global_max(tile_max_row, diag, tau):  # reference = max over every tile, not the running max
    skip = tile_max_row < np.max(tile_max_row) - tau
    skip[list(diag)] = False
    return skip


def _mut_gap_sign(tile_max_row, diag, tau):  # M + tau instead of M - tau
    n = tile_max_row.shape[0]
    skip = np.zeros(n, dtype=bool)
    m = -np.inf
    for j in range(n):
        if j not in diag and tile_max_row[j] < m + tau:
            skip[j] = True
        else:
            m = max(m, float(tile_max_row[j]))
    return skip


def _mut_diag_square(i, bm, bn, m_kv):  # diagonal = same block index, as if the tile were square
    return [i] if i < m_kv else []


def _mut_diag_touching(i, bm, bn, m_kv):  # blocks that merely touch the query block count as diagonal
    return [j for j in range(m_kv) if j * bn <= (i + 1) * bm and (j + 1) * bn >= i * bm]


def _mut_calib_square(tile_max_row, i, k, causal, block=1):  # off-diagonal set of a square tile
    cols = [j for j in (range(i) if causal else range(tile_max_row.shape[0])) if j != i]
    if len(cols) <= k:
        return -np.inf
    if k == 0:
        return np.inf
    vals = np.sort(tile_max_row[cols])[::-1]
    return 0.5 * (vals[k - 1] + vals[k])


_ORIG_TO_F64 = ob.to_f64


def _mut_to_f64_fp16(x):  # bf16 bits read as IEEE half precision
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return x.view(np.float16).astype(np.float64)
    return _ORIG_TO_F64(x)


def _mut_to_f64_shift(x):  # mantissa bits placed one position too low
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return _ORIG_TO_F64(x)


def _mut_override_transposed(q, k, v, thresholds, causal, block, blocks, skip_override=None,
                             gate_mode="threshold"):  # the mask read as [.., key block, query block]
    if skip_override is not None:
        skip_override = np.swapaxes(skip_override, -1, -2)
    return _ORIG_RUN_BLOCKS(q, k, v, thresholds, causal, block, blocks, skip_override, gate_mode)


def _mut_override_ignored(q, k, v, thresholds, causal, block, blocks, skip_override=None,
                          gate_mode="threshold"):  # the gate's own decisions kept
    return _ORIG_RUN_BLOCKS(q, k, v, thresholds, causal, block, blocks, None, gate_mode)


MUTANTS = [
    ("to_f64", _mut_to_f64_fp16, pins.test_bf16_decode_matches_library_conversion),
    ("to_f64", _mut_to_f64_shift, pins.test_bf16_decode_matches_library_conversion),
    ("run_blocks", _mut_override_transposed,
     lambda: pins.test_mask_override_equals_library_attention_under_the_mask(False, 256, 64)),
    ("run_blocks", _mut_override_ignored,
     lambda: pins.test_mask_override_equals_library_attention_under_the_mask(True, 256, 64)),
    ("gate", _mut_gate_le, lambda: pins.test_uniform_scores_tie_rule_closed_form(True)),
    ("gate", _mut_gate_no_bypass, lambda: pins.test_infinite_threshold_is_block_diagonal_attention(True)),
    ("block_scores", _mut_unscaled, lambda: pins.test_dense_threshold_equals_library_attention(True)),
    ("threshold_for", _mut_threshold_wrap, pins.test_threshold_table_reuses_last_entry),
    ("block_tile_maxima", _mut_tile_max_all,
     lambda: pins.test_oracle_matches_brute_force_streaming(True, 1, 2, 1, 256, 16, 4, 3)),
    ("run_blocks", _mut_gqa_modulo, lambda: pins.test_dense_threshold_equals_library_attention(False)),
    ("gate_gap", _mut_gap_global_max,
     lambda: gap_pins.test_gap_gate_matches_brute_force_streaming(True, 1, 2, 1, 256, 16, 4, 21)),
    ("gate_gap", _mut_gap_sign, lambda: gap_pins.test_uniform_scores_closed_form(True)),
    ("diagonal_blocks", _mut_diag_square,
     lambda: rect_pins.test_infinite_threshold_keeps_the_tiles_sharing_a_position(True, 256, (64, 32))),
    ("diagonal_blocks", _mut_diag_touching,
     lambda: rect_pins.test_infinite_threshold_keeps_the_tiles_sharing_a_position(False, 256, (32, 64))),
    ("calibrate_row", _mut_calib_square, lambda: rect_pins.test_rect_fixed_k_keeps_exactly_k(True, (64, 32))),
]


@pytest.mark.parametrize("name,mutant,pin", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_pin_catches_mutant(monkeypatch, name, mutant, pin):
    # the module's own calls and the package's re-export both see the mutant
    monkeypatch.setattr(ob, name, mutant)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, mutant)
    with pytest.raises((AssertionError, ValueError)):
        pin()
