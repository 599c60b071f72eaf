"""The forward paths return identical bits where they compute the same thing.

* Head pairs against causal block pairs: a causal layer whose query heads
  share one K/V runs as head pairs (G = 2); the same query heads with that K/V
  repeated per head run as causal block pairs (G = 1), whose two units'
  diagonals fall one step apart.  Every (head, query block) sees the same Q
  rows, keys, values and threshold, so out, lse, skip counts and the per-tile
  diagnostics must agree bit for bit.
* The pipelined kernel's tail instance against its aligned one: an aligned
  layer through ``bsfa_prefill`` / ``bsfa_prefill_ex`` and through
  ``bsfa_prefill_varlen`` with every sequence at full length (the instance
  that handles tails), for head pairs (causal and bidirectional) and
  bidirectional block pairs.

Each at threshold -inf, at a fixed-k point calibrated on the GPU, and at
thresholds equal to tile maxima (the median computed tile of each (head,
query block) of batch element 0, kept as a tie).
"""

import pytest
import torch

from block_sparse_flashattention_tiled_amd import accounting as acc
from block_sparse_flashattention_tiled_amd import binding as bb
from block_sparse_flashattention_tiled_amd import workloads as wl

pytestmark = pytest.mark.gpu

TAIL_CASES = {
    "headpair-causal": dict(base="llama8k", batch=2, seq_len=1024, heads_q=8, heads_kv=2),
    "headpair-bidirectional": dict(base="llama8k", batch=1, seq_len=1024, heads_q=4, heads_kv=2, causal=False),
    "blockpair-bidirectional": dict(base="llama8k", batch=2, seq_len=768, heads_q=3, heads_kv=1, causal=False),
}


def _threshold_sets(q, k, w):
    tile = (w.block, w.block)
    M = w.n_blocks
    tmax = bb.tile_max(q, k, w.causal, tile)
    kk = acc.grid_k_for_target(w.seq_len, w.block, w.block, 0.5, w.causal)
    return {
        "dense": torch.full((w.heads_q, M), float("-inf"), device="cuda"),
        "fixed-k": bb.calibrate(tmax, [kk], w.causal, tile, w.seq_len, w.head_dim)[0].contiguous(),
        "on-maxima": torch.nanmedian(tmax[0], dim=-1).values.contiguous(),
    }


def _assert_same(a, b, label):
    for n in ("out", "lse", "skip_counts", "tile_state"):
        assert torch.equal(a[n], b[n]), f"{label}: {n} differs"
    same = (a["tile_max"] == b["tile_max"]) | (torch.isnan(a["tile_max"]) & torch.isnan(b["tile_max"]))
    assert bool(same.all()), f"{label}: tile maxima differ"


def test_head_pairs_and_causal_block_pairs_agree():
    assert torch.cuda.is_available()
    w = wl.get_config("llama8k", batch=2, seq_len=1024, heads_q=4, heads_kv=2)
    data = wl.generate(w, seed=5)
    q = bb.bits_to_device(data["q"])
    # one K/V per pair of query heads (G = 2: head pairs) ...
    k2 = bb.bits_to_device(data["k"])
    v2 = bb.bits_to_device(data["v"])
    # ... and the same K/V repeated per query head (G = 1: causal block pairs)
    k1 = k2.repeat_interleave(2, dim=1).contiguous()
    v1 = v2.repeat_interleave(2, dim=1).contiguous()
    tile = (w.block, w.block)
    for label, thr in _threshold_sets(q, k2, w).items():
        print(f"[kernels-agree] {label}", flush=True)
        hp = bb.prefill(q, k2, v2, thr, True, tile, diagnostics=True)
        bp = bb.prefill(q, k1, v1, thr, True, tile, diagnostics=True)
        hp_prod = bb.prefill(q, k2, v2, thr, True, tile)
        bp_prod = bb.prefill(q, k1, v1, thr, True, tile)
        torch.cuda.synchronize()
        _assert_same(hp, bp, f"head pairs vs block pairs / {label}")
        for n in ("out", "lse", "skip_counts"):
            assert torch.equal(hp_prod[n], bp_prod[n]), f"production {n} differs / {label}"
            assert torch.equal(hp_prod[n], hp[n]), f"production vs diagnostics {n} / {label}"
        skipped = int((hp["tile_state"] == 2).sum())
        print(f"[kernels-agree] {label}: identical, {skipped} tiles skipped", flush=True)
        if label != "dense":
            assert skipped > 0


@pytest.mark.parametrize("name", list(TAIL_CASES))
def test_tail_instance_matches_aligned(name):
    assert torch.cuda.is_available()
    over = dict(TAIL_CASES[name])
    w = wl.get_config(over.pop("base"), **over)
    print(f"[tail-agree {name}] generating", flush=True)
    data = wl.generate(w, seed=3)
    q, k, v = (bb.bits_to_device(data[n]) for n in ("q", "k", "v"))
    tile = (w.block, w.block)
    lens = torch.full((w.batch,), w.seq_len, dtype=torch.int32, device="cuda")
    for label, thr in _threshold_sets(q, k, w).items():
        aligned = bb.prefill(q, k, v, thr, w.causal, tile)
        aligned_ex = bb.prefill(q, k, v, thr, w.causal, tile, diagnostics=True)
        tails = bb.prefill_varlen(q, k, v, thr, w.causal, tile, lens, diagnostics=True)
        torch.cuda.synchronize()
        _assert_same(aligned_ex, tails, f"{name}/{label}")
        for n in ("out", "lse", "skip_counts"):
            assert torch.equal(aligned[n], tails[n]), f"{name}/{label}: production {n} differs"
        skipped = int((tails["tile_state"] == 2).sum())
        print(f"[tail-agree {name}] {label}: identical, {skipped} tiles skipped", flush=True)
        if label != "dense":
            assert skipped > 0
