"""The two forward kernels return identical bits.

An aligned layer with 128 x 128 tiles at d = 128 runs through the pipelined
kernel (``bsfa_prefill``, ``bsfa_prefill_ex``); the same layer given to
``bsfa_prefill_varlen`` with every sequence at full length runs through the
tail-handling instances: the paired kernel's for block pairs, the pipelined
kernel's own for head pairs (its tail path must not change an aligned
result either).  Both form the tile maxima with the
same MFMA chains and reductions, gate alike, and sum the softmax and P~V in
the same order, so out, lse, skip counts and the per-tile diagnostics must
agree bit for bit, at any thresholds: dense, a fixed-k point calibrated on
the GPU, and thresholds set exactly on the kernels' own tile maxima.

Routes: head pairs (causal and bidirectional) and bidirectional block pairs
(an odd group), both on the pipelined side.
"""

import pytest
import torch

from block_sparse_flashattention_tiled_amd import accounting as acc
from block_sparse_flashattention_tiled_amd import binding as bb
from block_sparse_flashattention_tiled_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = {
    "headpair-causal": dict(base="llama8k", batch=2, seq_len=1024, heads_q=8, heads_kv=2),
    "headpair-bidirectional": dict(base="llama8k", batch=1, seq_len=1024, heads_q=4, heads_kv=2, causal=False),
    "blockpair-bidirectional": dict(base="llama8k", batch=2, seq_len=768, heads_q=3, heads_kv=1, causal=False),
}


@pytest.mark.parametrize("name", list(CASES))
def test_pipelined_and_paired_kernels_agree(name):
    assert torch.cuda.is_available()
    over = dict(CASES[name])
    w = wl.get_config(over.pop("base"), **over)
    print(f"[kernels-agree {name}] generating", flush=True)
    data = wl.generate(w, seed=3)
    q, k, v = (bb.bits_to_device(data[n]) for n in ("q", "k", "v"))
    tile = (w.block, w.block)
    M = w.n_blocks
    tmax = bb.tile_max(q, k, w.causal, tile)
    kk = acc.grid_k_for_target(w.seq_len, w.block, w.block, 0.5, w.causal)
    thr_fixed = bb.calibrate(tmax, [kk], w.causal, tile, w.seq_len, w.head_dim)[0].contiguous()
    # thresholds equal to a tile maximum of each (head, query block) of batch element 0: the
    # median computed tile, which is kept (a tie), tiles below it skipped
    on_max = torch.nanmedian(tmax[0], dim=-1).values.contiguous()
    cases = {
        "dense": torch.full((w.heads_q, M), float("-inf"), device="cuda"),
        "fixed-k": thr_fixed,
        "on-maxima": on_max,
    }
    lens = torch.full((w.batch,), w.seq_len, dtype=torch.int32, device="cuda")
    for label, thr in cases.items():
        print(f"[kernels-agree {name}] {label}", flush=True)
        pipe = bb.prefill(q, k, v, thr, w.causal, tile)
        pipe_ex = bb.prefill(q, k, v, thr, w.causal, tile, diagnostics=True)
        pair = bb.prefill_varlen(q, k, v, thr, w.causal, tile, lens, diagnostics=True)
        torch.cuda.synchronize()
        for n in ("out", "lse", "skip_counts"):
            assert torch.equal(pipe[n], pair[n]), f"{name}/{label}: {n} differs between the kernels"
            assert torch.equal(pipe_ex[n], pair[n]), f"{name}/{label}: {n} (diagnostics launch) differs"
        assert torch.equal(pipe_ex["tile_state"], pair["tile_state"]), f"{name}/{label}: tile states differ"
        same = (pipe_ex["tile_max"] == pair["tile_max"]) | (torch.isnan(pipe_ex["tile_max"]) &
                                                            torch.isnan(pair["tile_max"]))
        assert bool(same.all()), f"{name}/{label}: tile maxima differ"
        skipped = int((pair["tile_state"] == 2).sum())
        print(f"[kernels-agree {name}] {label}: identical, {skipped} tiles skipped", flush=True)
        if label != "dense":
            assert skipped > 0
