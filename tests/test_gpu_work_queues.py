"""The pipelined kernel's work queues on the GPU: slots reused, streams
overlapping.

Every 128 x 128, d = 128 forward launch takes the next slot of the library's
ring of 1,024 work-counter slots and zeroes it on its stream first.  These
tests check what that must guarantee, on outputs filled with NaN before each
launch, so that an item taken twice or never shows:

* more launches than the ring has slots, alternating a larger and a smaller
  layer on one stream, each output equal bit for bit to that layer's first;
* launches of two layers enqueued alternately on two streams without
  synchronisation between them, equal to the same launches run one by one;
* a launch captured in a graph and replayed, equal to the eager launch.
"""

import pytest
import torch

from block_sparse_flashattention_tiled_amd import accounting as acc
from block_sparse_flashattention_tiled_amd import binding as bb
from block_sparse_flashattention_tiled_amd import workloads as wl

pytestmark = pytest.mark.gpu

RING_SLOTS = 1024


def _layer(seq_len, heads_q, heads_kv, causal, seed):
    w = wl.get_config("llama8k", batch=1, seq_len=seq_len, heads_q=heads_q, heads_kv=heads_kv, causal=causal)
    data = wl.generate(w, seed=seed)
    q, k, v = (bb.bits_to_device(data[n]) for n in ("q", "k", "v"))
    tile = (w.block, w.block)
    tmax = bb.tile_max(q, k, w.causal, tile)
    kk = acc.grid_k_for_target(w.seq_len, w.block, w.block, 0.5, w.causal)
    thr = bb.calibrate(tmax, [kk], w.causal, tile, w.seq_len, w.head_dim)[0].contiguous()
    M = w.n_blocks
    return dict(w=w, q=q, k=k, v=v, thr=thr, shape=bb.make_shape(1, heads_q, heads_kv, seq_len, w.head_dim, M),
                block=bb.make_block(w.block),
                out=torch.empty((1, heads_q, seq_len, w.head_dim), device="cuda"),
                lse=torch.empty((1, heads_q, seq_len), device="cuda"),
                cnt=torch.empty((1, heads_q, M), dtype=torch.int32, device="cuda"))


def _launch(L, stream=None):
    L["out"].fill_(float("nan"))
    L["lse"].fill_(float("nan"))
    L["cnt"].fill_(-1)
    bb.bsfa_prefill(L["q"], L["k"], L["v"], L["out"], L["lse"], L["cnt"], L["thr"], L["shape"],
                    int(L["w"].causal), L["block"], stream)


def _snap(L):
    return L["out"].clone(), L["lse"].clone(), L["cnt"].clone()


def _same(L, ref, label):
    out, lse, cnt = ref
    assert torch.equal(L["out"], out), f"{label}: out differs"
    assert torch.equal(L["lse"], lse), f"{label}: lse differs"
    assert torch.equal(L["cnt"], cnt), f"{label}: skip counts differ"


def test_ring_slots_reused():
    assert torch.cuda.is_available()
    big = _layer(1024, 4, 2, True, seed=11)   # 16 work items: 2 head pairs x 8 query blocks
    small = _layer(384, 2, 1, True, seed=12)  # 3 work items: 1 head pair x 3 query blocks
    _launch(big)
    _launch(small)
    torch.cuda.synchronize()
    ref_big, ref_small = _snap(big), _snap(small)
    assert bool(torch.isfinite(ref_big[0]).all()) and bool(torch.isfinite(ref_small[0]).all())
    n = RING_SLOTS // 2 + 40  # two launches per round: the ring comes round and past its start
    for r in range(n):
        _launch(big)
        _launch(small)
        if r % 64 == 0 or r == n - 1:
            torch.cuda.synchronize()
            _same(big, ref_big, f"round {r}, larger layer")
            _same(small, ref_small, f"round {r}, smaller layer")
    print(f"[work-queues] {2 * n + 2} launches, outputs identical", flush=True)


@pytest.mark.parametrize("causal", [True, False])
def test_streams_overlap(causal):
    assert torch.cuda.is_available()
    a = _layer(4096, 8, 2, causal, seed=21)   # head pairs
    b = _layer(2048, 3, 1, causal, seed=22)   # head pairs and block pairs (causal), block pairs (bidirectional)
    _launch(a)
    _launch(b)
    torch.cuda.synchronize()
    ref_a, ref_b = _snap(a), _snap(b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for r in range(8):
        with torch.cuda.stream(s1):
            _launch(a, s1)
        with torch.cuda.stream(s2):
            _launch(b, s2)
    torch.cuda.synchronize()
    _same(a, ref_a, "stream 1")
    _same(b, ref_b, "stream 2")


def test_graph_replays():
    # a captured forward (the counter-zeroing kernel and the persistent kernel,
    # no memset node) replayed several times, with eager work and
    # synchronisation between the replays, each replay equal to the eager run
    assert torch.cuda.is_available()
    L = _layer(2048, 4, 2, True, seed=31)
    _launch(L)
    torch.cuda.synchronize()
    ref = _snap(L)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            bb.bsfa_prefill(L["q"], L["k"], L["v"], L["out"], L["lse"], L["cnt"], L["thr"], L["shape"],
                            int(L["w"].causal), L["block"], side)
    torch.cuda.synchronize()
    for r in range(4):
        L["out"].fill_(float("nan"))
        L["lse"].fill_(float("nan"))
        L["cnt"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(L, ref, f"replay {r}")
        _launch(L)  # eager work between the replays
        torch.cuda.synchronize()
        _same(L, ref, f"eager run after replay {r}")
