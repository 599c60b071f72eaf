"""GPU parity of bsfa_prefill_varlen (a padded batch of sequences of different
lengths, each attended alone) through the C ABI:

* every sequence against the oracle run on that sequence alone (mask exact:
  thresholds kept 2e-3 away from every tile maximum of every sequence);
* every sequence bit-identical to bsfa_prefill on a copy of that sequence;
* diagnostics past a sequence's last key block read as not computed;
* routes: head pairs (causal); block pairs whose second block lies past the end
  of a sequence (bidirectional); an odd group under causal masking (head pairs
  plus causal block pairs for its last head), also with an odd number of query
  blocks; a sequence of length 0.
"""

import numpy as np
import pytest
import torch

import oracle
from block_sparse_flashattention_tiled_amd import binding as bb
from block_sparse_flashattention_tiled_amd import workloads as wl
from parity_util import away_from, compare_blocks

pytestmark = pytest.mark.gpu

CASES = {
    "headpair-causal": (dict(base="llama8k", batch=3, seq_len=1024, heads_q=4, heads_kv=1), [1000, 257, 640], 3),
    "blockpair-bidirectional": (dict(base="llama8k", batch=3, seq_len=1024, heads_q=3, heads_kv=1, causal=False),
                                [900, 300, 1024], 2),
    "odd-group-with-empty": (dict(base="tiny", batch=3, seq_len=640, heads_q=3, heads_kv=1), [0, 640, 333], 3),
    "odd-group-odd-M": (dict(base="tiny", batch=3, seq_len=576, heads_q=3, heads_kv=1), [576, 0, 300], 3),
    # 2 x 4 heads: block pairs in the order that runs whole heads per XCD
    "mha-8-head-slots-causal": (dict(base="llama8k", batch=2, seq_len=640, heads_q=4, heads_kv=4), [640, 390], 2),
}


def _thresholds(data, lens, w, k):
    """Fixed-k thresholds [H, M] from the longest sequence, moved 2e-3 away from
    every tile maximum of every sequence."""
    M = w.n_blocks
    tms = []
    for b, n in enumerate(lens):
        if n == 0:
            continue
        tms.append(oracle.tile_maxima(data["q"][b:b + 1, :, :n], data["k"][b:b + 1, :, :n], w.causal, w.block)[0])
    longest = int(np.argmax(lens))
    n = lens[longest]
    base = oracle.calibrate_fixed_k(
        oracle.tile_maxima(data["q"][longest:longest + 1, :, :n], data["k"][longest:longest + 1, :, :n], w.causal,
                           w.block), k, w.causal)
    thr = np.full((w.heads_q, M), -np.inf, dtype=np.float32)
    thr[:, :base.shape[1]] = base
    for h in range(w.heads_q):
        for i in range(M):
            vals = np.concatenate([t[h, i][np.isfinite(t[h, i])] for t in tms if i < t.shape[1]] + [np.zeros(0)])
            thr[h, i] = np.float32(away_from(float(thr[h, i]), vals))
    return thr


@pytest.mark.parametrize("name", list(CASES))
def test_varlen_matches_oracle_and_single_sequences(name):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    bb.load_library()
    over, lens, k = CASES[name]
    over = dict(over)
    w = wl.get_config(over.pop("base"), **over)
    data = wl.generate(w, seed=0)
    thr = _thresholds(data, lens, w, k)
    q, kk, v = (bb.bits_to_device(data[n]) for n in ("q", "k", "v"))
    t = torch.from_numpy(thr).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    print(f"[varlen {name}] lens={lens} M={w.n_blocks} blk={w.block} causal={w.causal}", flush=True)
    var = bb.prefill_varlen(q, kk, v, t, w.causal, w.block, sl, diagnostics=True)
    prod = bb.prefill_varlen(q, kk, v, t, w.causal, w.block, sl)
    torch.cuda.synchronize()
    g = {n: x.cpu().numpy() for n, x in var.items()}
    pr = {n: x.cpu().numpy() for n, x in prod.items()}
    skipped = 0
    for b, n in enumerate(lens):
        if n == 0:
            continue
        Mb = -(-n // w.block)
        rows = slice(0, n)
        # production entry point: identical to the diagnostic one inside the sequence
        assert np.array_equal(pr["out"][b, :, rows], g["out"][b, :, rows])
        assert np.array_equal(pr["lse"][b, :, rows], g["lse"][b, :, rows])
        assert np.array_equal(pr["skip_counts"][b, :, :Mb], g["skip_counts"][b, :, :Mb])
        # the same sequence alone, through bsfa_prefill_ex
        one = bb.prefill(bb.bits_to_device(np.ascontiguousarray(data["q"][b:b + 1, :, :n])),
                         bb.bits_to_device(np.ascontiguousarray(data["k"][b:b + 1, :, :n])),
                         bb.bits_to_device(np.ascontiguousarray(data["v"][b:b + 1, :, :n])),
                         t[:, :Mb].contiguous(), w.causal, w.block, diagnostics=True)
        torch.cuda.synchronize()
        one = {x: y.cpu().numpy()[0] for x, y in one.items()}
        assert np.array_equal(one["out"], g["out"][b, :, rows]), f"b={b}: out differs from the lone sequence"
        assert np.array_equal(one["lse"], g["lse"][b, :, rows])
        assert np.array_equal(one["skip_counts"], g["skip_counts"][b, :, :Mb])
        assert np.array_equal(one["tile_state"], g["tile_state"][b, :, :Mb, :Mb])
        assert np.array_equal(one["tile_max"], g["tile_max"][b, :, :Mb, :Mb], equal_nan=True)
        # key blocks past the end of the sequence: not computed
        assert (g["tile_state"][b, :, :Mb, Mb:] == oracle.STATE_PRUNED).all()
        assert np.isnan(g["tile_max"][b, :, :Mb, Mb:]).all()
        # the oracle on this sequence alone
        blocks = [(0, h, i) for h in range(w.heads_q) for i in range(Mb)]
        ref = oracle.run_blocks(data["q"][b:b + 1, :, :n], data["k"][b:b + 1, :, :n], data["v"][b:b + 1, :, :n],
                                thr[:, :Mb], w.causal, w.block, blocks)
        gb = {x: g[x][b:b + 1, :, :n] if x in ("out", "lse") else g[x][b:b + 1, :, :Mb] for x in
              ("out", "lse", "skip_counts")}
        gb["tile_state"] = g["tile_state"][b:b + 1, :, :Mb, :Mb]
        gb["tile_max"] = g["tile_max"][b:b + 1, :, :Mb, :Mb]
        stats = compare_blocks(gb, ref, w.block, thr[:, :Mb], label=f"{name} b={b}")
        skipped += int(gb["skip_counts"].sum())
        print(f"[varlen {name}] b={b} n={n} {stats}", flush=True)
    assert skipped > 0


def test_varlen_writes_nothing_past_each_sequence():
    # outputs start as sentinels: rows past a sequence's end, counts of query blocks past its last block, and
    # everything of an empty sequence must keep them
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    bb.load_library()
    over, lens, k = CASES["odd-group-with-empty"]
    over = dict(over)
    w = wl.get_config(over.pop("base"), **over)
    data = wl.generate(w, seed=0)
    thr = _thresholds(data, lens, w, k)
    q, kk, v = (bb.bits_to_device(data[n]) for n in ("q", "k", "v"))
    B, H, N, d = w.batch, w.heads_q, w.seq_len, w.head_dim
    M = w.n_blocks
    out = torch.full((B, H, N, d), 1234.5, dtype=torch.float32, device="cuda")
    lse = torch.full((B, H, N), -777.0, dtype=torch.float32, device="cuda")
    counts = torch.full((B, H, M), -5, dtype=torch.int32, device="cuda")
    shape = bb.make_shape(B, H, w.heads_kv, N, d, thr.shape[1])
    bb.bsfa_prefill_varlen(q, kk, v, out, lse, counts, torch.from_numpy(thr).cuda(), shape, int(w.causal),
                           bb.make_block(w.block), torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    o, l, c = out.cpu().numpy(), lse.cpu().numpy(), counts.cpu().numpy()
    for b, n in enumerate(lens):
        Mb = -(-n // w.block)
        assert (o[b, :, n:] == np.float32(1234.5)).all() and (l[b, :, n:] == np.float32(-777.0)).all()
        assert (c[b, :, Mb:] == -5).all()
        assert np.isfinite(o[b, :, :n]).all() and (c[b, :, :Mb] >= 0).all()
