"""GPU parity of the entry points beside the hot path, through the C ABI:

* bsfa_prefill_gated with the gap gate (the running-maximum gate of the
  related methods) against the oracle's ``gate_mode="gap"``, mask exact;
* bsfa_prefill_bf16: bf16 output equal to the fp32 entry point's output
  rounded to nearest even, and within tolerance of the oracle;
* bsfa_calibrate_levels: every level equal to bsfa_calibrate_fixed_k for its k
  and to the oracle's fixed-k calibration.
"""

import numpy as np
import pytest
import torch

import oracle
from block_sparse_flashattention_tiled_amd import binding as bb
from block_sparse_flashattention_tiled_amd import workloads as wl
from parity_util import OUT_MAX, compare_blocks, gap_thresholds, margin_thresholds

pytestmark = pytest.mark.gpu


def _setup(over):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    bb.load_library()
    over = dict(over)
    w = wl.get_config(over.pop("base"), **over)
    data = wl.generate(w, seed=0)
    dev = {n: bb.bits_to_device(data[n]) for n in ("q", "k", "v")}
    return w, data, dev


GAP_CASES = {
    # routes: head pairs (G even, causal), block pairs (bidirectional), head pairs plus block pairs (odd G, causal), d64/b64
    "gap-headpair-causal": dict(base="llama8k", seq_len=2048, heads_q=4, heads_kv=1),
    "gap-blockpair-bidirectional": dict(base="dit32k", batch=1, heads_q=2, heads_kv=2, seq_len=1024,
                                        grid=(4, 8, 32)),
    "gap-odd-group": dict(base="llama8k", seq_len=1024, heads_q=3, heads_kv=1),
    "gap-d64-b64": dict(base="tiny", seq_len=1024, heads_q=2, heads_kv=1),
}


@pytest.mark.parametrize("name", list(GAP_CASES))
def test_gap_gate_matches_oracle(name):
    w, data, dev = _setup(GAP_CASES[name])
    tm = oracle.tile_maxima(data["q"], data["k"], w.causal, w.block)
    thr = gap_thresholds(tm, w.causal, base=1.0)
    t = torch.from_numpy(thr).cuda()
    diag = bb.prefill(dev["q"], dev["k"], dev["v"], t, w.causal, w.block, diagnostics=True, gate="gap")
    prod = bb.prefill(dev["q"], dev["k"], dev["v"], t, w.causal, w.block, gate="gap")
    torch.cuda.synchronize()
    g = {n: x.cpu().numpy() for n, x in diag.items()}
    for n in ("out", "lse", "skip_counts"):
        assert np.array_equal(prod[n].cpu().numpy(), g[n]), f"{name}: production {n} differs from diagnostics"
    M = w.n_blocks
    blocks = [(b, h, i) for b in range(w.batch) for h in range(w.heads_q) for i in range(M)]
    ref = oracle.run_blocks(data["q"], data["k"], data["v"], thr, w.causal, w.block, blocks, gate_mode="gap")
    stats = compare_blocks(g, ref, w.block, thr, label=name, exempt=False)
    skipped = int(g["skip_counts"].sum())
    assert skipped > 0, f"{name}: the gap should skip tiles ({stats})"
    print(name, "skipped", skipped, stats)


def test_infinite_gap_equals_dense_threshold():
    w, data, dev = _setup(dict(base="llama8k", seq_len=1024, heads_q=4, heads_kv=2))
    inf = torch.full((w.heads_q, 1), float("inf"), device="cuda")
    ninf = torch.full((w.heads_q, 1), float("-inf"), device="cuda")
    a = bb.prefill(dev["q"], dev["k"], dev["v"], inf, w.causal, w.block, gate="gap")
    b = bb.prefill(dev["q"], dev["k"], dev["v"], ninf, w.causal, w.block)
    torch.cuda.synchronize()
    for n in ("out", "lse", "skip_counts"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("over,k", [
    (dict(base="llama8k", seq_len=2048, heads_q=4, heads_kv=1), 5),      # head pairs
    (dict(base="llama8k", seq_len=1024, heads_q=3, heads_kv=1), 3),      # odd group
    (dict(base="tiny", batch=2, seq_len=512, heads_q=4, heads_kv=2), 3),  # d64, b64
])
def test_bf16_output(over, k):
    w, data, dev = _setup(over)
    tm = oracle.tile_maxima(data["q"], data["k"], w.causal, w.block)
    thr = margin_thresholds(tm, k, w.causal)
    t = torch.from_numpy(thr).cuda()
    f32 = bb.prefill(dev["q"], dev["k"], dev["v"], t, w.causal, w.block)
    b16 = bb.prefill(dev["q"], dev["k"], dev["v"], t, w.causal, w.block, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # same kernel arithmetic: the bf16 output is the fp32 output rounded to nearest even
    bits_gpu = b16["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    bits_ref = wl.f32_to_bf16_bits(f32["out"].cpu().numpy())
    assert np.array_equal(bits_gpu, bits_ref)
    assert torch.equal(b16["lse"], f32["lse"]) and torch.equal(b16["skip_counts"], f32["skip_counts"])
    # against the oracle: the fp32 tolerance plus half a bf16 ulp of the value
    M = w.n_blocks
    blocks = [(b, h, i) for b in range(w.batch) for h in range(w.heads_q) for i in range(M)]
    ref = oracle.run_blocks(data["q"], data["k"], data["v"], thr, w.causal, w.block, blocks)
    out = wl.bf16_bits_to_f32(bits_gpu).astype(np.float64)
    worst = 0.0
    for r in ref:
        o = out[r["b"], r["h"], r["i"] * w.block:(r["i"] + 1) * w.block]
        half_ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(r["out"]), 1e-30))).astype(int) - 8)
        excess = np.abs(o - r["out"]) - half_ulp
        worst = max(worst, float(excess.max()))
    assert worst <= OUT_MAX, worst


def test_calibrate_levels_equals_single_levels_and_oracle():
    w, data, dev = _setup(dict(base="llama8k", seq_len=2048, heads_q=4, heads_kv=2))
    tmax = bb.tile_max(dev["q"], dev["k"], w.causal, w.block)
    ks = [0, 2, 5, 40]  # 40 > every n_i at M = 16: the whole level is -inf
    levels = bb.calibrate_levels(tmax, ks, w.causal)
    torch.cuda.synchronize()
    tm_cpu = tmax.cpu().numpy().astype(np.float64)
    for li, kk in enumerate(ks):
        single = bb.calibrate_fixed_k(tmax, kk, w.causal)
        torch.cuda.synchronize()
        assert torch.equal(levels[li], single), f"level {li}"
        ref = oracle.calibrate_fixed_k(tm_cpu, kk, w.causal)
        got = levels[li].cpu().numpy().astype(np.float64)
        same_inf = (np.isinf(ref) == np.isinf(got)) & ((ref == got) | ~np.isinf(ref))
        assert same_inf.all(), f"level {li}: infinities differ"
        fin = np.isfinite(ref)
        np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-6, atol=1e-6)
    assert np.isinf(levels[3].cpu().numpy()).all() and (levels[3].cpu().numpy() < 0).all()


TIE_CASES = {
    # head pairs (causal), block pairs (bidirectional), 128 x 64 tiles (two gates per step)
    "tie-headpair-causal": (dict(base="llama8k", seq_len=1024, heads_q=4, heads_kv=1), (128, 128)),
    "tie-blockpair-bidirectional": (dict(base="llama8k", seq_len=1024, heads_q=2, heads_kv=2, causal=False),
                                    (128, 128)),
    "tie-headpair-causal-128x64": (dict(base="llama8k", seq_len=1024, heads_q=4, heads_kv=1), (128, 64)),
}


@pytest.mark.parametrize("name", list(TIE_CASES))
def test_threshold_ties_keep_the_tile(name):
    """The threshold gate skips an off-diagonal tile iff s_max < tau, strictly.
    The thresholds here sit exactly on the kernel's own fp32 tile maxima (and
    one ulp above them), which the oracle parity cases avoid on purpose: the
    production launch and the launch that writes the tile maxima must take the
    same decisions, and those decisions must follow the strict comparison."""
    over, tile = TIE_CASES[name]
    w, data, dev = _setup(over)
    M = -(-w.seq_len // tile[0])
    dense = bb.prefill(dev["q"], dev["k"], dev["v"], torch.full((w.heads_q, M), -np.inf, device="cuda"), w.causal,
                       tile, diagnostics=True)
    torch.cuda.synchronize()
    tmax = dense["tile_max"].cpu().numpy()[0]
    state = dense["tile_state"].cpu().numpy()[0]
    off = state == 1  # computed off-diagonal tiles (all kept at -inf)
    thr = np.full((w.heads_q, M), -np.inf, dtype=np.float32)
    n_tie = 0
    for h in range(w.heads_q):
        for i in range(M):
            vals = np.sort(tmax[h, i][off[h, i]])
            if vals.size == 0:
                continue
            t = np.float32(vals[vals.size // 2])
            if (h + i) % 2:
                t = np.nextafter(t, np.float32(np.inf))  # the tile at t is now below tau: skipped
            else:
                n_tie += 1  # the tile at t equals tau: kept
            thr[h, i] = t
    assert n_tie > 0
    t = torch.from_numpy(thr).cuda()
    diag = bb.prefill(dev["q"], dev["k"], dev["v"], t, w.causal, tile, diagnostics=True)
    prod = bb.prefill(dev["q"], dev["k"], dev["v"], t, w.causal, tile)
    torch.cuda.synchronize()
    g = {n: x.cpu().numpy() for n, x in diag.items()}
    assert np.array_equal(g["tile_max"], dense["tile_max"].cpu().numpy(), equal_nan=True)
    for n in ("out", "lse", "skip_counts"):
        assert np.array_equal(prod[n].cpu().numpy(), g[n]), f"{name}: production {n} differs from diagnostics"
    want_skip = off & (tmax < thr[:, :, None])
    assert np.array_equal(g["skip_counts"][0], want_skip.sum(axis=2)), name
    assert np.array_equal(g["tile_state"][0] == 2, want_skip), name
    ties = off & (tmax == thr[:, :, None])
    assert ties.any() and (g["tile_state"][0][ties] == 1).all(), f"{name}: a tile at tau must be kept"
