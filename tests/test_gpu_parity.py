"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Sizes the oracle finishes in seconds but that span many tiles.  Every case
runs the diagnostic entry point (skip mask and tile maxima compared tile by
tile) and the production entry point (must be bit-identical to it).
"""

import numpy as np
import pytest
import torch

import oracle
from block_sparse_flashattention_tiled_amd import binding as bb
from block_sparse_flashattention_tiled_amd import workloads as wl
from parity_util import compare_blocks, margin_thresholds

pytestmark = pytest.mark.gpu


def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    bb.load_library()


def _run_gpu(data, thr, causal, block, diagnostics=True):
    q = bb.bits_to_device(data["q"])
    k = bb.bits_to_device(data["k"])
    v = bb.bits_to_device(data["v"])
    t = torch.from_numpy(np.ascontiguousarray(thr, dtype=np.float32)).cuda()
    r = bb.prefill(q, k, v, t, causal, block, diagnostics=diagnostics)
    torch.cuda.synchronize()
    return {n: x.cpu().numpy() for n, x in r.items()}


CASES = {
    # name: (workload overrides, k or None (= -inf), threshold mode)
    "tiny": (dict(base="tiny"), 4, "calib"),
    "llama-2k-G4-d128-b128": (dict(base="llama8k", seq_len=2048, heads_q=4, heads_kv=1), 5, "calib"),
    "llama-1k-G1-d128-b64": (dict(base="llama8k", seq_len=1024, heads_q=2, heads_kv=2, block=64), 6, "calib"),
    "llama-1k-G2-d64-b128": (dict(base="llama8k", seq_len=1024, heads_q=2, heads_kv=1, head_dim=64), 2, "calib"),
    "tiny-d64-b64-batch2": (dict(base="tiny", batch=2, seq_len=512, heads_q=4, heads_kv=2), 3, "calib"),
    "dit-noncausal-b128": (dict(base="dit32k", batch=2, heads_q=2, heads_kv=2, seq_len=1024, grid=(4, 8, 32)), 3,
                           "calib"),
    "dit-noncausal-d64-b64": (dict(base="dit32k", batch=1, heads_q=2, heads_kv=2, seq_len=512, grid=(2, 8, 32),
                                   head_dim=64, block=64), 2, "calib"),
    "dense": (dict(base="llama8k", seq_len=1024, heads_q=4, heads_kv=2), None, "calib"),
    "diagonal-only": (dict(base="llama8k", seq_len=1024, heads_q=2, heads_kv=1), None, "+inf"),
    "one-threshold-per-head": (dict(base="llama8k", seq_len=1024, heads_q=2, heads_kv=1), 3, "t_len1"),
    "table-shorter-than-M": (dict(base="llama8k", seq_len=2048, heads_q=2, heads_kv=1), 4, "t_len4"),
    "single-tile": (dict(base="llama8k", seq_len=128, heads_q=2, heads_kv=1), None, "+inf"),
    # odd groups: causal (head pairs plus causal block pairs for the last head) and bidirectional (block pairs);
    # an odd number of blocks leaves the last block pair's second block past the end
    "odd-group-causal": (dict(base="llama8k", seq_len=1024, heads_q=3, heads_kv=1), 3, "calib"),
    "odd-group-bidirectional-even-M": (dict(base="llama8k", seq_len=1024, heads_q=3, heads_kv=1, causal=False), 2,
                                       "calib"),
    "bidirectional-odd-M": (dict(base="dit32k", batch=1, heads_q=2, heads_kv=2, seq_len=896, grid=(4, 7, 32)), 2,
                            "calib"),
    # sequence lengths that are not a multiple of the tile (partial last block),
    # through every route: head pairs, block pairs (even and odd M); both tile sizes
    "ragged-headpair-causal": (dict(base="llama8k", seq_len=1000, heads_q=4, heads_kv=1), 3, "calib"),
    "ragged-blockpair-bidirectional": (dict(base="llama8k", seq_len=1000, heads_q=3, heads_kv=1, causal=False), 2,
                                       "calib"),
    "ragged-odd-group-causal": (dict(base="llama8k", seq_len=700, heads_q=3, heads_kv=1), 2, "calib"),
    "ragged-odd-M-bidirectional-d64-b64": (dict(base="tiny", seq_len=900, heads_q=2, heads_kv=2, causal=False),
                                              2, "calib"),
    "ragged-headpair-d64-b64": (dict(base="tiny", seq_len=1000), 4, "calib"),
    "ragged-single-partial-tile": (dict(base="llama8k", seq_len=77, heads_q=2, heads_kv=1), None, "+inf"),
    "ragged-dense-bidirectional": (dict(base="llama8k", seq_len=333, heads_q=2, heads_kv=2, causal=False), None,
                                   "calib"),
    # causal block pairs (two neighbouring query blocks of one head): multi-head attention (G = 1) and the last head
    # of an odd group, whose other heads run in head pairs; with odd M the last pair's second block lies past the end
    "mha-causal-blockpair": (dict(base="llama8k", seq_len=1024, heads_q=2, heads_kv=2), 3, "calib"),
    "odd-group-causal-odd-M": (dict(base="llama8k", seq_len=1152, heads_q=3, heads_kv=1), 3, "calib"),
    "ragged-blockpair-causal": (dict(base="llama8k", seq_len=1000, heads_q=1, heads_kv=1), 2, "calib"),
    "ragged-odd-group-causal-odd-M": (dict(base="llama8k", seq_len=1100, heads_q=3, heads_kv=1), 2, "calib"),
    "blockpair-causal-d64-b64": (dict(base="tiny", seq_len=640, heads_q=2, heads_kv=2), 3, "calib"),
    "mha-causal-odd-M": (dict(base="llama8k", seq_len=1152, heads_q=2, heads_kv=2), 3, "calib"),
    "odd-group-5-causal": (dict(base="llama8k", seq_len=768, heads_q=5, heads_kv=1), 2, "calib"),
    # block-pair launches over a multiple of 8 heads take the order that runs whole heads per XCD
    "mha-8-heads-causal": (dict(base="llama8k", seq_len=768, heads_q=8, heads_kv=8), 2, "calib"),
    "mha-8-heads-causal-odd-M": (dict(base="llama8k", seq_len=640, heads_q=8, heads_kv=8), 2, "calib"),
    "dit-8-heads-bidirectional": (dict(base="dit32k", batch=2, heads_q=4, heads_kv=4, seq_len=512, grid=(2, 8, 32)),
                                  2, "calib"),
    "odd-group-causal-8-groups": (dict(base="llama8k", seq_len=512, heads_q=24, heads_kv=8), 2, "calib"),
    # degenerate shapes: a single token (one partial block, only the diagonal tile), and a threshold table
    # longer than the number of query blocks (entries past the last block are never read)
    "single-token-causal": (dict(base="llama8k", seq_len=1, heads_q=2, heads_kv=1), 3, "calib"),
    "single-token-bidirectional-d64": (dict(base="tiny", seq_len=1, heads_q=2, heads_kv=1, causal=False), 3,
                                       "calib"),
    "table-longer-than-M": (dict(base="llama8k", seq_len=1024, heads_q=4, heads_kv=2), 3, "t_long"),
}


def _make(name):
    over, k, mode = CASES[name]
    over = dict(over)
    w = wl.get_config(over.pop("base"), **over)
    data = wl.generate(w, seed=0)
    tm = oracle.tile_maxima(data["q"], data["k"], w.causal, w.block)
    if mode == "+inf":
        thr = np.full((w.heads_q, 1), np.inf, dtype=np.float32)
    elif mode == "t_len1":
        full = margin_thresholds(tm, k, w.causal)
        # one value per head: the median of the finite per-block thresholds, kept away from every s_max
        thr = np.array([[np.median(r[np.isfinite(r)])] for r in full], dtype=np.float32)
        thr = _nudge(tm, thr)
    elif mode == "t_long":
        full = margin_thresholds(tm, k, w.causal)
        # entries past the last query block: -inf would keep every tile if they were read
        thr = np.ascontiguousarray(np.concatenate([full, np.full((w.heads_q, 5), -np.inf, np.float32)], axis=1))
    elif mode == "t_len4":
        full = margin_thresholds(tm, k, w.causal)
        thr = _nudge(tm, np.ascontiguousarray(full[:, 6:10]))  # entries of blocks 6..9, reused past the table
    else:
        thr = margin_thresholds(tm, k, w.causal)
    return w, data, thr


def _nudge(tm, thr, margin=2e-3):
    """Move each threshold out of the 2e-3 band around every tile max it is compared with."""
    B, H, M, _ = tm.shape
    out = thr.copy()
    for h in range(H):
        for c in range(thr.shape[1]):
            rows = range(c, M) if c == thr.shape[1] - 1 else [c]
            vals = np.concatenate([tm[:, h, i][np.isfinite(tm[:, h, i])] for i in rows])
            t = float(out[h, c])
            while np.min(np.abs(vals - t)) <= margin:
                t += margin
            out[h, c] = np.float32(t)
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_parity_against_oracle(name):
    _gpu()
    w, data, thr = _make(name)
    print(f"[case {name}] B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} N={w.seq_len} d={w.head_dim} "
          f"blk={w.block} causal={w.causal} thr={thr.shape}", flush=True)
    gpu = _run_gpu(data, thr, w.causal, w.block, diagnostics=True)
    blocks = [(b, h, i) for b in range(w.batch) for h in range(w.heads_q) for i in range(w.n_blocks)]
    ref = oracle.run_blocks(data["q"], data["k"], data["v"], thr, w.causal, w.block, blocks)
    stats = compare_blocks(gpu, ref, w.block, thr, name)
    print(f"[case {name}] {stats} skipped={int(gpu['skip_counts'].sum())}", flush=True)
    # production entry point: bit-identical outputs
    prod = _run_gpu(data, thr, w.causal, w.block, diagnostics=False)
    for n in ("out", "lse", "skip_counts"):
        assert np.array_equal(prod[n], gpu[n], equal_nan=True), n


def test_deterministic_and_skipped_v_never_read():
    _gpu()
    w, data, thr = _make("llama-2k-G4-d128-b128")
    base = _run_gpu(data, thr, w.causal, w.block, diagnostics=True)
    again = _run_gpu(data, thr, w.causal, w.block, diagnostics=True)
    for n in base:
        assert np.array_equal(base[n], again[n], equal_nan=True), f"{n} differs between identical runs"
    # poison the V rows of tiles one query block skips; that block's results must not move a bit
    G = w.group
    checked = 0
    for h, i in [(0, 15), (3, 9), (1, 12)]:
        skipped = np.flatnonzero(base["tile_state"][0, h, i] == oracle.STATE_SKIPPED)
        if skipped.size == 0:
            continue
        v = data["v"].copy()
        for j in skipped:
            v[0, h // G, j * w.block:(j + 1) * w.block] = 0x7FC0  # bf16 quiet NaN
        pois = _run_gpu(dict(data, v=v), thr, w.causal, w.block, diagnostics=True)
        sl = slice(i * w.block, (i + 1) * w.block)
        assert np.array_equal(pois["out"][0, h, sl], base["out"][0, h, sl])
        assert np.array_equal(pois["lse"][0, h, sl], base["lse"][0, h, sl])
        assert np.array_equal(pois["tile_state"][0, h, i], base["tile_state"][0, h, i])
        checked += 1
    assert checked >= 2


@pytest.mark.parametrize("name", ["llama-2k-G4-d128-b128", "dit-noncausal-b128", "tiny-d64-b64-batch2",
                                  "ragged-headpair-causal", "ragged-odd-M-bidirectional-d64-b64"])
def test_tile_max_pass(name):
    _gpu()
    w, data, thr = _make(name)
    q, k = bb.bits_to_device(data["q"]), bb.bits_to_device(data["k"])
    tm_gpu = bb.tile_max(q, k, w.causal, w.block).cpu().numpy()
    diag = _run_gpu(data, thr, w.causal, w.block, diagnostics=True)
    # the calibration pass measures exactly what the gate compares
    assert np.array_equal(tm_gpu, diag["tile_max"], equal_nan=True)
    ref = oracle.tile_maxima(data["q"], data["k"], w.causal, w.block)
    assert np.array_equal(np.isnan(tm_gpu), np.isnan(ref))
    fin = np.isfinite(ref)
    err = np.abs(tm_gpu[fin] - ref[fin])
    assert (err <= 1e-4 + 1e-5 * np.abs(ref[fin])).all(), err.max()


@pytest.mark.parametrize("causal", [True, False])
def test_calibration_kernel_matches_oracle(causal):
    _gpu()
    rng = np.random.default_rng(5)
    S, H, M = 2, 3, 40
    tm = rng.normal(size=(S, H, M, M)).astype(np.float32)
    if causal:
        tm[:, :, np.triu_indices(M, 1)[0], np.triu_indices(M, 1)[1]] = np.nan
    dev = torch.from_numpy(tm).cuda()
    for k in (0, 1, 3, 7, M - 2, M - 1, M + 5):
        got = bb.calibrate_fixed_k(dev, k, causal).cpu().numpy()
        want = oracle.calibrate_fixed_k(tm.astype(np.float64), k, causal)
        assert np.array_equal(np.isneginf(got), np.isneginf(want)), k
        assert np.array_equal(np.isposinf(got), np.isposinf(want)), k
        fin = np.isfinite(want)
        np.testing.assert_allclose(got[fin], want[fin], rtol=2e-7, atol=1e-7, err_msg=f"k={k}")


def test_gpu_calibration_keeps_exactly_k():
    _gpu()
    w = wl.get_config("llama8k", seq_len=4096, heads_q=4, heads_kv=1)
    data = wl.generate(w, seed=3)
    q, k, v = (bb.bits_to_device(data[n]) for n in ("q", "k", "v"))
    tm = bb.tile_max(q, k, w.causal, w.block)
    tmn = tm.cpu().numpy()
    M = w.n_blocks
    for kk in (2, 9):
        thr = bb.calibrate_fixed_k(tm, kk, w.causal)
        res = bb.prefill(q, k, v, thr, w.causal, w.block)
        counts = res["skip_counts"].cpu().numpy()[0]
        want = np.maximum(np.arange(M) - kk, 0)
        for h in range(w.heads_q):
            for i in range(M):
                if counts[h, i] == want[i]:
                    continue
                vals = np.sort(tmn[0, h, i, :i])[::-1]
                # only a near-tie between the k-th and (k+1)-th maxima may shift the count by one
                assert abs(int(counts[h, i]) - int(want[i])) == 1
                assert np.spacing(np.float32(vals[kk])) * 2 >= abs(vals[kk - 1] - vals[kk])
