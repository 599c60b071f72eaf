"""GPU parity on rectangular tiles (B_M != B_N) through the C ABI.

The pages' A100 kernel uses 128 x 64 tiles (Sec. 5.1); the diagonal tiles
that bypass the gate are then the key blocks overlapping the query block's
positions (two 64-key blocks per 128-row query block, or one 128-key block
holding a 64-row query block).  Every case runs the diagnostic entry point
against the oracle tile by tile and the production entry point, which must
be bit-identical to it; the routes (head pairs, block pairs with even and odd
numbers of query blocks), partial last blocks, both gates, bf16 output, per-sequence
lengths, the tile-maximum pass and the calibration kernel are covered.
"""

import numpy as np
import pytest
import torch

import oracle
from block_sparse_flashattention_tiled_amd import binding as bb
from block_sparse_flashattention_tiled_amd import workloads as wl
from parity_util import OUT_MAX, away_from, compare_blocks, gap_thresholds, margin_thresholds

pytestmark = pytest.mark.gpu


def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    bb.load_library()


CASES = {
    # name: (workload overrides, tile, k (None = -inf), threshold mode)
    "headpair-causal-128x64": (dict(base="llama8k", seq_len=2048, heads_q=4, heads_kv=1), (128, 64), 8, "calib"),
    "headpair-causal-64x128": (dict(base="llama8k", seq_len=1024, heads_q=2, heads_kv=1), (64, 128), 3, "calib"),
    "headpair-causal-128x64-d64": (dict(base="tiny", seq_len=1024, heads_q=4, heads_kv=2), (128, 64), 5, "calib"),
    "headpair-causal-64x128-d64": (dict(base="tiny", seq_len=1024, heads_q=2, heads_kv=1), (64, 128), 2, "calib"),
    # odd group, causal: head pairs plus causal block pairs for the last head (M even, and M odd: the last pair's
    # second block past the end)
    "odd-group-causal-128x64": (dict(base="llama8k", seq_len=1024, heads_q=3, heads_kv=1), (128, 64), 4, "calib"),
    "odd-group-causal-64x128": (dict(base="llama8k", seq_len=1024, heads_q=3, heads_kv=1), (64, 128), 2, "calib"),
    "odd-group-causal-odd-M-128x64": (dict(base="llama8k", seq_len=1152, heads_q=3, heads_kv=1), (128, 64), 4, "calib"),
    "odd-group-causal-odd-M-64x128": (dict(base="llama8k", seq_len=1088, heads_q=3, heads_kv=1), (64, 128), 2, "calib"),
    "blockpair-causal-128x64": (dict(base="llama8k", seq_len=1024, heads_q=1, heads_kv=1), (128, 64), 5, "calib"),
    "blockpair-causal-64x128": (dict(base="llama8k", seq_len=1024, heads_q=2, heads_kv=2), (64, 128), 3, "calib"),
    "ragged-blockpair-causal-128x64-d64": (dict(base="tiny", seq_len=1000, heads_q=2, heads_kv=2), (128, 64), 4,
                                           "calib"),
    "blockpair-bidirectional-128x64": (dict(base="dit32k", batch=1, heads_q=1, heads_kv=1, seq_len=1024,
                                            grid=(4, 8, 32)), (128, 64), 5, "calib"),
    "blockpair-bidirectional-64x128": (dict(base="dit32k", batch=2, heads_q=1, heads_kv=1, seq_len=1024,
                                            grid=(4, 8, 32)), (64, 128), 3, "calib"),
    "odd-M-bidirectional-128x64": (dict(base="dit32k", batch=1, heads_q=1, heads_kv=1, seq_len=896,
                                           grid=(4, 7, 32)), (128, 64), 4, "calib"),
    "headpair-bidirectional-64x128-d64": (dict(base="tiny", seq_len=512, heads_q=2, heads_kv=1, causal=False),
                                          (64, 128), 1, "calib"),
    "dense-128x64": (dict(base="llama8k", seq_len=1024, heads_q=4, heads_kv=2), (128, 64), None, "calib"),
    "diagonal-only-128x64": (dict(base="llama8k", seq_len=1024, heads_q=2, heads_kv=1), (128, 64), None, "+inf"),
    "diagonal-only-64x128": (dict(base="llama8k", seq_len=1024, heads_q=2, heads_kv=1), (64, 128), None, "+inf"),
    # partial last blocks: N a multiple of neither side, or of only one of them
    "ragged-headpair-causal-128x64": (dict(base="llama8k", seq_len=1000, heads_q=4, heads_kv=1), (128, 64), 6,
                                      "calib"),
    "ragged-keys-only-causal-64x128": (dict(base="llama8k", seq_len=960, heads_q=2, heads_kv=1), (64, 128), 3,
                                       "calib"),
    "ragged-queries-only-bidirectional-128x64": (dict(base="llama8k", seq_len=960, heads_q=3, heads_kv=1,
                                                      causal=False), (128, 64), 4, "calib"),
    "ragged-odd-group-causal-64x128": (dict(base="llama8k", seq_len=700, heads_q=3, heads_kv=1), (64, 128), 2,
                                      "calib"),
    "ragged-bidirectional-d64-64x128": (dict(base="tiny", seq_len=900, heads_q=2, heads_kv=2, causal=False),
                                        (64, 128), 2, "calib"),
    "ragged-single-partial-tile-128x64": (dict(base="llama8k", seq_len=77, heads_q=2, heads_kv=1), (128, 64), None,
                                          "+inf"),
    "ragged-two-key-blocks-128x64": (dict(base="llama8k", seq_len=100, heads_q=2, heads_kv=1), (128, 64), None,
                                     "+inf"),
}


def _make(name):
    over, tile, k, mode = CASES[name]
    over = dict(over)
    w = wl.get_config(over.pop("base"), **over)
    data = wl.generate(w, seed=0)
    tm = oracle.tile_maxima(data["q"], data["k"], w.causal, tile)
    if mode == "+inf":
        thr = np.full((w.heads_q, 1), np.inf, dtype=np.float32)
    else:
        thr = margin_thresholds(tm, k, w.causal, block=tile)
    return w, tile, data, thr


def _dev(data):
    return tuple(bb.bits_to_device(data[n]) for n in ("q", "k", "v"))


def _run(data, thr, causal, tile, **kw):
    q, k, v = _dev(data)
    t = torch.from_numpy(np.ascontiguousarray(thr, dtype=np.float32)).cuda()
    r = bb.prefill(q, k, v, t, causal, tile, **kw)
    torch.cuda.synchronize()
    return {n: x.cpu().numpy() if x.dtype != torch.bfloat16 else x.float().cpu().numpy() for n, x in r.items()}


def _blocks(w, tile):
    M = -(-w.seq_len // tile[0])
    return [(b, h, i) for b in range(w.batch) for h in range(w.heads_q) for i in range(M)]


@pytest.mark.parametrize("name", list(CASES))
def test_rect_parity_against_oracle(name):
    _gpu()
    w, tile, data, thr = _make(name)
    print(f"[case {name}] B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} N={w.seq_len} d={w.head_dim} "
          f"tile={tile} causal={w.causal} thr={thr.shape}", flush=True)
    gpu = _run(data, thr, w.causal, tile, diagnostics=True)
    M, M_kv = -(-w.seq_len // tile[0]), -(-w.seq_len // tile[1])
    assert gpu["tile_state"].shape == (w.batch, w.heads_q, M, M_kv)
    ref = oracle.run_blocks(data["q"], data["k"], data["v"], thr, w.causal, tile, _blocks(w, tile))
    stats = compare_blocks(gpu, ref, tile, thr, name)
    print(f"[case {name}] {stats} skipped={int(gpu['skip_counts'].sum())}", flush=True)
    prod = _run(data, thr, w.causal, tile, diagnostics=False)
    for n in ("out", "lse", "skip_counts"):
        assert np.array_equal(prod[n], gpu[n], equal_nan=True), n


def test_rect_skipped_v_never_read():
    _gpu()
    w, tile, data, thr = _make("headpair-causal-128x64")
    base = _run(data, thr, w.causal, tile, diagnostics=True)
    bm, bn = tile
    checked = 0
    for h, i in [(0, 15), (3, 9), (1, 12)]:
        skipped = np.flatnonzero(base["tile_state"][0, h, i] == oracle.STATE_SKIPPED)
        if skipped.size == 0:
            continue
        v = data["v"].copy()
        for j in skipped:
            v[0, h // w.group, j * bn:(j + 1) * bn] = 0x7FC0  # bf16 quiet NaN
        pois = _run(dict(data, v=v), thr, w.causal, tile, diagnostics=True)
        sl = slice(i * bm, (i + 1) * bm)
        assert np.array_equal(pois["out"][0, h, sl], base["out"][0, h, sl])
        assert np.array_equal(pois["lse"][0, h, sl], base["lse"][0, h, sl])
        checked += 1
    assert checked >= 2


@pytest.mark.parametrize("name", ["headpair-causal-128x64", "blockpair-bidirectional-64x128",
                                  "ragged-headpair-causal-128x64", "ragged-keys-only-causal-64x128",
                                  "odd-M-bidirectional-128x64"])
def test_rect_tile_max_pass(name):
    _gpu()
    w, tile, data, thr = _make(name)
    q, k, _ = _dev(data)
    tm_gpu = bb.tile_max(q, k, w.causal, tile).cpu().numpy()
    diag = _run(data, thr, w.causal, tile, diagnostics=True)
    assert np.array_equal(tm_gpu, diag["tile_max"], equal_nan=True)
    ref = oracle.tile_maxima(data["q"], data["k"], w.causal, tile)
    assert np.array_equal(np.isnan(tm_gpu), np.isnan(ref))
    fin = np.isfinite(ref)
    err = np.abs(tm_gpu[fin] - ref[fin])
    assert (err <= 1e-4 + 1e-5 * np.abs(ref[fin])).all(), err.max()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("tile,N", [((128, 64), 2048), ((64, 128), 2048), ((128, 64), 1000), ((64, 128), 960),
                                    ((128, 128), 1000)])
def test_rect_calibration_kernel_matches_oracle(causal, tile, N):
    _gpu()
    rng = np.random.default_rng(7)
    S, H = 2, 3
    bm, bn = tile
    M, M_kv = -(-N // bm), -(-N // bn)
    tm = rng.normal(size=(S, H, M, M_kv)).astype(np.float32)
    if causal:  # tiles whose first key comes after the block's last query are not computed
        for i in range(M):
            for j in range(M_kv):
                if j * bn > min((i + 1) * bm, N) - 1:
                    tm[:, :, i, j] = np.nan
    dev = torch.from_numpy(tm).cuda()
    ks = [0, 1, 3, 7, M_kv - 3, M_kv + 5]
    got = bb.calibrate(dev, ks, causal, tile, N, 128).cpu().numpy()
    for lvl, kk in enumerate(ks):
        want = oracle.calibrate_fixed_k(tm.astype(np.float64), kk, causal, tile)
        g = got[lvl]
        assert np.array_equal(np.isneginf(g), np.isneginf(want)), kk
        assert np.array_equal(np.isposinf(g), np.isposinf(want)), kk
        fin = np.isfinite(want)
        np.testing.assert_allclose(g[fin], want[fin], rtol=2e-7, atol=1e-7, err_msg=f"k={kk}")


def test_rect_gpu_calibration_keeps_exactly_k():
    _gpu()
    w = wl.get_config("llama8k", seq_len=4096, heads_q=4, heads_kv=1)
    tile = (128, 64)
    data = wl.generate(w, seed=3)
    q, k, v = _dev(data)
    tm = bb.tile_max(q, k, w.causal, tile)
    tmn = tm.cpu().numpy()
    M = w.seq_len // 128
    thr = bb.calibrate(tm, [3, 11], w.causal, tile, w.seq_len, w.head_dim)
    for lvl, kk in enumerate((3, 11)):
        res = bb.prefill(q, k, v, thr[lvl].contiguous(), w.causal, tile)
        counts = res["skip_counts"].cpu().numpy()[0]
        want = np.maximum(2 * np.arange(M) - kk, 0)  # query block i: 2i off-diagonal key blocks
        for h in range(w.heads_q):
            for i in range(M):
                if counts[h, i] == want[i]:
                    continue
                vals = np.sort(tmn[0, h, i, :2 * i])[::-1]
                assert abs(int(counts[h, i]) - int(want[i])) == 1
                assert np.spacing(np.float32(vals[kk])) * 2 >= abs(vals[kk - 1] - vals[kk])


@pytest.mark.parametrize("name", ["headpair-causal-128x64", "blockpair-bidirectional-64x128",
                                  "ragged-headpair-causal-128x64"])
def test_rect_gap_gate(name):
    _gpu()
    w, tile, data, _ = _make(name)
    tm = oracle.tile_maxima(data["q"], data["k"], w.causal, tile)
    thr = gap_thresholds(tm, w.causal, base=1.0, block=tile)
    g = _run(data, thr, w.causal, tile, diagnostics=True, gate="gap")
    ref = oracle.run_blocks(data["q"], data["k"], data["v"], thr, w.causal, tile, _blocks(w, tile), gate_mode="gap")
    stats = compare_blocks(g, ref, tile, thr, label=name, exempt=False)
    assert int(g["skip_counts"].sum()) > 0, stats


def test_rect_bf16_output():
    _gpu()
    w, tile, data, thr = _make("ragged-headpair-causal-128x64")
    f32 = _run(data, thr, w.causal, tile)
    b16 = _run(data, thr, w.causal, tile, out_dtype=torch.bfloat16)
    want = torch.from_numpy(f32["out"]).to(torch.bfloat16).float().numpy()
    assert np.array_equal(b16["out"], want)
    assert np.array_equal(b16["lse"], f32["lse"]) and np.array_equal(b16["skip_counts"], f32["skip_counts"])
    assert np.abs(b16["out"] - f32["out"]).max() <= OUT_MAX * 4


@pytest.mark.parametrize("tile", [(128, 64), (64, 128)])
def test_rect_varlen(tile):
    _gpu()
    w = wl.get_config("llama8k", seq_len=1024, heads_q=4, heads_kv=2, batch=3)
    data = wl.generate(w, seed=9)
    lens = [1024, 700, 129]
    bm, bn = tile
    M = -(-w.seq_len // bm)
    thr = np.empty((w.heads_q, M), dtype=np.float32)
    # one table for the batch: fixed-k thresholds of the full-length sequence, moved
    # away from the tile maxima of every sequence at its own length
    tm_full = oracle.tile_maxima(data["q"][:1], data["k"][:1], w.causal, tile)
    base = oracle.calibrate_fixed_k(tm_full, 4, w.causal, tile)
    tms = [oracle.tile_maxima(data["q"][b:b + 1, :, :n], data["k"][b:b + 1, :, :n], w.causal, tile)
           for b, n in enumerate(lens)]
    for h in range(w.heads_q):
        for i in range(M):
            vals = np.concatenate([t[0, h, i][np.isfinite(t[0, h, i])] for t in tms if i < t.shape[2]])
            thr[h, i] = np.float32(away_from(float(base[h, i]), vals))
    q, k, v = _dev(data)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    t = torch.from_numpy(thr).cuda()
    r = bb.prefill_varlen(q, k, v, t, w.causal, tile, sl, diagnostics=True)
    torch.cuda.synchronize()
    g = {n: x.cpu().numpy() for n, x in r.items()}
    for b, n in enumerate(lens):
        Mb = -(-n // bm)
        sub = {key: data[key][b:b + 1, :, :n] for key in ("q", "k", "v")}
        ref = oracle.run_blocks(sub["q"], sub["k"], sub["v"], thr, w.causal, tile,
                                [(0, h, i) for h in range(w.heads_q) for i in range(Mb)])
        M_kv_b = -(-n // bn)
        gb = {"out": g["out"][b:b + 1, :, :n], "lse": g["lse"][b:b + 1, :, :n],
              "skip_counts": g["skip_counts"][b:b + 1, :, :Mb],
              "tile_state": g["tile_state"][b:b + 1, :, :Mb, :M_kv_b],
              "tile_max": g["tile_max"][b:b + 1, :, :Mb, :M_kv_b]}
        # key blocks past the sequence read as not computed
        assert (g["tile_state"][b, :, :Mb, M_kv_b:] == oracle.STATE_PRUNED).all()
        assert np.isnan(g["tile_max"][b, :, :Mb, M_kv_b:]).all()
        stats = compare_blocks(gb, ref, tile, thr, label=f"varlen {tile} b={b}")
        print(f"[varlen {tile} b={b} n={n}] {stats}", flush=True)
