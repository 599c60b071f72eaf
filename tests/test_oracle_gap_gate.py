"""Pins of the oracle's gap gate (the running-maximum gate of the related
methods, Sec. 3 "Related Work" of "Block Sparse Flash Attention") against
things other than itself (CPU only):

* an infinite gap skips nothing: the oracle must equal a library attention
  routine (torch scaled_dot_product_attention, float64);
* a pure-Python streaming loop that keeps the running maximum of the kept
  tiles itself (App. B.2 loop order) agrees to 1e-12;
* closed form for uniform scores: a non-negative gap keeps everything, a
  negative gap keeps the first visited tile and the diagonal only;
* invariants: the decisions do not change when every score of the query
  block is shifted by the same constant (unlike the stored-threshold gate),
  and a larger gap never skips more.
"""

import numpy as np
import pytest
import torch

import oracle
from block_sparse_flashattention_tiled_amd import workloads as wl
from brute_stream import brute_stream


def _inputs(seed, B, Hq, Hkv, N, d, scale=1.0):
    rng = np.random.default_rng(seed)
    q = wl.f32_to_bf16_bits(rng.standard_normal((B, Hq, N, d), dtype=np.float32) * np.float32(scale))
    k = wl.f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, d), dtype=np.float32) * np.float32(scale))
    v = wl.f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, d), dtype=np.float32))
    return q, k, v


def _nested(x):
    return oracle.to_f64(x).tolist()


@pytest.mark.parametrize("causal", [True, False])
def test_infinite_gap_is_dense_library_attention(causal):
    B, Hq, Hkv, N, d, blk = 1, 4, 2, 384, 64, 64
    q, k, v = _inputs(11, B, Hq, Hkv, N, d, scale=1.5)
    thr = np.full((Hq, 1), np.inf)
    r = oracle.run(q, k, v, thr, causal, blk, gate_mode="gap")
    assert (r["skip_counts"] == 0).all()
    G = Hq // Hkv
    qt = torch.from_numpy(oracle.to_f64(q))
    kt = torch.from_numpy(oracle.to_f64(k)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(oracle.to_f64(v)).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal).numpy()
    np.testing.assert_allclose(r["out"], ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize(
    "causal,B,Hq,Hkv,N,d,t_len,seed",
    [
        (True, 1, 2, 1, 256, 16, 4, 21),
        (False, 1, 2, 2, 256, 16, 1, 22),
        (True, 2, 1, 1, 256, 32, 2, 23),
    ],
)
def test_gap_gate_matches_brute_force_streaming(causal, B, Hq, Hkv, N, d, t_len, seed):
    blk = 64
    q, k, v = _inputs(seed, B, Hq, Hkv, N, d, scale=1.5)
    rng = np.random.default_rng(seed + 100)
    thr = rng.uniform(0.2, 1.5, size=(Hq, t_len))  # gaps in the scaled-score domain
    r = oracle.run(q, k, v, thr, causal, blk, gate_mode="gap")
    bo, bl, bs, _ = brute_stream(_nested(q), _nested(k), _nested(v), thr.tolist(), causal, blk, gate="gap")
    assert (np.array(bs) == r["skip_counts"]).all()
    assert r["skip_counts"].sum() > 0, "case should exercise the gate"
    np.testing.assert_allclose(np.array(bo), r["out"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(np.array(bl), r["lse"], atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [True, False])
def test_uniform_scores_closed_form(causal):
    # Q = 0: every score is 0, every tile max is 0.  Gap >= 0: 0 < 0 - gap never
    # holds, nothing is skipped.  Gap < 0: the first visited tile is kept
    # (nothing kept before it), then every off-diagonal tile is skipped.
    B, Hq, Hkv, N, d, blk = 1, 1, 1, 256, 16, 64
    _, k, v = _inputs(31, B, Hq, Hkv, N, d)
    q = np.zeros((B, Hq, N, d), dtype=np.uint16)
    M = N // blk
    vf = oracle.to_f64(v)[0, 0]
    r = oracle.run(q, k, v, np.full((Hq, 1), 0.25), causal, blk, gate_mode="gap")
    assert (r["skip_counts"] == 0).all()
    r = oracle.run(q, k, v, np.full((Hq, 1), -0.25), causal, blk, gate_mode="gap")
    for i in range(M):
        # key block 0 is visited first and kept (for i = 0 it is the diagonal);
        # every later off-diagonal block is skipped; the diagonal always passes
        n_off = i if causal else M - 1
        kept_off = 1 if i > 0 else 0
        assert r["skip_counts"][0, 0, i] == n_off - kept_off
        keys = set(range(0, blk)) | set(range(i * blk, (i + 1) * blk))
        for a in range(blk):
            qpos = i * blk + a
            vis = sorted(kk for kk in keys if not causal or kk <= qpos)
            np.testing.assert_allclose(r["out"][0, 0, qpos], vf[vis].mean(axis=0), atol=1e-12, rtol=0)


def test_decisions_invariant_under_a_common_shift():
    rng = np.random.default_rng(41)
    for _ in range(200):
        n = int(rng.integers(1, 20))
        i = int(rng.integers(0, n))
        row = rng.normal(0, 3, n)
        gap = float(rng.uniform(0, 4))
        base = oracle.gate_gap(row, [i], gap)
        for c in (-7.25, 3.5, 120.0):  # exact shifts in binary: no rounding flips a comparison
            assert (oracle.gate_gap(row + c, [i], gap) == base).all()
        # the stored-threshold gate is not shift invariant, so this is a property of the gap reading
    row = np.array([0.0, 2.0, 1.0])
    assert oracle.gate(row, [2], 0.5).tolist() != oracle.gate(row + 3.0, [2], 0.5).tolist()


def test_larger_gap_never_skips_more():
    rng = np.random.default_rng(43)
    for _ in range(200):
        n = int(rng.integers(2, 24))
        i = int(rng.integers(0, n))
        row = rng.normal(0, 2, n)
        gaps = np.sort(rng.uniform(-1, 5, 4))
        skips = [oracle.gate_gap(row, [i], g) for g in gaps]
        for a, b in zip(skips, skips[1:]):
            assert not (b & ~a).any()
        assert not skips[0][i] and not skips[-1][i]  # diagonal bypass
