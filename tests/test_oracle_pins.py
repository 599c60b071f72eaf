"""Pins of the CPU oracle against things other than itself (CPU only).

* threshold -inf everywhere: nothing is skipped, so the oracle must equal a
  library attention routine (torch's scaled_dot_product_attention, float64);
* threshold +inf everywhere: only diagonal tiles survive, i.e. block-diagonal
  attention, again checked block by block against the library routine;
* a pure-Python streaming loop (App. B.2 steps with the Sec. 4.4 gate);
* closed forms for uniform scores and the strict '<' tie rule;
* invariants: monotone in the threshold, skipped V rows never read, head
  permutation within a group, planted needles dominate their query.
"""

import math

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


def _sdpa(qf, kf, vf, causal):
    """torch SDPA in float64 on the CPU with KV heads expanded contiguously."""
    G = qf.shape[1] // kf.shape[1]
    qt = torch.from_numpy(qf)
    kt = torch.from_numpy(kf).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(vf).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal).numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_dense_threshold_equals_library_attention(causal):
    B, Hq, Hkv, N, d, blk = 2, 4, 2, 384, 64, 64
    q, k, v = _inputs(1, B, Hq, Hkv, N, d)
    thr = np.full((Hq, N // blk), -np.inf)
    r = oracle.run(q, k, v, thr, causal, blk)
    qf, kf, vf = oracle.to_f64(q), oracle.to_f64(k), oracle.to_f64(v)
    ref = _sdpa(qf, kf, vf, causal)
    np.testing.assert_allclose(r["out"], ref, atol=1e-12, rtol=0)
    assert (r["skip_counts"] == 0).all()
    # lse against torch.logsumexp of the (masked) score matrix
    G = Hq // Hkv
    s = torch.from_numpy(qf) @ torch.from_numpy(kf).repeat_interleave(G, 1).transpose(-1, -2) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(r["lse"], torch.logsumexp(s, -1).numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [True, False])
def test_infinite_threshold_is_block_diagonal_attention(causal):
    B, Hq, Hkv, N, d, blk = 1, 2, 1, 256, 32, 64
    q, k, v = _inputs(2, B, Hq, Hkv, N, d)
    M = N // blk
    thr = np.full((Hq, 1), np.inf)
    r = oracle.run(q, k, v, thr, causal, blk)
    qf, kf, vf = oracle.to_f64(q), oracle.to_f64(k), oracle.to_f64(v)
    for i in range(M):
        sl = slice(i * blk, (i + 1) * blk)
        ref = _sdpa(qf[:, :, sl], kf[:, :, sl], vf[:, :, sl], causal)
        np.testing.assert_allclose(r["out"][:, :, sl], ref, atol=1e-12, rtol=0)
    expect = np.arange(M) if causal else np.full(M, M - 1)
    assert (r["skip_counts"] == expect[None, None, :]).all()
    diag = np.eye(M, dtype=bool)
    assert (r["tile_state"][..., diag] == oracle.STATE_DIAGONAL).all()


def _nested(x):
    return oracle.to_f64(x).tolist()


def test_bf16_decode_matches_library_conversion():
    # every bf16 bit pattern decodes exactly as torch's bfloat16 -> float64
    # conversion does (NaN patterns to NaN, signed zeros kept)
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127  # exponent all ones, non-zero mantissa, either sign
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    # closed forms: sign, 8 exponent bits (bias 127), 7 mantissa bits
    assert oracle.to_f64(np.array([0x3F80, 0xC000, 0x3FC0, 0x0001, 0x7F7F, 0x7F80, 0xFF80], np.uint16)).tolist() == [
        1.0, -2.0, 1.5, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, math.inf, -math.inf]
    # float inputs pass through unchanged
    x = np.array([1.5, -2.25, np.inf, 3.0e-40], dtype=np.float32)
    assert np.array_equal(oracle.to_f64(x), x.astype(np.float64))


def _position_mask_sdpa(qf, kf, vf, skip, causal, bm, bn):
    """SDPA (float64, CPU) under a boolean mask built from positions: key k takes
    part for query q iff it is visible and tile (q // bm, k // bn) is not in
    ``skip`` [B, H_q, M_Q, M_KV]."""
    B, Hq, N, _ = qf.shape
    G = Hq // kf.shape[1]
    pos = np.arange(N)
    allowed = ~skip[:, :, pos[:, None] // bm, pos[None, :] // bn]
    if causal:
        allowed &= (pos[None, :] <= pos[:, None])[None, None]
    kt = torch.from_numpy(kf).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(vf).repeat_interleave(G, dim=1)
    mask = torch.from_numpy(allowed)
    out = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(qf), kt, vt, attn_mask=mask).numpy()
    s = torch.from_numpy(qf) @ kt.transpose(-1, -2) / math.sqrt(qf.shape[-1])
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), -1).numpy()
    return out, lse


@pytest.mark.parametrize("causal,N,block", [(True, 256, 64), (False, 256, 64), (True, 200, (64, 32)),
                                            (False, 224, (32, 64))])
def test_mask_override_equals_library_attention_under_the_mask(causal, N, block):
    # an externally supplied mask (the GPU's decisions on near-threshold tiles)
    # replaces the gate: the oracle must equal SDPA under that mask
    B, Hq, Hkv, d = 2, 4, 2, 32
    bm, bn = oracle.tile_shape(block)
    M, M_kv = -(-N // bm), -(-N // bn)
    q, k, v = _inputs(11, B, Hq, Hkv, N, d)
    rng = np.random.default_rng(12)
    skip = rng.random((B, Hq, M, M_kv)) < 0.5
    for i in range(M):
        skip[:, :, i, oracle.diagonal_blocks(i, bm, bn, M_kv)] = False
    thr = np.full((Hq, M), -np.inf)  # the gate alone would skip nothing
    r = oracle.run(q, k, v, thr, causal, block, skip_override=skip)
    ref, ref_lse = _position_mask_sdpa(oracle.to_f64(q), oracle.to_f64(k), oracle.to_f64(v), skip, causal, bm, bn)
    np.testing.assert_allclose(r["out"], ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(r["lse"], ref_lse, atol=1e-12, rtol=0)
    computed = r["tile_state"] != oracle.STATE_PRUNED
    assert ((r["tile_state"] == oracle.STATE_SKIPPED) == (skip & computed)).all()
    assert (r["skip_counts"] == (skip & computed).sum(-1)).all()
    assert r["skip_counts"].sum() > 0
    # a diagonal tile cannot be overridden to skipped
    bad = skip.copy()
    bad[0, 0, 0, 0] = True
    with pytest.raises(ValueError):
        oracle.run(q, k, v, thr, causal, block, skip_override=bad)


@pytest.mark.parametrize(
    "causal,B,Hq,Hkv,N,d,t_len,seed",
    [
        (True, 1, 2, 1, 256, 16, 4, 3),   # full table, GQA 2
        (True, 1, 2, 2, 256, 16, 2, 4),   # table shorter than M: clamp to last entry
        (False, 1, 2, 1, 192, 16, 1, 5),  # one threshold per head, bidirectional
        (True, 2, 1, 1, 256, 64, 2, 6),   # batch of two, d = 64
    ],
)
def test_oracle_matches_brute_force_streaming(causal, B, Hq, Hkv, N, d, t_len, seed):
    blk = 64
    q, k, v = _inputs(seed, B, Hq, Hkv, N, d, scale=1.5)
    # thresholds spread across the observed tile maxima so some tiles skip
    tm = oracle.tile_maxima(q, k, causal, blk)
    M = N // blk
    off = tm[..., ~np.eye(M, dtype=bool)]
    finite = off[np.isfinite(off)]
    rng = np.random.default_rng(seed + 100)
    thr = rng.uniform(np.quantile(finite, 0.2), np.quantile(finite, 0.8), size=(Hq, t_len))
    r = oracle.run(q, k, v, thr, causal, blk)
    bo, bl, bs, bt = brute_stream(_nested(q), _nested(k), _nested(v), thr.tolist(), causal, blk)
    assert (np.array(bs) == r["skip_counts"]).all()
    bt = np.array([[[[np.nan if x is None else x for x in row] for row in hh] for hh in bb] for bb in bt])
    np.testing.assert_allclose(bt, r["tile_max"], atol=1e-12, rtol=0)  # NaN positions must agree too
    assert r["skip_counts"].sum() > 0, "case should exercise the gate"
    np.testing.assert_allclose(np.array(bo), r["out"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(np.array(bl), r["lse"], atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [True, False])
def test_uniform_scores_tie_rule_closed_form(causal):
    # Q = 0 makes every score 0, so every tile max is 0.
    B, Hq, Hkv, N, d, blk = 1, 2, 1, 256, 32, 64
    M = N // blk
    _, k, v = _inputs(7, B, Hq, Hkv, N, d)
    q = np.zeros((B, Hq, N, d), np.uint16)
    vf = oracle.to_f64(v)[0, 0]
    pos = np.arange(N)
    # tau = 0: s_max == tau is not below it, so nothing is skipped (strict '<').
    r = oracle.run(q, k, v, np.zeros((Hq, 1)), causal, blk)
    assert (r["skip_counts"] == 0).all()
    if causal:
        ref = np.cumsum(vf, axis=0) / (pos + 1)[:, None]
        ref_lse = np.log(pos + 1.0)
    else:
        ref = np.broadcast_to(vf.mean(axis=0), (N, d))
        ref_lse = np.full(N, math.log(N))
    for h in range(Hq):
        np.testing.assert_allclose(r["out"][0, h], ref, atol=1e-12)
        np.testing.assert_allclose(r["lse"][0, h], ref_lse, atol=1e-12)
    # tau just above 0: every off-diagonal tile skips; the diagonal remains.
    r = oracle.run(q, k, v, np.full((Hq, 1), 1e-6), causal, blk)
    start = (pos // blk) * blk
    for h in range(Hq):
        for qp in range(N):
            hi = qp + 1 if causal else start[qp] + blk
            np.testing.assert_allclose(r["out"][0, h, qp], vf[start[qp]:hi].mean(axis=0), atol=1e-12)
            assert abs(r["lse"][0, h, qp] - math.log(hi - start[qp])) < 1e-12
    assert (r["skip_counts"][0, 0] == (np.arange(M) if causal else M - 1)).all()


def test_threshold_table_reuses_last_entry():
    # App. B.3: positions past the table reuse its last entry.  Entry 0 = +inf
    # (skip every off-diagonal tile), entry 1 = -inf (keep all): blocks 1.. M-1
    # must then equal dense attention and block 0 is its own diagonal anyway.
    B, Hq, Hkv, N, d, blk = 1, 2, 1, 384, 32, 64
    q, k, v = _inputs(14, B, Hq, Hkv, N, d)
    thr = np.array([[np.inf, -np.inf]] * Hq)
    r = oracle.run(q, k, v, thr, True, blk)
    ref = _sdpa(oracle.to_f64(q), oracle.to_f64(k), oracle.to_f64(v), True)
    np.testing.assert_allclose(r["out"], ref, atol=1e-12, rtol=0)
    assert (r["skip_counts"] == 0).all()


def test_nan_threshold_skips_nothing():
    q, k, v = _inputs(8, 1, 1, 1, 256, 16)
    r = oracle.run(q, k, v, np.full((1, 1), np.nan), True, 64)
    r0 = oracle.run(q, k, v, np.full((1, 1), -np.inf), True, 64)
    assert (r["skip_counts"] == 0).all()
    assert np.array_equal(r["out"], r0["out"])


def test_monotone_in_threshold():
    B, Hq, Hkv, N, d, blk = 1, 2, 1, 512, 32, 64
    q, k, v = _inputs(9, B, Hq, Hkv, N, d, scale=1.5)
    prev = None
    for tau in np.linspace(0.5, 4.0, 8):
        r = oracle.run(q, k, v, np.full((Hq, 1), tau), True, blk)
        skipped = r["tile_state"] == oracle.STATE_SKIPPED
        if prev is not None:
            assert (skipped | ~prev).all() and (skipped >= prev).all()
        prev = skipped
        assert (r["skip_counts"] == skipped.sum(-1)).all()


def test_skipped_value_rows_are_never_read():
    B, Hq, Hkv, N, d, blk = 1, 1, 1, 512, 32, 64
    q, k, v = _inputs(10, B, Hq, Hkv, N, d, scale=1.5)
    thr = np.full((Hq, 1), 2.0)
    base = oracle.run(q, k, v, thr, True, blk)
    M = N // blk
    for i in range(M):
        skipped = np.flatnonzero(base["tile_state"][0, 0, i] == oracle.STATE_SKIPPED)
        if skipped.size == 0:
            continue
        vp = oracle.to_f64(v).copy()
        for j in skipped:
            vp[0, 0, j * blk:(j + 1) * blk] = np.nan
        r = oracle.run_blocks(q, k, vp, thr, True, blk, [(0, 0, i)])[0]
        sl = slice(i * blk, (i + 1) * blk)
        assert np.array_equal(r["out"], base["out"][0, 0, sl])
        assert np.array_equal(r["lse"], base["lse"][0, 0, sl])


def test_head_permutation_within_group():
    B, Hq, Hkv, N, d, blk = 1, 4, 2, 256, 16, 64
    q, k, v = _inputs(11, B, Hq, Hkv, N, d, scale=1.5)
    rng = np.random.default_rng(11)
    thr = rng.uniform(1.0, 3.0, size=(Hq, 4))
    perm = np.array([1, 0, 3, 2])  # swaps stay within groups {0,1}, {2,3}
    r = oracle.run(q, k, v, thr, True, blk)
    rp = oracle.run(q[:, perm], k, v, thr[perm], True, blk)
    assert np.array_equal(rp["out"], r["out"][:, perm])
    assert np.array_equal(rp["skip_counts"], r["skip_counts"][:, perm])


def test_planted_needles_dominate():
    w = wl.get_config("tiny")
    data = wl.generate(w, seed=0)
    thr = np.full((w.heads_q, 1), -np.inf)
    vf = oracle.to_f64(data["v"])
    for b, h, qp, kp in data["planted"]:
        i = qp // w.block
        r = oracle.run_blocks(data["q"], data["k"], data["v"], thr, True, w.block, [(b, h, i)])[0]
        o = r["out"][qp - i * w.block]
        assert np.abs(o - vf[b, h // w.group, kp]).max() < 1e-3


def test_fixed_k_calibration_retains_exactly_k():
    B, Hq, Hkv, N, d, blk = 1, 2, 1, 1024, 32, 64
    q, k, v = _inputs(12, B, Hq, Hkv, N, d, scale=1.5)
    M = N // blk
    tm = oracle.tile_maxima(q, k, True, blk)
    for kk in (0, 1, 4, 9):
        thr = oracle.calibrate_fixed_k(tm, kk, True)
        r = oracle.run(q, k, v, thr, True, blk)
        kept_off = (r["tile_state"] == oracle.STATE_KEPT).sum(-1)
        expect = np.minimum(np.arange(M), kk)
        assert (kept_off == expect[None, None, :]).all()
        assert np.isneginf(thr[:, : kk + 1]).all()


def test_calibration_averages_samples():
    rng = np.random.default_rng(13)
    M = 8
    tm = rng.normal(size=(2, 1, M, M))
    tm[:, :, np.triu_indices(M, 1)[0], np.triu_indices(M, 1)[1]] = np.nan
    t0 = oracle.calibrate_fixed_k(tm[:1], 2, True)
    t1 = oracle.calibrate_fixed_k(tm[1:], 2, True)
    t = oracle.calibrate_fixed_k(tm, 2, True)
    np.testing.assert_allclose(t, 0.5 * (t0 + t1), atol=1e-15)
    # midpoint of the 2nd and 3rd largest off-diagonal maxima of row 5, sample 0
    vals = np.sort(tm[0, 0, 5, :5])[::-1]
    assert t0[0, 5] == pytest.approx(0.5 * (vals[1] + vals[2]), abs=1e-15)
