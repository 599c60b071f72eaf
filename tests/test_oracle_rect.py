"""Pins of the oracle on rectangular tiles, B_M != B_N (CPU only).

"Block Sparse Flash Attention" runs its A100 kernel on 128 x 64 tiles
(Sec. 5.1) and its H100 port on 128 x 224 (App. A.3); which tiles are
"diagonal" there is not stated.  The reading pinned here: the key blocks
whose positions overlap the query block's.  The pins reach the oracle from
outside its own index arithmetic:

* threshold -inf: torch scaled_dot_product_attention (float64), whatever the tile;
* threshold +inf: attention restricted to the keys sharing a tile with the
  query's own position, the allowed (query block, key block) pairs read off
  the positions themselves, against the library routine with that mask;
* the pure-Python streaming loop (App. B.2 steps with the Sec. 4.4 gate),
  which finds diagonal tiles by enumerating positions;
* the tile maxima of 2b x b and b x 2b tiles are maxima of the b x b ones;
* a fixed-k table keeps exactly min(k, n_i) off-diagonal tiles per query block.
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


def _sdpa(q, k, v, causal=False, mask=None):
    qf, kf, vf = (oracle.to_f64(x) for x in (q, k, v))
    G = qf.shape[1] // kf.shape[1]
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qf), torch.from_numpy(kf).repeat_interleave(G, 1),
        torch.from_numpy(vf).repeat_interleave(G, 1), is_causal=causal,
        attn_mask=None if mask is None else torch.from_numpy(mask)).numpy()


def _shared_tiles(N, bm, bn):
    """(query block, key block) pairs that hold a common position."""
    return {(p // bm, p // bn) for p in range(N)}


@pytest.mark.parametrize("causal,N,tile", [(True, 256, (64, 32)), (False, 200, (32, 64)), (True, 150, (64, 32)),
                                           (False, 130, (64, 32)), (True, 190, (32, 64)), (True, 100, (48, 32))])
def test_dense_rect_equals_library_attention(causal, N, tile):
    q, k, v = _inputs(61, 1, 4, 2, N, 16)
    bm, bn = tile
    r = oracle.run(q, k, v, np.full((4, 1), -np.inf), causal, tile)
    M, M_kv = -(-N // bm), -(-N // bn)
    assert r["out"].shape == (1, 4, N, 16) and r["skip_counts"].shape == (1, 4, M)
    assert r["tile_max"].shape == (1, 4, M, M_kv) and r["tile_state"].shape == (1, 4, M, M_kv)
    np.testing.assert_allclose(r["out"], _sdpa(q, k, v, causal), atol=1e-12, rtol=0)
    assert (r["skip_counts"] == 0).all()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N,tile", [(256, (64, 32)), (200, (64, 32)), (256, (32, 64)), (170, (32, 64)),
                                    (150, (48, 32))])
def test_infinite_threshold_keeps_the_tiles_sharing_a_position(causal, N, tile):
    bm, bn = tile
    q, k, v = _inputs(62, 1, 2, 1, N, 16)
    r = oracle.run(q, k, v, np.full((2, 1), np.inf), causal, tile)
    pairs = _shared_tiles(N, bm, bn)
    pos = np.arange(N)
    allowed = np.array([[(a // bm, c // bn) in pairs for c in pos] for a in pos])
    if causal:
        allowed &= pos[None, :] <= pos[:, None]
    np.testing.assert_allclose(r["out"], _sdpa(q, k, v, mask=allowed), atol=1e-12, rtol=0)
    # skip counts: every computed tile that shares no position with the query block
    M, M_kv = -(-N // bm), -(-N // bn)
    for i in range(M):
        computed = [j for j in range(M_kv)
                    if not causal or any(c <= a for a in range(i * bm, min((i + 1) * bm, N))
                                         for c in range(j * bn, min((j + 1) * bn, N)))]
        expect = sum(1 for j in computed if (i, j) not in pairs)
        assert (r["skip_counts"][:, :, i] == expect).all()
        st = r["tile_state"][0, 0, i]
        assert sorted(np.flatnonzero(st == oracle.STATE_DIAGONAL)) == sorted(j for (a, j) in pairs if a == i)


def _nested(x):
    return oracle.to_f64(x).tolist()


@pytest.mark.parametrize("causal,N,tile,gate", [(True, 160, (64, 32), "threshold"),
                                                (False, 150, (32, 64), "threshold"),
                                                (True, 130, (32, 64), "gap"),
                                                (False, 96, (48, 32), "threshold"),
                                                (True, 120, (32, 48), "threshold")])
def test_rect_matches_brute_force_streaming(causal, N, tile, gate):
    q, k, v = _inputs(63, 1, 2, 1, N, 8, scale=1.5)
    tm = oracle.tile_maxima(q, k, causal, tile)
    M = tm.shape[2]
    if gate == "gap":
        thr = np.full((2, M), 0.6)
    else:
        finite = tm[np.isfinite(tm)]
        thr = np.full((2, M), np.quantile(finite, 0.5))
    r = oracle.run(q, k, v, thr, causal, tile, gate_mode=gate)
    bo, bl, bs, bt = brute_stream(_nested(q), _nested(k), _nested(v), thr.tolist(), causal, tile, gate=gate)
    assert (np.array(bs) == r["skip_counts"]).all()
    assert r["skip_counts"].sum() > 0
    bt = np.array([[[[np.nan if x is None else x for x in row] for row in hh] for hh in bb] for bb in bt])
    np.testing.assert_allclose(bt, r["tile_max"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(np.array(bo), r["out"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(np.array(bl), r["lse"], atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [256, 232])
def test_rect_tile_maxima_are_maxima_of_square_ones(causal, N):
    b = 32
    q, k, _ = _inputs(64, 1, 2, 1, N, 16)
    sq = oracle.tile_maxima(q, k, causal, b)
    tall = oracle.tile_maxima(q, k, causal, (2 * b, b))   # two query blocks per tile
    wide = oracle.tile_maxima(q, k, causal, (b, 2 * b))   # two key blocks per tile
    # np.fmax ignores NaN (a tile not computed) unless both are NaN
    exp_tall = np.stack([np.fmax.reduce(sq[:, :, 2 * i: 2 * i + 2], axis=2) for i in range(tall.shape[2])], axis=2)
    exp_wide = np.stack([np.fmax.reduce(sq[:, :, :, 2 * j: 2 * j + 2], axis=3) for j in range(wide.shape[3])],
                        axis=3)
    np.testing.assert_array_equal(np.isnan(tall), np.isnan(exp_tall))
    np.testing.assert_array_equal(np.isnan(wide), np.isnan(exp_wide))
    np.testing.assert_allclose(tall, exp_tall, atol=1e-12, rtol=0)
    np.testing.assert_allclose(wide, exp_wide, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("tile", [(64, 32), (32, 64)])
def test_rect_fixed_k_keeps_exactly_k(causal, tile):
    N = 320
    q, k, v = _inputs(65, 1, 2, 1, N, 16)
    tm = oracle.tile_maxima(q, k, causal, tile)
    dense = oracle.run(q, k, v, np.full((2, 1), -np.inf), causal, tile)
    n_off = (dense["tile_state"][0] == oracle.STATE_KEPT).sum(axis=-1)  # [H, M] off-diagonal computed tiles
    for kk in (0, 1, 3):
        thr = oracle.calibrate_fixed_k(tm, kk, causal, tile)
        r = oracle.run(q, k, v, thr, causal, tile)
        kept = (r["tile_state"][0] == oracle.STATE_KEPT).sum(axis=-1)
        np.testing.assert_array_equal(kept, np.minimum(kk, n_off))
        np.testing.assert_array_equal(r["skip_counts"][0], n_off - np.minimum(kk, n_off))
