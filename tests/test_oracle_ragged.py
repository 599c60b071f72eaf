"""Pins of the oracle on sequence lengths that are not a multiple of the tile
(the last query block and key block are partial; positions >= N do not
exist), CPU only:

* threshold -inf: equals torch scaled_dot_product_attention (float64) over
  exactly N positions;
* threshold +inf: block-diagonal attention with a partial last block, block
  by block against the library routine;
* the pure-Python streaming loop (App. B.2 steps with the Sec. 4.4 gate) on
  the same ragged shapes;
* prefix consistency under causal masking: with every tile kept, the ragged
  run on the first N positions of an aligned sequence equals the first N rows
  of the aligned run - the missing tail cannot leak into the result.
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


def _sdpa(q, k, v, causal):
    qf, kf, vf = (oracle.to_f64(x) for x in (q, k, v))
    G = qf.shape[1] // kf.shape[1]
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qf), torch.from_numpy(kf).repeat_interleave(G, 1),
        torch.from_numpy(vf).repeat_interleave(G, 1), is_causal=causal).numpy()


@pytest.mark.parametrize("causal,N,blk", [(True, 300, 64), (False, 200, 64), (True, 65, 64), (False, 1, 64),
                                          (True, 130, 128)])
def test_dense_ragged_equals_library_attention(causal, N, blk):
    q, k, v = _inputs(51, 1, 4, 2, N, 32)
    M = -(-N // blk)
    r = oracle.run(q, k, v, np.full((4, 1), -np.inf), causal, blk)
    assert r["out"].shape == (1, 4, N, 32) and r["skip_counts"].shape == (1, 4, M)
    np.testing.assert_allclose(r["out"], _sdpa(q, k, v, causal), atol=1e-12, rtol=0)
    assert (r["skip_counts"] == 0).all()


@pytest.mark.parametrize("causal", [True, False])
def test_diagonal_only_ragged_is_block_diagonal(causal):
    N, blk = 200, 64
    q, k, v = _inputs(52, 1, 2, 1, N, 16)
    r = oracle.run(q, k, v, np.full((2, 1), np.inf), causal, blk)
    M = -(-N // blk)
    for i in range(M):
        sl = slice(i * blk, min((i + 1) * blk, N))
        ref = _sdpa(q[:, :, sl], k[:, :, sl], v[:, :, sl], causal)
        np.testing.assert_allclose(r["out"][:, :, sl], ref, atol=1e-12, rtol=0)
        assert (r["skip_counts"][:, :, i] == (i if causal else M - 1)).all()


def _nested(x):
    return oracle.to_f64(x).tolist()


@pytest.mark.parametrize("causal,N,gate", [(True, 230, "threshold"), (False, 150, "threshold"),
                                           (True, 200, "gap")])
def test_ragged_matches_brute_force_streaming(causal, N, gate):
    blk = 64
    q, k, v = _inputs(53, 1, 2, 1, N, 16, scale=1.5)
    tm = oracle.tile_maxima(q, k, causal, blk)
    M = -(-N // blk)
    assert tm.shape == (1, 2, M, M)
    if gate == "gap":
        thr = np.full((2, M), 0.6)
    else:
        off = tm[..., ~np.eye(M, dtype=bool)]
        finite = off[np.isfinite(off)]
        thr = np.full((2, M), np.quantile(finite, 0.5))
    r = oracle.run(q, k, v, thr, causal, blk, gate_mode=gate)
    bo, bl, bs, bt = brute_stream(_nested(q), _nested(k), _nested(v), thr.tolist(), causal, blk, gate=gate)
    assert (np.array(bs) == r["skip_counts"]).all()
    assert r["skip_counts"].sum() > 0
    bt = np.array([[[[np.nan if x is None else x for x in row] for row in hh] for hh in bb] for bb in bt])
    np.testing.assert_allclose(bt, r["tile_max"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(np.array(bo), r["out"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(np.array(bl), r["lse"], atol=1e-12, rtol=0)


def test_tail_of_a_longer_sequence_does_not_leak():
    # causal attention over the first N positions cannot see later ones, so the
    # causal ragged run must equal the first N rows of the aligned run when the
    # gate decisions agree; with T = -inf they do by construction
    N_full, N, blk = 256, 200, 64
    q, k, v = _inputs(54, 1, 2, 1, N_full, 16)
    thr = np.full((2, 1), -np.inf)
    full = oracle.run(q, k, v, thr, True, blk)
    part = oracle.run(q[:, :, :N], k[:, :, :N], v[:, :, :N], thr, True, blk)
    np.testing.assert_allclose(part["out"], full["out"][:, :, :N], atol=1e-12, rtol=0)
    np.testing.assert_allclose(part["lse"], full["lse"][:, :, :N], atol=1e-12, rtol=0)
