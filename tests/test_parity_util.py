"""CPU checks of the parity comparison itself (the acceptance rule for tiles
whose maximum lies within 1e-3 of the threshold): the oracle stands in for
the GPU, with one near-threshold tile decided the other way."""

import numpy as np
import pytest

import oracle
from block_sparse_flashattention_tiled_amd import workloads as wl
from parity_util import EXEMPT, compare_blocks, rerun_under_mask


def _setup():
    w = wl.get_config("tiny")
    data = wl.generate(w, seed=3)
    q, k, v = data["q"], data["k"], data["v"]
    blk, M = w.block, w.n_blocks
    tm = oracle.tile_maxima(q, k, True, blk)
    # the off-diagonal tile with the largest maximum of (h=1, i=M-1): removing
    # it changes that block's output by far more than the tolerance
    h, i = 1, M - 1
    j = int(np.nanargmax(tm[0, h, i, :i]))
    thr = np.full((w.heads_q, M), -np.inf)
    thr[h, i] = tm[0, h, i, j]  # exactly on the maximum: kept (strict '<'), inside the band
    blocks = [(0, hh, ii) for hh in range(w.heads_q) for ii in range(M)]
    ref = oracle.run_blocks(q, k, v, thr, True, blk, blocks)
    full = oracle.run(q, k, v, thr, True, blk)
    gpu = {n: full[n].copy() for n in ("out", "lse", "skip_counts", "tile_state", "tile_max")}
    gpu["out"] = gpu["out"].astype(np.float32)
    gpu["lse"] = gpu["lse"].astype(np.float32)
    return w, data, thr, blocks, ref, gpu, (h, i, j)


def _flip(gpu, data, thr, blk, h, i, j, outputs=True):
    """The "GPU" skips tile j of (h, i); its outputs follow that mask when ``outputs``."""
    gpu = {n: a.copy() for n, a in gpu.items()}
    gpu["tile_state"][0, h, i, j] = oracle.STATE_SKIPPED
    gpu["skip_counts"][0, h, i] += 1
    if outputs:
        r = rerun_under_mask((data["q"], data["k"], data["v"], True), thr, blk, 0, h, i,
                             gpu["tile_state"][0, h, i] == oracle.STATE_SKIPPED)
        gpu["out"][0, h, i * blk:(i + 1) * blk] = r["out"]
        gpu["lse"][0, h, i * blk:(i + 1) * blk] = r["lse"]
    return gpu


def test_identical_results_pass_with_the_band_counted():
    w, data, thr, blocks, ref, gpu, _ = _setup()
    st = compare_blocks(gpu, ref, w.block, thr, "same", inputs=(data["q"], data["k"], data["v"], True))
    assert st["exempt"] >= 1 and st["flipped"] == 0 and st["overridden"] == 0


def test_flipped_band_tile_is_compared_under_the_gpu_mask():
    w, data, thr, blocks, ref, gpu, (h, i, j) = _setup()
    g2 = _flip(gpu, data, thr, w.block, h, i, j)
    inputs = (data["q"], data["k"], data["v"], True)
    st = compare_blocks(g2, ref, w.block, thr, "flip", inputs=inputs)
    assert st["flipped"] == 1 and st["overridden"] == 1
    # the flip matters: the flipped outputs fail against the oracle's own mask
    assert np.abs(g2["out"][0, h] - gpu["out"][0, h]).max() > 10 * 1e-2
    # without the inputs the difference cannot be checked: an error
    with pytest.raises(AssertionError, match="mask-override"):
        compare_blocks(g2, ref, w.block, thr, "flip")
    # outputs that do not follow the GPU's own mask fail
    g3 = _flip(gpu, data, thr, w.block, h, i, j, outputs=False)
    with pytest.raises(AssertionError, match="out max-abs"):
        compare_blocks(g3, ref, w.block, thr, "stale", inputs=inputs)


def test_flip_outside_the_band_fails():
    w, data, thr, blocks, ref, gpu, (h, i, j) = _setup()
    thr2 = thr.copy()
    thr2[h, i] -= 4 * EXEMPT  # the tile is now clearly above its threshold
    ref2 = oracle.run_blocks(data["q"], data["k"], data["v"], thr2, True, w.block, blocks)
    g2 = _flip(gpu, data, thr2, w.block, h, i, j)
    with pytest.raises(AssertionError, match="tile_state differs"):
        compare_blocks(g2, ref2, w.block, thr2, "outside", inputs=(data["q"], data["k"], data["v"], True))
