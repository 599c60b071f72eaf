"""Helpers shared by the parity tests: threshold construction from the oracle
and comparison of the HIP path's results with the oracle's.

Acceptance (per tile / element, on identical bf16 inputs):
  * skip mask identical, except tiles whose oracle s_max lies within 1e-3 of
    the threshold (either decision is correct there);
  * out: max |diff| <= 1e-2 and mean |diff| <= 1e-3;
  * lse: max |diff| <= 1e-3;
  * skip_counts equal to the number of skipped tiles of the same run;
  * tile_max (diagnostic): |diff| <= 1e-4 + 1e-5 |s_max| (fp32 accumulation of
    exact bf16 products against float64).
Thresholds built by ``margin_thresholds`` keep every tile maximum at least
2e-3 away, so on those inputs the mask must match exactly.  Where a tile
inside the exempt band was decided differently (thresholds calibrated on the
GPU's own fp32 maxima sit exactly between two of them), the query block's
out and lse are compared with the oracle run under the GPU's mask instead
(``oracle.run_blocks(..., skip_override=...)``), which needs the inputs.
"""

from __future__ import annotations

import numpy as np

import oracle

OUT_MAX = 1e-2
OUT_MEAN = 1e-3
LSE_MAX = 1e-3
EXEMPT = 1e-3
TMAX_ABS = 1e-4
TMAX_REL = 1e-5


def away_from(t0: float, vals: np.ndarray, margin: float = 2e-3) -> float:
    """``t0`` if every value is more than ``margin`` away from it, else the
    middle of the nearest gap between consecutive values (or beyond the ends)
    that is wider than 2*margin."""
    vals = np.sort(vals[np.isfinite(vals)])
    if not np.isfinite(t0) or vals.size == 0 or np.min(np.abs(vals - t0)) > margin:
        return t0
    ext = np.concatenate(([vals[0] - 4 * margin], vals, [vals[-1] + 4 * margin]))
    mids = 0.5 * (ext[:-1] + ext[1:])
    cand = mids[(ext[1:] - ext[:-1]) > 2 * margin]
    return float(cand[np.argmin(np.abs(cand - t0))])


def _diag(i: int, block, m_kv: int):
    bm, bn = oracle.tile_shape(block)
    return oracle.diagonal_blocks(i, bm, bn, m_kv)


def margin_thresholds(tile_max: np.ndarray, k, causal: bool, margin: float = 2e-3, block=1) -> np.ndarray:
    """Fixed-k thresholds [H, M] (float32) from oracle tile maxima [B, H, M, M_KV]
    (``block``: the tile, for the diagonal sets; an int means square).

    Starts from the oracle's fixed-k calibration (averaged over the batch) and,
    where a tile maximum of any batch element lies within ``margin`` of it,
    moves the threshold to the middle of the nearest gap wider than
    2*margin between consecutive off-diagonal maxima.  ``k=None`` gives -inf.
    Rows with no finite tile maxima keep the calibrated value.
    """
    B, H, M, M_kv = tile_max.shape
    if k is None:
        return np.full((H, M), -np.inf, dtype=np.float32)
    thr = oracle.calibrate_fixed_k(tile_max, k, causal, block)
    out = thr.astype(np.float32)
    for h in range(H):
        for i in range(M):
            diag = _diag(i, block, M_kv)
            cols = [j for j in range(M_kv) if j not in diag]
            out[h, i] = np.float32(away_from(float(out[h, i]), tile_max[:, h, i, cols].ravel(), margin))
    return out


def gap_thresholds(tile_max: np.ndarray, causal: bool, base: float, margin: float = 2e-3,
                   step: float = 0.037, block=1) -> np.ndarray:
    """Gaps [H, M] (float32) for the gap gate, starting at ``base``, moved per
    (head, query block) until no off-diagonal tile of any batch element lies
    within ``margin`` of its decision boundary M - gap (float64, the oracle's
    visiting order), so that the masks of the two sides must agree exactly."""
    B, H, M, M_kv = tile_max.shape
    out = np.empty((H, M), dtype=np.float32)
    for h in range(H):
        for i in range(M):
            diag = _diag(i, block, M_kv)
            for t in range(200):
                gap = np.float32(base + step * ((t + 1) // 2) * (1 if t % 2 else -1))
                ok = True
                for b in range(B):
                    row = tile_max[b, h, i]
                    m = -np.inf
                    for j in range(M_kv):
                        if not np.isfinite(row[j]):
                            continue  # not computed
                        ref = m - float(gap)
                        if j not in diag and np.isfinite(ref) and abs(row[j] - ref) <= margin:
                            ok = False
                            break
                        if j in diag or not row[j] < ref:
                            m = max(m, row[j])
                    if not ok:
                        break
                if ok:
                    break
            else:
                raise RuntimeError("no gap with the required margin")
            out[h, i] = gap
    return out


def rerun_under_mask(inputs, thresholds: np.ndarray, block, b: int, h: int, i: int,
                     skip_row: np.ndarray) -> dict:
    """Oracle result of query block (b, h, i) with the skip decisions of its
    computed tiles taken from ``skip_row`` [M_KV] (bool) instead of its gate."""
    q, k, v, causal = inputs
    g = h // (q.shape[1] // k.shape[1])
    ov = np.zeros((1, 1, i + 1, skip_row.shape[0]), dtype=bool)
    ov[0, 0, i] = skip_row
    r = oracle.run_blocks(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], thresholds[h:h + 1],
                          causal, block, [(0, 0, i)], skip_override=ov)[0]
    r.update(b=b, h=h)
    return r


def compare_blocks(gpu: dict, ref_blocks, block, thresholds: np.ndarray, label: str = "",
                   exempt: bool = True, inputs=None):
    """Compare GPU outputs (numpy, full arrays) with oracle ``run_blocks`` results
    (``block``: an int for square tiles or (B_M, B_N)).

    ``exempt=False``: no tile is exempt from the mask comparison (inputs built
    with a margin around every decision boundary, e.g. ``gap_thresholds``).
    ``inputs``: (q, k, v, causal) as given to the oracle.  When the GPU decided
    a tile of the exempt band differently (known from its ``tile_state``), the
    block's out and lse are compared with the oracle under the GPU's mask;
    without ``inputs`` such a difference is an error.
    Returns a dict of statistics (``exempt``: tiles in the band; ``overridden``:
    blocks compared under the GPU's mask; ``flipped``: band tiles decided
    differently).  Raises AssertionError on any violation.
    """
    errs = []
    n_exempt = 0
    n_override = 0
    n_flipped = 0
    worst = 0.0
    abs_sum = 0.0
    count = 0
    lse_worst = 0.0
    tmax_worst = 0.0
    bm, _ = oracle.tile_shape(block)
    for r in ref_blocks:
        b, h, i = r["b"], r["h"], r["i"]
        sl = slice(i * bm, (i + 1) * bm)
        computed = np.isfinite(r["tile_max"])
        st_ref = r["tile_state"]
        if "tile_state" in gpu:
            st_gpu = gpu["tile_state"][b, h, i]
            tau = float(thresholds[h, min(i, thresholds.shape[1] - 1)])
            near = np.zeros_like(computed)
            near[computed] = np.abs(r["tile_max"][computed] - tau) <= EXEMPT
            near[st_ref == oracle.STATE_DIAGONAL] = False
            if not exempt:
                near[:] = False
            n_exempt += int(near.sum())
            bad = (st_gpu != st_ref) & ~near
            if bad.any():
                errs.append(f"{label} (b={b},h={h},i={i}): tile_state differs at j={np.flatnonzero(bad)[:8]}")
            flipped = (st_gpu != st_ref) & near
            if flipped.any():
                n_flipped += int(flipped.sum())
                if not np.isin(st_gpu[flipped], (oracle.STATE_KEPT, oracle.STATE_SKIPPED)).all():
                    errs.append(f"{label} (b={b},h={h},i={i}): invalid tile_state in the exempt band")
                elif inputs is None:
                    errs.append(f"{label} (b={b},h={h},i={i}): exempt tiles decided differently and no inputs "
                                "for the mask-override comparison")
                else:
                    r = rerun_under_mask(inputs, thresholds, block, b, h, i, st_gpu == oracle.STATE_SKIPPED)
                    n_override += 1
            skipped_gpu = int((st_gpu == oracle.STATE_SKIPPED).sum())
            if int(gpu["skip_counts"][b, h, i]) != skipped_gpu:
                errs.append(f"{label} (b={b},h={h},i={i}): skip_count {gpu['skip_counts'][b, h, i]} != "
                            f"{skipped_gpu} skipped tiles")
            tm = gpu["tile_max"][b, h, i]
            if not np.array_equal(np.isnan(tm), ~computed):
                errs.append(f"{label} (b={b},h={h},i={i}): tile_max NaN pattern differs")
            d = np.abs(tm[computed] - r["tile_max"][computed])
            tol = TMAX_ABS + TMAX_REL * np.abs(r["tile_max"][computed])
            tmax_worst = max(tmax_worst, float(d.max()) if d.size else 0.0)
            if (d > tol).any():
                errs.append(f"{label} (b={b},h={h},i={i}): tile_max off by {d.max():.3g}")
        elif int(gpu["skip_counts"][b, h, i]) != r["skip_count"]:
            errs.append(f"{label} (b={b},h={h},i={i}): skip_count {gpu['skip_counts'][b, h, i]} != "
                        f"{r['skip_count']}")
        o = gpu["out"][b, h, sl].astype(np.float64)
        diff = np.abs(o - r["out"])
        worst = max(worst, float(diff.max()))
        abs_sum += float(diff.sum())
        count += diff.size
        ld = np.abs(gpu["lse"][b, h, sl].astype(np.float64) - r["lse"])
        lse_worst = max(lse_worst, float(ld.max()))
    mean = abs_sum / max(count, 1)
    if worst > OUT_MAX:
        errs.append(f"{label}: out max-abs {worst:.3g} > {OUT_MAX}")
    if mean > OUT_MEAN:
        errs.append(f"{label}: out mean-abs {mean:.3g} > {OUT_MEAN}")
    if lse_worst > LSE_MAX:
        errs.append(f"{label}: lse max-abs {lse_worst:.3g} > {LSE_MAX}")
    stats = {"out_max": worst, "out_mean": mean, "lse_max": lse_worst, "tile_max_max": tmax_worst,
             "exempt": n_exempt, "flipped": n_flipped, "overridden": n_override, "blocks": len(ref_blocks)}
    assert not errs, "\n".join(errs[:20]) + f"\nstats={stats}"
    return stats
