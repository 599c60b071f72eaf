"""Brute-force streaming evaluation used to pin the oracle.

Pure-Python scalar loops (no numpy arithmetic, no BLAS) that follow the
tiled online-softmax procedure of "Block Sparse Flash Attention"
(paperpeel.com/paper/2512.07011), App. B.2 steps (1)-(6), with the gating
check of Sec. 4.4 inserted after each score tile: keep Q_i, stream K_j, form
the scaled scores of the tile, skip the tile when it is off the diagonal and
its maximum is below the threshold, otherwise update the running max and
normaliser, accumulate P~ V_j and rescale.  A tile is diagonal when some
position is both a query of its query block and a key of its key block; a
tile with no visible (query, key) pair is not computed.  Both are found by
enumerating positions, not by index arithmetic.

The oracle instead evaluates one softmax over the kept entries of each row;
the two agree only if online softmax with skips is the exact rearrangement
the pages claim, so this is an independent check.  Tiny inputs only.
"""

import math


def brute_stream(q, k, v, thresholds, causal, block, gate="threshold"):
    """q: [B][Hq][N][d] nested float lists (or arrays of Python floats);
    ``block``: B_M = B_N (int) or (B_M, B_N).

    ``gate="gap"``: the running-maximum gate instead of the stored threshold -
    skip an off-diagonal tile whose maximum is below (largest maximum of the
    tiles kept so far) minus the table entry.

    Returns (out, lse, skip_counts, tile_max) as nested lists; tile_max holds
    the maximum visible score of each computed tile (None where not computed).
    """
    B = len(q)
    Hq = len(q[0])
    N = len(q[0][0])
    d = len(q[0][0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    bm, bn = (block, block) if isinstance(block, int) else block
    M = -(-N // bm)  # the last blocks may be partial
    M_kv = -(-N // bn)
    t_len = len(thresholds[0])
    inv = 1.0 / math.sqrt(d)
    out = [[[None] * N for _ in range(Hq)] for _ in range(B)]
    lse = [[[None] * N for _ in range(Hq)] for _ in range(B)]
    skips = [[[0] * M for _ in range(Hq)] for _ in range(B)]
    tmax = [[[[None] * M_kv for _ in range(M)] for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(M):
                tau = thresholds[h][min(i, t_len - 1)]
                rows = list(range(i * bm, min((i + 1) * bm, N)))
                m_run = [-math.inf] * len(rows)
                l_run = [0.0] * len(rows)
                acc = [[0.0] * d for _ in range(len(rows))]
                kept_max = -math.inf
                for j in range(M_kv):
                    cols = list(range(j * bn, min((j + 1) * bn, N)))
                    diagonal = any(c in rows for c in cols)
                    s = [[None] * len(cols) for _ in range(len(rows))]
                    tile_max = -math.inf
                    for a, qr in enumerate(rows):
                        for c, kc in enumerate(cols):
                            if causal and kc > qr:
                                continue
                            dot = 0.0
                            qv = q[b][h][qr]
                            kv = k[b][g][kc]
                            for e in range(d):
                                dot += qv[e] * kv[e]
                            s[a][c] = dot * inv
                            if s[a][c] > tile_max:
                                tile_max = s[a][c]
                    if all(x is None for row in s for x in row):
                        continue  # no visible pair: not computed
                    tmax[b][h][i][j] = tile_max
                    if gate == "gap":
                        ref = math.nan if kept_max == -math.inf and tau == -math.inf else kept_max - tau
                    else:
                        ref = tau
                    if not diagonal and tile_max < ref:
                        skips[b][h][i] += 1
                        continue
                    kept_max = max(kept_max, tile_max)
                    for a in range(len(rows)):
                        vals = [(c, s[a][c]) for c in range(len(cols)) if s[a][c] is not None]
                        if not vals:
                            continue
                        m_new = max(m_run[a], max(x for _, x in vals))
                        alpha = 0.0 if m_run[a] == -math.inf else math.exp(m_run[a] - m_new)
                        l_run[a] *= alpha
                        row_acc = acc[a]
                        for e in range(d):
                            row_acc[e] *= alpha
                        for c, x in vals:
                            p = math.exp(x - m_new)
                            l_run[a] += p
                            vr = v[b][g][cols[c]]
                            for e in range(d):
                                row_acc[e] += p * vr[e]
                        m_run[a] = m_new
                for a, qr in enumerate(rows):
                    out[b][h][qr] = [x / l_run[a] for x in acc[a]]
                    lse[b][h][qr] = m_run[a] + math.log(l_run[a])
    return out, lse, skips, tmax
