"""Seeded synthetic inputs for block-sparse FlashAttention prefill.

This module only draws random numbers and rounds them to bfloat16.  It holds
none of the attention arithmetic (no scores, no softmax, no gate, no
thresholds), so the CPU oracle and the HIP path can both be fed from it
without sharing any of the method's code.

The pages ("Block Sparse Flash Attention", paperpeel.com/paper/2512.07011)
measure on RULER, LongBench and Needle-in-a-Haystack with Llama-3.1-8B and
Qwen2.5-7B.  None of those datasets or weights is available here, so these
generators stand in for them at the same layer shapes:

* ``tiny``      - 1 batch, 2 query heads over 1 KV head, N=1024, d=64, 64x64
                  tiles, causal; Q, K, V ~ N(0,1) with 8 planted keys equal to
                  4x a random query row.
* ``llama8k``   - Llama-3.1-8B layer (Sec. 5.1 / App. B.1: 32 heads, d=128),
                  8 KV heads, N=8192, causal.  Q and K share a smooth random
                  walk latent per KV group (local correlation), the first 64
                  keys point along the mean query (an attention sink, Sec. 2
                  "Empirical sparsity patterns"), and 1% of key positions are
                  planted needles.
* ``llama32k``  - the same generator at N=32768.
* ``gqa128k``   - N=131072, 32 query heads over 4 KV heads, 0.2% needles.
* ``dit32k``    - non-causal (App. B.3 "Practical considerations": the method
                  extends to bidirectional attention): B=2, 40 heads, no GQA,
                  N=32768 tokens on a 16x32x64 (t, y, x) grid; Q and K are a
                  spatially smooth random field plus white noise.

Every tensor is drawn in float32 and rounded to bfloat16 with
round-to-nearest-even; arrays are returned as the raw uint16 bit patterns so
both consumers read exactly the same bytes.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "CONFIGS",
    "get_config",
    "generate",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and generator recipe of one synthetic prefill attention layer."""

    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seq_len: int
    head_dim: int
    block: int
    causal: bool
    kind: str  # "tiny" | "llama" | "dit"
    skip_targets: Tuple[float, ...]
    needles: int = 0  # planted keys per (batch, KV group); "tiny" only
    needle_frac: float = 0.0  # planted keys as a fraction of key positions
    sink: int = 64  # number of sink keys ("llama")
    rho_len: float = 256.0  # correlation length of the latent walk ("llama")
    grid: Tuple[int, int, int] = (0, 0, 0)  # (t, y, x) token grid ("dit")
    blur: Tuple[float, float, float] = (1.0, 2.0, 2.0)  # Gaussian sigma ("dit")

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // self.block)  # the last block may be partial

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 2, 1, 1024, 64, 64, True, "tiny", (0.5,), needles=8),
    "llama8k": Workload("llama8k", 1, 32, 8, 8192, 128, 128, True, "llama", (0.5,), needle_frac=0.01),
    "llama32k": Workload(
        "llama32k", 1, 32, 8, 32768, 128, 128, True, "llama", (0.0, 0.6, 0.8, 0.9), needle_frac=0.01
    ),
    "gqa128k": Workload("gqa128k", 1, 32, 4, 131072, 128, 128, True, "llama", (0.95,), needle_frac=0.002),
    "dit32k": Workload(
        "dit32k", 2, 40, 40, 32768, 128, 128, False, "dit", (0.75,), grid=(16, 32, 64)
    ),
}


def get_config(name: str, **overrides) -> Workload:
    w = CONFIGS[name]
    return w.replace(**overrides) if overrides else w


# ---------------------------------------------------------------------------
# bfloat16 bit handling (round-to-nearest-even)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------


def _plant(q_bits, k_bits, b, g, group, count, lo, rng, taken):
    """Plant ``count`` keys K[b,g,kpos] = 4*Q[b,h,qpos] with kpos <= qpos.

    Multiplying a bfloat16 value by 4 only moves its exponent, so the planted
    key is exactly representable.  Key positions are distinct and >= ``lo``; a
    sequence with fewer free positions than ``count`` gets one per free position.
    """
    n = q_bits.shape[2]
    count = min(count, max(0, n - lo - sum(1 for t in taken if t >= lo)))
    planted = []
    while len(planted) < count:
        h = g * group + int(rng.integers(group))
        qpos = int(rng.integers(lo, n))
        kpos = int(rng.integers(lo, qpos + 1))
        if kpos in taken:
            continue
        taken.add(kpos)
        row = bf16_bits_to_f32(q_bits[b, h, qpos]) * np.float32(4.0)
        k_bits[b, g, kpos] = f32_to_bf16_bits(row)
        planted.append((h, qpos, kpos))
    return planted


def _gen_tiny(w: Workload, seed: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    shp_q = (w.batch, w.heads_q, w.seq_len, w.head_dim)
    shp_k = (w.batch, w.heads_kv, w.seq_len, w.head_dim)
    q = f32_to_bf16_bits(rng.standard_normal(shp_q, dtype=np.float32))
    k = f32_to_bf16_bits(rng.standard_normal(shp_k, dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal(shp_k, dtype=np.float32))
    planted = []
    for b in range(w.batch):
        for g in range(w.heads_kv):
            taken: set = set()
            for h, qp, kp in _plant(q, k, b, g, w.group, w.needles, 0, rng, taken):
                planted.append((b, h, qp, kp))
    return q, k, v, planted


def _smooth_walk(rng, n, d, rho):
    """Stationary AR(1) walk z_t = rho z_{t-1} + sqrt(1-rho^2) e_t, unit variance."""
    from scipy.signal import lfilter

    e = rng.standard_normal((n, d), dtype=np.float32).astype(np.float64)
    c = math.sqrt(1.0 - rho * rho)
    e[0] /= c  # so that z_0 = e_0 ~ N(0, I)
    return lfilter([c], [1.0, -rho], e, axis=0).astype(np.float32)


def _gen_llama(w: Workload, seed: int):
    n, d, G = w.seq_len, w.head_dim, w.group
    q = np.empty((w.batch, w.heads_q, n, d), np.uint16)
    k = np.empty((w.batch, w.heads_kv, n, d), np.uint16)
    v = np.empty((w.batch, w.heads_kv, n, d), np.uint16)
    rho = math.exp(-1.0 / w.rho_len)
    n_needles = int(round(w.needle_frac * n))
    children = np.random.SeedSequence(seed).spawn(w.batch * w.heads_kv)
    planted = []
    for b in range(w.batch):
        for g in range(w.heads_kv):
            rng = np.random.Generator(np.random.PCG64(children[b * w.heads_kv + g]))
            z = _smooth_walk(rng, n, d, rho)
            half_z = np.float32(0.5) * z
            for hh in range(G):
                q[b, g * G + hh] = f32_to_bf16_bits(half_z + rng.standard_normal((n, d), dtype=np.float32))
            kk = half_z + rng.standard_normal((n, d), dtype=np.float32)
            # attention sink: the first keys point along the mean query of the group
            qf = bf16_bits_to_f32(q[b, g * G : (g + 1) * G]).astype(np.float64)
            m = qf.mean(axis=(0, 1))
            m_hat = (m / np.linalg.norm(m)).astype(np.float32)
            s = min(w.sink, n)
            kk[:s] = np.float32(4.0 * math.sqrt(d)) * m_hat + rng.standard_normal((s, d), dtype=np.float32)
            k[b, g] = f32_to_bf16_bits(kk)
            v[b, g] = f32_to_bf16_bits(rng.standard_normal((n, d), dtype=np.float32))
            taken: set = set()
            lo = min(s, n - 1)
            for h, qp, kp in _plant(q, k, b, g, G, n_needles, lo, rng, taken):
                planted.append((b, h, qp, kp))
    return q, k, v, planted


def _gen_dit(w: Workload, seed: int):
    from scipy.ndimage import gaussian_filter

    t, y, x = w.grid
    n, d = w.seq_len, w.head_dim
    if t * y * x != n:
        raise ValueError(f"grid {w.grid} does not hold {n} tokens")
    if w.heads_q != w.heads_kv:
        raise ValueError("the DiT workload has no grouped-query heads")
    q = np.empty((w.batch, w.heads_q, n, d), np.uint16)
    k = np.empty_like(q)
    v = np.empty_like(q)
    children = np.random.SeedSequence(seed).spawn(w.batch * w.heads_q)
    sigma = (w.blur[0], w.blur[1], w.blur[2], 0.0)
    for b in range(w.batch):
        for h in range(w.heads_q):
            rng = np.random.Generator(np.random.PCG64(children[b * w.heads_q + h]))
            white = rng.standard_normal((t, y, x, d), dtype=np.float32)
            f = gaussian_filter(white, sigma=sigma, mode="wrap")
            f /= np.float32(f.std())
            # token n = (t*Y + y)*X + x, i.e. C order over (t, y, x)
            f = f.reshape(n, d)
            q[b, h] = f32_to_bf16_bits(f + rng.standard_normal((n, d), dtype=np.float32))
            k[b, h] = f32_to_bf16_bits(f + rng.standard_normal((n, d), dtype=np.float32))
            v[b, h] = f32_to_bf16_bits(rng.standard_normal((n, d), dtype=np.float32))
    return q, k, v, []


def generate(w: Workload, seed: int = 0) -> dict:
    """Draw one seeded input set for workload ``w``.

    Returns ``{"q", "k", "v"}`` as uint16 bfloat16 bit arrays of shape
    ``[B, H, N, d]`` (C order) plus ``"planted"``: a list of
    ``(b, h_q, q_pos, k_pos)`` for every planted key.
    """
    if w.kind == "tiny":
        q, k, v, planted = _gen_tiny(w, seed)
    elif w.kind == "llama":
        q, k, v, planted = _gen_llama(w, seed)
    elif w.kind == "dit":
        q, k, v, planted = _gen_dit(w, seed)
    else:
        raise ValueError(f"unknown workload kind {w.kind!r}")
    return {"q": q, "k": k, "v": v, "planted": planted, "workload": w, "seed": seed}


def random_thresholds(rng: np.random.Generator, heads_q: int, t_len: int, lo: float, hi: float) -> np.ndarray:
    """Uniform float32 thresholds in [lo, hi) of shape [heads_q, t_len]."""
    return rng.uniform(lo, hi, size=(heads_q, t_len)).astype(np.float32)
