"""Seeded generators: determinism, bf16 rounding, planted keys, shapes (CPU)."""

import hashlib

import numpy as np
import pytest

from block_sparse_flashattention_tiled_amd import workloads as wl


def _digest(d):
    h = hashlib.sha256()
    for n in ("q", "k", "v"):
        h.update(d[n].tobytes())
    return h.hexdigest()


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    b = wl.f32_to_bf16_bits(x)
    back = wl.bf16_bits_to_f32(b)
    # ties go to the even mantissa: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0 + 2**-6)
    assert back[3] == 1.0 and back[4] == -2.5
    # round trip is exact on bf16 values
    assert np.array_equal(wl.f32_to_bf16_bits(back), b)
    # against torch's own conversion
    import torch
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(tb, b)


def test_tiny_is_deterministic_and_planted_exactly():
    w = wl.get_config("tiny")
    a = wl.generate(w, seed=0)
    b = wl.generate(w, seed=0)
    c = wl.generate(w, seed=1)
    assert _digest(a) == _digest(b) != _digest(c)
    assert a["q"].shape == (1, 2, 1024, 64) and a["k"].shape == (1, 1, 1024, 64)
    assert len(a["planted"]) == 8
    kpos = [p[3] for p in a["planted"]]
    assert len(set(kpos)) == 8
    for bb, h, qp, kp in a["planted"]:
        assert kp <= qp
        assert np.array_equal(wl.bf16_bits_to_f32(a["k"][bb, 0, kp]), 4 * wl.bf16_bits_to_f32(a["q"][bb, h, qp]))


def test_llama_generator_small():
    w = wl.get_config("llama8k", seq_len=2048, heads_q=8, heads_kv=2)
    a = wl.generate(w, seed=0)
    assert _digest(a) == _digest(wl.generate(w, seed=0))
    assert a["q"].shape == (1, 8, 2048, 128) and a["v"].shape == (1, 2, 2048, 128)
    assert len(a["planted"]) == 2 * round(0.01 * 2048)
    for b, h, qp, kp in a["planted"]:
        assert 64 <= kp <= qp
        assert h // 4 in (0, 1)
    # the latent makes neighbouring keys correlated and distant ones not
    kf = wl.bf16_bits_to_f32(a["k"][0, 0, 64:]).astype(np.float64)
    near = np.mean(np.sum(kf[:-1] * kf[1:], axis=1))
    far = np.mean(np.sum(kf[:-1000] * kf[1000:], axis=1))
    assert near > 20 and abs(far) < 10  # 0.25 * d = 32 shared variance per step


def test_dit_generator_small():
    w = wl.get_config("dit32k", batch=1, heads_q=2, heads_kv=2, seq_len=2 * 8 * 16, grid=(2, 8, 16), head_dim=64)
    a = wl.generate(w, seed=0)
    assert a["q"].shape == (1, 2, 256, 64)
    qf = wl.bf16_bits_to_f32(a["q"][0, 0]).reshape(2, 8, 16, 64).astype(np.float64)
    # spatial neighbours along x share the smooth field
    assert np.mean(np.sum(qf[:, :, :-1] * qf[:, :, 1:], axis=-1)) > 0.4 * 64


def test_unaligned_length_has_a_partial_last_block():
    w = wl.get_config("tiny", seq_len=1000)
    d = wl.generate(w, seed=0)
    assert w.n_blocks == 16 and d["q"].shape[2] == 1000
    assert all(0 <= kp <= qp < 1000 for _, _, qp, kp in d["planted"])


@pytest.mark.parametrize("n", [1, 3, 8])
def test_sequence_shorter_than_the_needle_count(n):
    # eight needles want eight distinct key positions; a shorter sequence gets one per position and the
    # generator still ends
    w = wl.get_config("tiny", seq_len=n, causal=False)
    d = wl.generate(w, seed=0)
    kpos = [p[3] for p in d["planted"]]
    assert len(kpos) == min(8, n) and len(set(kpos)) == len(kpos)
    assert all(0 <= kp <= qp < n for _, _, qp, kp in d["planted"])
