"""C ABI checks that need no GPU: the library loads, exports every entry point
include/bsfa.h declares, validates shapes and rejects bad pointers before any
HIP call."""

import ctypes
import os
import re

import pytest

from block_sparse_flashattention_tiled_amd import binding as bb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bb.LIB_PATH):
        from block_sparse_flashattention_tiled_amd import build_lib

        build_lib.build()
    return bb.load_library()


def _declared():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(bsfa_\w+)\s*\(", src))
    return names


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert {"bsfa_prefill", "bsfa_prefill_ex", "bsfa_validate", "bsfa_status_string"} <= declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared but not exported"
    assert set(bb.EXPORTED) <= declared


def S(B=1, Hq=4, Hkv=2, N=1024, d=128, T=8):
    return bb.make_shape(B, Hq, Hkv, N, d, T)


@pytest.mark.parametrize(
    "shape,causal,blk,status",
    [
        (S(), 1, 128, 0),
        (S(d=64), 0, 64, 0),
        (S(N=1000), 1, 128, 0),      # not a multiple of the tile: the last block is partial
        (S(N=1), 0, 64, 0),          # a single position
        (S(Hq=3, Hkv=2), 1, 128, 2),  # H_q % H_kv
        (S(d=96), 1, 128, 3),        # unsupported head dim
        (S(), 1, 96, 3),             # unsupported tile
        (S(), 2, 128, 2),            # causal flag
        (S(T=0), 1, 128, 2),
        (S(B=0), 1, 128, 2),
        (S(N=-128), 1, 128, 2),
        # one head's K / V must fit in 2^31 - 1 bytes (32-bit buffer offsets)
        (S(B=1, Hq=1, Hkv=1, N=8_388_607, d=128, T=1), 1, 128, 0),
        (S(B=1, Hq=1, Hkv=1, N=8_388_608, d=128, T=1), 1, 128, 3),
        (S(B=1, Hq=1, Hkv=1, N=8_388_609, d=128, T=1), 1, 128, 3),
        (S(B=1, Hq=1, Hkv=1, N=16_777_215, d=64, T=1), 0, 64, 0),
        (S(B=1, Hq=1, Hkv=1, N=16_777_216, d=64, T=1), 0, 64, 3),
        (S(B=1, Hq=1, Hkv=1, N=16_777_217, d=64, T=1), 0, 64, 3),
        (S(B=1, Hq=1, Hkv=1, N=100_000_000, d=128, T=1), 1, 128, 3),
        (S(B=1, Hq=1, Hkv=1, N=2**30 + 1, d=64, T=1), 1, 64, 2),  # beyond INT32_MAX / 2
    ],
)
def test_validate(lib, shape, causal, blk, status):
    assert bb.bsfa_validate(shape, causal, bb.make_block(blk)) == status


def test_tile_shapes(lib):
    # every pairing of 64 and 128 has kernels; other sides do not
    for bm in (64, 128):
        for bn in (64, 128):
            assert bb.bsfa_validate(S(), 1, bb.make_block(bm, bn)) == 0
            assert bb.bsfa_validate(S(N=1000), 0, bb.make_block(bm, bn)) == 0
    for bm, bn in ((128, 32), (32, 128), (128, 224), (256, 64)):
        assert bb.bsfa_validate(S(), 1, bb.make_block(bm, bn)) == 3
    assert bb.bsfa_validate(S(), 1, bb.make_block(128, 0)) == 2
    assert bb.bsfa_validate(S(), 1, bb.make_block(-64, 64)) == 2


def test_calibrate_rejects_before_any_launch(lib):
    import ctypes

    good = 0x100000
    ks = (ctypes.c_int64 * 2)(2, 5)
    pks = ctypes.cast(ks, ctypes.c_void_p)
    f = lib.bsfa_calibrate
    blk = bb.make_block(128, 64)
    assert f(good, S(), 1, bb.make_block(128, 32), pks, 2, good, None) == 3   # tile without kernels
    assert f(good, S(Hq=3, Hkv=2), 1, blk, pks, 2, good, None) == 2           # shape
    assert f(good, S(), 2, blk, pks, 2, good, None) == 2                      # causal flag
    assert f(good, S(), 1, blk, None, 2, good, None) == 1                     # ks missing
    assert f(None, S(), 1, blk, pks, 2, good, None) == 1                      # tile maxima missing
    assert f(good, S(), 1, blk, pks, 0, good, None) == 2                      # no level
    bad = (ctypes.c_int64 * 2)(3, -1)
    assert f(good, S(), 1, blk, ctypes.cast(bad, ctypes.c_void_p), 2, good, None) == 2  # negative k
    assert f(good, S(N=64 * 20000), 1, bb.make_block(128, 64), pks, 2, good, None) == 3  # M_KV beyond the kernel
    assert f(good + 2, S(), 1, blk, pks, 2, good, None) == 4                  # misaligned tile maxima


def test_status_strings(lib):
    for s in range(6):
        assert bb.status_string(s) and bb.status_string(s) != "unknown status"
    assert bb.status_string(99) == "unknown status"


def test_null_and_misaligned_pointers_rejected_before_any_launch(lib):
    shape, blk = S(), bb.make_block(128)
    f = lib.bsfa_prefill
    good = 0x100000
    # required pointer missing
    assert f(None, good, good, good, None, None, good, shape, 1, blk, None) == 1
    assert f(good, good, good, good, None, None, None, shape, 1, blk, None) == 1
    # misaligned bf16 / fp32 buffers
    assert f(good + 2, good, good, good, None, None, good, shape, 1, blk, None) == 4
    assert f(good, good, good, good + 4, None, None, good, shape, 1, blk, None) == 4
    assert f(good, good, good, good, good + 2, None, good, shape, 1, blk, None) == 4
    # shape errors win over pointer errors
    assert f(None, None, None, None, None, None, None, S(Hq=3, Hkv=2), 1, blk, None) == 2
    assert lib.bsfa_prefill_ex(good, good, good, good, None, None, good, shape, 1, blk, None, good + 1,
                               None) == 4


def test_bf16_and_gated_entry_points_reject_before_any_launch(lib):
    shape, blk = S(), bb.make_block(128)
    good = 0x100000
    f = lib.bsfa_prefill_bf16
    assert f(good, good, good, None, None, None, good, shape, 1, blk, None) == 1  # no output
    assert f(good, good, good, good + 8, None, None, good, shape, 1, blk, None) == 4  # bf16 out not 16-B aligned
    assert f(None, None, None, None, None, None, None, S(Hq=3, Hkv=2), 1, blk, None) == 2
    g = lib.bsfa_prefill_gated
    for bad_gate in (-1, 2, 7):  # unknown gate: shape status, before the pointer checks
        assert g(good, good, good, good, None, None, good, shape, 1, blk, bad_gate, None, None, None) == 2
    assert g(good, good, good, None, None, None, good, shape, 1, blk, bb.GATE_GAP, None, None, None) == 1
    assert g(good, good, good, good, None, None, good, shape, 1, blk, bb.GATE_GAP, None, good + 2, None) == 4


def test_calibrate_levels_rejects_before_any_launch(lib):
    import ctypes

    good = 0x100000
    ks = (ctypes.c_int64 * 3)(2, 5, 9)
    f = lib.bsfa_calibrate_levels
    pks = ctypes.cast(ks, ctypes.c_void_p)
    assert f(good, 1, 4, 8, 1, None, 3, good, None) == 1        # ks missing
    assert f(good, 1, 4, 8, 1, pks, 0, good, None) == 2         # no level
    bad = (ctypes.c_int64 * 2)(3, -1)
    assert f(good, 1, 4, 8, 1, ctypes.cast(bad, ctypes.c_void_p), 2, good, None) == 2  # negative k
    assert f(good, 1, 4, 20000, 1, pks, 3, good, None) == 3     # M beyond the calibration kernel
    assert f(good + 2, 1, 4, 8, 1, pks, 3, good, None) == 4     # misaligned tile maxima
    assert f(good, 1, 4, 8, 2, pks, 3, good, None) == 2         # causal flag


def test_missing_library_raises_and_nothing_falls_back(monkeypatch, tmp_path):
    # with the shared library absent every entry point must fail loudly: there is no CPU path
    monkeypatch.setattr(bb, "LIB_PATH", str(tmp_path / "absent" / "libbsfa.so"))
    monkeypatch.setattr(bb, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        bb.load_library()
    with pytest.raises(RuntimeError):
        bb.bsfa_validate(S(), 1, bb.make_block(128))
    with pytest.raises(RuntimeError):
        bb.status_string(0)


def test_heads_past_32bit_offsets_rejected_by_every_entry_point(lib):
    # N d 2 > INT32_MAX: every entry point returns BSFA_ERR_UNSUPPORTED before any launch
    import ctypes

    good = 0x100000
    blk = bb.make_block(128)
    long_ = bb.make_shape(1, 2, 1, 8_388_608, 128, 1)
    ks = (ctypes.c_int64 * 1)(3)
    pks = ctypes.cast(ks, ctypes.c_void_p)
    assert lib.bsfa_prefill(good, good, good, good, None, None, good, long_, 1, blk, None) == 3
    assert lib.bsfa_prefill_ex(good, good, good, good, None, None, good, long_, 1, blk, good, good, None) == 3
    assert lib.bsfa_prefill_bf16(good, good, good, good, None, None, good, long_, 1, blk, None) == 3
    assert lib.bsfa_prefill_gated(good, good, good, good, None, None, good, long_, 1, blk, 1, None, None, None) == 3
    assert lib.bsfa_prefill_varlen(good, good, good, good, None, None, good, long_, 1, blk, good, None, None,
                                   None) == 3
    assert lib.bsfa_tile_max(good, good, good, long_, 1, blk, None) == 3
    assert lib.bsfa_calibrate(good, long_, 1, blk, pks, 1, good, None) == 3
