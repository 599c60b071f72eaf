"""ctypes binding of ``libbsfa.so`` (the C ABI declared in ``include/bsfa.h``).

Argument marshalling only: torch tensors are checked for dtype, shape,
contiguity and device, their device pointers and torch's current HIP stream
are passed to the library, and a non-zero status raises.  All computation
happens in the library's HIP kernels.  There is no fallback: if the library
has not been built, every entry point raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbsfa.so")

BSFA_OK = 0
TILE_PRUNED, TILE_KEPT, TILE_SKIPPED, TILE_DIAGONAL = 0, 1, 2, 3
GATE_THRESHOLD, GATE_GAP = 0, 1
GATES = {"threshold": GATE_THRESHOLD, "gap": GATE_GAP}

EXPORTED = (
    "bsfa_prefill",
    "bsfa_prefill_ex",
    "bsfa_prefill_bf16",
    "bsfa_prefill_gated",
    "bsfa_prefill_varlen",
    "bsfa_tile_max",
    "bsfa_calibrate_fixed_k",
    "bsfa_calibrate_levels",
    "bsfa_calibrate",
    "bsfa_validate",
    "bsfa_status_string",
)


class BsfaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("n_heads_q", ctypes.c_int64),
        ("n_heads_kv", ctypes.c_int64),
        ("seq_len", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("thr_len", ctypes.c_int64),
    ]


class BsfaBlock(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32)]


class BsfaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libbsfa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m block_sparse_flashattention_tiled_amd.build_lib` (there is no fallback path)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.bsfa_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, BsfaShape, i32, BsfaBlock, vp]
    lib.bsfa_prefill.restype = i32
    lib.bsfa_prefill_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, BsfaShape, i32, BsfaBlock, vp, vp, vp]
    lib.bsfa_prefill_ex.restype = i32
    lib.bsfa_prefill_bf16.argtypes = [vp, vp, vp, vp, vp, vp, vp, BsfaShape, i32, BsfaBlock, vp]
    lib.bsfa_prefill_bf16.restype = i32
    lib.bsfa_prefill_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, BsfaShape, i32, BsfaBlock, i32, vp, vp, vp]
    lib.bsfa_prefill_gated.restype = i32
    lib.bsfa_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, BsfaShape, i32, BsfaBlock, vp, vp, vp, vp]
    lib.bsfa_prefill_varlen.restype = i32
    lib.bsfa_calibrate_levels.argtypes = [vp, i64, i64, i64, i32, vp, i64, vp, vp]
    lib.bsfa_calibrate_levels.restype = i32
    lib.bsfa_tile_max.argtypes = [vp, vp, vp, BsfaShape, i32, BsfaBlock, vp]
    lib.bsfa_tile_max.restype = i32
    lib.bsfa_calibrate_fixed_k.argtypes = [vp, i64, i64, i64, i32, i64, vp, vp]
    lib.bsfa_calibrate_fixed_k.restype = i32
    lib.bsfa_calibrate.argtypes = [vp, BsfaShape, i32, BsfaBlock, vp, i64, vp, vp]
    lib.bsfa_calibrate.restype = i32
    lib.bsfa_validate.argtypes = [BsfaShape, i32, BsfaBlock]
    lib.bsfa_validate.restype = i32
    lib.bsfa_status_string.argtypes = [i32]
    lib.bsfa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def make_shape(batch, n_heads_q, n_heads_kv, seq_len, head_dim, thr_len) -> BsfaShape:
    return BsfaShape(batch, n_heads_q, n_heads_kv, seq_len, head_dim, thr_len)


def make_block(bm: int, bn: Optional[int] = None) -> BsfaBlock:
    return BsfaBlock(bm, bm if bn is None else bn)


def as_block(block) -> BsfaBlock:
    """A BsfaBlock from an int (square tile), a (bm, bn) pair or a BsfaBlock."""
    if isinstance(block, BsfaBlock):
        return block
    if isinstance(block, (tuple, list)):
        return make_block(int(block[0]), int(block[1]))
    return make_block(int(block))


def n_blocks(seq_len: int, block: BsfaBlock) -> Tuple[int, int]:
    """(M, M_KV): query blocks ceil(N / bm) and key blocks ceil(N / bn); the last may be partial."""
    return (-(-seq_len // block.bm) if block.bm > 0 else 0, -(-seq_len // block.bn) if block.bn > 0 else 0)


def status_string(status: int) -> str:
    return load_library().bsfa_status_string(int(status)).decode()


def bsfa_validate(shape: BsfaShape, causal: int, block: BsfaBlock) -> int:
    """Host-only shape check; returns the status code."""
    return int(load_library().bsfa_validate(shape, int(causal), block))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(t, name, dtype, shape, device):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_all(q, k, v, out, lse, skip_counts, thresholds, shape, block, tile_state=None, tile_max=None,
               out_dtype=torch.float32):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    B, Hq, Hkv, N, d, T = (shape.batch, shape.n_heads_q, shape.n_heads_kv, shape.seq_len, shape.head_dim,
                           shape.thr_len)
    M, Mkv = n_blocks(N, block)
    _check(q, "q", torch.bfloat16, (B, Hq, N, d), dev)
    _check(k, "k", torch.bfloat16, (B, Hkv, N, d), dev)
    _check(v, "v", torch.bfloat16, (B, Hkv, N, d), dev)
    _check(out, "out", out_dtype, (B, Hq, N, d), dev)
    _check(lse, "lse", torch.float32, (B, Hq, N), dev)
    _check(skip_counts, "skip_counts", torch.int32, (B, Hq, M), dev)
    _check(thresholds, "thresholds", torch.float32, (Hq, T), dev)
    _check(tile_state, "tile_state", torch.uint8, (B, Hq, M, Mkv), dev)
    _check(tile_max, "tile_max", torch.float32, (B, Hq, M, Mkv), dev)


def bsfa_prefill(q, k, v, out, lse, skip_counts, thresholds, shape: BsfaShape, causal: int,
                 block: BsfaBlock, stream=None) -> None:
    """C ABI ``bsfa_prefill`` on torch tensors (see include/bsfa.h)."""
    st = bsfa_validate(shape, causal, block)
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_prefill")
    _check_all(q, k, v, out, lse, skip_counts, thresholds, shape, block)
    st = load_library().bsfa_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(skip_counts), _ptr(thresholds),
        shape, int(causal), block, _stream(stream))
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_prefill")


def bsfa_prefill_ex(q, k, v, out, lse, skip_counts, thresholds, shape: BsfaShape, causal: int,
                    block: BsfaBlock, tile_state, tile_max, stream=None) -> None:
    """C ABI ``bsfa_prefill_ex`` on torch tensors (see include/bsfa.h)."""
    st = bsfa_validate(shape, causal, block)
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_prefill_ex")
    _check_all(q, k, v, out, lse, skip_counts, thresholds, shape, block, tile_state, tile_max)
    st = load_library().bsfa_prefill_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(skip_counts), _ptr(thresholds),
        shape, int(causal), block, _ptr(tile_state), _ptr(tile_max), _stream(stream))
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_prefill_ex")


def bsfa_prefill_bf16(q, k, v, out, lse, skip_counts, thresholds, shape: BsfaShape, causal: int,
                      block: BsfaBlock, stream=None) -> None:
    """C ABI ``bsfa_prefill_bf16`` on torch tensors: ``out`` is bf16 (see include/bsfa.h)."""
    st = bsfa_validate(shape, causal, block)
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_prefill_bf16")
    _check_all(q, k, v, out, lse, skip_counts, thresholds, shape, block, out_dtype=torch.bfloat16)
    st = load_library().bsfa_prefill_bf16(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(skip_counts), _ptr(thresholds),
        shape, int(causal), block, _stream(stream))
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_prefill_bf16")


def bsfa_prefill_gated(q, k, v, out, lse, skip_counts, thresholds, shape: BsfaShape, causal: int,
                       block: BsfaBlock, gate: int, tile_state=None, tile_max=None, stream=None) -> None:
    """C ABI ``bsfa_prefill_gated`` on torch tensors (see include/bsfa.h)."""
    st = bsfa_validate(shape, causal, block)
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_prefill_gated")
    _check_all(q, k, v, out, lse, skip_counts, thresholds, shape, block, tile_state, tile_max)
    st = load_library().bsfa_prefill_gated(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(skip_counts), _ptr(thresholds),
        shape, int(causal), block, int(gate), _ptr(tile_state), _ptr(tile_max), _stream(stream))
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_prefill_gated")


def bsfa_prefill_varlen(q, k, v, out, lse, skip_counts, thresholds, shape: BsfaShape, causal: int,
                        block: BsfaBlock, seq_lens, tile_state=None, tile_max=None, stream=None) -> None:
    """C ABI ``bsfa_prefill_varlen``: ``seq_lens`` is an int32 [B] device tensor (see include/bsfa.h)."""
    st = bsfa_validate(shape, causal, block)
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_prefill_varlen")
    _check_all(q, k, v, out, lse, skip_counts, thresholds, shape, block, tile_state, tile_max)
    _check(seq_lens, "seq_lens", torch.int32, (shape.batch,), q.device)
    if seq_lens is None:
        raise ValueError("seq_lens is required")
    st = load_library().bsfa_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(skip_counts), _ptr(thresholds),
        shape, int(causal), block, _ptr(seq_lens), _ptr(tile_state), _ptr(tile_max), _stream(stream))
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_prefill_varlen")


def bsfa_calibrate_levels(tile_max, n_samples: int, n_heads: int, n_blocks: int, causal: int, ks,
                          thresholds, stream=None) -> None:
    """C ABI ``bsfa_calibrate_levels``: ``ks`` is a host sequence of ints, ``thresholds``
    a [len(ks), H, M] fp32 device tensor (see include/bsfa.h)."""
    dev = tile_max.device
    ks = [int(x) for x in ks]
    _check(tile_max, "tile_max", torch.float32, (n_samples, n_heads, n_blocks, n_blocks), dev)
    _check(thresholds, "thresholds", torch.float32, (len(ks), n_heads, n_blocks), dev)
    arr = (ctypes.c_int64 * max(len(ks), 1))(*ks)
    st = load_library().bsfa_calibrate_levels(_ptr(tile_max), n_samples, n_heads, n_blocks, int(causal),
                                              ctypes.cast(arr, ctypes.c_void_p), len(ks), _ptr(thresholds),
                                              _stream(stream))
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_calibrate_levels")


def bsfa_tile_max(q, k, tile_max, shape: BsfaShape, causal: int, block: BsfaBlock, stream=None) -> None:
    """C ABI ``bsfa_tile_max`` on torch tensors (see include/bsfa.h)."""
    st = bsfa_validate(shape, causal, block)
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_tile_max")
    dev = q.device
    B, Hq, Hkv, N, d = shape.batch, shape.n_heads_q, shape.n_heads_kv, shape.seq_len, shape.head_dim
    M, Mkv = n_blocks(N, block)
    _check(q, "q", torch.bfloat16, (B, Hq, N, d), dev)
    _check(k, "k", torch.bfloat16, (B, Hkv, N, d), dev)
    _check(tile_max, "tile_max", torch.float32, (B, Hq, M, Mkv), dev)
    st = load_library().bsfa_tile_max(_ptr(q), _ptr(k), _ptr(tile_max), shape, int(causal), block, _stream(stream))
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_tile_max")


def bsfa_calibrate_fixed_k(tile_max, n_samples: int, n_heads: int, n_blocks: int, causal: int, k: int,
                           thresholds, stream=None) -> None:
    """C ABI ``bsfa_calibrate_fixed_k`` on torch tensors (see include/bsfa.h)."""
    dev = tile_max.device
    _check(tile_max, "tile_max", torch.float32, (n_samples, n_heads, n_blocks, n_blocks), dev)
    _check(thresholds, "thresholds", torch.float32, (n_heads, n_blocks), dev)
    st = load_library().bsfa_calibrate_fixed_k(_ptr(tile_max), n_samples, n_heads, n_blocks, int(causal), int(k),
                                               _ptr(thresholds), _stream(stream))
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_calibrate_fixed_k")


def bsfa_calibrate(tile_max, shape: BsfaShape, causal: int, block: BsfaBlock, ks, thresholds,
                   stream=None) -> None:
    """C ABI ``bsfa_calibrate``: tile maxima [B, H_q, M, M_KV] of a ``bsfa_tile_max`` call with
    the same shape / causal / block, ``ks`` a host sequence of ints, ``thresholds`` a
    [len(ks), H_q, M] fp32 device tensor (see include/bsfa.h)."""
    st = bsfa_validate(shape, causal, block)
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_calibrate")
    dev = tile_max.device
    ks = [int(x) for x in ks]
    M, Mkv = n_blocks(shape.seq_len, block)
    _check(tile_max, "tile_max", torch.float32, (shape.batch, shape.n_heads_q, M, Mkv), dev)
    _check(thresholds, "thresholds", torch.float32, (len(ks), shape.n_heads_q, M), dev)
    arr = (ctypes.c_int64 * max(len(ks), 1))(*ks)
    st = load_library().bsfa_calibrate(_ptr(tile_max), shape, int(causal), block, ctypes.cast(arr, ctypes.c_void_p),
                                       len(ks), _ptr(thresholds), _stream(stream))
    if st != BSFA_OK:
        raise BsfaError(st, "bsfa_calibrate")


def tile_max(q: torch.Tensor, k: torch.Tensor, causal: bool, block, stream=None) -> torch.Tensor:
    """Allocate and fill the [B, H_q, M, M_KV] tile maxima (``bsfa_tile_max``);
    ``block`` is an int (square) or (bm, bn)."""
    B, Hq, N, d = q.shape
    shape = make_shape(B, Hq, k.shape[1], N, d, 1)
    blk = as_block(block)
    M, Mkv = n_blocks(N, blk)
    out = torch.empty((B, Hq, M, Mkv), dtype=torch.float32, device=q.device)
    bsfa_tile_max(q, k, out, shape, int(causal), blk, stream)
    return out


def calibrate_fixed_k(tile_maxima: torch.Tensor, k: Optional[int], causal: bool, stream=None) -> torch.Tensor:
    """Fixed-k threshold table [H, M] from square-tile maxima [S, H, M, M]; k=None gives -inf (dense).
    Any tile shape: ``calibrate``."""
    S, H, M, _ = tile_maxima.shape
    if k is None:
        return torch.full((H, M), float("-inf"), dtype=torch.float32, device=tile_maxima.device)
    thr = torch.empty((H, M), dtype=torch.float32, device=tile_maxima.device)
    bsfa_calibrate_fixed_k(tile_maxima, S, H, M, int(causal), int(k), thr, stream)
    return thr


def calibrate_levels(tile_maxima: torch.Tensor, ks, causal: bool, stream=None) -> torch.Tensor:
    """Threshold tensor [len(ks), H, M]: one fixed-k table per sparsity level (square tiles)."""
    S, H, M, _ = tile_maxima.shape
    thr = torch.empty((len(ks), H, M), dtype=torch.float32, device=tile_maxima.device)
    bsfa_calibrate_levels(tile_maxima, S, H, M, int(causal), ks, thr, stream)
    return thr


def calibrate(tile_maxima: torch.Tensor, ks, causal: bool, block, seq_len: int, head_dim: int,
              stream=None) -> torch.Tensor:
    """Threshold tensor [len(ks), H, M] for any tile shape (``bsfa_calibrate``); ``tile_maxima``
    [S, H, M, M_KV] as returned by ``tile_max`` for a sequence of ``seq_len`` positions."""
    S, H, M, _ = tile_maxima.shape
    blk = as_block(block)
    shape = make_shape(S, H, 1, seq_len, head_dim, M)
    thr = torch.empty((len(ks), H, M), dtype=torch.float32, device=tile_maxima.device)
    bsfa_calibrate(tile_maxima, shape, int(causal), blk, ks, thr, stream)
    return thr


def prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, thresholds: torch.Tensor, causal: bool,
                   block, seq_lens: torch.Tensor, diagnostics: bool = False, stream=None) -> dict:
    """Allocate the outputs and run ``bsfa_prefill_varlen`` (padded batch, int32 device lengths).
    Entries past each sequence are left as allocated (torch.empty)."""
    B, Hq, N, d = q.shape
    shape = make_shape(B, Hq, k.shape[1], N, d, thresholds.shape[1])
    blk = as_block(block)
    M, Mkv = n_blocks(N, blk)
    dev = q.device
    res = {
        "out": torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
        "lse": torch.empty((B, Hq, N), dtype=torch.float32, device=dev),
        "skip_counts": torch.empty((B, Hq, M), dtype=torch.int32, device=dev),
    }
    if diagnostics:
        res["tile_state"] = torch.empty((B, Hq, M, Mkv), dtype=torch.uint8, device=dev)
        res["tile_max"] = torch.empty((B, Hq, M, Mkv), dtype=torch.float32, device=dev)
    bsfa_prefill_varlen(q, k, v, res["out"], res["lse"], res["skip_counts"], thresholds, shape, int(causal), blk,
                        seq_lens, res.get("tile_state"), res.get("tile_max"), stream)
    return res


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, thresholds: torch.Tensor, causal: bool,
            block, diagnostics: bool = False, stream=None, gate: str = "threshold",
            out_dtype: torch.dtype = torch.float32) -> dict:
    """Allocate the outputs and run the forward pass.

    ``bsfa_prefill`` by default; ``bsfa_prefill_ex`` with diagnostics;
    ``bsfa_prefill_gated`` for ``gate="gap"``; ``bsfa_prefill_bf16`` for a
    bf16 output (threshold gate, no diagnostics).
    q: bf16 [B, H_q, N, d]; k, v: bf16 [B, H_kv, N, d]; thresholds: fp32 [H_q, T_len];
    block: an int (square tile) or (bm, bn).
    Returns a dict of device tensors: out, lse, skip_counts (+ tile_state, tile_max).
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    shape = make_shape(B, Hq, Hkv, N, d, thresholds.shape[1])
    blk = as_block(block)
    M, Mkv = n_blocks(N, blk)
    dev = q.device
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    if gate not in GATES:
        raise ValueError(f"gate must be one of {sorted(GATES)}")
    res = {
        "out": torch.empty((B, Hq, N, d), dtype=out_dtype, device=dev),
        "lse": torch.empty((B, Hq, N), dtype=torch.float32, device=dev),
        "skip_counts": torch.empty((B, Hq, M), dtype=torch.int32, device=dev),
    }
    if out_dtype == torch.bfloat16:
        if diagnostics or gate != "threshold":
            raise ValueError("the bf16 output entry point has the threshold gate and no diagnostics")
        bsfa_prefill_bf16(q, k, v, res["out"], res["lse"], res["skip_counts"], thresholds, shape, int(causal), blk,
                          stream)
        return res
    if gate != "threshold":
        if diagnostics:
            res["tile_state"] = torch.empty((B, Hq, M, Mkv), dtype=torch.uint8, device=dev)
            res["tile_max"] = torch.empty((B, Hq, M, Mkv), dtype=torch.float32, device=dev)
        bsfa_prefill_gated(q, k, v, res["out"], res["lse"], res["skip_counts"], thresholds, shape, int(causal),
                           blk, GATES[gate], res.get("tile_state"), res.get("tile_max"), stream)
        return res
    if diagnostics:
        res["tile_state"] = torch.empty((B, Hq, M, Mkv), dtype=torch.uint8, device=dev)
        res["tile_max"] = torch.empty((B, Hq, M, Mkv), dtype=torch.float32, device=dev)
        bsfa_prefill_ex(q, k, v, res["out"], res["lse"], res["skip_counts"], thresholds, shape, int(causal), blk,
                        res["tile_state"], res["tile_max"], stream)
    else:
        bsfa_prefill(q, k, v, res["out"], res["lse"], res["skip_counts"], thresholds, shape, int(causal), blk,
                     stream)
    return res


def bits_to_device(bits, device="cuda") -> torch.Tensor:
    """uint16 bfloat16 bit patterns (numpy) -> bf16 device tensor with the same bytes."""
    import numpy as np

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)
