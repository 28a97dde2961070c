"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Holds random-number generation and dtype conversion of inputs only (see
gen.c); none of the method's arithmetic lives here.  Both sides of every
parity test read the bytes this module produces.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

SEED_BASE = 0xC5A20000


def build() -> str:
    """Compile gen.c into libsynth.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
    lib.synth_word.argtypes = [u64, u64]
    lib.synth_word.restype = u64
    for name in ("synth_normal_f32", "synth_normal_bf16", "synth_normal_e4m3"):
        getattr(lib, name).argtypes = [u64, u64, i64, vp]
        getattr(lib, name).restype = None
    lib.synth_normal_rows_f32.argtypes = [u64, vp, i64, i64, vp]
    lib.synth_normal_rows_f32.restype = None
    for name in ("synth_to_bf16", "synth_to_e4m3"):
        getattr(lib, name).argtypes = [vp, i64, vp]
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def seed(cfg: int, stream: int) -> int:
    """Seed of one input tensor: base + 1000*workload + stream id."""
    return SEED_BASE + 1000 * cfg + stream


def word(seed_: int, n: int) -> int:
    """Raw 64-bit word n of stream seed_ (counter-based SplitMix64)."""
    return int(_load().synth_word(seed_, n))


def normal_f32(seed_: int, n: int, offset: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """Elements offset .. offset+n-1 of the N(0,1) stream seed_, as float32."""
    if out is None:
        out = np.empty(n, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == n
    _load().synth_normal_f32(seed_, offset, n, out.ctypes.data)
    return out


def normal_rows_f32(seed_: int, row_ids, row_len: int) -> np.ndarray:
    """Rows row_ids of the stream viewed as [*, row_len]; float32 [len(row_ids), row_len]."""
    ids = np.ascontiguousarray(np.asarray(row_ids, dtype=np.int64))
    out = np.empty((ids.size, row_len), dtype=np.float32)
    _load().synth_normal_rows_f32(seed_, ids.ctypes.data, ids.size, row_len, out.ctypes.data)
    return out


def normal_bf16(seed_: int, n: int, offset: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """N(0,1) stream rounded to bf16 (RNE); returns the uint16 bit patterns."""
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    _load().synth_normal_bf16(seed_, offset, n, out.ctypes.data)
    return out


def normal_e4m3(seed_: int, n: int, offset: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """N(0,1) stream rounded to fp8 e4m3fn (RNE, saturating); returns uint8 bit patterns."""
    if out is None:
        out = np.empty(n, dtype=np.uint8)
    assert out.dtype == np.uint8 and out.flags.c_contiguous and out.size == n
    _load().synth_normal_e4m3(seed_, offset, n, out.ctypes.data)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().synth_to_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().synth_to_e4m3(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_idx(dtype: str, seed_: int, n: int, offset: int = 0) -> np.ndarray:
    """Index-vector stream in the named storage dtype ('bf16' -> uint16 bits, 'e4m3' -> uint8 bits,
    'fp4' -> the fp32 values, which each side packs with its own FP4 codec)."""
    if dtype == "fp4":
        return normal_f32(seed_, n, offset)
    if dtype == "bf16":
        return normal_bf16(seed_, n, offset)
    if dtype == "e4m3":
        return normal_e4m3(seed_, n, offset)
    raise ValueError(f"unknown index dtype {dtype!r}")
