"""CSA2 CPU oracle - TEST INFRASTRUCTURE ONLY.

Python access (ctypes + numpy) to the plain C oracle in csa2_oracle.c.  Only the
tests, the smoke check and the bench's CPU-baseline leg may import this module;
the GPU library never uses it and shares no code with it.  The oracle's
readings of the method, and the passages they follow, are listed at the top of
csa2_oracle.c.

Storage conventions (identical to the inputs the GPU path receives):
  bf16 tensors are uint16 bit patterns, fp8 e4m3fn tensors are uint8 bit patterns,
  index dtype code 0 = bf16, 1 = e4m3, 2 = FP4 keys (e2m1 codes [.., K/2] plus fp32
  scales per 32 elements [.., K/32], the cache codec) with bf16 index queries.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

IDX_DTYPES = {"bf16": 0, "e4m3": 1, "fp4": 2}
MODES = {"F": 0, "Ri": 1, "Ru": 2}


def build() -> str:
    """Compile the oracle (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=gnu11",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float


class _Group(ctypes.Structure):
    _fields_ = [("B", i32), ("N_cap", i64), ("D", i32), ("H_I", i32), ("d_I", i32),
                ("idx_dtype", i32), ("k", i32), ("codes", vp), ("scales", vp), ("ikeys", vp),
                ("n_valid", vp), ("sel", vp), ("has_entries", i32), ("has_selection", i32),
                ("sel_qs", i32), ("ikey_scales", vp), ("pool_blocks", i32), ("pool", vp),
                ("has_pool", i32), ("pool_qs", i32)]


class _Layer(ctypes.Structure):
    _fields_ = [("Qs", i32), ("Hq", i32), ("q", vp), ("iq", vp), ("wk", vp), ("wv", vp),
                ("W", i32), ("wlen", vp), ("new_entry", vp), ("new_ikey", vp),
                ("sm_scale", f32), ("out", vp), ("lse", vp)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.orc_e2m1_value.argtypes = [ctypes.c_int]
    lib.orc_e2m1_value.restype = ctypes.c_double
    lib.orc_fp4_pack.argtypes = [vp, i64, ctypes.c_int, vp, vp]
    lib.orc_fp4_pack.restype = None
    lib.orc_fp4_dequant.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    lib.orc_fp4_dequant.restype = None
    lib.orc_idx_value.argtypes = [ctypes.c_int, vp, i64]
    lib.orc_idx_value.restype = ctypes.c_double
    lib.orc_exact_dot_f32.argtypes = [vp, vp, ctypes.c_int]
    lib.orc_exact_dot_f32.restype = ctypes.c_float
    lib.orc_exact_sum_f32.argtypes = [vp, ctypes.c_int]
    lib.orc_exact_sum_f32.restype = ctypes.c_float
    lib.orc_index_score.argtypes = [ctypes.c_int, vp, vp, vp, i64, i64, i64, ctypes.c_int,
                                    ctypes.c_int, vp, vp]
    lib.orc_index_score.restype = None
    lib.orc_topk.argtypes = [vp, i64, i64, i64, vp, ctypes.c_int, vp]
    lib.orc_topk.restype = None
    lib.orc_pool_blocks.argtypes = [vp, i64, i64, vp, ctypes.c_int, vp]
    lib.orc_pool_blocks.restype = None
    lib.orc_pool_topk.argtypes = [vp, i64, i64, vp, vp, ctypes.c_int, ctypes.c_int, vp]
    lib.orc_pool_topk.restype = None
    lib.orc_attend.argtypes = [vp, i64, i64, ctypes.c_int, ctypes.c_int, vp, vp, i64, vp,
                               ctypes.c_int, vp, vp, ctypes.c_int, vp, f32, vp, vp]
    lib.orc_attend.restype = None
    lib.orc_layer_step.argtypes = [ctypes.c_int, ctypes.POINTER(_Layer), ctypes.POINTER(_Group)]
    lib.orc_layer_step.restype = ctypes.c_int
    lib.orc_cache_bytes.argtypes = [i64, i64, i64, i64]
    lib.orc_cache_bytes.restype = i64
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return None if a is None else a.ctypes.data


def e2m1_value(code: int) -> float:
    return float(_load().orc_e2m1_value(int(code)))


def fp4_pack(x: np.ndarray):
    """x float32 [rows, dim] -> (codes uint8 [rows, dim/2], scales float32 [rows, dim/32])."""
    x = _c(x, np.float32)
    rows, dim = x.shape
    assert dim % 32 == 0
    codes = np.empty((rows, dim // 2), dtype=np.uint8)
    scales = np.empty((rows, dim // 32), dtype=np.float32)
    _load().orc_fp4_pack(x.ctypes.data, rows, dim, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def fp4_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    rows = codes.shape[0]
    dim = codes.shape[1] * 2
    out = np.empty((rows, dim), dtype=np.float64)
    _load().orc_fp4_dequant(codes.ctypes.data, scales.ctypes.data, rows, dim, out.ctypes.data)
    return out


def idx_values(dtype: str, bits: np.ndarray) -> np.ndarray:
    """Decode stored index elements to float64 with the oracle's own decoder."""
    bits = np.ascontiguousarray(bits)
    lib = _load()
    code = IDX_DTYPES[dtype]
    flat = bits.reshape(-1)
    return np.array([lib.orc_idx_value(code, flat.ctypes.data, i) for i in range(flat.size)],
                    dtype=np.float64).reshape(bits.shape)


def exact_dot_f32(a: np.ndarray, b: np.ndarray) -> np.float32:
    a = _c(a, np.float64)
    b = _c(b, np.float64)
    assert a.size == b.size
    return np.float32(_load().orc_exact_dot_f32(a.ctypes.data, b.ctypes.data, a.size))


def exact_sum_f32(t: np.ndarray) -> np.float32:
    t = _c(t, np.float64)
    return np.float32(_load().orc_exact_sum_f32(t.ctypes.data, t.size))


def index_score(dtype: str, iq: np.ndarray, ik: np.ndarray, n_valid_row=None, ik_scales=None) -> np.ndarray:
    """iq [B, Qs, H, d] and ik [B, N, H, d] stored bits -> exact fp32 scores [B, Qs, N].
    dtype 'fp4': iq bf16 bits, ik e2m1 codes [B, N, H, d/2], ik_scales float32 [B, N, H*d/32]."""
    B, Qs, H, d = iq.shape
    N = ik.shape[1]
    if dtype == "fp4":
        assert ik.shape == (B, N, H, d // 2) and ik_scales is not None
        iq = _c(iq, np.uint16)
        ik = _c(ik, np.uint8)
        ks = _c(ik_scales, np.float32)
        assert ks.shape == (B, N, H * d // 32)
    else:
        assert ik.shape == (B, N, H, d)
        st = np.uint16 if dtype == "bf16" else np.uint8
        iq = _c(iq, st)
        ik = _c(ik, st)
        ks = None
    nv = None if n_valid_row is None else _c(n_valid_row, np.int64)
    out = np.empty((B, Qs, N), dtype=np.float32)
    _load().orc_index_score(IDX_DTYPES[dtype], iq.ctypes.data, ik.ctypes.data, _p(ks), B, Qs, N, H, d,
                            _p(nv), out.ctypes.data)
    return out


def topk(scores: np.ndarray, k: int, n_valid=None) -> np.ndarray:
    """scores float32 [R, N] -> int32 [R, k] ascending indices, -1 padded."""
    s = _c(scores, np.float32)
    R, N = s.shape
    nv = None if n_valid is None else _c(n_valid, np.int64)
    out = np.empty((R, k), dtype=np.int32)
    _load().orc_topk(s.ctypes.data, R, N, N, _p(nv), k, out.ctypes.data)
    return out


POOL_BLOCK = 8


def pool_blocks(scores: np.ndarray, P: int, n_valid) -> np.ndarray:
    """Hierarchical pool: scores float32 [R, N], n_valid [R] -> int32 [R, P], the P blocks of 8
    positions with the largest block score (max over the block's valid positions), ascending."""
    s = _c(scores, np.float32)
    R, N = s.shape
    nv = _c(n_valid, np.int64)
    out = np.empty((R, P), dtype=np.int32)
    _load().orc_pool_blocks(s.ctypes.data, R, N, nv.ctypes.data, P, out.ctypes.data)
    return out


def pool_topk(scores: np.ndarray, pool: np.ndarray, k: int, n_valid) -> np.ndarray:
    """Top-k over the valid positions of the pool's blocks only: int32 [R, k] ascending, -1 padded."""
    s = _c(scores, np.float32)
    R, N = s.shape
    pl = _c(pool, np.int32)
    nv = _c(n_valid, np.int64)
    out = np.empty((R, k), dtype=np.int32)
    _load().orc_pool_topk(s.ctypes.data, R, N, nv.ctypes.data, pl.ctypes.data, pl.shape[1], k,
                          out.ctypes.data)
    return out


def attend(q, codes, scales, idx, wk, wv, W, sm_scale, wlen=None):
    """q bf16 bits [B, Qs, Hq, D]; codes [B, N, D/2]; scales [B, N, D/32]; idx [B*Qs, k];
    wk, wv bf16 bits [B, Qs+W-1, D] -> (out float32 [B, Qs, Hq, D], lse float32 [B, Qs, Hq])."""
    q = _c(q, np.uint16)
    B, Qs, Hq, D = q.shape
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    N = codes.shape[1]
    idx = _c(idx, np.int32)
    k = idx.shape[-1]
    wk = _c(wk, np.uint16)
    wv = _c(wv, np.uint16)
    assert wk.shape == (B, Qs + W - 1, D) and wv.shape == wk.shape
    wl = None if wlen is None else _c(wlen, np.int32)
    out = np.empty((B, Qs, Hq, D), dtype=np.float32)
    lse = np.empty((B, Qs, Hq), dtype=np.float32)
    _load().orc_attend(q.ctypes.data, B, Qs, Hq, D, codes.ctypes.data, scales.ctypes.data, N,
                       idx.ctypes.data, k, wk.ctypes.data, wv.ctypes.data, W, _p(wl),
                       float(sm_scale), out.ctypes.data, lse.ctypes.data)
    return out, lse


def cache_bytes(entries: int, numbers: int, copies: int, bits: int) -> int:
    return int(_load().orc_cache_bytes(entries, numbers, copies, bits))


class Group:
    """One sharing group's state: FP4 entries, index keys, valid counts and the shared selection."""

    def __init__(self, codes, scales, ikeys, n_valid, idx_dtype: str, k: int, max_rows: int,
                 has_entries: bool = True, ikey_scales=None, pool_blocks: int = 0):
        """ikeys [B, N, H, d] stored bits; 'fp4': e2m1 codes [B, N, H, d/2] and
        ikey_scales float32 [B, N, H*d/32].  pool_blocks > 0: hierarchical search (Full keeps a
        pool of that many 8-position blocks per row, Reindex ranks only the pool)."""
        self.codes = _c(codes, np.uint8)
        self.scales = _c(scales, np.float32)
        self.idx_dtype = idx_dtype
        st = np.uint16 if idx_dtype == "bf16" else np.uint8
        self.ikeys = _c(ikeys, st)
        self.B, self.N_cap, H_I, d_I = self.ikeys.shape
        self.ikey_scales = None
        if idx_dtype == "fp4":
            d_I *= 2
            self.ikey_scales = _c(ikey_scales, np.float32)
        self.n_valid = _c(n_valid, np.int64)
        self.sel = np.full((max_rows, k), -1, dtype=np.int32)
        self.pool = np.full((max_rows, max(pool_blocks, 1)), -1, dtype=np.int32)
        self._g = _Group(self.B, self.N_cap, self.codes.shape[2] * 2, H_I, d_I,
                         IDX_DTYPES[idx_dtype], k, self.codes.ctypes.data, self.scales.ctypes.data,
                         self.ikeys.ctypes.data, self.n_valid.ctypes.data, self.sel.ctypes.data,
                         int(has_entries), 0, 0, _p(self.ikey_scales), pool_blocks,
                         self.pool.ctypes.data, 0, 0)

    @property
    def has_selection(self) -> bool:
        return bool(self._g.has_selection)

    def layer_step(self, mode: str, q, W, sm_scale, wk, wv, iq=None, new_entry=None, new_ikey=None,
                   wlen=None):
        """Run one layer; returns (status, out, lse)."""
        q = _c(q, np.uint16)
        B, Qs, Hq, D = q.shape
        st = self.ikeys.dtype
        qt = np.uint16 if self.idx_dtype == "fp4" else st  # fp4 keys take bf16 queries
        iq = None if iq is None else _c(iq, qt)
        wk = _c(wk, np.uint16)
        wv = _c(wv, np.uint16)
        ne = None if new_entry is None else _c(new_entry, np.float32)
        nk = None if new_ikey is None else _c(new_ikey, np.float32 if self.idx_dtype == "fp4" else st)
        wl = None if wlen is None else _c(wlen, np.int32)
        out = np.zeros((B, Qs, Hq, D), dtype=np.float32)
        lse = np.zeros((B, Qs, Hq), dtype=np.float32)
        L = _Layer(Qs, Hq, q.ctypes.data, _p(iq), wk.ctypes.data, wv.ctypes.data, W, _p(wl),
                   _p(ne), _p(nk), float(sm_scale), out.ctypes.data, lse.ctypes.data)
        rc = _load().orc_layer_step(MODES[mode], ctypes.byref(L), ctypes.byref(self._g))
        return rc, out, lse
