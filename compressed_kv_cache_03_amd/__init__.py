"""Python binding of libcsa2 (CSA2 layer step for MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels behind
the C ABI declared in include/csa2.h.  PyTorch provides device memory and the
current stream.  There is no fallback: if libcsa2.so is missing or a call fails,
an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_STATE, ERR_HIP = range(6)
MODE = {"F": 0, "Ri": 1, "Ru": 2, "full": 0, "reindex": 1, "reuse": 2}
IDX_DTYPE = {"bf16": 0, "e4m3": 1, "fp4": 2}

vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class CGroup(ctypes.Structure):
    _fields_ = [("B", i32), ("N_cap", i64), ("D", i32), ("H_I", i32), ("d_I", i32),
                ("idx_dtype", ctypes.c_int), ("k", i32), ("codes", vp), ("scales", vp),
                ("ikeys", vp), ("n_valid", vp), ("n_valid_max", i64), ("sel", vp),
                ("sel_rows", i32), ("has_entries", i32), ("has_selection", i32), ("sel_qs", i32),
                ("ikey_scales", vp), ("pool_blocks", i32), ("pool", vp), ("has_pool", i32),
                ("pool_qs", i32)]

POOL_BLOCK = 8  # entries per block of a hierarchical group's pool
STATIC_SCRATCH_BYTES = 128 << 20  # scratch of csa2_layer_step_noalloc, per GPU


class CLayerArgs(ctypes.Structure):
    _fields_ = [("Qs", i32), ("Hq", i32), ("q", vp), ("iq", vp), ("wk", vp), ("wv", vp),
                ("W", i32), ("wlen", vp), ("new_entry", vp), ("new_ikey", vp),
                ("sm_scale", f32), ("out", vp), ("lse", vp), ("index_events", vp * 2)]


class Csa2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python compressed_kv_cache_03_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.csa2_status_str.argtypes = [ctypes.c_int]
    lib.csa2_status_str.restype = ctypes.c_char_p
    lib.csa2_version.argtypes = []
    lib.csa2_version.restype = ctypes.c_char_p
    lib.csa2_fp4_pack.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.csa2_index_score.argtypes = [vp, vp, vp, ctypes.c_int, i32, i32, i64, i32, i32, i64, i32, vp, vp]
    lib.csa2_topk_workspace_bytes.argtypes = [i64, i64, i32]
    lib.csa2_topk_workspace_bytes.restype = sz
    lib.csa2_topk.argtypes = [vp, i64, i64, i64, vp, i32, vp, vp, sz, vp]
    lib.csa2_attend_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.csa2_attend_workspace_bytes.restype = sz
    lib.csa2_sparse_attend.argtypes = [vp, i32, i32, i32, i32, vp, vp, i64, vp, i32, vp, vp, i32,
                                       vp, f32, vp, vp, vp, sz, vp]
    lib.csa2_layer_workspace_bytes.argtypes = [ctypes.POINTER(CGroup), i32, i32, i32]
    lib.csa2_layer_workspace_bytes.restype = sz
    lib.csa2_layer_step.argtypes = [ctypes.c_int, ctypes.POINTER(CLayerArgs), ctypes.POINTER(CGroup),
                                    vp, sz, vp]
    lib.csa2_layer_step_noalloc.argtypes = [ctypes.c_int, ctypes.POINTER(CLayerArgs), ctypes.POINTER(CGroup),
                                            vp]
    lib.csa2_group_image_bytes.argtypes = [ctypes.POINTER(CGroup)]
    lib.csa2_group_image_bytes.restype = sz
    lib.csa2_group_save.argtypes = [ctypes.POINTER(CGroup), vp, sz, vp]
    lib.csa2_group_restore.argtypes = [ctypes.POINTER(CGroup), vp, sz, vp]
    lib.csa2_cache_bytes.argtypes = [i64, i64, i64, i64]
    lib.csa2_cache_bytes.restype = i64
    for name in ("csa2_fp4_pack", "csa2_index_score", "csa2_topk", "csa2_sparse_attend",
                 "csa2_layer_step", "csa2_layer_step_noalloc", "csa2_group_save", "csa2_group_restore"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def lib():
    return _load()


def status_str(status: int) -> str:
    return _load().csa2_status_str(status).decode()


def version() -> str:
    return _load().csa2_version().decode()


def _check(status: int, where: str):
    if status != OK:
        raise Csa2Error(status, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def cache_bytes(entries: int, numbers: int, copies: int, bits: int) -> int:
    return int(_load().csa2_cache_bytes(entries, numbers, copies, bits))


def fp4_pack(x: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
             stream=None):
    """x fp32 [..., dim] -> (codes uint8 [..., dim/2], scales fp32 [..., dim/32])."""
    _dev(x, "x")
    assert x.dtype == torch.float32
    dim = x.shape[-1]
    rows = x.numel() // dim if dim else 0
    if codes is None:
        codes = torch.empty(*x.shape[:-1], dim // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(*x.shape[:-1], dim // 32, dtype=torch.float32, device=x.device)
    _check(_load().csa2_fp4_pack(x.data_ptr(), rows, dim, codes.data_ptr(), scales.data_ptr(),
                                 _stream(stream)), "csa2_fp4_pack")
    return codes, scales


def index_score(iq: torch.Tensor, ik: torch.Tensor, dtype: str, out: torch.Tensor | None = None,
                stream=None, ik_scales: torch.Tensor | None = None, causal_offset: int = -1,
                exact: bool = True) -> torch.Tensor:
    """iq [B, Qs, H, d] and ik [B, N, H, d] (uint8 for e4m3, int16/bf16/uint16 bits for bf16)
    -> exact fp32 scores [B, Qs, N].  dtype 'fp4': iq bf16 bits, ik the e2m1 codes
    [B, N, H, d/2] and ik_scales fp32 [B, N, H*d/32].  causal_offset c >= 0: row i scores
    entries j <= c + i and gets -inf for the rest."""
    _dev(iq, "iq")
    _dev(ik, "ik")
    B, Qs, H, d = iq.shape
    N = ik.shape[1]
    if dtype == "fp4":
        if ik_scales is None:
            raise ValueError("fp4 index keys need ik_scales")
        _dev(ik_scales, "ik_scales")
    if out is None:
        out = torch.empty(B, Qs, N, dtype=torch.float32, device=iq.device)
    _check(_load().csa2_index_score(iq.data_ptr(), ik.data_ptr(), _ptr(ik_scales), IDX_DTYPE[dtype], B, Qs,
                                    N, H, d, int(causal_offset), int(bool(exact)), out.data_ptr(),
                                    _stream(stream)), "csa2_index_score")
    return out


def _events(pair):
    """Raw hipEvent_t handles of a pair of created torch.cuda.Event, or (None, None)."""
    if pair is None:
        return (vp * 2)(None, None)
    handles = [int(e.cuda_event) for e in pair]
    if not all(handles):
        raise ValueError("index_events must be created (record them once) before use")
    return (vp * 2)(*handles)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def topk(scores: torch.Tensor, k: int, n_valid: torch.Tensor | None = None,
         out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """scores fp32 [R, N] -> int32 [R, k] ascending indices, -1 padded."""
    _dev(scores, "scores")
    R, N = scores.shape
    L = _load()
    if out is None:
        out = torch.empty(R, k, dtype=torch.int32, device=scores.device)
    need = L.csa2_topk_workspace_bytes(R, max(N, 1), k)
    if ws is None:
        ws = _workspace(need, scores.device)
    _check(L.csa2_topk(scores.data_ptr(), R, N, N, _ptr(n_valid), k, out.data_ptr(), ws.data_ptr(),
                       ws.numel(), _stream(stream)), "csa2_topk")
    return out


def sparse_attend(q, codes, scales, idx, wk, wv, W: int, sm_scale: float, wlen=None, out=None,
                  lse=None, ws=None, stream=None):
    """q bf16 [B, Qs, Hq, D]; codes [B, N, D/2]; scales [B, N, D/32]; idx int32 [B*Qs, k];
    wk, wv bf16 [B, Qs+W-1, D] -> (out fp32 [B, Qs, Hq, D], lse fp32 [B, Qs, Hq])."""
    B, Qs, Hq, D = q.shape
    N = codes.shape[1]
    k = idx.shape[-1]
    L = _load()
    if out is None:
        out = torch.empty(B, Qs, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(B, Qs, Hq, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = _workspace(L.csa2_attend_workspace_bytes(B, Qs, Hq, D, k, W), q.device)
    _check(L.csa2_sparse_attend(q.data_ptr(), B, Qs, Hq, D, codes.data_ptr(), scales.data_ptr(), N,
                                idx.data_ptr(), k, _ptr(wk), _ptr(wv), W, _ptr(wlen), float(sm_scale),
                                out.data_ptr(), _ptr(lse), ws.data_ptr(), ws.numel(), _stream(stream)),
           "csa2_sparse_attend")
    return out, lse


class Group:
    """A sharing group: FP4 entries, index keys, valid counts and the shared selection.

    The tensors are device tensors owned by this object; the C struct handed to the
    library points at them.
    """

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, ikeys: torch.Tensor,
                 n_valid: torch.Tensor, idx_dtype: str, k: int, sel_rows: int,
                 n_valid_max: int | None = None, has_entries: bool = True,
                 ikey_scales: torch.Tensor | None = None, pool_blocks: int = 0):
        """ikeys [B, N_cap, H_I, d_I] in idx_dtype; for 'fp4' the e2m1 codes
        [B, N_cap, H_I, d_I/2] and ikey_scales fp32 [B, N_cap, H_I*d_I/32].
        pool_blocks > 0 makes the group hierarchical: Full keeps a pool of that many
        blocks of POOL_BLOCK entries per query row, Reindex searches only the pool."""
        for name, t in (("codes", codes), ("scales", scales), ("ikeys", ikeys), ("n_valid", n_valid)):
            _dev(t, name)
        B, N_cap, H_I, d_I = ikeys.shape
        if idx_dtype == "fp4":
            if ikey_scales is None:
                raise ValueError("fp4 index keys need ikey_scales")
            _dev(ikey_scales, "ikey_scales")
            d_I *= 2
        self.ikey_scales = ikey_scales
        self.codes, self.scales, self.ikeys = codes, scales, ikeys
        self.n_valid = n_valid.to(torch.int32)
        self.sel = torch.full((sel_rows, k), -1, dtype=torch.int32, device=codes.device)
        self.pool = torch.full((sel_rows, max(pool_blocks, 1)), -1, dtype=torch.int32, device=codes.device)
        nvm = int(self.n_valid.max().item()) if n_valid_max is None else int(n_valid_max)
        self.c = CGroup(B, N_cap, codes.shape[-1] * 2, H_I, d_I, IDX_DTYPE[idx_dtype], k,
                        codes.data_ptr(), scales.data_ptr(), ikeys.data_ptr(), self.n_valid.data_ptr(),
                        nvm, self.sel.data_ptr(), sel_rows, int(has_entries), 0, 0, _ptr(ikey_scales),
                        int(pool_blocks), self.pool.data_ptr(), 0, 0)
        self._ws = None

    @property
    def has_selection(self) -> bool:
        return bool(self.c.has_selection)

    def set_n_valid_max(self, v: int):
        self.c.n_valid_max = int(v)

    def workspace_bytes(self, Qs: int, Hq: int, W: int) -> int:
        return int(_load().csa2_layer_workspace_bytes(ctypes.byref(self.c), Qs, Hq, W))

    def workspace(self, Qs: int, Hq: int, W: int) -> torch.Tensor:
        need = self.workspace_bytes(Qs, Hq, W)
        if self._ws is None or self._ws.numel() < need:
            self._ws = _workspace(need, self.codes.device)
        return self._ws

    def layer_step(self, mode: str, q, wk, wv, W: int, sm_scale: float, iq=None, new_entry=None,
                   new_ikey=None, wlen=None, out=None, lse=None, ws=None, stream=None, index_events=None):
        """One CSA2 layer in mode 'F' (Full), 'Ri' (Reindex) or 'Ru' (Reuse); returns (out, lse).
        index_events: optional pair of created torch.cuda.Event (enable_timing) that the library
        records around the layer's index-scoring kernels."""
        B, Qs, Hq, D = q.shape
        if out is None:
            out = torch.empty(B, Qs, Hq, D, dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty(B, Qs, Hq, dtype=torch.float32, device=q.device)
        if ws is None:
            ws = self.workspace(Qs, Hq, W)
        a = CLayerArgs(Qs, Hq, q.data_ptr(), _ptr(iq), _ptr(wk), _ptr(wv), W, _ptr(wlen),
                       _ptr(new_entry), _ptr(new_ikey), float(sm_scale), out.data_ptr(), _ptr(lse),
                       _events(index_events))
        st = _load().csa2_layer_step(MODE[mode], ctypes.byref(a), ctypes.byref(self.c), ws.data_ptr(),
                                     ws.numel(), _stream(stream))
        _check(st, f"csa2_layer_step({mode})")
        return out, lse

    def layer_step_noalloc(self, mode: str, q, wk, wv, W: int, sm_scale: float, iq=None, new_entry=None,
                           new_ikey=None, wlen=None, out=None, lse=None, stream=None):
        """layer_step through csa2_layer_step_noalloc: the library's own per-GPU scratch replaces
        the workspace.  out and lse must be given to allocate nothing here either."""
        B, Qs, Hq, D = q.shape
        if out is None:
            out = torch.empty(B, Qs, Hq, D, dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty(B, Qs, Hq, dtype=torch.float32, device=q.device)
        a = CLayerArgs(Qs, Hq, q.data_ptr(), _ptr(iq), _ptr(wk), _ptr(wv), W, _ptr(wlen),
                       _ptr(new_entry), _ptr(new_ikey), float(sm_scale), out.data_ptr(), _ptr(lse))
        st = _load().csa2_layer_step_noalloc(MODE[mode], ctypes.byref(a), ctypes.byref(self.c), _stream(stream))
        _check(st, f"csa2_layer_step_noalloc({mode})")
        return out, lse

    def image_bytes(self) -> int:
        """Size of the group's host-tier image (entries, keys, selection and pool)."""
        return int(_load().csa2_group_image_bytes(ctypes.byref(self.c)))

    def save(self, host: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Copy the group into a host byte tensor (pinned by default); asynchronous."""
        n = self.image_bytes()
        if host is None:
            host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
        if host.device.type != "cpu" or not host.is_contiguous():
            raise ValueError("host image must be a contiguous CPU tensor")
        st = _load().csa2_group_save(ctypes.byref(self.c), host.data_ptr(), host.numel() * host.element_size(),
                                     _stream(stream))
        _check(st, "csa2_group_save")
        return host

    def restore(self, host: torch.Tensor, stream=None):
        """Copy a host image back into the group's device buffers; asynchronous."""
        if host.device.type != "cpu" or not host.is_contiguous():
            raise ValueError("host image must be a contiguous CPU tensor")
        st = _load().csa2_group_restore(ctypes.byref(self.c), host.data_ptr(),
                                        host.numel() * host.element_size(), _stream(stream))
        _check(st, "csa2_group_restore")

    def step_status(self, mode: str, **kw) -> int:
        """Like layer_step but returns the status code instead of raising."""
        try:
            self.layer_step(mode, **kw)
            return OK
        except Csa2Error as e:
            return e.status
