"""Seeded host inputs of a workload: identical bytes for the oracle and the GPU path.

Stream ids and layouts are listed in workloads.py.  A case may shrink B / N / Qs from a
workload's full size; the recipe (N(0,1), dtypes, k, window) is the workload's.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import normal_bf16, normal_f32, normal_idx
from .workloads import Workload


@dataclasses.dataclass
class Inputs:
    wl: Workload
    cache_x: list      # per group: fp32 [B, N, D]
    ikeys: list        # per group: bits [B, N, H, d] (fp4 keys: fp32 values, packed by each side)
    layers: list       # per layer: dict(q, iq, wk, wv, new_entry, new_ikey)
    n_valid: np.ndarray  # int32 [B]


def idx_np_dtype(wl: Workload):
    return np.uint16 if wl.idx_dtype == "bf16" else np.uint8


def query_dtype(wl: Workload) -> str:
    """Storage dtype of the index queries: bf16 queries go with FP4 keys."""
    return "bf16" if wl.idx_dtype == "fp4" else wl.idx_dtype


def make_inputs(wl: Workload, n_valid=None, groups=None) -> Inputs:
    B, N, D, H, d, Qs, W, Hq = wl.B, wl.N, wl.D, wl.H_I, wl.d_I, wl.Qs, wl.W, wl.Hq
    G = wl.groups if groups is None else groups
    cache_x, ikeys, layers = [], [], []
    for g in range(G):
        cache_x.append(normal_f32(wl.seed(wl.stream(g, 0, 0)), B * N * D).reshape(B, N, D))
        ikeys.append(normal_idx(wl.idx_dtype, wl.seed(wl.stream(g, 0, 1)), B * N * H * d)
                     .reshape(B, N, H, d))
        for li, mode in enumerate(wl.pattern):
            st = lambda kind: wl.seed(wl.stream(g, li, kind))  # noqa: E731
            L = dict(
                mode=mode,
                q=normal_bf16(st(3), B * Qs * Hq * D).reshape(B, Qs, Hq, D),
                wk=normal_bf16(st(4), B * (Qs + W - 1) * D).reshape(B, Qs + W - 1, D),
                wv=normal_bf16(st(5), B * (Qs + W - 1) * D).reshape(B, Qs + W - 1, D),
                iq=None, new_entry=None, new_ikey=None, group=g)
            if mode in ("F", "Ri"):
                L["iq"] = normal_idx(query_dtype(wl), st(2), B * Qs * H * d).reshape(B, Qs, H, d)
            if mode == "F":
                L["new_entry"] = normal_f32(st(6), B * Qs * D).reshape(B, Qs, D)
                L["new_ikey"] = normal_idx(wl.idx_dtype, st(7), B * Qs * H * d).reshape(B, Qs, H, d)
            layers.append(L)
    nv = np.full(B, N, np.int32) if n_valid is None else np.asarray(n_valid, np.int32)
    return Inputs(wl, cache_x, ikeys, layers, nv)
