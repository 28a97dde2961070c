"""C-ABI library: it loads, exports every declared entry point, and validates its
arguments on the host before anything reaches the GPU (no device is touched here)."""
import ctypes
import os
import re

import pytest

import compressed_kv_cache_03_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

FAKE = 0x10000  # aligned, never dereferenced: validation fails before any launch


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(csa2.LIB_PATH)
    names = _declared()
    assert {"csa2_fp4_pack", "csa2_index_score", "csa2_topk", "csa2_sparse_attend",
            "csa2_layer_step"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    for code, name in enumerate(["CSA2_OK", "CSA2_ERR_INVALID_ARG", "CSA2_ERR_UNSUPPORTED",
                                 "CSA2_ERR_WORKSPACE", "CSA2_ERR_STATE", "CSA2_ERR_HIP"]):
        assert csa2.status_str(code) == name
    assert csa2.version().startswith("csa2-gfx950")


def test_cache_bytes_worked_figure_and_overflow():
    assert csa2.cache_bytes(4096, 128, 16, 8) == 8388608
    assert csa2.cache_bytes(4096, 128, 4, 8) == 2097152
    assert csa2.cache_bytes(-1, 1, 1, 8) == -1
    assert csa2.cache_bytes(1 << 40, 1 << 20, 1 << 10, 8) == -1


def test_fp4_pack_validation():
    L = csa2.lib()
    assert L.csa2_fp4_pack(FAKE, 4, 48, FAKE, FAKE, None) == csa2.ERR_INVALID_ARG  # dim % 32
    assert L.csa2_fp4_pack(FAKE, -1, 128, FAKE, FAKE, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_fp4_pack(None, 4, 128, FAKE, FAKE, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_fp4_pack(FAKE + 4, 4, 128, FAKE, FAKE, None) == csa2.ERR_INVALID_ARG  # misaligned
    assert L.csa2_fp4_pack(None, 0, 128, None, None, None) == csa2.OK  # empty: no-op


def test_index_score_validation():
    L = csa2.lib()
    assert L.csa2_index_score(FAKE, FAKE, None, 0, 1, 1, 10, 64, 65, -1, 1, FAKE, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_index_score(FAKE, FAKE, None, 7, 1, 1, 10, 4, 64, -1, 1, FAKE, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_index_score(FAKE, FAKE, None, 0, 1, 0, 10, 4, 64, -1, 1, FAKE, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_index_score(None, FAKE, None, 0, 1, 1, 10, 4, 64, -1, 1, FAKE, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_index_score(FAKE, FAKE, None, 0, 1, 1, 1 << 31, 4, 64, -1, 1, FAKE, None) == csa2.ERR_UNSUPPORTED
    assert L.csa2_index_score(FAKE, FAKE, None, 0, 1, 1, 0, 4, 64, -1, 1, FAKE, None) == csa2.OK
    # FP4 keys need their scales, and whole 32-element blocks
    assert L.csa2_index_score(FAKE, FAKE, None, 2, 1, 1, 10, 4, 64, -1, 1, FAKE, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_index_score(FAKE, FAKE, FAKE, 2, 1, 1, 10, 1, 48, -1, 1, FAKE, None) == csa2.ERR_INVALID_ARG
    # causal offsets below -1 are invalid; 0 and beyond are accepted for any N
    assert L.csa2_index_score(FAKE, FAKE, None, 0, 1, 1, 10, 4, 64, -2, 1, FAKE, None) == csa2.ERR_INVALID_ARG
    # a launch beyond 2^32 - 1 work-items (B*Qs*N about 4.3e9) is refused before anything is enqueued
    assert L.csa2_index_score(FAKE, FAKE, None, 0, 4096, 1, 1 << 20, 4, 64, -1, 1, FAKE, None) == csa2.ERR_UNSUPPORTED
    assert L.csa2_index_score(FAKE, FAKE, None, 0, 64, 64, 1 << 20, 4, 64, 5, 0, FAKE, None) == csa2.ERR_UNSUPPORTED
    assert L.csa2_fp4_pack(FAKE, 1 << 33, 128, FAKE, FAKE, None) == csa2.ERR_UNSUPPORTED


def test_topk_validation():
    L = csa2.lib()
    need = L.csa2_topk_workspace_bytes(4, 1000, 16)
    assert need > 4 * 4096 * 4
    assert L.csa2_topk(FAKE, 4, 1000, 1000, None, 0, FAKE, FAKE, need, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_topk(FAKE, 4, 1000, 999, None, 8, FAKE, FAKE, need, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_topk(FAKE, 4, 1000, 1000, None, 8, FAKE, FAKE, need - 1, None) == csa2.ERR_WORKSPACE
    assert L.csa2_topk(FAKE, 4, 1000, 1000, None, 8, FAKE, None, need, None) == csa2.ERR_WORKSPACE


def test_attend_validation():
    L = csa2.lib()
    need = L.csa2_attend_workspace_bytes(2, 1, 16, 128, 64, 128)
    args = [FAKE, 2, 1, 16, 128, FAKE, FAKE, 100, FAKE, 64, FAKE, FAKE, 128, None, 0.0884, FAKE,
            FAKE, FAKE, need, None]
    bad_d = list(args)
    bad_d[4] = 100
    assert L.csa2_sparse_attend(*bad_d) == csa2.ERR_INVALID_ARG
    bad_h = list(args)
    bad_h[3] = 33
    assert L.csa2_sparse_attend(*bad_h) == csa2.ERR_INVALID_ARG
    nan = list(args)
    nan[14] = float("nan")
    assert L.csa2_sparse_attend(*nan) == csa2.ERR_INVALID_ARG
    small = list(args)
    small[18] = need - 1
    assert L.csa2_sparse_attend(*small) == csa2.ERR_WORKSPACE


def _group(**over):
    g = csa2.CGroup(2, 1000, 128, 4, 64, 0, 64, FAKE, FAKE, FAKE, FAKE, 1000, FAKE, 2, 1, 0, 0)
    for k, v in over.items():
        setattr(g, k, v)
    return g


def _args(**over):
    a = csa2.CLayerArgs(1, 16, FAKE, FAKE, FAKE, FAKE, 128, None, FAKE, FAKE, 0.0884, FAKE, FAKE)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def _step(mode, g, a, ws_bytes=None):
    L = csa2.lib()
    need = L.csa2_layer_workspace_bytes(ctypes.byref(g), a.Qs, a.Hq, a.W)
    return L.csa2_layer_step(mode, ctypes.byref(a), ctypes.byref(g), FAKE,
                             need if ws_bytes is None else ws_bytes, None)


def test_layer_step_state_machine_errors():
    # Reuse before any selection, Reindex with no entries: state errors, nothing launched
    assert _step(2, _group(), _args()) == csa2.ERR_STATE
    assert _step(1, _group(has_entries=0), _args()) == csa2.ERR_STATE
    # Reuse of a selection made for another Qs
    assert _step(2, _group(has_selection=1, sel_qs=4), _args()) == csa2.ERR_STATE


def test_layer_step_argument_errors():
    assert _step(3, _group(), _args()) == csa2.ERR_INVALID_ARG               # unknown mode
    assert _step(0, _group(D=100), _args()) == csa2.ERR_INVALID_ARG          # D % 32
    assert _step(0, _group(k=0), _args()) == csa2.ERR_INVALID_ARG            # k < 1
    assert _step(0, _group(k=1001), _args()) == csa2.ERR_INVALID_ARG         # k > N_cap
    assert _step(0, _group(n_valid_max=1001), _args()) == csa2.ERR_INVALID_ARG
    assert _step(0, _group(), _args(new_entry=None)) == csa2.ERR_INVALID_ARG  # Full needs new rows
    assert _step(1, _group(), _args(iq=None)) == csa2.ERR_INVALID_ARG        # Reindex needs iq
    assert _step(0, _group(sel_rows=1), _args()) == csa2.ERR_INVALID_ARG     # sel too small
    assert _step(0, _group(), _args(Hq=0)) == csa2.ERR_INVALID_ARG
    assert _step(0, _group(), _args(), ws_bytes=100) == csa2.ERR_WORKSPACE
    assert _step(0, _group(B=70000), _args()) == csa2.ERR_UNSUPPORTED
    # launches beyond 2^32 - 1 work-items are refused before the Full layer writes anything:
    # the decode score stream (B * N > 4.3e9) and the prefill score GEMM
    big = dict(B=8192, N_cap=1 << 20, n_valid_max=1 << 20, sel_rows=8192)
    assert _step(0, _group(**big), _args()) == csa2.ERR_UNSUPPORTED
    assert _step(1, _group(**big), _args()) == csa2.ERR_UNSUPPORTED
    pre = dict(B=1, N_cap=1 << 30, n_valid_max=1 << 30, idx_dtype=1, sel_rows=60000)
    assert _step(0, _group(**pre), _args(Qs=60000)) == csa2.ERR_UNSUPPORTED


def test_group_image_bytes_and_save_restore_validation():
    L = csa2.lib()
    g = _group()  # B=2, N_cap=1000, D=128, 4x64 bf16, k=64, n_valid_max=1000, no selection
    per_entry = 128 // 2 + 128 // 32 * 4 + 4 * 64 * 2  # codes + scales + bf16 keys
    assert L.csa2_group_image_bytes(ctypes.byref(g)) == 2 * 1000 * per_entry
    gs = _group(has_selection=1, sel_qs=1, n_valid_max=300, idx_dtype=1)
    per_entry8 = 128 // 2 + 128 // 32 * 4 + 4 * 64
    assert L.csa2_group_image_bytes(ctypes.byref(gs)) == 2 * 300 * per_entry8 + 2 * 1 * 64 * 4
    assert L.csa2_group_image_bytes(ctypes.byref(_group(D=100))) == 0
    assert L.csa2_group_image_bytes(ctypes.byref(_group(has_selection=1, sel_qs=2))) == 0  # sel_rows 2 < B*2
    need = L.csa2_group_image_bytes(ctypes.byref(g))
    # every error is found before a copy is queued
    assert L.csa2_group_save(ctypes.byref(g), None, need, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_group_save(ctypes.byref(g), FAKE, need - 1, None) == csa2.ERR_WORKSPACE
    assert L.csa2_group_save(ctypes.byref(_group(has_entries=0)), FAKE, need, None) == csa2.ERR_STATE
    assert L.csa2_group_restore(ctypes.byref(g), FAKE, need - 1, None) == csa2.ERR_WORKSPACE
    assert L.csa2_group_restore(ctypes.byref(_group(codes=None)), FAKE, need, None) == csa2.ERR_INVALID_ARG


def test_fp4_index_keys_validation_and_image():
    # FP4 keys: the group needs its key scales; the image carries them after the codes
    assert _step(0, _group(idx_dtype=2), _args()) == csa2.ERR_INVALID_ARG
    assert _step(0, _group(idx_dtype=2, H_I=1, d_I=48, ikey_scales=FAKE), _args()) == csa2.ERR_INVALID_ARG
    L = csa2.lib()
    g = _group(idx_dtype=2, ikey_scales=FAKE, n_valid_max=10)
    per_entry = 128 // 2 + 128 // 32 * 4 + 4 * 64 // 2 + 4 * 64 // 32 * 4
    assert L.csa2_group_image_bytes(ctypes.byref(g)) == 2 * 10 * per_entry


def test_hierarchical_pool_validation_and_image():
    # a pool needs room for k entries, at most one block per 8 cache slots, and a buffer
    assert _step(0, _group(pool_blocks=-1), _args()) == csa2.ERR_INVALID_ARG
    assert _step(0, _group(pool_blocks=7, pool=FAKE), _args()) == csa2.ERR_INVALID_ARG    # 56 < k = 64
    assert _step(0, _group(pool_blocks=126, pool=FAKE), _args()) == csa2.ERR_INVALID_ARG  # > 1000/8 blocks
    assert _step(0, _group(pool_blocks=8), _args()) == csa2.ERR_INVALID_ARG               # no pool buffer
    # Reindex in a hierarchical group needs the pool of a Full layer with the same Qs
    assert _step(1, _group(pool_blocks=8, pool=FAKE), _args()) == csa2.ERR_STATE
    assert _step(1, _group(pool_blocks=8, pool=FAKE, has_pool=1, pool_qs=2), _args()) == csa2.ERR_STATE
    L = csa2.lib()
    g = _group(n_valid_max=10, has_selection=1, sel_qs=1, pool_blocks=8, pool=FAKE, has_pool=1, pool_qs=1)
    per_entry = 128 // 2 + 128 // 32 * 4 + 4 * 64 * 2
    assert L.csa2_group_image_bytes(ctypes.byref(g)) == 2 * 10 * per_entry + 2 * 64 * 4 + 2 * 8 * 4
    assert L.csa2_group_save(ctypes.byref(_group(has_pool=1, pool_qs=1, pool_blocks=8)), FAKE, 10 ** 9,
                             None) == csa2.ERR_INVALID_ARG  # image with a pool needs the buffer


def test_layer_step_noalloc_validation():
    # the same checks as csa2_layer_step, then the scratch limit; all before any HIP call
    L = csa2.lib()
    ab = lambda g, a, mode=0: L.csa2_layer_step_noalloc(mode, ctypes.byref(a), ctypes.byref(g), None)  # noqa: E731
    assert ab(_group(), _args(), mode=2) == csa2.ERR_STATE
    assert ab(_group(D=100), _args()) == csa2.ERR_INVALID_ARG
    assert ab(_group(B=70000), _args()) == csa2.ERR_UNSUPPORTED
    # a layer whose workspace exceeds the static scratch is refused
    g = _group(B=64, N_cap=131072, n_valid_max=131072, sel_rows=64 * 5)
    assert L.csa2_layer_workspace_bytes(ctypes.byref(g), 5, 16, 128) > csa2.STATIC_SCRATCH_BYTES
    assert ab(g, _args(Qs=5)) == csa2.ERR_WORKSPACE
    assert L.csa2_layer_workspace_bytes(ctypes.byref(g), 1, 16, 128) <= csa2.STATIC_SCRATCH_BYTES


def test_out_of_range_enums_are_rejected():
    # a C caller can pass any integer where an enum is declared: rejected, nothing launched
    L = csa2.lib()
    assert L.csa2_index_score(FAKE, FAKE, None, 3, 1, 1, 10, 4, 64, -1, 1, FAKE, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_index_score(FAKE, FAKE, None, -1, 1, 1, 10, 4, 64, -1, 1, FAKE, None) == csa2.ERR_INVALID_ARG
    assert _step(7, _group(), _args()) == csa2.ERR_INVALID_ARG
    assert _step(-1, _group(), _args()) == csa2.ERR_INVALID_ARG
    assert _step(0, _group(idx_dtype=9), _args()) == csa2.ERR_INVALID_ARG
    assert L.csa2_layer_workspace_bytes(ctypes.byref(_group(idx_dtype=9)), 1, 16, 128) == 0
    assert L.csa2_group_image_bytes(ctypes.byref(_group(idx_dtype=-3))) == 0
