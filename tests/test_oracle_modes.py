"""Pins of the oracle's layer modes and cache accounting.

Mode semantics ("DeepSeek-V4.1-Flash", section "Sharing the cache across layers"):
Full computes its own entries and selection, Reindex shares entries but selects
afresh, Reuse shares both; every layer keeps its own queries and window.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _group(dtype="bf16", B=2, N=64, H=2, d=64, D=64, k=8, seed=200):
    x = synth.normal_f32(synth.seed(0, seed), B * N * D).reshape(B * N, D)
    codes, scales = oracle.fp4_pack(x)
    ik = synth.normal_idx(dtype, synth.seed(0, seed + 1), B * N * H * d).reshape(B, N, H, d)
    g = oracle.Group(codes.reshape(B, N, D // 2), scales.reshape(B, N, D // 32), ik,
                     np.full(B, N, np.int64), dtype, k, max_rows=B)
    return g


def _layer(B=2, H=2, d=64, D=64, Hq=4, W=8, seed=300, dtype="bf16"):
    q = synth.normal_bf16(synth.seed(0, seed), B * Hq * D).reshape(B, 1, Hq, D)
    iq = synth.normal_idx(dtype, synth.seed(0, seed + 1), B * H * d).reshape(B, 1, H, d)
    wk = synth.normal_bf16(synth.seed(0, seed + 2), B * W * D).reshape(B, W, D)
    wv = synth.normal_bf16(synth.seed(0, seed + 3), B * W * D).reshape(B, W, D)
    ne = synth.normal_f32(synth.seed(0, seed + 4), B * D).reshape(B, 1, D)
    nk = synth.normal_idx(dtype, synth.seed(0, seed + 5), B * H * d).reshape(B, 1, H, d)
    return dict(q=q, iq=iq, wk=wk, wv=wv, new_entry=ne, new_ikey=nk, W=W, sm_scale=0.125)


def _checksum(g):
    return (g.codes.tobytes(), g.scales.tobytes(), g.ikeys.tobytes())


def test_reuse_equals_full_given_identical_indices():
    g = _group()
    L = _layer()
    rc, out_f, lse_f = g.layer_step("F", **L)
    assert rc == 0
    rc, out_r, lse_r = g.layer_step("Ru", q=L["q"], wk=L["wk"], wv=L["wv"], W=L["W"],
                                    sm_scale=L["sm_scale"])
    assert rc == 0
    assert np.array_equal(out_f.view(np.uint32), out_r.view(np.uint32))
    assert np.array_equal(lse_f.view(np.uint32), lse_r.view(np.uint32))


def test_reindex_with_full_query_reproduces_selection_and_writes_nothing():
    g = _group()
    L = _layer()
    assert g.layer_step("F", **L)[0] == 0
    sel_full = g.sel.copy()
    before = _checksum(g)
    rc, out_ri, _ = g.layer_step("Ri", q=L["q"], iq=L["iq"], wk=L["wk"], wv=L["wv"], W=L["W"],
                                 sm_scale=L["sm_scale"])
    assert rc == 0
    assert np.array_equal(g.sel, sel_full)
    assert _checksum(g) == before
    L2 = _layer(seed=400)
    rc, _, _ = g.layer_step("Ri", q=L2["q"], iq=L2["iq"], wk=L2["wk"], wv=L2["wv"], W=8, sm_scale=0.125)
    assert rc == 0 and _checksum(g) == before
    # the fresh selection is the top-k of the new index query's scores
    s = oracle.index_score("bf16", L2["iq"], g.ikeys)
    assert np.array_equal(g.sel, oracle.topk(s.reshape(2, -1), 8))
    sel_ri = g.sel.copy()
    assert g.layer_step("Ru", q=L2["q"], wk=L2["wk"], wv=L2["wv"], W=8, sm_scale=0.125)[0] == 0
    assert np.array_equal(g.sel, sel_ri) and _checksum(g) == before


def test_full_writes_the_new_entry_at_the_last_valid_slot():
    g = _group()
    L = _layer()
    old = _checksum(g)
    assert g.layer_step("F", **L)[0] == 0
    c, s = oracle.fp4_pack(L["new_entry"].reshape(2, 64))
    assert np.array_equal(g.codes[:, -1], c) and np.array_equal(g.scales[:, -1], s)
    assert np.array_equal(g.ikeys[:, -1], L["new_ikey"][:, 0])
    assert g.codes[:, :-1].tobytes() == np.frombuffer(old[0], np.uint8).reshape(g.codes.shape)[:, :-1].tobytes()


def test_state_errors():
    g = _group()
    L = _layer()
    rc, _, _ = g.layer_step("Ru", q=L["q"], wk=L["wk"], wv=L["wv"], W=8, sm_scale=0.125)
    assert rc == 4  # Reuse before any selection
    g2 = oracle.Group(g.codes, g.scales, g.ikeys, g.n_valid, "bf16", 8, 2, has_entries=False)
    rc, _, _ = g2.layer_step("Ri", q=L["q"], iq=L["iq"], wk=L["wk"], wv=L["wv"], W=8, sm_scale=0.125)
    assert rc == 4  # Reindex on a group with no entries


def test_cache_bytes_worked_figure():
    rows = [list(map(int, l.split())) for l in open(os.path.join(GOLDEN, "cache_figure.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 2
    for entries, numbers, copies, bits, want in rows:
        assert oracle.cache_bytes(entries, numbers, copies, bits) == want
    assert rows[0][4] == 8 * 2 ** 20 and rows[1][4] == 2 * 2 ** 20
