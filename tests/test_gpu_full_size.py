"""Parity at the workloads' full sizes, in the launch configuration the bench times.

The decode workloads (batch 32 x 65,536 entries, the draft-block, FP4-key and
hierarchical variants, and batch 8 x 262,144 entries) are compared against the
oracle in full: every selection bit-exact, every attention output within the
stated tolerance.  The prefill chunk (4,096 queries against 131,072 causal
entries) is too large for the oracle as a whole; its GPU selection is checked
for validity on every row and against the oracle exactly on 256 sampled rows
(every 256-row tile edge and the last 64 rows among them), attention included.
"""
import numpy as np
import pytest
import torch

import compressed_kv_cache_03_amd as csa2
import oracle
from cases import make_inputs, rel_err
from synth.workloads import W2, W3, W4, W5, W6, W7, W8
from test_gpu_parity import TOL, Run, dev, host

pytestmark = pytest.mark.gpu


def test_w2_full_size():
    Run(W2).check_all()


def test_w3_full_size_fp8():
    Run(W3).check_all()


def test_w6_full_size_draft_block():
    Run(W6).check_all()


def test_w7_full_size_fp4_index_keys():
    Run(W7).check_all()


def test_w8_full_size_hierarchical():
    Run(W8).check_all()


def test_w5_full_size_stack_two_sequences_against_the_oracle():
    # the 16-layer stack (4 groups of Full/Reindex/Reuse/Reuse, batch 64 x 131,072 entries) runs
    # whole on the GPU; sequences are independent, so the oracle follows the first and the last
    wl = W5
    B, N, D = wl.B, wl.N, wl.D
    seqs = np.array([0, B - 1])
    inp = make_inputs(wl)
    g_gpu, g_orc = [], []
    for g in range(wl.groups):
        x = dev(inp.cache_x[g])
        gc, gs = csa2.fp4_pack(x)
        del x
        g_gpu.append(csa2.Group(gc, gs, dev(inp.ikeys[g]), dev(inp.n_valid), wl.idx_dtype, wl.k, sel_rows=B))
        oc, os_ = oracle.fp4_pack(np.ascontiguousarray(inp.cache_x[g][seqs]).reshape(-1, D))
        g_orc.append(oracle.Group(oc.reshape(2, N, D // 2), os_.reshape(2, N, D // 32),
                                  np.ascontiguousarray(inp.ikeys[g][seqs]), inp.n_valid[seqs].astype(np.int64),
                                  wl.idx_dtype, wl.k, max_rows=2))
        inp.cache_x[g] = inp.ikeys[g] = None  # the host copies are no longer needed
    torch.cuda.synchronize()
    for li, L in enumerate(inp.layers):
        g, mode = L["group"], L["mode"]
        kw = dict(q=L["q"], wk=L["wk"], wv=L["wv"], W=wl.W, sm_scale=np.float32(wl.sm_scale))
        if L["iq"] is not None:
            kw["iq"] = L["iq"]
        if L["new_entry"] is not None:
            kw["new_entry"] = L["new_entry"]
            kw["new_ikey"] = L["new_ikey"]
        go, _ = g_gpu[g].layer_step(mode, **{k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in kw.items()})
        rc, ro, _ = g_orc[g].layer_step(mode, **{k: (np.ascontiguousarray(v[seqs]) if isinstance(v, np.ndarray) else v)
                                                 for k, v in kw.items()})
        assert rc == 0
        torch.cuda.synchronize()
        assert np.array_equal(host(g_gpu[g].sel)[seqs], g_orc[g].sel[:2]), (li, mode)
        err = rel_err(host(go)[seqs], ro)
        assert err <= TOL, (li, mode, err)


def test_w4_full_size_prefill_sampled_rows():
    wl = W4
    B, N, D, Qs, W, k = wl.B, wl.N, wl.D, wl.Qs, wl.W, wl.k
    assert B == 1
    inp = make_inputs(wl)
    L = inp.layers[0]
    x = inp.cache_x[0]

    # GPU: the whole chunk, as the bench runs it
    gc, gs = csa2.fp4_pack(dev(x))
    grp = csa2.Group(gc, gs, dev(inp.ikeys[0]), dev(inp.n_valid), wl.idx_dtype, k, sel_rows=B * Qs)
    out, _ = grp.layer_step("F", q=dev(L["q"]), iq=dev(L["iq"]), wk=dev(L["wk"]), wv=dev(L["wv"]), W=W,
                            sm_scale=wl.sm_scale, new_entry=dev(L["new_entry"]), new_ikey=dev(L["new_ikey"]))
    torch.cuda.synchronize()
    sel = host(grp.sel)[:Qs]
    out = host(out).reshape(Qs, wl.Hq, D)

    # every row: ascending distinct valid indices, min(k, visible) of them, then -1
    visible = N - Qs + 1 + np.arange(Qs)
    take = np.minimum(k, visible)
    pos = np.arange(k)[None, :]
    assert np.all((sel >= 0) == (pos < take[:, None]))
    d = np.diff(sel.astype(np.int64), axis=1)
    assert np.all(d[pos[:, 1:] < take[:, None]] > 0)
    assert np.all(sel < visible[:, None])

    # oracle on sampled rows: the cache after the chunk's own write (rows N-Qs..N-1
    # packed from the new entries; their index keys stored), then the row's exact
    # causal scores, top-k and joint attention with its own window rows
    codes, scales = oracle.fp4_pack(x.reshape(N, D))
    ncodes, nscales = oracle.fp4_pack(L["new_entry"].reshape(Qs, D))
    codes = codes.reshape(N, D // 2).copy()
    scales = scales.reshape(N, D // 32).copy()
    codes[N - Qs:] = ncodes.reshape(Qs, D // 2)
    scales[N - Qs:] = nscales.reshape(Qs, D // 32)
    ikeys = inp.ikeys[0].copy()
    ikeys[0, N - Qs:] = L["new_ikey"][0]
    # 256 rows: both sides of every 256-row tile edge, the first rows, the last 64
    # (the ones that see the chunk's own new entries most) and random rows
    rows = {0, 1} | {e + o for e in range(256, Qs, 256) for o in (-1, 0)} | set(range(Qs - 64, Qs))
    rng = np.random.default_rng(4096)
    while len(rows) < 256:
        rows.add(int(rng.integers(0, Qs)))
    rows = np.array(sorted(rows))
    nv = visible[rows].astype(np.int64)
    sc = oracle.index_score(wl.idx_dtype, np.ascontiguousarray(L["iq"][:, rows]), ikeys, n_valid_row=nv)
    ref_sel = oracle.topk(sc.reshape(len(rows), N), k, n_valid=nv)
    bad = [int(i) for i, r in zip(rows, ref_sel) if not np.array_equal(sel[i], r)]
    assert not bad, bad
    for t, i in enumerate(rows):
        ro, _ = oracle.attend(L["q"][:, i:i + 1], codes.reshape(1, N, D // 2), scales.reshape(1, N, D // 32),
                              ref_sel[t:t + 1], L["wk"][:, i:i + W], L["wv"][:, i:i + W], W,
                              np.float32(wl.sm_scale))
        err = rel_err(out[i], ro.reshape(wl.Hq, D))
        assert err <= TOL, (i, err)


def test_w4_full_size_prefill_run_to_run_bitwise():
    # candidate regions are filled through atomics, so their order varies between
    # runs; the selection (sorted) and the attention over it must not
    wl = W4
    inp = make_inputs(wl)
    L = inp.layers[0]
    gc, gs = csa2.fp4_pack(dev(inp.cache_x[0]))
    keys = dev(inp.ikeys[0])
    kw = dict(q=dev(L["q"]), iq=dev(L["iq"]), wk=dev(L["wk"]), wv=dev(L["wv"]), W=wl.W, sm_scale=wl.sm_scale,
              new_entry=dev(L["new_entry"]), new_ikey=dev(L["new_ikey"]))
    runs = []
    for _ in range(2):
        grp = csa2.Group(gc.clone(), gs.clone(), keys.clone(), dev(inp.n_valid), wl.idx_dtype, wl.k,
                         sel_rows=wl.B * wl.Qs)
        out, lse = grp.layer_step("F", **kw)
        torch.cuda.synchronize()
        runs.append((host(grp.sel), host(out), host(lse)))
    assert np.array_equal(runs[0][0], runs[1][0])
    assert np.array_equal(runs[0][1].view(np.uint32), runs[1][1].view(np.uint32))
    assert np.array_equal(runs[0][2].view(np.uint32), runs[1][2].view(np.uint32))


def test_w2_full_size_host_tier_round_trip_resumes_against_the_oracle():
    # the bench's host-tier leg at its size: the group after its Full layer goes to a
    # pinned host image (about 1.24 GB), its device buffers are overwritten, the image
    # comes back, every stored byte and the selection are as before, and the Reindex and
    # Reuse layers that follow still match the oracle, which never left the host
    run = Run(W2)
    mode, gi, ro, rl, go, gl = run.layer(0)
    assert mode == "F"
    g = run.g_gpu[0]
    assert np.array_equal(host(g.sel), run.g_orc[0].sel)
    before = [t.clone() for t in (g.codes, g.scales, g.ikeys, g.sel)]
    image = g.save()
    torch.cuda.synchronize()
    assert image.numel() == g.image_bytes()
    g.codes.fill_(0x5A)
    g.scales.fill_(float("nan"))
    g.ikeys.fill_(0x7FC1)
    g.sel.fill_(-7)
    g.restore(image)
    torch.cuda.synchronize()
    for a, b in zip(before, (g.codes, g.scales, g.ikeys, g.sel)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    del before
    for li in range(1, 4):
        mode, gi, ro, rl, go, gl = run.layer(li)
        assert np.array_equal(host(g.sel), run.g_orc[0].sel), (li, mode)
        assert rel_err(go, ro) <= TOL, (li, mode)
        assert np.allclose(gl, rl, rtol=0, atol=TOL), (li, mode)
