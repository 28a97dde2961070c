"""csa2_layer_step_noalloc (the layer step on the library's per-GPU static scratch) against
csa2_layer_step with a caller workspace: two group runs in a row, the second smaller, so the
second runs on scratch the first left behind; then the w2 group at full size.  Named to be
collected last."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_03_amd as csa2
from cases import make_inputs, rel_err
from synth.workloads import W2, W8

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3


def dev(a):
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint16): np.int16}.get(a.dtype)
    return torch.from_numpy(a.view(view) if view is not None else a).to(DEV)


def _groups(wl, n_valid):
    inp = make_inputs(wl, n_valid=n_valid)
    B, N, D = wl.B, wl.N, wl.D
    out = []
    for _ in range(2):  # one group per entry point, same bytes
        codes, scales = csa2.fp4_pack(dev(inp.cache_x[0]))
        out.append(csa2.Group(codes, scales, dev(inp.ikeys[0]), dev(inp.n_valid), wl.idx_dtype, wl.k,
                              sel_rows=B * wl.Qs, pool_blocks=wl.pool_blocks))
    return inp, out[0], out[1]


def _run_both(wl, n_valid):
    print(f"noalloc case: {wl.name} B={wl.B} N={wl.N} n_valid={n_valid}", flush=True)
    inp, g_ws, g_st = _groups(wl, n_valid)
    for li, L in enumerate(inp.layers):
        kw = dict(q=dev(L["q"]), wk=dev(L["wk"]), wv=dev(L["wv"]), W=wl.W, sm_scale=wl.sm_scale)
        if L["iq"] is not None:
            kw["iq"] = dev(L["iq"])
        if L["new_entry"] is not None:
            kw["new_entry"] = dev(L["new_entry"])
            kw["new_ikey"] = dev(L["new_ikey"])
        o1, l1 = g_ws.layer_step(L["mode"], **kw)
        o2 = torch.empty_like(o1)
        l2 = torch.empty_like(l1)
        g_st.layer_step_noalloc(L["mode"], out=o2, lse=l2, **kw)
        torch.cuda.synchronize()
        assert torch.equal(g_ws.sel, g_st.sel), (li, L["mode"])
        assert rel_err(o2.cpu().numpy(), o1.cpu().numpy()) <= TOL, (li, L["mode"])
        assert np.allclose(l2.cpu().numpy(), l1.cpu().numpy(), rtol=0, atol=TOL)
        if wl.pool_blocks:
            assert torch.equal(g_ws.pool, g_st.pool)
    assert torch.equal(g_ws.codes, g_st.codes) and torch.equal(g_ws.ikeys, g_st.ikeys)


def test_noalloc_matches_workspace_entry_point_twice_second_smaller():
    _run_both(W2.scaled(B=8, N=40000), n_valid=[40000, 39000, 1, 20000, 40000, 7, 2048, 33333])
    _run_both(W8.scaled(B=3, N=9000, k=500, pool_blocks=200), n_valid=[9000, 4500, 8001])


def test_noalloc_full_size_decode_group():
    # the w2 group at its full size (30 MiB of scratch), after the smaller calls above
    _run_both(W2, n_valid=None)
