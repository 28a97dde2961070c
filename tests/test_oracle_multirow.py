"""Pins of the oracle's multi-row steps and partial windows.

Three behaviours that every prefill, draft-block and ragged-window parity case rests on:

* causal visibility ("Why Is DeepSeek V4.1 Flash So Fast?", section 3: each query
  retrieves from the compressed positions before it).  Row i of a Qs-row step sits at
  entry n_valid-Qs+i and sees entries j <= n_valid-Qs+i;
* where a Full layer writes the step's new rows ("DeepSeek-V4.1-Flash", "Sharing the
  cache across layers": Full makes its own entries): row i goes to slot n_valid-Qs+i;
* the partial window ("Why Is DeepSeek V4.1 Flash So Fast?", section 3, the 128-token
  window; "Inference-Efficient LLMs", section 4: every mode keeps its own window
  state).  Query i uses buffer rows i..i+W-1 of the [Qs+W-1] buffer, of which only the
  last wlen rows are valid, i.e. rows max(i, Qs+W-1-wlen) .. i+W-1.

Each expected value below is written from those statements alone: a Python sort for the
selection, the pinned FP4 codec for the written rows, and a scipy softmax over an
explicit row list for the window.  A misplaced cut-off, a reversed row order or a window
start off by one fails here.
"""
import numpy as np
import pytest
import scipy.special

import oracle
import synth


def _bf16(x):
    return synth.bf16_bits_to_f32(x).astype(np.float64)


def _brute_topk(row, k, visible):
    order = sorted(range(visible), key=lambda j: (-float(row[j]), j))
    sel = sorted(order[:k])
    return sel + [-1] * (k - len(sel))


def _multirow_case(B=3, N=48, Qs=4, H=2, d=32, D=64, Hq=2, W=6, seed=700, dtype="bf16"):
    x = synth.normal_f32(synth.seed(0, seed), B * N * D).reshape(B * N, D)
    codes, scales = oracle.fp4_pack(x)
    ik = synth.normal_idx(dtype, synth.seed(0, seed + 1), B * N * H * d).reshape(B, N, H, d)
    nv = np.array([N, N - 7, Qs + 3][:B], np.int64)  # ragged; the last one barely holds the step
    layer = dict(
        q=synth.normal_bf16(synth.seed(0, seed + 2), B * Qs * Hq * D).reshape(B, Qs, Hq, D),
        iq=synth.normal_idx(dtype, synth.seed(0, seed + 3), B * Qs * H * d).reshape(B, Qs, H, d),
        wk=synth.normal_bf16(synth.seed(0, seed + 4), B * (Qs + W - 1) * D).reshape(B, Qs + W - 1, D),
        wv=synth.normal_bf16(synth.seed(0, seed + 5), B * (Qs + W - 1) * D).reshape(B, Qs + W - 1, D),
        new_entry=synth.normal_f32(synth.seed(0, seed + 6), B * Qs * D).reshape(B, Qs, D),
        new_ikey=synth.normal_idx(dtype, synth.seed(0, seed + 7), B * Qs * H * d).reshape(B, Qs, H, d),
        W=W, sm_scale=0.125)
    return codes.reshape(B, N, D // 2), scales.reshape(B, N, D // 32), ik, nv, layer


@pytest.mark.parametrize("k", [5, 48])
def test_full_multirow_step_cutoff_and_write_slots(k):
    B, N, Qs = 3, 48, 4
    codes, scales, ik, nv, L = _multirow_case(B=B, N=N, Qs=Qs)
    g = oracle.Group(codes.copy(), scales.copy(), ik.copy(), nv, "bf16", k, max_rows=B * Qs)
    rc, _, _ = g.layer_step("F", **L)
    assert rc == 0

    # write slots: new row i of sequence b lands at n_valid[b]-Qs+i, nothing else changes
    want_codes, want_scales, want_keys = codes.copy(), scales.copy(), ik.copy()
    for b in range(B):
        c, s = oracle.fp4_pack(L["new_entry"][b])
        for i in range(Qs):
            slot = int(nv[b]) - Qs + i
            want_codes[b, slot], want_scales[b, slot] = c[i], s[i]
            want_keys[b, slot] = L["new_ikey"][b, i]
    assert np.array_equal(g.codes, want_codes)
    assert np.array_equal(g.scales.view(np.uint32), want_scales.view(np.uint32))
    assert np.array_equal(g.ikeys, want_keys)

    # selection: row i of sequence b ranks entries 0 .. n_valid[b]-Qs+i only
    s_all = oracle.index_score("bf16", L["iq"], want_keys)  # [B, Qs, N], no cut-off
    for b in range(B):
        for i in range(Qs):
            visible = int(nv[b]) - Qs + i + 1
            assert g.sel[b * Qs + i].tolist() == _brute_topk(s_all[b, i], k, visible), (b, i)
    if k >= N:  # every visible entry is kept: the count is the cut-off itself
        for b in range(B):
            for i in range(Qs):
                assert int((g.sel[b * Qs + i] >= 0).sum()) == int(nv[b]) - Qs + i + 1


def test_reindex_multirow_step_uses_the_same_cutoff():
    B, N, Qs, k = 3, 48, 4, 6
    codes, scales, ik, nv, L = _multirow_case(B=B, N=N, Qs=Qs, seed=720)
    g = oracle.Group(codes, scales, ik.copy(), nv, "bf16", k, max_rows=B * Qs)
    keys_before = g.ikeys.copy()
    rc, _, _ = g.layer_step("Ri", q=L["q"], iq=L["iq"], wk=L["wk"], wv=L["wv"], W=L["W"],
                            sm_scale=L["sm_scale"])
    assert rc == 0
    assert np.array_equal(g.ikeys, keys_before)
    s_all = oracle.index_score("bf16", L["iq"], keys_before)
    for b in range(B):
        for i in range(Qs):
            assert g.sel[b * Qs + i].tolist() == _brute_topk(s_all[b, i], k, int(nv[b]) - Qs + i + 1)


def test_draft_block_rows_see_each_other_causally():
    """Planted: entry slot n_valid-Qs+i scores highest for every row; row i must keep the new
    entries 0..i and none of i+1..Qs-1."""
    B, N, Qs, H, d, k = 1, 40, 5, 1, 32, 5
    codes, scales, ik, nv, L = _multirow_case(B=1, N=N, Qs=Qs, H=H, d=d, seed=740)
    one = synth.to_bf16_bits(np.full(H * d, 1.0, np.float32)).reshape(1, 1, H, d)
    L["iq"] = np.repeat(one, Qs, axis=1)
    L["new_ikey"] = synth.to_bf16_bits(np.full((1, Qs, H, d), 8.0, np.float32))  # score 256 >> others
    g = oracle.Group(codes, scales, ik, nv, "bf16", k, max_rows=Qs)
    assert g.layer_step("F", **L)[0] == 0
    base = int(nv[0]) - Qs
    for i in range(Qs):
        row = set(g.sel[i].tolist())
        assert {base + t for t in range(i + 1)} <= row, (i, sorted(row))
        assert not ({base + t for t in range(i + 1, Qs)} & row), (i, sorted(row))


def _window_reference(q_row, sel_keys, wk_b, wv_b, rows, scale):
    keys = np.concatenate([sel_keys, _bf16(wk_b[rows])]) if len(rows) else sel_keys
    vals = np.concatenate([sel_keys, _bf16(wv_b[rows])]) if len(rows) else sel_keys
    logits = scale * _bf16(q_row) @ keys.T
    return scipy.special.softmax(logits, axis=-1) @ vals, scipy.special.logsumexp(logits, axis=-1)


@pytest.mark.parametrize("poison", [False, True])
def test_partial_window_rows(poison):
    B, N, Qs, D, Hq, W, k = 5, 24, 3, 64, 2, 6, 4
    wrows = Qs + W - 1
    q =synth.normal_bf16(synth.seed(0, 770), B * Qs * Hq * D).reshape(B, Qs, Hq, D)
    x = synth.normal_f32(synth.seed(0, 771), B * N * D).reshape(B * N, D)
    codes, scales = oracle.fp4_pack(x)
    codes, scales = codes.reshape(B, N, D // 2), scales.reshape(B, N, D // 32)
    wk = synth.normal_bf16(synth.seed(0, 772), B * wrows * D).reshape(B, wrows, D)
    wv = synth.normal_bf16(synth.seed(0, 773), B * wrows * D).reshape(B, wrows, D)
    wlen = np.array([1, 4, 5, wrows - 1, wrows], np.int32)  # 0 < wlen <= Qs+W-1
    if poison:  # rows before the valid tail must never be read: fill them with NaN / Inf
        nan_bits, inf_bits = np.uint16(0x7FC0), np.uint16(0x7F80)
        for b in range(B):
            wk[b, : wrows - wlen[b]] = nan_bits
            wv[b, : wrows - wlen[b]] = inf_bits
    rng = np.random.default_rng(5)
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(B * Qs)]).astype(np.int32)
    out, lse = oracle.attend(q, codes, scales, idx, wk, wv, W, 0.125, wlen=wlen)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    for b in range(B):
        deq = oracle.fp4_dequant(codes[b], scales[b])
        for i in range(Qs):
            first = max(i, wrows - int(wlen[b]))
            rows = list(range(first, i + W))
            ref, ref_lse = _window_reference(q[b, i], deq[idx[b * Qs + i]], wk[b], wv[b], rows, 0.125)
            assert np.allclose(out[b, i], ref, rtol=0, atol=1e-6), (b, i, rows)
            assert np.allclose(lse[b, i], ref_lse, rtol=1e-6, atol=0), (b, i)


def test_partial_window_through_the_layer_step():
    """The layer step passes wlen through to the attention of every mode."""
    B, N, Qs, k = 3, 48, 4, 6
    codes, scales, ik, nv, L = _multirow_case(B=B, N=N, Qs=Qs, seed=780)
    wrows = Qs + L["W"] - 1
    wlen = np.array([2, wrows - 3, wrows], np.int32)
    g = oracle.Group(codes, scales, ik, nv, "bf16", k, max_rows=B * Qs)
    rc, out, lse = g.layer_step("F", wlen=wlen, **L)
    assert rc == 0
    o2, l2 = oracle.attend(L["q"], g.codes, g.scales, g.sel, L["wk"], L["wv"], L["W"], L["sm_scale"],
                           wlen=wlen)
    assert np.array_equal(out.view(np.uint32), o2.view(np.uint32))
    for b in range(B):
        deq = oracle.fp4_dequant(g.codes[b], g.scales[b])
        for i in range(Qs):
            sel = [j for j in g.sel[b * Qs + i] if j >= 0]
            rows = list(range(max(i, wrows - int(wlen[b])), i + L["W"]))
            ref, _ = _window_reference(L["q"][b, i], deq[sel], L["wk"][b], L["wv"][b], rows, L["sm_scale"])
            assert np.allclose(out[b, i], ref, rtol=0, atol=1e-6)
