"""Pins of the oracle's sparse attention.

The main pin: with k equal to the whole cache, sparse attention must equal a dense
textbook softmax attention over the dequantised cache plus the window, written
separately here with numpy/scipy.  Further closed forms: window only, a single key,
equal logits, the empty set, and invariance under reordering.
"""
import numpy as np
import pytest
import scipy.special

import oracle
import synth


def _bf16(x):
    return synth.bf16_bits_to_f32(x).astype(np.float64)


def _inputs(B=2, Qs=1, Hq=4, D=64, N=48, W=8, seed=70):
    q = synth.normal_bf16(synth.seed(0, seed), B * Qs * Hq * D).reshape(B, Qs, Hq, D)
    x = synth.normal_f32(synth.seed(0, seed + 1), B * N * D).reshape(B * N, D)
    codes, scales = oracle.fp4_pack(x)
    codes = codes.reshape(B, N, D // 2)
    scales = scales.reshape(B, N, D // 32)
    wk = synth.normal_bf16(synth.seed(0, seed + 2), B * (Qs + W - 1) * D).reshape(B, Qs + W - 1, D)
    wv = synth.normal_bf16(synth.seed(0, seed + 3), B * (Qs + W - 1) * D).reshape(B, Qs + W - 1, D)
    return q, codes, scales, wk, wv


def dense_reference(q, keys, vals, scale):
    """Textbook attention for one query row: softmax(scale * q K^T) V for every head."""
    qv = _bf16(q)  # [Hq, D]
    logits = scale * qv @ keys.T
    p = scipy.special.softmax(logits, axis=-1)
    return p @ vals, scipy.special.logsumexp(logits, axis=-1)


@pytest.mark.parametrize("Qs", [1, 3])
def test_full_selection_equals_dense_attention(Qs):
    B, Hq, D, N, W = 2, 4, 64, 48, 8
    q, codes, scales, wk, wv = _inputs(B, Qs, Hq, D, N, W)
    scale = np.float32(1.0 / np.sqrt(D))
    idx = np.tile(np.arange(N, dtype=np.int32), (B * Qs, 1))
    out, lse = oracle.attend(q, codes, scales, idx, wk, wv, W, scale)
    for b in range(B):
        deq = oracle.fp4_dequant(codes[b], scales[b])
        for i in range(Qs):
            keys = np.concatenate([deq, _bf16(wk[b, i:i + W])])
            vals = np.concatenate([deq, _bf16(wv[b, i:i + W])])
            ref, ref_lse = dense_reference(q[b, i], keys, vals, float(scale))
            assert np.allclose(out[b, i], ref, rtol=0, atol=1e-6)
            assert np.allclose(lse[b, i], ref_lse, rtol=1e-6, atol=0)


def test_window_only_is_textbook_sliding_window():
    B, Qs, Hq, D, N, W = 1, 2, 4, 64, 16, 8
    q, codes, scales, wk, wv = _inputs(B, Qs, Hq, D, N, W, seed=80)
    idx = np.full((B * Qs, 5), -1, dtype=np.int32)
    out, _ = oracle.attend(q, codes, scales, idx, wk, wv, W, 0.125)
    for i in range(Qs):
        ref, _ = dense_reference(q[0, i], _bf16(wk[0, i:i + W]), _bf16(wv[0, i:i + W]), 0.125)
        assert np.allclose(out[0, i], ref, atol=1e-6, rtol=0)


def test_single_key_returns_its_value():
    B, Hq, D, N, W = 1, 4, 64, 16, 4
    q, codes, scales, wk, wv = _inputs(B, 1, Hq, D, N, W, seed=90)
    idx = np.array([[5, -1, -1]], dtype=np.int32)
    out, lse = oracle.attend(q, codes, scales, idx, wk, wv, W, 0.125, wlen=np.array([0], np.int32))
    deq = oracle.fp4_dequant(codes[0, 5:6], scales[0, 5:6])[0]
    for h in range(Hq):
        assert np.array_equal(out[0, 0, h], deq.astype(np.float32))
        z = 0.125 * float(_bf16(q[0, 0, h]) @ deq)
        assert np.isclose(lse[0, 0, h], z, rtol=1e-6)


def test_equal_logits_give_the_mean():
    B, Hq, D, N, W = 1, 2, 64, 12, 4
    _, codes, scales, wk, wv = _inputs(B, 1, Hq, D, N, W, seed=100)
    q = np.zeros((B, 1, Hq, D), dtype=np.uint16)  # all logits 0
    idx = np.array([[0, 3, 7]], dtype=np.int32)
    out, lse = oracle.attend(q, codes, scales, idx, wk, wv, W, 0.125)
    deq = oracle.fp4_dequant(codes[0], scales[0])
    vals = np.concatenate([deq[[0, 3, 7]], _bf16(wv[0])])
    assert np.allclose(out[0, 0, 0], vals.mean(axis=0), atol=1e-7)
    assert np.isclose(lse[0, 0, 0], np.log(7.0))


def test_empty_set_gives_zero_and_neg_inf():
    _, codes, scales, wk, wv = _inputs(1, 1, 2, 64, 8, 4, seed=110)
    q = synth.normal_bf16(1, 128).reshape(1, 1, 2, 64)
    idx = np.full((1, 4), -1, dtype=np.int32)
    out, lse = oracle.attend(q, codes, scales, idx, wk, wv, 4, 0.125, wlen=np.array([0], np.int32))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_permutation_invariance():
    B, Hq, D, N, W = 1, 4, 64, 40, 8
    q, codes, scales, wk, wv = _inputs(B, 1, Hq, D, N, W, seed=120)
    rng = np.random.default_rng(0)
    idx = np.sort(rng.choice(N, 20, replace=False)).astype(np.int32)[None, :]
    out1, lse1 = oracle.attend(q, codes, scales, idx, wk, wv, W, 0.125)
    perm = rng.permutation(W)
    out2, lse2 = oracle.attend(q, codes, scales, idx[:, ::-1].copy(), wk[:, perm], wv[:, perm], W, 0.125)
    assert np.allclose(out1, out2, atol=1e-13, rtol=0) and np.allclose(lse1, lse2, atol=1e-12)
