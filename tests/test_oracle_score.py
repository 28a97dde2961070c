"""Pins of the oracle's index score: fp32 round-to-nearest-even of the exact sum.

Checked against exact rational arithmetic (fractions.Fraction) with an independent
fp32 rounding, planted rounding ties, cancellation, integer-valued closed forms and
the single-head plain dot product.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def round_f32(fr: Fraction) -> np.float32:
    """Exact rational -> nearest fp32, ties to even (IEEE binary32, with subnormals)."""
    if fr == 0:
        return np.float32(0.0)
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    qe = max(e - 23, -149)
    n = a / (Fraction(2) ** qe)
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * Fraction(2) ** qe
    f = np.float32(np.inf) if val >= Fraction(2) ** 128 else np.float32(float(val))
    return -f if neg else f


def exact_dot(a, b) -> np.float32:
    return round_f32(sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b)), Fraction(0)))


def _bf16_vals(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _e4m3_vals(bits):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def _wide_bf16(rng, n):
    sign = rng.integers(0, 2, n)
    exp = rng.integers(-70, 70, n)
    mant = rng.integers(0, 128, n)
    vals = (1 + mant / 128.0) * np.exp2(exp.astype(np.float64)) * np.where(sign, -1, 1)
    return synth.to_bf16_bits(vals.astype(np.float32))


def test_exact_dot_random_wide_exponents():
    rng = np.random.default_rng(7)
    for _ in range(300):
        n = int(rng.integers(1, 300))
        a = _bf16_vals(_wide_bf16(rng, n))
        b = _bf16_vals(_wide_bf16(rng, n))
        got = oracle.exact_dot_f32(a, b)
        want = exact_dot(a, b)
        assert got.view(np.uint32) == want.view(np.uint32), (n, got, want)


def test_exact_dot_planted_ties_and_cancellation():
    cases = [
        ([1.0, 2.0 ** -24], 1.0),                               # midpoint -> even (1.0)
        ([1.0, 3 * 2.0 ** -24], 1.0 + 2.0 ** -22),              # midpoint -> even (up)
        ([1.0, 2.0 ** -24, 2.0 ** -80], 1.0 + 2.0 ** -23),      # just above the midpoint
        ([1.0, 2.0 ** -24, -2.0 ** -80], 1.0),                  # just below
        ([-1.0, -(2.0 ** -24), -(2.0 ** -80)], -(1.0 + 2.0 ** -23)),
        ([2.0 ** 60, -(2.0 ** 60), 3.0], 3.0),                  # catastrophic cancellation
        ([2.0 ** 100, 1.0, -(2.0 ** 100)], 1.0),
        ([2.0 ** -140, 2.0 ** -140], 2.0 ** -139),              # fp32 subnormal result
        ([2.0 ** -151], 0.0),                                   # below half the least subnormal
        ([3 * 2.0 ** -151], 2.0 ** -149),                       # rounds up to the least subnormal
        ([1.0, -1.0], 0.0),
    ]
    for terms, want in cases:
        t = np.array(terms, dtype=np.float64)
        got = oracle.exact_dot_f32(t, np.ones_like(t))
        # bitwise, so an exact zero must come out as +0
        assert got.view(np.uint32) == np.float32(want).view(np.uint32), (terms, got, want)


def test_exact_dot_integer_inputs_give_integer_scores():
    rng = np.random.default_rng(3)
    a = rng.integers(-200, 200, size=(50, 256)).astype(np.float64)
    b = rng.integers(-200, 200, size=(50, 256)).astype(np.float64)
    for i in range(50):
        want = int(np.dot(a[i].astype(np.int64), b[i].astype(np.int64)))
        assert abs(want) < 2 ** 24
        assert oracle.exact_dot_f32(a[i], b[i]) == np.float32(want)


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_index_score_matches_rational_brute_force(dtype):
    B, Qs, N, H, d = 2, 2, 40, 4, 64
    iq = synth.normal_idx(dtype, synth.seed(0, 60), B * Qs * H * d).reshape(B, Qs, H, d)
    ik = synth.normal_idx(dtype, synth.seed(0, 61), B * N * H * d).reshape(B, N, H, d)
    s = oracle.index_score(dtype, iq, ik)
    dec = _bf16_vals if dtype == "bf16" else _e4m3_vals
    qv, kv = dec(iq), dec(ik)
    for b in range(B):
        for i in range(Qs):
            for j in range(N):
                want = exact_dot(qv[b, i].reshape(-1), kv[b, j].reshape(-1))
                assert s[b, i, j].view(np.uint32) == want.view(np.uint32)


def test_index_score_single_head_is_plain_dot():
    # with small-integer bf16 inputs every partial sum is exact in fp64, so the exact
    # score equals the ordinary fp64 dot product rounded to fp32
    rng = np.random.default_rng(4)
    iq = synth.to_bf16_bits(rng.integers(-8, 8, (1, 1, 1, 64)).astype(np.float32))
    ik = synth.to_bf16_bits(rng.integers(-8, 8, (1, 33, 1, 64)).astype(np.float32))
    s = oracle.index_score("bf16", iq, ik)[0, 0]
    q = _bf16_vals(iq).reshape(64)
    k = _bf16_vals(ik).reshape(33, 64)
    assert np.array_equal(s, (k @ q).astype(np.float32))


def test_index_score_n_valid_masks_with_neg_inf():
    iq = synth.normal_idx("bf16", synth.seed(0, 62), 64).reshape(1, 1, 1, 64)
    ik = synth.normal_idx("bf16", synth.seed(0, 63), 10 * 64).reshape(1, 10, 1, 64)
    s = oracle.index_score("bf16", iq, ik, n_valid_row=np.array([6]))
    assert np.all(np.isneginf(s[0, 0, 6:])) and np.all(np.isfinite(s[0, 0, :6]))


def test_e4m3_decoder_matches_torch_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ours = oracle.idx_values("e4m3", codes)
    ref = _e4m3_vals(codes)
    assert np.array_equal(ours, ref) and np.array_equal(np.signbit(ours), np.signbit(ref))
    assert math.isnan(oracle.idx_values("e4m3", np.array([0x7F], np.uint8))[0])


# FP4 index keys (the cache codec reused by the indexer): value = e2m1(code) * scale
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX e2m1 magnitudes, codes 0..7


def _fp4_key_values(codes, scales):
    """codes uint8 [..., K/2] (element 2i in the low nibble), scales float32 [..., K/32]
    -> exact Fractions [..., K] as nested lists, written out from the format."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    K = scales.shape[-1] * 32
    flat_c = codes.reshape(-1, K // 2)
    flat_s = scales.reshape(-1, K // 32)
    out = []
    for row_c, row_s in zip(flat_c, flat_s):
        vals = []
        for e in range(K):
            nib = (int(row_c[e // 2]) >> (4 * (e % 2))) & 15
            mag = Fraction(E2M1[nib & 7])
            vals.append((-mag if nib & 8 else mag) * Fraction(float(row_s[e // 32])))
        out.append(vals)
    return out


def test_index_score_fp4_keys_match_rational_brute_force():
    rng = np.random.default_rng(21)
    B, Qs, N, H, d = 1, 3, 25, 2, 64
    K = H * d
    iq = _wide_bf16(rng, B * Qs * K).reshape(B, Qs, H, d)
    codes = rng.integers(0, 256, (B, N, H, d // 2)).astype(np.uint8)
    # scales over many binades, some subnormal, some zero
    sc = (rng.random((B, N, K // 32)) + 0.5) * np.exp2(rng.integers(-140, 100, (B, N, K // 32)))
    sc[0, 3, 1] = 0.0
    sc[0, 5, 0] = 2.0 ** -149
    scales = sc.astype(np.float32)
    s = oracle.index_score("fp4", iq, codes, ik_scales=scales)
    qv = _bf16_vals(iq).reshape(B, Qs, K)
    kv = _fp4_key_values(codes, scales)
    for i in range(Qs):
        for j in range(N):
            want = round_f32(sum((Fraction(float(qv[0, i, e])) * kv[j][e] for e in range(K)), Fraction(0)))
            assert s[0, i, j].view(np.uint32) == want.view(np.uint32), (i, j)


def test_index_score_fp4_keys_planted_ties_and_cancellation():
    # q = 1 on two elements whose key values sum to an fp32 midpoint or cancel exactly
    K = 64
    iq = synth.to_bf16_bits(np.zeros((1, 1, 1, K), np.float32))
    iq[0, 0, 0, 0] = synth.to_bf16_bits(np.array([1.0], np.float32))[0]
    iq[0, 0, 0, 32] = iq[0, 0, 0, 0]
    codes = np.zeros((1, 3, 1, K // 2), np.uint8)
    scales = np.ones((1, 3, K // 32), np.float32)
    # entry 0: 1.0 + 2^-24 (a tie between 1 and 1+2^-23, rounds to even = 1.0)
    codes[0, 0, 0, 0], codes[0, 0, 0, 16] = 0x2, 0x2          # e2m1 1.0 in both blocks
    scales[0, 0] = [1.0, 2.0 ** -24]
    # entry 1: 1.0 + 3*2^-24 (a tie between 1+2^-23 and 1+2^-22, rounds to even = 1+2^-22)
    codes[0, 1, 0, 0], codes[0, 1, 0, 16] = 0x2, 0x5          # 1.0 and 3.0
    scales[0, 1] = [1.0, 2.0 ** -24]
    # entry 2: 6 * 2^100 - 6 * 2^100 = +0
    codes[0, 2, 0, 0], codes[0, 2, 0, 16] = 0x7, 0xF          # +6 and -6
    scales[0, 2] = [2.0 ** 100, 2.0 ** 100]
    s = oracle.index_score("fp4", iq, codes, ik_scales=scales)[0, 0]
    assert s[0] == np.float32(1.0)
    assert s[1] == np.float32(1.0 + 2.0 ** -22)
    assert s[2] == 0.0 and not np.signbit(s[2])
