"""Pins of the oracle's FP4 codec (e2m1 elements, fp32 scale per 32 elements).

The element table comes from the OCP MX format definition (tests/golden/e2m1_table.txt);
packing is checked against an independent brute-force nearest search in exact
rational arithmetic, an exhaustive sweep at scale 1, and closed-form properties.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _golden_table():
    rows = []
    for line in open(os.path.join(GOLDEN, "e2m1_table.txt")):
        if line.startswith("#") or not line.strip():
            continue
        c, v = line.split()
        rows.append((int(c, 16), float(v)))
    return rows


def test_e2m1_table_exhaustive():
    table = _golden_table()
    assert len(table) == 16
    for code, val in table:
        got = oracle.e2m1_value(code)
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def _nearest_code_exact(x: float, scale: float) -> int:
    """Brute force: the grid point v*scale nearest to x, ties to the even magnitude code."""
    fx, fs = Fraction(abs(x)), Fraction(scale)
    d = [abs(fx - Fraction(v) * fs) for v in GRID]
    best = min(d)
    cands = [c for c in range(8) if d[c] == best]
    c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return c | (8 if np.signbit(x) else 0)


def _unpack(codes: np.ndarray) -> np.ndarray:
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def test_pack_random_blocks_against_exact_brute_force():
    rng = np.random.default_rng(1)
    rows = 96
    x = synth.normal_f32(synth.seed(0, 50), rows * 128).reshape(rows, 128)
    # spread block magnitudes over many binades, including fp32 subnormal territory
    mag = np.float32(2.0) ** rng.integers(-140, 60, size=(rows, 4)).astype(np.float32)
    x = (x.reshape(rows, 4, 32) * mag[:, :, None]).reshape(rows, 128).astype(np.float32)
    codes, scales = oracle.fp4_pack(x)
    el = _unpack(codes)
    for r in range(rows):
        for b in range(4):
            blk = x[r, 32 * b:32 * b + 32]
            amax = np.float32(np.max(np.abs(blk)))
            assert scales[r, b] == np.float32(amax / np.float32(6.0))
            for i in range(32):
                assert el[r, 32 * b + i] == _nearest_code_exact(float(blk[i]), float(scales[r, b]))


def test_pack_ties_go_to_even_code():
    # scale 1 (block amax 6): the seven decision points are exact ties
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect = [0, 2, 2, 4, 4, 6, 6]  # even neighbour of each pair
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 6.0
    x[0, 1:8] = ties
    x[0, 8:15] = -np.array(ties)
    codes, scales = oracle.fp4_pack(x)
    el = _unpack(codes)[0]
    assert scales[0, 0] == 1.0
    assert el[1:8].tolist() == expect
    assert el[8:15].tolist() == [c | 8 for c in expect]
    assert el[0] == 7


def test_pack_exhaustive_sweep_at_scale_one():
    # every fp32 value in [2^-4, 6] (and its negative) against a vectorised nearest search;
    # at scale 1 the distances |x - v| are exact in fp64
    lo = np.float32(2.0 ** -4).view(np.uint32)
    hi = np.float32(6.0).view(np.uint32)
    allv = np.arange(lo, hi + 1, dtype=np.uint32).view(np.float32)
    grid = np.array(GRID)
    step = 31 * (1 << 17)
    for start in range(0, allv.size, step):
        v = allv[start:start + step]
        nblk = -(-v.size // 31)
        pad = np.zeros(nblk * 31, dtype=np.float32)
        pad[:v.size] = v
        sign = np.where(np.arange(pad.size) % 2 == 0, 1.0, -1.0).astype(np.float32)
        pad *= sign
        blocks = np.concatenate([np.full((nblk, 1), 6.0, np.float32), pad.reshape(nblk, 31)], axis=1)
        codes, scales = oracle.fp4_pack(blocks.reshape(-1, 32))
        assert np.all(scales == 1.0)
        el = _unpack(codes)[:, 1:].reshape(-1)
        d = np.abs(np.abs(pad.astype(np.float64))[:, None] - grid[None, :])
        best = d.min(axis=1, keepdims=True)
        is_best = d == best
        ntie = is_best.sum(axis=1)
        first = np.argmax(is_best, axis=1)
        even_pick = np.where(first % 2 == 0, first, first + 1)
        want = np.where(ntie == 1, first, even_pick) | np.where(np.signbit(pad), 8, 0)
        assert np.array_equal(el, want.astype(np.uint8))


def test_pack_closed_form_properties():
    x = synth.normal_f32(synth.seed(0, 51), 4096 * 128).reshape(4096, 128)
    codes, scales = oracle.fp4_pack(x)
    deq = oracle.fp4_dequant(codes, scales)
    s = np.repeat(scales.astype(np.float64), 32, axis=1)
    # widest grid gap is 4 -> 6 (2 * scale), so the error never exceeds one scale
    assert np.all(np.abs(deq - x) <= s)
    # the block maximum maps to +-6 exactly (code 7 or 15)
    el = _unpack(codes)
    blk = np.abs(x).reshape(4096, 4, 32)
    arg = blk.argmax(axis=2)
    top = np.take_along_axis(el.reshape(4096, 4, 32), arg[:, :, None], axis=2)[:, :, 0]
    assert np.all((top & 7) == 7)
    # values already on the grid round-trip exactly
    g = np.array(GRID + [-v for v in GRID], dtype=np.float32)
    y = np.resize(g, (8, 32)).astype(np.float32) * np.float32(0.375)
    y[:, 0] = 6 * 0.375
    c2, s2 = oracle.fp4_pack(y)
    assert np.all(s2 == np.float32(0.375))
    assert np.array_equal(oracle.fp4_dequant(c2, s2), y.astype(np.float64))


def test_pack_zero_block_keeps_sign():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 1::2] = -0.0
    codes, scales = oracle.fp4_pack(x)
    assert scales[0, 0] == 0.0
    el = _unpack(codes)[0]
    assert el[0::2].tolist() == [0] * 16 and el[1::2].tolist() == [8] * 16


def test_nibble_order_low_is_even_element():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 6.0   # code 7 in the low nibble of byte 0
    x[0, 1] = -3.0  # code 0xD in the high nibble
    codes, _ = oracle.fp4_pack(x)
    assert codes[0, 0] == 0xD7
