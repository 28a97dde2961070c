"""Seeded input generator: determinism, distribution and the storage conversions."""
import numpy as np
import pytest
import scipy.stats
import torch

import synth


def _py_splitmix64(seed, count):
    """SplitMix64 as a sequential generator (state += GAMMA; output = mix(state))."""
    M = (1 << 64) - 1
    state = seed & M
    out = []
    for _ in range(count):
        state = (state + 0x9E3779B97F4A7C15) & M
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        out.append(z ^ (z >> 31))
    return out


def test_counter_form_equals_sequential_splitmix64():
    # word n of a stream is output n+1 of SplitMix64 started from state mix(seed)
    seed = synth.seed(2, 7)
    state0 = _py_splitmix64(seed - 0x9E3779B97F4A7C15, 1)[0]  # mix(seed)
    seq = _py_splitmix64(state0, 40)
    assert [synth.word(seed, n) for n in range(40)] == seq


def test_normal_deterministic_and_offsets():
    s = synth.seed(1, 3)
    a = synth.normal_f32(s, 10001)
    b = synth.normal_f32(s, 10001)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = synth.normal_f32(s, 501, offset=4321)
    assert np.array_equal(c, a[4321:4822])
    rows = synth.normal_rows_f32(s, [3, 0, 7], 100)
    assert np.array_equal(rows[0], a[300:400]) and np.array_equal(rows[2], a[700:800])
    assert not np.array_equal(synth.normal_f32(synth.seed(1, 4), 100), a[:100])


def test_normal_distribution():
    x = synth.normal_f32(synth.seed(9, 1), 2_000_000).astype(np.float64)
    assert abs(x.mean()) < 3e-3
    assert abs(x.std() - 1.0) < 3e-3
    assert abs(scipy.stats.kurtosis(x)) < 2e-2
    assert scipy.stats.kstest(x[:200_000], "norm").pvalue > 1e-4
    assert np.abs(x).max() < 8.6  # sqrt(-2 ln 2^-53) bounds Box-Muller with 53-bit uniforms


def test_bf16_rne_matches_torch():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000],
                    dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    x = bits.view(np.float32)
    finite = np.isfinite(x)
    ours = synth.to_bf16_bits(x[finite])
    ref = torch.from_numpy(x[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_rne_matches_torch_and_saturates():
    rng = np.random.default_rng(5)
    # dense sweep over every fp32 exponent the format reaches, plus random mantissas
    e = np.arange(-20, 10)
    m = rng.integers(0, 1 << 23, size=(e.size, 4000), dtype=np.uint32)
    m[:, :64] = (np.arange(64, dtype=np.uint32) << 17)  # exact ties and their neighbours
    m[:, 64:128] = (np.arange(64, dtype=np.uint32) << 17) + 1
    bits = (((e[:, None] + 127).astype(np.uint32) << 23) | m).reshape(-1)
    x = np.concatenate([bits.view(np.float32), -bits.view(np.float32), [0.0, -0.0]]).astype(np.float32)
    x = x[np.abs(x) <= 464.0]
    ours = synth.to_e4m3_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    big = np.array([448.0, 465.0, 1e6, np.inf, -500.0], dtype=np.float32)
    assert synth.to_e4m3_bits(big).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_e4m3_all_codes_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(synth.to_e4m3_bits(vals), codes)


@pytest.mark.parametrize("dt", ["bf16", "e4m3"])
def test_fused_streams_equal_convert_of_f32(dt):
    s = synth.seed(3, 11)
    x = synth.normal_f32(s, 5000, offset=17)
    fused = synth.normal_idx(dt, s, 5000, offset=17)
    conv = synth.to_bf16_bits(x) if dt == "bf16" else synth.to_e4m3_bits(x)
    assert np.array_equal(fused, conv)
