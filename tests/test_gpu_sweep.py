"""GPU parity over seeded random shapes and value ranges: the exact index scores (every key
dtype, index width, row count, causal offset and exponent spread) and the top-k selection
(row lengths on every path, valid counts, ties), each compared bit for bit with the oracle.

Each case is drawn from its own seed, so a failure names a reproducible case.  Shapes stay
small enough for the oracle to finish in a fraction of a second per case.
"""
import numpy as np
import pytest
import torch

import compressed_kv_cache_03_amd as csa2
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

WIDTHS = {"bf16": [(1, 64), (2, 64), (4, 64), (3, 32), (2, 128), (4, 128)],
          "e4m3": [(1, 128), (2, 64), (4, 64), (2, 128), (3, 64)],
          "fp4": [(4, 64), (2, 128), (1, 64), (3, 32)]}


def dev(a):
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}.get(a.dtype)
    return torch.from_numpy(a.view(view) if view is not None else a).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def _bits_eq(a, b):
    return np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def _values(rng, shape, spread):
    """N(0,1) values times 2^e, e drawn per element from [-spread, spread], with some exact zeros."""
    x = rng.standard_normal(shape) * np.exp2(rng.integers(-spread, spread + 1, shape))
    x[rng.random(shape) < 0.01] = 0.0
    return x.astype(np.float32)


def _score_case(seed):
    rng = np.random.default_rng(7000 + seed)
    dtype = ["bf16", "e4m3", "fp4"][seed % 3]
    H, d = WIDTHS[dtype][rng.integers(len(WIDTHS[dtype]))]
    B = int(rng.integers(1, 4))
    Qs = int(rng.choice([1, 2, 5]))
    N = int(rng.integers(1, 5001))
    causal = -1 if rng.random() < 0.5 else int(rng.integers(0, N + 10))
    spread = int(rng.choice([0, 3, 20, 60]))
    ks = None
    if dtype == "bf16":
        iq = synth.to_bf16_bits(_values(rng, (B, Qs, H, d), spread))
        ik = synth.to_bf16_bits(_values(rng, (B, N, H, d), spread))
    elif dtype == "e4m3":
        iq = synth.to_e4m3_bits(_values(rng, (B, Qs, H, d), min(spread, 4)))
        ik = synth.to_e4m3_bits(_values(rng, (B, N, H, d), min(spread, 4)))
    else:
        iq = synth.to_bf16_bits(_values(rng, (B, Qs, H, d), spread))
        ik = rng.integers(0, 256, (B, N, H, d // 2)).astype(np.uint8)
        ks = ((rng.random((B, N, H * d // 32)) + 0.5) *
              np.exp2(rng.integers(-40 - spread, 40 + spread + 1, (B, N, H * d // 32)))).astype(np.float32)
        ks[:, ::11, 0] = 0.0
    return dtype, iq, ik, ks, causal, (B, Qs, H, d, N, spread)


@pytest.mark.parametrize("seed", range(96))
def test_index_score_sweep(seed):
    dtype, iq, ik, ks, causal, shape = _score_case(seed)
    B, Qs, H, d, N, _ = shape
    got = csa2.index_score(dev(iq), dev(ik), dtype, ik_scales=None if ks is None else dev(ks),
                           causal_offset=causal)
    torch.cuda.synchronize()
    nv = None
    if causal >= 0:
        nv = np.minimum(np.array([[causal + i + 1 for i in range(Qs)]] * B, np.int64).reshape(-1), N)
    ref = oracle.index_score(dtype, iq, ik, n_valid_row=nv, ik_scales=ks)
    # entries a causal row does not see read -inf on both sides; exact sums beyond fp32
    # round to +-inf on both sides
    assert _bits_eq(host(got), ref), (seed, dtype, shape, causal)


def _topk_case(seed):
    rng = np.random.default_rng(9000 + seed)
    R = int(rng.choice([1, 3, 8, 40, 300]))
    N = int(rng.choice([1, 7, 4096, 8193, 20000, 65536, 140001]))
    if R * N > 6_000_000:
        R = max(1, 6_000_000 // N)
    k = int(rng.choice([1, 5, 100, 2048, 3000]))
    levels = int(rng.choice([3, 100, 1 << 20]))
    s = (rng.integers(0, levels, (R, N)).astype(np.float32) - levels / 2) * np.float32(0.25)
    s[rng.random((R, N)) < 0.001] = -np.inf
    s[rng.random((R, N)) < 0.001] = -0.0
    nv = rng.integers(0, N + 1, R).astype(np.int32)
    nv[0] = N
    return s, k, nv


@pytest.mark.parametrize("seed", range(48))
def test_topk_sweep(seed):
    s, k, nv = _topk_case(seed)
    got = csa2.topk(dev(s), k, n_valid=dev(nv))
    torch.cuda.synchronize()
    ref = oracle.topk(s, k, n_valid=nv.astype(np.int64))
    assert np.array_equal(host(got), ref), (seed, s.shape, k)


# ---------------------------------------------------------------- whole layer steps
def _layer_case(seed):
    """A workload recipe at random sizes: index width, entry width, query heads, window,
    rows per step, selection size, valid counts and (hierarchical recipes) pool size."""
    from synth.workloads import W1, W2, W3, W4, W6, W7, W8
    rng = np.random.default_rng(11000 + seed)
    base = [W1, W2, W3, W6, W7, W8, W4][seed % 7]
    dt = base.idx_dtype
    if base is W4:  # prefill chunks on the matrix-core selection: K of 128 or 256
        H, d = [(2, 64), (4, 64), (1, 128)][rng.integers(3)]
        Qs = int(rng.choice([2, 33, 96]))
    else:
        H, d = WIDTHS[dt][rng.integers(len(WIDTHS[dt]))]
        Qs = base.Qs if base.Qs > 1 else int(rng.choice([1, 1, 2, 5]))
    B = int(rng.integers(1, 4))
    N = int(rng.integers(max(Qs, 20), 6001))
    k = int(rng.integers(1, min(N, 700) + 1))
    # head counts that leave the last group of 16 partly empty, entry widths of every
    # kernel instance kind (odd and even numbers of 32-element blocks)
    kw = dict(B=B, N=N, H_I=H, d_I=d, Qs=Qs, k=k, Hq=int(rng.choice([1, 3, 4, 16, 17, 32])),
              D=int(rng.choice([32, 64, 96, 128, 160, 256])), W=int(rng.choice([0, 1, 17, 128, 200])))
    if base.pool_blocks:
        blocks = (N + 7) // 8
        kw["pool_blocks"] = int(rng.integers(min((k + 7) // 8, blocks), blocks + 1))
    nv = rng.integers(Qs, N + 1, B)
    if rng.random() < 0.5:
        nv[rng.integers(B)] = N
    return base.scaled(**kw), [int(v) for v in nv]


@pytest.mark.parametrize("seed", range(84))
def test_layer_step_sweep(seed):
    from test_gpu_parity import Run
    wl, nv = _layer_case(seed)
    print(seed, wl, nv, flush=True)
    Run(wl, n_valid=nv).check_all()
