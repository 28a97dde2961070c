"""GPU parity: every C-ABI entry point against the CPU oracle on identical seeded inputs.

Bars: FP4 bytes, index scores and top-k index sets bit-exact; attention outputs within
2e-3 max relative error per (row, head) (max|g-r| / max|r|), fp32 accumulation.
"""
import numpy as np
import pytest
import torch

import compressed_kv_cache_03_amd as csa2
import oracle
import synth
from cases import make_inputs, rel_err
from synth.workloads import W1, W2, W3, W4, W5, W6, W7, W8

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}.get(a.dtype)
    t = torch.from_numpy(a.view(view) if view is not None else a)
    return t.to(DEV)


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def bits_eq(a, b):
    return np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


# ---------------------------------------------------------------- S1 pack
def test_pack_parity():
    rng = np.random.default_rng(11)
    x = synth.normal_f32(synth.seed(1, 0), 4096 * 128).reshape(4096, 128)
    wide = (synth.normal_f32(synth.seed(0, 900), 512 * 128).reshape(512, 4, 32)
            * np.float32(2.0) ** rng.integers(-140, 60, (512, 4, 1)).astype(np.float32)).reshape(512, 128)
    ties = np.zeros((8, 128), np.float32)
    ties[:, 0::32] = 6.0
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    for blk in range(4):
        ties[:, 32 * blk + 1:32 * blk + 8] = t
        ties[:, 32 * blk + 8:32 * blk + 15] = -t
    ties[7] = 0.0
    ties[7, 1::2] = -0.0
    x = np.concatenate([x, wide.astype(np.float32), ties]).astype(np.float32)
    codes, scales = csa2.fp4_pack(dev(x))
    torch.cuda.synchronize()
    oc, os_ = oracle.fp4_pack(x)
    assert bits_eq(host(codes), oc)
    assert bits_eq(host(scales), os_)


# ---------------------------------------------------------------- S2 scores
@pytest.mark.parametrize("dtype,H,d", [("bf16", 1, 64), ("bf16", 4, 64), ("bf16", 3, 64),
                                       ("e4m3", 4, 64), ("e4m3", 1, 64), ("e4m3", 2, 128)])
@pytest.mark.parametrize("Qs", [1, 3])
def test_index_score_parity(dtype, H, d, Qs):
    B, N = 2, 2999
    iq = synth.normal_idx(dtype, synth.seed(0, 910), B * Qs * H * d).reshape(B, Qs, H, d)
    ik = synth.normal_idx(dtype, synth.seed(0, 911), B * N * H * d).reshape(B, N, H, d)
    got = csa2.index_score(dev(iq), dev(ik), dtype)
    torch.cuda.synchronize()
    ref = oracle.index_score(dtype, iq, ik)
    assert bits_eq(host(got), ref)


@pytest.mark.parametrize("dtype,H,d", [("bf16", 4, 64), ("e4m3", 4, 64), ("bf16", 3, 32), ("fp4", 4, 64)])
@pytest.mark.parametrize("causal", [0, 1000, 2990, 5000])
def test_index_score_causal_offset(dtype, H, d, causal):
    # row i of a causal chunk scores entries j <= causal + i and reads -inf beyond
    B, Qs, N = 2, 12, 2999
    if dtype == "fp4":
        rng = np.random.default_rng(causal + 1)
        iq, ik, ks = _fp4_key_case(rng, B, N, H, d)
        iq = np.concatenate([iq] * (Qs // 2), axis=1)
        g_ks, o_ks = dev(ks), ks
    else:
        iq = synth.normal_idx(dtype, synth.seed(0, 912), B * Qs * H * d).reshape(B, Qs, H, d)
        ik = synth.normal_idx(dtype, synth.seed(0, 913), B * N * H * d).reshape(B, N, H, d)
        g_ks = o_ks = None
    got = csa2.index_score(dev(iq), dev(ik), dtype, ik_scales=g_ks, causal_offset=causal, exact=False)
    torch.cuda.synchronize()
    nv = np.array([[causal + i + 1 for i in range(Qs)]] * B, np.int64).reshape(-1)
    ref = oracle.index_score(dtype, iq, ik, n_valid_row=np.minimum(nv, N), ik_scales=o_ks)
    assert bits_eq(host(got), ref)


def test_index_score_fp8_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    n = codes.size
    iq = np.zeros((1, 1, 4, 64), np.uint8)
    iq[0, 0, 0, 0] = 0x38  # 1.0
    iq[0, 0, 2, 5] = 0xC0  # -2.0
    ik = np.zeros((1, n, 4, 64), np.uint8)
    ik[0, :, 0, 0] = codes
    ik[0, :, 2, 5] = codes[::-1]
    got = csa2.index_score(dev(iq), dev(ik), "e4m3")
    torch.cuda.synchronize()
    assert bits_eq(host(got), oracle.index_score("e4m3", iq, ik))


def test_index_score_bf16_rounding_ties_take_exact_path():
    # sums that land exactly on (or a hair beside) an fp32 rounding midpoint, extreme
    # exponent spreads and cancellation: the fp64 pass cannot certify these
    one = 0x3F80
    b = lambda v: int(synth.to_bf16_bits(np.array([v], np.float32))[0])  # noqa: E731
    rows = [
        {0: 1.0, 1: 2.0 ** -24},
        {0: 1.0, 1: 3 * 2.0 ** -24},
        {0: 1.0, 1: 2.0 ** -24, 2: 2.0 ** -80},
        {0: 1.0, 1: 2.0 ** -24, 2: -(2.0 ** -80)},
        {0: 2.0 ** 100, 1: 1.0, 2: -(2.0 ** 100)},
        {0: 2.0 ** 60, 1: -(2.0 ** 60), 2: 3.0},
        {0: 2.0 ** -126, 1: 2.0 ** -130},
        {0: 0.0},
        {0: -(2.0 ** -120), 1: 2.0 ** -120},
    ]
    N = len(rows) * 37
    ik = np.zeros((1, N, 1, 64), np.uint16)
    for j in range(N):
        for e, v in rows[j % len(rows)].items():
            ik[0, j, 0, e] = b(v)
        ik[0, j, 0, 10 + j % 50] = b(2.0 ** -(j % 90)) if j % 3 == 0 else 0
    iq = np.zeros((1, 1, 1, 64), np.uint16)
    iq[0, 0, 0, :3] = one
    iq[0, 0, 0, 10:60] = b(1.0)
    got = csa2.index_score(dev(iq), dev(ik), "bf16")
    torch.cuda.synchronize()
    assert bits_eq(host(got), oracle.index_score("bf16", iq, ik))


@pytest.mark.parametrize("qexp,kexp,zeros", [(0, 0, False), (-70, -70, False), (-60, -62, True),
                                             (60, 66, False), (-20, 40, True)])
def test_index_score_bf16_products_at_the_fp32_range(qexp, kexp, zeros):
    # bf16 x bf16 products are formed in fp32: scaled so that products underflow
    # into fp32's subnormal range (-70, -70; -60, -62), overflow it (60, 66), or
    # stay inside it; zero query and key elements widen the bound on the smallest
    # product.  K = 256 (the decode shape), several workgroups and a ragged tail.
    rng = np.random.default_rng(2024 + qexp)
    B, N, H, d = 2, 1500, 4, 64
    q = rng.standard_normal((B, 1, H, d)) * 2.0 ** qexp
    k = rng.standard_normal((B, N, H, d)) * 2.0 ** kexp
    if zeros:
        q[:, :, 0, :5] = 0.0
        k[:, ::3, 1, 7] = 0.0
    iq = synth.to_bf16_bits(q.astype(np.float32))
    ik = synth.to_bf16_bits(k.astype(np.float32))
    got = csa2.index_score(dev(iq), dev(ik), "bf16")
    torch.cuda.synchronize()
    assert bits_eq(host(got), oracle.index_score("bf16", iq, ik))


def _fp4_key_case(rng, B, N, H, d):
    # wide-exponent bf16 queries; every code byte; block scales over many binades
    K = H * d
    iq = synth.to_bf16_bits(((rng.random((B, 2, H, d)) - 0.5) *
                             np.exp2(rng.integers(-60, 60, (B, 2, H, d)))).astype(np.float32))
    codes = rng.integers(0, 256, (B, N, H, d // 2)).astype(np.uint8)
    sc = (rng.random((B, N, K // 32)) + 0.5) * np.exp2(rng.integers(-126, 100, (B, N, K // 32)))
    sc[:, ::7, 0] = 0.0
    return iq, codes, sc.astype(np.float32)


@pytest.mark.parametrize("H,d", [(4, 64), (2, 256), (3, 32)])
def test_index_score_fp4_keys_bit_exact(H, d):
    # (4, 64) and (2, 256) run the streaming kernel, (3, 32) the generic one
    rng = np.random.default_rng(H * 100 + d)
    B, N = 2, 3000
    iq, codes, scales = _fp4_key_case(rng, B, N, H, d)
    got = csa2.index_score(dev(iq), dev(codes), "fp4", ik_scales=dev(scales))
    torch.cuda.synchronize()
    assert bits_eq(host(got), oracle.index_score("fp4", iq, codes, ik_scales=scales))


def test_index_score_fp4_keys_rounding_ties_take_exact_path():
    # two blocks whose values sum to an fp32 midpoint: the certificate cannot decide,
    # the exact accumulator rounds to even
    K = 256
    iq = np.zeros((1, 1, 1, K), np.uint16)
    iq[0, 0, 0, 0] = synth.to_bf16_bits(np.array([1.0], np.float32))[0]
    iq[0, 0, 0, 32] = iq[0, 0, 0, 0]
    N = 64
    codes = np.zeros((1, N, 1, K // 2), np.uint8)
    scales = np.ones((1, N, K // 32), np.float32)
    for j in range(N):
        codes[0, j, 0, 0], codes[0, j, 0, 16] = 0x2, (0x2, 0x5, 0xA, 0xD)[j % 4]  # 1 and +-1, +-3
        scales[0, j, 1] = 2.0 ** -(24 + j % 16)
    got = csa2.index_score(dev(iq), dev(codes), "fp4", ik_scales=dev(scales))
    torch.cuda.synchronize()
    assert bits_eq(host(got), oracle.index_score("fp4", iq, codes, ik_scales=scales))


def _bf16_fields(rng, fields):
    """bf16 bits with the given exponent fields, random sign and mantissa."""
    fields = np.asarray(fields, np.int64)
    return ((rng.integers(0, 2, fields.shape) << 15) | (fields << 7) |
            rng.integers(0, 128, fields.shape)).astype(np.uint16)


@pytest.mark.parametrize("case", ["normal", "band1", "band3", "beyond", "subnormal", "zeros", "edges"])
def test_index_score_fp4_mfma_bands(case):
    # FP4 keys with K = 256 score on the matrix cores when every query block's values lie within
    # 28 binades of the block's largest (bands of 7 binades, one or two band pairs) and the
    # exponents are moderate; other rows take the per-thread fp64 path.  Each case mixes rows of
    # both kinds with ragged N (3000 = 2048 + 952) and three rows per sequence.
    rng = np.random.default_rng(["normal", "band1", "band3", "beyond", "subnormal", "zeros", "edges"].index(case))
    B, Qs, N, H, d = 2, 3, 3000, 4, 64
    K = H * d
    R = B * Qs
    emax = 127 + rng.integers(-3, 4, (R, K // 32, 1))
    if case == "normal":
        iq = synth.to_bf16_bits(rng.normal(size=(R, K)).astype(np.float32))
    elif case in ("band1", "band3", "beyond"):
        span = 14 if case == "band1" else 28
        f = emax - rng.integers(0, span, (R, K // 32, 32))
        f[:, :, 0] = emax[:, :, 0]
        f[:, :, 1] = emax[:, :, 0] - (span - 1)  # the deepest band's lowest binade
        if case == "beyond":
            f[0, 3, 5] = emax[0, 3, 0] - 28
        iq = _bf16_fields(rng, f).reshape(R, K)
    elif case == "subnormal":
        iq = synth.to_bf16_bits(rng.normal(size=(R, K)).astype(np.float32))
        iq[1, 77] = 0x0005
        iq[4, 3] = 0x8041
    elif case == "zeros":
        iq = synth.to_bf16_bits(rng.normal(size=(R, K)).astype(np.float32))
        iq[rng.random((R, K)) < 0.3] = 0
        iq[0, 64:96] = 0x8000  # a block of -0
        iq[2, :] = 0
    else:  # edges: block maxima at the ends of the MFMA range and just outside it
        f = emax - rng.integers(0, 10, (R, K // 32, 32))
        for row, top in enumerate([64 + 9, 63, 220, 221, 127, 64]):
            f[row] += top - emax[row]
            f[row, :, 0] = top
        iq = _bf16_fields(rng, np.maximum(f, 1)).reshape(R, K)
    iq = iq.reshape(B, Qs, H, d)
    codes = rng.integers(0, 256, (B, N, H, d // 2)).astype(np.uint8)
    sc = ((rng.random((B, N, K // 32)) + 0.5) * np.exp2(rng.integers(-20, 20, (B, N, K // 32))) *
          np.where(rng.random((B, N, K // 32)) < 0.2, -1.0, 1.0))
    sc[:, ::11, 3] = 0.0
    scales = sc.astype(np.float32)
    for causal in (-1, N - Qs - 100):
        got = csa2.index_score(dev(iq), dev(codes), "fp4", ik_scales=dev(scales), causal_offset=causal)
        torch.cuda.synchronize()
        nv = None if causal < 0 else np.tile(causal + 1 + np.arange(Qs), B).astype(np.int64)
        want = oracle.index_score("fp4", iq, codes, n_valid_row=nv, ik_scales=scales)
        assert bits_eq(host(got), want), case


def _fp4_row_queries(rng, R, K):
    """bf16 index queries of three kinds by row: N(0,1) values (one band pair on the
    matrix cores), values spread over 28 binades below each block's largest (two band
    pairs), and one value 28 binades down (outside the bands: the per-thread path)."""
    emax = 127 + rng.integers(-3, 4, (R, K // 32, 1))
    f = emax - rng.integers(0, 28, (R, K // 32, 32))
    f[:, :, 0] = emax[:, :, 0]
    f[:, :, 1] = emax[:, :, 0] - 27
    iq = _bf16_fields(rng, f).reshape(R, K)
    iq[0::3] = synth.to_bf16_bits(rng.normal(size=(len(range(0, R, 3)), K)).astype(np.float32))
    iq[2::3, 37] = ((iq[2::3, 37].astype(np.int64) & 0x807f) |
                    ((emax[2::3, 1, 0] - 28) << 7)).astype(np.uint16)
    return iq


@pytest.mark.parametrize("B,N,causal", [(32, 65536, -1), (200, 3000, -1), (64, 8192, 5000), (40, 5000, -1),
                                        (33, 4097, 4096)])
def test_index_score_fp4_mfma_decode_shapes(B, N, causal):
    # FP4 keys with K = 256 and one query row per sequence on the matrix-core scorer, bit for bit
    # at the FP4-key decode shape (32 x 65,536: 4,096 workgroups of 512 entries) and at shapes
    # whose rows end inside a block: 200 rows of 6 blocks (the last of 440 entries), 64 rows cut
    # at 5,001 entries, 40 rows of 10 blocks (the last of 392) and 33 rows that end on a 1-entry
    # block.  Rows cycle through one band pair, two band pairs and the per-thread path
    rng = np.random.default_rng(B * 7 + N)
    K = 256
    iq = _fp4_row_queries(rng, B, K).reshape(B, 1, 4, 64)
    codes = rng.integers(0, 256, (B, N, 4, 32)).astype(np.uint8)
    sc = ((rng.random((B, N, K // 32)) + 0.5) * np.exp2(rng.integers(-20, 20, (B, N, K // 32))) *
          np.where(rng.random((B, N, K // 32)) < 0.2, -1.0, 1.0))
    sc[:, ::11, 3] = 0.0
    scales = sc.astype(np.float32)
    got = csa2.index_score(dev(iq), dev(codes), "fp4", ik_scales=dev(scales), causal_offset=causal)
    torch.cuda.synchronize()
    nv = None if causal < 0 else np.full(B, min(causal + 1, N), np.int64)
    want = oracle.index_score("fp4", iq, codes, n_valid_row=nv, ik_scales=scales)
    assert bits_eq(host(got), want)


def test_w7_scaled_fp4_ragged_batch():
    # the FP4-key recipe at batch 40: Full scores every sequence's valid entries on the
    # matrix-core scorer with the digit histogram (rows from 1 to 5,000 valid entries, most
    # ending inside a block, one with a single entry)
    rng = np.random.default_rng(78)
    nv = rng.integers(1, 5001, 40)
    nv[[0, 7, 19]] = [5000, 1, 513]
    Run(W7.scaled(B=40, N=5000, k=300), n_valid=[int(v) for v in nv]).check_all()


# ---------------------------------------------------------------- S3 top-k
def _topk_scores(R, N, seed):
    rng = np.random.default_rng(seed)
    s = rng.normal(size=(R, N)).astype(np.float32) * 16
    for r in range(R):
        src, dst = rng.integers(0, N, 300), rng.integers(0, N, 300)
        s[r, dst] = s[r, src]
    s[0, :] = 3.0
    s[1, ::2] = 0.0
    s[1, 1::2] = -0.0
    s[2, rng.integers(0, N, 50)] = -np.inf
    s[3] = np.round(s[3])  # heavy ties everywhere
    return s


@pytest.mark.parametrize("k", [1, 100, 2048, 19999, 25000])
def test_topk_parity(k):
    R, N = 7, 20000
    s = _topk_scores(R, N, k)
    nv = np.array([N, N, 12345, N, 0, 4097, 77], np.int32)
    got = csa2.topk(dev(s), k, n_valid=dev(nv))
    torch.cuda.synchronize()
    ref = oracle.topk(s, k, n_valid=nv.astype(np.int64))
    assert np.array_equal(host(got), ref)


@pytest.mark.parametrize("k", [1, 700, 4099])
def test_topk_parity_unaligned_rows(k):
    # an odd row length: rows start off 16-byte boundaries, so every score is
    # read one at a time
    R, N = 5, 4099
    s = _topk_scores(R, N, 11 + k)
    nv = np.array([N, 4098, 17, N, 1], np.int32)
    got = csa2.topk(dev(s), k, n_valid=dev(nv))
    torch.cuda.synchronize()
    assert np.array_equal(host(got), oracle.topk(s, k, n_valid=nv.astype(np.int64)))


@pytest.mark.parametrize("R,N", [(4, 200003), (8, 262144), (4, (1 << 19) - 3)])
def test_topk_parity_long_rows_sliced(R, N):
    # a few rows longer than 2^17 entries take the sliced path (compaction spread
    # over the chip, then one final workgroup per row); ties, signed zeros, -inf
    # and short valid counts as in the row-kernel tests
    for k in (1, 2048, 9000):
        s = _topk_scores(R, N, 31 + k)
        nv = np.array([N, N - 7, 131073, 9, N, 150000, 1, N][:R], np.int32)
        got = csa2.topk(dev(s), k, n_valid=dev(nv))
        torch.cuda.synchronize()
        assert np.array_equal(host(got), oracle.topk(s, k, n_valid=nv.astype(np.int64))), (R, N, k)


def test_topk_parity_long_row_multi_pass_slices():
    # beyond 2^24 entries a slice spans several 4096-entry compaction passes
    N = (1 << 24) + 5000
    rng = np.random.default_rng(5)
    s = rng.normal(size=(1, N)).astype(np.float32)
    s[0, rng.integers(0, N, 4000)] = s[0, rng.integers(0, N, 4000)]
    for k in (2048, 7000):
        got = csa2.topk(dev(s), k)
        torch.cuda.synchronize()
        assert np.array_equal(host(got), oracle.topk(s, k))


# ---------------------------------------------------------------- S5+S6 attend
@pytest.mark.parametrize("B,Qs,Hq,D,W,k,wlen", [
    (3, 1, 16, 128, 128, 300, None),
    (3, 1, 16, 128, 128, 300, [128, 5, 0]),
    (2, 4, 16, 128, 128, 64, None),
    (2, 3, 4, 64, 8, 40, [8, 2]),
    (1, 1, 32, 256, 16, 33, None),
    (2, 3, 16, 96, 40, 70, [40, 3]),        # odd number of scale blocks
    (1, 1, 8, 160, 128, 200, None),
    (1, 1100, 16, 128, 16, 64, None),       # enough rows for one split per row
    (2, 1, 16, 128, 128, 0, [128, 50]),     # window only
    (2, 2, 16, 128, 0, 96, None),           # no window
])
def test_attend_parity(B, Qs, Hq, D, W, k, wlen):
    N = 3000
    rng = np.random.default_rng(B * 100 + Qs * 10 + Hq + D)
    x = synth.normal_f32(synth.seed(0, 920), B * N * D).reshape(B * N, D)
    oc, os_ = oracle.fp4_pack(x)
    oc, os_ = oc.reshape(B, N, D // 2), os_.reshape(B, N, D // 32)
    gc, gs = csa2.fp4_pack(dev(x.reshape(B, N, D)))
    q = synth.normal_bf16(synth.seed(0, 921), B * Qs * Hq * D).reshape(B, Qs, Hq, D)
    wk = synth.normal_bf16(synth.seed(0, 922), B * (Qs + W - 1) * D).reshape(B, Qs + W - 1, D)
    wv = synth.normal_bf16(synth.seed(0, 923), B * (Qs + W - 1) * D).reshape(B, Qs + W - 1, D)
    idx = np.full((B * Qs, k), -1, np.int32)
    for r in range(B * Qs):
        m = int(rng.integers(0, k + 1))
        idx[r, :m] = np.sort(rng.choice(N, m, replace=False))
    wl = None if wlen is None else np.array(wlen, np.int32)
    out, lse = csa2.sparse_attend(dev(q), gc, gs, dev(idx), dev(wk), dev(wv), W, 1 / np.sqrt(D),
                                  wlen=None if wl is None else dev(wl))
    torch.cuda.synchronize()
    ro, rl = oracle.attend(q, oc, os_, idx, wk, wv, W, np.float32(1 / np.sqrt(D)), wlen=wl)
    assert rel_err(host(out), ro) <= TOL
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(host(lse)))
    assert np.allclose(host(lse)[fin], rl[fin], rtol=0, atol=TOL)
    assert np.all(host(out)[~fin] == 0)


def test_attend_never_reads_invalid_window_rows_or_empty_slots():
    # rows before the valid tail of the window hold NaN / Inf, and the record every
    # empty (-1) slot is clamped to has a NaN scale: none of them may reach the result
    B, Qs, Hq, D, W, k, N = 3, 3, 16, 128, 40, 70, 500
    rng = np.random.default_rng(77)
    x = synth.normal_f32(synth.seed(0, 930), B * N * D).reshape(B * N, D)
    oc, os_ = oracle.fp4_pack(x)
    oc, os_ = oc.reshape(B, N, D // 2), os_.reshape(B, N, D // 32)
    os_[:, 0, :] = np.nan
    wrows = Qs + W - 1
    q = synth.normal_bf16(synth.seed(0, 931), B * Qs * Hq * D).reshape(B, Qs, Hq, D)
    wk = synth.normal_bf16(synth.seed(0, 932), B * wrows * D).reshape(B, wrows, D)
    wv = synth.normal_bf16(synth.seed(0, 933), B * wrows * D).reshape(B, wrows, D)
    wl = np.array([5, 1, wrows - 2], np.int32)
    for b in range(B):
        wk[b, : wrows - wl[b]] = 0x7FC0  # NaN
        wv[b, : wrows - wl[b]] = 0x7F80  # +Inf
    idx = np.full((B * Qs, k), -1, np.int32)
    for r in range(B * Qs):
        m = int(rng.integers(1, k - 5))
        idx[r, :m] = np.sort(rng.choice(np.arange(1, N), m, replace=False))
    out, lse = csa2.sparse_attend(dev(q), dev(oc), dev(os_), dev(idx), dev(wk), dev(wv), W, 1 / np.sqrt(D),
                                  wlen=dev(wl))
    torch.cuda.synchronize()
    ro, rl = oracle.attend(q, oc, os_, idx, wk, wv, W, np.float32(1 / np.sqrt(D)), wlen=wl)
    assert np.all(np.isfinite(ro)) and np.all(np.isfinite(host(out)))
    assert rel_err(host(out), ro) <= TOL
    assert np.allclose(host(lse), rl, rtol=0, atol=TOL)


# ---------------------------------------------------------------- S4 layer steps
class Run:
    """One workload run through both sides, layer by layer."""

    def __init__(self, wl, n_valid=None, ikeys=None, iq=None):
        self.wl = wl
        self.inp = make_inputs(wl, n_valid=n_valid)
        if ikeys is not None:  # replace every group's index keys (same shape and dtype)
            self.inp.ikeys = [ikeys(g, k) for g, k in enumerate(self.inp.ikeys)]
        if iq is not None:
            for L in self.inp.layers:
                if L["iq"] is not None:
                    L["iq"] = iq(L["iq"])
        B, N, D, H, d = wl.B, wl.N, wl.D, wl.H_I, wl.d_I
        self.g_gpu, self.g_orc = [], []
        for g in range(wl.groups):
            x = self.inp.cache_x[g]
            oc, os_ = oracle.fp4_pack(x.reshape(B * N, D))
            gc, gs = csa2.fp4_pack(dev(x))
            if wl.idx_dtype == "fp4":
                # FP4 index keys: each side packs the fp32 key values with its own codec
                K = H * d
                kx = self.inp.ikeys[g].reshape(B * N, K)
                okc, oks = oracle.fp4_pack(kx)
                gkc, gks = csa2.fp4_pack(dev(kx))
                o_keys, o_ks = okc.reshape(B, N, H, d // 2), oks.reshape(B, N, K // 32)
                g_keys, g_ks = gkc.reshape(B, N, H, d // 2), gks.reshape(B, N, K // 32)
            else:
                o_keys, o_ks = self.inp.ikeys[g].copy(), None
                g_keys, g_ks = dev(self.inp.ikeys[g]), None
            self.g_orc.append(oracle.Group(oc.reshape(B, N, D // 2), os_.reshape(B, N, D // 32), o_keys,
                                           self.inp.n_valid.astype(np.int64), wl.idx_dtype, wl.k,
                                           max_rows=B * wl.Qs, ikey_scales=o_ks,
                                           pool_blocks=wl.pool_blocks))
            self.g_gpu.append(csa2.Group(gc, gs, g_keys, dev(self.inp.n_valid), wl.idx_dtype, wl.k,
                                         sel_rows=B * wl.Qs, ikey_scales=g_ks, pool_blocks=wl.pool_blocks))

    def layer(self, li):
        L = self.inp.layers[li]
        g = L["group"]
        mode = L["mode"]
        kw = dict(q=L["q"], wk=L["wk"], wv=L["wv"], W=self.wl.W, sm_scale=np.float32(self.wl.sm_scale))
        if L["iq"] is not None:
            kw["iq"] = L["iq"]
        if L["new_entry"] is not None:
            kw["new_entry"] = L["new_entry"]
            kw["new_ikey"] = L["new_ikey"]
        rc, ro, rl = self.g_orc[g].layer_step(mode, **kw)
        assert rc == 0
        gkw = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in kw.items()}
        go, gl = self.g_gpu[g].layer_step(mode, **gkw)
        torch.cuda.synchronize()
        return mode, g, ro, rl, host(go), host(gl)

    def check_all(self):
        for li in range(len(self.inp.layers)):
            mode, g, ro, rl, go, gl = self.layer(li)
            assert np.array_equal(host(self.g_gpu[g].sel), self.g_orc[g].sel), (li, mode)
            err = rel_err(go, ro)
            assert err <= TOL, (li, mode, err)
            assert np.allclose(gl, rl, rtol=0, atol=TOL), (li, mode)
            if mode == "F":
                assert bits_eq(host(self.g_gpu[g].codes), self.g_orc[g].codes)
                assert bits_eq(host(self.g_gpu[g].scales), self.g_orc[g].scales)
                assert bits_eq(host(self.g_gpu[g].ikeys), self.g_orc[g].ikeys)
                if self.g_orc[g].ikey_scales is not None:
                    assert bits_eq(host(self.g_gpu[g].ikey_scales), self.g_orc[g].ikey_scales)
                if self.wl.pool_blocks:
                    R, P = self.wl.B * self.wl.Qs, self.wl.pool_blocks
                    assert np.array_equal(host(self.g_gpu[g].pool)[:R, :P], self.g_orc[g].pool[:R, :P])


def test_layer_step_w1_full_size():
    Run(W1).check_all()


def test_group_w2_scaled_ragged():
    Run(W2.scaled(B=3, N=10000), n_valid=[10000, 7777, 9001]).check_all()


def test_w3_scaled_fp8():
    Run(W3.scaled(B=2, N=9000), n_valid=[9000, 5000]).check_all()


@pytest.mark.parametrize("B,N,causal", [(40, 5000, -1), (40, 5000, 2047), (33, 4097, 4096), (300, 1200, -1)])
def test_index_score_e4m3_persistent_stream(B, N, causal):
    # e4m3 keys with K = 256 and one query row per sequence: once rows x 512-entry blocks exceed
    # 256 the stream runs as resident workgroups over runs of a row's blocks.  40 x 10 blocks
    # gives 6 workgroups per row with 2 blocks each (one with none); 33 x 9 blocks ends every row
    # on a 1-entry block; 300 rows take one workgroup each over 3 blocks
    iq = synth.normal_idx("e4m3", synth.seed(0, 960), B * 4 * 64).reshape(B, 1, 4, 64)
    ik = synth.normal_idx("e4m3", synth.seed(0, 961), B * N * 4 * 64).reshape(B, N, 4, 64)
    got = csa2.index_score(dev(iq), dev(ik), "e4m3", causal_offset=causal)
    torch.cuda.synchronize()
    nv = None if causal < 0 else np.full(B, min(causal + 1, N), np.int64)
    ref = oracle.index_score("e4m3", iq, ik, n_valid_row=nv)
    assert bits_eq(host(got), ref)


def test_w3_scaled_persistent_stream_ragged():
    # the long-context recipe at batch 40: Full scores every sequence's valid entries through
    # the persistent stream (rows from 1 to 5,000 valid entries, blocks cut mid-run)
    rng = np.random.default_rng(77)
    nv = rng.integers(1, 5001, 40)
    nv[[0, 7, 19]] = [5000, 1, 513]
    Run(W3.scaled(B=40, N=5000, k=300), n_valid=[int(v) for v in nv]).check_all()


def test_group_save_restore_resumes_bitwise():
    # Full and Reindex, then the group goes to a pinned host image, its device
    # buffers are overwritten, the image comes back, and the two Reuse layers
    # give the same bits as an uninterrupted run
    wl = W2.scaled(B=3, N=6000, k=500)
    nv = [5000, 6000, 4321]  # n_valid_max below N_cap: strided copies
    ref = Run(wl, n_valid=nv)
    ref_out = [ref.layer(li)[4:] for li in range(4)]
    run = Run(wl, n_valid=nv)
    for li in range(2):
        run.layer(li)
    g = run.g_gpu[0]
    n = int(max(nv))
    before = [host(t).copy() for t in (g.codes[:, :n], g.scales[:, :n], g.ikeys[:, :n], g.sel)]
    image = g.save()
    torch.cuda.synchronize()
    assert image.numel() == g.image_bytes()
    g.codes.fill_(0x5A)
    g.scales.fill_(float("nan"))
    g.ikeys.fill_(0x7FC1)
    g.sel.fill_(-7)
    g.restore(image)
    torch.cuda.synchronize()
    after = [host(t) for t in (g.codes[:, :n], g.scales[:, :n], g.ikeys[:, :n], g.sel)]
    for a, b in zip(before, after):
        assert bits_eq(a, b)
    for li in range(2, 4):
        mode, gi, ro, rl, go, gl = run.layer(li)
        assert mode == "Ru"
        assert bits_eq(go, ref_out[li][0]) and bits_eq(gl, ref_out[li][1]), li
        # and the resumed layers still match the oracle, which never left the host
        assert np.array_equal(host(run.g_gpu[gi].sel), run.g_orc[gi].sel)
        assert rel_err(go, ro) <= TOL and np.allclose(gl, rl, rtol=0, atol=TOL), li


def test_hierarchical_group_save_restore_keeps_the_pool():
    # saved after Full: the image carries the pool, and the Reindex that follows
    # the restore searches the same pool as an uninterrupted run
    wl = W8.scaled(B=2, N=3000, k=200, pool_blocks=50)
    nv = [3000, 2500]
    ref = Run(wl, n_valid=nv)
    ref_res = [ref.layer(li) for li in range(2)]
    ref_sel = host(ref.g_gpu[0].sel).copy()
    run = Run(wl, n_valid=nv)
    run.layer(0)
    g = run.g_gpu[0]
    pool_before = host(g.pool).copy()
    image = g.save()
    torch.cuda.synchronize()
    assert image.numel() == g.image_bytes()
    g.pool.fill_(-3)
    g.sel.fill_(-7)
    g.restore(image)
    torch.cuda.synchronize()
    assert bits_eq(host(g.pool), pool_before)
    mode, _, ro, rl, go, gl = run.layer(1)
    assert mode == "Ri"
    assert np.array_equal(host(g.sel), ref_sel)
    assert bits_eq(go, ref_res[1][4]) and bits_eq(gl, ref_res[1][5])
    # the Reindex after the restore against the oracle's own pool and selection
    assert np.array_equal(host(g.sel), run.g_orc[0].sel)
    assert np.array_equal(host(g.pool)[:, :50], run.g_orc[0].pool[:, :50])
    assert rel_err(go, ro) <= TOL and np.allclose(gl, rl, rtol=0, atol=TOL)


def test_w7_scaled_fp4_index_keys():
    Run(W7.scaled(B=3, N=6000, k=600), n_valid=[6000, 4097, 5555]).check_all()


def test_w8_scaled_hierarchical_ragged():
    # 125 blocks of 8 per row, 60 kept: Reindex ranks 480 candidates
    Run(W8.scaled(B=3, N=1000, k=100, pool_blocks=60), n_valid=[1000, 411, 999]).check_all()


def test_w8_hierarchical_pool_covers_every_block():
    Run(W8.scaled(B=2, N=800, k=64, pool_blocks=100), n_valid=[800, 123]).check_all()


def test_w8_hierarchical_all_scores_equal():
    # equal keys: every block ties, the pool is the first blocks and Reindex the first entries
    Run(W8.scaled(B=2, N=2000, k=50, pool_blocks=20), n_valid=[2000, 1501],
        ikeys=lambda g, k: np.full_like(k, k.flat[0])).check_all()


def _fp4_band_queries(iq):
    # rows of every kind the FP4 matrix-core scorer meets, by row index mod 4: one band pair,
    # two band pairs (a value 20 binades below its block's largest), and rows it leaves to the
    # queue (a value 30 binades below, or a subnormal)
    out = iq.copy()
    flat = out.reshape(-1, out.shape[-2] * out.shape[-1])
    for r in range(flat.shape[0]):
        emax = int(((flat[r, :32] >> 7) & 0xFF).max())
        kind = r % 4
        if kind in (1, 2):
            flat[r, 5] = ((emax - (20 if kind == 1 else 30)) << 7) | 0x35
        elif kind == 3:
            flat[r, 9] = 0x0003
    return out


def test_w7_fp4_keys_rows_outside_the_bands():
    Run(W7.scaled(B=4, N=3000, k=300), n_valid=[3000, 2999, 1234, 3000], iq=_fp4_band_queries).check_all()


def test_w8_hierarchical_fp4_keys_and_draft_rows():
    Run(W8.scaled(B=2, N=3000, k=120, pool_blocks=40, idx_dtype="fp4"), n_valid=[3000, 2222]).check_all()
    Run(W8.scaled(B=2, N=3000, k=120, pool_blocks=40, Qs=5), n_valid=[3000, 1999]).check_all()


def test_w8_pool_size_layer_step():
    # the real pool (2,048 blocks = 16,384 candidates) over 20,000 entries
    Run(W8.scaled(B=2, N=20000), n_valid=[20000, 17003]).check_all()


def test_verify5_w6_scaled():
    # a draft block of 5 queries per sequence through Full/Reindex/Reuse/Reuse
    Run(W6.scaled(B=3, N=5000, k=700)).check_all()


def test_verify5_w6_ragged_n_valid():
    Run(W6.scaled(B=4, N=3000, k=256), n_valid=[3000, 2048, 300, 5]).check_all()


def _tie_keys(g, k):
    # the index keys of the bf16 tie cases: sums on (or a hair beside) fp32
    # midpoints, extreme exponent spreads, cancellation
    b = lambda v: int(synth.to_bf16_bits(np.array([v], np.float32))[0])  # noqa: E731
    pats = [{0: 1.0, 1: 2.0 ** -24}, {0: 1.0, 1: 3 * 2.0 ** -24}, {0: 1.0, 1: 2.0 ** -24, 2: 2.0 ** -80},
            {0: 2.0 ** 100, 1: 1.0, 2: -(2.0 ** 100)}, {0: 2.0 ** 60, 1: -(2.0 ** 60), 2: 3.0},
            {0: 2.0 ** -126, 1: 2.0 ** -130}, {0: -(2.0 ** -120), 1: 2.0 ** -120}]
    out = np.zeros_like(k)
    B, N = k.shape[:2]
    flat = out.reshape(B, N, -1)
    for j in range(N):
        for e, v in pats[j % len(pats)].items():
            flat[:, j, e] = b(v)
        flat[:, j, 10 + j % 50] = b(2.0 ** -(j % 90)) if j % 3 == 0 else 0
    return out


def _tie_queries(iq):
    out = np.zeros_like(iq)
    flat = out.reshape(iq.shape[0], iq.shape[1], -1)
    flat[:, :, :3] = 0x3F80
    flat[:, :, 10:60] = 0x3F80
    flat[:, 1::2, 64:] = synth.to_bf16_bits(np.array([0.5], np.float32))[0]  # rows differ past 64
    return out


def test_draft_rows_share_key_loads_ties_and_groups():
    # several query rows per sequence go through the shared-load scorer; undecided
    # scores are queued and recomputed exactly (heavy ties make the selection
    # depend on every bit)
    Run(W6.scaled(B=2, N=999, k=100, H_I=2, d_I=64), ikeys=_tie_keys, iq=_tie_queries).check_all()
    Run(W6.scaled(B=2, N=1500, k=200, Qs=3), n_valid=[1500, 1001]).check_all()
    Run(W6.scaled(B=2, N=1500, k=200, Qs=7, H_I=2, d_I=64), n_valid=[1500, 777]).check_all()


def test_prefill_w4_scaled():
    Run(W4.scaled(N=6000, Qs=96, k=512)).check_all()


# Prefill chunks with e4m3 index keys select through the MFMA candidate path
# (sampled threshold, filtered score GEMM, exact band) or its exact row fallback.
def test_prefill_mfma_large_k_ragged():
    Run(W4.scaled(B=2, N=40000, Qs=300, k=2048), n_valid=[40000, 23456]).check_all()


def test_prefill_mfma_k128_every_entry_a_candidate():
    # k close to the visible count: the threshold admits every entry
    Run(W4.scaled(N=3000, Qs=64, k=2048, H_I=1, d_I=128)).check_all()


def _e4m3_small_ints(a, seed):
    # keys and queries in {-1, 0, +1}: integer scores with many exact ties
    rng = np.random.default_rng(seed)
    vals = np.array([0xB8, 0x00, 0x38], np.uint8)  # -1, 0, +1 in e4m3
    return vals[rng.integers(0, 3, a.shape)]


def test_prefill_mfma_exact_ties_take_lower_index():
    Run(W4.scaled(N=20000, Qs=128, k=512),
        ikeys=lambda g, k: _e4m3_small_ints(k, 7 + g),
        iq=lambda q: _e4m3_small_ints(q, 99)).check_all()


def test_prefill_mfma_all_equal_scores_fall_back():
    # identical keys: every score ties, the candidate list overflows, and every
    # row is recomputed by the exact row kernel
    Run(W4.scaled(N=20000, Qs=32, k=512),
        ikeys=lambda g, k: np.full_like(k, 0x38)).check_all()


def _time_layer(run, li, reps=3):
    # GPU time of repeating layer li (a Full layer rewrites the same entries, so the
    # repeat is idempotent), HIP events on the layer's stream
    L = run.inp.layers[li]
    kw = dict(q=dev(L["q"]), wk=dev(L["wk"]), wv=dev(L["wv"]), W=run.wl.W, sm_scale=run.wl.sm_scale,
              iq=dev(L["iq"]), new_entry=dev(L["new_entry"]), new_ikey=dev(L["new_ikey"]))
    g = run.g_gpu[L["group"]]
    g.layer_step(L["mode"], **kw)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(reps):
        g.layer_step(L["mode"], **kw)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def test_prefill_mfma_rows_beyond_2_18_visible_entries():
    # a 1M-token context compressed 4x holds 2^18 entries; a chunk on top of it makes
    # every row see more.  The band selection writes its output in passes of 2^18
    # entries, so these rows stay on the MFMA path: bit-exact against the oracle, and
    # fast (a row recomputed by the exact fallback alone would take > 10 ms)
    run = Run(W4.scaled(N=(1 << 18) + 3000, Qs=48, k=512))
    run.check_all()
    ms = _time_layer(run, 0)
    print(f"prefill chunk of 48 rows over {(1 << 18) + 3000} entries: {ms:.3f} ms")
    assert ms < 8.0, ms


def test_prefill_k_above_the_mfma_band_limit_takes_the_exact_path():
    # k beyond what the band selection holds (3k + 2048 candidates in LDS): the chunk is
    # scored and selected on the exact path instead, still bit-exact
    Run(W4.scaled(N=12000, Qs=40, k=2100), n_valid=[12000]).check_all()


def _e4m3_values(bits):
    """Exact values of e4m3fn bit patterns (no NaN among the inputs here)."""
    b = bits.astype(np.int64)
    e, m = (b >> 3) & 15, b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where(b & 0x80, -mag, mag)


def _group_exp(bits):
    """Largest e4m3 exponent (unbiased; zero and subnormal count as -6) of each group of 8
    consecutive elements along the last axis."""
    f = ((bits.astype(np.int64) >> 3) & 15).reshape(*bits.shape[:-1], -1, 8).max(-1)
    return np.maximum(f, 1) - 7


def _mfma_band_bound(qb, kb):
    """Bound on |s^ - s| for every (row, entry) pair of e4m3 bit rows qb [R][K] and kb [N][K],
    under the measured model of v_mfma_scale_f32_16x16x128_f8f6f4: each product is cut toward
    zero to a multiple of 2^(ea + eb - 13) of its group of 8 (error < 2^(eq_g + ek_g - 10) per
    group), and the group sums are added in fp32 (2 K/8 + 1 roundings, u = 2^-23, doubled)."""
    K = qb.shape[1]
    qv, kv = _e4m3_values(qb), _e4m3_values(kb)
    n = 2 * (K // 8) + 1
    gam = n * 2.0 ** -23 / (1 - n * 2.0 ** -23)
    E = 2 * gam * np.sqrt((qv * qv).sum(1))[:, None] * np.sqrt((kv * kv).sum(1))[None, :]
    T = np.exp2(_group_exp(qb)) @ np.exp2(_group_exp(kb)).T * 2.0 ** -10
    return E + T, qv, kv


def _trunc_groups(n, K, big, small):
    """Rows whose every group of 8 holds e4m3 codes (big, small x 7)."""
    x = np.full((n, K // 8, 8), small, np.uint8)
    x[:, :, 0] = big
    return x.reshape(n, K)


def test_mfma_score_error_within_the_band_bound():
    # The prefill selection trusts |s^ - s| <= delta for the fp32 MFMA scores s^.  The bound
    # follows the instruction's measured behaviour (see _mfma_band_bound); the kernel uses it
    # with the sequence's largest key exponent per group.  With N <= 2048 the threshold-sample
    # GEMM runs at stride 1, so the workspace holds s^ for every (row, entry); they are read
    # back and checked against the exact sums on adversarial e4m3 inputs: all-subnormal rows,
    # +-448 cancellation with small terms, random bit patterns, and groups of one 448 x 448
    # product with seven products just below the group's truncation step (7 x 1 < 2^3): the
    # last lose 49 per group, more than an fp32-summation bound allows.
    rng = np.random.default_rng(448)
    B, N, Qs, H, d, Hq, D, W, k = 1, 2048, 80, 4, 64, 16, 128, 8, 64
    K = H * d
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)

    def kind(n, t, side):
        if t == 0:  # N(0,1) rounded to e4m3
            return synth.to_e4m3_bits(rng.normal(size=(n, K)).astype(np.float32))
        if t == 1:  # subnormals only
            return (rng.integers(1, 8, (n, K)) | (rng.integers(0, 2, (n, K)) << 7)).astype(np.uint8)
        if t == 2:  # +-448 with small terms mixed in: large partial sums that cancel
            x = np.where(rng.random((n, K)) < 0.5, 0x7E, 0xFE).astype(np.uint8)
            small = rng.random((n, K)) < 0.25
            x[small] = rng.integers(1, 0x30, int(small.sum())).astype(np.uint8)
            return x
        if t == 4:  # (448, 7 x 7) against (448, 1 x 7) in every group
            return _trunc_groups(n, K, 0x7E, 0x4E if side == "q" else 0x38)
        return codes[rng.integers(0, codes.size, (n, K))]  # any bit pattern

    iq = np.concatenate([kind(Qs // 5, t, "q") for t in range(5)]).reshape(B, Qs, H, d)
    ik = np.concatenate([kind(N // 5 + (N % 5 if t == 0 else 0), t, "k") for t in range(5)])
    ik = ik[rng.permutation(N)].reshape(B, N, H, d)
    new_ikey = kind(Qs, 3, "k").reshape(B, Qs, H, d)
    x = synth.normal_f32(synth.seed(0, 940), B * N * D).reshape(B, N, D)
    gc, gs = csa2.fp4_pack(dev(x))
    grp = csa2.Group(gc, gs, dev(ik), dev(np.array([N], np.int32)), "e4m3", k, sel_rows=Qs)
    q = synth.normal_bf16(synth.seed(0, 941), B * Qs * Hq * D).reshape(B, Qs, Hq, D)
    wk = synth.normal_bf16(synth.seed(0, 942), B * (Qs + W - 1) * D).reshape(B, Qs + W - 1, D)
    ne = synth.normal_f32(synth.seed(0, 943), B * Qs * D).reshape(B, Qs, D)
    ws = grp.workspace(Qs, Hq, W)
    grp.layer_step("F", q=dev(q), iq=dev(iq), wk=dev(wk), wv=dev(wk), W=W, sm_scale=0.125,
                   new_entry=dev(ne), new_ikey=dev(new_ikey), ws=ws)
    torch.cuda.synchronize()
    # the workspace starts with the exact-score rows [Qs][N] (fp32, 256-byte aligned), then
    # the sample scores [Qs][ncols] (ncols = N at stride 1)
    off = (Qs * N * 4 + 255) // 256 * 256
    samp = host(ws[off:off + Qs * N * 4].view(torch.float32)).reshape(Qs, N).astype(np.float64)
    keys = ik[0].reshape(N, K).copy()
    keys[N - Qs:] = new_ikey[0].reshape(Qs, K)
    bound, qv, kv = _mfma_band_bound(iq[0].reshape(Qs, K), keys)
    exact = qv @ kv.T  # e4m3 products and their partial sums are exact in fp64
    visible = np.arange(N)[None, :] <= (N - Qs + np.arange(Qs))[:, None]
    assert np.all(np.isneginf(samp[~visible]))
    err = np.abs(samp - exact)[visible]
    b = bound[visible]
    assert np.all(err <= b), float((err - b).max())
    ratio = float((err / np.where(b > 0, b, 1.0)).max())
    # the fp32-summation bound alone (2 gamma_(K-1) ||q|| ||k||) is exceeded by the truncation rows
    gam = (K - 1) * 2.0 ** -23 / (1 - (K - 1) * 2.0 ** -23)
    old = (2 * gam * np.sqrt((qv * qv).sum(1))[:, None] * np.sqrt((kv * kv).sum(1))[None, :])[visible]
    old_ratio = float((err / np.where(old > 0, old, 1.0)).max())
    print(f"MFMA score error: worst |s^ - s| / bound = {ratio:.3e}, / fp32-summation bound = {old_ratio:.3e} "
          f"over {int(visible.sum())} scores")
    assert old_ratio > 1.0
    assert np.all(err[b == 0] == 0)


def test_prefill_mfma_truncation_cannot_hide_an_entry():
    # Entry 5 has the highest exact score, 32 * (256 * 256 + 7 * 7.5), but the MFMA cuts its
    # 7.5 x 1 products below their groups' truncation step (2^3 next to 256 x 256), so its s^
    # sits 1680 below its score, while the k entries 10.. score 168 less than it, exactly
    # (their one extra product, 7.5 x 208, is a multiple of 8).  An fp32-summation bound
    # (about 514 here, with the key truncation) would rule entry 5 out; the band must reach it:
    # the selection is {5, 10, ..., 10+k-2}.
    rng = np.random.default_rng(5)
    B, N, Qs, H, d, Hq, D, W, k = 1, 2048, 16, 4, 64, 16, 128, 8, 64
    K = H * d
    iq = _trunc_groups(Qs, K, 0x78, 0x4F).reshape(B, Qs, H, d)
    neg = lambda n: synth.to_e4m3_bits(-np.abs(rng.normal(size=(n, K)) * 10).astype(np.float32))
    ik = neg(N)
    ik[5] = _trunc_groups(1, K, 0x78, 0x38)[0]
    ik[10:10 + k] = _trunc_groups(k, K, 0x78, 0x00)
    ik[10:10 + k, 1] = 0x75  # 208 next to the query's 7.5 in group 0: +1560, exact
    ik = ik.reshape(B, N, H, d)
    new_ikey = neg(Qs).reshape(B, Qs, H, d)
    x = synth.normal_f32(synth.seed(0, 950), B * N * D).reshape(B, N, D)
    gc, gs = csa2.fp4_pack(dev(x))
    grp = csa2.Group(gc, gs, dev(ik), dev(np.array([N], np.int32)), "e4m3", k, sel_rows=Qs)
    q = synth.normal_bf16(synth.seed(0, 951), B * Qs * Hq * D).reshape(B, Qs, Hq, D)
    wk = synth.normal_bf16(synth.seed(0, 952), B * (Qs + W - 1) * D).reshape(B, Qs + W - 1, D)
    ne = synth.normal_f32(synth.seed(0, 953), B * Qs * D).reshape(B, Qs, D)
    grp.layer_step("F", q=dev(q), iq=dev(iq), wk=dev(wk), wv=dev(wk), W=W, sm_scale=0.125,
                   new_entry=dev(ne), new_ikey=dev(new_ikey))
    torch.cuda.synchronize()
    keys = ik[0].reshape(N, K).copy()
    keys[N - Qs:] = new_ikey[0].reshape(Qs, K)
    nv = (N - Qs + 1 + np.arange(Qs)).astype(np.int64)
    s = oracle.index_score("e4m3", iq[0].reshape(1, Qs, H, d), keys.reshape(1, N, H, d), n_valid_row=nv)
    want = oracle.topk(s.reshape(Qs, N), k, n_valid=nv)
    assert np.array_equal(want[0], np.r_[5, np.arange(10, 10 + k - 1)])
    assert np.array_equal(host(grp.sel).reshape(Qs, k), want)


def test_stack_w5_scaled():
    Run(W5.scaled(B=2, N=5000, groups=2), n_valid=[5000, 4321]).check_all()


def test_n_valid_below_k_pads():
    Run(W2.scaled(B=2, N=3000, k=2048), n_valid=[3000, 1500]).check_all()


def test_modes_write_nothing_and_reuse_equals_full():
    run = Run(W2.scaled(B=2, N=5000))
    L = run.inp.layers
    g = run.g_gpu[0]
    go_full = run.layer(0)[4]
    snap = [t.clone() for t in (g.codes, g.scales, g.ikeys)]
    sel_full = g.sel.clone()
    # Reuse with the Full layer's own query and window reproduces its output bit for bit
    out, lse = g.layer_step("Ru", q=dev(L[0]["q"]), wk=dev(L[0]["wk"]), wv=dev(L[0]["wv"]),
                            W=run.wl.W, sm_scale=run.wl.sm_scale)
    torch.cuda.synchronize()
    assert bits_eq(host(out), go_full)
    # Reindex with the Full layer's index query selects the same entries
    g.layer_step("Ri", q=dev(L[0]["q"]), iq=dev(L[0]["iq"]), wk=dev(L[0]["wk"]), wv=dev(L[0]["wv"]),
                 W=run.wl.W, sm_scale=run.wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(g.sel, sel_full)
    for a, b in zip(snap, (g.codes, g.scales, g.ikeys)):
        assert torch.equal(a, b)
    # Reuse does not touch the selection either
    g.layer_step("Ru", q=dev(L[3]["q"]), wk=dev(L[3]["wk"]), wv=dev(L[3]["wv"]), W=run.wl.W,
                 sm_scale=run.wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(g.sel, sel_full)


def test_run_to_run_determinism():
    run = Run(W3.scaled(B=2, N=4000))
    L = run.inp.layers[0]
    g = run.g_gpu[0]
    args = dict(q=dev(L["q"]), iq=dev(L["iq"]), wk=dev(L["wk"]), wv=dev(L["wv"]), W=run.wl.W,
                sm_scale=run.wl.sm_scale)
    o1, l1 = g.layer_step("Ri", **args)
    s1 = g.sel.clone()
    o1 = o1.clone()
    o2, l2 = g.layer_step("Ri", **args)
    torch.cuda.synchronize()
    assert torch.equal(s1, g.sel) and torch.equal(o1, o2)
