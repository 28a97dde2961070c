"""Pins of the oracle's hierarchical search ("Inference-Efficient LLMs", section 5,
Hierarchical Sparse Indexing: an earlier Full layer keeps a candidate pool of blocks
of 8 positions, later Reindex layers rank only inside it).

The block rule (a block's score is the largest index score of its valid positions)
is a reading; the pins check the oracle against properties that do not restate its
sort: a pairwise dominance test for the pool, a rank count for the pool-restricted
top-k, the containment theorem that the max rule gives, and the special cases that
reduce to the plain top-k.
"""
import numpy as np
import pytest

import oracle

BLK = oracle.POOL_BLOCK


def beats(a, b):
    """(score, index) order: higher score first, then lower index; -0 == +0."""
    return a[0] > b[0] or (a[0] == b[0] and a[1] < b[1])


def block_key(row, j, nv):
    vals = [float(row[t]) for t in range(j * BLK, min((j + 1) * BLK, nv))]
    return (max(vals), j)


def check_pool(row, nv, P, pool):
    nb = (nv + BLK - 1) // BLK
    kept = [int(x) for x in pool if x >= 0]
    assert kept == sorted(kept)
    assert len(kept) == min(P, nb)
    assert all(x == -1 for x in pool[len(kept):])
    assert all(0 <= x < nb for x in kept)
    inside = set(kept)
    keys = {j: block_key(row, j, nv) for j in range(nb)}
    # every kept block beats every block left out
    for a in inside:
        for b in range(nb):
            if b not in inside:
                assert beats(keys[a], keys[b]), (a, b, keys[a], keys[b])


def rank_count_topk(row, cand, k):
    """Candidate j is kept iff fewer than k candidates beat it."""
    keys = {j: (float(row[j]), j) for j in cand}
    sel = sorted(j for j in cand if sum(beats(keys[i], keys[j]) for i in cand) < k)
    return sel + [-1] * (k - len(sel))


def tied_scores(rng, R, N):
    # a few distinct values so that ties are everywhere, +0 and -0 included
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 2.0, 3.0], dtype=np.float32)
    return vals[rng.integers(0, len(vals), (R, N))]


@pytest.mark.parametrize("seed", range(4))
def test_pool_blocks_dominance(seed):
    rng = np.random.default_rng(100 + seed)
    R, N = 6, 203
    s = rng.normal(size=(R, N)).astype(np.float32) if seed % 2 else tied_scores(rng, R, N)
    nv = rng.integers(1, N + 1, R)
    nv[0] = N
    nv[1] = 8 * 7 + 3  # partial last block
    for P in (1, 3, 8, 26, 40):
        pool = oracle.pool_blocks(s, P, nv)
        for r in range(R):
            check_pool(s[r], int(nv[r]), P, pool[r])


def test_pool_ignores_positions_past_n_valid():
    s = np.zeros((1, 64), dtype=np.float32)
    s[0, 21] = 1.0       # block 2, valid
    s[0, 44] = 100.0     # block 5, but position 44 >= n_valid = 43
    s[0, 42] = 0.5       # block 5, valid
    pool = oracle.pool_blocks(s, 2, [43])
    assert pool[0].tolist() == [2, 5]
    pool = oracle.pool_blocks(s, 1, [43])
    assert pool[0].tolist() == [2]


def test_pool_all_equal_takes_first_blocks():
    s = np.full((2, 100), 7.0, dtype=np.float32)
    pool = oracle.pool_blocks(s, 4, [100, 17])
    assert pool[0].tolist() == [0, 1, 2, 3]
    assert pool[1].tolist() == [0, 1, 2, -1]  # 17 positions make 3 blocks


@pytest.mark.parametrize("seed", range(4))
def test_pool_topk_rank_count(seed):
    rng = np.random.default_rng(200 + seed)
    R, N = 5, 160
    s = tied_scores(rng, R, N) if seed % 2 else rng.normal(size=(R, N)).astype(np.float32)
    nv = rng.integers(1, N + 1, R)
    nv[0] = 8 * 11 + 5
    pool = np.full((R, 9), -1, dtype=np.int32)
    for r in range(R):
        nb = (int(nv[r]) + BLK - 1) // BLK
        blocks = sorted(rng.choice(nb, size=min(nb, int(rng.integers(1, 10))), replace=False))
        pool[r, :len(blocks)] = blocks
    for k in (1, 5, 30, 72, 80):
        got = oracle.pool_topk(s, pool, k, nv)
        for r in range(R):
            cand = [b * BLK + t for b in pool[r] if b >= 0 for t in range(BLK) if b * BLK + t < nv[r]]
            assert got[r].tolist() == rank_count_topk(s[r], cand, k), (r, k)


@pytest.mark.parametrize("seed", range(6))
def test_flat_topk_lies_inside_a_pool_of_at_least_k_blocks(seed):
    # under the max rule, a top-k position's block is beaten by fewer than k blocks
    rng = np.random.default_rng(300 + seed)
    R, N = 4, 400
    s = tied_scores(rng, R, N) if seed % 2 else rng.normal(size=(R, N)).astype(np.float32)
    nv = rng.integers(1, N + 1, R)
    for k in (1, 4, 13, 40):
        flat = oracle.topk(s, k, n_valid=nv)
        for P in (k, k + 3):
            pool = oracle.pool_blocks(s, P, nv)
            inpool = oracle.pool_topk(s, pool, k, nv)
            for r in range(R):
                blocks = set(int(x) for x in pool[r] if x >= 0)
                assert all(j // BLK in blocks for j in flat[r] if j >= 0)
                # so ranking inside the pool gives back the flat selection
                assert inpool[r].tolist() == flat[r].tolist()


def test_pool_covering_every_block_is_the_flat_topk():
    rng = np.random.default_rng(7)
    s = rng.normal(size=(3, 90)).astype(np.float32)
    nv = np.array([90, 41, 8])
    pool = oracle.pool_blocks(s, 12, nv)
    for k in (1, 10, 50):
        assert np.array_equal(oracle.pool_topk(s, pool, k, nv), oracle.topk(s, k, n_valid=nv))


def _group(rng, B, N, P, k, nv):
    D, H, d = 32, 1, 16
    x = rng.normal(size=(B * N, D)).astype(np.float32)
    codes, scales = oracle.fp4_pack(x)
    import synth
    ik = synth.to_bf16_bits(rng.normal(size=(B, N, H, d)).astype(np.float32))
    return oracle.Group(codes.reshape(B, N, D // 2), scales.reshape(B, N, D // 32), ik,
                        np.asarray(nv, np.int64), "bf16", k, max_rows=B, pool_blocks=P)


def _layer_inputs(rng, B, D=32, H=1, d=16, W=2, Hq=2):
    import synth
    bf = lambda *sh: synth.to_bf16_bits(rng.normal(size=sh).astype(np.float32))
    return dict(q=bf(B, 1, Hq, D), W=W, sm_scale=0.25, wk=bf(B, W, D), wv=bf(B, W, D),
                iq=bf(B, 1, H, d))


def test_layer_modes_keep_and_use_the_pool():
    import synth
    rng = np.random.default_rng(11)
    B, N, P, k = 2, 120, 4, 6
    nv = [120, 77]
    g = _group(rng, B, N, P, k, nv)
    full = _layer_inputs(rng, B)
    full["new_entry"] = rng.normal(size=(B, 1, 32)).astype(np.float32)
    full["new_ikey"] = synth.to_bf16_bits(rng.normal(size=(B, 1, 1, 16)).astype(np.float32))
    rc, _, _ = g.layer_step("F", **full)
    assert rc == 0
    nv_row = np.asarray(nv, np.int64)
    s_full = oracle.index_score("bf16", full["iq"], g.ikeys, nv_row)[:, 0, :]
    assert np.array_equal(g.pool[:, :P], oracle.pool_blocks(s_full, P, nv_row))
    assert np.array_equal(g.sel, oracle.topk(s_full, k, n_valid=nv_row))
    ri = _layer_inputs(rng, B)
    rc, _, _ = g.layer_step("Ri", **ri)
    assert rc == 0
    s_ri = oracle.index_score("bf16", ri["iq"], g.ikeys, nv_row)[:, 0, :]
    assert np.array_equal(g.sel, oracle.pool_topk(s_ri, g.pool[:, :P], k, nv_row))
    for r in range(B):
        assert all(j // BLK in set(g.pool[r, :P].tolist()) for j in g.sel[r] if j >= 0)


def test_reindex_needs_a_pool_from_a_full_layer_of_the_same_rows():
    rng = np.random.default_rng(12)
    B, N = 1, 64
    g = _group(rng, B, N, 2, 4, [64])
    rc, _, _ = g.layer_step("Ri", **_layer_inputs(rng, B))
    assert rc == 4  # no Full layer has built the pool yet
