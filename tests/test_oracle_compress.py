"""Pins for the oracle's block statistics, selection and extraction (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from tests import brute


def rand_qk(seed, n, d=16):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, d)), r.standard_normal((n, d))


# ---------------------------------------------------------------- block statistics
def test_uniform_closed_form_masses():
    n = 256
    q, k = rand_qk(0, n)
    A = oracle.causal_map(q, k, 0.0)
    M = oracle.block_masses(A)
    for r in range(4):
        rows = np.arange(64 * r, 64 * r + 64)
        for c in range(r):
            assert math.isclose(M[r, c], float(np.sum(64.0 / (rows + 1))), rel_tol=1e-13)
        assert math.isclose(M[r, r], float(np.sum((rows - 64 * r + 1) / (rows + 1))), rel_tol=1e-13)
        assert np.all(M[r, r + 1:] == 0)
    assert M[0, 0] == pytest.approx(64.0, rel=1e-14)


@pytest.mark.parametrize("n", [64, 200, 257])
def test_block_rows_sum_to_row_count(n):
    q, k = rand_qk(n, n)
    A = oracle.causal_map(q, k, 0.8, 4.0)
    M = oracle.block_masses(A)
    R = M.shape[0]
    for r in range(R):
        assert math.isclose(M[r, : r + 1].sum(), min(64, n - 64 * r), rel_tol=1e-12)


def test_masses_brute_force_small_blocks():
    q, k = rand_qk(3, 13, 4)
    A = oracle.causal_map(q, k, 0.9, 4.0)
    B = brute.causal_map(q.tolist(), k.tolist(), 0.9, 4.0)
    M = oracle.block_masses(A, block=4)
    for r in range(4):
        for c in range(r + 1):
            ref = sum(B[i][j] for i in range(4 * r, min(4 * r + 4, 13)) for j in range(4 * c, min(4 * c + 4, 13)))
            assert math.isclose(M[r, c], ref, rel_tol=1e-12)


def test_row_stats_reproduce_map():
    q, k = rand_qk(5, 100)
    m, l = oracle.row_stats(q, k, 0.7, 4.0)
    A = oracle.causal_map(q, k, 0.7, 4.0)
    s = 0.7 * (q @ k.T)
    s[:, 0] += 4.0
    i, j = np.tril_indices(100)
    assert np.allclose(np.exp(s[i, j] - m[i]) / l[i], A[i, j], rtol=1e-12)
    assert np.allclose(m, np.array([s[t, : t + 1].max() for t in range(100)]))
    assert (l >= 1.0).all()


# ---------------------------------------------------------------- selection
@pytest.mark.parametrize("seed", range(12))
def test_greedy_matches_subset_enumeration(seed):
    r = np.random.default_rng(seed)
    nb = int(r.integers(1, 13))
    masses = r.uniform(0.0, 1.0, nb) ** 3
    tau = float(r.uniform(0.3, 0.99))
    kept = oracle.select_blocks(masses, tau)
    size, best, winners = brute.best_subset(masses.tolist(), tau)
    assert len(kept) == size
    assert kept in winners
    assert masses[kept].sum() / masses.sum() >= tau


def test_selection_edge_cases():
    m = np.array([0.1, 0.5, 0.2, 0.2])
    assert oracle.select_blocks(m, 1.0) == [0, 1, 2, 3]
    assert oracle.select_blocks(m, 2.0) == [0, 1, 2, 3]
    assert oracle.select_blocks(m, 1e-9) == [1]
    assert oracle.select_blocks(np.array([64.0]), 0.95) == [0]
    # ties go to the lower column: 0.2 (col 2) is taken before 0.2 (col 3)
    assert oracle.select_blocks(m, 0.6) == [1, 2]
    assert oracle.select_blocks(m, 0.75) == [1, 2, 3]


def test_selection_margin_values():
    m = np.array([0.1, 0.5, 0.25, 0.15])  # sorted: 0.5, 0.25, 0.15, 0.1
    # tau = 0.7: keep 0.5 + 0.25 = 0.75; gap 0.25 - 0.15 = 0.1; over 0.05; room 0.7 - 0.5 = 0.2
    assert math.isclose(oracle.selection_margin(m, 0.7), 0.05, rel_tol=1e-12)
    # tau = 0.76: keep 3 (0.9); gap 0.05; over 0.14; room 0.01
    assert math.isclose(oracle.selection_margin(m, 0.76), 0.01, rel_tol=1e-9)
    assert oracle.selection_margin(m, 1.0) == math.inf


# ---------------------------------------------------------------- extraction
def test_extracted_blocks_equal_rounded_map():
    n, tau = 200, 0.9
    q, k = rand_qk(9, n)
    res = oracle.compress_head(q, k, 1.1, 4.0, tau)
    A = oracle.causal_map(q, k, 1.1, 4.0)
    Ap = np.pad(A, ((0, 56), (0, 56)))
    for r, cols in enumerate(res["kept"]):
        kept_mass = 0.0
        for t, c in enumerate(cols):
            blk = Ap[64 * r: 64 * r + 64, 64 * c: 64 * c + 64]
            assert np.array_equal(res["blocks"][r][t], oracle.round_bf16(blk))
            kept_mass += blk.sum()
        assert kept_mass >= tau * min(64, n - 64 * r) * (1 - 1e-12)
    # diagonal blocks hold zeros above the diagonal and outside the sequence
    for r, cols in enumerate(res["kept"]):
        for t, c in enumerate(cols):
            blk = res["blocks"][r][t]
            if c == r:
                assert np.all(blk[np.triu_indices(64, 1)] == 0)
            if r == 3:
                assert np.all(blk[8:] == 0) and (c < 3 or np.all(blk[:, 8:] == 0))


def test_block_compress_layout_varlen():
    r = np.random.default_rng(10)
    lens = [70, 128, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H = 2
    q = r.standard_normal((H, cu[-1], 8))
    k = r.standard_normal((H, cu[-1], 8))
    scale, bias = np.array([0.9, 1.2]), np.array([4.0, 0.0])
    out = oracle.block_compress(q, k, scale, bias, cu, 0.8)
    Rs = [2, 2, 1]
    assert out["r_tot"] == 5 and out["nb_tot"] == 3 + 3 + 1
    assert len(out["row_ptr"]) == H * 5 + 1
    g = 0
    for h in range(H):
        off = 0
        for s, n in enumerate(lens):
            single = oracle.compress_head(q[h, cu[s]:cu[s + 1]], k[h, cu[s]:cu[s + 1]], scale[h], bias[h], 0.8)
            for rr in range(Rs[s]):
                cols = out["col_idx"][out["row_ptr"][g]: out["row_ptr"][g + 1]]
                assert list(cols) == single["kept"][rr]
                assert np.array_equal(out["vals"][out["row_ptr"][g]: out["row_ptr"][g + 1]], single["blocks"][rr])
                tri = out["masses"][h, off + rr * (rr + 1) // 2: off + rr * (rr + 1) // 2 + rr + 1]
                assert np.array_equal(tri, single["masses"][rr, : rr + 1])
                g += 1
            off += Rs[s] * (Rs[s] + 1) // 2
            assert np.array_equal(out["row_stats"][h, cu[s]:cu[s + 1], 0], single["m"])


def test_block_compress_empty_sequence():
    """A zero-length sequence in the batch has no block-rows: the block-sparse
    output equals that of the batch without it."""
    r = np.random.default_rng(11)
    lens = [70, 0, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = r.standard_normal((2, cu[-1], 8))
    k = r.standard_normal((2, cu[-1], 8))
    scale, bias = np.array([0.9, 1.2]), np.array([4.0, 0.0])
    a = oracle.block_compress(q, k, scale, bias, cu, 0.8)
    b = oracle.block_compress(q, k, scale, bias, np.array([0, 70, 75]), 0.8)
    assert a["r_tot"] == b["r_tot"] == 3
    for key in ("row_ptr", "col_idx", "vals", "masses", "row_stats"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("n,tau", [(200, 0.9), (256, 0.95), (130, 1.0)])
def test_block_row_matches_whole_head(n, tau):
    """The per-block-row oracle (used for sampled checks of long sequences) gives
    exactly the whole-head oracle's masses, kept set, margin, blocks and row
    statistics for every block-row, including a ragged last one."""
    rng = np.random.default_rng(11 + n)
    q = rng.standard_normal((n, 16))
    k = rng.standard_normal((n, 16))
    scale, bias = 0.6, 3.0
    whole = oracle.compress_head(q, k, scale, bias, tau)
    for r in range(whole["R"]):
        one = oracle.compress_block_row(q, k, scale, bias, r, tau)
        np.testing.assert_allclose(one["masses"], whole["masses"][r, : r + 1], rtol=1e-12, atol=1e-15)
        assert one["kept"] == whole["kept"][r]
        assert one["margin"] == pytest.approx(whole["margins"][r], rel=1e-9, abs=1e-12)
        np.testing.assert_array_equal(one["blocks"], whole["blocks"][r])
        rows = slice(64 * r, min(64 * (r + 1), n))
        np.testing.assert_allclose(one["m"], whole["m"][rows], rtol=1e-12)
        np.testing.assert_allclose(one["l"], whole["l"][rows], rtol=1e-12)


def test_block_row_uniform_closed_form():
    """Scale 0, no sink: every visible entry of row i is 1/(i+1), so an
    off-diagonal block of block-row r has mass 64 * sum_{i in r} 1/(i+1) and the
    diagonal block sum_{i in r} (i - 64r + 1)/(i+1)."""
    n, r = 320, 3
    q = np.ones((n, 8))
    k = np.ones((n, 8))
    one = oracle.compress_block_row(q, k, 0.0, 0.0, r, 1.0)
    i = np.arange(64 * r, 64 * (r + 1))
    off = 64 * np.sum(1.0 / (i + 1))
    diag = np.sum((i - 64 * r + 1) / (i + 1))
    np.testing.assert_allclose(one["masses"][:r], off, rtol=1e-13)
    np.testing.assert_allclose(one["masses"][r], diag, rtol=1e-13)
    assert one["kept"] == list(range(r + 1))


@pytest.mark.parametrize("n,kb0,tau", [(300, 2, 0.9), (256, 3, 0.95), (70, 1, 1.0)])
def test_chunk_equals_rows_of_whole_prompt(n, kb0, tau):
    """A prefill chunk (the last n - 64 kb0 queries against all n keys) compresses to
    exactly the block-rows kb0 .. of the whole prompt's compression: the same
    masses, kept sets, blocks and row statistics (the map rows are the same rows of
    one causal softmax)."""
    rng = np.random.default_rng(n + kb0)
    q = rng.standard_normal((n, 16))
    k = rng.standard_normal((n, 16))
    whole = oracle.compress_head(q, k, 0.6, 3.0, tau)
    chunk = oracle.compress_head(q[64 * kb0:], k, 0.6, 3.0, tau)
    assert chunk["kb0"] == kb0 and chunk["R"] == whole["R"] - kb0
    for r in range(chunk["R"]):
        ra = kb0 + r
        np.testing.assert_allclose(chunk["masses"][r, : ra + 1], whole["masses"][ra, : ra + 1], rtol=1e-12,
                                   atol=1e-15)
        assert not chunk["masses"][r, ra + 1:].any()
        if whole["margins"][ra] > 1e-9:
            assert chunk["kept"][r] == whole["kept"][ra]
            np.testing.assert_allclose(chunk["blocks"][r], whole["blocks"][ra], rtol=2 ** -8, atol=0)
    np.testing.assert_allclose(chunk["m"], whole["m"][64 * kb0:], rtol=1e-12)
    np.testing.assert_allclose(chunk["l"], whole["l"][64 * kb0:], rtol=1e-12)
    with pytest.raises(ValueError):  # a chunk must start on a block boundary
        oracle.compress_head(q[64 * kb0 + 1:], k, 0.6, 3.0, tau)


def test_block_compress_layout_with_chunks():
    """Varlen layout with chunked sequences: row pointers, masses at offset
    r kb0 + r(r+1)/2 per sequence, and per-sequence results equal to compress_head."""
    rng = np.random.default_rng(3)
    lq, lk = [70, 128, 5], [198, 128, 69]
    H = 2
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    cu_k = np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((H, int(cu_q[-1]), 16))
    k = rng.standard_normal((H, int(cu_k[-1]), 16))
    scale, bias = np.array([0.5, 0.8]), np.array([2.0, 0.0])
    out = oracle.block_compress(q, k, scale, bias, cu_q, 0.85, cu_k=cu_k, used_k=lk)
    R = [(n + 63) // 64 for n in lq]
    kb = [(b - a) // 64 for a, b in zip(lq, lk)]
    assert out["nb_tot"] == sum(r * x + r * (r + 1) // 2 for r, x in zip(R, kb))
    g = 0
    for h in range(H):
        off = 0
        for s in range(3):
            res = oracle.compress_head(q[h, cu_q[s]: cu_q[s + 1]], k[h, cu_k[s]: cu_k[s + 1]], scale[h], bias[h], 0.85)
            for r in range(R[s]):
                o = off + r * kb[s] + r * (r + 1) // 2
                assert np.array_equal(out["masses"][h, o: o + kb[s] + r + 1], res["masses"][r, : kb[s] + r + 1])
                assert out["kept"][g] == res["kept"][r]
                assert list(out["col_idx"][out["row_ptr"][g]: out["row_ptr"][g + 1]]) == res["kept"][r]
                g += 1
            off += R[s] * kb[s] + R[s] * (R[s] + 1) // 2
    assert g == H * sum(R)
