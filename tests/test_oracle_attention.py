"""Pins for the oracle's causal maps and storage rounding (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import brute


def rand_qk(seed, nq, nk, d):
    r = np.random.default_rng(seed)
    return r.standard_normal((nq, d)), r.standard_normal((nk, d))


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("n", [1, 5, 64, 130])
def test_rows_sum_to_one_and_causal(n):
    q, k = rand_qk(n, n, n, 16)
    A = oracle.causal_map(q, k, 0.7, 2.0)
    assert np.allclose(A.sum(axis=1), 1.0, atol=1e-13)
    assert (A >= 0).all()
    assert np.all(A[np.triu_indices(n, 1)] == 0.0)
    assert A[0, 0] == 1.0


# ---------------------------------------------------------------- closed forms
def test_scale_zero_is_uniform_over_prefix():
    n = 200
    q, k = rand_qk(1, n, n, 8)
    A = oracle.causal_map(q, k, 0.0, 0.0)
    i, j = np.tril_indices(n)
    assert np.allclose(A[i, j], 1.0 / (i + 1), rtol=1e-14)


@pytest.mark.parametrize("b", [4.0, -3.0])
def test_scale_zero_with_sink(b):
    n = 100
    q, k = rand_qk(2, n, n, 8)
    A = oracle.causal_map(q, k, 0.0, b)
    eb = math.exp(b)
    i = np.arange(n)
    assert np.allclose(A[:, 0], eb / (eb + i), rtol=1e-13)
    for r in range(1, n):
        assert np.allclose(A[r, 1: r + 1], 1.0 / (eb + r), rtol=1e-13)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed,nq,nk,scale,bias", [
    (0, 7, 7, 0.35, 0.0), (1, 16, 16, 0.9, 4.0), (2, 3, 11, 0.5, 4.0), (3, 1, 9, 1.3, -1.0),
])
def test_brute_force_tiny(seed, nq, nk, scale, bias):
    q, k = rand_qk(seed, nq, nk, 6)
    A = oracle.causal_map(q, k, scale, bias)
    B = np.array(brute.causal_map(q.tolist(), k.tolist(), scale, bias))
    assert np.allclose(A, B, rtol=1e-12, atol=1e-15)


def test_decode_row_is_last_row_of_extended_prefill():
    q, k = rand_qk(5, 40, 40, 12)
    full = oracle.causal_map(q, k, 0.4, 4.0)
    for t in [0, 17, 39]:
        row = oracle.causal_map(q[t: t + 1], k[: t + 1], 0.4, 4.0)
        assert np.allclose(row[0], full[t, : t + 1], rtol=1e-13, atol=1e-16)


def test_varlen_is_concatenation():
    r = np.random.default_rng(3)
    lens = [5, 64, 17]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, d = 3, 8
    q = r.standard_normal((H, cu[-1], d))
    k = r.standard_normal((H, cu[-1], d))
    scale = np.array([0.3, 0.5, 1.0])
    bias = np.array([0.0, 4.0, 0.0])
    maps = oracle.attn_maps(q, k, scale, bias, cu, cu)
    for h in range(H):
        for s in range(len(lens)):
            sl = slice(cu[s], cu[s + 1])
            assert np.array_equal(maps[h][s], oracle.causal_map(q[h, sl], k[h, sl], scale[h], bias[h]))


def test_empty_sequences_in_batch():
    """A sequence with no query rows has an empty map (0 rows, its key count wide),
    packs to nothing and leaves the other sequences' maps unchanged."""
    r = np.random.default_rng(4)
    lq, lk = [5, 0, 0, 9], [5, 0, 4, 12]
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    q = r.standard_normal((2, cq[-1], 8))
    k = r.standard_normal((2, ck[-1], 8))
    scale, bias = np.array([0.5, 1.0]), np.array([4.0, 0.0])
    maps = oracle.attn_maps(q, k, scale, bias, cq, ck)
    for h in range(2):
        assert maps[h][1].shape == (0, 0) and maps[h][2].shape == (0, 4)
        assert oracle.pack_rows(maps[h][2]).size == 0 == oracle.packed_size(0, 4)
        for s in (0, 3):
            want = oracle.causal_map(q[h, cq[s]:cq[s + 1]], k[h, ck[s]:ck[s + 1]], scale[h], bias[h])
            assert np.array_equal(maps[h][s], want)
            assert np.allclose(want.sum(axis=1), 1.0, rtol=0, atol=1e-13)


def test_identity_against_torch_sdpa():
    """Library special case: map @ V equals torch's scaled_dot_product_attention (float64, CPU)."""
    r = np.random.default_rng(11)
    n, d, scale, b = 50, 16, 0.3, 4.0
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    A = oracle.causal_map(q, k, scale, b)
    mask = torch.zeros(n, n, dtype=torch.float64)
    mask[torch.ones(n, n, dtype=torch.bool).triu(1)] = float("-inf")
    mask[:, 0] += b
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None], torch.tensor(k)[None, None], torch.tensor(v)[None, None],
        attn_mask=mask[None, None], scale=scale)[0, 0].numpy()
    assert np.allclose(A @ v, ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- packing
def test_packed_layout_indices():
    q, k = rand_qk(8, 9, 9, 4)
    A = oracle.causal_map(q, k, 0.5)
    p = oracle.pack_rows(A)
    assert len(p) == oracle.packed_size(9, 9) == 45
    for i in range(9):
        for j in range(i + 1):
            assert p[i * (i + 1) // 2 + j] == A[i, j]
    # bottom-right rows: row i starts at i*(nk-nq) + i(i+1)/2
    q, k = rand_qk(9, 3, 10, 4)
    A = oracle.causal_map(q, k, 0.5)
    p = oracle.pack_rows(A)
    assert len(p) == oracle.packed_size(3, 10) == 3 * 7 + 6
    for i in range(3):
        start = i * 7 + i * (i + 1) // 2
        assert np.array_equal(p[start: start + 7 + i + 1], A[i, : 8 + i])


# ---------------------------------------------------------------- rounding
def test_round_bf16_matches_torch_on_float32_values():
    """Library special case: for float32 inputs torch's bf16 cast is round-to-nearest-even."""
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-30, 30, 20000),
                        r.uniform(0, 1, 20000)]).astype(np.float32)
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_and_no_double_rounding():
    one = 1.0
    assert oracle.round_bf16(one + 2.0 ** -8) == 1.0                       # tie -> even
    assert oracle.round_bf16(one + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6         # tie -> even (up)
    assert oracle.round_bf16(one + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7  # above the tie
    assert oracle.round_bf16(2.0 ** -130) == 2.0 ** -130                    # bf16 subnormal
    assert oracle.round_bf16(0.0) == 0.0
    assert oracle.round_bf16(-(one + 2.0 ** -7)) == -(one + 2.0 ** -7)
