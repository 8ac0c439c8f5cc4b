"""Pins for the oracle's cosine head mapping (CPU only)."""
import math

import numpy as np
import pytest
from scipy.spatial import distance

import oracle
from tests import brute


def special_maps(n):
    """Uniform causal map U (A_ij = 1/(i+1)), identity I, and all-on-key-0 sink S."""
    U = np.tril(np.ones((n, n))) / (np.arange(n)[:, None] + 1.0)
    I = np.eye(n)
    S = np.zeros((n, n))
    S[:, 0] = 1.0
    return U, I, S


def test_closed_forms_at_512():
    n = 512
    U, I, S = special_maps(n)
    flat = lambda A: oracle.pack_rows(A)
    cos = oracle.cosine_matrix(np.stack([flat(U), flat(I)]), np.stack([flat(I), flat(S)]))
    Hn = sum(1.0 / t for t in range(1, n + 1))
    assert math.isclose(cos[0, 0], math.sqrt(Hn / n), rel_tol=1e-13)   # cos(U, I)
    assert math.isclose(cos[0, 1], math.sqrt(Hn / n), rel_tol=1e-13)   # cos(U, S)
    assert math.isclose(cos[1, 1], 1.0 / n, rel_tol=1e-13)             # cos(I, S)
    assert math.isclose(cos[1, 0], 1.0, rel_tol=1e-14)                  # cos(I, I)
    assert math.isclose(math.sqrt(Hn / n), 0.1153842, abs_tol=5e-8)


def test_against_scipy_cosine_distance():
    r = np.random.default_rng(0)
    R = r.uniform(0, 1, (5, 300))
    S = r.uniform(0, 1, (7, 300))
    cos = oracle.cosine_matrix(R, S)
    for h in range(5):
        for j in range(7):
            assert math.isclose(cos[h, j], 1.0 - distance.cosine(R[h], S[j]), rel_tol=1e-12)


def test_brute_force_and_properties():
    r = np.random.default_rng(1)
    R = r.uniform(0, 1, (3, 40))
    S = r.uniform(0, 1, (4, 40))
    cos = oracle.cosine_matrix(R, S)
    for h in range(3):
        for j in range(4):
            assert math.isclose(cos[h, j], brute.cosine(R[h].tolist(), S[j].tolist()), rel_tol=1e-12)
    assert np.allclose(np.diag(oracle.cosine_matrix(S, S)), 1.0, atol=1e-14)
    assert np.allclose(oracle.cosine_matrix(S, R), cos.T, atol=1e-15)
    assert np.allclose(oracle.cosine_matrix(3.0 * R, 0.25 * S), cos, atol=1e-15)
    assert (cos >= 0).all() and (cos <= 1 + 1e-15).all()


def test_argmax_permutation_ties_and_margin():
    r = np.random.default_rng(2)
    R = r.uniform(0, 1, (6, 50))
    S = r.uniform(0, 1, (5, 50))
    cos, arg, margin = oracle.head_map(R, S)
    perm = r.permutation(5)
    _, arg_p, margin_p = oracle.head_map(R, S[perm])
    assert np.array_equal(perm[arg_p], arg)
    assert np.allclose(margin_p, margin)
    srt = np.sort(cos, axis=1)
    assert np.allclose(margin, srt[:, -1] - srt[:, -2])
    # exact ties (integer-valued maps: every sum is exact) go to the lowest sender index
    a = np.array([[1.0, 2.0, 0.0, 1.0]])
    b, c = np.array([0.0, 1.0, 2.0, 0.0]), np.array([2.0, 4.0, 0.0, 2.0])
    _, arg_t, margin_t = oracle.head_map(a, np.stack([b, c, a[0], c]))
    assert arg_t[0] == 1 and margin_t[0] == 0.0
    _, arg_t, _ = oracle.head_map(a, np.stack([b, a[0], c]))
    assert arg_t[0] == 1
    # one sender gives margin +inf
    _, _, m1 = oracle.head_map(R, S[:1])
    assert np.isinf(m1).all()


def test_maps_from_attention_score_highest_on_themselves():
    """A receiver map identical to one sender map maps to it with cosine 1."""
    r = np.random.default_rng(4)
    n, d = 64, 8
    maps = [oracle.pack_rows(oracle.causal_map(r.standard_normal((n, d)), r.standard_normal((n, d)), 1.0, b))
            for b in (0.0, 4.0, 0.0)]
    cos, arg, _ = oracle.head_map(np.stack([maps[2], maps[0]]), np.stack(maps))
    assert list(arg) == [2, 0]
    assert math.isclose(cos[0, 2], 1.0, rel_tol=1e-14)
