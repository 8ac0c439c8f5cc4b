"""Pins for the oracle's mapped x V pass and mapping helpers (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sender_maps(seed, hs, n, d=8, biases=None):
    r = np.random.default_rng(seed)
    q = r.standard_normal((hs, n, d))
    k = r.standard_normal((hs, n, d))
    biases = biases if biases is not None else [4.0 * (j % 2) for j in range(hs)]
    return q, k, np.stack([oracle.causal_map(q[j], k[j], 0.9, biases[j]) for j in range(hs)])


def test_identity_mixing_is_ordinary_attention_torch_sdpa():
    """Library special case: identity M reproduces causal attention (torch SDPA, float64, CPU)."""
    hs, n, d = 3, 40, 8
    q, k, maps = sender_maps(0, hs, n, d, biases=[4.0, 0.0, 4.0])
    v = np.random.default_rng(1).standard_normal((hs, n, 16))
    O = oracle.mapped_av_dense(maps, np.eye(hs), v)
    for j, b in enumerate([4.0, 0.0, 4.0]):
        mask = torch.zeros(n, n, dtype=torch.float64)
        mask[torch.ones(n, n, dtype=torch.bool).triu(1)] = float("-inf")
        mask[:, 0] += b
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[j])[None], torch.tensor(k[j])[None], torch.tensor(v[j])[None],
            attn_mask=mask[None], scale=0.9)[0].numpy()
        assert np.allclose(O[j], ref, rtol=1e-11, atol=1e-12)


def test_brute_force_tiny():
    _, _, maps = sender_maps(2, 3, 6, 4)
    r = np.random.default_rng(3)
    M = r.normal(0, 0.5, (2, 3))
    V = r.standard_normal((2, 6, 3))
    O = oracle.mapped_av_dense(maps, M, V)
    B = np.array(brute.mapped_av(maps.tolist(), M.tolist(), V.tolist()))
    assert np.allclose(O, B, rtol=1e-12, atol=1e-14)


def test_linear_in_M_onehot_and_row0():
    hs, hr, n = 4, 3, 30
    _, _, maps = sender_maps(4, hs, n)
    r = np.random.default_rng(5)
    V = r.standard_normal((hr, n, 8))
    M1, M2 = r.normal(size=(hr, hs)), r.normal(size=(hr, hs))
    O1 = oracle.mapped_av_dense(maps, M1, V)
    O2 = oracle.mapped_av_dense(maps, M2, V)
    assert np.allclose(oracle.mapped_av_dense(maps, 2.0 * M1 - 3.0 * M2, V), 2.0 * O1 - 3.0 * O2, atol=1e-12)
    pi = [2, 0, 3]
    Oh = oracle.mapped_av_dense(maps, oracle.onehot_mix(np.array(pi), hs), V)
    for h in range(hr):
        assert np.allclose(Oh[h], maps[pi[h]] @ V[h], atol=1e-14)
    # row 0 only sees key 0 with probability 1 in every sender map
    assert np.allclose(O1[:, 0], M1.sum(axis=1)[:, None] * V[:, 0], atol=1e-13)


def test_stochastic_mixing_keeps_rows_normalised():
    _, _, maps = sender_maps(6, 4, 25)
    M = np.random.default_rng(7).uniform(0, 1, (5, 4))
    M /= M.sum(axis=1, keepdims=True)
    B = oracle.mix_maps(maps, M)
    assert np.allclose(B.sum(axis=2), 1.0, atol=1e-13)
    assert (B >= 0).all()


def test_full_retention_bsr_equals_dense():
    """tau >= 1 keeps every causal block: the sparse pass equals the dense pass on rounded maps."""
    r = np.random.default_rng(8)
    lens = [130, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    hs, hr = 3, 2
    q = r.standard_normal((hs, cu[-1], 8))
    k = r.standard_normal((hs, cu[-1], 8))
    scale, bias = np.full(hs, 0.8), np.array([4.0, 0.0, 0.0])
    bsr = oracle.block_compress(q, k, scale, bias, cu, 1.0)
    M = r.normal(size=(1, hr, hs))
    V = r.standard_normal((hr, cu[-1], 8))
    rows = [(s, rr) for s in range(2) for rr in range((lens[s] + 63) // 64)]
    out = oracle.mapped_av_bsr_rows(bsr["row_ptr"], bsr["col_idx"], bsr["vals"], hs, lens, M, V, cu, rows)
    for s, n in enumerate(lens):
        maps = np.stack([oracle.round_bf16(oracle.causal_map(q[j, cu[s]:cu[s + 1]], k[j, cu[s]:cu[s + 1]],
                                                              scale[j], bias[j])) for j in range(hs)])
        dense = oracle.mapped_av_dense(maps, M[0], V[:, cu[s]:cu[s + 1]])
        got = np.concatenate([out[(s, rr)] for rr in range((n + 63) // 64)], axis=1)
        assert np.allclose(got, dense, rtol=1e-12, atol=1e-13)


def test_dropped_blocks_are_zero_in_bsr_rows():
    r = np.random.default_rng(9)
    n, hs = 256, 2
    q = r.standard_normal((hs, n, 8))
    k = r.standard_normal((hs, n, 8))
    bsr = oracle.block_compress(q, k, np.full(hs, 2.0), np.zeros(hs), np.array([0, n]), 0.5)
    for g in range(hs * 4):
        rr = g % 4
        rows = oracle.dense_from_bsr_rows(bsr["row_ptr"], bsr["col_idx"], bsr["vals"], g, n, rr)
        kept = set(bsr["kept"][g])
        for c in range(4):
            blk = rows[:, 64 * c: 64 * c + 64]
            if c not in kept:
                assert not blk.any()


# ---------------------------------------------------------------- layer order
def test_iam_layer_order_golden():
    with open(os.path.join(GOLDEN, "iam_mapped_layers.json")) as f:
        g = json.load(f)
    assert oracle.mapped_layers(g["n_layers"], g["ratio"]) == g["layers"]


def test_layer_order_properties():
    assert oracle.mapped_layers(80, 0.2) == list(range(79, 63, -1))
    assert oracle.mapped_layers(80, 0.1) == list(range(79, 71, -1))
    full = oracle.mapped_layers(80, 1.0)
    assert len(full) == 64 and min(full) == 16 and len(set(full)) == 64
    assert oracle.mapped_layers(80, 0.0) == []
    assert oracle.mapped_layers(40, 0.5) == list(range(39, 31, -1)) + list(range(8, 20))


def test_chunk_rows_equal_whole_prompt_rows():
    """mapped_av over a chunk's block-rows (queries at the end of a longer key span)
    equals the same rows of the whole prompt's pass; a BSR whose rows are listed by
    (begin, end) pairs out of order gives the same result as the packed one."""
    rng = np.random.default_rng(11)
    n, kb0, Hs, Hr = 200, 2, 3, 2
    q = rng.standard_normal((Hs, n, 16))
    k = rng.standard_normal((Hs, n, 16))
    sc, bi = np.array([0.5, 0.7, 0.9]), np.zeros(Hs)
    whole = oracle.block_compress(q, k, sc, bi, np.array([0, n]), 0.9)
    chunk = oracle.block_compress(q[:, 64 * kb0:], k, sc, bi, np.array([0, n - 64 * kb0]), 0.9,
                                  cu_k=np.array([0, n]), used_k=[n])
    M = rng.standard_normal((1, Hr, Hs))
    V = rng.standard_normal((Hr, n, 8))
    R = (n + 63) // 64
    ow = oracle.mapped_av_bsr_rows(whole["row_ptr"], whole["col_idx"], whole["vals"], Hs, [n], M, V,
                                   np.array([0]), [(0, r) for r in range(R)])
    oc = oracle.mapped_av_bsr_rows(chunk["row_ptr"], chunk["col_idx"], chunk["vals"], Hs, [n - 64 * kb0], M, V,
                                   np.array([0]), [(0, r) for r in range(R - kb0)], lengths_k=[n])
    for r in range(R - kb0):
        if all(whole["margins"][j * R + kb0 + r] > 1e-9 for j in range(Hs)):
            np.testing.assert_allclose(oc[(0, r)], ow[(0, kb0 + r)], rtol=1e-12, atol=1e-12)
    # rows given by (begin, end), stored in reverse order
    rp = chunk["row_ptr"]
    order = list(range(len(rp) - 1))[::-1]
    beg, end, cols, vals = np.zeros(len(order), np.int64), np.zeros(len(order), np.int64), [], []
    pos = 0
    for g in order:
        a, b = int(rp[g]), int(rp[g + 1])
        beg[g], end[g] = pos, pos + b - a
        cols.extend(chunk["col_idx"][a:b])
        vals.append(chunk["vals"][a:b])
        pos += b - a
    ob = oracle.mapped_av_bsr_rows(np.append(beg, 0), np.array(cols), np.concatenate(vals), Hs, [n - 64 * kb0], M,
                                   V, np.array([0]), [(0, r) for r in range(R - kb0)], lengths_k=[n], row_end=end)
    for key in oc:
        assert np.array_equal(ob[key], oc[key])
