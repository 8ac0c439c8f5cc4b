"""The pins catch plausible mistakes: each test plants one in a copy of an oracle
function (on the CPU) and checks that a pin that passes on the real oracle fails."""
import numpy as np
import pytest

import oracle
from tests import test_oracle_attention as ta
from tests import test_oracle_compress as tc
from tests import test_oracle_cosine as tcos


def _mutant_map(kind):
    def causal_map(q, k, scale, bias=0.0):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        nq, nk = q.shape[0], k.shape[0]
        s = float(scale) * ((k @ q.T).T if kind != "transposed" else (k @ q.T))
        if kind == "bias_last":
            s[:, -1] += float(bias)
        elif kind != "no_bias":
            s[:, 0] += float(bias)
        pos = (nk - nq) + np.arange(nq)
        if kind == "strict_mask":
            vis = np.arange(nk)[None, :] < np.maximum(pos[:, None], 1)
        elif kind == "top_left":
            vis = np.arange(nk)[None, :] <= np.arange(nq)[:, None]
        else:
            vis = np.arange(nk)[None, :] <= pos[:, None]
        s = np.where(vis, s, -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        return e / e.sum(axis=1, keepdims=True)
    return causal_map


@pytest.mark.parametrize("kind,pin", [
    ("bias_last", lambda: ta.test_scale_zero_with_sink(4.0)),
    ("no_bias", lambda: ta.test_brute_force_tiny(1, 16, 16, 0.9, 4.0)),
    ("strict_mask", lambda: ta.test_scale_zero_is_uniform_over_prefix()),
    ("transposed", lambda: ta.test_brute_force_tiny(0, 7, 7, 0.35, 0.0)),
    ("top_left", lambda: ta.test_decode_row_is_last_row_of_extended_prefill()),
])
def test_attention_mutants_are_caught(monkeypatch, kind, pin):
    monkeypatch.setattr(oracle, "causal_map", _mutant_map(kind))
    with pytest.raises(AssertionError):
        pin()


def test_selection_tie_mutant_is_caught(monkeypatch):
    def select_high_tie(mass_row, tau):
        w = np.asarray(mass_row, dtype=np.float64)
        w = w / w.sum()
        order = sorted(range(len(w)), key=lambda c: (-w[c], -c))
        kept, cum = [], 0.0
        for c in order:
            kept.append(c)
            cum += w[c]
            if cum >= tau:
                break
        return sorted(kept)
    monkeypatch.setattr(oracle, "select_blocks", select_high_tie)
    with pytest.raises(AssertionError):
        tc.test_selection_edge_cases()


def test_selection_strict_threshold_mutant_is_caught(monkeypatch):
    def select_keep_one_more(mass_row, tau):
        if tau >= 1.0:
            return list(range(len(mass_row)))
        w = np.asarray(mass_row, dtype=np.float64) / np.sum(mass_row)
        order = sorted(range(len(w)), key=lambda c: (-w[c], c))
        kept, cum = [], 0.0
        for c in order:
            if cum >= tau:
                break
            kept.append(c)
            cum += w[c]
        return sorted(kept + ([order[len(kept)]] if len(kept) < len(w) else []))
    monkeypatch.setattr(oracle, "select_blocks", select_keep_one_more)
    with pytest.raises(AssertionError):
        for seed in range(12):
            tc.test_greedy_matches_subset_enumeration(seed)


def test_cosine_without_sqrt_is_caught(monkeypatch):
    def cos_nosqrt(recv, send):
        r = np.asarray(recv, dtype=np.float64)
        s = np.asarray(send, dtype=np.float64)
        return (r @ s.T) / ((r * r).sum(1)[:, None] * (s * s).sum(1)[None, :])
    monkeypatch.setattr(oracle, "cosine_matrix", cos_nosqrt)
    with pytest.raises(AssertionError):
        tcos.test_closed_forms_at_512()
