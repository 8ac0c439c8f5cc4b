"""Host-side mapping decisions (test infrastructure only).

IAM Method 2: on the 80-layer model the layers that tolerate mapping best are
the last two 8-layer sub-blocks (64-80) and sub-blocks 2-4 (16-40); the first two
sub-blocks (0-16) must not be mapped. For a requested ratio, layers are taken
from the last layer backwards down to layer 64, and if more are needed, from
layer 16 upwards.

Readings: layers are 0-indexed; the number mapped is round-half-up(ratio * L);
for a depth other than 80 the cut points scale with depth (0.8 L and 0.2 L,
rounded half up); the forward run continues up to 0.8 L - 1 and the first 0.2 L
layers are never mapped (more layers than that are not available).

IAM Method 4: the head map fixed at prefill is a per-head argmax over sender
heads; as a mixing matrix it is one-hot. Its thresholds: a prompt shorter than
tau_e is first extended by ordinary generation to tau_e tokens, and only then is
the mapping built; for a context longer than tau_t the similarity is computed on
a truncated context. Readings: the generated tokens belong to the context the
maps are taken over, and truncation keeps the first tau_t tokens.
"""
import math

import numpy as np


def _half_up(x):
    return int(math.floor(x + 0.5))


def mapped_layers(n_layers, ratio):
    """Mapped receiver layers in priority order (first ``round(ratio * L)`` of the order)."""
    hi = _half_up(0.8 * n_layers)
    lo = _half_up(0.2 * n_layers)
    order = list(range(n_layers - 1, hi - 1, -1)) + list(range(lo, hi))
    return order[: max(0, min(_half_up(ratio * n_layers), len(order)))]


def onehot_mix(argmax, n_send):
    """One-hot mixing matrix from head-map indices: ``argmax`` [B, Hr] -> M [B, Hr, Hs]."""
    a = np.asarray(argmax)
    M = np.zeros(a.shape + (n_send,), dtype=np.float64)
    np.put_along_axis(M, a[..., None], 1.0, axis=-1)
    return M


def mapping_plan(prompt_len, tau_e, tau_t):
    """IAM Method 4 thresholds for one request: (tokens generated before the head
    map is built, number of leading context tokens the similarity uses)."""
    if prompt_len < 0 or tau_e < 0 or tau_t < 1:
        raise ValueError("bad lengths")
    gen = tau_e - prompt_len if prompt_len < tau_e else 0
    context = prompt_len + gen
    return gen, (context if context <= tau_t else tau_t)
