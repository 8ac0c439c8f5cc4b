"""Head mapping by cosine similarity of flattened maps (test infrastructure only).

IAM Method 1: the small and the large model's attention matrices are flattened
into vectors and compared; cosine similarity works best. IAM Method 4: at
prefill, every head of every mapped layer of the large model is paired with the
most similar head among all of the small model's maps.

Readings: the cosine is taken over the stored (rounded) maps; the flattened
vector holds the causal entries only (the zeros above the diagonal add nothing to
either dot products or norms, so the value is the same as over the full square);
ties in the argmax go to the lowest sender index; the decision margin is the gap
between the best and second-best cosine (+inf with a single sender). A zero
vector has cosine 0 with everything.
"""
import numpy as np


def cosine_matrix(recv, send):
    """cos[h, j] = <r_h, s_j> / (|r_h| |s_j|) in float64. ``recv`` [Hr, L], ``send`` [Hs, L]."""
    r = np.asarray(recv, dtype=np.float64)
    s = np.asarray(send, dtype=np.float64)
    dots = r @ s.T
    nr = np.sqrt((r * r).sum(axis=1))
    ns = np.sqrt((s * s).sum(axis=1))
    den = nr[:, None] * ns[None, :]
    with np.errstate(invalid="ignore", divide="ignore"):
        cos = np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
    return cos


def head_map(recv, send):
    """(cos [Hr, Hs], argmax [Hr] int, margin [Hr]) for one mapping problem."""
    cos = cosine_matrix(recv, send)
    arg = np.argmax(cos, axis=1)  # first index of the maximum: lowest index wins ties
    if cos.shape[1] > 1:
        srt = np.sort(cos, axis=1)
        margin = srt[:, -1] - srt[:, -2]
    else:
        margin = np.full(cos.shape[0], np.inf)
    return cos, arg.astype(np.int64), margin
