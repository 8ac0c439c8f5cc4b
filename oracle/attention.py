"""Causal attention probability maps (test infrastructure only).

Follows GLIDE sections II-A/II-B: a query at position i attends to every key at
position j <= i through a scaled dot product normalised by softmax. IAM Method 4
needs these maps explicitly (which is why it cannot use a fused flash kernel).

Readings (the pages are silent on these):
* logit s_ij = scale_h * <q_i, k_j> + bias_h * [j == 0]; scale_h = beta_h / sqrt(d)
  is given per head, and the optional per-head bias is added after scaling to the
  first key of every row (the "sink" of the synthetic workloads);
* a query block shorter than its key block sits at the end of it (bottom-right
  alignment): query row i of a sequence with nq queries and nk keys is key
  position nk - nq + i and sees keys 0 .. nk - nq + i (a decode row attends to
  the whole context including itself);
* sequences packed together are independent.
"""
import numpy as np


def seq_lengths(cu, used=None):
    """Per-sequence lengths: ``used[s]`` if given, else ``cu[s+1] - cu[s]``."""
    cu = np.asarray(cu, dtype=np.int64)
    if used is not None:
        return [int(x) for x in np.asarray(used)]
    return [int(cu[s + 1] - cu[s]) for s in range(len(cu) - 1)]


def causal_map(q, k, scale, bias=0.0):
    """Exact causal softmax map of one head and one sequence, float64 ``[nq, nk]``.

    ``q`` ``[nq, d]`` and ``k`` ``[nk, d]`` hold the stored input values.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    if nq > nk:
        raise ValueError("more queries than keys")
    if nq == 0:  # a sequence with no query rows has an empty map
        return np.zeros((0, nk))
    s = float(scale) * (q @ k.T)
    if nk > 0:
        s[:, 0] += float(bias)
    pos = (nk - nq) + np.arange(nq)
    visible = np.arange(nk)[None, :] <= pos[:, None]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def attn_maps(q, k, scale, bias, cu_q, cu_k, used_q=None, used_k=None, heads=None):
    """Maps of every (head, sequence): ``out[h][s]`` float64 ``[nq_s, nk_s]``.

    ``q`` ``[H, Tq, d]``, ``k`` ``[H, Tk, d]`` (float arrays of the stored values);
    sequence s uses query rows ``cu_q[s] .. cu_q[s] + nq_s`` and key rows
    ``cu_k[s] .. cu_k[s] + nk_s``.
    """
    lq = seq_lengths(cu_q, used_q)
    lk = seq_lengths(cu_k, used_k)
    hs = range(q.shape[0]) if heads is None else heads
    bias = np.zeros(q.shape[0]) if bias is None else bias
    out = []
    for h in hs:
        per = []
        for s in range(len(lq)):
            qs = q[h, cu_q[s]: cu_q[s] + lq[s]]
            ks = k[h, cu_k[s]: cu_k[s] + lk[s]]
            per.append(causal_map(qs, ks, scale[h], bias[h]))
        out.append(per)
    return out


def packed_size(nq, nk):
    """Number of visible entries of a causal map with bottom-right alignment."""
    return nq * (nk - nq) + nq * (nq + 1) // 2


def pack_rows(A):
    """Flatten the visible (causal) entries of a map row by row.

    Row i contributes its first nk - nq + i + 1 entries, so row i starts at
    i * (nk - nq) + i * (i + 1) / 2; for a square map that is i(i+1)/2 + j.
    """
    nq, nk = A.shape
    return np.concatenate([A[i, : nk - nq + i + 1] for i in range(nq)]) if nq else np.zeros(0)
