"""Mapped attention times the receiver's V (test infrastructure only).

MapFlow article, approach section: a receiver layer that reuses the sender's
maps forms each of its heads' maps as a learned linear combination of the
sender's head maps, then applies them to its own value vectors.
Storage-and-execution section: the fused kernel reads the sparse blocks, mixes
the heads and multiplies by V without rebuilding the receiver's dense map.
IAM Method 4 (decode): a mapped layer takes the small model's attention row for
the new token directly; with a one-hot mixing matrix this is the same
operation on a single row.

Definition: O_h = (sum_j M[h, j] * A_j) @ V_h in float64, where A_j is sender
map j as stored (the dense map, or its block-sparse form with zeros off the kept
blocks). Readings: M may differ per sequence; the receiver has one V per head;
kept probabilities are used as stored (no renormalisation).
"""
import numpy as np


def mix_maps(maps, M):
    """B[h] = sum_j M[h, j] * maps[j]; ``maps`` [Hs, nq, nk], ``M`` [Hr, Hs] -> [Hr, nq, nk]."""
    maps = np.asarray(maps, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    out = np.zeros((M.shape[0],) + maps.shape[1:])
    for h in range(M.shape[0]):
        for j in range(M.shape[1]):
            out[h] += M[h, j] * maps[j]
    return out


def mapped_av_dense(maps, M, V):
    """One sequence: ``maps`` [Hs, nq, nk], ``M`` [Hr, Hs], ``V`` [Hr, nk, d] -> O [Hr, nq, d]."""
    B = mix_maps(maps, M)
    V = np.asarray(V, dtype=np.float64)
    return np.stack([B[h] @ V[h] for h in range(B.shape[0])])


def dense_from_bsr_rows(row_ptr, col_idx, vals, g, n, r, block=64, row_end=None):
    """Rows ``r*64 .. r*64+63`` (all ``n`` key columns) of one map from block-row ``g``
    of a BSR; the row's blocks are ``row_ptr[g] .. row_end[g]`` (``row_end``
    defaults to ``row_ptr[g + 1]``)."""
    R = (n + block - 1) // block
    out = np.zeros((block, R * block))
    end = int(row_ptr[g + 1]) if row_end is None else int(row_end[g])
    for t in range(int(row_ptr[g]), end):
        c = int(col_idx[t])
        out[:, c * block:(c + 1) * block] = vals[t]
    return out[:, :n]


def mapped_av_bsr_rows(row_ptr, col_idx, vals, n_send, lengths, M, V, cu_k, rows, block=64,
                       lengths_k=None, row_end=None):
    """O rows of a block-sparse mapped pass, computed one block-row at a time.

    ``lengths`` per sequence (query rows), ``lengths_k`` its keys (default: the
    same; more keys than queries: the queries are a chunk at the end of the
    sequence and their block-rows see key blocks up to kb0 + r); ``M`` [S or 1,
    Hr, Hs]; ``V`` [Hr, Tk, d] with sequence s at key rows ``cu_k[s] ..``; ``rows``
    is a list of (sequence, block-row) pairs. Returns {(s, r): O [Hr,
    rows_in_block, d]}. The block-sparse arrays are indexed as head-major, then
    sequence, then block-row; ``row_end`` (optional) gives each block-row's end
    when the rows are not stored back to back.
    """
    lengths_k = list(lengths) if lengths_k is None else list(lengths_k)
    Rs = [(n + block - 1) // block for n in lengths]
    r_tot = sum(Rs)
    roff = np.concatenate([[0], np.cumsum(Rs)]).astype(np.int64)
    M = np.asarray(M, dtype=np.float64)
    out = {}
    for (s, r) in rows:
        n, nk = lengths[s], lengths_k[s]
        nr = min(block, n - r * block)
        Ms = M[s] if M.shape[0] > 1 else M[0]
        maps = np.stack([dense_from_bsr_rows(row_ptr, col_idx, vals, j * r_tot + roff[s] + r, nk, r, block,
                                             row_end)[:nr] for j in range(n_send)])
        Vs = np.asarray(V[:, cu_k[s]: cu_k[s] + nk], dtype=np.float64)
        out[(s, r)] = mapped_av_dense(maps, Ms, Vs)
    return out
