"""Block-sparse compression of causal maps (test infrastructure only).

MapFlow article, storage-and-execution section: because attention mass is not
spread evenly, regions are kept by importance -- cumulative attention
probability -- and the map is stored in a block-sparse format of regular 2-D
blocks; compression runs in two phases, block-level statistics first and then
extraction of the kept blocks, without first producing the dense map.

The oracle computes the exact dense map in float64 (it is the definition, not a
fast path) and applies the two phases to it.

Readings (the page gives no numbers or tie rules):
* blocks are 64 x 64, laid out per sequence from its first token; block (r, c)
  exists for c <= r; an edge block of a sequence whose length is not a multiple
  of 64 is zero-padded;
* the statistic of a block is its probability mass, the sum of the exact
  (unrounded) map over the block;
* per block-row, masses are normalised by their sum (the number of rows in the
  block-row, up to rounding), ordered largest first with ties to the lower
  column, and the shortest prefix whose running sum (in that order) reaches
  tau is kept; tau >= 1 keeps every causal block; kept probabilities are not
  renormalised;
* kept blocks are stored as bf16 (round to nearest even) in row-major 64 x 64
  order, zeros above the diagonal; block order is head, then sequence, then
  block-row, then column ascending.
"""
import math

import numpy as np

from .attention import causal_map, seq_lengths
from .numerics import round_bf16

BLOCK = 64


def block_masses(A, block=BLOCK):
    """Lower-triangular block masses ``[R, R]`` of a square causal map ``A`` (float64)."""
    n = A.shape[0]
    R = (n + block - 1) // block
    pad = R * block - n
    Ap = np.pad(np.asarray(A, dtype=np.float64), ((0, pad), (0, pad)))
    m = Ap.reshape(R, block, R, block).sum(axis=(1, 3))
    return np.tril(m)


def _sorted_weights(mass_row):
    w = np.asarray(mass_row, dtype=np.float64)
    w = w / w.sum()
    order = sorted(range(len(w)), key=lambda c: (-w[c], c))
    return w, order


def select_blocks(mass_row, tau):
    """Kept columns (ascending) of one block-row given its masses ``mass_row[0..r]``."""
    n = len(mass_row)
    if tau >= 1.0:
        return list(range(n))
    w, order = _sorted_weights(mass_row)
    kept, cum = [], 0.0
    for c in order:
        kept.append(c)
        cum += w[c]
        if cum >= tau:
            break
    return sorted(kept)


def selection_margin(mass_row, tau):
    """Distance of one block-row's selection from flipping, in normalised-mass units.

    The smallest of: the gap between the last kept and first dropped weight, the
    overshoot of the kept running sum above tau, and how far the running sum one
    block earlier stays below tau. +inf when tau >= 1 (nothing is decided).
    """
    n = len(mass_row)
    if tau >= 1.0:
        return math.inf
    w, order = _sorted_weights(mass_row)
    cum, prev, k = 0.0, 0.0, 0
    for c in order:
        prev = cum
        cum += w[c]
        k += 1
        if cum >= tau:
            break
    gap = w[order[k - 1]] - w[order[k]] if k < n else math.inf
    return min(gap, cum - tau, tau - prev)


def row_stats(q, k, scale, bias):
    """(m_i, l_i): row maximum of the logits and sum of exp(logit - m_i) (natural units).

    Query row i sits at key position nk - nq + i (bottom-right alignment) and sees
    keys 0 .. nk - nq + i.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    if nq == 0:  # an empty sequence has no rows
        return np.zeros(0), np.zeros(0)
    s = float(scale) * (q @ k.T)
    s[:, 0] += float(bias)
    vis = np.arange(nk)[None, :] <= (nk - nq + np.arange(nq))[:, None]
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    l = np.exp(s - m[:, None]).sum(axis=1)
    return m, l


def compress_head(q, k, scale, bias, tau, block=BLOCK):
    """Both phases for one head and one sequence.

    The sequence has nk = len(k) keys and nq = len(q) <= nk query rows, the last
    nq positions (a prefill chunk at the end of its context; nq = nk for a whole
    prompt). The block grid starts at the sequence's first token, so nk - nq must
    be a multiple of the block size: block-row r of the chunk is block-row
    kb0 + r of the sequence (kb0 = (nk - nq) / 64) and has blocks c = 0 .. kb0 + r.

    Returns dict with ``masses`` [R, C] (R = ceil(nq / 64) block-rows, C = ceil(nk
    / 64) block columns; row r is meaningful up to column kb0 + r, zero after),
    ``kept`` (list of column lists), ``margins`` [R], ``blocks`` (list over rows of
    float64 bf16-rounded ``[k_r, 64, 64]`` arrays), ``m``, ``l`` row statistics and
    ``kb0``.
    """
    A = causal_map(q, k, scale, bias)
    nq, nk = A.shape
    if (nk - nq) % block:
        raise ValueError("a query chunk must start on a block boundary of its sequence")
    kb0 = (nk - nq) // block
    R = (nq + block - 1) // block
    C = (nk + block - 1) // block
    Ap = np.pad(A, ((0, R * block - nq), (0, C * block - nk)))
    masses = Ap.reshape(R, block, C, block).sum(axis=(1, 3))
    kept, margins, blocks = [], np.zeros(R), []
    for r in range(R):
        row = masses[r, : kb0 + r + 1]
        cols = select_blocks(row, tau)
        kept.append(cols)
        margins[r] = selection_margin(row, tau)
        if cols:
            b = np.stack([Ap[r * block:(r + 1) * block, c * block:(c + 1) * block] for c in cols])
            blocks.append(round_bf16(b))
        else:
            blocks.append(np.zeros((0, block, block)))
    m, l = row_stats(q, k, scale, bias)
    return dict(masses=masses, kept=kept, margins=margins, blocks=blocks, m=m, l=l, n=nq, R=R, kb0=kb0)


def compress_block_row(q, k, scale, bias, r, tau, block=BLOCK):
    """Both phases for block-row ``r`` of one head and one sequence, for sampled
    checks of long sequences: the map rows of the block-row are the exact causal
    softmax of those queries against keys ``0 .. 64 r + 63`` (so the same rows as
    ``compress_head``'s map, without forming the rest of it).

    Returns dict with ``masses`` [r + 1], ``kept`` (ascending columns), ``margin``,
    ``blocks`` (float64 bf16-rounded ``[k, 64, 64]``, zero above the diagonal and
    past the sequence), ``rows`` (the exact float64 map rows of the block-row,
    ``[64, 64 (r + 1)]``, zero-padded likewise) and the row statistics ``m``, ``l``
    of the block-row's queries (natural units).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n = q.shape[0]
    i0, i1 = r * block, min((r + 1) * block, n)
    kend = i1  # keys 0 .. i1 - 1 are visible to some query of the block-row
    A = causal_map(q[i0:i1], k[:kend], scale, bias)  # [i1 - i0, kend]; bottom-right alignment
    rows = np.zeros((block, (r + 1) * block))
    rows[: i1 - i0, :kend] = A
    masses = rows.reshape(block, r + 1, block).sum(axis=(0, 2))
    cols = select_blocks(masses, tau)
    margin = selection_margin(masses, tau)
    blocks = (round_bf16(np.stack([rows[:, c * block:(c + 1) * block] for c in cols]))
              if cols else np.zeros((0, block, block)))
    s = float(scale) * (q[i0:i1] @ k[:kend].T)
    s[:, 0] += float(bias)
    vis = np.arange(kend)[None, :] <= np.arange(i0, i1)[:, None]
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    l = np.exp(s - m[:, None]).sum(axis=1)
    return dict(masses=masses, kept=cols, margin=margin, blocks=blocks, rows=rows, m=m, l=l)


def block_compress(q, k, scale, bias, cu, tau, used=None, block=BLOCK, heads=None,
                   keep_values=True, cu_k=None, used_k=None):
    """Whole compression over heads and packed sequences, in the library's layout.

    Sequence s uses query rows ``cu[s] ..`` and key rows ``cu_k[s] ..`` (``cu_k``
    defaults to ``cu``), ``used[s]`` queries (default: the ``cu`` spacing) and
    ``used_k[s]`` keys (default: as many as queries); with more keys than queries
    the queries are a chunk at the end of the sequence (``compress_head``).

    Returns dict with:
    * ``row_ptr`` [H * R_tot + 1] int64, ``col_idx`` [nnz], ``vals`` [nnz, 64, 64]
      float64 (bf16-rounded) when ``keep_values``;
    * ``masses`` [H, NB_tot]: per sequence, block-row r's kb0 + r + 1 masses at
      offset_s + r kb0 + r(r+1)/2 (lower-triangular for whole prompts),
      ``row_stats`` [H, T, 2] (m, l) at each query row;
    * ``margins`` [H * R_tot] selection margins; ``kept`` flat list of column lists.
    """
    lens = seq_lengths(cu, used)
    lens_k = list(lens) if used_k is None else [int(x) for x in used_k]
    cu = np.asarray(cu, dtype=np.int64)
    cu_k = cu if cu_k is None else np.asarray(cu_k, dtype=np.int64)
    hs = list(range(q.shape[0])) if heads is None else list(heads)
    bias = np.zeros(q.shape[0]) if bias is None else bias
    Rs = [(n + block - 1) // block for n in lens]
    kb0s = [(nk - n) // block for n, nk in zip(lens, lens_k)]
    r_tot = sum(Rs)
    nb_tot = sum(R * kb + R * (R + 1) // 2 for R, kb in zip(Rs, kb0s))
    T = int(q.shape[1])
    masses = np.zeros((len(hs), nb_tot))
    stats = np.zeros((len(hs), T, 2))
    counts, kept_all, margins, vals = [], [], [], []
    for hi, h in enumerate(hs):
        off = 0
        for s, n in enumerate(lens):
            qs = q[h, cu[s]: cu[s] + n]
            ks = k[h, cu_k[s]: cu_k[s] + lens_k[s]]
            res = compress_head(qs, ks, scale[h], bias[h], tau, block)
            R, kb = Rs[s], kb0s[s]
            for r in range(R):
                o = off + r * kb + r * (r + 1) // 2
                masses[hi, o: o + kb + r + 1] = res["masses"][r, : kb + r + 1]
                counts.append(len(res["kept"][r]))
                kept_all.append(res["kept"][r])
                margins.append(res["margins"][r])
                if keep_values and len(res["kept"][r]):
                    vals.append(res["blocks"][r])
            off += R * kb + R * (R + 1) // 2
            stats[hi, cu[s]: cu[s] + n, 0] = res["m"]
            stats[hi, cu[s]: cu[s] + n, 1] = res["l"]
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.array([c for cols in kept_all for c in cols], dtype=np.int64)
    out = dict(row_ptr=row_ptr, col_idx=col_idx, masses=masses, row_stats=stats,
               margins=np.array(margins), kept=kept_all, r_tot=r_tot, nb_tot=nb_tot,
               lengths=lens, lengths_k=lens_k, nnz=int(row_ptr[-1]))
    if keep_values:
        out["vals"] = np.concatenate(vals) if vals else np.zeros((0, block, block))
    return out
