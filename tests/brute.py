"""Pure-Python brute force for tiny shapes: loops and ``math`` only, no numpy.

Independent of the oracle's code; used to pin it. Every function restates the
definition element by element.
"""
import itertools
import math


def causal_map(q, k, scale, bias=0.0):
    """Softmax over keys j <= nk - nq + i of scale * q_i . k_j (+ bias on key 0)."""
    nq, nk = len(q), len(k)
    out = []
    for i in range(nq):
        last = nk - nq + i
        logits = []
        for j in range(last + 1):
            dot = 0.0
            for a, b in zip(q[i], k[j]):
                dot += a * b
            logits.append(scale * dot + (bias if j == 0 else 0.0))
        mx = max(logits)
        ex = [math.exp(x - mx) for x in logits]
        z = sum(ex)
        out.append([e / z for e in ex] + [0.0] * (nk - last - 1))
    return out


def cosine(a, b):
    dot = sum(x * y for x, y in zip(a, b))
    na = math.sqrt(sum(x * x for x in a))
    nb = math.sqrt(sum(y * y for y in b))
    return dot / (na * nb) if na > 0 and nb > 0 else 0.0


def best_subset(masses, tau):
    """Among subsets whose normalised mass reaches tau: smallest size, then largest mass.

    Returns (size, best mass, list of subsets achieving both) by enumeration.
    """
    total = sum(masses)
    n = len(masses)
    for size in range(1, n + 1):
        best, winners = -1.0, []
        for sub in itertools.combinations(range(n), size):
            m = sum(masses[c] for c in sub)
            if m / total >= tau:
                if m > best + 1e-15:
                    best, winners = m, [sorted(sub)]
                elif abs(m - best) <= 1e-15:
                    winners.append(sorted(sub))
        if winners:
            return size, best, winners
    return n, total, [list(range(n))]


def mapped_av(maps, M, V):
    """O[h][i][e] = sum_j sum_s M[h][s] * maps[s][i][j] * V[h][j][e]."""
    hr, hs = len(M), len(M[0])
    nq, nk, d = len(maps[0]), len(maps[0][0]), len(V[0][0])
    out = []
    for h in range(hr):
        rows = []
        for i in range(nq):
            row = []
            for e in range(d):
                acc = 0.0
                for j in range(nk):
                    b = 0.0
                    for s in range(hs):
                        b += M[h][s] * maps[s][i][j]
                    acc += b * V[h][j][e]
                row.append(acc)
            rows.append(row)
        out.append(rows)
    return out
