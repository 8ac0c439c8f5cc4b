"""Helpers for GPU tests: moving seeded inputs to the device and comparing with the oracle."""
import numpy as np
import torch

import synth


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host64(t):
    """GPU tensor (bf16 or fp32) -> float64 numpy, exact."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(bits_or_f32):
    """Stored input values as float64 (bf16 bits widened exactly, or fp32)."""
    a = np.asarray(bits_or_f32)
    if a.dtype == np.uint16:
        return synth.bf16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def bf16_bits_from_f64(x):
    """Exactly-representable bf16 values (float64) -> uint16 bits."""
    return synth.bf16_from_f32(np.asarray(x, dtype=np.float32))


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return num / den if den > 0 else num


def blocks_to_panels(vals):
    """Row-major 64x64 blocks [nnz, 64, 64] -> the library's stored layout (four
    16-column panels per block, each row-major), returned as [nnz, 64, 64]."""
    v = np.asarray(vals)
    return np.ascontiguousarray(v.reshape(-1, 64, 4, 16).transpose(0, 2, 1, 3)).reshape(-1, 64, 64)


def blocks_from_panels(vals):
    """Inverse of blocks_to_panels."""
    v = np.asarray(vals)
    return np.ascontiguousarray(v.reshape(-1, 4, 64, 16).transpose(0, 2, 1, 3)).reshape(-1, 64, 64)


def tile_v(V, lens, cu):
    """Token-major V [H, T, 128] (uint16 bf16 bits) -> the tiled operand layout the
    library documents: [H, sum ceil(len/64), 64 * 128], block c of sequence s at
    block offset sum_{u<s} ceil(len_u/64); element ((ks*4+dt)*64 + L)*8 + e of a
    block is V[key 64c + 16ks + 8(L//32) + e][feature 32dt + L%32], zero past the end."""
    V = np.asarray(V)
    H = V.shape[0]
    nb = [(n + 63) // 64 for n in lens]
    out = np.zeros((H, sum(nb), 64 * 128), dtype=V.dtype)
    dt, ks, L, e = np.meshgrid(np.arange(4), np.arange(4), np.arange(64), np.arange(8), indexing="ij")
    key = 16 * ks + 8 * (L // 32) + e
    feat = 32 * dt + L % 32
    pos = (((ks * 4 + dt) * 64 + L) * 8 + e).ravel()
    b0 = 0
    for s, n in enumerate(lens):
        for c in range(nb[s]):
            blk = np.zeros((H, 64, 128), dtype=V.dtype)
            m = min(64, n - 64 * c)
            blk[:, :m] = V[:, cu[s] + 64 * c: cu[s] + 64 * c + m]
            out[:, b0 + c, pos] = blk[:, key.ravel(), feat.ravel()]
        b0 += nb[s]
    return out


def greedy_mismatches(mass_packed, row_ptr, col, R_list, tau, head_off=0, min_margin=1e-6, kb0_list=None):
    """Selection validity on every block-row, from the library's own masses.

    ``mass_packed``: one head's masses over its sequences, each packed
    lower-triangular (offset + r(r+1)/2 + c); ``R_list``: block-rows per sequence;
    ``head_off``: index of the head's first block-row in ``row_ptr``; ``kb0_list``:
    per sequence, the first block-row of a prefill chunk (its block-row r holds
    kb0 + r + 1 masses from r kb0 + r(r+1)/2; default 0, whole prompts). For every
    block-row the greedy shortest prefix (weight descending, ties to the lower
    column, running sum >= tau) is recomputed in float64 from those masses and
    compared with the kept columns the library returned. Returns (rows compared,
    list of mismatching rows whose margin under the library's masses exceeds
    ``min_margin``, rows skipped for a smaller margin).
    """
    import oracle
    bad, skipped, n = [], 0, 0
    off, g = 0, head_off
    kb0_list = kb0_list or [0] * len(R_list)
    for R, kb in zip(R_list, kb0_list):
        for r in range(R):
            o = off + r * kb + r * (r + 1) // 2
            mrow = np.asarray(mass_packed[o: o + kb + r + 1], dtype=np.float64)
            kept = [int(c) for c in col[row_ptr[g]: row_ptr[g + 1]]]
            n += 1
            if mrow.sum() > 0:
                want = oracle.select_blocks(mrow, tau)
                if kept != want:
                    if oracle.selection_margin(mrow, tau) > min_margin:
                        bad.append(g)
                    else:
                        skipped += 1
            g += 1
        off += R * kb + R * (R + 1) // 2
    return n, bad, skipped
