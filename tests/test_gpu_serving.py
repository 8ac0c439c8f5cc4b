"""GPU parity of the serving-side rows of the path: prefill chunks (a query chunk
at the end of a longer key prefix, the block grid from the sequence start), V read
through a page table, block-sparse rows listed by (begin, end) in a shared pool,
and the prefix-hash cache flow of MapFlow's storage-and-execution section: a
request whose prompt shares a prefix with a cached one reuses the cached sender
block-rows, compresses only its own chunk, and two receivers are served from the
assembled state. Expected values come from the float64 oracle; the reuse paths
must also give the bits of the direct computation."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import (dev_bf16, dev_f32, dev_i32, f64, host64, rel_l2, blocks_from_panels, blocks_to_panels,
                            bf16_bits_from_f64, greedy_mismatches)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def cma():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cross_model_attention_causal_amd as c
    c.load_library()
    return c


def _chunk_inputs(seed, H, lq, lk, d=128):
    """Q rows for the chunks (the last lq of each sequence), K rows for all lk keys."""
    x = synth.attention_inputs(seed, H, lk, d=d)
    cu_k = x["cu_q"]
    q_full = x["q"]
    q = np.concatenate([q_full[:, cu_k[s] + lk[s] - lq[s]: cu_k[s] + lk[s]] for s in range(len(lq))], axis=1)
    return dict(q=np.ascontiguousarray(q), q_full=q_full, k=x["k"], scale=x["scale"], bias=x["bias"],
                cu_q=synth.cu_from_lengths(lq), cu_k=cu_k)


@pytest.mark.parametrize("d", [128, 64])
def test_chunked_compress_matches_oracle(cma, d):
    lq, lk = [448, 70, 128, 0], [576, 198, 128, 64]
    H, tau = 3, 0.9
    say(f"chunked block_compress d={d} lq={lq} lk={lk}")
    x = _chunk_inputs(951 + d, H, lq, lk, d)
    vl = cma.Varlen(x["cu_q"], x["cu_k"], used_q=lq, used_k=lk)
    out = cma.block_compress(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_f32(x["scale"]), dev_f32(x["bias"]), vl, tau,
                             want_mass=True, want_stats=True)
    torch.cuda.synchronize()
    ref = oracle.block_compress(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], tau, used=lq,
                                cu_k=x["cu_k"], used_k=lk)
    nnz = int(out["nnz"].item())
    row_ptr = host64(out["row_ptr"]).astype(np.int64)
    col = host64(out["col_idx"][:nnz]).astype(np.int64)
    vals = blocks_from_panels(host64(out["vals"][:nnz]))
    mass = host64(out["block_mass"])
    assert mass.shape == ref["masses"].shape
    assert rel_l2(mass, ref["masses"]) <= 1e-5
    st = host64(out["row_stats"])
    assert rel_l2(st[..., 1], ref["row_stats"][..., 1]) <= 1e-5
    assert np.max(np.abs(st[..., 0] - ref["row_stats"][..., 0])) <= 1e-4
    same = 0
    for g in range(len(ref["kept"])):
        gk = list(col[row_ptr[g]: row_ptr[g + 1]])
        if ref["margins"][g] > 1e-4:
            assert gk == ref["kept"][g], g
        if gk == ref["kept"][g] and gk:
            a, b = row_ptr[g], ref["row_ptr"][g]
            assert rel_l2(vals[a: a + len(gk)], ref["vals"][b: b + len(gk)]) <= 1e-2
            same += 1
    R_list = [(n + 63) // 64 for n in lq]
    kb0 = [(b - a) // 64 for a, b in zip(lq, lk)]
    for h in range(H):
        _, bad, _ = greedy_mismatches(mass[h], row_ptr, col, R_list, tau, head_off=h * sum(R_list), kb0_list=kb0)
        assert not bad
    say(f"  nnz={nnz} (oracle {ref['nnz']}), {same} block-rows compared")


@pytest.fixture(scope="module")
def prompt_pair(cma):
    """Prompt A (1024 tokens) and prompt B sharing A's first 640 tokens (10
    block-rows), both as 16 sender heads; B's own 384 tokens are new."""
    H, n, shared = 16, 1024, 640
    xa = synth.attention_inputs(961, H, [n], d=128)
    xb = synth.attention_inputs(962, H, [n], d=128)
    for key in ("q", "k"):
        xb[key] = xb[key].copy()
        xb[key][:, :shared] = xa[key][:, :shared]
    xb["scale"], xb["bias"] = xa["scale"], xa["bias"]
    rng = np.random.default_rng(963)
    tok_a = rng.integers(0, 50000, n).astype(np.int32)
    tok_b = np.concatenate([tok_a[:shared], rng.integers(0, 50000, n - shared).astype(np.int32)])
    return dict(xa=xa, xb=xb, tok_a=tok_a, tok_b=tok_b, H=H, n=n, shared=shared)


def test_chunk_rows_equal_whole_prompt_rows(cma, prompt_pair):
    """B's last 384 queries compressed as a chunk over its 1024 keys give the same
    bits as block-rows 10 .. 15 of B compressed whole."""
    P = prompt_pair
    xb, H, n, sh = P["xb"], P["H"], P["n"], P["shared"]
    q, k, sc, bi = dev_bf16(xb["q"]), dev_bf16(xb["k"]), dev_f32(xb["scale"]), dev_f32(xb["bias"])
    full = cma.block_compress(q, k, sc, bi, cma.Varlen([0, n]), 0.95, want_mass=True)
    chunk = cma.block_compress(q[:, sh:].contiguous(), k, sc, bi,
                               cma.Varlen([0, n - sh], [0, n], used_q=[n - sh], used_k=[n]), 0.95, want_mass=True)
    torch.cuda.synchronize()
    R, kb0 = n // 64, sh // 64
    rf, rc = host64(full["row_ptr"]).astype(np.int64), host64(chunk["row_ptr"]).astype(np.int64)
    for h in range(H):
        for r in range(R - kb0):
            gf, gc = h * R + kb0 + r, h * (R - kb0) + r
            a, b = int(rf[gf]), int(rf[gf + 1])
            c0, c1 = int(rc[gc]), int(rc[gc + 1])
            assert torch.equal(chunk["col_idx"][c0:c1], full["col_idx"][a:b]), (h, r)
            assert torch.equal(chunk["vals"][c0:c1].view(torch.int16), full["vals"][a:b].view(torch.int16)), (h, r)
    say("  chunk block-rows bitwise equal to the whole prompt's")


def _paged(cma, v, vl, n_pages, seed):
    """V tiled into a page pool through a shuffled page table."""
    rng = np.random.default_rng(seed)
    nkb = [(int(x) + 63) // 64 for x in vl.lens_k]
    stride = max(nkb) + 3
    perm = rng.permutation(n_pages)
    table = np.full((vl.n_seqs, stride), -1, dtype=np.int32)
    used = 0
    for s, m in enumerate(nkb):
        table[s, :m] = perm[used: used + m]
        used += m
    pages = torch.zeros((v.shape[0], n_pages, 64 * 128), dtype=torch.bfloat16, device="cuda")
    tab = dev_i32(table)
    cma.tile_v_paged(v, vl, pages, tab)
    return dict(pages=pages, table=tab)


@pytest.mark.parametrize("Hs", [24, 40])
def test_mapped_av_chunks_and_paged_v(cma, Hs):
    """The fused pass (learned M) and the indexed pass over chunked block-sparse
    maps, against the oracle; V token-major (tiled in the workspace), tiled by the
    caller and paged through a shuffled table all give the same bits. With 40
    senders the fused pass runs as two sender groups."""
    lq, lk = [448, 70, 128], [576, 198, 128]
    Hr, Hv = 20, 10
    say(f"mapped_av on chunks lq={lq} lk={lk} Hs={Hs} Hr={Hr} Hv={Hv}")
    x = _chunk_inputs(971, Hs, lq, lk)
    ref = oracle.block_compress(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], 0.9, used=lq,
                                cu_k=x["cu_k"], used_k=lk)
    vl = cma.Varlen(x["cu_q"], x["cu_k"], used_q=lq, used_k=lk)
    src = dict(row_ptr=dev_i32(ref["row_ptr"]), col_idx=dev_i32(ref["col_idx"]),
               vals=dev_bf16(bf16_bits_from_f64(blocks_to_panels(ref["vals"]))), n_block_rows=ref["r_tot"],
               n_key_blocks=vl.n_key_blocks)
    Tq, Tk = int(x["cu_q"][-1]), int(x["cu_k"][-1])
    V = synth.values(972, Hv, Tk, 128)
    M = synth.mix_matrix_learned(973, Hr, Hs)
    v = dev_bf16(V)
    O = cma.mapped_av(src, Hs, dev_f32(M), Hr, v, vl, q_rows=Tq, v_heads=Hv)
    vt = cma.tile_v(v, vl, vl.n_key_blocks)
    Ot = cma.mapped_av(src, Hs, dev_f32(M), Hr, vt, vl, q_rows=Tq, v_heads=Hv, v_layout=cma.V_TILED, k_rows=Tk)
    pv = _paged(cma, v, vl, 40, 974)
    Op = cma.mapped_av(src, Hs, dev_f32(M), Hr, pv, vl, q_rows=Tq, v_heads=Hv, v_layout=cma.V_PAGED, k_rows=Tk)
    idx = (np.arange(Hr) * 7 % Hs).astype(np.int32)[None, :]
    Oi = cma.mapped_av(src, Hs, dev_i32(idx), Hr, v, vl, q_rows=Tq, v_heads=Hv, out_dtype=torch.float32)
    Oip = cma.mapped_av(src, Hs, dev_i32(idx), Hr, pv, vl, q_rows=Tq, v_heads=Hv, v_layout=cma.V_PAGED, k_rows=Tk,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(O, Ot) and torch.equal(O, Op)
    assert torch.equal(Oi, Oip)
    rows = [(s, r) for s in range(len(lq)) for r in range((lq[s] + 63) // 64)]
    Vr = np.repeat(f64(V), Hr // Hv, axis=0)
    oo = oracle.mapped_av_bsr_rows(ref["row_ptr"], ref["col_idx"], ref["vals"], Hs, lq, M, Vr, x["cu_k"], rows,
                                   lengths_k=lk)
    Mo = oracle.onehot_mix(idx, Hs)
    oi = oracle.mapped_av_bsr_rows(ref["row_ptr"], ref["col_idx"], ref["vals"], Hs, lq, Mo, Vr, x["cu_k"], rows,
                                   lengths_k=lk)
    got, goti = host64(O), host64(Oi)
    refO, refI = np.zeros_like(got), np.zeros_like(goti)
    for (s, r), o in oo.items():
        a = x["cu_q"][s] + 64 * r
        refO[:, a: a + o.shape[1]] = o
        refI[:, a: a + o.shape[1]] = oi[(s, r)]
    assert rel_l2(got, oracle.round_bf16(refO)) <= 1e-2
    assert rel_l2(goti, refI) <= 1e-5
    say("  fused and indexed passes on chunks match the oracle; token-major, tiled and paged V bitwise equal")


def test_prefix_cache_serving_flow(cma, prompt_pair):
    """A's compressed block-rows are cached under their prefix hashes. B shares A's
    first 640 tokens: the lookup finds 10 block-rows, only B's last 384 queries
    are compressed (a chunk over all 1024 keys), and the state assembled from the
    cache and the chunk (rows given by begin / end in one block pool) serves two
    receivers stacked in one call (8 and 12 heads, their own V heads, paged V),
    bit for bit as B compressed whole and, on sampled rows, as the oracle."""
    P = prompt_pair
    xa, xb, H, n, sh = P["xa"], P["xb"], P["H"], P["n"], P["shared"]
    R, kb0, seed = n // 64, sh // 64, 0x5EED
    sc, bi = dev_f32(xa["scale"]), dev_f32(xa["bias"])
    vl = cma.Varlen([0, n])
    # request A: compress, cache every block-row
    A = cma.block_compress(dev_bf16(xa["q"]), dev_bf16(xa["k"]), sc, bi, vl, 0.95)
    torch.cuda.synchronize()
    nnz_a = int(A["nnz"].item())
    rp_a = host64(A["row_ptr"]).astype(np.int64)
    index = cma.PrefixIndex(H, 1024)
    hashes_a = cma.prefix_hashes(P["tok_a"], seed)
    for r in range(R):
        beg = [rp_a[h * R + r] for h in range(H)]
        cnt = [rp_a[h * R + r + 1] - rp_a[h * R + r] for h in range(H)]
        assert index.insert(0, hashes_a[r], beg, cnt) == 0
    # request B: look up its prefix, compress only the rest
    hashes_b = cma.prefix_hashes(P["tok_b"], seed)
    hits, beg, cnt = index.lookup(0, hashes_b)
    assert hits == kb0
    qb, kb = dev_bf16(xb["q"]), dev_bf16(xb["k"])
    C = cma.block_compress(qb[:, sh:].contiguous(), kb, sc, bi,
                           cma.Varlen([0, n - sh], [0, n], used_q=[n - sh], used_k=[n]), 0.95)
    torch.cuda.synchronize()
    nnz_c = int(C["nnz"].item())
    rp_c = host64(C["row_ptr"]).astype(np.int64)
    # one pool: A's blocks, then the chunk's; B's rows by (begin, end)
    pool_col = torch.cat([A["col_idx"][:nnz_a], C["col_idx"][:nnz_c]])
    pool_vals = torch.cat([A["vals"][:nnz_a], C["vals"][:nnz_c]]).contiguous()
    row_beg = np.zeros(H * R, dtype=np.int32)
    row_end = np.zeros(H * R, dtype=np.int32)
    for h in range(H):
        for r in range(R):
            g = h * R + r
            if r < hits:
                row_beg[g], row_end[g] = beg[r, h], beg[r, h] + cnt[r, h]
            else:
                gc = h * (R - kb0) + r - kb0
                row_beg[g], row_end[g] = nnz_a + rp_c[gc], nnz_a + rp_c[gc + 1]
    state = dict(row_ptr=dev_i32(row_beg), row_end=dev_i32(row_end), col_idx=pool_col, vals=pool_vals,
                 n_block_rows=R)
    # B compressed whole, for comparison
    Bw = cma.block_compress(qb, kb, sc, bi, vl, 0.95)
    # two receivers stacked: 8 heads over 4 V heads, 12 heads over 6 V heads (group 2)
    M1, M2 = synth.mix_matrix_learned(981, 8, H), synth.mix_matrix_learned(982, 12, H)
    V1, V2 = synth.values(983, 4, n, 128), synth.values(984, 6, n, 128)
    Ms = np.concatenate([M1, M2], axis=1)
    v = dev_bf16(np.concatenate([V1, V2]))
    pv = _paged(cma, v, vl, 32, 985)
    O_cache = cma.mapped_av(state, H, dev_f32(Ms), 20, pv, vl, v_heads=10, v_layout=cma.V_PAGED, k_rows=n)
    O_whole = cma.mapped_av(Bw, H, dev_f32(Ms), 20, v, vl, v_heads=10)
    idx = (np.arange(20) * 3 % H).astype(np.int32)[None, :]
    I_cache = cma.mapped_av(state, H, dev_i32(idx), 20, pv, vl, v_heads=10, v_layout=cma.V_PAGED, k_rows=n)
    I_whole = cma.mapped_av(Bw, H, dev_i32(idx), 20, v, vl, v_heads=10)
    torch.cuda.synchronize()
    assert torch.equal(O_cache, O_whole)
    assert torch.equal(I_cache, I_whole)
    # the oracle on two block-rows: one from the cache, one from the chunk
    got = host64(O_cache)
    Vr = np.repeat(f64(np.concatenate([V1, V2])), 2, axis=0)
    for r in (kb0 - 1, R - 1):
        refs = [oracle.compress_block_row(f64(xb["q"][j]), f64(xb["k"][j]), xb["scale"][j], xb["bias"][j], r, 0.95)
                for j in range(H)]
        mixed = np.zeros((20, 64, 64 * (r + 1)))
        for j in range(H):
            g = j * R + r
            cols = host64(pool_col[row_beg[g]: row_end[g]]).astype(int)
            if refs[j]["margin"] > 1e-4:
                assert list(cols) == refs[j]["kept"], (r, j)
            Aj = np.zeros((64, 64 * (r + 1)))
            for c in cols:
                Aj[:, 64 * c: 64 * c + 64] = oracle.round_bf16(refs[j]["rows"][:, 64 * c: 64 * c + 64])
            mixed += Ms[0][:, j, None, None] * Aj[None]
        ref = np.stack([mixed[h] @ Vr[h, : 64 * (r + 1)] for h in range(20)])
        assert rel_l2(got[:, 64 * r: 64 * r + 64], oracle.round_bf16(ref)) <= 1e-2, r
    index.close()
    say(f"  prefix hits {hits}/{R} block-rows; cached + chunk state equals the whole prompt's bits; oracle rows match")
