"""GPU parity at the workloads' full sizes, on sampled outputs the oracle can
compute one by one, plus properties checked over every output.

Each test runs the library exactly as the benchmark does (same entry points,
same layouts and workspaces) on the full-size seeded inputs, then checks:
* sampled outputs element by element against the float64 oracle (relative L2
  1e-5 for fp32 results, 1e-2 for bf16 results; argmax and kept sets bit-exact
  where the oracle's decision margin exceeds 1e-4);
* size-independent properties over all outputs (kept mass reaches tau under the
  library's own masses, at least one kept block per row, sorted columns).
No expected value comes from the library: the oracle computes its own maps,
block statistics, selections and mixing matrices from the same inputs.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import dev_bf16, dev_f32, f64, host64, rel_l2, blocks_from_panels, greedy_mismatches

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


# ------------------------------------------------------------------ IAM head mapping, 512 tokens
def test_cfg2_head_mapping_full(cma):
    """2560 LLM maps x 336 SLM maps over 131,328 causal entries (bf16)."""
    t0 = time.time()
    x = synth.cfg2()
    Hs, Hr, n = x["n_send"], x["n_recv"], x["n"]
    say(f"cfg2: inputs in {time.time() - t0:.1f}s; Hs={Hs} Hr={Hr} n={n}")
    L = n * (n + 1) // 2
    vl = cma.Varlen(x["cu"])
    sm = cma.attn_maps(dev_bf16(x["send_q"]), dev_bf16(x["send_k"]), dev_f32(x["send_scale"]),
                       dev_f32(x["send_bias"]), vl)
    rm = cma.attn_maps(dev_bf16(x["recv_q"]), dev_bf16(x["recv_k"]), dev_f32(x["recv_scale"]),
                       dev_f32(x["recv_bias"]), vl)
    cos, arg, mar = cma.head_map_cosine(rm, sm, 1, Hr, Hs, L, L, 0, L, 0)
    torch.cuda.synchronize()
    say(f"cfg2: GPU done at {time.time() - t0:.1f}s")
    # oracle: every sender map, a sample of receiver maps (bf16-rounded as stored)
    S = np.stack([oracle.round_bf16(oracle.pack_rows(oracle.causal_map(
        f64(x["send_q"][j]), f64(x["send_k"][j]), x["send_scale"][j], x["send_bias"][j]))) for j in range(Hs)])
    rs = np.linspace(0, Hr - 1, 24).astype(int)
    R = np.stack([oracle.round_bf16(oracle.pack_rows(oracle.causal_map(
        f64(x["recv_q"][h]), f64(x["recv_k"][h]), x["recv_scale"][h], x["recv_bias"][h]))) for h in rs])
    say(f"cfg2: oracle maps at {time.time() - t0:.1f}s")
    ocos, oarg, omar = oracle.head_map(R, S)
    # sampled maps as stored
    sm_h, rm_h = host64(sm[[0, 100, 335]]), host64(rm[rs[:3]])
    for a, b in zip(sm_h, S[[0, 100, 335]]):
        assert rel_l2(a, b) <= 1e-2
    for a, b in zip(rm_h, R[:3]):
        assert rel_l2(a, b) <= 1e-2
    gcos, garg, gmar = host64(cos)[0], host64(arg)[0].astype(int), host64(mar)[0]
    assert rel_l2(gcos[rs], ocos) <= 1e-5
    big = omar > 1e-4
    assert np.array_equal(garg[rs][big], oarg[big])
    say(f"cfg2: {big.sum()}/{len(rs)} sampled heads above the margin line, all argmax equal")
    # every receiver: the argmax is a valid sender and its cosine is the row maximum
    assert garg.min() >= 0 and garg.max() < Hs
    assert np.all(gcos[np.arange(Hr), garg] >= gcos.max(axis=1) - 1e-7)
    assert np.all((gcos >= -1e-6) & (gcos <= 1 + 1e-6))


# ------------------------------------------------------------------ block-sparse compression, 8192 tokens
@pytest.fixture(scope="module")
def cfg3_run(cma):
    t0 = time.time()
    x = synth.cfg3()
    H, n, tau = x["n_heads"], x["n"], x["tau"]
    vl = cma.Varlen(x["cu"])
    q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
    out = cma.block_compress(q, k, dev_f32(x["scale"]), dev_f32(x["bias"]), vl, tau, want_mass=True,
                             want_stats=True, workspace=cma.Workspace())
    torch.cuda.synchronize()
    say(f"cfg3: inputs + GPU compression in {time.time() - t0:.1f}s, nnz={int(out['nnz'].item())}")
    return x, vl, out


def test_cfg3_compress_full(cma, cfg3_run):
    """32 heads x 8192 tokens, tau = 0.95: sampled block-rows against the oracle,
    selection invariants over every block-row."""
    x, vl, out = cfg3_run
    H, n, tau = x["n_heads"], x["n"], x["tau"]
    R = n // 64
    nnz = int(out["nnz"].item())
    row_ptr = host64(out["row_ptr"]).astype(np.int64)
    col = host64(out["col_idx"][:nnz]).astype(np.int64)
    mass = host64(out["block_mass"])
    stats = host64(out["row_stats"])
    assert row_ptr[0] == 0 and row_ptr[-1] == nnz and np.all(np.diff(row_ptr) >= 1)
    # invariants on every block-row, under the library's own masses
    tri0 = lambda r: r * (r + 1) // 2
    worst = np.inf
    for h in range(H):
        for r in range(R):
            g = h * R + r
            cs = col[row_ptr[g]: row_ptr[g + 1]]
            assert np.all(np.diff(cs) > 0) and cs[0] >= 0 and cs[-1] <= r
            mrow = mass[h, tri0(r): tri0(r) + r + 1]
            worst = min(worst, mrow[cs].sum() / mrow.sum() - tau)
    assert worst >= -1e-6
    say(f"cfg3: kept mass reaches tau on all {H * R} block-rows (min overshoot {worst:.2e})")
    # every block-row: the kept set is the greedy prefix of the library's own masses
    skipped = 0
    for h in range(H):
        _, bad, sk = greedy_mismatches(mass[h], row_ptr, col, [R], tau, head_off=h * R)
        assert not bad, (h, bad[:5])
        skipped += sk
    say(f"cfg3: greedy prefix of the library's masses on all {H * R} block-rows ({skipped} within 1e-6)")
    # sampled block-rows against the oracle
    exempt = checked = 0
    for h in (0, 7, 19, 31):
        for r in (0, 1, 63, 126, 127):
            ref = oracle.compress_block_row(f64(x["q"][h]), f64(x["k"][h]), x["scale"][h], x["bias"][h], r, tau)
            mrow = mass[h, tri0(r): tri0(r) + r + 1]
            assert rel_l2(mrow, ref["masses"]) <= 1e-5
            rows = slice(64 * r, 64 * r + 64)
            assert np.max(np.abs(stats[h, rows, 0] - ref["m"])) <= 1e-4
            assert rel_l2(stats[h, rows, 1], ref["l"]) <= 1e-5
            g = h * R + r
            cs = list(col[row_ptr[g]: row_ptr[g + 1]])
            if ref["margin"] > 1e-4:
                assert cs == ref["kept"], (h, r)
            if cs == ref["kept"]:
                v = blocks_from_panels(host64(out["vals"][row_ptr[g]: row_ptr[g + 1]]))
                assert rel_l2(v, ref["blocks"]) <= 1e-2
                checked += 1
            else:
                exempt += 1
    say(f"cfg3: {checked} sampled block-rows equal, {exempt} exempt (margin <= 1e-4)")


# ------------------------------------------------------------------ fused mapped x V, 8192 tokens
def _bsr_row_reference(refs, kept_lib, Hs, R, r):
    """A block-sparse structure holding only block-row ``r`` of every sender, with
    the library's own kept columns and, at each, the exact float64 map block
    rounded to bf16 (so the comparison covers every sampled row, whatever the
    selection margin)."""
    counts = np.zeros(Hs * R, dtype=np.int64)
    cis, vvs = [], []
    for j in range(Hs):
        cols = kept_lib[j]
        counts[j * R + r] = len(cols)
        cis.append(np.asarray(cols, dtype=np.int64))
        vvs.append(oracle.round_bf16(np.stack([refs[j]["rows"][:, 64 * c: 64 * c + 64] for c in cols]))
                   if cols else np.zeros((0, 64, 64)))
    rp = np.concatenate([[0], np.cumsum(counts)])
    return rp, np.concatenate(cis), np.concatenate(vvs)


def test_cfg4_mapped_av_full(cma, cfg3_run):
    """24 receiver heads over the 32-head compressed maps of the 8192-token
    sequence, learned M, token-major V through the workspace (as benchmarked).
    Sampled block-rows (four of them past block-row 32): every sender whose
    oracle margin exceeds 1e-4 must keep exactly the oracle's columns, and the
    output is compared with the oracle's mixed product over the library's kept
    columns (exact map blocks rounded to bf16)."""
    x, vl, bsr = cfg3_run
    y = synth.cfg4()
    Hs, Hr, n = y["n_send"], y["n_recv"], y["n"]
    R = n // 64
    O = cma.mapped_av(bsr, Hs, dev_f32(y["M"]), Hr, dev_bf16(y["v"]), vl, workspace=cma.Workspace())
    torch.cuda.synchronize()
    nnz = int(bsr["nnz"].item())
    row_ptr = host64(bsr["row_ptr"]).astype(np.int64)
    col = host64(bsr["col_idx"][:nnz]).astype(np.int64)
    got = host64(O)
    V = f64(y["v"])
    M = y["M"].astype(np.float64)  # [1, Hr, Hs]: one matrix for the sequence
    sample = (0, 2, 40, 64, 100, 127)
    compared, long_rows, decided = 0, 0, 0
    for r in sample:
        refs = [oracle.compress_block_row(f64(x["q"][j]), f64(x["k"][j]), x["scale"][j], x["bias"][j], r, x["tau"])
                for j in range(Hs)]
        kept_lib = [list(col[row_ptr[j * R + r]: row_ptr[j * R + r + 1]]) for j in range(Hs)]
        for j in range(Hs):
            if refs[j]["margin"] > 1e-4:
                assert kept_lib[j] == refs[j]["kept"], (r, j)
                decided += 1
        rp, ci, vv = _bsr_row_reference(refs, kept_lib, Hs, R, r)
        ref = oracle.mapped_av_bsr_rows(rp, ci, vv, Hs, [n], M, V, np.array([0, n]), [(0, r)])[(0, r)]
        assert rel_l2(got[:, 64 * r: 64 * r + 64], oracle.round_bf16(ref)) <= 1e-2, r
        compared += 1
        long_rows += r >= 32
    assert compared == len(sample) and long_rows >= 3
    say(f"cfg4: {compared} sampled block-rows compared ({long_rows} past block-row 32); "
        f"{decided} decided sender selections equal the oracle's")
    assert np.isfinite(got).all()


def test_cfg4_mapped_av_sender_groups_full(cma, cfg3_run):
    """The fused pass over 64 senders at full size (two groups of 32, the second
    pass adding into the output): the 32-head compression of the 8192-token
    sequence stacked twice. Mixing the two copies with weights M[:, :32] and
    M[:, 32:] equals mixing one copy with their sum, so the output is compared
    with the oracle's product for the summed weights on sampled block-rows."""
    x, vl, bsr = cfg3_run
    y = synth.cfg4()
    Hs, Hr, n = y["n_send"], y["n_recv"], y["n"]
    R = n // 64
    nnz = int(bsr["nnz"].item())
    rp = bsr["row_ptr"][: Hs * R + 1]
    stacked = dict(row_ptr=torch.cat([rp[:-1], rp + nnz]), col_idx=torch.cat([bsr["col_idx"][:nnz]] * 2),
                   vals=torch.cat([bsr["vals"][:nnz]] * 2), n_block_rows=R)
    M2 = synth.mix_matrix_learned(171, Hr, 2 * Hs).astype(np.float32)
    O = cma.mapped_av(stacked, 2 * Hs, dev_f32(M2), Hr, dev_bf16(y["v"]), vl, workspace=cma.Workspace())
    torch.cuda.synchronize()
    got = host64(O)
    del stacked
    row_ptr = host64(bsr["row_ptr"]).astype(np.int64)
    col = host64(bsr["col_idx"][:nnz]).astype(np.int64)
    V = f64(y["v"])
    Msum = M2[..., :Hs].astype(np.float64) + M2[..., Hs:].astype(np.float64)
    for r in (3, 77, 126):
        refs = [oracle.compress_block_row(f64(x["q"][j]), f64(x["k"][j]), x["scale"][j], x["bias"][j], r, x["tau"])
                for j in range(Hs)]
        kept_lib = [list(col[row_ptr[j * R + r]: row_ptr[j * R + r + 1]]) for j in range(Hs)]
        rp_, ci, vv = _bsr_row_reference(refs, kept_lib, Hs, R, r)
        ref = oracle.mapped_av_bsr_rows(rp_, ci, vv, Hs, [n], Msum, V, np.array([0, n]), [(0, r)])[(0, r)]
        assert rel_l2(got[:, 64 * r: 64 * r + 64], oracle.round_bf16(ref)) <= 1e-2, r
    assert np.isfinite(got).all()
    say("cfg4 with 64 senders (two stacked copies): 3 sampled block-rows equal the oracle's summed-weight product")


# ------------------------------------------------------------------ serving mix, one mapped layer
def test_cfg5_serving_layer_full(cma):
    """64 x 512 + 4 x 8192 prompts packed varlen, 28 sender / 64 receiver heads:
    prefix maps and per-prompt cosine head maps, one-hot M, block compression of
    every prompt, fused mapped x V with the one-hot M, and decode rows at two
    steps. Sampled prompts, heads and block-rows against the oracle."""
    t0 = time.time()
    x = synth.cfg5_layer(0)
    Hs, Hr, tt, nsh, dec = x["n_send"], x["n_recv"], x["tau_t"], x["n_short"], x["decode"]
    pl, st = x["prompt_lengths"], x["store_lengths"]
    cp, cs = x["cu_prompt"], x["cu_store"]
    P = len(pl)
    L = tt * (tt + 1) // 2
    say(f"cfg5: inputs in {time.time() - t0:.1f}s")
    sq, sk = dev_bf16(x["send_q"]), dev_bf16(x["send_k"])
    ss, sb = dev_f32(x["send_scale"]), dev_f32(x["send_bias"])
    # prefix maps (each prompt's first tau_t tokens) and head map per prompt
    vl_s = cma.Varlen(cp, cs, used_q=[tt] * P, used_k=[tt] * P)
    vl_r = cma.Varlen(np.arange(P + 1) * tt)
    sm = cma.attn_maps(sq, sk, ss, sb, vl_s)
    rm = cma.attn_maps(dev_bf16(x["recv_q"]), dev_bf16(x["recv_k"]), dev_f32(x["recv_scale"]),
                       dev_f32(x["recv_bias"]), vl_r)
    cos, arg, mar = cma.head_map_cosine(rm, sm, P, Hr, Hs, L, P * L, L, P * L, L)
    Mo = cma.onehot_mix(arg, Hs)
    # compression and the fused pass over the prompts
    vl_p = cma.Varlen(cp, cs, used_q=pl, used_k=pl)
    bsr = cma.block_compress(sq, sk, ss, sb, vl_p, 0.95, workspace=cma.Workspace())
    v = dev_bf16(x["v"])
    O = cma.mapped_av(bsr, Hs, Mo, Hr, v, vl_p, q_rows=int(cp[-1]), workspace=cma.Workspace())
    # the same with the argmax as sender indices (each head reads only its sender)
    Oi = cma.mapped_av(bsr, Hs, arg, Hr, v, vl_p, q_rows=int(cp[-1]), workspace=cma.Workspace())
    # decode rows at steps 0 and dec - 1 for the short prompts
    dec_out = {}
    for t in (0, dec - 1):
        vl_d = cma.Varlen(np.arange(nsh + 1), cs[: nsh + 1], used_q=[1] * nsh, used_k=[tt + t + 1] * nsh)
        qd = dev_bf16(np.ascontiguousarray(x["send_dec_q"][t]))
        rows = cma.attn_maps(qd, sk, ss, sb, vl_d, layout=cma.DENSE, out_dtype=torch.float32)
        od = cma.mapped_av(("dense", rows, cma.DENSE), Hs, Mo[:nsh].contiguous(), Hr, v, vl_d, q_rows=nsh)
        dec_out[t] = (host64(rows), host64(od))
    torch.cuda.synchronize()
    say(f"cfg5: GPU done at {time.time() - t0:.1f}s")
    assert arg.dtype == torch.int32 and torch.equal(Oi, O)
    del Oi
    garg, gcos = host64(arg).astype(int), host64(cos)
    nnz = int(bsr["nnz"].item())
    row_ptr = host64(bsr["row_ptr"]).astype(np.int64)
    col = host64(bsr["col_idx"][:nnz]).astype(np.int64)
    Og = host64(O)
    nblk = [(n + 63) // 64 for n in pl]
    roff = np.concatenate([[0], np.cumsum(nblk)])
    R_tot = int(roff[-1])
    V = x["v"]
    checked_rows = 0
    for p in (0, 37, 64, 67):
        # head map of prompt p
        S = np.stack([oracle.round_bf16(oracle.pack_rows(oracle.causal_map(
            f64(x["send_q"][j, cp[p]: cp[p] + tt]), f64(x["send_k"][j, cs[p]: cs[p] + tt]),
            x["send_scale"][j], x["send_bias"][j]))) for j in range(Hs)])
        Rm = np.stack([oracle.round_bf16(oracle.pack_rows(oracle.causal_map(
            f64(x["recv_q"][h, p * tt: (p + 1) * tt]), f64(x["recv_k"][h, p * tt: (p + 1) * tt]),
            x["recv_scale"][h], x["recv_bias"][h]))) for h in range(Hr)])
        ocos, oarg, omar = oracle.head_map(Rm, S)
        assert rel_l2(gcos[p], ocos) <= 1e-5
        big = omar > 1e-4
        assert np.array_equal(garg[p][big], oarg[big]), p
        # fused pass on two block-rows of the prompt, for heads whose mapping is decided
        n = pl[p]
        heads = [h for h in (0, 21, 42, 63) if big[h]]
        for r in sorted({0, nblk[p] - 1}):
            for h in heads:
                j = oarg[h]
                ref = oracle.compress_block_row(f64(x["send_q"][j, cp[p]: cp[p] + n]),
                                                f64(x["send_k"][j, cs[p]: cs[p] + n]),
                                                x["send_scale"][j], x["send_bias"][j], r, 0.95)
                g = j * R_tot + roff[p] + r
                kept = [int(c) for c in col[row_ptr[g]: row_ptr[g + 1]]]
                if ref["margin"] > 1e-4:
                    assert kept == ref["kept"], (p, r, j)
                # the oracle's product over the library's kept columns (exact map
                # blocks rounded to bf16)
                Vh = f64(V[h, cs[p]: cs[p] + n])
                o = np.zeros((64, Vh.shape[1]))
                for c in kept:
                    kk = min(64, n - 64 * c)
                    blk = oracle.round_bf16(ref["rows"][:, 64 * c: 64 * c + 64])
                    o += blk[:, :kk] @ Vh[64 * c: 64 * c + kk]
                rr = min(64, n - 64 * r)
                got = Og[h, cp[p] + 64 * r: cp[p] + 64 * r + rr]
                assert rel_l2(got, oracle.round_bf16(o[:rr])) <= 1e-2, (p, r, h)
                checked_rows += 1
        # decode rows (short prompts)
        if p < nsh:
            for t, (rows, od) in dec_out.items():
                ctx = tt + t + 1
                ks = slice(cs[p], cs[p] + ctx)
                for h in heads[:2]:
                    j = oarg[h]
                    a = oracle.causal_map(f64(x["send_dec_q"][t, j, p][None, :]), f64(x["send_k"][j, ks]),
                                          x["send_scale"][j], x["send_bias"][j])[0]
                    width = rows.shape[1] // nsh
                    assert rel_l2(rows[j, p * width: p * width + ctx], a) <= 1e-5
                    o = a @ f64(V[h, ks])
                    assert rel_l2(od[h, p], oracle.round_bf16(o)) <= 1e-2
    assert checked_rows >= 8
    say(f"cfg5: {checked_rows} sampled (prompt, block-row, head) outputs compared; total {time.time() - t0:.1f}s")
