"""GPU parity at small sizes: every stage against the oracle on the same seeded inputs.

Shapes span several tiles and end in ragged tails (lengths not multiples of 64,
head counts not multiples of the tile widths). Tolerances: relative L2 1e-5 for
fp32 outputs and 1e-2 for bf16 outputs (fp32 accumulation); head-map indices and
kept-block sets bit-exact wherever the oracle's decision margin exceeds 1e-4.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import (dev_bf16, dev_f32, dev_i32, f64, host64, rel_l2, bf16_bits_from_f64, tile_v,
                            blocks_to_panels, blocks_from_panels, greedy_mismatches)

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


# ------------------------------------------------------------------ tiny fp32 workload
def test_cfg1_tiny_fp32_all_stages(cma):
    say("cfg1: tiny fp32, 128 tokens, d=64, 4 sender / 2 receiver heads")
    x = synth.cfg1()
    vl = cma.Varlen(x["cu"], x["cu"])
    n = x["n"]
    # stage 1: dense fp32 maps
    sm = cma.attn_maps(dev_f32(x["send_q"]), dev_f32(x["send_k"]), dev_f32(x["send_scale"]),
                       dev_f32(x["send_bias"]), vl, layout=cma.DENSE, out_dtype=torch.float32)
    rm = cma.attn_maps(dev_f32(x["recv_q"]), dev_f32(x["recv_k"]), dev_f32(x["recv_scale"]),
                       dev_f32(x["recv_bias"]), vl, layout=cma.DENSE, out_dtype=torch.float32)
    torch.cuda.synchronize()
    S = np.stack([oracle.causal_map(f64(x["send_q"][j]), f64(x["send_k"][j]), 0.125) for j in range(4)])
    R = np.stack([oracle.causal_map(f64(x["recv_q"][j]), f64(x["recv_k"][j]), 0.125) for j in range(2)])
    Sr, Rr = oracle.round_f32(S), oracle.round_f32(R)
    assert rel_l2(host64(sm).reshape(4, n, n), Sr) <= 1e-5
    assert rel_l2(host64(rm).reshape(2, n, n), Rr) <= 1e-5
    # stage 2: cosine 2 x 4 on oracle-stored maps
    cos, arg, mar = cma.head_map_cosine(dev_f32(Rr.reshape(2, -1)), dev_f32(Sr.reshape(4, -1)), 1, 2, 4,
                                        n * n, n * n, 0, n * n, 0)
    torch.cuda.synchronize()
    ocos, oarg, omar = oracle.head_map(Rr.reshape(2, -1), Sr.reshape(4, -1))
    assert rel_l2(host64(cos)[0], ocos) <= 1e-5
    for h in range(2):
        if omar[h] > 1e-4:
            assert int(arg[0, h]) == oarg[h]
    # stage 4: dense mapped x V, fp32, on oracle-stored maps
    O = cma.mapped_av(("dense", dev_f32(Sr.reshape(4, -1)), cma.DENSE), 4, dev_f32(x["M"]), 2,
                      dev_f32(x["v"]), vl, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oO = oracle.mapped_av_dense(Sr, x["M"][0].astype(np.float64), f64(x["v"]))
    assert rel_l2(host64(O), oracle.round_f32(oO)) <= 1e-5
    # chained: GPU maps feed GPU mapped_av
    O2 = cma.mapped_av(("dense", sm, cma.DENSE), 4, dev_f32(x["M"]), 2, dev_f32(x["v"]), vl,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_l2(host64(O2), oracle.round_f32(oO)) <= 1e-5


# ------------------------------------------------------------------ attn_maps bf16
# "short": every sequence has at most 512 keys (the one-pass kernel, K resident in
# LDS), with an empty sequence; "long": one sequence past 512 keys (the two-sweep
# kernel); "prefix": more keys than queries, so a unit's first block-row already
# sees several key blocks.
ATTN_CASES = {
    "short": ([130, 64, 0, 7, 200], None),
    "long": ([600, 64, 7, 200], None),
    "prefix": ([130, 64, 7, 200], [300, 64, 100, 512]),
}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("layout", ["packed", "dense"])
@pytest.mark.parametrize("case", list(ATTN_CASES))
def test_attn_maps_bf16_varlen(cma, d, layout, case):
    lens, klens = ATTN_CASES[case]
    say(f"attn_maps bf16 d={d} layout={layout} case={case} lens={lens} k_lens={klens}")
    x = synth.attention_inputs(101 + d, 5, lens, d=d, k_lengths=klens)
    vl = cma.Varlen(x["cu_q"], x["cu_k"])
    lay = cma.PACKED if layout == "packed" else cma.DENSE
    outs = {}
    for out_dtype, tol in ((torch.bfloat16, 1e-2), (torch.float32, 1e-5)):
        maps = cma.attn_maps(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_f32(x["scale"]), dev_f32(x["bias"]),
                             vl, layout=lay, out_dtype=out_dtype)
        torch.cuda.synchronize()
        got = host64(maps)
        outs[out_dtype] = got
        q, k = f64(x["q"]), f64(x["k"])
        om = oracle.attn_maps(q, k, x["scale"], x["bias"], x["cu_q"], x["cu_k"])
        rnd = oracle.round_bf16 if out_dtype == torch.bfloat16 else oracle.round_f32
        for h in range(5):
            ref = np.concatenate([(oracle.pack_rows(A) if lay == cma.PACKED else A.ravel()) for A in om[h]])
            assert got.shape[1] == ref.size
            err = rel_l2(got[h], rnd(ref))
            assert err <= tol, (h, err)
            if out_dtype == torch.bfloat16:
                # stored values: at most one bf16 step from the oracle's rounding
                assert np.max(np.abs(got[h] - rnd(ref)) / np.maximum(np.abs(ref), 1e-30)) <= 2 ** -7
    # the bf16 map is the round-to-nearest-even of the very same fp32 value
    assert np.array_equal(outs[torch.bfloat16], oracle.round_bf16(outs[torch.float32]))


def test_attn_maps_decode_rows(cma):
    """Query rows at the end of longer key spans (bottom-right alignment)."""
    lq, lk = [1, 3, 1], [513, 77, 1000]
    say(f"attn_maps decode rows lq={lq} lk={lk}")
    x = synth.attention_inputs(7, 4, lq, d=128, k_lengths=lk)
    vl = cma.Varlen(x["cu_q"], x["cu_k"])
    for lay in (cma.PACKED, cma.DENSE):
        maps = cma.attn_maps(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_f32(x["scale"]), dev_f32(x["bias"]),
                             vl, layout=lay, out_dtype=torch.float32)
        torch.cuda.synchronize()
        got = host64(maps)
        om = oracle.attn_maps(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], x["cu_k"])
        for h in range(4):
            ref = np.concatenate([(oracle.pack_rows(A) if lay == cma.PACKED else A.ravel()) for A in om[h]])
            assert rel_l2(got[h], oracle.round_f32(ref)) <= 1e-5


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_attn_maps_single_rows(cma, d, out_bf16):
    """One query per sequence (decode): the single-row kernel, key counts from 1
    (only the sink key) to several thousand, both layouts."""
    lq, lk = [1, 1, 1, 1, 1], [1, 513, 64, 2001, 130]
    say(f"attn_maps single rows d={d} out_bf16={out_bf16} lk={lk}")
    x = synth.attention_inputs(17, 3, lq, d=d, k_lengths=lk)
    vl = cma.Varlen(x["cu_q"], x["cu_k"])
    om = oracle.attn_maps(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], x["cu_k"])
    for lay in (cma.PACKED, cma.DENSE):
        maps = cma.attn_maps(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_f32(x["scale"]), dev_f32(x["bias"]),
                             vl, layout=lay, out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
        torch.cuda.synchronize()
        got = host64(maps)
        for h in range(3):
            ref = np.concatenate([A.ravel() for A in om[h]])
            if out_bf16:
                assert rel_l2(got[h], oracle.round_bf16(ref)) <= 1e-2
            else:
                assert rel_l2(got[h], oracle.round_f32(ref)) <= 1e-5


# ------------------------------------------------------------------ cosine bf16
def test_head_map_cosine_bf16(cma):
    n = 200
    lens = [n]
    say("head_map_cosine bf16: 130 receivers x 37 senders over 20100 entries")
    xs = synth.attention_inputs(201, 37, lens, d=128, heads_per_layer=37)
    xr = synth.attention_inputs(202, 130, lens, d=128, heads_per_layer=65)
    S = np.stack([oracle.pack_rows(oracle.causal_map(f64(xs["q"][j]), f64(xs["k"][j]), xs["scale"][j], xs["bias"][j]))
                  for j in range(37)])
    R = np.stack([oracle.pack_rows(oracle.causal_map(f64(xr["q"][j]), f64(xr["k"][j]), xr["scale"][j], xr["bias"][j]))
                  for j in range(130)])
    Sb, Rb = oracle.round_bf16(S), oracle.round_bf16(R)
    L = Sb.shape[1]
    # pad rows to a multiple of 8 elements (16-byte aligned rows)
    Lp = (L + 7) // 8 * 8
    Sp = np.zeros((37, Lp)); Sp[:, :L] = Sb
    Rp = np.zeros((130, Lp)); Rp[:, :L] = Rb
    cos, arg, mar = cma.head_map_cosine(dev_bf16(bf16_bits_from_f64(Rp)), dev_bf16(bf16_bits_from_f64(Sp)),
                                        1, 130, 37, L, Lp, 0, Lp, 0)
    torch.cuda.synchronize()
    ocos, oarg, omar = oracle.head_map(Rb, Sb)
    assert rel_l2(host64(cos)[0], ocos) <= 1e-5
    big = omar > 1e-4
    assert np.array_equal(host64(arg)[0][big].astype(int), oarg[big])
    assert np.allclose(host64(mar)[0], omar, atol=1e-5)


def test_head_map_cosine_batched_strided(cma):
    """Batched problems addressed with head and batch strides, like per-prompt mapping."""
    B, Hr, Hs, L = 3, 20, 28, 4100
    say(f"head_map_cosine batched B={B} Hr={Hr} Hs={Hs} L={L}")
    r = np.random.default_rng(5)
    Lp = 4104
    # layout [head][batch][Lp] for both, like attn_maps output over several sequences
    R = r.uniform(0, 1, (Hr, B, Lp)) ** 4
    S = r.uniform(0, 1, (Hs, B, Lp)) ** 4
    R[..., L:] = 0
    S[..., L:] = 0
    Rb, Sb = oracle.round_bf16(R), oracle.round_bf16(S)
    cos, arg, mar = cma.head_map_cosine(dev_bf16(bf16_bits_from_f64(Rb)), dev_bf16(bf16_bits_from_f64(Sb)),
                                        B, Hr, Hs, L, B * Lp, Lp, B * Lp, Lp)
    torch.cuda.synchronize()
    for b in range(B):
        ocos, oarg, omar = oracle.head_map(Rb[:, b, :L], Sb[:, b, :L])
        assert rel_l2(host64(cos)[b], ocos) <= 1e-5
        big = omar > 1e-4
        assert np.array_equal(host64(arg)[b][big].astype(int), oarg[big])


@pytest.mark.parametrize("Hs,L", [(100, 1000), (200, 24676), (384, 50001)])
def test_head_map_cosine_sender_tiles(cma, Hs, L):
    """Sender counts that take the 4-, 8- and 12-tile forms of the Gram, with a
    ragged receiver tile, splits of one and of several full K-steps and a
    partial last step."""
    Hr = 150
    say(f"head_map_cosine Hr={Hr} Hs={Hs} L={L}")
    r = np.random.default_rng(Hs + L)
    Lp = (L + 7) // 8 * 8
    R = np.zeros((Hr, Lp)); R[:, :L] = r.uniform(0, 1, (Hr, L)) ** 4
    S = np.zeros((Hs, Lp)); S[:, :L] = r.uniform(0, 1, (Hs, L)) ** 4
    Rb, Sb = oracle.round_bf16(R), oracle.round_bf16(S)
    cos, arg, mar = cma.head_map_cosine(dev_bf16(bf16_bits_from_f64(Rb)), dev_bf16(bf16_bits_from_f64(Sb)),
                                        1, Hr, Hs, L, Lp, 0, Lp, 0)
    torch.cuda.synchronize()
    ocos, oarg, omar = oracle.head_map(Rb[:, :L], Sb[:, :L])
    assert rel_l2(host64(cos)[0], ocos) <= 1e-5
    big = omar > 1e-4
    assert np.array_equal(host64(arg)[0][big].astype(int), oarg[big])
    assert np.allclose(host64(mar)[0], omar, atol=1e-5)


# ------------------------------------------------------------------ block compress
@pytest.mark.parametrize("tau", [0.9, 1.0])
def test_block_compress_small(cma, tau):
    lens = [200, 64, 130, 5]
    H = 3
    say(f"block_compress lens={lens} H={H} tau={tau}")
    x = synth.attention_inputs(301, H, lens, d=128)
    vl = cma.Varlen(x["cu_q"], x["cu_k"])
    out = cma.block_compress(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_f32(x["scale"]), dev_f32(x["bias"]),
                             vl, tau, want_mass=True, want_stats=True)
    torch.cuda.synchronize()
    ref = oracle.block_compress(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], tau)
    nnz = int(out["nnz"].item())
    row_ptr = host64(out["row_ptr"]).astype(np.int64)
    col = host64(out["col_idx"][:nnz]).astype(np.int64)
    vals = blocks_from_panels(host64(out["vals"][:nnz]))
    assert rel_l2(host64(out["block_mass"]), ref["masses"]) <= 1e-5
    st = host64(out["row_stats"])
    assert rel_l2(st[..., 1], ref["row_stats"][..., 1]) <= 1e-5
    assert np.max(np.abs(st[..., 0] - ref["row_stats"][..., 0])) <= 1e-4
    exempt = 0
    for g in range(len(ref["kept"])):
        gk = list(col[row_ptr[g]: row_ptr[g + 1]])
        if ref["margins"][g] > 1e-4:
            assert gk == ref["kept"][g], g
        elif gk != ref["kept"][g]:
            exempt += 1
        if gk == ref["kept"][g] and gk:
            a, b = row_ptr[g], ref["row_ptr"][g]
            assert rel_l2(vals[a: a + len(gk)], ref["vals"][b: b + len(gk)]) <= 1e-2
    # every block-row, exempt or not: the kept set is the greedy prefix of the
    # library's own masses (where those masses decide it by more than 1e-6)
    R_list = [(n + 63) // 64 for n in lens]
    mass = host64(out["block_mass"])
    for h in range(H):
        _, bad, _ = greedy_mismatches(mass[h], row_ptr, col, R_list, tau, head_off=h * sum(R_list))
        assert not bad, (h, bad)
    say(f"  nnz={nnz} oracle={ref['nnz']} exempt rows differing={exempt}")


def test_block_compress_longest_sequence(cma):
    """A 16384-token sequence (256 block-rows, the longest the block table
    holds) beside a short one: sampled block-rows against the oracle."""
    lens = [16384, 300]
    H, tau = 2, 0.95
    say(f"block_compress lens={lens} H={H} tau={tau}")
    x = synth.attention_inputs(311, H, lens, d=128)
    vl = cma.Varlen(x["cu_q"], x["cu_k"])
    out = cma.block_compress(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_f32(x["scale"]), dev_f32(x["bias"]),
                             vl, tau, want_mass=True, want_stats=True)
    torch.cuda.synchronize()
    nnz = int(out["nnz"].item())
    row_ptr = host64(out["row_ptr"]).astype(np.int64)
    col = host64(out["col_idx"][:nnz]).astype(np.int64)
    mass = host64(out["block_mass"])
    stats = host64(out["row_stats"])
    R = [(n + 63) // 64 for n in lens]
    tri0 = lambda r: r * (r + 1) // 2
    checked = exempt = 0
    for h in range(H):
        for s, rows in ((0, (0, 1, 127, 128, 200, 254, 255)), (1, range(R[1]))):
            a, b = int(x["cu_q"][s]), int(x["cu_q"][s + 1])
            q, k = f64(x["q"][h, a:b]), f64(x["k"][h, a:b])
            g0 = h * sum(R) + sum(R[:s])
            m0 = h * sum(tri0(r) for r in R) + sum(tri0(r) for r in R[:s])  # mass offset of this (h, s)
            for r in rows:
                ref = oracle.compress_block_row(q, k, x["scale"][h], x["bias"][h], r, tau)
                mrow = mass.reshape(-1)[m0 + tri0(r): m0 + tri0(r) + r + 1]
                assert rel_l2(mrow, ref["masses"]) <= 1e-5, (h, s, r)
                rr = slice(a + 64 * r, min(a + 64 * r + 64, b))
                assert np.max(np.abs(stats[h, rr, 0] - ref["m"])) <= 1e-4
                assert rel_l2(stats[h, rr, 1], ref["l"]) <= 1e-5
                g = g0 + r
                cs = list(col[row_ptr[g]: row_ptr[g + 1]])
                if ref["margin"] > 1e-4:
                    assert cs == ref["kept"], (h, s, r)
                if cs == ref["kept"]:
                    v = blocks_from_panels(host64(out["vals"][row_ptr[g]: row_ptr[g + 1]]))
                    assert rel_l2(v, ref["blocks"]) <= 1e-2
                    checked += 1
                else:
                    exempt += 1
    for h in range(H):
        n_rows, bad, _ = greedy_mismatches(mass[h], row_ptr, col, R, tau, head_off=h * sum(R))
        assert not bad, (h, bad)
    say(f"  {checked} sampled block-rows equal, {exempt} exempt (margin <= 1e-4); greedy prefix of the "
        f"library's masses on all {H * sum(R)} block-rows")


# ------------------------------------------------------------------ mapped_av block-sparse
# v_heads: grouped V (receiver head h reads V head h // (n_recv // v_heads));
# None = one V per receiver head. The oracle gets V repeated per group.
@pytest.mark.parametrize("n_recv,v_layout,v_heads", [(24, "token", None), (7, "token", None), (24, "key", None),
                                                     (24, "tiled", None), (7, "tiled", None), (24, "token", 6),
                                                     (24, "tiled", 8), (24, "key", 3)])
def test_mapped_av_bsr_small(cma, n_recv, v_layout, v_heads):
    lens = [200, 64, 130]
    n_send = 32
    n_v = v_heads or n_recv
    say(f"mapped_av bsr lens={lens} n_send={n_send} n_recv={n_recv} v_heads={n_v} v_layout={v_layout}")
    x = synth.attention_inputs(401, n_send, lens, d=128)
    ref = oracle.block_compress(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], 0.9)
    M = synth.mix_matrix_learned(402, n_recv, n_send)
    T = int(x["cu_q"][-1])
    V = synth.values(403, n_v, T, 128)
    vl = cma.Varlen(x["cu_q"], x["cu_q"])
    src = dict(row_ptr=dev_i32(ref["row_ptr"]), col_idx=dev_i32(ref["col_idx"]),
               vals=dev_bf16(bf16_bits_from_f64(blocks_to_panels(ref["vals"]))), n_block_rows=ref["r_tot"])
    if v_layout == "key":
        O = cma.mapped_av(src, n_send, dev_f32(M), n_recv, dev_bf16(np.ascontiguousarray(V.transpose(0, 2, 1))), vl,
                          out_dtype=torch.bfloat16, v_layout=cma.V_KEY_MAJOR, v_heads=v_heads)
    elif v_layout == "tiled":
        O = cma.mapped_av(src, n_send, dev_f32(M), n_recv, dev_bf16(tile_v(V, lens, x["cu_q"])), vl,
                          out_dtype=torch.bfloat16, v_layout=cma.V_TILED, k_rows=T, v_heads=v_heads)
    else:
        O = cma.mapped_av(src, n_send, dev_f32(M), n_recv, dev_bf16(V), vl, out_dtype=torch.bfloat16,
                          v_heads=v_heads)
    torch.cuda.synchronize()
    got = host64(O)
    rows = [(s, r) for s in range(len(lens)) for r in range((lens[s] + 63) // 64)]
    Vr = np.repeat(f64(V), n_recv // n_v, axis=0)
    oo = oracle.mapped_av_bsr_rows(ref["row_ptr"], ref["col_idx"], ref["vals"], n_send, lens, M, Vr,
                                   x["cu_q"], rows)
    refO = np.zeros_like(got)
    for (s, r), o in oo.items():
        a = x["cu_q"][s] + 64 * r
        refO[:, a: a + o.shape[1]] = o
    assert rel_l2(got, oracle.round_bf16(refO)) <= 1e-2


# More senders than the fused pass stages at once (32): one pass per group of 32
# senders, each later pass adding into the output. The oracle mixes all senders
# at once; bf16 output is rounded once per group, so it keeps the bf16 bar.
@pytest.mark.parametrize("n_send,n_recv,out_f32", [(40, 12, True), (64, 24, False), (33, 7, True)])
def test_mapped_av_bsr_sender_groups(cma, n_send, n_recv, out_f32):
    lens = [200, 64, 130]
    say(f"mapped_av bsr sender groups lens={lens} n_send={n_send} n_recv={n_recv} out_f32={out_f32}")
    x = synth.attention_inputs(411, n_send, lens, d=128)
    ref = oracle.block_compress(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], 0.9)
    M = synth.mix_matrix_learned(412, n_recv, n_send)
    T = int(x["cu_q"][-1])
    V = synth.values(413, n_recv, T, 128)
    vl = cma.Varlen(x["cu_q"], x["cu_q"])
    src = dict(row_ptr=dev_i32(ref["row_ptr"]), col_idx=dev_i32(ref["col_idx"]),
               vals=dev_bf16(bf16_bits_from_f64(blocks_to_panels(ref["vals"]))), n_block_rows=ref["r_tot"])
    O = cma.mapped_av(src, n_send, dev_f32(M), n_recv, dev_bf16(V), vl,
                      out_dtype=torch.float32 if out_f32 else torch.bfloat16)
    torch.cuda.synchronize()
    got = host64(O)
    rows = [(s, r) for s in range(len(lens)) for r in range((lens[s] + 63) // 64)]
    oo = oracle.mapped_av_bsr_rows(ref["row_ptr"], ref["col_idx"], ref["vals"], n_send, lens, M, f64(V),
                                   x["cu_q"], rows)
    refO = np.zeros_like(got)
    for (s, r), o in oo.items():
        a = x["cu_q"][s] + 64 * r
        refO[:, a: a + o.shape[1]] = o
    assert rel_l2(got, refO if out_f32 else oracle.round_bf16(refO)) <= 1e-2


# ------------------------------------------------------------------ mapped_av, one sender per head
# Sender indices per (sequence, receiver head) as the cosine argmax gives them:
# O_h = A_{idx[h]} V_{h // g}. The oracle gets the one-hot M; the general path
# with that M must give the same bits (its mix of a one-hot row is exact).
@pytest.mark.parametrize("lens,n_recv,v_layout,v_heads,shared,out_f32", [
    ([200, 64, 130], 64, "token", None, False, False),
    ([130, 0, 64, 257], 13, "key", None, False, True),
    ([200, 64, 130], 64, "tiled", 16, True, False),
    ([64 * 9 + 5], 24, "token", 8, False, True),
])
def test_mapped_av_indexed_small(cma, lens, n_recv, v_layout, v_heads, shared, out_f32):
    n_send = 28
    n_v = v_heads or n_recv
    say(f"mapped_av indexed lens={lens} n_send={n_send} n_recv={n_recv} v_heads={n_v} v_layout={v_layout} "
        f"shared={shared} out_f32={out_f32}")
    x = synth.attention_inputs(431, n_send, lens, d=128)
    ref = oracle.block_compress(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], 0.9)
    S = len(lens)
    rng = np.random.default_rng(432)
    idx = rng.integers(0, n_send, size=(1 if shared else S, n_recv)).astype(np.int32)
    if n_recv == 13:
        idx[:, 3], idx[:, 7] = -1, n_send  # out of range: zero rows
    M = np.zeros((idx.shape[0], n_recv, n_send))
    for b in range(idx.shape[0]):
        for h in range(n_recv):
            if 0 <= idx[b, h] < n_send:
                M[b, h, idx[b, h]] = 1.0
    T = int(x["cu_q"][-1])
    V = synth.values(433, n_v, T, 128)
    vl = cma.Varlen(x["cu_q"], x["cu_q"])
    src = dict(row_ptr=dev_i32(ref["row_ptr"]), col_idx=dev_i32(ref["col_idx"]),
               vals=dev_bf16(bf16_bits_from_f64(blocks_to_panels(ref["vals"]))), n_block_rows=ref["r_tot"])
    od = torch.float32 if out_f32 else torch.bfloat16
    if v_layout == "key":
        vv, kw = dev_bf16(np.ascontiguousarray(V.transpose(0, 2, 1))), dict(v_layout=cma.V_KEY_MAJOR)
    elif v_layout == "tiled":
        vv, kw = dev_bf16(tile_v(V, lens, x["cu_q"])), dict(v_layout=cma.V_TILED, k_rows=T)
    else:
        vv, kw = dev_bf16(V), {}
    O = cma.mapped_av(src, n_send, dev_i32(idx), n_recv, vv, vl, out_dtype=od, v_heads=v_heads, **kw)
    Og = cma.mapped_av(src, n_send, dev_f32(M), n_recv, vv, vl, out_dtype=od, v_heads=v_heads, **kw)
    torch.cuda.synchronize()
    assert torch.equal(O, Og)
    got = host64(O)
    rows = [(s_, r) for s_ in range(S) for r in range((lens[s_] + 63) // 64)]
    Vr = np.repeat(f64(V), n_recv // n_v, axis=0)
    oo = oracle.mapped_av_bsr_rows(ref["row_ptr"], ref["col_idx"], ref["vals"], n_send, lens, M, Vr,
                                   x["cu_q"], rows)
    refO = np.zeros_like(got)
    for (s_, r), o in oo.items():
        a = x["cu_q"][s_] + 64 * r
        refO[:, a: a + o.shape[1]] = o
    if out_f32:
        assert rel_l2(got, refO) <= 1e-5
    else:
        assert rel_l2(got, oracle.round_bf16(refO)) <= 1e-2
    if n_recv == 13:
        assert not got[[3, 7]].any()


@pytest.mark.parametrize("key_major", [False, True])
def test_tile_v(cma, key_major):
    """cma.tile_v writes the documented tiled layout (bit for bit, zeros past each
    sequence's end), and the fused pass on the tiled copy equals the one that tiles
    V itself."""
    lens = [200, 64, 130, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, R = int(cu[-1]), sum((n + 63) // 64 for n in lens)
    say(f"tile_v lens={lens} key_major={key_major}")
    V = synth.values(441, 6, T, 128)
    vl = cma.Varlen(cu, cu)
    if key_major:
        vv, lay = dev_bf16(np.ascontiguousarray(V.transpose(0, 2, 1))), cma.V_KEY_MAJOR
    else:
        vv, lay = dev_bf16(V), cma.V_TOKEN_MAJOR
    got = cma.tile_v(vv, vl, R, v_layout=lay)
    torch.cuda.synchronize()
    assert np.array_equal(host64(got), f64(tile_v(V, lens, cu)))
    # the fused pass: tiled by the caller vs tiled inside the call
    n_send = 8
    x = synth.attention_inputs(442, n_send, lens, d=128)
    ref = oracle.block_compress(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], 0.9)
    src = dict(row_ptr=dev_i32(ref["row_ptr"]), col_idx=dev_i32(ref["col_idx"]),
               vals=dev_bf16(bf16_bits_from_f64(blocks_to_panels(ref["vals"]))), n_block_rows=ref["r_tot"])
    M = dev_f32(synth.mix_matrix_learned(443, 6, n_send))
    O1 = cma.mapped_av(src, n_send, M, 6, vv, vl, v_layout=lay)
    O2 = cma.mapped_av(src, n_send, M, 6, got, vl, v_layout=cma.V_TILED, k_rows=T)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)


def test_mapped_av_two_receivers_stacked(cma):
    """Two receivers served from one sender state: their heads stacked in one call
    (M rows and V heads concatenated, each with its own grouped V) give exactly the
    outputs of two separate calls, and match the oracle."""
    lens = [200, 64, 130]
    n_send = 32
    say(f"mapped_av two receivers stacked lens={lens}")
    x = synth.attention_inputs(411, n_send, lens, d=128)
    ref = oracle.block_compress(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], 0.9)
    T = int(x["cu_q"][-1])
    vl = cma.Varlen(x["cu_q"], x["cu_q"])
    src = dict(row_ptr=dev_i32(ref["row_ptr"]), col_idx=dev_i32(ref["col_idx"]),
               vals=dev_bf16(bf16_bits_from_f64(blocks_to_panels(ref["vals"]))), n_block_rows=ref["r_tot"])
    # receiver 1: 24 heads, 8 V heads; receiver 2: 12 heads, 4 V heads (group 3 in both)
    M1, M2 = synth.mix_matrix_learned(412, 24, n_send), synth.mix_matrix_learned(413, 12, n_send)
    V1, V2 = synth.values(414, 8, T, 128), synth.values(415, 4, T, 128)
    O1 = cma.mapped_av(src, n_send, dev_f32(M1), 24, dev_bf16(V1), vl, v_heads=8)
    O2 = cma.mapped_av(src, n_send, dev_f32(M2), 12, dev_bf16(V2), vl, v_heads=4)
    Ms = np.concatenate([M1, M2], axis=1)  # [1, 36, n_send]
    Os = cma.mapped_av(src, n_send, dev_f32(Ms), 36, dev_bf16(np.concatenate([V1, V2])), vl, v_heads=12)
    torch.cuda.synchronize()
    assert torch.equal(Os[:24], O1) and torch.equal(Os[24:], O2)
    rows = [(s_, r) for s_ in range(len(lens)) for r in range((lens[s_] + 63) // 64)]
    Vr = np.repeat(f64(np.concatenate([V1, V2])), 3, axis=0)
    oo = oracle.mapped_av_bsr_rows(ref["row_ptr"], ref["col_idx"], ref["vals"], n_send, lens, Ms, Vr, x["cu_q"], rows)
    got = host64(Os)
    refO = np.zeros_like(got)
    for (s_, r), o in oo.items():
        a0 = x["cu_q"][s_] + 64 * r
        refO[:, a0: a0 + o.shape[1]] = o
    assert rel_l2(got, oracle.round_bf16(refO)) <= 1e-2


@pytest.mark.parametrize("key_major,v_heads", [(False, None), (True, None), (False, 3), (True, 2)])
def test_mapped_av_dense_decode_rows(cma, key_major, v_heads):
    """Decode rows: one query per sequence over long contexts, one-hot and learned M;
    optionally grouped V (the oracle gets V repeated per group)."""
    lq, lk = [1, 1, 2], [1000, 513, 300]
    n_send, n_recv = 28, 6
    n_v = v_heads or n_recv
    say(f"mapped_av dense decode rows lq={lq} lk={lk} key_major={key_major} v_heads={n_v}")
    x = synth.attention_inputs(501, n_send, lq, d=128, k_lengths=lk)
    om = oracle.attn_maps(f64(x["q"]), f64(x["k"]), x["scale"], x["bias"], x["cu_q"], x["cu_k"])
    maps = np.stack([np.concatenate([A.ravel() for A in om[j]]) for j in range(n_send)])
    mapsr = oracle.round_f32(maps)
    Tk = int(x["cu_k"][-1])
    V = synth.values(502, n_v, Tk, 128)
    Vr = np.repeat(f64(V), n_recv // n_v, axis=0)
    vl = cma.Varlen(x["cu_q"], x["cu_k"])
    Ml = synth.mix_matrix_learned(503, n_recv, n_send, n_batch=3)
    Moh = oracle.onehot_mix(np.array([[5, 0, 27, 3, 3, 9], [1, 2, 3, 4, 5, 6], [0, 0, 0, 0, 0, 0]]), n_send).astype(np.float32)
    for M in (Ml, Moh):
        vd = dev_bf16(np.ascontiguousarray(V.transpose(0, 2, 1))) if key_major else dev_bf16(V)
        O = cma.mapped_av(("dense", dev_f32(mapsr), cma.DENSE), n_send, dev_f32(M), n_recv, vd, vl,
                          out_dtype=torch.float32, q_rows=int(x["cu_q"][-1]),
                          v_layout=cma.V_KEY_MAJOR if key_major else cma.V_TOKEN_MAJOR, v_heads=v_heads)
        torch.cuda.synchronize()
        got = host64(O)
        off = 0
        for s_ in range(3):
            A = mapsr[:, off: off + lq[s_] * lk[s_]].reshape(n_send, lq[s_], lk[s_])
            off += lq[s_] * lk[s_]
            ref = oracle.mapped_av_dense(A, M[s_].astype(np.float64), Vr[:, x["cu_k"][s_]: x["cu_k"][s_] + lk[s_]])
            assert rel_l2(got[:, x["cu_q"][s_]: x["cu_q"][s_] + lq[s_]], oracle.round_f32(ref)) <= 1e-5


def test_onehot_and_layers(cma):
    arg = dev_i32(np.array([[2, 0, 5], [1, 1, 0]]))
    M = host64(cma.onehot_mix(arg, 4))
    exp = np.zeros((2, 3, 4))
    for b, row in enumerate([[2, 0, 5], [1, 1, 0]]):
        for h, j in enumerate(row):
            if j < 4:
                exp[b, h, j] = 1.0  # index 5 is out of range: all-zero row
    assert np.array_equal(M, exp)
    assert cma.mapped_layers(80, 0.5) == oracle.mapped_layers(80, 0.5)
