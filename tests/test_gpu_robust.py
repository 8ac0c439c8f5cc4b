"""GPU tests of properties beyond element-wise parity: bitwise determinism of the
whole chain, the block-sparse capacity protocol, head dimension 64 in the
compressor, long-context decode rows (IAM's 8192 + 512 setting) and rows longer
than the maxima a caller passed, and non-finite inputs staying local to the rows
they touch. Expected values come from the float64 oracle or from the library's
own earlier outputs (determinism, locality), never from stored GPU results."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import (dev_bf16, dev_f32, dev_i32, f64, host64, rel_l2, blocks_from_panels,
                            greedy_mismatches)

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


def _chain(cma, xs, xr, lens, V, M, arg_heads):
    """Every stage once: maps, cosine head map, compression, the general and the
    indexed fused pass, and decode rows with their dense mapped x V."""
    vl = cma.Varlen(xs["cu_q"], xs["cu_k"])
    q, k = dev_bf16(xs["q"]), dev_bf16(xs["k"])
    sc, bi = dev_f32(xs["scale"]), dev_f32(xs["bias"])
    sm = cma.attn_maps(q, k, sc, bi, vl)
    rm = cma.attn_maps(dev_bf16(xr["q"]), dev_bf16(xr["k"]), dev_f32(xr["scale"]), dev_f32(xr["bias"]), vl)
    # cosine head map on the first sequence's maps (rows padded to 16-byte strides)
    L0 = lens[0] * (lens[0] + 1) // 2
    Lp = (L0 + 7) // 8 * 8
    Hs, Hr = xs["q"].shape[0], xr["q"].shape[0]
    sp = torch.zeros((Hs, Lp), dtype=torch.bfloat16, device="cuda")
    rp = torch.zeros((Hr, Lp), dtype=torch.bfloat16, device="cuda")
    sp[:, :L0] = sm[:, :L0]
    rp[:, :L0] = rm[:, :L0]
    cos, arg, mar = cma.head_map_cosine(rp, sp, 1, Hr, Hs, L0, Lp, 0, Lp, 0)
    bsr = cma.block_compress(q, k, sc, bi, vl, 0.9, want_mass=True, want_stats=True)
    v = dev_bf16(V)
    O = cma.mapped_av(bsr, Hs, dev_f32(M), Hr, v, vl)
    Oi = cma.mapped_av(bsr, Hs, dev_i32(arg_heads), Hr, v, vl)
    # decode rows: the last token of every sequence as a query over its prefix
    n_s = len(lens)
    vl_d = cma.Varlen(np.arange(n_s + 1), xs["cu_k"], used_q=[1] * n_s, used_k=lens)
    qd = q[:, torch.as_tensor(xs["cu_q"][1:] - 1, dtype=torch.long, device="cuda")].contiguous()
    rows = cma.attn_maps(qd, k, sc, bi, vl_d, layout=cma.DENSE, out_dtype=torch.float32)
    od = cma.mapped_av(("dense", rows, cma.DENSE), Hs, dev_f32(M), Hr, v, vl_d, q_rows=n_s)
    torch.cuda.synchronize()
    return dict(sm=sm, rm=rm, cos=cos, arg=arg, mar=mar, row_ptr=bsr["row_ptr"], nnz=bsr["nnz"],
                col=bsr["col_idx"], vals=bsr["vals"], mass=bsr["block_mass"], stats=bsr["row_stats"],
                O=O, Oi=Oi, rows=rows, od=od)


def test_determinism_full_chain(cma):
    """Two runs of the whole chain on the same inputs give identical bits in every
    output (fixed-order reductions, no floating-point atomics)."""
    lens = [1000, 64, 777]
    Hs, Hr = 16, 24
    say(f"determinism: lens={lens} Hs={Hs} Hr={Hr}")
    xs = synth.attention_inputs(901, Hs, lens, d=128)
    xr = synth.attention_inputs(902, Hr, lens, d=128)
    V = synth.values(903, Hr, int(xs["cu_q"][-1]), 128)
    M = synth.mix_matrix_learned(904, Hr, Hs)
    arg_heads = (np.arange(Hr) * 5 % Hs).astype(np.int32)[None, :]
    a = _chain(cma, xs, xr, lens, V, M, arg_heads)
    b = _chain(cma, xs, xr, lens, V, M, arg_heads)
    nnz = int(a["nnz"].item())
    assert nnz == int(b["nnz"].item())
    for key in a:
        x, y = a[key], b[key]
        if key in ("col", "vals"):
            x, y = x[:nnz], y[:nnz]
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y), key
    say(f"  every output bitwise equal over two runs (nnz={nnz})")


def test_capacity_overflow_and_retry(cma):
    """nnz > capacity: row_ptr and nnz are written, col_idx and vals are left
    untouched; a retry with capacity = nnz gives the full result."""
    lens = [300, 130]
    H = 4
    say(f"capacity protocol: lens={lens} H={H}")
    x = synth.attention_inputs(911, H, lens, d=128)
    vl = cma.Varlen(x["cu_q"], x["cu_k"])
    q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
    sc, bi = dev_f32(x["scale"]), dev_f32(x["bias"])
    full = cma.block_compress(q, k, sc, bi, vl, 0.9)
    torch.cuda.synchronize()
    nnz = int(full["nnz"].item())
    cap = nnz // 2
    sentinel_c, sentinel_v = -7, torch.tensor(-3.0, dtype=torch.bfloat16)
    small = dict(row_ptr=torch.full((H * vl.n_block_rows + 1,), -1, dtype=torch.int32, device="cuda"),
                 col_idx=torch.full((cap,), sentinel_c, dtype=torch.int32, device="cuda"),
                 vals=torch.full((cap, 64, 64), float(sentinel_v), dtype=torch.bfloat16, device="cuda"),
                 nnz=torch.zeros(1, dtype=torch.int32, device="cuda"), capacity=cap)
    out = cma.block_compress(q, k, sc, bi, vl, 0.9, bsr=small)
    torch.cuda.synchronize()
    assert int(out["nnz"].item()) == nnz > cap
    assert torch.equal(out["row_ptr"], full["row_ptr"])
    assert bool((small["col_idx"] == sentinel_c).all())
    assert bool((small["vals"] == sentinel_v).all())
    retry = cma.block_compress(q, k, sc, bi, vl, 0.9, capacity=nnz)
    torch.cuda.synchronize()
    assert torch.equal(retry["row_ptr"], full["row_ptr"])
    assert torch.equal(retry["col_idx"][:nnz], full["col_idx"][:nnz])
    assert torch.equal(retry["vals"][:nnz], full["vals"][:nnz])
    say(f"  nnz={nnz} > capacity={cap}: arrays untouched; retry equal")


@pytest.mark.parametrize("tau", [0.9, 1.0])
def test_block_compress_d64(cma, tau):
    """Head dimension 64 through both compression phases, ragged varlen."""
    lens = [200, 64, 130, 5, 0]
    H = 3
    say(f"block_compress d=64 lens={lens} H={H} tau={tau}")
    x = synth.attention_inputs(921, H, lens, d=64)
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
    T = int(x["cu_q"][-1])
    assert rel_l2(st[:, :T, 1], ref["row_stats"][:, :T, 1]) <= 1e-5
    assert np.max(np.abs(st[:, :T, 0] - ref["row_stats"][:, :T, 0])) <= 1e-4
    same = 0
    for g in range(len(ref["kept"])):
        gk = list(col[row_ptr[g]: row_ptr[g + 1]])
        if ref["margins"][g] > 1e-4:
            assert gk == ref["kept"][g], g
        if gk == ref["kept"][g] and gk:
            a, b = row_ptr[g], ref["row_ptr"][g]
            assert rel_l2(vals[a: a + len(gk)], ref["vals"][b: b + len(gk)]) <= 1e-2
            same += 1
    R_list = [(n + 63) // 64 for n in lens]
    mass = host64(out["block_mass"])
    for h in range(H):
        _, bad, _ = greedy_mismatches(mass[h], row_ptr, col, R_list, tau, head_off=h * sum(R_list))
        assert not bad
    say(f"  nnz={nnz} (oracle {ref['nnz']}), {same} block-rows with equal kept sets compared")


# ------------------------------------------------------------------ IAM long-context decode
@pytest.fixture(scope="module")
def long_dec():
    x = synth.long_decode()
    return x


@pytest.mark.parametrize("step", [0, 255, 511])
def test_long_context_decode_rows(cma, long_dec, step):
    """IAM's 8192 + 512 decode at batch 4: at generation step t every prompt's new
    token attends over 8193 + t keys. Sender rows (the single-row kernel) and the
    mapped x V of 24 receiver heads with the learned M and with the one-hot head
    map (the dense pass, whose mixed-row window holds 8192 keys, so these
    contexts take two windows), against the oracle on sampled heads."""
    x = long_dec
    P, n, ctx, Hs, Hr = x["n_prompts"], x["n"], x["ctx"], x["n_send"], x["n_recv"]
    nk = n + 1 + step
    say(f"long decode: step {step}, {P} prompts at context {nk}, Hs={Hs} Hr={Hr}")
    vl = cma.Varlen(np.arange(P + 1), x["cu_k"], used_q=[1] * P, used_k=[nk] * P)
    k, sc, bi = dev_bf16(x["send_k"]), dev_f32(x["send_scale"]), dev_f32(x["send_bias"])
    qd = dev_bf16(np.ascontiguousarray(x["dec_q"][step]))
    rows = cma.attn_maps(qd, k, sc, bi, vl, layout=cma.DENSE, out_dtype=torch.float32)
    v = dev_bf16(x["v"])
    onehot = (np.arange(Hr) * 7 % Hs)
    Mo = oracle.onehot_mix(np.tile(onehot, (P, 1)), Hs).astype(np.float32)
    O_l = cma.mapped_av(("dense", rows, cma.DENSE), Hs, dev_f32(x["M"]), Hr, v, vl, q_rows=P)
    O_o = cma.mapped_av(("dense", rows, cma.DENSE), Hs, dev_f32(Mo), Hr, v, vl, q_rows=P,
                        out_dtype=torch.float32)
    # the same launches without a workspace: each row in one workgroup
    O_l1 = cma.mapped_av(("dense", rows, cma.DENSE), Hs, dev_f32(x["M"]), Hr, v, vl, q_rows=P, split_rows=False)
    O_o1 = cma.mapped_av(("dense", rows, cma.DENSE), Hs, dev_f32(Mo), Hr, v, vl, q_rows=P,
                         out_dtype=torch.float32, split_rows=False)
    torch.cuda.synchronize()
    R = host64(rows).reshape(Hs, P, nk)
    Ol, Oo = host64(O_l), host64(O_o)
    # split and unsplit rows add the same terms in different orders
    assert rel_l2(host64(O_o1), Oo) <= 1e-6
    assert rel_l2(host64(O_l1), Ol) <= 1e-2
    M = x["M"][0].astype(np.float64)
    for p in (0, P - 1):
        ks = slice(int(x["cu_k"][p]), int(x["cu_k"][p]) + nk)
        A = np.stack([oracle.causal_map(f64(x["dec_q"][step, j, p][None, :]), f64(x["send_k"][j, ks]),
                                        x["send_scale"][j], x["send_bias"][j])[0] for j in range(Hs)])
        assert rel_l2(R[:, p], oracle.round_f32(A)) <= 1e-5, p
        Vp = f64(x["v"][:, ks])
        for h in (0, 5, Hr - 1):
            ref_l = (M[h] @ A) @ Vp[h]
            assert rel_l2(Ol[h, p], oracle.round_bf16(ref_l)) <= 1e-2, (p, h)
            ref_o = A[onehot[h]] @ Vp[h]
            assert rel_l2(Oo[h, p], oracle.round_f32(ref_o)) <= 1e-5, (p, h)
    say("  sender rows (fp32, 1e-5) and mapped x V (learned M bf16 1e-2, one-hot fp32 1e-5) match")


def test_rows_longer_than_the_stated_maximum(cma, long_dec):
    """A caller that passes max_seqlen_k below a row's true length still gets the
    whole row: the single-row kernel's LDS holds max_seqlen_k keys and the longer
    row is computed window by window (three windows here)."""
    x = long_dec
    P, n, Hs = x["n_prompts"], x["n"], x["n_send"]
    nk = n + 512
    vl = cma.Varlen(np.arange(P + 1), x["cu_k"], used_q=[1] * P, used_k=[nk] * P)
    k, sc, bi = dev_bf16(x["send_k"]), dev_f32(x["send_scale"]), dev_f32(x["send_bias"])
    qd = dev_bf16(np.ascontiguousarray(x["dec_q"][511]))
    full = cma.attn_maps(qd, k, sc, bi, vl, layout=cma.DENSE, out_dtype=torch.float32)
    vl.max_k = 3000  # understated: rows of 8704 keys take three windows of 3000
    part = cma.attn_maps(qd, k, sc, bi, vl, layout=cma.DENSE, out_dtype=torch.float32)
    torch.cuda.synchronize()
    R = host64(part).reshape(Hs, P, nk)
    for p in (0, P - 1):
        ks = slice(int(x["cu_k"][p]), int(x["cu_k"][p]) + nk)
        for j in (0, 13, Hs - 1):
            a = oracle.causal_map(f64(x["dec_q"][511, j, p][None, :]), f64(x["send_k"][j, ks]),
                                  x["send_scale"][j], x["send_bias"][j])[0]
            assert rel_l2(R[j, p], oracle.round_f32(a)) <= 1e-5
    assert rel_l2(host64(part), host64(full)) <= 1e-6
    say("  understated max_seqlen_k: rows of 8704 keys computed in windows, equal to the oracle")


# ------------------------------------------------------------------ non-finite inputs
def test_nonfinite_inputs_stay_local(cma):
    """A NaN in one query row of one head makes only that head's map row (and
    that block-row's statistics) non-finite; every other head and row keeps the
    bits of a clean run, and the kept sets stay valid. A NaN in one receiver V
    entry changes only the rows of that head that read it."""
    lens = [300, 200]
    H = 4
    say(f"non-finite: lens={lens} H={H}")
    x = synth.attention_inputs(931, H, lens, d=128)
    vl = cma.Varlen(x["cu_q"], x["cu_k"])
    qn = x["q"].copy()
    bad_row = 130  # sequence 0, block-row 2
    qn[1, bad_row, 5] = 0x7FC0  # bf16 NaN
    k, sc, bi = dev_bf16(x["k"]), dev_f32(x["scale"]), dev_f32(x["bias"])
    clean = cma.attn_maps(dev_bf16(x["q"]), k, sc, bi, vl, layout=cma.DENSE, out_dtype=torch.float32)
    dirty = cma.attn_maps(dev_bf16(qn), k, sc, bi, vl, layout=cma.DENSE, out_dtype=torch.float32)
    c_b = cma.block_compress(dev_bf16(x["q"]), k, sc, bi, vl, 0.9)
    d_b = cma.block_compress(dev_bf16(qn), k, sc, bi, vl, 0.9)
    torch.cuda.synchronize()
    n0 = lens[0]
    C, D = host64(clean), host64(dirty)
    assert np.array_equal(C[[0, 2, 3]], D[[0, 2, 3]])
    row = D[1, bad_row * n0: (bad_row + 1) * n0]
    assert not np.isfinite(row[: bad_row + 1]).any()
    mask = np.ones(D.shape[1], dtype=bool)
    mask[bad_row * n0: (bad_row + 1) * n0] = False
    assert np.array_equal(C[1][mask], D[1][mask])
    # compression: other heads bitwise equal; the affected head's kept sets valid
    R_list = [(n + 63) // 64 for n in lens]
    R_tot = sum(R_list)
    rp_c, rp_d = host64(c_b["row_ptr"]).astype(np.int64), host64(d_b["row_ptr"]).astype(np.int64)
    nnz_d = int(d_b["nnz"].item())
    col_c = host64(c_b["col_idx"][: int(c_b["nnz"].item())]).astype(np.int64)
    col_d = host64(d_b["col_idx"][:nnz_d]).astype(np.int64)
    for h in range(H):
        for g in range(h * R_tot, (h + 1) * R_tot):
            kd = col_d[rp_d[g]: rp_d[g + 1]]
            r = g - h * R_tot
            r_loc = r if r < R_list[0] else r - R_list[0]
            assert len(kd) >= 1 and np.all(np.diff(kd) > 0) and kd[0] >= 0 and kd[-1] <= r_loc
            if h != 1 or r != 2:
                assert np.array_equal(kd, col_c[rp_c[g]: rp_c[g + 1]]), (h, g)
    # V: a NaN at key t of receiver head 2 reaches only that head's rows from the
    # first row of t's block-row on (a kept block multiplies all of its keys, and
    # 0 x NaN is NaN, as in the float64 definition)
    Hs, Hr = H, 3
    M = synth.mix_matrix_learned(932, Hr, Hs)
    V = synth.values(933, Hr, int(x["cu_q"][-1]), 128)
    Vn = V.copy()
    t = 150
    Vn[2, t, 7] = 0x7FC0
    O_c = cma.mapped_av(c_b, Hs, dev_f32(M), Hr, dev_bf16(V), vl)
    O_d = cma.mapped_av(c_b, Hs, dev_f32(M), Hr, dev_bf16(Vn), vl)
    torch.cuda.synchronize()
    Oc, Od = host64(O_c), host64(O_d)
    assert np.array_equal(Oc[:2], Od[:2])
    assert np.array_equal(Oc[2, : t // 64 * 64], Od[2, : t // 64 * 64])
    assert not np.isfinite(Od[2, t]).all()
    assert np.array_equal(Oc[2, n0:], Od[2, n0:])
    say("  non-finite values stay in the rows that read them")
