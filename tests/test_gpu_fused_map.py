"""GPU parity of the fused head mapping (receiver maps formed on chip inside the
Gram producer, never stored) against the float64 oracle's cosine of the stored
(bf16-rounded) maps, and against the unfused library path (maps stored, then the
Gram). Tolerances: cosines relative L2 1e-5, argmax exact where the oracle's
top-1 minus top-2 margin exceeds 1e-4."""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import dev_bf16, dev_f32, f64, host64, rel_l2

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


@pytest.mark.parametrize("lens,Hr,Hs", [([200, 64, 130], 40, 150), ([512], 24, 32), ([37, 96], 7, 5)])
def test_fused_head_map_small(cma, lens, Hr, Hs):
    say(f"fused head map lens={lens} Hr={Hr} Hs={Hs}")
    xs = synth.attention_inputs(1001, Hs, lens, d=128)
    xr = synth.attention_inputs(1002, Hr, lens, d=128)
    vl = cma.Varlen(xs["cu_q"], xs["cu_k"])
    sm = cma.attn_maps(dev_bf16(xs["q"]), dev_bf16(xs["k"]), dev_f32(xs["scale"]), dev_f32(xs["bias"]), vl,
                       layout=cma.DENSE)
    rq, rk = dev_bf16(xr["q"]), dev_bf16(xr["k"])
    rsc, rbi = dev_f32(xr["scale"]), dev_f32(xr["bias"])
    cos, arg, mar = cma.head_map_fused(rq, rk, rsc, rbi, sm, Hs, vl)
    # the unfused library path: receiver maps stored (dense, same values), then the Gram per sequence
    rm = cma.attn_maps(rq, rk, rsc, rbi, vl, layout=cma.DENSE)
    torch.cuda.synchronize()
    gcos, garg, gmar = host64(cos), host64(arg).astype(int), host64(mar)
    off = 0
    for b, n in enumerate(lens):
        S = np.stack([oracle.round_bf16(oracle.causal_map(f64(xs["q"][j, xs["cu_q"][b]: xs["cu_q"][b] + n]),
                                                          f64(xs["k"][j, xs["cu_k"][b]: xs["cu_k"][b] + n]),
                                                          xs["scale"][j], xs["bias"][j])).ravel() for j in range(Hs)])
        R = np.stack([oracle.round_bf16(oracle.causal_map(f64(xr["q"][h, xr["cu_q"][b]: xr["cu_q"][b] + n]),
                                                          f64(xr["k"][h, xr["cu_k"][b]: xr["cu_k"][b] + n]),
                                                          xr["scale"][h], xr["bias"][h])).ravel() for h in range(Hr)])
        ocos, oarg, omar = oracle.head_map(R, S)
        assert rel_l2(gcos[b], ocos) <= 1e-5, b
        big = omar > 1e-4
        assert np.array_equal(garg[b][big], oarg[big]), b
        assert np.allclose(gmar[b], omar, atol=1e-5)
        # against the stored-map path of the library on the same sequence
        L = n * n
        Lp = (L + 7) // 8 * 8
        sp = torch.zeros((Hs, Lp), dtype=torch.bfloat16, device="cuda")
        rp = torch.zeros((Hr, Lp), dtype=torch.bfloat16, device="cuda")
        sp[:, :L] = sm[:, off: off + L]
        rp[:, :L] = rm[:, off: off + L]
        c2, a2, _ = cma.head_map_cosine(rp, sp, 1, Hr, Hs, L, Lp, 0, Lp, 0)
        torch.cuda.synchronize()
        assert rel_l2(gcos[b], host64(c2)[0]) <= 1e-5
        off += L
    say(f"  cosines and decided argmaxes match the oracle and the stored-map path")


def test_fused_head_map_iam_full(cma):
    """The IAM head-mapping workload: 2560 large-model maps against 336 small-model
    maps of one 512-token prompt; the sender maps are stored (dense bf16), the
    receivers' 2560 maps never are. Sampled receivers against the oracle, and
    every receiver's argmax is its row's maximum."""
    t0 = time.time()
    x = synth.cfg2()
    Hs, Hr, n = x["n_send"], x["n_recv"], x["n"]
    vl = cma.Varlen(x["cu"])
    sm = cma.attn_maps(dev_bf16(x["send_q"]), dev_bf16(x["send_k"]), dev_f32(x["send_scale"]),
                       dev_f32(x["send_bias"]), vl, layout=cma.DENSE)
    cos, arg, mar = cma.head_map_fused(dev_bf16(x["recv_q"]), dev_bf16(x["recv_k"]), dev_f32(x["recv_scale"]),
                                       dev_f32(x["recv_bias"]), sm, Hs, vl)
    torch.cuda.synchronize()
    say(f"cfg2 fused: GPU done at {time.time() - t0:.1f}s")
    S = np.stack([oracle.round_bf16(oracle.pack_rows(oracle.causal_map(
        f64(x["send_q"][j]), f64(x["send_k"][j]), x["send_scale"][j], x["send_bias"][j]))) for j in range(Hs)])
    rs = np.linspace(0, Hr - 1, 24).astype(int)
    R = np.stack([oracle.round_bf16(oracle.pack_rows(oracle.causal_map(
        f64(x["recv_q"][h]), f64(x["recv_k"][h]), x["recv_scale"][h], x["recv_bias"][h]))) for h in rs])
    ocos, oarg, omar = oracle.head_map(R, S)
    gcos, garg = host64(cos)[0], host64(arg)[0].astype(int)
    assert rel_l2(gcos[rs], ocos) <= 1e-5
    big = omar > 1e-4
    assert np.array_equal(garg[rs][big], oarg[big])
    assert garg.min() >= 0 and garg.max() < Hs
    assert np.all(gcos[np.arange(Hr), garg] >= gcos.max(axis=1) - 1e-7)
    say(f"cfg2 fused: {big.sum()}/{len(rs)} sampled heads above the margin line, all argmax equal; "
        f"total {time.time() - t0:.1f}s")
