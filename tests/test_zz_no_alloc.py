"""The allocation-free compression entry point (cma_block_compress_noalloc),
called through the C ABI, gives the same bits as cma_block_compress with a
caller workspace, on two calls in a row (the second smaller, so the shared
static scratch holds the first call's contents)."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev_bf16, dev_f32

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


def _outputs(cma, H, vl, T, cap):
    dev = "cuda"
    n_tri = int(sum(((int(n) + 63) // 64) * ((int(n) + 63) // 64 + 1) // 2 for n in vl.lens_q))
    return dict(row_ptr=torch.full((H * vl.n_block_rows + 1,), -5, dtype=torch.int32, device=dev),
                col_idx=torch.full((cap,), -5, dtype=torch.int32, device=dev),
                vals=torch.zeros((cap, 64, 64), dtype=torch.bfloat16, device=dev),
                nnz=torch.zeros(1, dtype=torch.int32, device=dev),
                mass=torch.zeros((H, n_tri), dtype=torch.float32, device=dev),
                stats=torch.zeros((H, T, 2), dtype=torch.float32, device=dev))


def _call(cma, fn, x, vl, H, tau, out, ws=None):
    lib = cma.load_library()
    q, k = dev_bf16(x["q"]), dev_bf16(x["k"])
    sc, bi = dev_f32(x["scale"]), dev_f32(x["bias"])
    T = x["q"].shape[1]
    cvl = vl.c(T, x["k"].shape[1])
    cap = out["col_idx"].numel()
    args = [q.data_ptr(), k.data_ptr(), cma.BF16, H, x["q"].shape[2], ctypes.byref(cvl), sc.data_ptr(),
            bi.data_ptr(), float(tau), vl.n_block_rows, out["row_ptr"].data_ptr(), out["col_idx"].data_ptr(),
            out["vals"].data_ptr(), cap, out["nnz"].data_ptr(), out["mass"].data_ptr(), out["stats"].data_ptr()]
    stream = torch.cuda.current_stream().cuda_stream
    if fn == "noalloc":
        rc = lib.cma_block_compress_noalloc(*args, stream)
    else:
        rc = lib.cma_block_compress(*args, ws.data_ptr(), ws.numel(), stream)
    torch.cuda.synchronize()
    assert rc == 0, lib.cma_last_error()
    return q, k, sc, bi  # keep the inputs alive until the work is done


@pytest.mark.parametrize("lens,H,tau", [([1000, 64, 777, 5], 8, 0.9)])
def test_noalloc_matches_workspace_call_twice(cma, lens, H, tau):
    # the second call is smaller (fewer heads, shorter sequences)
    cases = [(lens, H, 911), ([300, 130], 3, 912)]
    lib = cma.load_library()
    for lens_i, H_i, seed in cases:
        say(f"noalloc: lens={lens_i} H={H_i} tau={tau}")
        x = synth.attention_inputs(seed, H_i, lens_i, d=128)
        vl = cma.Varlen(x["cu_q"], x["cu_k"])
        T = int(x["cu_q"][-1])
        cap = cma.bsr_max_blocks(H_i, lens_i)
        ws_bytes = lib.cma_block_compress_workspace(H_i, vl.n_block_rows, vl.max_q, T)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        ref = _outputs(cma, H_i, vl, T, cap)
        got = _outputs(cma, H_i, vl, T, cap)
        _call(cma, "workspace", x, vl, H_i, tau, ref, ws)
        _call(cma, "noalloc", x, vl, H_i, tau, got)
        nnz = int(ref["nnz"].item())
        assert int(got["nnz"].item()) == nnz
        assert torch.equal(got["row_ptr"], ref["row_ptr"])
        assert torch.equal(got["col_idx"][:nnz], ref["col_idx"][:nnz])
        assert torch.equal(got["vals"][:nnz].view(torch.int16), ref["vals"][:nnz].view(torch.int16))
        assert torch.equal(got["mass"].view(torch.int32), ref["mass"].view(torch.int32))
        assert torch.equal(got["stats"].view(torch.int32), ref["stats"].view(torch.int32))
        say(f"  nnz={nnz}: every output bitwise equal to the workspace call")
