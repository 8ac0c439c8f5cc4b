"""The C-ABI library loads on a machine without a GPU, exports every function
include/cma.h declares, and its host-only calls and argument validation work
without touching a device (no compute call is made here)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cma.h")
LIB = os.path.join(ROOT, "cross_model_attention_causal_amd", "libcma.so")


def declared_functions():
    import glob
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)  # drop comments
        names |= set(re.findall(r"\b(cma_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from cross_model_attention_causal_amd import build
        build.build()
    return ctypes.CDLL(LIB)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 15, names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_host_helpers(lib):
    assert lib.cma_version() == 100
    lib.cma_maps_elems.restype = ctypes.c_int64
    lib.cma_maps_elems.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lq = np.array([5, 64, 3], dtype=np.int32)
    lk = np.array([5, 70, 3], dtype=np.int32)
    packed = lib.cma_maps_elems(3, lq.ctypes.data, lk.ctypes.data, 1)
    dense = lib.cma_maps_elems(3, lq.ctypes.data, lk.ctypes.data, 0)
    want_packed = sum(oracle.packed_size(int(a), int(b)) for a, b in zip(lq, lk))
    assert packed == want_packed
    assert dense == int(np.sum(lq.astype(np.int64) * lk))
    bad = np.array([4], dtype=np.int32)  # nq > nk
    assert lib.cma_maps_elems(1, np.array([5], dtype=np.int32).ctypes.data, bad.ctypes.data, 1) == -1
    lib.cma_bsr_max_blocks.restype = ctypes.c_int64
    lib.cma_bsr_max_blocks.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lens = np.array([200, 64, 5], dtype=np.int32)
    R = (lens + 63) // 64
    assert lib.cma_bsr_max_blocks(3, 3, lens.ctypes.data) == 3 * int(np.sum(R * (R + 1) // 2))


@pytest.mark.parametrize("n_layers,ratio", [(80, 0.5), (24, 0.5), (40, 0.25), (10, 1.0), (80, 0.0)])
def test_mapped_layers_match_oracle(lib, n_layers, ratio):
    lib.cma_mapped_layers.argtypes = [ctypes.c_int32, ctypes.c_double, ctypes.c_void_p, ctypes.c_int32]
    out = np.zeros(n_layers, dtype=np.int32)
    k = lib.cma_mapped_layers(n_layers, ratio, out.ctypes.data, n_layers)
    assert list(out[:k]) == list(oracle.mapped_layers(n_layers, ratio))


# IAM Method 4 thresholds, worked by hand from the rule (extend a short prompt by
# generation to tau_e, then take the similarity over at most the first tau_t tokens):
# (prompt length, tau_e, tau_t) -> (tokens generated first, similarity prefix)
PLAN_CASES = [
    ((100, 256, 512), (156, 256)),   # short prompt: generate 156, map over 256
    ((256, 256, 512), (0, 256)),     # exactly tau_e: map at prefill
    ((300, 256, 512), (0, 300)),     # between the thresholds: the whole prompt
    ((512, 256, 512), (0, 512)),
    ((8192, 256, 512), (0, 512)),    # long prompt: truncated to the first 512 tokens
    ((0, 256, 512), (256, 256)),     # empty prompt
    ((100, 600, 512), (500, 512)),   # tau_e above tau_t: generate to 600, use 512
    ((7, 0, 1), (0, 1)),
]


@pytest.mark.parametrize("args,want", PLAN_CASES)
def test_mapping_plan_oracle_worked_cases(args, want):
    assert oracle.mapping_plan(*args) == want


def test_mapping_plan_matches_oracle(lib):
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    lib.cma_mapping_plan.argtypes = [I32, P, I32, I32, P, P]
    lib.cma_mapping_plan.restype = ctypes.c_int
    rng = np.random.default_rng(11)
    for tau_e, tau_t in [(0, 1), (256, 512), (600, 512), (512, 512), (1, 8192)]:
        p = np.concatenate([rng.integers(0, 9000, 200), [0, tau_e, tau_t, max(0, tau_e - 1), tau_t + 1]]).astype(np.int32)
        gen = np.full(p.size, -7, dtype=np.int32)
        sim = np.full(p.size, -7, dtype=np.int32)
        assert lib.cma_mapping_plan(p.size, p.ctypes.data, tau_e, tau_t, gen.ctypes.data, sim.ctypes.data) == 0
        want = [oracle.mapping_plan(int(x), tau_e, tau_t) for x in p]
        assert list(zip(gen.tolist(), sim.tolist())) == want
    # invalid arguments: an error and nothing written
    bad = np.array([5, -1], dtype=np.int32)
    gen = np.full(2, -7, dtype=np.int32)
    sim = np.full(2, -7, dtype=np.int32)
    assert lib.cma_mapping_plan(2, bad.ctypes.data, 10, 20, gen.ctypes.data, sim.ctypes.data) == -1
    assert gen.tolist() == [-7, -7]
    ok = np.array([5], dtype=np.int32)
    assert lib.cma_mapping_plan(1, ok.ctypes.data, 10, 0, gen.ctypes.data, sim.ctypes.data) == -1
    assert lib.cma_mapping_plan(1, ok.ctypes.data, -1, 20, gen.ctypes.data, sim.ctypes.data) == -1
    assert lib.cma_mapping_plan(-1, None, 10, 20, None, None) == -1
    assert lib.cma_mapping_plan(0, None, 10, 20, None, None) == 0


def test_mapping_plan_binding():
    import cross_model_attention_causal_amd as cma
    lens = [100, 256, 8192, 0]
    gen, sim = cma.mapping_plan(lens, 256, 512)
    assert list(zip(gen, sim)) == [oracle.mapping_plan(p, 256, 512) for p in lens]
    with pytest.raises(cma.CmaError):
        cma.mapping_plan([-3], 256, 512)


def test_validation_errors_without_device(lib):
    """Bad arguments are rejected before any device work, with a message."""
    lib.cma_last_error.restype = ctypes.c_char_p
    # NULL varlen
    rc = lib.cma_attn_maps(None, None, 1, 1, 128, None, None, None, None, 1, 1, ctypes.c_int64(0), None)
    assert rc == -1
    assert lib.cma_last_error()
    # head map with zero problems is a no-op; negative sizes are rejected
    rc = lib.cma_head_map_cosine(None, None, 1, -1, 1, 1, ctypes.c_int64(1), ctypes.c_int64(0), ctypes.c_int64(0),
                                 ctypes.c_int64(0), ctypes.c_int64(0), None, None, None, None, ctypes.c_size_t(0),
                                 None)
    assert rc < 0
    lib.cma_mapped_layers.argtypes = [ctypes.c_int32, ctypes.c_double, ctypes.c_void_p, ctypes.c_int32]
    assert lib.cma_mapped_layers(-1, 0.5, None, 0) == -1


def test_golden_layer_order(lib):
    """The 80-layer, 50% mapping order the IAM notes give (fixture with citation)."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "iam_mapped_layers.json")))
    lib.cma_mapped_layers.argtypes = [ctypes.c_int32, ctypes.c_double, ctypes.c_void_p, ctypes.c_int32]
    out = np.zeros(g["n_layers"], dtype=np.int32)
    k = lib.cma_mapped_layers(g["n_layers"], g["ratio"], out.ctypes.data, g["n_layers"])
    assert list(out[:k]) == g["layers"]


def test_binding_rejects_undersized_tensors():
    """The binding checks tensor sizes before passing raw pointers (CPU tensors are
    rejected too, but the size checks come first for the shapes tested here)."""
    torch = pytest.importorskip("torch")
    import cross_model_attention_causal_amd as cma
    cma.load_library()

    class VL:  # the host fields the checks read
        n_seqs = 1
        cu_q_host = np.array([0, 64])
        cu_k_host = np.array([0, 64])
        lens_q = np.array([64])
        lens_k = np.array([64])
        n_block_rows = 1

        def maps_elems(self, layout):
            return 64 * 65 // 2

    q = torch.zeros(2, 64, 128)
    with pytest.raises(ValueError):  # k has fewer heads than q
        cma.attn_maps(q, torch.zeros(1, 64, 128), torch.zeros(2), None, VL())
    with pytest.raises(ValueError):  # rows past the end of k
        cma.attn_maps(q, torch.zeros(2, 32, 128), torch.zeros(2), None, VL())
    with pytest.raises(ValueError):  # one scale for two heads
        cma.attn_maps(q, torch.zeros(2, 64, 128), torch.zeros(1), None, VL())
    with pytest.raises(ValueError):  # V with fewer heads than receivers
        cma.mapped_av(("dense", torch.zeros(4, 2080), cma.PACKED), 4, torch.zeros(1, 3, 4), 3,
                      torch.zeros(2, 64, 128), VL())


def test_indexed_workspace_and_validation(lib):
    """cma_mapped_av_indexed: the workspace size follows its layout (tiled V, then
    the per-sequence block-row offsets, the head order and the pair table, each
    on a 256-byte boundary), and bad arguments are rejected before any device
    work (the pointers below are never dereferenced)."""
    from cross_model_attention_causal_amd import _CMapsSrc, _CVarlen, SRC_BSR, SRC_DENSE, V_TILED, V_TOKEN_MAJOR
    P, I32, I64, SZ, INT = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    lib.cma_last_error.restype = ctypes.c_char_p
    ws = lib.cma_mapped_av_indexed_workspace
    ws.restype, ws.argtypes = SZ, [P, I32, I32, I32, I32, INT]
    r256 = lambda x: (x + 255) // 256 * 256
    src = _CMapsSrc()
    src.kind, src.n_block_rows = SRC_BSR, 37
    for layout in (V_TOKEN_MAJOR, V_TILED):
        n_recv, n_v, n_seqs = 64, 16, 5
        vt = 0 if layout == V_TILED else r256(n_v * 37 * 64 * 128 * 2)
        want = vt + r256(4 * n_seqs) + r256(4 * n_seqs * n_recv) + r256(4 * ((37 + n_seqs) // 2 + 1))
        assert ws(ctypes.byref(src), n_recv, n_v, 128, n_seqs, layout) == want
    dense = _CMapsSrc()
    dense.kind = SRC_DENSE
    assert ws(ctypes.byref(dense), 64, 16, 128, 5, V_TOKEN_MAJOR) == 0

    call = lib.cma_mapped_av_indexed
    call.argtypes = [P, I32, P, I64, I32, I32, P, INT, INT, I32, P, P, INT, P, SZ, P]
    fake = 0x1000
    src.row_ptr = src.col_idx = src.vals = fake
    vl = _CVarlen()
    vl.n_seqs, vl.cu_seqlens_q, vl.cu_seqlens_k = 2, fake, fake
    vl.max_seqlen_q = vl.max_seqlen_k = 128
    vl.total_q = vl.total_k = 256

    def run(s=src, n_send=8, n_recv=16, n_v=16, v_dt=1, d=128, ws_bytes=1 << 30):
        return call(ctypes.byref(s) if s is not None else None, n_send, fake, 0, n_recv, n_v, fake, v_dt,
                    V_TOKEN_MAJOR, d, ctypes.byref(vl), fake, 1, fake, ws_bytes, None)

    assert run(s=None) == -1                  # no source
    assert run(s=dense) == -2                 # dense maps have no indexed form
    assert run(n_v=5) == -1                   # V heads must divide receiver heads
    assert run(v_dt=0) == -2                  # fp32 V
    assert run(d=64) == -2
    assert run(n_recv=300, n_v=300) == -2     # more receiver heads than the head sort holds
    assert run(n_send=0) == -2
    assert run(ws_bytes=64) == -3             # workspace too small
    assert lib.cma_last_error()

    tile = lib.cma_tile_v
    tile.argtypes = [P, INT, I32, I32, P, I32, P, P]
    assert tile(fake, V_TILED, 4, 128, ctypes.byref(vl), 4, fake, None) == -1   # input must be untiled
    assert tile(fake, V_TOKEN_MAJOR, 4, 64, ctypes.byref(vl), 4, fake, None) == -2
    assert tile(fake, V_TOKEN_MAJOR, 4, 128, ctypes.byref(vl), 4, None, None) == -1
    assert tile(fake, V_TOKEN_MAJOR, 4, 128, ctypes.byref(vl), 0, fake, None) == -1


def test_workspace_too_small_is_enospc(lib):
    """Each call that takes a workspace rejects a short one with CMA_ENOSPC before
    any device work (the fake pointers below are never dereferenced)."""
    from cross_model_attention_causal_amd import _CMapsSrc, _CVarlen, SRC_BSR, V_TOKEN_MAJOR
    P, I32, I64, SZ, INT, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int,
                               ctypes.c_float)
    lib.cma_last_error.restype = ctypes.c_char_p
    fake = 0x1000
    vl = _CVarlen()
    vl.n_seqs, vl.cu_seqlens_q, vl.cu_seqlens_k = 2, fake, fake
    vl.max_seqlen_q = vl.max_seqlen_k = 128
    vl.total_q = vl.total_k = 256

    # head_map_cosine
    cws = lib.cma_head_map_cosine_workspace
    cws.restype, cws.argtypes = SZ, [I32, I32, I32, I64, INT]
    need = cws(1, 24, 32, 131328, 1)
    assert need > 0
    cos = lib.cma_head_map_cosine
    cos.argtypes = [P, P, INT, I32, I32, I32, I64, I64, I64, I64, I64, P, P, P, P, SZ, P]
    args = (fake, fake, 1, 1, 24, 32, 131328, 131328, 0, 131328, 0, fake, fake, fake)
    assert cos(*args, fake, need - 1, None) == -3
    assert b"workspace" in lib.cma_last_error()
    assert cos(*args, None, need, None) == -3

    # block_compress
    bws = lib.cma_block_compress_workspace
    bws.restype, bws.argtypes = SZ, [I32, I32, I32, I64]
    need = bws(4, 4, 128, 256)
    assert need >= 4 * 4 * (4 + 32) + 4 * 256 * 4
    comp = lib.cma_block_compress
    comp.argtypes = [P, P, INT, I32, I32, P, P, P, F, I32, P, P, P, I64, P, P, P, P, SZ, P]
    head = (fake, fake, 1, 4, 128, ctypes.byref(vl), fake, None, 0.95, 4, fake, fake, fake, 40, fake, None, None)
    assert comp(*head, fake, need - 1, None) == -3
    assert comp(*head, None, need, None) == -3
    bad_tau = head[:8] + (0.0,) + head[9:]
    assert comp(*bad_tau, fake, need, None) == -1                  # tau must be > 0
    d96 = head[:4] + (96,) + head[5:]
    assert comp(*d96, fake, need, None) == -2                      # head dim 96 is not built

    # mapped_av, block-sparse source with token-major V (V is tiled in the workspace)
    src = _CMapsSrc()
    src.kind, src.n_block_rows = SRC_BSR, 4
    src.row_ptr = src.col_idx = src.vals = fake
    mws = lib.cma_mapped_av_workspace
    mws.restype, mws.argtypes = SZ, [P, I32, I32, I64, INT]
    need = mws(ctypes.byref(src), 24, 128, 256, V_TOKEN_MAJOR)
    assert need == 24 * 4 * 64 * 128 * 2
    mav = lib.cma_mapped_av
    mav.argtypes = [P, I32, P, I64, I32, I32, P, INT, INT, I32, P, P, INT, P, SZ, P]
    run = lambda ws, nb: mav(ctypes.byref(src), 32, fake, 0, 24, 24, fake, 1, V_TOKEN_MAJOR, 128, ctypes.byref(vl),
                             fake, 1, ws, nb, None)
    assert run(fake, need - 1) == -3
    assert run(None, need) == -3
    assert run(fake + 8, need) == -1                               # workspace must be 16-byte aligned
    # more senders than two groups of 32: refused before any device work
    assert mav(ctypes.byref(src), 65, fake, 0, 24, 24, fake, 1, V_TOKEN_MAJOR, 128, ctypes.byref(vl),
               fake, 1, fake, need, None) == -2
    assert b"n_send" in lib.cma_last_error()


def test_noalloc_compress_rejects_oversized_scratch(lib):
    """cma_block_compress_noalloc refuses (CMA_ENOSPC, before any device work) a
    problem whose scratch would exceed its static array of 16 MiB."""
    from cross_model_attention_causal_amd import _CVarlen
    P, I32, I64, SZ, INT, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int,
                               ctypes.c_float)
    lib.cma_last_error.restype = ctypes.c_char_p
    ws = lib.cma_block_compress_workspace
    ws.restype, ws.argtypes = SZ, [I32, I32, I32, I64]
    fn = lib.cma_block_compress_noalloc
    fn.argtypes = [P, P, INT, I32, I32, P, P, P, F, I32, P, P, P, I64, P, P, P, P]
    fake = 0x1000
    big_T = 1 << 22
    assert ws(2, big_T // 64, 64, big_T) > (16 << 20)
    vl = _CVarlen()
    vl.n_seqs, vl.cu_seqlens_q, vl.cu_seqlens_k = 1, fake, fake
    vl.max_seqlen_q = vl.max_seqlen_k = 64
    vl.total_q = vl.total_k = big_T
    rc = fn(fake, fake, 1, 2, 128, ctypes.byref(vl), fake, None, 0.9, big_T // 64, fake, fake, fake, 0, fake,
            None, None, None)
    assert rc == -3
    assert b"scratch" in lib.cma_last_error()


def test_bsr_capacity_counts_chunk_blocks(lib):
    """cma_bsr_capacity: every block a compression can keep, prefill chunks included
    (block-row r of a chunk starting at block-row kb0 has kb0 + r + 1 blocks)."""
    lib.cma_bsr_capacity.restype = ctypes.c_int64
    lib.cma_bsr_capacity.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lq = np.array([448, 70, 128, 0], dtype=np.int32)
    lk = np.array([576, 198, 128, 64], dtype=np.int32)
    want = sum(len(oracle.select_blocks(np.ones(((b - a) // 64) + r + 1), 1.0))
               for a, b in zip(lq, lk) for r in range((int(a) + 63) // 64))
    assert lib.cma_bsr_capacity(3, 4, lq.ctypes.data, lk.ctypes.data) == 3 * want
    lib.cma_bsr_max_blocks.restype = ctypes.c_int64
    lib.cma_bsr_max_blocks.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert lib.cma_bsr_capacity(2, 4, lq.ctypes.data, None) == lib.cma_bsr_max_blocks(2, 4, lq.ctypes.data)
    assert lib.cma_bsr_capacity(2, 1, lk.ctypes.data, lq.ctypes.data) == -1  # fewer keys than queries
