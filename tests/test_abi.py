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
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)  # drop comments
    return sorted(set(re.findall(r"\b(cma_[a-z0-9_]+)\s*\(", text)))


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
