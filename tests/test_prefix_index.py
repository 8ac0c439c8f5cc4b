"""Prefix-hash index of cached sender block-rows (MapFlow, storage and execution,
second component), on the CPU: the library's chain hashes equal the oracle's,
which are pinned to the FNV-1a hash's published test vectors, and the index's
insert / lookup / erase / eviction behaviour equals a plain ordered-dictionary
model of the same rules over a long random sequence of operations."""
import ctypes
import threading

import numpy as np
import pytest

import oracle

# Published 64-bit FNV-1a test vectors (the hash's reference test suite by its
# authors, Fowler, Noll and Vo): input bytes -> hash.
FNV1A64_VECTORS = [(b"", 0xCBF29CE484222325), (b"a", 0xAF63DC4C8601EC8C), (b"foobar", 0x85944171F73967E8)]


@pytest.fixture(scope="module")
def cma():
    import cross_model_attention_causal_amd as c
    c.load_library()
    return c


def test_oracle_fnv1a64_published_vectors():
    for data, want in FNV1A64_VECTORS:
        assert oracle.fnv1a64(data) == want


def test_library_fnv1a64_equals_oracle(cma):
    lib = cma.load_library()
    for data, want in FNV1A64_VECTORS:
        buf = ctypes.create_string_buffer(data, max(1, len(data)))
        assert lib.cma_fnv1a64(buf, len(data)) == want
    rng = np.random.default_rng(1)
    for n in (1, 7, 64, 1000):
        data = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert lib.cma_fnv1a64(data, n) == oracle.fnv1a64(data)


def test_chain_hashes_equal_oracle_and_carry_the_prefix(cma):
    rng = np.random.default_rng(2)
    tokens = rng.integers(-2 ** 31, 2 ** 31, 64 * 9 + 17, dtype=np.int64).astype(np.int32)
    for seed in (0, 12345, 2 ** 64 - 1):
        got = cma.prefix_hashes(tokens, seed)
        want = oracle.prefix_hashes(tokens, seed)
        assert len(got) == 9 and [int(x) for x in got] == want  # the partial last block is not hashed
    base = [int(x) for x in cma.prefix_hashes(tokens, 7)]
    t2 = tokens.copy()
    t2[64 * 4 + 10] += 1  # a token of block 4 changes: blocks 0-3 keep their hashes, 4.. all change
    changed = [int(x) for x in cma.prefix_hashes(t2, 7)]
    assert changed[:4] == base[:4] and all(a != b for a, b in zip(changed[4:], base[4:]))
    assert [int(x) for x in cma.prefix_hashes(tokens, 8)][0] != base[0]  # the seed is part of the chain
    assert len(cma.prefix_hashes(tokens[:63], 0)) == 0


def test_index_matches_model_under_random_operations(cma):
    H, cap = 3, 40
    ix = cma.PrefixIndex(H, cap)
    model = oracle.PrefixIndexModel(cap)
    rng = np.random.default_rng(3)
    keys = [(int(l), int(h)) for l, h in zip(rng.integers(0, 3, 90), rng.integers(0, 2 ** 63, 90, dtype=np.int64))]
    for step in range(3000):
        op = rng.integers(0, 10)
        layer, h = keys[rng.integers(0, len(keys))]
        if op < 4:
            val = rng.integers(0, 10 ** 6, 2 * H).astype(np.int32)
            rc = ix.insert(layer, h, val[:H], val[H:])
            ok = model.insert(layer, h, (tuple(val[:H]), tuple(val[H:])))
            assert (rc == 0) == ok and (rc == 0 or rc == cma.CMA_ENOSPC)
        elif op < 7:
            run = [keys[i] for i in rng.integers(0, len(keys), rng.integers(1, 6))]
            run = [(layer, hh) for _, hh in run]
            n, b, c = ix.lookup(layer, [hh for _, hh in run])
            want = model.lookup(layer, [hh for _, hh in run])
            assert n == len(want)
            for i, (wb, wc) in enumerate(want):
                assert tuple(b[i]) == wb and tuple(c[i]) == wc
        elif op < 8:
            assert bool(ix.erase(layer, h)) == model.erase(layer, h)
        elif op < 9:
            ev = ix.evict_lru()
            mv = model.evict_lru()
            assert (ev is None) == (mv is None)
            if ev is not None:
                assert ev[0] == mv[0] and tuple(ev[1]) == mv[1][0] and tuple(ev[2]) == mv[1][1]
        assert len(ix) == len(model.d)
    ix.close()


def test_index_rejects_bad_arguments_and_is_thread_safe(cma):
    lib = cma.load_library()
    assert not lib.cma_prefix_index_create(0, 10)
    assert not lib.cma_prefix_index_create(4, 0)
    ix = cma.PrefixIndex(2, 100000)
    assert ix.insert(0, 1, [-1, 0], [1, 1]) == cma.CMA_EINVAL
    assert lib.cma_prefix_index_lookup(None, 0, None, 0, None, None) == cma.CMA_EINVAL

    def worker(t):
        for i in range(2000):
            assert ix.insert(t, i, [i, i], [1, 2]) == 0

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert len(ix) == 16000
    n, b, c = ix.lookup(5, np.arange(2000, dtype=np.uint64))
    assert n == 2000 and np.array_equal(b[:, 0], np.arange(2000)) and np.all(c[:, 1] == 2)
    ix.close()
