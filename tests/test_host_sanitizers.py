"""The host-only part of the library (the prefix-hash index) built with the host
sanitizers: AddressSanitizer + UndefinedBehaviorSanitizer in one build,
ThreadSanitizer in another, each linked with a small driver
(`tests/sanitize/prefix_index_driver.cpp`). The driver runs a seeded script of
index operations whose printed results must equal the oracle's model of the
index (`oracle/prefix.py`), then calls the API with invalid arguments and from
eight threads at once; any sanitizer report fails the test. CPU only (g++)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import prefix as oprefix

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "cross_model_attention_causal_amd", "csrc", "prefix_index.hip")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "prefix_index_driver.cpp")
CMA_OK, CMA_ENOSPC = 0, -3

BUILDS = {
    "asan_ubsan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
    "tsan": ["-fsanitize=thread"],
}


def make_script(seed=7, n_heads=3, capacity=6):
    """A seeded operation script and the lines the oracle's model expects."""
    rng = np.random.default_rng(seed)
    model = oprefix.PrefixIndexModel(capacity)
    ops, want = [f"C {n_heads} {capacity}"], []
    for n, hseed in ((0, 1), (63, 2), (64, 3), (130, 4), (256, 2 ** 64 - 1)):
        tok = rng.integers(-2 ** 31, 2 ** 31, size=n, dtype=np.int64)
        ops.append(f"H {hseed} {n} " + " ".join(str(int(t)) for t in tok))
        want.append(" ".join(["H"] + [str(h) for h in oprefix.prefix_hashes(tok.astype(np.int32), hseed)]))
    keys = [int(k) for k in rng.integers(0, 2 ** 64, size=9, dtype=np.uint64)]
    for _ in range(300):
        kind = rng.integers(0, 6)
        layer = int(rng.integers(0, 2))
        if kind <= 1:
            key = keys[int(rng.integers(0, len(keys)))]
            b = [int(x) for x in rng.integers(0, 1000, size=n_heads)]
            c = [int(x) for x in rng.integers(0, 64, size=n_heads)]
            ops.append(f"I {layer} {key} " + " ".join(f"{x} {y}" for x, y in zip(b, c)))
            want.append(f"I {CMA_OK if model.insert(layer, key, (b, c)) else CMA_ENOSPC}")
        elif kind == 2:
            hs = [keys[int(i)] for i in rng.integers(0, len(keys), size=int(rng.integers(0, 5)))]
            ops.append(f"L {layer} {len(hs)} " + " ".join(str(h) for h in hs))
            found = model.lookup(layer, hs)
            want.append(" ".join([f"L {len(found)}"] + [f"{x} {y}" for b, c in found for x, y in zip(b, c)]))
        elif kind == 3:
            key = keys[int(rng.integers(0, len(keys)))]
            ops.append(f"E {layer} {key}")
            want.append(f"E {1 if model.erase(layer, key) else 0}")
        elif kind == 4:
            ops.append("V")
            got = model.evict_lru()
            if got is None:
                want.append("V 0")
            else:
                (ly, h), (b, c) = got
                want.append(" ".join([f"V 1 {ly} {h}"] + [f"{x} {y}" for x, y in zip(b, c)]))
        else:
            ops.append("S")
            want.append(f"S {len(model.d)}")
    return "\n".join(ops) + "\n", want


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
@pytest.mark.parametrize("build", sorted(BUILDS))
def test_prefix_index_under_sanitizers(tmp_path, build):
    exe = str(tmp_path / f"driver_{build}")
    cmd = ["g++", "-std=c++17", "-O1", "-g", *BUILDS[build], "-I", os.path.join(ROOT, "include"), DRIVER,
           "-x", "c++", SRC, "-x", "none", "-pthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "cannot find" in r.stderr and "san" in r.stderr:
        pytest.skip(f"{build} runtime not installed")
    assert r.returncode == 0, r.stderr[-2000:]
    script, want = make_script()
    path = tmp_path / "script.txt"
    path.write_text(script)
    # verify_asan_link_order=0: the environment may preload a library ahead of the runtime
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe, str(path)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-3000:]
    for bad in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer", "ERROR: LeakSanitizer"):
        assert bad not in r.stderr, r.stderr[-3000:]
    got = r.stdout.splitlines()
    assert len(got) == len(want)
    for i, (g, w) in enumerate(zip(got, want)):
        assert g.split() == w.split(), (i, g, w)
