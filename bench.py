#!/usr/bin/env python3
"""Benchmark of the map-reuse hot path on one MI355X.

Metric: mapped-attention prefill tokens/s at 8192 ctx, with the fraction of the
HBM / MFMA roofline reached by the dominant kernel.

Workload (synthetic, seeded): 4 prompts x 8192 tokens (IAM's long-context batch),
one mapped layer of a Ministral-like 8B -> 3B pair: 32 sender heads, 24 receiver
heads, d = 128, bf16. One step runs every stage of the path once:
  1. attn_maps        sender (32) and receiver (24) maps on each prompt's first
                      512 tokens (IAM's truncated head-mapping input), packed bf16
  2. head_map_cosine  4 problems of 24 x 32 over 131,328 entries -> argmax, margin
  3. onehot_mix       IAM head map as a per-prompt one-hot mixing matrix
  4. block_compress   32 heads x 4 x 8192 tokens, 64x64 blocks, tau = 0.95
  5. mapped_av        V tiled into the fused kernel's operand order, then the fused
                      block-sparse mix x V for 24 receiver heads (learned M)
  6. decode row       first generated token: sender rows over 8193 keys, then
                      mapped x V with the one-hot IAM head map
plus the host-side mapped-layer order. Inputs are resident in HBM before timing;
the receiver's V is token-major [heads, tokens, d].

Prints one JSON line. ``--gpus N`` with N > 1 is not supported: the benchmark runs
on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prompts", type=int, default=4)
    ap.add_argument("--ctx", type=int, default=8192)
    ap.add_argument("--tau", type=float, default=0.95)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-headline", action="store_true",
                    help="skip the single-sequence headline figures (H1: fused mapped x V, H2: block "
                         "compression, each on one 8192-token sequence)")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the check of the last step's outputs (sampled fused-pass rows, the decode "
                         "rows and prompt 0's head map) against the oracle")
    ap.add_argument("--no-measured-ceilings", dest="measured_ceilings", action="store_false",
                    help="skip the probes run after the timed steps (the stages' fractions of the "
                         "measured ceilings)")
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--stage-figures", action="store_true",
                    help="instead of the step: time each stage at its own workload (512-token head "
                         "mapping; 32-head x 8192-token compression; the fused pass over it) and print "
                         "one JSON line per workload with every kernel's roofline fraction")
    ap.add_argument("--peaks", action="store_true",
                    help="only run the ceiling probes (HBM read and copy, 32x32x16 bf16 MFMA rate, L2 -> CU "
                         "read bandwidth) and print one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB five times (for scaling hardware byte counters)")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch.
    Hardware counters of this run give the factor that turns counter readings into
    bytes for the kernels measured with the same counters."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "launches": 5}), flush=True)


# share of an HBM-bound kernel's algorithmic bytes that are written (the rest read),
# for its fraction of the probes' read and write ceilings
WRITE_SHARE = {"k_attn_maps_short": 0.5, "k_attn_maps": 0.5, "k_tile_v": 0.5, "k_attn_rows": 4 / 260,
               "k_block_extract": 0.94}


def peaks(reps=5):
    """Print the chip's ceilings as the library's probes measure them (one JSON line)."""
    print(json.dumps(measure_ceilings(reps)), flush=True)


def measure_ceilings(reps=5):
    """The chip's ceilings as the library's probes measure them (cma_probe.h): median
    of ``reps`` launches each, timed with HIP events on the current stream."""
    import ctypes
    import torch
    import cross_model_attention_causal_amd as cma

    lib = cma.load_library()
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.cma_probe_read.argtypes = [P, I64, I32, I32, P, P]
    lib.cma_probe_copy.argtypes = [P, P, I64, I32, P]
    lib.cma_probe_mfma.argtypes = [I32, I32, P, P]
    lib.cma_probe_l2.argtypes = [P, I32, I32, I32, P, P]
    lib.cma_probe_write.argtypes = [P, I64, I32, I32, P]
    lib.cma_probe_valu.argtypes = [I32, I32, I32, P, P]
    lib.cma_probe_lds.argtypes = [I32, I32, P, P]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream().cuda_stream

    def med(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert fn() == 0
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    out = {"probe": "ceilings", "compute_units": cus, "reps": reps, "clocks_before": clocks()}
    big = 4 << 30
    a = torch.ones(big // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(cus * 8 * 512, dtype=torch.int32, device="cuda")
    # reads: grid-stride and per-workgroup contiguous; the ceiling is the better
    rd = {}
    for mode, name in ((0, "stride"), (1, "contig")):
        t = med(lambda: lib.cma_probe_read(a.data_ptr(), big, cus * 8, mode, sink.data_ptr(), st))
        rd[name] = round(big / (t * 1e-3) / 1e9, 1)
    out["hbm_read_GBps_by_pattern"] = rd
    out["hbm_read_GBps"] = max(rd.values())
    half = big // 2
    b = torch.empty(half // 4, dtype=torch.float32, device="cuda")
    t = med(lambda: lib.cma_probe_copy(a.data_ptr(), b.data_ptr(), half, cus * 8, st))
    out["hbm_copy_GBps_read_plus_write"] = round(2 * half / (t * 1e-3) / 1e9, 1)
    # writes: plain and non-temporal stores, grid-stride and per-workgroup
    # contiguous; the ceiling is the best of the four
    wr = {}
    for mode, name in ((0, "plain_stride"), (1, "nt_stride"), (2, "plain_contig"), (3, "nt_contig")):
        t = med(lambda: lib.cma_probe_write(a.data_ptr(), big, cus * 8, mode, st))
        wr[name] = round(big / (t * 1e-3) / 1e9, 1)
    out["hbm_write_GBps_by_pattern"] = wr
    out["hbm_write_GBps"] = max(wr.values())
    del a, b
    # vector-unit rates: lane-operations per clock per SIMD (4 SIMDs per CU) at 2.4 GHz
    n_wg, iters = cus * 8, 4096
    o = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    for kind, name in ((0, "exp2"), (1, "fma")):
        t = med(lambda: lib.cma_probe_valu(kind, n_wg, iters, o.data_ptr(), st))
        out[f"valu_{name}_lane_ops_per_clk_per_simd_at_2p4GHz"] = round(
            n_wg * 256 * iters * 8 / (t * 1e-3) / (4 * cus) / 2.4e9, 2)
    n_wg, iters = cus * 4, 20000
    o = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    t = med(lambda: lib.cma_probe_mfma(n_wg, iters, o.data_ptr(), st))
    flops = n_wg * 4 * iters * 8 * 2 * 32 * 32 * 16
    out["mfma_32x32x16_bf16_TFLOPs"] = round(flops / (t * 1e-3) / 1e12, 1)
    l2b, l2it = 2 << 20, 200
    buf = torch.ones(l2b // 2, dtype=torch.bfloat16, device="cuda")
    t = med(lambda: lib.cma_probe_l2(buf.data_ptr(), l2b, l2it, cus * 2, sink.data_ptr(), st))
    moved = cus * 2 * l2it * l2b
    out["l2_to_cu_GBps"] = round(moved / (t * 1e-3) / 1e9, 1)
    out["l2_to_cu_B_per_clk_per_cu_at_2p4GHz"] = round(moved / (t * 1e-3) / 2.4e9 / cus, 1)
    # LDS: one 512-thread workgroup per CU (64 KB each), 16-byte reads
    lds_it = 4096
    t = med(lambda: lib.cma_probe_lds(cus, lds_it, sink.data_ptr(), st))
    lds_bytes = cus * 512 * lds_it * 8 * 16
    out["lds_read_B_per_clk_per_cu_at_2p4GHz"] = round(lds_bytes / (t * 1e-3) / 2.4e9 / cus, 1)
    out["clocks_after"] = clocks()
    del buf, sink, o
    torch.cuda.empty_cache()
    return out


def clocks():
    """The current shader and memory clocks of device 0 as the amdgpu driver's sysfs
    files list them (the entry marked '*'); None where they cannot be read. Read from
    files, with no child process, so it also works under a profiler."""
    import torch
    try:
        p = torch.cuda.get_device_properties(0)
        dev = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
    except (AttributeError, RuntimeError):
        return None
    got = {}
    for key in ("sclk", "mclk", "fclk"):
        try:
            with open(f"{dev}/pp_dpm_{key}") as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        got[key] = line.split(":", 1)[-1].strip(" *\n")
        except OSError:
            pass
    return got or None


def cache_flush():
    """A function that evicts the 256 MB last-level cache (MALL) by reading a 512 MB
    buffer with the read probe on the current stream. A read leaves clean lines
    behind: a write flush would leave up to 256 MB of dirty lines that the next
    kernel's reads must first write back, slowing it for reasons of the flush's own."""
    import ctypes
    import torch
    import cross_model_attention_causal_amd as cma

    lib = cma.load_library()
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.cma_probe_read.argtypes = [P, I64, I32, I32, P, P]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(cus * 8 * 512, dtype=torch.int32, device="cuda")

    def flush():
        st = torch.cuda.current_stream().cuda_stream
        assert lib.cma_probe_read(buf.data_ptr(), buf.numel(), cus * 8, 1, sink.data_ptr(), st) == 0

    flush()
    torch.cuda.synchronize()
    return flush


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_figures(reps=20, warmup=3):
    """Each stage at its own workload: the 512-token head mapping (maps of 336 small-
    and 2560 large-model heads, the 2560 x 336 cosine), the 32-head x 8192-token
    compression at tau 0.95, the fused pass of 24 receiver heads over it, and
    one mapped layer of the varlen serving mix (its prefill chain and one decode
    step). Per kernel: average launch time from HIP events on the launch stream, the
    algorithmic work per launch, and the fraction of the roofline that binds it; per
    workload call: p10, median and p90 of ``reps`` timed calls after ``warmup``."""
    import torch
    import cross_model_attention_causal_amd as cma
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cma.load_library()
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to("cuda")
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")

    # the probes' ceilings, for fractions of what this GPU measurably sustains
    cei = measure_ceilings(3)
    log("ceilings: " + json.dumps({k: v for k, v in cei.items() if k.startswith(("hbm", "mfma"))}))
    # Every timed call starts with the last-level cache (the 256 MB MALL) flushed by
    # reading a 512 MB buffer, outside the timed interval, so that no stage is timed
    # on inputs left in the cache by its previous call.
    flush = cache_flush()

    def timed(fn, work):
        """work: kernel -> (bound, work per launch[, share of the bytes written])."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        cma.timing_reset()
        cma.timing_enable(True)
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        for i in range(reps):
            flush()
            e0[i].record()
            fn()
            e1[i].record()
        torch.cuda.synchronize()
        cma.timing_enable(False)
        kt = cma.timing_collect()
        call = np.array([e0[i].elapsed_time(e1[i]) for i in range(reps)])
        out = {"call_ms": {"p10": round(float(np.percentile(call, 10)), 4), "median": round(float(np.median(call)), 4),
                           "p90": round(float(np.percentile(call, 90)), 4), "reps": reps}}
        for name, (ms, cnt) in kt.items():
            e = dict(ms=round(ms / cnt, 4), launches_per_call=cnt // reps)
            if name in work:
                bound, amount = work[name][:2]
                wf = work[name][2] if len(work[name]) > 2 else WRITE_SHARE.get(name, 0.0)
                sec = ms / cnt * 1e-3
                if bound == "hbm":
                    ach, peak, unit = amount / sec / 1e9, HBM_PEAK_GBS, "GB/s"
                    mpeak = 1.0 / ((1.0 - wf) / cei["hbm_read_GBps"] + wf / cei["hbm_write_GBps"])
                else:
                    ach, peak, unit = amount / sec / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
                    mpeak = cei["mfma_32x32x16_bf16_TFLOPs"]
                e.update(bound=bound, work_per_launch=amount, achieved=round(ach, 1), peak=peak, unit=unit,
                         frac=round(ach / peak, 4), measured_peak=round(mpeak, 1),
                         frac_of_measured=round(ach / mpeak, 4))
            out[name] = e
        return out

    # 512-token head mapping
    t0 = time.time()
    x = synth.cfg2()
    log(f"head-mapping inputs in {time.time() - t0:.1f}s")
    Hs, Hr, n = x["n_send"], x["n_recv"], x["n"]
    L = n * (n + 1) // 2
    vl = cma.Varlen(x["cu"])
    sq, sk, rq, rk = bf(x["send_q"]), bf(x["send_k"]), bf(x["recv_q"]), bf(x["recv_k"])
    ss, sb, rs, rb = f32(x["send_scale"]), f32(x["send_bias"]), f32(x["recv_scale"]), f32(x["recv_bias"])
    st = {}

    def maps():
        st["s"] = cma.attn_maps(sq, sk, ss, sb, vl)
        st["r"] = cma.attn_maps(rq, rk, rs, rb, vl)
    maps_bytes = (Hs + Hr) * (2 * n * 128 * 2 + L * 2) / 2  # per launch, average of the two
    k_maps = timed(maps, {"k_attn_maps_short": ("hbm", maps_bytes), "k_attn_maps": ("hbm", maps_bytes)})
    k_cos = timed(lambda: cma.head_map_cosine(st["r"], st["s"], 1, Hr, Hs, L, L, 0, L, 0),
                  {"k_gram_bf16": ("mfma", 2 * Hr * Hs * L)})
    print(json.dumps({"workload": f"head mapping: one {n}-token prompt, {Hs} small-model and {Hr} large-model "
                                  "maps (d=128, bf16), packed causal, and the Hr x Hs cosine with argmax",
                      "call_ms": {"maps": k_maps.pop("call_ms"), "cosine": k_cos.pop("call_ms")},
                      "kernels": {**k_maps, **k_cos}}), flush=True)
    del st
    # the same head mapping with the large model's maps formed inside the Gram
    # producer (never stored): the small model's maps stored dense, then the fused pass
    fz = {}

    def fused():
        fz["s"] = cma.attn_maps(sq, sk, ss, sb, vl, layout=cma.DENSE)
        fz["r"] = cma.head_map_fused(rq, rk, rs, rb, fz["s"], Hs, vl, workspace=fz.setdefault("ws", cma.Workspace()))
    s_bytes = Hs * (2 * n * 128 * 2 + n * n * 2)
    k_fused = timed(fused, {"k_attn_maps_short": ("hbm", s_bytes),
                            "k_head_map_fused": ("mfma", 2 * Hr * Hs * L + 2 * Hr * L * 128)})
    tot = sum(e["ms"] * e["launches_per_call"] for e in k_fused.values() if "launches_per_call" in e)
    print(json.dumps({"workload": f"fused head mapping: the same {Hr} x {Hs} problem, {Hs} small-model maps stored "
                                  f"(dense bf16), the {Hr} large-model maps formed on chip inside the Gram "
                                  "(work: Gram products + one QK^T pass over the causal entries)",
                      "total_ms": round(tot, 4), "kernels": k_fused}), flush=True)
    del fz, sq, sk, rq, rk

    # 32-head x 8192-token compression, then the fused pass over it
    t0 = time.time()
    x = synth.cfg3()
    y = synth.cfg4()
    log(f"compression inputs in {time.time() - t0:.1f}s")
    H, n, tau = x["n_heads"], x["n"], x["tau"]
    vl = cma.Varlen(x["cu"])
    q, k = bf(x["q"]), bf(x["k"])
    sc, bi = f32(x["scale"]), f32(x["bias"])
    ws = cma.Workspace()
    res = {}

    def comp():
        res["bsr"] = cma.block_compress(q, k, sc, bi, vl, tau, workspace=ws)
    comp()
    torch.cuda.synchronize()
    nnz = int(res["bsr"]["nnz"].item())
    qk = 2 * H * n * 128 * 2
    k_comp = timed(comp, {"k_block_stats": ("mfma", H * (n * (n + 1) // 2) * 128 * 2),
                          "k_block_extract": ("hbm", nnz * 8192 + nnz * 4 + qk,
                                              nnz * 8196 / (nnz * 8196 + qk))})
    causal = (n // 64) * (n // 64 + 1) // 2
    print(json.dumps({"workload": f"block compression: {H} heads x {n} tokens (d=128, bf16), 64x64 blocks, "
                                  f"tau={tau}", "kept_block_fraction": round(nnz / (H * causal), 4),
                      "kernels": k_comp}), flush=True)
    Hs, Hr = y["n_send"], y["n_recv"]
    M, V = f32(y["M"]), bf(y["v"])
    wsv = cma.Workspace()
    r_tot = n // 64
    k_mav = timed(lambda: cma.mapped_av(res["bsr"], Hs, M, Hr, V, vl, workspace=wsv),
                  {"k_mapped_av_bsr": ("hbm", nnz * 8192 + 2 * Hr * n * 128 * 2 + (Hs * r_tot + 1 + nnz) * 4),
                   "k_tile_v": ("hbm", 2 * Hr * n * 128 * 2)})
    print(json.dumps({"workload": f"fused mapped x V: {Hr} receiver heads over the {Hs}-head compressed maps "
                                  f"above, learned M, token-major bf16 V (d=128)", "kernels": k_mav}), flush=True)
    # the same with grouped V: 8 V heads, each shared by 3 receiver heads
    Hv = 8
    Vg = V[:Hv].contiguous()
    k_gqa = timed(lambda: cma.mapped_av(res["bsr"], Hs, M, Hr, Vg, vl, workspace=wsv, v_heads=Hv),
                  {"k_mapped_av_bsr": ("hbm", nnz * 8192 + (Hv + Hr) * n * 128 * 2 + (Hs * r_tot + 1 + nnz) * 4),
                   "k_tile_v": ("hbm", 2 * Hv * n * 128 * 2)})
    print(json.dumps({"workload": f"fused mapped x V with grouped V: {Hr} receiver heads reading {Hv} V heads "
                                  f"({Hr // Hv} per V head), otherwise as above", "kernels": k_gqa}), flush=True)
    # a prefill chunk: the last 4096 queries of the 8192-token prompt over all its
    # keys (compression of the chunk, then the fused pass with V read through a
    # shuffled page table)
    ch = n // 2
    vl_c = cma.Varlen([0, ch], [0, n], used_q=[ch], used_k=[n])
    qc = q[:, n - ch:].contiguous()
    res_c = {}

    def comp_chunk():
        res_c["bsr"] = cma.block_compress(qc, k, sc, bi, vl_c, tau, workspace=ws)
    comp_chunk()
    torch.cuda.synchronize()
    nnz_c = int(res_c["bsr"]["nnz"].item())
    n_pages = n // 64 + 16
    table = torch.from_numpy(np.random.default_rng(5).permutation(n_pages)[: n // 64].astype(np.int32)).view(
        1, -1).to("cuda")
    pages = torch.zeros((Hr, n_pages, 64 * 128), dtype=torch.bfloat16, device="cuda")
    cma.tile_v_paged(V, cma.Varlen([0, n]), pages, table)
    pv = dict(pages=pages, table=table)
    chunk_flops = H * sum((n - ch + i + 1) for i in range(ch)) * 128 * 2
    k_cc = timed(comp_chunk, {"k_block_stats": ("mfma", chunk_flops),
                              "k_block_extract": ("hbm", nnz_c * 8192 + nnz_c * 4 + H * (ch + n) * 128 * 2,
                                                  nnz_c * 8196 / (nnz_c * 8196 + H * (ch + n) * 128 * 2))})
    k_cm = timed(lambda: cma.mapped_av(res_c["bsr"], Hs, M, Hr, pv, vl_c, q_rows=ch, v_layout=cma.V_PAGED,
                                       k_rows=n),
                 {"k_mapped_av_bsr": ("hbm", nnz_c * 8192 + Hr * (ch + n) * 128 * 2
                                      + (Hs * (ch // 64) + 1 + nnz_c) * 4)})
    print(json.dumps({"workload": f"prefill chunk: the last {ch} queries of the {n}-token prompt over its {n} keys, "
                                  f"{H} sender heads compressed at tau={tau}, then {Hr} receiver heads with V read "
                                  "through a page table of 64-key pages", "kernels_compress": k_cc,
                      "kernels_mapped_av": k_cm}), flush=True)
    del res_c, pages, pv, qc
    # two such receivers served from the one sender state: separate calls, then one
    # call with their heads stacked (each sender column read once per XCD)
    M2 = torch.cat([M, M.flip(1)], dim=1).contiguous()
    V2 = torch.cat([Vg, Vg.flip(0)]).contiguous()
    k_two = timed(lambda: (cma.mapped_av(res["bsr"], Hs, M, Hr, Vg, vl, workspace=wsv, v_heads=Hv),
                           cma.mapped_av(res["bsr"], Hs, M2[:, Hr:].contiguous(), Hr, V2[Hv:], vl, workspace=wsv,
                                         v_heads=Hv)), {})
    k_stack = timed(lambda: cma.mapped_av(res["bsr"], Hs, M2, 2 * Hr, V2, vl, workspace=wsv, v_heads=2 * Hv), {})
    print(json.dumps({"workload": f"two receivers of {Hr} heads ({Hv} V heads each) on the one sender state: two "
                                  "calls against one call with the heads stacked",
                      "two_calls_ms": round(sum(v["ms"] * v["launches_per_call"] for v in k_two.values() if "launches_per_call" in v), 4),
                      "stacked_ms": round(sum(v["ms"] * v["launches_per_call"] for v in k_stack.values() if "launches_per_call" in v), 4),
                      "kernels_two_calls": k_two, "kernels_stacked": k_stack}), flush=True)
    del res, q, k, M, V, Vg, M2, V2, ws, wsv

    # the varlen serving mix, one mapped layer: the prefill chain over all 68
    # prompts, then one decode step of the 64 short prompts at the longest context
    t0 = time.time()
    x = synth.cfg5_layer(0)
    log(f"serving-mix inputs in {time.time() - t0:.1f}s")
    Hs, Hr, tt, nsh, dec = x["n_send"], x["n_recv"], x["tau_t"], x["n_short"], x["decode"]
    pl, cp, cs = x["prompt_lengths"], x["cu_prompt"], x["cu_store"]
    P, L = len(pl), tt * (tt + 1) // 2
    sq, sk = bf(x["send_q"]), bf(x["send_k"])
    ss, sb = f32(x["send_scale"]), f32(x["send_bias"])
    rq, rk, rs, rb = bf(x["recv_q"]), bf(x["recv_k"]), f32(x["recv_scale"]), f32(x["recv_bias"])
    v = bf(x["v"])
    vl_s = cma.Varlen(cp, cs, used_q=[tt] * P, used_k=[tt] * P)
    vl_r = cma.Varlen(np.arange(P + 1) * tt)
    vl_p = cma.Varlen(cp, cs, used_q=pl, used_k=pl)
    ws, wsv = cma.Workspace(), cma.Workspace()
    st = {}

    def prefill():
        sm = cma.attn_maps(sq, sk, ss, sb, vl_s)
        rm = cma.attn_maps(rq, rk, rs, rb, vl_r)
        _, st["arg"], _ = cma.head_map_cosine(rm, sm, P, Hr, Hs, L, P * L, L, P * L, L)
        st["bsr"] = cma.block_compress(sq, sk, ss, sb, vl_p, 0.95, workspace=ws)
        # one sender per receiver head: the argmax itself selects the maps
        st["O"] = cma.mapped_av(st["bsr"], Hs, st["arg"], Hr, v, vl_p, q_rows=int(cp[-1]), workspace=wsv)
    prefill()
    torch.cuda.synchronize()
    nnz = int(st["bsr"]["nnz"].item())
    tri = sum(n * (n + 1) // 2 for n in pl)
    r_tot = sum((n + 63) // 64 for n in pl)
    tokens = int(cp[-1])
    # blocks of the senders in use: each prompt's kept blocks of the senders its heads map to
    rp = st["bsr"]["row_ptr"].cpu().numpy().astype(np.int64)
    argh = st["arg"].cpu().numpy()
    roff = np.concatenate([[0], np.cumsum([(n + 63) // 64 for n in pl])])
    used_blocks = sum(int(rp[j * r_tot + roff[p_ + 1]] - rp[j * r_tot + roff[p_]])
                      for p_ in range(P) for j in set(argh[p_].tolist()))
    # blocks multiplied by the indexed pass: each receiver head's sender's kept blocks
    head_blocks = sum(int(rp[j * r_tot + roff[p_ + 1]] - rp[j * r_tot + roff[p_]])
                      for p_ in range(P) for j in argh[p_].tolist())
    maps_bytes = P * (Hs + Hr) * (2 * tt * 128 * 2 + L * 2) / 2
    idx_bytes = used_blocks * 8192 + 2 * Hr * tokens * 128 * 2 + (Hs * r_tot + 1 + nnz) * 4
    # 64 x 64 x 128 multiply-adds per (receiver head, block): ~2 TFLOP against ~3 GB,
    # so the matrix cores, not HBM, bound the indexed pass
    idx_flops = head_blocks * 64 * 64 * 128 * 2
    k_pre = timed(prefill, {"k_attn_maps_short": ("hbm", maps_bytes),
                            # 68 small problems (64 x 28): ~20 flop per byte, far below
                            # the ridge, so the maps' bytes bound the Gram here
                            "k_gram_bf16": ("hbm", P * (Hr + Hs) * L * 2),
                            "k_block_stats": ("mfma", Hs * tri * 128 * 2),
                            "k_block_extract": ("hbm", nnz * 8192 + nnz * 4 + 2 * Hs * tokens * 128 * 2,
                                                nnz * 8196 / (nnz * 8196 + 2 * Hs * tokens * 128 * 2)),
                            "k_mapped_av_idx": ("mfma", idx_flops),
                            "k_tile_v": ("hbm", 2 * Hr * tokens * 128 * 2)})
    pre_ms = sum(e["ms"] * e["launches_per_call"] for e in k_pre.values() if "launches_per_call" in e)
    # the general fused pass on the same problem, with the argmax as a one-hot M
    st["M"] = cma.onehot_mix(st["arg"], Hs)
    k_gen = timed(lambda: cma.mapped_av(st["bsr"], Hs, st["M"], Hr, v, vl_p, q_rows=tokens, workspace=wsv),
                  {"k_mapped_av_bsr": ("hbm", idx_bytes)})
    print(json.dumps({"workload": f"serving mix, one mapped layer, prefill: {P} prompts ({nsh} x {pl[0]} + "
                                  f"{P - nsh} x {pl[-1]} tokens) packed varlen, {Hs} sender / {Hr} receiver heads "
                                  f"(d=128, bf16): prefix maps (tau_t={tt}), per-prompt cosine head maps, one-hot "
                                  "M, block compression at tau 0.95, fused mapped x V",
                      "kernel_ms_per_layer": round(pre_ms, 4), "kept_block_fraction":
                      round(nnz / (Hs * sum((n // 64) * (n // 64 + 1) // 2 for n in pl)), 4),
                      "kernels": k_pre, "general_path_one_hot_M": k_gen}), flush=True)
    t = dec - 1
    ctx = tt + t + 1
    vl_d = cma.Varlen(np.arange(nsh + 1), cs[: nsh + 1], used_q=[1] * nsh, used_k=[ctx] * nsh)
    qd = bf(x["send_dec_q"][t])
    Md = st["M"][:nsh].contiguous()

    def decode():
        rows = cma.attn_maps(qd, sk, ss, sb, vl_d, layout=cma.DENSE, out_dtype=torch.float32)
        st["od"] = cma.mapped_av(("dense", rows, cma.DENSE), Hs, Md, Hr, v, vl_d, q_rows=nsh)
    k_dec = timed(decode, {"k_attn_rows": ("hbm", Hs * nsh * ctx * (128 * 2 + 4)),
                           "k_mapped_av_dense": ("hbm", Hr * nsh * ctx * (128 * 2 + 4))})
    dec_ms = sum(e["ms"] * e["launches_per_call"] for e in k_dec.values() if "launches_per_call" in e)
    print(json.dumps({"workload": f"serving mix, one mapped layer, one decode step: {nsh} prompts at context "
                                  f"{ctx}, sender rows over {Hs} heads and the one-hot mapped x V of {Hr} receiver "
                                  "heads", "kernel_ms_per_step": round(dec_ms, 4), "kernels": k_dec}), flush=True)


def long_decode_figures(reps=20):
    """IAM's long-context decode (8192 + 512 at batch 4), one generation step at its
    longest context (8704 keys): the sender rows over 32 heads, then the mapped x V
    of 24 receiver heads with a one-hot head map."""
    import torch
    import cross_model_attention_causal_amd as cma
    import synth

    x = synth.long_decode()
    P, n, dec, Hs, Hr = x["n_prompts"], x["n"], x["decode"], x["n_send"], x["n_recv"]
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to("cuda")
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    t = dec - 1
    ctx = n + 1 + t
    vl = cma.Varlen(np.arange(P + 1), x["cu_k"], used_q=[1] * P, used_k=[ctx] * P)
    k, sc, bi, v = bf(x["send_k"]), f32(x["send_scale"]), f32(x["send_bias"]), bf(x["v"])
    qd = bf(x["dec_q"][t])
    Mo = torch.zeros((P, Hr, Hs), dtype=torch.float32, device="cuda")
    Mo[:, torch.arange(Hr), torch.arange(Hr) * 7 % Hs] = 1.0
    st = {}

    def step():
        st["rows"] = cma.attn_maps(qd, k, sc, bi, vl, layout=cma.DENSE, out_dtype=torch.float32)
        st["o"] = cma.mapped_av(("dense", st["rows"], cma.DENSE), Hs, Mo, Hr, v, vl, q_rows=P)
    cei = measure_ceilings(3)
    # the step's K and V (~0.5 GB) would fit the 256 MB last-level cache in part:
    # it is flushed (a 512 MB read) before every timed step
    flush = cache_flush()
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    cma.timing_reset()
    cma.timing_enable(True)
    for i in range(reps):
        flush()
        step()
    torch.cuda.synchronize()
    cma.timing_enable(False)
    kt = cma.timing_collect()
    work = {"k_attn_rows": Hs * P * (128 * 2 + ctx * (128 * 2 + 4)), "k_mapped_av_dense": Hr * P * ctx * (128 * 2 + 4)}
    kern = {}
    for name, (ms, cnt) in kt.items():
        e = dict(ms=round(ms / cnt, 4), launches_per_step=cnt // reps)
        if name in work:
            ach = work[name] / (ms / cnt * 1e-3) / 1e9
            wf = WRITE_SHARE.get(name, 0.0)
            mpeak = 1.0 / ((1.0 - wf) / cei["hbm_read_GBps"] + wf / cei["hbm_write_GBps"])
            e.update(bound="hbm", work_per_launch=work[name], achieved=round(ach, 1), peak=HBM_PEAK_GBS,
                     unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4), measured_peak=round(mpeak, 1),
                     frac_of_measured=round(ach / mpeak, 4))
        kern[name] = e
    step_ms = sum(e["ms"] * e["launches_per_step"] for e in kern.values())
    print(json.dumps({"workload": f"IAM long-context decode, one step at context {ctx}: {P} prompts, sender rows "
                                  f"over {Hs} heads, one-hot mapped x V of {Hr} receiver heads (bf16, d=128)",
                      "kernel_ms_per_step": round(step_ms, 4), "tokens_per_s": round(P / (step_ms * 1e-3), 1),
                      "kernels": kern}), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        return calibrate_copy()
    if args.peaks:
        return peaks()
    if args.stage_figures:
        stage_figures()
        return long_decode_figures()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; sharding over several GPUs is a design "
                          "note, not a supported run (use --gpus 1)", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import cross_model_attention_causal_amd as cma
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cma.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    P, n = args.prompts, args.ctx
    t0 = time.time()
    x = synth.prefill_batch(n_prompts=P, n=n)
    log(f"inputs generated in {time.time() - t0:.1f}s")
    Hs, Hr, tau_t, slot = x["n_send"], x["n_recv"], x["tau_t"], x["slot"]

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    send_q, send_k = bf(x["send_q"]), bf(x["send_k"])
    recv_q, recv_k = bf(x["recv_q"]), bf(x["recv_k"])
    v = bf(x["v"])  # token-major V [24, P*slot, 128], as a V projection writes it
    dec_q = bf(x["dec_q"])
    s_scale, s_bias = f32(x["send_scale"]), f32(x["send_bias"])
    r_scale, r_bias = f32(x["recv_scale"]), f32(x["recv_bias"])
    M = f32(x["M"])

    vl_pref = cma.Varlen(x["cu_q"], x["cu_k"], used_q=[n] * P, used_k=[n] * P)
    vl_map_s = cma.Varlen(x["cu_q"], x["cu_k"], used_q=[tau_t] * P, used_k=[tau_t] * P)
    vl_map_r = cma.Varlen(x["cu_t"], x["cu_t"])
    vl_dec = cma.Varlen(np.arange(P + 1), x["cu_k"], used_q=[1] * P, used_k=[n + 1] * P)

    L = tau_t * (tau_t + 1) // 2
    sm = torch.empty((Hs, vl_map_s.maps_elems(cma.PACKED)), dtype=torch.bfloat16, device=dev)
    rm = torch.empty((Hr, vl_map_r.maps_elems(cma.PACKED)), dtype=torch.bfloat16, device=dev)
    assert sm.shape[1] == P * L and L % 8 == 0
    cap = cma.bsr_max_blocks(Hs, [n] * P)
    bsr_buf = dict(row_ptr=torch.empty(Hs * vl_pref.n_block_rows + 1, dtype=torch.int32, device=dev),
                   col_idx=torch.empty(cap, dtype=torch.int32, device=dev),
                   vals=torch.empty((cap, 64, 64), dtype=torch.bfloat16, device=dev),
                   nnz=torch.empty(1, dtype=torch.int32, device=dev), capacity=cap)
    ws_c, ws_v = cma.Workspace(), cma.Workspace()
    O = torch.empty((Hr, P * n, 128), dtype=torch.bfloat16, device=dev)
    vt = torch.empty((Hr, vl_pref.n_block_rows, 64 * 128), dtype=torch.bfloat16, device=dev)
    rows = torch.empty((Hs, vl_dec.maps_elems(cma.DENSE)), dtype=torch.float32, device=dev)
    od = torch.empty((Hr, P, 128), dtype=torch.bfloat16, device=dev)
    state = {}

    # The head mapping and the decode row (steps 1-3 and 6) and the tiling of V do
    # not depend on the compression (step 4): they run on a second stream of the
    # same (default) priority beside it; the fused pass (step 5) waits for the
    # tiled V. Each step starts both streams together and ends when both are done.
    side = torch.cuda.Stream()
    v_ready = torch.cuda.Event()

    def step():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        layers = cma.mapped_layers(80, 0.5)                                  # host: layer order
        with torch.cuda.stream(side):
            cma.tile_v(v, vl_pref, vl_pref.n_block_rows, out=vt)                 # 5a
            v_ready.record(side)
            cma.attn_maps(send_q, send_k, s_scale, s_bias, vl_map_s, out=sm)     # 1
            cma.attn_maps(recv_q, recv_k, r_scale, r_bias, vl_map_r, out=rm)
            cos, arg, mar = cma.head_map_cosine(rm, sm, P, Hr, Hs, L, P * L, L, P * L, L)  # 2
            Mdec = cma.onehot_mix(arg, Hs)                                       # 3
            cma.attn_maps(dec_q, send_k, s_scale, s_bias, vl_dec, layout=cma.DENSE,
                          out_dtype=torch.float32, out=rows)                      # 6
            cma.mapped_av(("dense", rows, cma.DENSE), Hs, Mdec, Hr, v, vl_dec, out=od, q_rows=P)
        bsr = cma.block_compress(send_q, send_k, s_scale, s_bias, vl_pref, args.tau,
                                 workspace=ws_c, bsr=bsr_buf)                 # 4
        main.wait_event(v_ready)
        cma.mapped_av(bsr, Hs, M, Hr, vt, vl_pref, out=O, q_rows=P * n, v_layout=cma.V_TILED,
                      k_rows=v.shape[1], workspace=ws_v)                      # 5
        main.wait_stream(side)
        state.update(arg=arg, mar=mar, cos=cos, bsr=bsr, layers=layers)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    cma.timing_reset()
    cma.timing_enable(True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    # one event between consecutive steps (each step ends with the main stream
    # waiting for the side stream), so every step's own time is known too
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    cma.timing_enable(False)
    kt = cma.timing_collect()
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    tokens = P * n
    value = tokens / (ms_step / 1e3)

    nnz = int(state["bsr"]["nnz"].item())
    r_tot = vl_pref.n_block_rows
    causal_blocks = P * (n // 64) * (n // 64 + 1) // 2
    kept_frac = nnz / (Hs * causal_blocks)

    # algorithmic work per launch: work per unit (bytes or flops) times the units of one launch
    def per_launch(name):
        ms, cnt = kt.get(name, (0.0, 0))
        return (ms / cnt if cnt else float("nan")), cnt

    stage = {}
    # fused mapped x V: kept sender blocks + V + O + block index
    b_mav = nnz * 8192 + 2 * Hr * tokens * 128 * 2 + (Hs * r_tot + 1 + nnz) * 4
    # block statistics: QK^T over the causal entries (MFMA flops)
    f_stats = Hs * P * (n * (n + 1) // 2) * 128 * 2
    # extraction: kept blocks written + Q and K read
    b_ext = nnz * 8192 + nnz * 4 + 2 * Hs * tokens * 128 * 2
    # maps: sender and receiver prefix maps, one launch each (Q, K read + packed bf16
    # written; per launch the average of the two); the decode row (q row + 8193 keys
    # read, fp32 row written), one launch
    b_maps = (Hs + Hr) * P * (2 * tau_t * 128 * 2 + L * 2) / 2
    b_rows = Hs * P * (128 * 2 + (n + 1) * (128 * 2 + 4))
    # cosine Gram: MFMA flops over all receiver x sender pairs
    f_gram = 2 * P * Hr * Hs * L
    # (bound, work per launch, share of the bytes that are written)
    specs = {
        "k_mapped_av_bsr": ("hbm", b_mav, Hr * tokens * 128 * 2 / b_mav),
        "k_block_stats": ("mfma", f_stats, 0.0),
        "k_block_extract": ("hbm", b_ext, nnz * 8196 / b_ext),
        "k_attn_maps_short": ("hbm", b_maps, L * 2 / (2 * tau_t * 128 * 2 + L * 2)),
        "k_attn_rows": ("hbm", b_rows, 4 / (128 * 2 + 4)),
        "k_tile_v": ("hbm", 2 * Hr * tokens * 128 * 2, 0.5),
        "k_gram_bf16": ("mfma", f_gram, 0.0),
    }
    # the probes' ceilings, measured after the timed steps (the measured-ceiling
    # fraction of an HBM kernel prices its reads at the read probe's rate and its
    # writes at the write probe's)
    cei = measure_ceilings(3) if args.measured_ceilings else None
    for name, (bound, work, wf) in specs.items():
        ms, cnt = per_launch(name)
        if not cnt:
            continue
        if bound == "hbm":
            ach, peak, unit = work / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
            mpeak = 1.0 / ((1.0 - wf) / cei["hbm_read_GBps"] + wf / cei["hbm_write_GBps"]) if cei else None
        else:
            ach, peak, unit = work / (ms * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
            mpeak = cei["mfma_32x32x16_bf16_TFLOPs"] if cei else None
        stage[name] = dict(ms=round(ms, 4), launches=cnt, bound=bound, achieved=round(ach, 1),
                           peak=peak, unit=unit, frac=round(ach / peak, 4))
        if mpeak:
            stage[name].update(measured_peak=round(mpeak, 1), frac_of_measured=round(ach / mpeak, 4))
    for name, (ms, cnt) in kt.items():
        if name not in stage:
            stage[name] = dict(ms=round(ms / cnt, 4), launches=cnt)

    # dominant kernel among those with a roofline
    dom = max((k for k in stage if "bound" in stage[k]), key=lambda k: stage[k]["ms"] * stage[k]["launches"])
    d = stage[dom]
    # HBM bytes per launch of the dominant kernel from the committed counter run
    # (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel of known size); null when
    # the kernel's source or the shared headers changed since that run.
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        try:
            t = json.load(open(tpath))[dom]
            h = hashlib.sha256()
            for f in [t["source"]] + list(t.get("headers", [])):
                h.update(open(os.path.join(ROOT, "cross_model_attention_causal_amd", "csrc", f), "rb").read())
            if h.hexdigest() == t["sha256"]:
                traffic = t["bytes_per_launch"]
        except (KeyError, OSError, ValueError):
            traffic = None
    roofline = dict(kernel=dom, bound=d["bound"], achieved=d["achieved"], peak=d["peak"], unit=d["unit"],
                    frac=d["frac"], traffic=traffic)

    result = {
        "metric": "mapped-attention prefill tokens/s at 8192 ctx; % of HBM/MFMA roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"prefill of {P} prompts x {n} tokens, one mapped layer, 32 sender -> 24 receiver "
                        "heads, d=128: maps + cosine head map on the 512-token prefix, block_compress "
                        f"tau={args.tau}, fused mapped_av, first decode row",
            "prompts": P, "ctx": n, "n_send": Hs, "n_recv": Hr, "d": 128, "tau": args.tau,
            "tau_t": tau_t, "global_batch": P, "seq_len": n, "parallelism": "none (1 GPU)",
        },
        "roofline": roofline,
        # the same kernel against the ceilings the probes measured on this GPU after
        # the timed steps (cma_probe.h), beside the vendor peak above
        "roofline_measured": (dict(kernel=dom, ceiling=d.get("measured_peak"), unit=d["unit"],
                                   frac=d.get("frac_of_measured"),
                                   probes={k: cei[k] for k in ("hbm_read_GBps", "hbm_write_GBps",
                                                               "hbm_copy_GBps_read_plus_write",
                                                               "mfma_32x32x16_bf16_TFLOPs")})
                              if cei else None),
        "kept_block_fraction": round(kept_frac, 4),
        "stages": stage,
        "wall_s_timed_region": round(wall, 3),
        "step_ms_percentiles": {"p10": round(float(np.percentile(step_ms, 10)), 4),
                                "median": round(float(np.median(step_ms)), 4),
                                "p90": round(float(np.percentile(step_ms, 90)), 4)},
    }
    check_ok = True
    if not args.no_check:
        result["check"] = check_outputs(x, state, O, od, P, n, args.tau)
        check_ok = result["check"]["ok"]

    if not args.no_headline:
        del state, bsr_buf, O, vt, rows
        torch.cuda.empty_cache()
        result["headline"] = headline_figures()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x, P, n, tokens, args.tau)

    print(json.dumps(result), flush=True)
    if not check_ok:
        sys.exit(1)


def headline_figures(reps=10):
    """Headline figures. On one 8192-token prompt (32 sender heads, tau = 0.95; 24
    receiver heads, learned M, token-major V): H2 = 8192 / t(block compression:
    statistics, scan, extraction) and H1 = 8192 / t(mapped x V: V tiling and the
    fused pass). On four 8192-token prompts (28 sender heads, 64 receiver heads with
    one sender each): H3 = 4 * 8192 / (t(block compression) + t(indexed mapped x
    V)). Each time is the median over ``reps`` calls from HIP events on the launch
    stream around the whole call, with the per-kernel averages beside them."""
    import torch
    import cross_model_attention_causal_amd as cma
    import synth

    x, y = synth.cfg3(), synth.cfg4()
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to("cuda")
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    H, n, tau = x["n_heads"], x["n"], x["tau"]
    vl = cma.Varlen(x["cu"])
    q, k, sc, bi = bf(x["q"]), bf(x["k"]), f32(x["scale"]), f32(x["bias"])
    M, V = f32(y["M"]), bf(y["v"])
    ws, wsv, res = cma.Workspace(), cma.Workspace(), {}

    def comp():
        res["bsr"] = cma.block_compress(q, k, sc, bi, vl, tau, workspace=ws)

    def mav():
        res["O"] = cma.mapped_av(res["bsr"], y["n_send"], M, y["n_recv"], V, vl, workspace=wsv)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        cma.timing_reset()
        cma.timing_enable(True)
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        cma.timing_enable(False)
        kt = cma.timing_collect()
        return float(np.median(ms)), {kname: round(t / c, 4) for kname, (t, c) in kt.items()}

    t_c, k_c = timed(comp)
    t_m, k_m = timed(mav)
    nnz = int(res["bsr"]["nnz"].item())
    del res["bsr"], res["O"]
    # H3: the serving mix's four 8192-token prompts, one mapped layer: 28 sender
    # heads compressed, then 64 receiver heads through the indexed pass (one sender
    # per head; seeded random senders stand in for the cosine argmax)
    P3, Hs3, Hr3 = 4, 28, 64
    x3 = synth.attention_inputs(20260035, Hs3, [n] * P3, d=128)
    vl3 = cma.Varlen(x3["cu_q"])
    q3, k3, sc3, bi3 = bf(x3["q"]), bf(x3["k"]), f32(x3["scale"]), f32(x3["bias"])
    v3 = bf(synth.values(20260036, Hr3, P3 * n, 128))
    snd = np.random.Generator(np.random.PCG64(np.random.SeedSequence(20260037))).integers(0, Hs3, (P3, Hr3))
    snd3 = torch.from_numpy(snd.astype(np.int32)).to("cuda")
    ws3, wsv3 = cma.Workspace(), cma.Workspace()

    def comp3():
        res["bsr3"] = cma.block_compress(q3, k3, sc3, bi3, vl3, tau, workspace=ws3)

    def mav3():
        res["O3"] = cma.mapped_av(res["bsr3"], Hs3, snd3, Hr3, v3, vl3, workspace=wsv3)

    t_c3, k_c3 = timed(comp3)
    t_m3, k_m3 = timed(mav3)
    return {"workload": f"one {n}-token prompt: block compression of {H} sender heads (tau={tau}), then "
                        f"mapped x V of {y['n_recv']} receiver heads (learned M, token-major bf16 V, d=128)",
            "H1_tokens_per_s": round(n / (t_m * 1e-3), 1), "H1_ms": round(t_m, 4),
            "H2_tokens_per_s": round(n / (t_c * 1e-3), 1), "H2_ms": round(t_c, 4),
            "kept_block_fraction": round(nnz / (H * (n // 64) * (n // 64 + 1) // 2), 4),
            "kernel_ms": {**k_c, **k_m},
            "H3_workload": f"{P3} prompts of {n} tokens, one mapped layer: block compression of {Hs3} sender "
                           f"heads (tau={tau}), then {Hr3} receiver heads with one sender each (indexed pass, "
                           "token-major bf16 V)",
            "H3_tokens_per_s": round(P3 * n / ((t_c3 + t_m3) * 1e-3), 1), "H3_ms": round(t_c3 + t_m3, 4),
            "H3_kernel_ms": {**k_c3, **k_m3}}


def check_outputs(x, state, O, od, P, n, tau):
    """The last timed step's own outputs against the oracle, on a sample: prompt 0's
    cosine head map (argmax equal wherever the oracle's margin exceeds 1e-4, cosines
    at 1e-5), every prompt's decode row through the one-hot mapped x V (bf16, 1e-2),
    and four block-rows of the fused pass (prompts 0 and P-1): every sender whose
    oracle selection margin exceeds 1e-4 keeps exactly the oracle's columns, and O
    equals the oracle's product over the kept columns (bf16, relative L2 1e-2)."""
    import oracle

    t0 = time.perf_counter()
    f64 = lambda b: (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)
    rel = lambda a, b: float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))
    Hs, Hr, tau_t, slot = x["n_send"], x["n_recv"], x["tau_t"], x["slot"]
    arg = state["arg"].cpu().numpy().astype(np.int64)
    cos_g = state["cos"].cpu().numpy().astype(np.float64) if state.get("cos") is not None else None
    out = dict(ok=True)
    # head map of prompt 0
    S = np.stack([oracle.round_bf16(oracle.pack_rows(oracle.causal_map(
        f64(x["send_q"][j, :tau_t]), f64(x["send_k"][j, :tau_t]), x["send_scale"][j], x["send_bias"][j])))
        for j in range(Hs)])
    R = np.stack([oracle.round_bf16(oracle.pack_rows(oracle.causal_map(
        f64(x["recv_q"][h, :tau_t]), f64(x["recv_k"][h, :tau_t]), x["recv_scale"][h], x["recv_bias"][h])))
        for h in range(Hr)])
    ocos, oarg, omar = oracle.head_map(R, S)
    big = omar > 1e-4
    out["head_map_decided"] = int(big.sum())
    out["head_map_ok"] = bool(np.array_equal(arg[0][big], oarg[big]) and
                              (cos_g is None or rel(cos_g[0], ocos) <= 1e-5))
    # decode rows: oracle rows over n + 1 keys, one-hot by the library's argmax
    odg = od.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for p in range(P):
        ks = slice(p * slot, p * slot + n + 1)
        A = np.stack([oracle.causal_map(f64(x["dec_q"][j, p][None, :]), f64(x["send_k"][j, ks]),
                                        x["send_scale"][j], x["send_bias"][j])[0] for j in range(Hs)])
        ref = np.stack([A[arg[p, h]] @ f64(x["v"][h, ks]) for h in range(Hr)])
        worst = max(worst, rel(odg[:, p], oracle.round_bf16(ref)))
    out["decode_rel_l2"] = round(worst, 6)
    # fused pass: sampled block-rows, reference on the library's kept columns
    bsr = state["bsr"]
    nnz = int(bsr["nnz"].item())
    row_ptr = bsr["row_ptr"].cpu().numpy().astype(np.int64)
    col = bsr["col_idx"][:nnz].cpu().numpy().astype(np.int64)
    Rb = n // 64
    r_tot = P * Rb
    M = x["M"][0].astype(np.float64)
    worst_o, decided, sel_ok = 0.0, 0, True
    for p, r in sorted({(0, 0), (0, min(64, Rb - 1)), (0, Rb - 1), (P - 1, Rb // 2)}):
        qs, ks = slice(p * n, p * n + n), slice(p * slot, p * slot + n)
        mixed = np.zeros((Hr, 64, 64 * (r + 1)))
        for j in range(Hs):
            ref = oracle.compress_block_row(f64(x["send_q"][j, qs]), f64(x["send_k"][j, ks]), x["send_scale"][j],
                                            x["send_bias"][j], r, tau)
            g = j * r_tot + p * Rb + r
            kept = [int(c) for c in col[row_ptr[g]: row_ptr[g + 1]]]
            if ref["margin"] > 1e-4:
                decided += 1
                sel_ok &= kept == ref["kept"]
            A = np.zeros((64, 64 * (r + 1)))
            for c in kept:
                A[:, 64 * c: 64 * c + 64] = oracle.round_bf16(ref["rows"][:, 64 * c: 64 * c + 64])
            mixed += M[:, j, None, None] * A[None]
        Vp = f64(x["v"][:, p * slot: p * slot + 64 * (r + 1)])
        ref_o = np.stack([mixed[h] @ Vp[h] for h in range(Hr)])
        got = O[:, p * n + 64 * r: p * n + 64 * r + 64].float().cpu().numpy().astype(np.float64)
        worst_o = max(worst_o, rel(got, oracle.round_bf16(ref_o)))
    out["fused_rel_l2"] = round(worst_o, 6)
    out["fused_decided_selections"] = decided
    out["selections_ok"] = bool(sel_ok)
    out["ok"] = bool(out["head_map_ok"] and sel_ok and worst <= 1e-2 and worst_o <= 1e-2)
    out["seconds"] = round(time.perf_counter() - t0, 1)
    return out


def cpu_baseline(x, P, n, tokens, tau):
    """The oracle, as it stands, on a bounded sample of one step; scaled to tokens/s.

    Sample (prompt 0 only): all 56 prefix maps and the 24 x 32 cosine problem;
    block compression of 1 of the 32 sender heads; the mapped x V pass for five
    block-rows spread over the prompt (r = 0, 31, 63, 95, 127); the decode row.
    Each part is scaled by the fraction of the step it covers.
    """
    import oracle
    import synth

    cores = len(os.sched_getaffinity(0))
    f64 = lambda b: synth.bf16_to_f32(b).astype(np.float64)
    tau_t, slot, Hs, Hr = x["tau_t"], x["slot"], x["n_send"], x["n_recv"]
    parts = {}
    # 1+2: prefix maps and cosine for prompt 0 (x P prompts)
    t = time.perf_counter()
    S = np.stack([oracle.round_bf16(oracle.pack_rows(oracle.causal_map(
        f64(x["send_q"][j, :tau_t]), f64(x["send_k"][j, :tau_t]), x["send_scale"][j], x["send_bias"][j])))
        for j in range(Hs)])
    R = np.stack([oracle.round_bf16(oracle.pack_rows(oracle.causal_map(
        f64(x["recv_q"][j, :tau_t]), f64(x["recv_k"][j, :tau_t]), x["recv_scale"][j], x["recv_bias"][j])))
        for j in range(Hr)])
    oracle.head_map(R, S)
    parts["maps_cosine"] = (time.perf_counter() - t) * P
    # 4: one head's compression (x Hs heads x P prompts)
    t = time.perf_counter()
    oracle.compress_head(f64(x["send_q"][0, :n]), f64(x["send_k"][0, :n]), x["send_scale"][0],
                         x["send_bias"][0], tau)
    parts["block_compress"] = (time.perf_counter() - t) * Hs * P
    # 5: mapped x V rows on a block-sparse structure holding the sampled block-rows
    R_ = n // 64
    sample = [0, 31, 63, 95, 127] if R_ == 128 else sorted(set([0, R_ // 2, R_ - 1]))
    counts = np.zeros(Hs * R_, dtype=np.int64)
    cols = []
    for j in range(Hs):
        for r in range(R_):
            if r in sample:
                counts[j * R_ + r] = r + 1
                cols.extend(range(r + 1))
    row_ptr = np.concatenate([[0], np.cumsum(counts)])
    vals = np.full((len(cols), 64, 64), 1.0 / 8192)
    V = f64(x["v"][:, :n])
    t = time.perf_counter()
    oracle.mapped_av_bsr_rows(row_ptr, np.array(cols), vals, Hs, [n], x["M"], V, np.array([0, n]),
                              [(0, r) for r in sample])
    frac = sum(r + 1 for r in sample) / (R_ * (R_ + 1) / 2)
    parts["mapped_av"] = (time.perf_counter() - t) / frac * P
    # 6: decode row for prompt 0 (x P)
    t = time.perf_counter()
    rows = np.stack([oracle.causal_map(f64(x["dec_q"][j, :1]), f64(x["send_k"][j, :n + 1]), x["send_scale"][j],
                                       x["send_bias"][j]) for j in range(Hs)])
    Mo = oracle.onehot_mix(np.arange(Hr) % Hs, Hs)
    oracle.mapped_av_dense(rows, Mo, f64(x["v"][:, :n + 1]))
    parts["decode"] = (time.perf_counter() - t) * P
    total = sum(parts.values())
    blas = "unknown"
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {}).get("name", "unknown")
    except Exception:
        pass
    return {
        "value": round(tokens / total, 3),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "blas": blas,
        "sample": "prompt 0 of the step: all 56 prefix maps + the 24x32 cosine problem (x4 prompts); "
                  "compression of 1 of 32 sender heads (x128); mapped x V for block-rows 0,31,63,95,127 "
                  "(scaled by their share of the 8256 causal blocks, x4); the decode row (x4). "
                  "Estimated oracle seconds per step: " + ", ".join(f"{k} {v:.1f}" for k, v in parts.items()),
        "est_seconds_per_step": round(total, 1),
    }


if __name__ == "__main__":
    main()
