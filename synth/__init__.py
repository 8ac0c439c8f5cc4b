"""Seeded synthetic inputs for the attention-map reuse path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no logits, softmax, cosine, block statistics or mixing).
Both the CPU oracle tests and the GPU path read the very same arrays, so the two
sides always start from identical bytes.

Conventions
-----------
* Generator: numpy PCG64 seeded with ``SeedSequence(20260000 + cfg)`` for the five
  named workloads; per-tensor streams are spawned from that sequence in the order
  documented in each function, so adding a tensor never changes earlier ones.
* bf16 tensors are held as ``uint16`` bit patterns (round-to-nearest-even from a
  float32 draw). ``bf16_to_f32`` widens them exactly.
* Layout: head-major ``[H, T, d]``; several sequences are packed along ``T`` and
  described by ``cu_seqlens`` (int32, ``n_seqs + 1`` start offsets).

The workloads stand in for the pages' models and data, which are not available:
IAM's Qwen2-72B/Qwen2-0.5B pair (512+512 at batch 64, 8192+512 at batch 4) and
MapFlow's Ministral3-8B -> 3B pair. Queries, keys and values are N(0, 1); every
head's logit scale is 1/sqrt(d) times a sharpness drawn from U[1, 4); half of the
heads of each layer get a +4 "sink" bias on key 0.
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20260000


# ----------------------------------------------------------------------------- bf16 bits
def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = np.where(nan, (u >> 16) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed_seq: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_seq))


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def head_scales(rng: np.random.Generator, n_layers: int, heads_per_layer: int, d: int,
                sharp: bool = True, sink: bool = True, sink_value: float = 4.0):
    """Per-head logit scale (float32, = sharpness / sqrt(d)) and key-0 bias (float32).

    Draw order: sharpness for all heads, then one permutation per layer choosing
    the sink heads (exactly half of each layer's heads, rounded down).
    """
    n = n_layers * heads_per_layer
    beta = rng.uniform(1.0, 4.0, size=n) if sharp else np.ones(n)
    scale = (beta / np.sqrt(d)).astype(np.float32)
    bias = np.zeros(n, dtype=np.float32)
    if sink:
        for layer in range(n_layers):
            pick = rng.permutation(heads_per_layer)[: heads_per_layer // 2]
            bias[layer * heads_per_layer + pick] = np.float32(sink_value)
    return scale, bias


# ----------------------------------------------------------------------------- generic
def attention_inputs(seed: int, n_heads: int, lengths, d: int = 128, dtype: str = "bf16",
                     sharp: bool = True, sink: bool = True, heads_per_layer: int | None = None,
                     k_lengths=None):
    """Q, K for ``n_heads`` heads over sequences of the given lengths.

    ``k_lengths`` (optional) makes the key side longer than the query side per
    sequence (decode rows sit at the end of their sequence).
    Stream order: [q, k, head scales].
    """
    ss = np.random.SeedSequence(seed)
    s_q, s_k, s_h = ss.spawn(3)
    lq = list(lengths)
    lk = list(k_lengths) if k_lengths is not None else lq
    tq, tk = int(sum(lq)), int(sum(lk))
    if dtype == "bf16":
        q = _normal_bf16(_rng(s_q), (n_heads, tq, d))
        k = _normal_bf16(_rng(s_k), (n_heads, tk, d))
    else:
        q = _rng(s_q).standard_normal(size=(n_heads, tq, d), dtype=np.float32)
        k = _rng(s_k).standard_normal(size=(n_heads, tk, d), dtype=np.float32)
    hpl = heads_per_layer or n_heads
    scale, bias = head_scales(_rng(s_h), n_heads // hpl, hpl, d, sharp=sharp, sink=sink)
    return dict(q=q, k=k, scale=scale, bias=bias, cu_q=cu_from_lengths(lq),
                cu_k=cu_from_lengths(lk), d=d, dtype=dtype)


def values(seed: int, n_heads: int, total: int, d: int = 128, dtype: str = "bf16"):
    rng = _rng(np.random.SeedSequence(seed))
    if dtype == "bf16":
        return _normal_bf16(rng, (n_heads, total, d))
    return rng.standard_normal(size=(n_heads, total, d), dtype=np.float32)


def mix_matrix_learned(seed: int, n_recv: int, n_send: int, n_batch: int = 1, sigma: float = 0.2):
    """Learned-style head mixing weights: N(0, sigma) plus 1.0 on the diagonal h == j."""
    rng = _rng(np.random.SeedSequence(seed))
    m = rng.normal(0.0, sigma, size=(n_batch, n_recv, n_send))
    for h in range(min(n_recv, n_send)):
        m[:, h, h] += 1.0
    return m.astype(np.float32)


# ----------------------------------------------------------------------------- named workloads
D = 128


def cfg1():
    """Tiny fp32 case: one 128-token sequence, d = 64, sender 4 heads, receiver 2 heads.

    Scale 1/8 (= 1/sqrt(64)), no sharpness, no sink. Stream order:
    [sender q, sender k, receiver q, receiver k, receiver v, M].
    """
    ss = np.random.SeedSequence(BASE_SEED + 1)
    s = ss.spawn(6)
    n, d = 128, 64
    f = lambda st, h: _rng(st).standard_normal(size=(h, n, d), dtype=np.float32)
    out = dict(
        send_q=f(s[0], 4), send_k=f(s[1], 4), recv_q=f(s[2], 2), recv_k=f(s[3], 2),
        v=f(s[4], 2), d=d, n=n,
        send_scale=np.full(4, 0.125, np.float32), send_bias=np.zeros(4, np.float32),
        recv_scale=np.full(2, 0.125, np.float32), recv_bias=np.zeros(2, np.float32),
        cu=cu_from_lengths([n]),
    )
    m = _rng(s[5]).uniform(0.0, 1.0, size=(1, 2, 4))
    out["M"] = (m / m.sum(axis=2, keepdims=True)).astype(np.float32)
    return out


def cfg2(n_slm_layers: int = 24, n_llm_layers: int = 40, n: int = 512):
    """IAM head mapping on one 512-token prompt.

    SLM: 24 layers x 14 heads = 336 maps; LLM mapped layers: 40 x 64 = 2560 maps.
    The SLM and LLM rows are stacked along the head axis: heads [0, 336) are the
    SLM (sender) maps and [336, 2896) the LLM (receiver) maps. Smaller layer
    counts give the same distribution at reduced size.
    Stream order: [slm q, slm k, slm heads, llm q, llm k, llm heads].
    """
    ss = np.random.SeedSequence(BASE_SEED + 2)
    s = ss.spawn(6)
    hs, hr = n_slm_layers * 14, n_llm_layers * 64
    q_s = _normal_bf16(_rng(s[0]), (hs, n, D))
    k_s = _normal_bf16(_rng(s[1]), (hs, n, D))
    sc_s, b_s = head_scales(_rng(s[2]), n_slm_layers, 14, D)
    q_r = _normal_bf16(_rng(s[3]), (hr, n, D))
    k_r = _normal_bf16(_rng(s[4]), (hr, n, D))
    sc_r, b_r = head_scales(_rng(s[5]), n_llm_layers, 64, D)
    return dict(send_q=q_s, send_k=k_s, send_scale=sc_s, send_bias=b_s,
                recv_q=q_r, recv_k=k_r, recv_scale=sc_r, recv_bias=b_r,
                cu=cu_from_lengths([n]), n=n, d=D, n_send=hs, n_recv=hr)


def cfg3(n: int = 8192, n_heads: int = 32, tau: float = 0.95):
    """Block-sparse compression input: 32 heads, one 8192-token sequence, d = 128.

    Stream order: [q, k, heads]. Sharpness and sink as for the IAM workload, with
    the 32 heads treated as one layer.
    """
    ss = np.random.SeedSequence(BASE_SEED + 3)
    s = ss.spawn(3)
    q = _normal_bf16(_rng(s[0]), (n_heads, n, D))
    k = _normal_bf16(_rng(s[1]), (n_heads, n, D))
    scale, bias = head_scales(_rng(s[2]), 1, n_heads, D)
    return dict(q=q, k=k, scale=scale, bias=bias, cu=cu_from_lengths([n]), n=n, d=D,
                tau=float(tau), n_heads=n_heads)


def cfg4(n: int = 8192, n_recv: int = 24, n_send: int = 32):
    """Fused mapped x V pass: receiver V [24, 8192, 128] bf16 and M [24, 32] fp32.

    The sender's block-sparse maps are the compressor's output on the cfg3 input.
    Stream order: [v, M].
    """
    ss = np.random.SeedSequence(BASE_SEED + 4)
    s = ss.spawn(2)
    v = _normal_bf16(_rng(s[0]), (n_recv, n, D))
    r = _rng(s[1])
    m = r.normal(0.0, 0.2, size=(1, n_recv, n_send))
    for h in range(min(n_recv, n_send)):
        m[0, h, h] += 1.0
    return dict(v=v, M=m.astype(np.float32), n=n, d=D, n_recv=n_recv, n_send=n_send)


def cfg5_lengths(n_short: int = 64, short: int = 512, n_long: int = 4, long: int = 8192,
                 decode: int = 512):
    """Prompt lengths and key-side storage lengths of the serving mix.

    Short prompts reserve room for their decode steps on the key/value side.
    """
    prompt = [short] * n_short + [long] * n_long
    store = [short + decode] * n_short + [long] * n_long
    return prompt, store


def cfg5_layer(slot: int, n_short: int = 64, short: int = 512, n_long: int = 4, long: int = 8192,
               decode: int = 512, n_send: int = 28, n_recv: int = 64, tau_t: int = 512):
    """Inputs of one mapped layer of the batched varlen serving mix.

    * sender Q for the prompt tokens ``[28, T_prompt, 128]`` (packed by prompt lengths),
    * sender K on the key-side layout ``[28, T_store, 128]`` (short prompts reserve
      ``decode`` slots for generated tokens),
    * sender decode queries ``[decode, 28, n_short, 128]`` (step-major, one row per
      short prompt per step),
    * receiver Q/K on each prompt's first ``tau_t`` tokens ``[64, n_prompts * tau_t, 128]``
      (used only to build the head map),
    * receiver V on the key-side layout ``[64, T_store, 128]``.

    Two independently seeded layers (slot 0 and 1) alternate over the mapped-layer
    slots. Stream order: [send q, send k, send heads, send decode q, recv q, recv k,
    recv heads, v].
    """
    ss = np.random.SeedSequence([BASE_SEED + 5, slot])
    s = ss.spawn(8)
    prompt, store = cfg5_lengths(n_short, short, n_long, long, decode)
    tp, ts = sum(prompt), sum(store)
    n_pr = len(prompt)
    out = dict(
        send_q=_normal_bf16(_rng(s[0]), (n_send, tp, D)),
        send_k=_normal_bf16(_rng(s[1]), (n_send, ts, D)),
    )
    out["send_scale"], out["send_bias"] = head_scales(_rng(s[2]), 1, n_send, D)
    out["send_dec_q"] = _normal_bf16(_rng(s[3]), (decode, n_send, n_short, D))
    out["recv_q"] = _normal_bf16(_rng(s[4]), (n_recv, n_pr * tau_t, D))
    out["recv_k"] = _normal_bf16(_rng(s[5]), (n_recv, n_pr * tau_t, D))
    out["recv_scale"], out["recv_bias"] = head_scales(_rng(s[6]), 1, n_recv, D)
    out["v"] = _normal_bf16(_rng(s[7]), (n_recv, ts, D))
    out.update(prompt_lengths=prompt, store_lengths=store, cu_prompt=cu_from_lengths(prompt),
               cu_store=cu_from_lengths(store), tau_t=tau_t, n_short=n_short, decode=decode,
               n_send=n_send, n_recv=n_recv, d=D)
    return out


def prefill_batch(n_prompts: int = 4, n: int = 8192, n_send: int = 32, n_recv: int = 24,
                  tau_t: int = 512, seed_offset: int = 0):
    """Long-context prefill batch: ``n_prompts`` prompts of ``n`` tokens, one mapped layer.

    The Ministral-like 8B -> 3B pair of the block-sparse workloads (32 sender
    heads, 24 receiver heads, d = 128), batched as in IAM's long-context setting
    (8192-token prompts at batch 4). Key-side tensors reserve one extra slot per
    prompt (rounded up to 8 rows) for the first generated token.

    * ``send_q`` [32, P*n, 128]; ``send_k`` [32, P*slot, 128] (prompt keys + decode key)
    * ``recv_q``/``recv_k`` [24, P*tau_t, 128]: the receiver's own queries/keys on each
      prompt's first tau_t tokens (IAM's truncated head-mapping input)
    * ``v`` [24, P*slot, 128]: receiver values for prompt and decode keys
    * ``dec_q`` [32, P, 128]: sender query of the first generated token per prompt
    * ``M`` [1, 24, 32]: learned-style mixing weights (N(0, 0.2) + 1 on the diagonal)
    Stream order: [send q, send k, send heads, recv q, recv k, recv heads, v, M, dec q].
    """
    ss = np.random.SeedSequence([BASE_SEED + 40 + seed_offset, n_prompts, n])
    s = ss.spawn(9)
    slot = (n + 1 + 7) // 8 * 8
    out = dict(
        send_q=_normal_bf16(_rng(s[0]), (n_send, n_prompts * n, D)),
        send_k=_normal_bf16(_rng(s[1]), (n_send, n_prompts * slot, D)),
    )
    out["send_scale"], out["send_bias"] = head_scales(_rng(s[2]), 1, n_send, D)
    out["recv_q"] = _normal_bf16(_rng(s[3]), (n_recv, n_prompts * tau_t, D))
    out["recv_k"] = _normal_bf16(_rng(s[4]), (n_recv, n_prompts * tau_t, D))
    out["recv_scale"], out["recv_bias"] = head_scales(_rng(s[5]), 1, n_recv, D)
    out["v"] = _normal_bf16(_rng(s[6]), (n_recv, n_prompts * slot, D))
    r = _rng(s[7])
    m = r.normal(0.0, 0.2, size=(1, n_recv, n_send))
    for h in range(min(n_recv, n_send)):
        m[0, h, h] += 1.0
    out["M"] = m.astype(np.float32)
    out["dec_q"] = _normal_bf16(_rng(s[8]), (n_send, n_prompts, D))
    out.update(n_prompts=n_prompts, n=n, slot=slot, tau_t=tau_t, n_send=n_send, n_recv=n_recv, d=D,
               cu_q=cu_from_lengths([n] * n_prompts), cu_k=cu_from_lengths([slot] * n_prompts),
               cu_t=cu_from_lengths([tau_t] * n_prompts))
    return out


def long_decode(n_prompts: int = 4, n: int = 8192, decode: int = 512, n_send: int = 32, n_recv: int = 24):
    """IAM's long-context decode: ``n_prompts`` prompts of ``n`` tokens, each followed
    by ``decode`` generated tokens whose mapped layers reuse the sender's attention
    row over the growing context (8192 + 512 at batch 4 in the IAM efficiency setting).

    * ``send_k`` [32, P*(n+decode), 128]: sender keys of the prompt and generated tokens
    * ``dec_q`` [decode, 32, P, 128]: sender query of each generated token (step-major)
    * ``v`` [24, P*(n+decode), 128]: receiver values of the same positions
    * ``M`` [1, 24, 32]: learned-style mixing weights (N(0, 0.2) + 1 on the diagonal)
    Stream order: [send k, send heads, dec q, v, M].
    """
    ss = np.random.SeedSequence([BASE_SEED + 45, n_prompts, n, decode])
    s = ss.spawn(5)
    ctx = n + decode
    out = dict(send_k=_normal_bf16(_rng(s[0]), (n_send, n_prompts * ctx, D)))
    out["send_scale"], out["send_bias"] = head_scales(_rng(s[1]), 1, n_send, D)
    out["dec_q"] = _normal_bf16(_rng(s[2]), (decode, n_send, n_prompts, D))
    out["v"] = _normal_bf16(_rng(s[3]), (n_recv, n_prompts * ctx, D))
    r = _rng(s[4])
    m = r.normal(0.0, 0.2, size=(1, n_recv, n_send))
    for h in range(min(n_recv, n_send)):
        m[0, h, h] += 1.0
    out["M"] = m.astype(np.float32)
    out.update(n_prompts=n_prompts, n=n, decode=decode, ctx=ctx, n_send=n_send, n_recv=n_recv, d=D,
               cu_k=cu_from_lengths([ctx] * n_prompts))
    return out
